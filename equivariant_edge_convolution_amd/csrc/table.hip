// Radial tables: the radial chain up to the folded last layer, r -> s2(r) =
// silu(silu(b(r) W1) W2) (64 hidden units per species pair), as piecewise
// polynomials of degree 10 on dyadic pieces of [0, rc] ("FastMACE rewrite
// screens", OPT6-T05 radial_tables: per species pair, degree-10 Chebyshev
// tables on dyadic pieces, values and r-derivatives certified against
// binary64; OPT6-T04 for the accuracy premise).
//
// Pieces: 2^K coarse pieces of width h0 = rc / 2^K, coarse piece c split into
// 2^d(c) equal sub-pieces, d(c) <= TAB_DMAX the smallest level at which the
// binary64 interpolants are within TAB_TOL of the network (the short-range
// pieces, where the chain's amplitude is largest, take the finest levels).
// Built in binary64 once per model: each sub-piece is interpolated at the 11
// Chebyshev points of the first kind, and the interpolant is stored in float32
// in power form in the sub-piece variable t in [-1, 1]
//   r = c h0 + (f + (t + 1) / 2) h0 / 2^d,   s2_j(r) ~ sum_m a[c][f][m][j] t^m,
// which Horner's rule evaluates in float32 (on these pieces the power-form
// coefficients of the interpolant stay within a small multiple of the
// function's size, so no cancellation is amplified).  The certificate is the
// largest error of the stored (float32) table against the binary64 network,
// for values and for r-derivatives, each relative to the largest magnitude of
// that output over its piece, over 16 points per piece between the nodes.
#include <math.h>

#include "eec_device.hpp"
#include "eec_internal.hpp"

namespace eec {
namespace {

constexpr int TAB_T = 64;       // one thread per hidden unit
constexpr int CHECKS = 16;      // certificate points per piece

// s2(r) and ds2/dr of one pair in binary64, thread j = hidden unit j; the
// basis, z1 and s1 go through LDS.
struct Net64 {
  double b[NB], db[NB];
  double s1[HID], ds1[HID];
};

__device__ void net64(double r, double rc, const float* __restrict__ W1, const float* __restrict__ W2, Net64& sh,
                      double& s2, double& ds2) {
  const int j = threadIdx.x;
  if (j < NB) {
    const double n = (double)(j + 1), x = r / rc;
    double sn, cn;
    sincos(n * PI / rc * r, &sn, &cn);
    double u = 0.0, du = 0.0;
    if (x < 1.0) {
      const double x2 = x * x, x5 = x2 * x2 * x, x6 = x5 * x;
      u = 1.0 + x6 * (-28.0 + x * (48.0 - 21.0 * x));
      du = -168.0 * x5 * (1.0 - x) * (1.0 - x) / rc;
    }
    const double b = sn / r * u;
    sh.b[j] = b;
    sh.db[j] = (n * PI / rc * cn * u + sn * du) / r - b / r;
  }
  __syncthreads();
  double z1 = 0.0, dz1 = 0.0;
  for (int n = 0; n < NB; ++n) {
    const double w = (double)W1[n * HID + j];
    z1 += sh.b[n] * w;
    dz1 += sh.db[n] * w;
  }
  {
    const double sg = 1.0 / (1.0 + exp(-z1));
    sh.s1[j] = z1 * sg;
    sh.ds1[j] = sg * (1.0 + z1 * (1.0 - sg)) * dz1;
  }
  __syncthreads();
  double z2 = 0.0, dz2 = 0.0;
  for (int k = 0; k < HID; ++k) {
    const double w = (double)W2[k * HID + j];
    z2 += sh.s1[k] * w;
    dz2 += sh.ds1[k] * w;
  }
  const double sg = 1.0 / (1.0 + exp(-z2));
  s2 = z2 * sg;
  ds2 = sg * (1.0 + z2 * (1.0 - sg)) * dz2;
  __syncthreads();  // sh is rewritten by the next call
}

// Largest of v over the block's 64 threads (every thread gets it).
__device__ double block_max(double v, double* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  __syncthreads();
  if (threadIdx.x == 0) red[0] = v;
  __syncthreads();
  return red[0];
}

// Block (pair p, coarse piece c), 64 threads (thread j = unit j).  Levels d =
// 0, 1, ... are tried in turn: the 2^d sub-pieces of c are interpolated and
// the binary64 interpolants checked against the network at CHECKS points per
// sub-piece; the first level whose errors (values and r-derivatives, relative
// to each unit's largest magnitude over the sub-piece) are all <= TAB_TOL is
// kept (else the last).  Slots f < 2^d of c hold its sub-pieces, the unused
// slots f >= 2^d zeros (every word of the table is written).
__global__ void __launch_bounds__(TAB_T) k_table_build(int K, double rc, const float* __restrict__ W1,
                                                       const float* __restrict__ W2, float* __restrict__ tab,
                                                       int32_t* __restrict__ level,
                                                       unsigned long long* __restrict__ cert) {
  __shared__ Net64 sh;
  __shared__ double red[1];
  const int nc = 1 << K, p = blockIdx.x / nc, c = blockIdx.x % nc, j = threadIdx.x;
  const float* w1 = W1 + (size_t)p * NB * HID;
  const float* w2 = W2 + (size_t)p * HID * HID;
  const double h0 = rc / (double)nc;
  double cv = 0.0, cd = 0.0;  // certificate of the kept level (float32 coefficients)
  int kept = TAB_DMAX;
  for (int d = 0; d <= TAB_DMAX; ++d) {
    const int nf = 1 << d;
    const double h = ldexp(h0, -d);
    double tv = 0.0, td = 0.0;  // truncation errors of this level (binary64 coefficients)
    cv = 0.0;
    cd = 0.0;
    for (int f = 0; f < nf; ++f) {
      const double r0 = c * h0 + f * h;
      double fv[TAB_NC];
      double scale = 0.0, dscale = 0.0;
      for (int i = 0; i < TAB_NC; ++i) {
        const double x = cos(PI * (i + 0.5) / TAB_NC);
        double v, dv;
        net64(r0 + 0.5 * (x + 1.0) * h, rc, w1, w2, sh, v, dv);
        fv[i] = v;
        scale = fmax(scale, fabs(v));
        dscale = fmax(dscale, fabs(dv));
      }
      double cc[TAB_NC];
      for (int m = 0; m < TAB_NC; ++m) {
        double acc = 0.0;
        for (int i = 0; i < TAB_NC; ++i) acc += fv[i] * cos(PI * m * (i + 0.5) / TAB_NC);
        cc[m] = (m == 0 ? 1.0 : 2.0) / TAB_NC * acc;
      }
      // power form: a = sum_m c_m (power coefficients of T_m), T_{m+1} = 2 t T_m - T_{m-1}
      double a[TAB_NC], tm1[TAB_NC], tm[TAB_NC];
      for (int q = 0; q < TAB_NC; ++q) {
        a[q] = 0.0;
        tm1[q] = 0.0;
        tm[q] = 0.0;
      }
      tm1[0] = 1.0;
      tm[1] = 1.0;
      a[0] = cc[0];
      for (int q = 0; q < TAB_NC; ++q) a[q] += cc[1] * tm[q];
      for (int m = 2; m < TAB_NC; ++m) {
        double nx[TAB_NC];
        nx[0] = -tm1[0];
        for (int q = 1; q < TAB_NC; ++q) nx[q] = 2.0 * tm[q - 1] - tm1[q];
        for (int q = 0; q < TAB_NC; ++q) {
          tm1[q] = tm[q];
          tm[q] = nx[q];
          a[q] += cc[m] * nx[q];
        }
      }
      float af[TAB_NC];
      float* out = tab + (((size_t)(p * nc + c) * TAB_SUB + f) * TAB_NC) * HID + 2 * (j & 31) + (j >> 5);
      for (int m = 0; m < TAB_NC; ++m) {
        af[m] = (float)a[m];
        out[m * HID] = af[m];
      }
      double ev = 0.0, ed = 0.0, fev = 0.0, fed = 0.0;
      for (int q = 0; q < CHECKS; ++q) {
        const double t = -1.0 + (2.0 * q + 1.0) / CHECKS;
        double v, dv;
        net64(r0 + 0.5 * (t + 1.0) * h, rc, w1, w2, sh, v, dv);
        scale = fmax(scale, fabs(v));
        dscale = fmax(dscale, fabs(dv));
        double pv = a[TAB_NC - 1], pd = 0.0, qv = (double)af[TAB_NC - 1], qd = 0.0;
        for (int m = TAB_NC - 2; m >= 0; --m) {
          pd = pd * t + pv;
          pv = pv * t + a[m];
          qd = qd * t + qv;
          qv = qv * t + (double)af[m];
        }
        ev = fmax(ev, fabs(pv - v));
        ed = fmax(ed, fabs(pd * (2.0 / h) - dv));
        fev = fmax(fev, fabs(qv - v));
        fed = fmax(fed, fabs(qd * (2.0 / h) - dv));
      }
      auto rel = [](double e, double sc) {
        const double x = sc > 0.0 ? e / sc : (e > 0.0 ? INFINITY : 0.0);
        return x != x ? INFINITY : x;
      };
      tv = fmax(tv, rel(ev, scale));
      td = fmax(td, rel(ed, dscale));
      cv = fmax(cv, rel(fev, scale));
      cd = fmax(cd, rel(fed, dscale));
    }
    const double worst = block_max(fmax(tv, td), red);
    if (worst <= TAB_TOL || d == TAB_DMAX) {
      if (j == 0) level[p * nc + c] = d;
      kept = d;
      break;
    }
  }
  for (int f = 1 << kept; f < TAB_SUB; ++f) {
    float* out = tab + (((size_t)(p * nc + c) * TAB_SUB + f) * TAB_NC) * HID + 2 * (j & 31) + (j >> 5);
    for (int m = 0; m < TAB_NC; ++m) out[m * HID] = 0.f;
  }
  if (cert != nullptr) {
    atomicMax(cert, (unsigned long long)__double_as_longlong(cv));
    atomicMax(cert + 1, (unsigned long long)__double_as_longlong(cd));
  }
}

__global__ void k_cert_clear(unsigned long long* cert) {
  if (threadIdx.x < 2) cert[threadIdx.x] = 0ull;
}

}  // namespace

size_t table_floats(int n_species, int log2_pieces) {
  return (size_t)n_species * n_species * ((size_t)1 << log2_pieces) * TAB_SUB * TAB_NC * HID;
}

size_t table_levels(int n_species, int log2_pieces) {
  return (size_t)n_species * n_species * ((size_t)1 << log2_pieces);
}

void launch_table_build(hipStream_t s, const eec_model* m, int log2_pieces, float* tab, int32_t* level,
                        double* cert) {
  auto* c = reinterpret_cast<unsigned long long*>(cert);
  if (c != nullptr) k_cert_clear<<<1, 64, 0, s>>>(c);
  const int P = m->n_species * m->n_species;
  k_table_build<<<P << log2_pieces, TAB_T, 0, s>>>(log2_pieces, m->cutoff, m->W1, m->W2, tab, level, c);
}

}  // namespace eec

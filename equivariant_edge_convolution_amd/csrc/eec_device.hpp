// Device building blocks shared by the gfx950 kernels of the edge convolution.
//
// Lane conventions (wave64, FP32 matrix cores, v_mfma_f32_32x32x2_f32):
//   A operand lane l holds A[l % 32][l / 32], B operand lane l holds
//   B[l / 32][l % 32], and accumulator register r of lane l holds
//   D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
// An edge tile is 32 edges; edge slot s = l % 32 and the lane half h = l / 32.
// With edges on the N (column) side, the accumulator registers of one layer are
// directly the B operand of the next layer (the K index is permuted the same
// way on the weight side), so the three-layer radial chain runs without any
// cross-lane data movement.  In that layout, register r of 32-row tile t of a
// lane in half h holds feature 32 t + fperm(r) + 4 h of edge s.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace eec {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int NB = 32;   // radial basis functions
constexpr int HID = 64;  // hidden width of the radial network
constexpr int NLM = 16;  // (lmax + 1)^2 harmonics, lmax = 3
constexpr double PI = 3.14159265358979323846;

// Row (within a 32-row accumulator tile, lane half 0) held by accumulator register r.
__device__ __forceinline__ constexpr int fperm(int r) { return ((r >> 2) << 3) | (r & 3); }

// Basis row index carried by row rho of the transposed-W1 tile, chosen so that a
// lane in half h holds basis functions 16 h .. 16 h + 15 in registers 0..15.
__device__ __forceinline__ int basis_of_row(int rho) {
  int h = (rho >> 2) & 1;
  int r = ((rho >> 3) << 2) | (rho & 3);
  return 16 * h + r;
}

__device__ __forceinline__ f32x16 mfma32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// 16x16x4 tiles: A lane l holds A[l % 16][l / 16], B lane l holds
// B[l / 16][l % 16], accumulator register i of lane l holds D[4 (l / 16) + i][l % 16].
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 zero4() {
  f32x4 z;
#pragma unroll
  for (int i = 0; i < 4; ++i) z[i] = 0.f;
  return z;
}

// Exchange 16-lane rows between two registers: on return `a` holds rows
// (a0, b0, a2, b2) and `b` rows (a1, b1, a3, b3) of the inputs (row k = lanes
// 16 k .. 16 k + 15).  Regroups a 32-wide tile layout into 16-wide ones.
__device__ __forceinline__ void swap_rows16(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// dE/dd of an edge: one 12-byte row (three floats, no padding) of the
// gradient array g [E][3], written by the backward kernels and gathered by
// the force scatter.
__device__ __forceinline__ void store_grad_row(float* __restrict__ g, int64_t e, float x, float y, float z) {
  static_assert(sizeof(float3) == 12, "float3 rows of 12 bytes");
  *reinterpret_cast<float3*>(g + 3 * e) = make_float3(x, y, z);
}
__device__ __forceinline__ float3 load_grad_row(const float* __restrict__ g, int64_t e) {
  return *reinterpret_cast<const float3*>(g + 3 * e);
}

// XOR-swizzled row-major weight tile in LDS: element (row, col) of a matrix
// with `ncols` columns (a multiple of 32).  Reads along a row (lanes over
// columns) and down a column (lanes over rows) are both bank-conflict free.
__device__ __forceinline__ int swz(int row, int col, int ncols) {
  return row * ncols + (col ^ (row & 31));
}

// ---------------------------------------------------------------- geometry
// d = (x_j - x_i) + n * L component-wise in binary64, r2 = (dx*dx + dy*dy) + dz*dz,
// with no contraction into fused multiply-adds, so that the cutoff decision
// and the edge vector are the same bits the neighbour list used.
__device__ __forceinline__ void edge_vector(const double* __restrict__ pos, int i, int j,
                                            const int8_t* __restrict__ sh, double Lx, double Ly,
                                            double Lz, double d[3]) {
#pragma clang fp contract(off)
  d[0] = (pos[3 * j + 0] - pos[3 * i + 0]) + (double)sh[0] * Lx;
  d[1] = (pos[3 * j + 1] - pos[3 * i + 1]) + (double)sh[1] * Ly;
  d[2] = (pos[3 * j + 2] - pos[3 * i + 2]) + (double)sh[2] * Lz;
}

__device__ __forceinline__ double norm2_nofma(const double d[3]) {
#pragma clang fp contract(off)
  double r2 = (d[0] * d[0] + d[1] * d[1]) + d[2] * d[2];
  return r2;
}

// ---------------------------------------------------------------- basis
// Polynomial cutoff envelope of exponent 6 and its derivative (binary64).
__device__ __forceinline__ double envelope(double x) {
  if (x >= 1.0) return 0.0;
  double x2 = x * x, x3 = x2 * x, x6 = x3 * x3;
  return 1.0 + x6 * (-28.0 + x * (48.0 - 21.0 * x));
}
__device__ __forceinline__ double envelope_d(double x) {
  if (x >= 1.0) return 0.0;
  double x2 = x * x, x5 = x2 * x2 * x, om = 1.0 - x;
  return -168.0 * x5 * om * om;
}

// Start of the basis recurrence of a lane half h: the sine and cosine of
// n0 theta, n0 = 16 h + 1, theta = pi r / rc, and of the step theta.  One
// binary64 sincos; the n0 = 17 start comes from four angle doublings
// (16 theta) and one rotation by theta, which costs a few ulps of binary64.
struct BasisStart {
  double s, c;    // sin, cos of n0 theta
  double sp, cp;  // sin, cos of (n0 - 1) theta
  double c1;      // cos theta
};

__device__ __forceinline__ BasisStart basis_start(double r, double rc, int h) {
  BasisStart b;
  double s1, c1;
  sincos(PI / rc * r, &s1, &c1);
  double s = s1, c = c1;
#pragma unroll
  for (int k = 0; k < 4; ++k) {  // 2^4 theta
    const double s2 = 2.0 * s * c;
    const double c2 = (c - s) * (c + s);
    s = s2;
    c = c2;
  }
  const double s17 = s * c1 + c * s1, c17 = c * c1 - s * s1;
  b.s = h ? s17 : s1;
  b.c = h ? c17 : c1;
  b.sp = h ? s : 0.0;
  b.cp = h ? c : 1.0;
  b.c1 = c1;
  return b;
}

// Basis functions n = n0 .. n0 + 15 of b_n = sin(n pi r / rc) / r * env(r / rc)
// by the three-term recurrence sin((n+1)t) = 2 cos t sin(nt) - sin((n-1)t) (and
// the same for cos) in binary64 from a BasisStart; optionally db_n / dr.
template <bool DERIV>
__device__ __forceinline__ void basis16_from(const BasisStart& st, double r, double rc, int n0,
                                             float b[16], float db[16]) {
  double s = st.s, sp = st.sp, c = st.c, cp = st.cp;
  const double two_c1 = 2.0 * st.c1;
  const double x = r / rc;
  const double env = envelope(x);
  const double inv_r = 1.0 / r;
  const double A = inv_r * env;                                        // b_n = s_n A
  const double Bd = DERIV ? inv_r * (envelope_d(x) / rc - A) : 0.0;   // db_n = c_n n k A + s_n Bd
  const double kA0 = PI / rc * A;
  double kA = (double)n0 * kA0;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    b[k] = (float)(s * A);
    if (DERIV) {
      db[k] = (float)(c * kA + s * Bd);
      kA += kA0;
      const double cn = two_c1 * c - cp;
      cp = c;
      c = cn;
    }
    const double sn = two_c1 * s - sp;
    sp = s;
    s = sn;
  }
}

// Basis functions n0 = 16 h + 1 .. 16 h + 16 of a lane half h (and derivatives).
template <bool DERIV>
__device__ __forceinline__ void basis16(double r, double rc, int n0, float b[16], float db[16]) {
  const BasisStart st = basis_start(r, rc, n0 > 1 ? 1 : 0);
  basis16_from<DERIV>(st, r, rc, n0, b, db);
}

// Float32 basis of the folded kernels (float32, as the rest of the network).
// x = r / rc is carried as a float32 head and tail.  Lane half h starts its
// recurrence from the angle pi x (h = 0) or 16 pi x (h = 1; 16 x is exact in
// float32): sincospif of the head, corrected to first order by the tail, so
// both starts carry the binary64 x and neither is built by angle doublings
// (whose errors grow with every doubling and bias the upper half).
struct BasisSeed {
  float x, xl;    // r / rc: float32 head and tail
  float s1, c1;   // sin, cos of pi x (every lane)
  float sa, ca;   // sin, cos of m pi x, m = 1 (h = 0) or 16 (h = 1)
  float inv_r;
};

// Lanes 0-31 of v to both halves of the wave.
__device__ __forceinline__ float lower_half(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]);
}

__device__ __forceinline__ void sincos_pi_split(float xh, float xl, float m, float& s, float& c) {
  float sh, ch;
  sincospif(m * xh, &sh, &ch);
  const float d = (float)PI * (m * xl);
  s = fmaf(d, ch, sh);
  c = fmaf(-d, sh, ch);
}

// The seed of an edge from its binary64 length (lane half h; the two halves of
// the wave hold the same edges).
__device__ __forceinline__ BasisSeed basis_seed(double r, double inv_rc, float inv_r, int h) {
  const double xd = r * inv_rc;
  BasisSeed sd;
  sd.x = (float)xd;
  sd.xl = (float)(xd - (double)sd.x);
  sincos_pi_split(sd.x, sd.xl, h ? 16.f : 1.f, sd.sa, sd.ca);
  sd.s1 = lower_half(sd.sa);
  sd.c1 = lower_half(sd.ca);
  sd.inv_r = inv_r;
  return sd;
}

// The same seed from a stored head, tail, sin pi x and cos pi x.
__device__ __forceinline__ BasisSeed basis_seed_stored(float x, float xl, float s1, float c1, float inv_r, int h) {
  BasisSeed sd;
  sd.x = x;
  sd.xl = xl;
  sd.s1 = s1;
  sd.c1 = c1;
  sincos_pi_split(x, xl, h ? 16.f : 1.f, sd.sa, sd.ca);
  sd.inv_r = inv_r;
  return sd;
}

// Basis functions n = 16 h + 1 .. 16 h + 16 of a lane half h in float32 (and
// db_n / dr) by the three-term recurrence sin((n+1)t) = 2 cos t sin(nt) -
// sin((n-1)t) (and the same for cos); half 1 starts at n = 17 by one rotation
// of its 16 pi x by pi x.  The envelope is zero from x = 1 on, so past the
// cutoff every b_n and db_n is an exact zero.
template <bool DERIV>
__device__ __forceinline__ void basis16f(const BasisSeed& sd, float inv_rc, int h, float b[16], float db[16]) {
  const float s17 = fmaf(sd.sa, sd.c1, sd.ca * sd.s1), c17 = fmaf(sd.ca, sd.c1, -(sd.sa * sd.s1));
  float sn = h ? s17 : sd.s1, cn = h ? c17 : sd.c1;
  float sp = h ? sd.sa : 0.f, cp = h ? sd.ca : 1.f;
  const float x = sd.x;
  float env = 0.f, envd = 0.f;
  if (x < 1.f) {
    const float x2 = x * x, x5 = x2 * x2 * x, x6 = x5 * x, om = 1.f - x;
    env = fmaf(x6, fmaf(x, fmaf(-21.f, x, 48.f), -28.f), 1.f);
    envd = -168.f * x5 * om * om * inv_rc;
  }
  const float A = sd.inv_r * env;                            // b_n = s_n A
  const float Bd = DERIV ? sd.inv_r * (envd - A) : 0.f;     // db_n = c_n n (pi / rc) A + s_n Bd
  const float kA0 = (float)PI * inv_rc * A;
  const float two_c1 = 2.f * sd.c1;
  const int n0 = 16 * h + 1;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    b[k] = sn * A;
    if (DERIV) {
      db[k] = fmaf(cn, (float)(n0 + k) * kA0, sn * Bd);
      const float cx = fmaf(two_c1, cn, -cp);
      cp = cn;
      cn = cx;
    }
    const float sx = fmaf(two_c1, sn, -sp);
    sp = sn;
    sn = sx;
  }
}

// ---------------------------------------------------------------- harmonics
// Real component-normalised harmonics l <= 3 of a unit vector (x, y, z),
// flat index l*l + l + m, m = -l..l, z polar, no Condon-Shortley phase.
struct SphC {
  static constexpr float s3 = 1.7320508075688772f;     // sqrt 3
  static constexpr float s15 = 3.8729833462074170f;    // sqrt 15
  static constexpr float s5h = 1.1180339887498949f;    // sqrt 5 / 2
  static constexpr float s15h = 1.9364916731037085f;   // sqrt 15 / 2
  static constexpr float s70q = 2.0916500663351889f;   // sqrt 70 / 4
  static constexpr float s105 = 10.246950765959598f;   // sqrt 105
  static constexpr float s42q = 1.6201851746019651f;   // sqrt 42 / 4
  static constexpr float s7h = 1.3228756555322954f;    // sqrt 7 / 2
  static constexpr float s105h = 5.1234753829797990f;  // sqrt 105 / 2
};

__device__ __forceinline__ void sph16(float x, float y, float z, float Y[16]) {
  const float x2 = x * x, y2 = y * y, z2 = z * z;
  Y[0] = 1.f;
  Y[1] = SphC::s3 * y;
  Y[2] = SphC::s3 * z;
  Y[3] = SphC::s3 * x;
  Y[4] = SphC::s15 * x * y;
  Y[5] = SphC::s15 * y * z;
  Y[6] = SphC::s5h * (3.f * z2 - 1.f);
  Y[7] = SphC::s15 * x * z;
  Y[8] = SphC::s15h * (x2 - y2);
  Y[9] = SphC::s70q * y * (3.f * x2 - y2);
  Y[10] = SphC::s105 * x * y * z;
  Y[11] = SphC::s42q * y * (5.f * z2 - 1.f);
  Y[12] = SphC::s7h * z * (5.f * z2 - 3.f);
  Y[13] = SphC::s42q * x * (5.f * z2 - 1.f);
  Y[14] = SphC::s105h * z * (x2 - y2);
  Y[15] = SphC::s70q * x * (x2 - 3.f * y2);
}

// G = sum_k w_k grad P_k(x, y, z) of the polynomials above (before projection
// onto the tangent plane of the unit sphere).
__device__ __forceinline__ void sph16_grad_dot(float x, float y, float z, const float w[16],
                                               float G[3]) {
  const float x2 = x * x, y2 = y * y, z2 = z * z;
  float gx = 0.f, gy = 0.f, gz = 0.f;
  gy += w[1] * SphC::s3;
  gz += w[2] * SphC::s3;
  gx += w[3] * SphC::s3;
  gx += w[4] * SphC::s15 * y;          gy += w[4] * SphC::s15 * x;
  gy += w[5] * SphC::s15 * z;          gz += w[5] * SphC::s15 * y;
  gz += w[6] * SphC::s5h * 6.f * z;
  gx += w[7] * SphC::s15 * z;          gz += w[7] * SphC::s15 * x;
  gx += w[8] * SphC::s15h * 2.f * x;   gy -= w[8] * SphC::s15h * 2.f * y;
  gx += w[9] * SphC::s70q * 6.f * x * y;
  gy += w[9] * SphC::s70q * 3.f * (x2 - y2);
  gx += w[10] * SphC::s105 * y * z;    gy += w[10] * SphC::s105 * x * z;
  gz += w[10] * SphC::s105 * x * y;
  gy += w[11] * SphC::s42q * (5.f * z2 - 1.f);
  gz += w[11] * SphC::s42q * 10.f * y * z;
  gz += w[12] * SphC::s7h * (15.f * z2 - 3.f);
  gx += w[13] * SphC::s42q * (5.f * z2 - 1.f);
  gz += w[13] * SphC::s42q * 10.f * x * z;
  gx += w[14] * SphC::s105h * 2.f * x * z;
  gy -= w[14] * SphC::s105h * 2.f * y * z;
  gz += w[14] * SphC::s105h * (x2 - y2);
  gx += w[15] * SphC::s70q * 3.f * (x2 - y2);
  gy -= w[15] * SphC::s70q * 6.f * x * y;
  G[0] = gx;
  G[1] = gy;
  G[2] = gz;
}

// ---------------------------------------------------------------- activations
__device__ __forceinline__ float sigmoid(float z) {
  return __builtin_amdgcn_rcpf(1.f + __expf(-z));
}
__device__ __forceinline__ float silu(float z) { return z * sigmoid(z); }
__device__ __forceinline__ float silu_d(float z) {
  const float s = sigmoid(z);
  return s * (1.f + z * (1.f - s));
}

}  // namespace eec

// Building blocks of the FP32 matrix-core radial chain shared by the kernels
// of radial.hip (direct path) and fold.hip (reassociated last layer): weight
// staging in LDS, the edge geometry of a lane, the first two network layers
// with edges on the N side, and the pair-grouped work scheduling.
#pragma once
#include <algorithm>

#include "eec_device.hpp"
#include "eec_internal.hpp"

namespace eec {
namespace chain {

constexpr int MAXP = 16;

// Weights in LDS, row-major with one padding column: a wave reading along a row
// (lanes over columns) or down a column (lanes over rows) touches 32 distinct
// banks either way, and every address is a per-lane base plus an immediate.
constexpr int LDH = HID + 1;  // row stride of W1 [32][64] and W2 [64][64]
template <int C>
struct Lds {
  static constexpr int NC = 4 * C;
  static constexpr int LD3 = NC + 1;            // row stride of W3 [64][NC]
  static constexpr int W1 = 0;
  static constexpr int W2 = W1 + NB * LDH;
  static constexpr int W3 = W2 + HID * LDH;
  static constexpr int FLOATS = W3 + HID * LD3;  // 90752 B (C=64), 156288 B (C=128)
};

struct EdgeIn {
  const double* pos;
  double Lx, Ly, Lz, rc;
  double inv_rc;              // 1 / rc
  float inv_rc_f;             // 1 / rc rounded to float32
  const int32_t* recv;
  const int32_t* col;
  const int8_t* shift;
  const int32_t* species;
  int32_t n_atoms;
  int64_t n_edges;
};

struct Sched {
  const int32_t* perm;        // pair-grouped order -> CSR edge; NULL = identity
  const int64_t* pair_start;  // [P+1] group offsets in that order; NULL = one group [0, E)
  int P;
  int64_t e0, e1;             // CSR edge range to process
};

struct SchedState {
  int64_t q0[MAXP], q1[MAXP];
  int bstart[MAXP + 1];
  int ntile[MAXP];
};

// Lower bound of CSR index `e` among positions [lo, hi) of a pair group.
__device__ __forceinline__ int64_t group_lower_bound(const int32_t* perm, int64_t lo, int64_t hi, int64_t e) {
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if ((int64_t)perm[mid] < e) lo = mid + 1; else hi = mid;
  }
  return lo;
}

template <int W>
__device__ __forceinline__ void sched_init(const Sched& sc, SchedState& st) {
  const int t = threadIdx.x;
  if (t < sc.P) {
    int64_t q0, q1;
    if (sc.perm == nullptr) {
      q0 = sc.e0;
      q1 = sc.e1;
    } else {
      const int64_t g0 = sc.pair_start[t], g1 = sc.pair_start[t + 1];
      q0 = group_lower_bound(sc.perm, g0, g1, sc.e0);
      q1 = group_lower_bound(sc.perm, q0, g1, sc.e1);
    }
    st.q0[t] = q0;
    st.q1[t] = q1;
    st.ntile[t] = (int)((q1 - q0 + 31) / 32);
  }
  __syncthreads();
  if (t == 0) {
    int acc = 0;
    for (int p = 0; p < sc.P; ++p) {
      st.bstart[p] = acc;
      acc += (st.ntile[p] + W - 1) / W;
    }
    st.bstart[sc.P] = acc;
  }
  __syncthreads();
}

// A row-major [rows][cols] global matrix (cols a multiple of 4) into LDS with
// row stride ld, by the whole workgroup: 16-byte loads when the source allows.
__device__ __forceinline__ void stage_rows(float* lds, int ld, const float* __restrict__ g, int rows, int cols,
                                           float scale = 1.f) {
  if ((reinterpret_cast<uintptr_t>(g) & 15) == 0) {
    const float4* g4 = reinterpret_cast<const float4*>(g);
    const int n4 = rows * cols / 4;
    for (int k = threadIdx.x; k < n4; k += blockDim.x) {
      const float4 v = g4[k];
      float* d = lds + ((4 * k) / cols) * ld + (4 * k) % cols;
      d[0] = v.x * scale;
      d[1] = v.y * scale;
      d[2] = v.z * scale;
      d[3] = v.w * scale;
    }
  } else {
    for (int k = threadIdx.x; k < rows * cols; k += blockDim.x) lds[(k / cols) * ld + k % cols] = g[k] * scale;
  }
}

// The same for a [ROWS][COLS] matrix staged by a workgroup of NT threads, in
// rounds: each thread issues up to STAGE_WORDS 16-byte loads before it stores
// any of them, so a round costs one memory latency (the loop above waits on
// every load before its store); the cap keeps the words in flight within the
// registers the kernels leave free.
constexpr int STAGE_WORDS = 4;
template <int ROWS, int COLS, int NT>
__device__ __forceinline__ void stage_rows_all(float* lds, int ld, const float* __restrict__ g, float scale = 1.f) {
  static_assert(COLS % 4 == 0, "rows of whole 16-byte words");
  constexpr int N4 = ROWS * COLS / 4, PER = (N4 + NT - 1) / NT;
  if ((reinterpret_cast<uintptr_t>(g) & 15) != 0) {
    stage_rows(lds, ld, g, ROWS, COLS, scale);
    return;
  }
  const float4* g4 = reinterpret_cast<const float4*>(g);
#pragma unroll
  for (int u0 = 0; u0 < PER; u0 += STAGE_WORDS) {
    constexpr int R = PER < STAGE_WORDS ? PER : STAGE_WORDS;
    float4 v[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int k = (int)threadIdx.x + (u0 + u) * NT;
      if (u0 + u < PER && k < N4) v[u] = g4[k];
    }
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int k = (int)threadIdx.x + (u0 + u) * NT;
      if (u0 + u < PER && k < N4) {
        float* d = lds + ((4 * k) / COLS) * ld + (4 * k) % COLS;
        d[0] = v[u].x * scale;
        d[1] = v[u].y * scale;
        d[2] = v[u].z * scale;
        d[3] = v[u].w * scale;
      }
    }
  }
}

template <int C, int NT>
__device__ __forceinline__ void stage_weights(float* lds, const float* __restrict__ W1, const float* __restrict__ W2,
                              const float* __restrict__ W3, int p, float w1_scale = 1.f) {
  constexpr int NC = Lds<C>::NC;
  stage_rows_all<NB, HID, NT>(lds + Lds<C>::W1, LDH, W1 + (size_t)p * NB * HID, w1_scale);
  stage_rows_all<HID, HID, NT>(lds + Lds<C>::W2, LDH, W2 + (size_t)p * HID * HID);
  stage_rows_all<HID, NC, NT>(lds + Lds<C>::W3, Lds<C>::LD3, W3 + (size_t)p * HID * NC);
}


// Schedule of a run of NMFMA matrix instructions whose B operands come from
// LDS (one read per PER instructions): PRE reads are issued ahead and each group
// of PER instructions is followed by the next read, so PRE reads stay in flight.
// Left alone the scheduler issues each read just before its use and waits on
// it, which stalls the matrix pipe for the LDS latency every PER instructions.
template <int NMFMA, int PER, int PRE>
__device__ __forceinline__ void pipeline_lds_mfma() {
  __builtin_amdgcn_sched_group_barrier(0x100, PRE, 0);
#pragma unroll
  for (int k = 0; k < NMFMA / PER - PRE; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, PER * PRE, 0);
}

// Input hidden feature of K-step ks (0..31) carried by a lane of half h when the
// 64 hidden features sit in two edges-on-N accumulator tiles: hid_k0(ks) + 4 h.
__device__ __forceinline__ constexpr int hid_k0(int ks) { return 32 * (ks >> 4) + fperm(ks & 15); }

// z1 = b W1 (edges on N): two 32-feature tiles.
__device__ __forceinline__ void layer1(const float* __restrict__ w1s, const float b[16], int s, int h,
                                       f32x16 z[2]) {
  const float* w = w1s + 16 * h * LDH + s;  // W1[16 h + ks][32 m + s]
  z[0] = zero16();
  z[1] = zero16();
#pragma unroll
  for (int ks = 0; ks < 16; ++ks)
#pragma unroll
    for (int m = 0; m < 2; ++m) z[m] = mfma32(w[ks * LDH + 32 * m], b[ks], z[m]);
  pipeline_lds_mfma<32, 2, 6>();
}

// z2 = s1 W2 (edges on N).
__device__ __forceinline__ void layer2(const float* __restrict__ w2s, const f32x16 s1[2], int s, int h,
                                       f32x16 z[2]) {
  const float* w = w2s + 4 * h * LDH + s;  // W2[hid_k0(ks) + 4 h][32 m + s]
  z[0] = zero16();
  z[1] = zero16();
#pragma unroll
  for (int ks = 0; ks < 32; ++ks) {
    const float bv = s1[ks >> 4][ks & 15];
#pragma unroll
    for (int m = 0; m < 2; ++m) z[m] = mfma32(w[hid_k0(ks) * LDH + 32 * m], bv, z[m]);
  }
  pipeline_lds_mfma<64, 2, 6>();
}

// s = silu(z) and d = silu'(z) from one sigmoid evaluation.  d is pinned to
// registers here: left to itself the compiler sinks it to its late use and
// keeps both z and the sigmoid live instead, twice the registers.
__device__ __forceinline__ void silu_and_deriv(const f32x16 z[2], f32x16 s[2], f32x16 d[2]) {
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float zz = z[m][r], sg = sigmoid(zz);
      s[m][r] = zz * sg;
      float dd = sg * (1.f + zz * (1.f - sg));
      asm volatile("" : "+v"(dd));
      d[m][r] = dd;
    }
}

__device__ __forceinline__ void silu_tiles(const f32x16 z[2], f32x16 s[2]) {
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[m][r] = silu(z[m][r]);
}

// The chain with the first layer's weights scaled by KEXP = -log2(e) (the
// one-species folded kernels stage KEXP W1): z1' = KEXP z1, so 2^{z'} = e^{-z}
// enters the sigmoid with no multiply, and s' = z' sigma(z) = KEXP silu(z)
// carries the same factor into the next layer (z2' = s1' W2 = KEXP z2) and on
// into T.  The derivative sigma + (s' / KEXP)(1 - sigma) = silu'(z) is
// unscaled.  Two vector instructions fewer per unit with its derivative, one
// without.
constexpr float KEXP = -1.44269504088896341f;
constexpr float KEXP_INV2 = 0.480453013918201424667f;  // 1 / KEXP^2 = (ln 2)^2
__device__ __forceinline__ float sigmoid_kexp(float zs) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(zs));
}

__device__ __forceinline__ void silu_and_deriv_kexp(const f32x16 z[2], f32x16 s[2], f32x16 d[2]) {
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float zz = z[m][r], sg = sigmoid_kexp(zz), ss = zz * sg;
      s[m][r] = ss;
      float dd = fmaf(fmaf(-sg, ss, ss), 1.f / KEXP, sg);
      asm volatile("" : "+v"(dd));
      d[m][r] = dd;
    }
}

__device__ __forceinline__ void silu_tiles_kexp(const f32x16 z[2], f32x16 s[2]) {
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[m][r] = z[m][r] * sigmoid_kexp(z[m][r]);
}

template <bool K>
__device__ __forceinline__ void silu_and_deriv_t(const f32x16 z[2], f32x16 s[2], f32x16 d[2]) {
  if (K) silu_and_deriv_kexp(z, s, d); else silu_and_deriv(z, s, d);
}
template <bool K>
__device__ __forceinline__ void silu_tiles_t(const f32x16 z[2], f32x16 s[2]) {
  if (K) silu_tiles_kexp(z, s); else silu_tiles(z, s);
}

// Geometry of the edge a lane works on (binary64, as the neighbour list).
struct Geo {
  double r;
  float ux, uy, uz, inv_r;
  int i, j;
};

// Edge e whose receiver the caller already knows (the unit's own atom).
__device__ __forceinline__ Geo edge_geo_at(const EdgeIn& in, int64_t e, int i) {
  Geo g;
  int j = in.col[e];
  i = min(max(i, 0), in.n_atoms - 1);
  j = min(max(j, 0), in.n_atoms - 1);
  double d[3];
  edge_vector(in.pos, i, j, in.shift + 3 * e, in.Lx, in.Ly, in.Lz, d);
  const double r2 = norm2_nofma(d);
  const double r = sqrt(r2);
  const double ir = 1.0 / r;
  g.r = r;
  g.inv_r = (float)ir;
  g.ux = (float)(d[0] * ir);
  g.uy = (float)(d[1] * ir);
  g.uz = (float)(d[2] * ir);
  g.i = i;
  g.j = j;
  return g;
}

__device__ __forceinline__ Geo edge_geo(const EdgeIn& in, int64_t e) { return edge_geo_at(in, e, in.recv[e]); }

// The global loads behind an edge's geometry (sender position and image shift).
struct EdgeRaw {
  double xj, yj, zj;
  int sx, sy, sz;
};

__device__ __forceinline__ EdgeRaw edge_raw(const EdgeIn& in, int64_t e) {
  EdgeRaw w;
  const int j = min(max(in.col[e], 0), in.n_atoms - 1);
  w.xj = in.pos[3 * j + 0];
  w.yj = in.pos[3 * j + 1];
  w.zj = in.pos[3 * j + 2];
  const int8_t* sh = in.shift + 3 * e;
  w.sx = sh[0];
  w.sy = sh[1];
  w.sz = sh[2];
  return w;
}

// edge_geo_at from prefetched loads and the receiver's position xi: the same
// binary64 operations in the same order as edge_vector.
__device__ __forceinline__ Geo geo_from_raw(const EdgeIn& in, const EdgeRaw& w, const double xi[3]) {
#pragma clang fp contract(off)
  double d[3];
  d[0] = (w.xj - xi[0]) + (double)w.sx * in.Lx;
  d[1] = (w.yj - xi[1]) + (double)w.sy * in.Ly;
  d[2] = (w.zj - xi[2]) + (double)w.sz * in.Lz;
  const double r2 = norm2_nofma(d);
  const double r = sqrt(r2);
  const double ir = 1.0 / r;
  Geo g;
  g.r = r;
  g.inv_r = (float)ir;
  g.ux = (float)(d[0] * ir);
  g.uy = (float)(d[1] * ir);
  g.uz = (float)(d[2] * ir);
  g.i = -1;
  g.j = -1;
  return g;
}


// Work units of the receiver-aligned kernels: (ordered species pair p, receiver i).
struct Units {
  const int32_t* row_ptr;
  const int32_t* species;
  const int32_t* perm;   // pair-grouped order -> CSR edge (S > 1); NULL when S == 1
  const int32_t* seg;    // [S][N][2] position range of unit (i, s) in that order (S > 1)
  int32_t n_atoms;
  int S;
};

// W1 and W2 only (the reassociated kernels read the last layer from global
// memory), by a workgroup of NT threads with every load issued first.
constexpr int W12_FLOATS = NB * LDH + HID * LDH;
template <int NT>
__device__ __forceinline__ void stage_w12(float* lds, const float* __restrict__ W1,
                                          const float* __restrict__ W2, int p, float w1_scale = 1.f) {
  stage_rows_all<NB, HID, NT>(lds, LDH, W1 + (size_t)p * NB * HID, w1_scale);
  stage_rows_all<HID, HID, NT>(lds + NB * LDH, LDH, W2 + (size_t)p * HID * HID);
}

// Position range [qa, qb) of unit (p, i) in the pair-grouped order; false when
// receiver i belongs to another pair's group.
__device__ __forceinline__ bool unit_range(const Units& un, int p, int i, int& qa, int& qb) {
  const int S = un.S;
  if (S == 1) {
    qa = un.row_ptr[i];
    qb = un.row_ptr[i + 1];
    return true;
  }
  if (min(max(un.species[i], 0), S - 1) != p / S) return false;
  const int zs = p % S;
  qa = un.seg[2 * ((size_t)zs * un.n_atoms + i)];
  qb = un.seg[2 * ((size_t)zs * un.n_atoms + i) + 1];
  return true;
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace chain
}  // namespace eec

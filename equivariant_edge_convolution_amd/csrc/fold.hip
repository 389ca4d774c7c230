// The energy/force call with the linear last radial layer moved past the
// edge sum (exact algebra, the fold of "deepmd-kit PR #6108", What: a frozen
// linear map applied after a linear reduction may be applied once, after it).
//
// Forward, per (pair p = (Z_i, s), receiver i) unit:
//   T_{k,lm} = sum_{e in row i, Z_j = s} s2_{e,k} Y_{e,lm}          (matrix cores, K = edges)
//   A^{(s)}_{i,lm,c} = h_{s,c} sum_k T_{k,lm} W3_p[k, l(lm) C + c]   (per receiver)
// instead of R_e = s2_e W3 for every edge: 45,056 -> 12,288 + 2,048 flop per
// edge plus 131,072 flop per unit.
// Backward, per unit, with Abar = dE/dA:
//   M_{lm,k} = sum_c Abar_{i,lm,c} h_{s,c} W3_p[k, l(lm) C + c]      (per receiver)
//   Ybar_{e,lm} = sum_k s2_{e,k} M_{lm,k},   s2bar_{e,k} = sum_lm M_{lm,k} Y_{e,lm}
// which replace recomputing R (32,768 flop/edge) and s2bar = Rbar W3^T
// (32,768 flop/edge) by 4,096 flop/edge.  The rest of the backward (SiLU
// derivatives, W2^T, W1^T, the radial and angular chain rule) is the direct
// path's.
#include "chain.hpp"

namespace eec {
namespace {
using namespace chain;

// ------------------------------------------------------------------ per-wave LDS
// Every unit belongs to one wave; its LDS region holds, in turn,
//   forward:  ysm [32][17] harmonics of the tile's edges (zero rows for padding),
//             tsm [64][16] T of the unit, staged for the last layer;
//   backward: ahsm [C][AHS] dE/dA_{lm,c} h_c by channel row (several species),
//             then (written once every ahsm or tsm row has been read) msm
//             [16][65] M of the unit, and ybsm [32][17] dE/dY of the tile's edges.
constexpr int AHS = NLM + 4;  // row stride of the staged dE/dA h rows (16-byte aligned)
template <int C>
struct FoldLds {
  static constexpr int YSM = 0, TSM = 32 * (NLM + 1), FWD = TSM + HID * NLM;
  static constexpr int AHSM = 0, MSM = 0, YBSM = NLM * (HID + 1), BWD_M = YBSM + 32 * (NLM + 1);
  static constexpr int BWD = C * AHS > BWD_M ? C * AHS : BWD_M;
  static constexpr int FWD_ONLY = FWD, BWD_ONLY = BWD, FUSED = FWD > BWD_M ? FWD : BWD_M;
};

template <int C>
struct WaveLds {
  float (*ysm)[NLM + 1];
  float (*tsm)[NLM];
  float (*ahsm)[AHS];
  float (*msm)[HID + 1];
  float (*ybsm)[NLM + 1];
  __device__ explicit WaveLds(float* base) {
    ysm = reinterpret_cast<float (*)[NLM + 1]>(base + FoldLds<C>::YSM);
    tsm = reinterpret_cast<float (*)[NLM]>(base + FoldLds<C>::TSM);
    ahsm = reinterpret_cast<float (*)[AHS]>(base + FoldLds<C>::AHSM);
    msm = reinterpret_cast<float (*)[HID + 1]>(base + FoldLds<C>::MSM);
    ybsm = reinterpret_cast<float (*)[NLM + 1]>(base + FoldLds<C>::YBSM);
  }
};

// ------------------------------------------------------------------ stash
// One-species fused kernel: what the backward tiles of a unit need from its
// forward tiles, kept in a per-wave scratch region instead of recomputing the
// radial basis and the first two layers.  Row of an edge (ZROW floats):
//   [0, 64)    silu'(z1) by hidden index
//   [64, 128)  z2 by hidden index
//   [128, 136) u_x, u_y, u_z, 1/r, and the basis seed: x = r / rc as a float32
//              head and tail, sin pi x, cos pi x
// A unit's first STASH_TILES tiles are kept; further tiles (rows denser than
// STASH_TILES * 32 edges) recompute.  The live rows of all waves (about 176
// MB for a 4096-atom diamond: 2,048 waves, 158 edges each, 544 bytes an edge)
// are read back mostly from the caches between the forward and the backward
// of a unit (marking those reads non-temporal made the kernel 13 % slower),
// which is cheaper than recomputing the basis and the two layers.
constexpr int ZROW = 2 * HID + 8;
constexpr int STASH_TILES = 6;

// ------------------------------------------------------------------ tiles
// Edge of lane slot s in the tile starting at position q0 of a unit whose edges
// sit at positions [qa, qb) of the work order (`perm` maps positions to CSR
// edges; NULL = identity).  Padding slots repeat the unit's first edge.
__device__ __forceinline__ int64_t tile_edge(const int32_t* perm, int q0, int qa, int qb, int s) {
  const int q = q0 + s;
  const int qq = q < qb ? q : qa;
  return perm ? (int64_t)perm[qq] : (int64_t)qq;
}

// Receiver position of unit atom i.
struct Recv {
  double x[3];
};
__device__ __forceinline__ Recv recv_pos(const EdgeIn& in, int i) {
  i = min(max(i, 0), in.n_atoms - 1);
  return Recv{{in.pos[3 * i], in.pos[3 * i + 1], in.pos[3 * i + 2]}};
}

// Stash rows of the tile at position q0 of a unit starting at qa, in the
// region `zw` of the wave; NULL when the tile is past the kept ones.
__device__ __forceinline__ float* stash_tile(float* zw, int q0, int qa) {
  const int t = (q0 - qa) >> 5;
  return zw != nullptr && t < STASH_TILES ? zw + (size_t)t * 32 * ZROW : nullptr;
}

// ------------------------------------------------------------------ forward
// One 32-edge tile [q0, q0 + 32) of a unit: T += s2^T Y over the tile.  With a
// stash tile zs, also its rows (edge slot k at zs + k ZROW).
template <bool K = false, bool PAD = true>
__device__ __forceinline__ void fwd_tile(const EdgeIn& in, const int32_t* perm, const Recv& xi,
                                         const float* w1s, const float* w2s, float (*ysm)[NLM + 1],
                                         int q0, int qa, int qb, int s, int h, f32x4 T[4], float* zs) {
  const bool valid = q0 + s < qb;
  const Geo g = geo_from_raw(in, edge_raw(in, tile_edge(perm, q0, qa, qb, s)), xi.x);
  const BasisSeed sd = basis_seed(g.r, in.inv_rc, g.inv_r, h);
  // With PAD, stash rows are written for all 32 slots, padding slots too
  // (they hold the padding edge; the tile's 32 rows exist and slots past the
  // unit's end are never read back), so no lane-dependent branch splits the
  // stores: cheaper where tiles are full (one species).  Without PAD only the
  // unit's own rows are written: less traffic where units are short and
  // tiles half empty (several species).
  if (zs != nullptr && h == 0 && (PAD || valid)) {
    float* row = zs + s * ZROW + 2 * HID;
    *reinterpret_cast<float4*>(row) = make_float4(g.ux, g.uy, g.uz, g.inv_r);
    *reinterpret_cast<float4*>(row + 4) = make_float4(sd.x, sd.xl, sd.s1, sd.c1);
  }
  f32x16 z[2], a[2];
  {
    float bas[16];
    basis16f<false>(sd, in.inv_rc_f, h, bas, nullptr);
    layer1(w1s, bas, s, h, z);
  }
  if (zs != nullptr) {
    f32x16 d[2];
    silu_and_deriv_t<K>(z, a, d);  // s1 and silu'(z1), edges on N: hidden hid_k0(ks) + 4h
    if (PAD || valid) {
      float* row = zs + s * ZROW + 4 * h;
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<float4*>(row + 32 * m + 8 * j) =
              make_float4(d[m][4 * j], d[m][4 * j + 1], d[m][4 * j + 2], d[m][4 * j + 3]);
    }
  } else {
    silu_tiles_t<K>(z, a);  // s1, edges on N
  }
  // z2 with edges on M: register r of tile m = edge fperm(r) + 4h, hidden 32 m + s
  {
    const float* w = w2s + 4 * h * LDH + s;  // W2[hid_k0(ks) + 4 h][32 m + s]
    z[0] = zero16();
    z[1] = zero16();
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) {
      const float av = a[ks >> 4][ks & 15];
#pragma unroll
      for (int m = 0; m < 2; ++m) z[m] = mfma32(av, w[hid_k0(ks) * LDH + 32 * m], z[m]);
    }
    pipeline_lds_mfma<64, 2, 6>();
  }
  if (zs != nullptr) {
    // z2 rows: register r of tile m is edge slot fperm(r) + 4h, hidden 32 m + s
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int k = fperm(r) + 4 * h;
      if (PAD || q0 + k < qb) {
        float* row = zs + k * ZROW + HID + s;
        row[0] = z[0][r];
        row[32] = z[1][r];
      }
    }
  }
  silu_tiles_t<K>(z, a);  // s2, edges on M
  {
    float Y[16];
    sph16(g.ux, g.uy, g.uz, Y);
#pragma unroll
    for (int k = 0; k < 8; ++k) ysm[s][8 * h + k] = valid ? (h ? Y[8 + k] : Y[k]) : 0.f;  // static indices
  }
  wave_sync_lds();
  // T[hidden][lm] += sum over this tile's edges on 16x16x4 tiles (N = the 16
  // harmonics exactly).  Swapping rows of registers r and r + 4 of tile m
  // leaves, in lane j + 16 q, hidden 32 m + j (register r) and 32 m + 16 + j
  // (register r + 4) of edge fperm(r) + off(q), off = 0, 8, 4, 12: the A
  // operands of hidden blocks 2m and 2m + 1 for K = those four edges.
  {
    const int j = s & 15, qk = (s >> 4) + 2 * h;
    const float* yrow = &ysm[8 * (qk & 1) + 4 * (qk >> 1)][j];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int rr = 0; rr < 12; rr = (rr == 3 ? 8 : rr + 1)) {
        float lo = a[m][rr], hi = a[m][rr + 4];
        swap_rows16(lo, hi);
        const float yv = yrow[fperm(rr) * (NLM + 1)];
        T[2 * m] = mfma16(lo, yv, T[2 * m]);
        T[2 * m + 1] = mfma16(hi, yv, T[2 * m + 1]);
      }
    pipeline_lds_mfma<32, 2, 6>();
  }
  wave_sync_lds();
}

// The multi-species kernel's LDS copy of W3 (C = 64): W3I[k][c][l] = W3[k][l C + c],
// the four degrees of a channel in one 16-byte word, rows of W3I_LD floats
// (a multiple of 4; 260 mod 64 = 4, so a wave reading one word per row or one
// per channel touches every bank once per 16 lanes).
constexpr int W3I_LD = 4 * 64 + 4;
constexpr int W3I_FLOATS = HID * W3I_LD;

// Stages W3[p] into the interleaved layout, by a workgroup of NT threads, in
// rounds of STAGE_WORDS 16-byte words W3[k][l C + 4 q .. 4 q + 3] per thread
// (all of a round's loads before its stores: one memory latency per round),
// each spread over the four channels' words (degree l in slot l).
template <int NT>
__device__ __forceinline__ void stage_w3i(float* lds, const float* __restrict__ W3p) {
  constexpr int C = 64, N4 = HID * 4 * C / 4, PER = N4 / NT;
  static_assert(N4 % NT == 0, "whole words per thread");
  if ((reinterpret_cast<uintptr_t>(W3p) & 15) != 0) {
    for (int t = threadIdx.x; t < HID * C; t += blockDim.x) {
      const int k = t / C, c = t % C;
      const float* src = W3p + (size_t)k * 4 * C + c;
      *reinterpret_cast<float4*>(lds + k * W3I_LD + 4 * c) = make_float4(src[0], src[C], src[2 * C], src[3 * C]);
    }
    return;
  }
  const float4* g4 = reinterpret_cast<const float4*>(W3p);
  static_assert(PER % STAGE_WORDS == 0, "whole rounds");
#pragma unroll
  for (int u0 = 0; u0 < PER; u0 += STAGE_WORDS) {
    float4 v[STAGE_WORDS];
#pragma unroll
    for (int u = 0; u < STAGE_WORDS; ++u) v[u] = g4[threadIdx.x + (u0 + u) * NT];
#pragma unroll
    for (int u = 0; u < STAGE_WORDS; ++u) {
      const int w = threadIdx.x + (u0 + u) * NT;  // word w: row k = w / 64, degree l = (w / 16) % 4, channels 4 (w % 16) ..
      const int k = w >> 6, l = (w >> 4) & 3, c = 4 * (w & 15);
      float* d = lds + k * W3I_LD + 4 * c + l;
      d[0] = v[u].x;
      d[4] = v[u].y;
      d[8] = v[u].z;
      d[12] = v[u].w;
    }
  }
}

// T of the unit to LDS, then acc[q][lm] = sum_k T[k][lm] W3[k][l(lm) C + c]
// for channel c = lane + 64 q (the h_c factor is the caller's).  W3[k][j] is
// w3[k * SK + j] (global memory: SK = 4 C), or SK = 0: the interleaved LDS
// copy W3I (C = 64).
template <int C, int SK>
__device__ __forceinline__ void unit_last_layer(const f32x4 T[4], float (*tsm)[NLM], const float* w3,
                                                int lane, float acc[C / 64][NLM]) {
  constexpr int CPL = C / 64;
  // T block b register i, lane l: hidden 16 b + 4 (l / 16) + i, harmonic l % 16
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) tsm[16 * b + 4 * (lane >> 4) + i][lane & 15] = T[b][i];
  wave_sync_lds();
#pragma unroll
  for (int q = 0; q < CPL; ++q)
#pragma unroll
    for (int k = 0; k < NLM; ++k) acc[q][k] = 0.f;
#pragma unroll 4
  for (int k = 0; k < HID; ++k) {
    float t[NLM];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float4 x = *reinterpret_cast<const float4*>(&tsm[k][4 * v]);
      t[4 * v] = x.x; t[4 * v + 1] = x.y; t[4 * v + 2] = x.z; t[4 * v + 3] = x.w;
    }
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      float w0, wl1, wl2, wl3;
      if (SK == 0) {  // the interleaved LDS copy: W3I[k][c][l], rows of W3I_LD floats
        const float4 w = *reinterpret_cast<const float4*>(w3 + (size_t)k * W3I_LD + 4 * (lane + 64 * q));
        w0 = w.x; wl1 = w.y; wl2 = w.z; wl3 = w.w;
      } else {
        const float* wr = w3 + (size_t)k * SK + lane + 64 * q;
        w0 = wr[0]; wl1 = wr[C]; wl2 = wr[2 * C]; wl3 = wr[3 * C];
      }
      acc[q][0] += t[0] * w0;
#pragma unroll
      for (int lm = 1; lm < 4; ++lm) acc[q][lm] += t[lm] * wl1;
#pragma unroll
      for (int lm = 4; lm < 9; ++lm) acc[q][lm] += t[lm] * wl2;
#pragma unroll
      for (int lm = 9; lm < 16; ++lm) acc[q][lm] += t[lm] * wl3;
    }
  }
  wave_sync_lds();  // every tsm read done before the region is reused
}

template <int C, int W>
__global__ void __launch_bounds__(64 * W)
k_fold_forward(EdgeIn in, Units un, const float* __restrict__ W1, const float* __restrict__ W2,
               const float* __restrict__ W3, const float* __restrict__ emb, float* __restrict__ A_out) {
  constexpr int CPL = C / 64;
  __shared__ float w12[W12_FLOATS];
  __shared__ __align__(16) float wbuf[W][FoldLds<C>::FWD_ONLY];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const WaveLds<C> L(wbuf[wave]);
  const float* w1s = w12;
  const float* w2s = w12 + NB * LDH;
  const int N = un.n_atoms, S = un.S, P = S * S;
  const int nbp = (N + W - 1) / W;
  int loaded = -1;
  for (int b = blockIdx.x; b < P * nbp; b += gridDim.x) {
    const int p = b / nbp;
    if (p != loaded) {
      __syncthreads();
      stage_w12<64 * W>(w12, W1, W2, p);
      __syncthreads();
      loaded = p;
    }
    const int i = (b - p * nbp) * W + wave;
    int qa, qb;
    if (i >= N || !unit_range(un, p, i, qa, qb)) continue;
    int s = lane & 31, h = lane >> 5;
    asm volatile("" : "+v"(s), "+v"(h));
    const int zs = p % S;
    f32x4 T[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) T[b] = zero4();
    const Recv xi = recv_pos(in, i);
    for (int q0 = qa; q0 < qb; q0 += 32)
      fwd_tile(in, un.perm, xi, w1s, w2s, L.ysm, q0, qa, qb, s, h, T, nullptr);
    float acc[CPL][NLM];
    unit_last_layer<C, 4 * C>(T, L.tsm, W3 + (size_t)p * HID * 4 * C, lane, acc);
    float* ao = A_out + ((size_t)zs * N + i) * NLM * C;
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      const int c = lane + 64 * q;
      const float hc = emb[(size_t)zs * C + c];
#pragma unroll
      for (int k = 0; k < NLM; ++k) ao[k * C + c] = hc * acc[q][k];
    }
  }
}

// ------------------------------------------------------------------ backward
// M[lm][k] = sum_c (dE/dA h)[lm][c] W3[k][l(lm) C + c] from the staged ahsm rows
// (lane = hidden k), into msm over the ahsm region.  W3[k][j] of this lane's k
// is wt[j * SJ] (the transposed copy in global memory: SJ = 64), or SJ = 0:
// wt = row k of the interleaved LDS copy W3I (C = 64).
template <int C, int SJ>
__device__ __forceinline__ void unit_M(float (*ahsm)[AHS], const float* wt, int lane, float (*msm)[HID + 1]) {
  float macc[NLM];
#pragma unroll
  for (int lm = 0; lm < NLM; ++lm) macc[lm] = 0.f;
#pragma unroll 4
  for (int c = 0; c < C; ++c) {
    float av[NLM];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float4 x = *reinterpret_cast<const float4*>(&ahsm[c][4 * v]);
      av[4 * v] = x.x; av[4 * v + 1] = x.y; av[4 * v + 2] = x.z; av[4 * v + 3] = x.w;
    }
    float w0, wl1, wl2, wl3;
    if (SJ == 0) {  // the interleaved LDS copy, wt = row k of W3I
      const float4 w = *reinterpret_cast<const float4*>(wt + 4 * c);
      w0 = w.x; wl1 = w.y; wl2 = w.z; wl3 = w.w;
    } else {
      w0 = wt[(size_t)c * SJ]; wl1 = wt[(size_t)(C + c) * SJ];
      wl2 = wt[(size_t)(2 * C + c) * SJ]; wl3 = wt[(size_t)(3 * C + c) * SJ];
    }
    macc[0] += av[0] * w0;
#pragma unroll
    for (int lm = 1; lm < 4; ++lm) macc[lm] += av[lm] * wl1;
#pragma unroll
    for (int lm = 4; lm < 9; ++lm) macc[lm] += av[lm] * wl2;
#pragma unroll
    for (int lm = 9; lm < 16; ++lm) macc[lm] += av[lm] * wl3;
  }
  wave_sync_lds();  // msm overlays ahsm
#pragma unroll
  for (int lm = 0; lm < NLM; ++lm) msm[lm][lane] = macc[lm];
  wave_sync_lds();
}

// One 32-edge tile of the backward of a unit: g = dE/dd of its edges.  The
// geometry, silu'(z1) and z2 come from the stash tile zs when given, else are
// recomputed.
template <bool K = false>
__device__ __forceinline__ void bwd_tile(const EdgeIn& in, const Recv& xi, const int32_t* perm,
                                         const float* w1s, const float* w2s, float (*msm)[HID + 1],
                                         float (*ybsm)[NLM + 1], int q0, int qa, int qb, int s, int h,
                                         float* __restrict__ gout, const float* zs) {
  const bool valid = q0 + s < qb;
  const int64_t e = tile_edge(perm, q0, qa, qb, s);
  Geo g;
  BasisSeed sd;
  f32x16 d1[2], d2[2], s2[2];  // silu'(z1), silu'(z2), silu(z2); edges on N
  if (zs != nullptr) {
    const float* row = zs + (valid ? s : 0) * ZROW;
    const float4 u = *reinterpret_cast<const float4*>(row + 2 * HID);
    const float4 bs = *reinterpret_cast<const float4*>(row + 2 * HID + 4);
    g.ux = u.x;
    g.uy = u.y;
    g.uz = u.z;
    g.inv_r = u.w;
    sd = basis_seed_stored(bs.x, bs.y, bs.z, bs.w, u.w, h);
    f32x16 z[2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 v1 = *reinterpret_cast<const float4*>(row + 4 * h + 32 * m + 8 * j);
        const float4 v2 = *reinterpret_cast<const float4*>(row + HID + 4 * h + 32 * m + 8 * j);
        d1[m][4 * j] = v1.x; d1[m][4 * j + 1] = v1.y; d1[m][4 * j + 2] = v1.z; d1[m][4 * j + 3] = v1.w;
        z[m][4 * j] = v2.x; z[m][4 * j + 1] = v2.y; z[m][4 * j + 2] = v2.z; z[m][4 * j + 3] = v2.w;
      }
    silu_and_deriv_t<K>(z, s2, d2);
  } else {
    g = geo_from_raw(in, edge_raw(in, e), xi.x);
    sd = basis_seed(g.r, in.inv_rc, g.inv_r, h);
    f32x16 z[2], s1[2];
    {
      float bas[16];
      basis16f<false>(sd, in.inv_rc_f, h, bas, nullptr);
      layer1(w1s, bas, s, h, z);
    }
    silu_and_deriv_t<K>(z, s1, d1);
    layer2(w2s, s1, s, h, z);
    silu_and_deriv_t<K>(z, s2, d2);
  }
  __builtin_amdgcn_sched_barrier(0);
  // Ybar[edge][lm] = sum_k s2[edge][k] M[lm][k] on 16x16x4 tiles: swapping rows
  // of registers r and r + 4 of tile mm leaves, in lane j + 16 q, edge j
  // (register r) and edge 16 + j (register r + 4) at hidden 32 mm + fperm(r) +
  // off(q), off = 0, 8, 4, 12: the A operands of edge blocks 0 and 1.
  f32x4 yb[2];
  yb[0] = zero4();
  yb[1] = zero4();
  {
    const int j = s & 15, qk = (s >> 4) + 2 * h;
    const float* mrow = &msm[j][8 * (qk & 1) + 4 * (qk >> 1)];
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
#pragma unroll
      for (int rr = 0; rr < 12; rr = (rr == 3 ? 8 : rr + 1)) {
        float lo = s2[mm][rr], hi = s2[mm][rr + 4];
        swap_rows16(lo, hi);
        const float bv = mrow[32 * mm + fperm(rr)];
        yb[0] = mfma16(lo, bv, yb[0]);
        yb[1] = mfma16(hi, bv, yb[1]);
      }
    pipeline_lds_mfma<32, 2, 6>();
  }
  __builtin_amdgcn_sched_barrier(0);
  // s2bar[k][edge] = sum_lm M[lm][k] Y[edge][lm]  (edges on N; K pairs (2ks, 2ks + 1))
  f32x16 sb[2];
  sb[0] = zero16();
  sb[1] = zero16();
  {
    float Y[16];
    sph16(g.ux, g.uy, g.uz, Y);
    const float* mc = &msm[h][s];  // M[2 ks + h][32 m + s]
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const float bv = h ? Y[2 * ks + 1] : Y[2 * ks];
#pragma unroll
      for (int m = 0; m < 2; ++m) sb[m] = mfma32(mc[2 * ks * (HID + 1) + 32 * m], bv, sb[m]);
    }
    pipeline_lds_mfma<16, 2, 6>();
  }
  __builtin_amdgcn_sched_barrier(0);
  // Ybar to the lanes that own the edges (block b register i of lane l: edge
  // 16 b + 4 (l / 16) + i, harmonic l % 16), contracted with the harmonic gradients
  {
    const int l = s + 32 * h;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) ybsm[16 * b + 4 * (l >> 4) + i][l & 15] = yb[b][i];
  }
  wave_sync_lds();
  float G[3];
  {
    float ybe[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) ybe[k] = ybsm[s][k];
    sph16_grad_dot(g.ux, g.uy, g.uz, ybe, G);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) sb[m][r] *= d2[m][r];  // z2bar
  f32x16 s1b[2];
  s1b[0] = zero16();
  s1b[1] = zero16();
  const float* w2c = w2s + s * LDH + 4 * h;  // W2[32 m + s][hid_k0(ks) + 4 h]
#pragma unroll
  for (int ks = 0; ks < 32; ++ks) {
    const float bv = sb[ks >> 4][ks & 15];
#pragma unroll
    for (int m = 0; m < 2; ++m) s1b[m] = mfma32(w2c[32 * m * LDH + hid_k0(ks)], bv, s1b[m]);
  }
  pipeline_lds_mfma<64, 2, 6>();
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) s1b[m][r] *= d1[m][r];  // z1bar
  f32x16 bb = zero16();
  const float* w1c = w1s + basis_of_row(s) * LDH + 4 * h;
#pragma unroll
  for (int ks = 0; ks < 32; ++ks) bb = mfma32(w1c[hid_k0(ks)], s1b[ks >> 4][ks & 15], bb);
  pipeline_lds_mfma<32, 2, 6>();
  __builtin_amdgcn_sched_barrier(0);
  float rbar = 0.f;
  {
    float bas[16], dbas[16];
    basis16f<true>(sd, in.inv_rc_f, h, bas, dbas);  // cheaper to redo than to keep live
#pragma unroll
    for (int r = 0; r < 16; ++r) rbar += bb[r] * dbas[r];
  }
  rbar += __shfl_xor(rbar, 32);
  const float gu = G[0] * g.ux + G[1] * g.uy + G[2] * g.uz;
  if (valid && h == 0) {
    store_grad_row(gout, e, rbar * g.ux + (G[0] - gu * g.ux) * g.inv_r, rbar * g.uy + (G[1] - gu * g.uy) * g.inv_r,
                   rbar * g.uz + (G[2] - gu * g.uz) * g.inv_r);
  }
  wave_sync_lds();
}

template <int C, int W>
__global__ void __launch_bounds__(64 * W)
k_fold_backward(EdgeIn in, Units un, const float* __restrict__ W1, const float* __restrict__ W2,
                const float* __restrict__ W3T, const float* __restrict__ emb,
                const float* __restrict__ Abar, float* __restrict__ gout) {
  constexpr int NC = 4 * C, CPL = C / 64;
  __shared__ float w12[W12_FLOATS];
  __shared__ __align__(16) float wbuf[W][FoldLds<C>::BWD_ONLY];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const WaveLds<C> L(wbuf[wave]);
  const float* w1s = w12;
  const float* w2s = w12 + NB * LDH;
  const int N = un.n_atoms, S = un.S, P = S * S;
  const int nbp = (N + W - 1) / W;
  int loaded = -1;
  for (int b = blockIdx.x; b < P * nbp; b += gridDim.x) {
    const int p = b / nbp;
    if (p != loaded) {
      __syncthreads();
      stage_w12<64 * W>(w12, W1, W2, p);
      __syncthreads();
      loaded = p;
    }
    const int i = (b - p * nbp) * W + wave;
    int qa, qb;
    if (i >= N || !unit_range(un, p, i, qa, qb) || qb <= qa) continue;
    int s = lane & 31, h = lane >> 5;
    asm volatile("" : "+v"(s), "+v"(h));
    const int zs = p % S;
    // stage Abar_i h_s (lane = channel)
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      const int c = lane + 64 * q;
      const float hc = emb[(size_t)zs * C + c];
      const float* ar = Abar + (size_t)i * NLM * C + c;
#pragma unroll
      for (int lm = 0; lm < NLM; ++lm) L.ahsm[c][lm] = ar[lm * C] * hc;
    }
    wave_sync_lds();
    unit_M<C, HID>(L.ahsm, W3T + (size_t)p * NC * HID + lane, lane, L.msm);
    const Recv xi = recv_pos(in, i);
    for (int q0 = qa; q0 < qb; q0 += 32)
      bwd_tile(in, xi, un.perm, w1s, w2s, L.msm, L.ybsm, q0, qa, qb, s, h, gout, nullptr);
  }
}

// M_i and E_i from the staged T of the unit through the Gram matrices (lane =
// hidden k).  g(k') returns G_0..G_3[k][k'] for this lane's k.
template <typename GF>
__device__ __forceinline__ float gram_epilogue(const float (*tsm)[NLM], int lane, GF&& g, float macc[NLM]) {
#pragma unroll
  for (int lm = 0; lm < NLM; ++lm) macc[lm] = 0.f;
#pragma unroll 4
  for (int kk = 0; kk < HID; ++kk) {
    float t[NLM];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float4 x = *reinterpret_cast<const float4*>(&tsm[kk][4 * v]);
      t[4 * v] = x.x; t[4 * v + 1] = x.y; t[4 * v + 2] = x.z; t[4 * v + 3] = x.w;
    }
    const float4 gv = g(kk);
    const float g0 = gv.x, g1 = gv.y, g2 = gv.z, g3 = gv.w;
    macc[0] += g0 * t[0];
#pragma unroll
    for (int lm = 1; lm < 4; ++lm) macc[lm] += g1 * t[lm];
#pragma unroll
    for (int lm = 4; lm < 9; ++lm) macc[lm] += g2 * t[lm];
#pragma unroll
    for (int lm = 9; lm < 16; ++lm) macc[lm] += g3 * t[lm];
  }
  float esum = 0.f;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float4 x = *reinterpret_cast<const float4*>(&tsm[lane][4 * v]);
    esum += x.x * macc[4 * v] + x.y * macc[4 * v + 1] + x.z * macc[4 * v + 2] + x.w * macc[4 * v + 3];
  }
  for (int off = 32; off > 0; off >>= 1) esum += __shfl_xor(esum, off);
  return 0.5f * esum;
}

// The readout of one receiver by the W = 8 waves of a workgroup: T (the sum of
// the waves' partials, in wave order) into tw, then wave w forms M for
// harmonics 2w and 2w + 1 (lane = hidden unit k, G_l read from global memory
// along rows: G is symmetric) into msh, and its share of E_i = 1/2 sum T.M
// into esh[w].  Returns E_i (the shares in wave order) to every thread.  M and
// E_i are multiplied by `scale` (1 / KEXP^2 when T carries the factor KEXP of
// the scaled chain: M then carries 1 / KEXP, which the backward's scaled s2
// cancels).
template <int W, int TSM_OFF, int STRIDE>
__device__ __forceinline__ float gram_epilogue_split(float* tw, const float* wbase, const float* __restrict__ G,
                                                     int lane, int wave, float (*msh)[HID + 1], float* esh,
                                                     float scale = 1.f) {
  static_assert(W == 8, "two harmonics per wave");
  for (int e = threadIdx.x; e < HID * NLM; e += 64 * W) {
    float v = tw[e];
#pragma unroll
    for (int w = 1; w < W; ++w) v += wbase[w * STRIDE + TSM_OFF + e];
    tw[e] = v;
  }
  __syncthreads();
  const float(*tsm)[NLM] = reinterpret_cast<const float(*)[NLM]>(tw);
  const int lm0 = 2 * wave, lm1 = lm0 + 1;
  const int l0 = lm0 == 0 ? 0 : (lm0 < 4 ? 1 : (lm0 < 9 ? 2 : 3));
  const int l1 = lm1 < 4 ? 1 : (lm1 < 9 ? 2 : 3);
  const float* g0 = G + (size_t)l0 * HID * HID + lane;
  const float* g1 = G + (size_t)l1 * HID * HID + lane;
  float m0 = 0.f, m1 = 0.f;
#pragma unroll 16
  for (int kk = 0; kk < HID; ++kk) {
    m0 += g0[kk * HID] * tsm[kk][lm0];
    m1 += g1[kk * HID] * tsm[kk][lm1];
  }
  msh[lm0][lane] = m0 * scale;
  msh[lm1][lane] = m1 * scale;
  float es = tsm[lane][lm0] * m0 + tsm[lane][lm1] * m1;
  for (int off = 32; off > 0; off >>= 1) es += __shfl_xor(es, off);
  if (lane == 0) esh[wave] = es;
  __syncthreads();
  float e = 0.f;
#pragma unroll
  for (int w = 0; w < W; ++w) e += esh[w];
  return 0.5f * e * scale;
}

// The same for the two receivers of a pair at once (the second only when
// `two`): the partial T of receiver r summed into tw[r], then each wave's two
// harmonics of both receivers from one pass over its rows of G (both
// receivers share them), so the L2 latency of those loads is paid once per
// pair.  Each receiver's sums run in the same order as above.  E_i of the
// receivers into e[0], e[1].
template <int W, int TSM_OFF, int STRIDE>
__device__ __forceinline__ void gram_epilogue_pair(float* tw0, const float* wbase, float* tw1, bool two,
                                                   const float* __restrict__ G, int lane, int wave,
                                                   float (*msh0)[HID + 1], float (*msh1)[HID + 1],
                                                   float (*esh)[W], float scale, float e[2]) {
  static_assert(W == 8, "two harmonics per wave");
  for (int x = threadIdx.x; x < HID * NLM; x += 64 * W) {
    float v = tw0[x];
#pragma unroll
    for (int w = 1; w < W; ++w) v += wbase[w * STRIDE + TSM_OFF + x];
    tw0[x] = v;
    if (two) {
      float u = tw1[x];
#pragma unroll
      for (int w = 1; w < W; ++w) u += tw1[w * HID * NLM + x];
      tw1[x] = u;
    }
  }
  __syncthreads();
  const float(*t0)[NLM] = reinterpret_cast<const float(*)[NLM]>(tw0);
  const float(*t1)[NLM] = reinterpret_cast<const float(*)[NLM]>(tw1);
  const int lm0 = 2 * wave, lm1 = lm0 + 1;
  const int l0 = lm0 == 0 ? 0 : (lm0 < 4 ? 1 : (lm0 < 9 ? 2 : 3));
  const int l1 = lm1 < 4 ? 1 : (lm1 < 9 ? 2 : 3);
  const float* g0 = G + (size_t)l0 * HID * HID + lane;
  const float* g1 = G + (size_t)l1 * HID * HID + lane;
  float m00 = 0.f, m01 = 0.f, m10 = 0.f, m11 = 0.f;
  if (two) {
#pragma unroll 16
    for (int kk = 0; kk < HID; ++kk) {
      const float a = g0[kk * HID], b = g1[kk * HID];
      m00 += a * t0[kk][lm0];
      m01 += b * t0[kk][lm1];
      m10 += a * t1[kk][lm0];
      m11 += b * t1[kk][lm1];
    }
  } else {
#pragma unroll 16
    for (int kk = 0; kk < HID; ++kk) {
      m00 += g0[kk * HID] * t0[kk][lm0];
      m01 += g1[kk * HID] * t0[kk][lm1];
    }
  }
  msh0[lm0][lane] = m00 * scale;
  msh0[lm1][lane] = m01 * scale;
  float es0 = t0[lane][lm0] * m00 + t0[lane][lm1] * m01;
  for (int off = 32; off > 0; off >>= 1) es0 += __shfl_xor(es0, off);
  if (lane == 0) esh[0][wave] = es0;
  if (two) {
    msh1[lm0][lane] = m10 * scale;
    msh1[lm1][lane] = m11 * scale;
    float es1 = t1[lane][lm0] * m10 + t1[lane][lm1] * m11;
    for (int off = 32; off > 0; off >>= 1) es1 += __shfl_xor(es1, off);
    if (lane == 0) esh[1][wave] = es1;
  }
  __syncthreads();
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    s0 += esh[0][w];
    s1 += two ? esh[1][w] : 0.f;
  }
  e[0] = 0.5f * s0 * scale;
  e[1] = 0.5f * s1 * scale;
}

// ------------------------------------------------------------------ fused (one species)
// With one species, receiver i's unit holds its whole row, and the backward of
// the unit needs only M_i, which depends on nothing but the unit's own forward:
// one wave runs forward tiles -> T_i -> E_i and M_i -> backward tiles.  The
// quadratic readout needs no A at all: with A_{lm,c} = h_c sum_k W3[k, lC+c]
// T_{lm,k} and E_i = sum_c w_c sum_lm A^2, the per-degree Gram matrices
//   G_l[k][k'] = sum_c 2 w_c h_c^2 W3[k][lC+c] W3[k'][lC+c]     (k_gram, per call)
// give M_{lm} = G_{l(lm)} T_{lm} and E_i = 1/2 sum_lm T_{lm} . M_{lm}: one
// 64 x 64 contraction per harmonic per receiver, whatever C is, instead of A
// (16 x 64 x C) and M (16 x C x 64).  G (64 KB) sits in LDS beside W1 and W2,
// interleaved by degree: GI[k][k'][l] = G_l[k][k'], the four degrees of an
// entry in one 16-byte word, rows of GI_LD floats (a multiple of 4; 260 mod
// 64 = 4, so 16 lanes reading one word each from rows k touch every bank once).
constexpr int GI_LD = 4 * HID + 4;
constexpr int GRAM_FLOATS = HID * GI_LD;

// G in global memory ([l][k][k']) into the interleaved LDS layout, by a
// workgroup of NT threads.  Thread t takes LDS entries t, t + NT, ... in LDS
// order (row k, then 4 k' + l), so a wave's stores are consecutive words
// (no bank conflicts), and issues all its loads before the first store (one
// memory latency instead of one per entry; the loads of one instruction fall
// in four 64-byte runs of G, one per degree).
template <int NT>
__device__ __forceinline__ void stage_gram(float* gs, const float* __restrict__ G) {
  constexpr int NE = 4 * HID * HID, PER = NE / NT;
  static_assert(NE % NT == 0, "whole entries per thread");
  float v[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int t = threadIdx.x + u * NT;
    const int k = t >> 8, j = t & 255;  // j = 4 k' + l
    v[u] = G[((j & 3) << 12) + (k << 6) + (j >> 2)];
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int t = threadIdx.x + u * NT;
    gs[(t >> 8) * GI_LD + (t & 255)] = v[u];
  }
}

// G_l[k][k'] for one species pair.  Block (l, four rows k): the degree-l
// columns of W3 (64 x C) in LDS (16-byte loads where W3 allows, all issued
// before the first store), one entry per thread, binary64 sums over c.
constexpr int GRAM_T = 256;
constexpr int GRAM_BLOCKS = 4 * HID * HID / GRAM_T;
template <int C>
__global__ void __launch_bounds__(GRAM_T) k_gram(const float* __restrict__ W3, const float* __restrict__ emb,
                                                 const float* __restrict__ w_read, float* __restrict__ G) {
  __shared__ float w3l[HID][C + 1];  // [k][c]
  __shared__ double d[C];            // 2 w_c h_c^2
  constexpr int ROWS = GRAM_T / HID, Q = C / 4, PER = HID * Q / GRAM_T;
  const int l = blockIdx.x / (HID / ROWS), k0 = ROWS * (blockIdx.x % (HID / ROWS));
  float4 v[PER];
  if ((reinterpret_cast<uintptr_t>(W3) & 15) == 0) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int t = threadIdx.x + u * GRAM_T;
      v[u] = *reinterpret_cast<const float4*>(W3 + (size_t)(t / Q) * 4 * C + l * C + 4 * (t % Q));
    }
  } else {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int t = threadIdx.x + u * GRAM_T;
      const float* q = W3 + (size_t)(t / Q) * 4 * C + l * C + 4 * (t % Q);
      v[u] = make_float4(q[0], q[1], q[2], q[3]);
    }
  }
  for (int c = threadIdx.x; c < C; c += GRAM_T) d[c] = 2.0 * (double)w_read[c] * (double)emb[c] * (double)emb[c];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int t = threadIdx.x + u * GRAM_T;
    float* row = &w3l[t / Q][4 * (t % Q)];
    row[0] = v[u].x;
    row[1] = v[u].y;
    row[2] = v[u].z;
    row[3] = v[u].w;
  }
  __syncthreads();
  const int k = k0 + threadIdx.x / HID, kk = threadIdx.x % HID;
  double acc = 0.0;
#pragma unroll 8
  for (int c = 0; c < C; ++c) acc += d[c] * (double)w3l[k][c] * (double)w3l[kk][c];
  G[((size_t)l * HID + k) * HID + kk] = (float)acc;
}

template <int C, int W>
__global__ void __launch_bounds__(64 * W)
k_fold_fused(EdgeIn in, Units un, const float* __restrict__ W1, const float* __restrict__ W2,
             const float* __restrict__ G, float* __restrict__ ei, float* __restrict__ gout,
             float* __restrict__ stash) {
  __shared__ __align__(16) float wl[W12_FLOATS + GRAM_FLOATS];
  __shared__ __align__(16) float wbuf[W][FoldLds<C>::FUSED];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const WaveLds<C> L(wbuf[wave]);
  const float* w1s = wl;
  const float* w2s = wl + NB * LDH;
  float* gs = wl + W12_FLOATS;
  const int N = un.n_atoms;
  const int nbp = (N + W - 1) / W;
  stage_w12<64 * W>(wl, W1, W2, 0, KEXP);  // the scaled chain (KEXP)
  stage_gram<64 * W>(gs, G);
  __syncthreads();
  for (int b = blockIdx.x; b < nbp; b += gridDim.x) {
    const int i = b * W + wave;
    if (i >= N) continue;
    int s = lane & 31, h = lane >> 5;
    asm volatile("" : "+v"(s), "+v"(h));
    const int qa = un.row_ptr[i], qb = un.row_ptr[i + 1];
    f32x4 T[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) T[b] = zero4();
    const Recv xi = recv_pos(in, i);
    float* zw = stash + (size_t)(blockIdx.x * W + wave) * STASH_TILES * 32 * ZROW;
    for (int q0 = qa; q0 < qb; q0 += 32)
      fwd_tile<true>(in, nullptr, xi, w1s, w2s, L.ysm, q0, qa, qb, s, h, T, stash_tile(zw, q0, qa));
    // T block b register r, lane l: hidden 16 b + 4 (l / 16) + r, harmonic l % 16
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) L.tsm[16 * b + 4 * (lane >> 4) + r][lane & 15] = T[b][r];
    wave_sync_lds();
    // M[lm][k] = sum_k' G_l(lm)[k][k'] T[k'][lm] and E_i = 1/2 sum T M (lane = hidden k)
    float macc[NLM];
    const float* g = gs + lane * GI_LD;
    const float e2 = gram_epilogue(L.tsm, lane, [&](int kk) { return *reinterpret_cast<const float4*>(g + 4 * kk); },
                                   macc);
    if (lane == 0) ei[i] = e2 * KEXP_INV2;  // T carries KEXP
    if (qb <= qa) continue;
    wave_sync_lds();  // msm overlays tsm
#pragma unroll
    for (int lm = 0; lm < NLM; ++lm) L.msm[lm][lane] = macc[lm] * KEXP_INV2;  // M / KEXP
    wave_sync_lds();
    for (int q0 = qa; q0 < qb; q0 += 32)
      bwd_tile<true>(in, xi, nullptr, w1s, w2s, L.msm, L.ybsm, q0, qa, qb, s, h, gout, stash_tile(zw, q0, qa));
  }
}

// ------------------------------------------------------------------ split (one species, few receivers)
// With fewer receivers than the chip has wave slots, one wave per receiver
// leaves most CUs idle and one receiver's tiles in sequence are the whole
// call.  Here a workgroup takes two receivers at a time (i and i + gridDim.x)
// and its W waves share their tiles, in one list (the first receiver's, then
// the second's; wave w: tiles w, w + W, ...): five tiles a receiver fill eight
// waves better in pairs than alone (no SIMD runs three tiles where one runs
// one).  Each wave sums its partial T of each receiver into LDS; the readout
// adds them up per receiver and forms M and E_i from G in global memory (G is
// symmetric, so lane k reads G_l[k'][k] along a row), and every wave runs the
// backward of its own tiles from its own stash rows.
template <int C, int W>
__global__ void __launch_bounds__(64 * W)
k_fold_split(EdgeIn in, Units un, const float* __restrict__ W1, const float* __restrict__ W2,
             const float* __restrict__ G, float* __restrict__ ei, float* __restrict__ gout,
             float* __restrict__ stash) {
  __shared__ float w12[W12_FLOATS];
  __shared__ __align__(16) float wbuf[W][FoldLds<C>::FUSED];
  __shared__ __align__(16) float tsm2[W][HID * NLM];  // the waves' partial T of the second receiver
  __shared__ __align__(16) float msh[2][NLM][HID + 1];  // M of the two receivers, read by every wave
  __shared__ float esh2[2][W];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const WaveLds<C> L(wbuf[wave]);
  const float* w1s = w12;
  const float* w2s = w12 + NB * LDH;
  const int N = un.n_atoms;
  stage_w12<64 * W>(w12, W1, W2, 0, KEXP);  // the scaled chain (KEXP)
  __syncthreads();
  float* zw = stash + (size_t)(blockIdx.x * W + wave) * STASH_TILES * 32 * ZROW;
  // T block b register r, lane l: hidden 16 b + 4 (l / 16) + r, harmonic l % 16
  auto put_t = [&](const f32x4 T[4], float* dst) {
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(16 * b + 4 * (lane >> 4) + r) * NLM + (lane & 15)] = T[b][r];
  };
  for (int i0 = blockIdx.x; i0 < N; i0 += 2 * gridDim.x) {
    int s = lane & 31, h = lane >> 5;
    asm volatile("" : "+v"(s), "+v"(h));
    const int i1 = i0 + gridDim.x;
    const int qa[2] = {un.row_ptr[i0], i1 < N ? un.row_ptr[i1] : 0};
    const int qb[2] = {un.row_ptr[i0 + 1], i1 < N ? un.row_ptr[i1 + 1] : 0};
    const int n0 = (qb[0] - qa[0] + 31) >> 5, n1 = (qb[1] - qa[1] + 31) >> 5;
    const Recv xi[2] = {recv_pos(in, i0), recv_pos(in, i1 < N ? i1 : i0)};
    f32x4 T[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) T[b] = zero4();
    int cur = 0, j = 0;
    for (int t = wave; t < n0 + n1; t += W, ++j) {
      const int r = t < n0 ? 0 : 1;
      if (r != cur) {  // the first receiver's partial is complete
        put_t(T, &L.tsm[0][0]);
#pragma unroll
        for (int b = 0; b < 4; ++b) T[b] = zero4();
        cur = 1;
      }
      const int q0 = qa[r] + 32 * (r ? t - n0 : t);
      fwd_tile<true>(in, nullptr, xi[r], w1s, w2s, L.ysm, q0, qa[r], qb[r], s, h, T,
                     j < STASH_TILES ? zw + (size_t)j * 32 * ZROW : nullptr);
    }
    if (cur == 0) {
      put_t(T, &L.tsm[0][0]);
#pragma unroll
      for (int b = 0; b < 4; ++b) T[b] = zero4();
    }
    if (i1 < N) put_t(T, tsm2[wave]);
    __syncthreads();
    {
      float e2[2];
      gram_epilogue_pair<W, FoldLds<C>::TSM, FoldLds<C>::FUSED>(&wbuf[0][FoldLds<C>::TSM], &wbuf[0][0], &tsm2[0][0],
                                                                 i1 < N, G, lane, wave, msh[0], msh[1], esh2,
                                                                 KEXP_INV2, e2);
      if (threadIdx.x == 0) {
        ei[i0] = e2[0];
        if (i1 < N) ei[i1] = e2[1];
      }
    }
    __syncthreads();
    j = 0;
    for (int t = wave; t < n0 + n1; t += W, ++j) {
      const int r = t < n0 ? 0 : 1;
      const int q0 = qa[r] + 32 * (r ? t - n0 : t);
      bwd_tile<true>(in, xi[r], nullptr, w1s, w2s, msh[r], L.ybsm, q0, qa[r], qb[r], s, h, gout,
                     j < STASH_TILES ? zw + (size_t)j * 32 * ZROW : nullptr);
    }
    __syncthreads();  // msh and the wave buffers are rewritten for the next pair
  }
}

// ------------------------------------------------------------------ radial tables
// The one-species fused call with s2 and ds2/dr read from the radial tables
// (piecewise polynomials of the chain r -> s2, degree TAB_DEG in the piece
// variable t) in place of the basis, the first two layers and their SiLUs:
// the forward tile evaluates s2 and ds2/dr by Horner's rule (lane s: hidden
// units s and s + 32 of 16 edges, the layout the second layer leaves), keeps
// both in the stash rows, and accumulates T as the network kernel does; the
// backward tile takes rbar = sum_k s2bar_k ds2_k/dr directly.  An edge at or
// beyond the table's end (r >= rc) contributes exactly zero.
struct TabArgs {
  const float2* tab;     // [coarse c][sub-piece f < TAB_SUB][m][32] pairs (hidden j, j + 32)
  const int32_t* level;  // [coarse c] sub-pieces 2^level
  double inv_h0;         // 2^K / rc: r -> r / h0
  int n_coarse;
};

// The slice of a table set that belongs to species pair p.
__device__ __forceinline__ TabArgs tab_pair(const TabArgs& ta, int p) {
  TabArgs t = ta;
  t.tab += (size_t)p * ta.n_coarse * TAB_SUB * TAB_NC * 32;
  t.level += (size_t)p * ta.n_coarse;
  return t;
}

// Sub-piece and local variable of an edge at distance r (binary64, then
// float32): u = r / h0, coarse c = floor(u), w = (u - c) 2^d(c), f = floor(w),
// t = 2 (w - f) - 1 in [-1, 1), dt/dr = 2^(d+1) / h0.  Returned as (t, slot
// c TAB_SUB + f or -1 for "no value", dt/dr, 0).
__device__ __forceinline__ float4 tab_locate(const TabArgs& ta, double r, bool valid) {
  const double u = r * ta.inv_h0;
  const double cf = floor(u);
  const bool in_range = valid && cf >= 0.0 && cf < (double)ta.n_coarse;
  const int c = in_range ? (int)cf : 0;
  const int d = min(max(ta.level[c], 0), TAB_DMAX);
  const double w = ldexp(u - cf, d);
  const double ff = fmin(floor(w), (double)((1 << d) - 1));
  const float t = in_range ? (float)(2.0 * (w - ff) - 1.0) : 0.f;
  const int slot = in_range ? c * TAB_SUB + (int)ff : -1;
  return make_float4(t, __int_as_float(slot), (float)ldexp(2.0 * ta.inv_h0, d), 0.f);
}

// Value and t-derivative of the pair of units at `c` (TAB_NC coefficients, 32 float2 apart).
__device__ __forceinline__ void tab_horner(const float2* __restrict__ c, float t, float2& v, float2& d) {
  float2 cc[TAB_NC];
#pragma unroll
  for (int m = 0; m < TAB_NC; ++m) cc[m] = c[32 * m];
  v = cc[TAB_DEG];
  d = make_float2(0.f, 0.f);
#pragma unroll
  for (int m = TAB_DEG - 1; m >= 0; --m) {
    d.x = d.x * t + v.x;
    d.y = d.y * t + v.y;
    v.x = v.x * t + cc[m].x;
    v.y = v.y * t + cc[m].y;
  }
}

template <bool PAD = true>
__device__ __forceinline__ void fwd_tile_tab(const EdgeIn& in, const int32_t* perm, const Recv& xi,
                                             const TabArgs& ta, float4* tp, float (*ysm)[NLM + 1], int q0, int qa,
                                             int qb, int s, int h, f32x4 T[4], float* zs) {
  const bool valid = q0 + s < qb;
  const Geo g = geo_from_raw(in, edge_raw(in, tile_edge(perm, q0, qa, qb, s)), xi.x);
  if (zs != nullptr && h == 0 && (PAD || valid)) {  // as fwd_tile
    float* row = zs + s * ZROW + 2 * HID;
    float rw[2];
    __builtin_memcpy(rw, &g.r, sizeof(double));
    *reinterpret_cast<float4*>(row) = make_float4(g.ux, g.uy, g.uz, g.inv_r);
    *reinterpret_cast<float2*>(row + 4) = make_float2(rw[0], rw[1]);
  }
  if (h == 0) tp[s] = tab_locate(ta, g.r, valid);
  {
    float Y[16];
    sph16(g.ux, g.uy, g.uz, Y);
#pragma unroll
    for (int k = 0; k < 8; ++k) ysm[s][8 * h + k] = valid ? (h ? Y[8 + k] : Y[k]) : 0.f;  // static indices
  }
  wave_sync_lds();
  // s2 with edges on M: register r of tile m = edge fperm(r) + 4h, hidden 32 m + s.
  // Edges in pairs, the coefficients of the next pair loading while this
  // pair's Horner steps run (a scheduling fence after each pair keeps the
  // look-ahead at one pair, within the registers).  The stash rows are
  // written as they come, padding rows too (a tile's 32 rows exist; rows past
  // the unit's end are never read), so no lane-dependent branch splits the
  // sequence.
  f32x16 a[2];
  float2 cc[2][2][TAB_NC];
  float4 loc[2][2];
  auto fetch = [&](int g, float2 (&dst)[2][TAB_NC], float4 (&lc)[2]) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      lc[q] = tp[fperm(2 * g + q) + 4 * h];
      const float2* c = ta.tab + (size_t)max(__float_as_int(lc[q].y), 0) * TAB_NC * 32 + s;
#pragma unroll
      for (int m = 0; m < TAB_NC; ++m) dst[q][m] = c[32 * m];
    }
  };
  fetch(0, cc[0], loc[0]);
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    if (g + 1 < 8) fetch(g + 1, cc[(g + 1) & 1], loc[(g + 1) & 1]);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r = 2 * g + q;
      const float4 e = loc[g & 1][q];
      const float on = __float_as_int(e.y) >= 0 ? 1.f : 0.f;
      const float2* c = cc[g & 1][q];
      float2 v = c[TAB_DEG], d = make_float2(0.f, 0.f);
#pragma unroll
      for (int m = TAB_DEG - 1; m >= 0; --m) {
        d.x = d.x * e.x + v.x;
        d.y = d.y * e.x + v.y;
        v.x = v.x * e.x + c[m].x;
        v.y = v.y * e.x + c[m].y;
      }
      a[0][r] = v.x * on;
      a[1][r] = v.y * on;
      if (zs != nullptr) {
        float* row = zs + (fperm(r) + 4 * h) * ZROW + s;
        row[0] = d.x * e.z * on;
        row[32] = d.y * e.z * on;
        row[HID] = a[0][r];
        row[HID + 32] = a[1][r];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // T[hidden][lm] += s2^T Y over the tile on 16x16x4 tiles (as fwd_tile)
  {
    const int j = s & 15, qk = (s >> 4) + 2 * h;
    const float* yrow = &ysm[8 * (qk & 1) + 4 * (qk >> 1)][j];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int rr = 0; rr < 12; rr = (rr == 3 ? 8 : rr + 1)) {
        float lo = a[m][rr], hi = a[m][rr + 4];
        swap_rows16(lo, hi);
        const float yv = yrow[fperm(rr) * (NLM + 1)];
        T[2 * m] = mfma16(lo, yv, T[2 * m]);
        T[2 * m + 1] = mfma16(hi, yv, T[2 * m + 1]);
      }
    pipeline_lds_mfma<32, 2, 6>();
  }
  wave_sync_lds();
}

__device__ __forceinline__ void bwd_tile_tab(const EdgeIn& in, const Recv& xi, const int32_t* perm,
                                             const TabArgs& ta, float (*msm)[HID + 1], float (*ybsm)[NLM + 1],
                                             int q0, int qa, int qb, int s, int h, float* __restrict__ gout,
                                             const float* zs) {
  const bool valid = q0 + s < qb;
  const int64_t e = tile_edge(perm, q0, qa, qb, s);
  Geo g;
  f32x16 ds[2], s2[2];  // ds2/dr and s2, edges on N: register 4j + i of tile m = hidden 4h + 32m + 8j + i
  if (zs != nullptr) {
    const float* row = zs + (valid ? s : 0) * ZROW;
    const float4 u = *reinterpret_cast<const float4*>(row + 2 * HID);
    const float2 rw = *reinterpret_cast<const float2*>(row + 2 * HID + 4);
    g.ux = u.x;
    g.uy = u.y;
    g.uz = u.z;
    g.inv_r = u.w;
    __builtin_memcpy(&g.r, &rw, sizeof(double));
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 v1 = *reinterpret_cast<const float4*>(row + 4 * h + 32 * m + 8 * j);
        const float4 v2 = *reinterpret_cast<const float4*>(row + HID + 4 * h + 32 * m + 8 * j);
        ds[m][4 * j] = v1.x; ds[m][4 * j + 1] = v1.y; ds[m][4 * j + 2] = v1.z; ds[m][4 * j + 3] = v1.w;
        s2[m][4 * j] = v2.x; s2[m][4 * j + 1] = v2.y; s2[m][4 * j + 2] = v2.z; s2[m][4 * j + 3] = v2.w;
      }
  } else {
    g = geo_from_raw(in, edge_raw(in, e), xi.x);
    const float4 loc = tab_locate(ta, g.r, valid);
    const int piece = __float_as_int(loc.y);
    const float on = piece >= 0 ? 1.f : 0.f;
    const float2* c = ta.tab + (size_t)max(piece, 0) * TAB_NC * 32 + 4 * h;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float2 v, d;
        tab_horner(c + 8 * j + i, loc.x, v, d);  // units 4h + 8j + i and + 32
        s2[0][4 * j + i] = v.x * on;
        s2[1][4 * j + i] = v.y * on;
        ds[0][4 * j + i] = d.x * loc.z * on;
        ds[1][4 * j + i] = d.y * loc.z * on;
      }
  }
  __builtin_amdgcn_sched_barrier(0);
  // Ybar[edge][lm] = sum_k s2[edge][k] M[lm][k] on 16x16x4 tiles (as bwd_tile)
  f32x4 yb[2];
  yb[0] = zero4();
  yb[1] = zero4();
  {
    const int j = s & 15, qk = (s >> 4) + 2 * h;
    const float* mrow = &msm[j][8 * (qk & 1) + 4 * (qk >> 1)];
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
#pragma unroll
      for (int rr = 0; rr < 12; rr = (rr == 3 ? 8 : rr + 1)) {
        float lo = s2[mm][rr], hi = s2[mm][rr + 4];
        swap_rows16(lo, hi);
        const float bv = mrow[32 * mm + fperm(rr)];
        yb[0] = mfma16(lo, bv, yb[0]);
        yb[1] = mfma16(hi, bv, yb[1]);
      }
    pipeline_lds_mfma<32, 2, 6>();
  }
  __builtin_amdgcn_sched_barrier(0);
  // s2bar[k][edge] = sum_lm M[lm][k] Y[edge][lm]  (edges on N)
  f32x16 sb[2];
  sb[0] = zero16();
  sb[1] = zero16();
  {
    float Y[16];
    sph16(g.ux, g.uy, g.uz, Y);
    const float* mc = &msm[h][s];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const float bv = h ? Y[2 * ks + 1] : Y[2 * ks];
#pragma unroll
      for (int m = 0; m < 2; ++m) sb[m] = mfma32(mc[2 * ks * (HID + 1) + 32 * m], bv, sb[m]);
    }
    pipeline_lds_mfma<16, 2, 6>();
  }
  __builtin_amdgcn_sched_barrier(0);
  {
    const int l = s + 32 * h;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) ybsm[16 * b + 4 * (l >> 4) + i][l & 15] = yb[b][i];
  }
  wave_sync_lds();
  float G[3];
  {
    float ybe[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) ybe[k] = ybsm[s][k];
    sph16_grad_dot(g.ux, g.uy, g.uz, ybe, G);
  }
  float rbar = 0.f;
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) rbar += sb[m][r] * ds[m][r];
  rbar += __shfl_xor(rbar, 32);
  const float gu = G[0] * g.ux + G[1] * g.uy + G[2] * g.uz;
  if (valid && h == 0) {
    store_grad_row(gout, e, rbar * g.ux + (G[0] - gu * g.ux) * g.inv_r, rbar * g.uy + (G[1] - gu * g.uy) * g.inv_r,
                   rbar * g.uz + (G[2] - gu * g.uz) * g.inv_r);
  }
  wave_sync_lds();
}

// Few receivers: a workgroup per receiver, its W waves sharing the row's tiles
// (as k_fold_split), s2 and ds2/dr from the radial table.
template <int C, int W>
__global__ void __launch_bounds__(64 * W)
k_fold_split_table(EdgeIn in, Units un, TabArgs ta, const float* __restrict__ G, float* __restrict__ ei,
                   float* __restrict__ gout, float* __restrict__ stash) {
  __shared__ __align__(16) float wbuf[W][FoldLds<C>::FUSED];
  __shared__ __align__(16) float msh[NLM][HID + 1];  // M of the receiver, read by every wave
  __shared__ float esh[W];
  __shared__ float4 tpb[W][32];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const WaveLds<C> L(wbuf[wave]);
  const int N = un.n_atoms;
  float* zw = stash + (size_t)(blockIdx.x * W + wave) * STASH_TILES * 32 * ZROW;
  for (int i = blockIdx.x; i < N; i += gridDim.x) {
    int s = lane & 31, h = lane >> 5;
    asm volatile("" : "+v"(s), "+v"(h));
    const int qa = un.row_ptr[i], qb = un.row_ptr[i + 1];
    const Recv xi = recv_pos(in, i);
    f32x4 T[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) T[b] = zero4();
    int j = 0;
    for (int q0 = qa + 32 * wave; q0 < qb; q0 += 32 * W, ++j)
      fwd_tile_tab(in, nullptr, xi, ta, tpb[wave], L.ysm, q0, qa, qb, s, h, T,
                   j < STASH_TILES ? zw + (size_t)j * 32 * ZROW : nullptr);
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) L.tsm[16 * b + 4 * (lane >> 4) + r][lane & 15] = T[b][r];
    __syncthreads();
    {
      const float e2 = gram_epilogue_split<W, FoldLds<C>::TSM, FoldLds<C>::FUSED>(
          &wbuf[0][FoldLds<C>::TSM], &wbuf[0][0], G, lane, wave, msh, esh);
      if (threadIdx.x == 0) ei[i] = e2;
    }
    __syncthreads();
    j = 0;
    for (int q0 = qa + 32 * wave; q0 < qb; q0 += 32 * W, ++j)
      bwd_tile_tab(in, xi, nullptr, ta, msh, L.ybsm, q0, qa, qb, s, h, gout,
                   j < STASH_TILES ? zw + (size_t)j * 32 * ZROW : nullptr);
    __syncthreads();  // msh and the wave buffers are rewritten for the next receiver
  }
}

template <int C, int W>
__global__ void __launch_bounds__(64 * W)
k_fold_table(EdgeIn in, Units un, TabArgs ta, const float* __restrict__ G, float* __restrict__ ei,
             float* __restrict__ gout, float* __restrict__ stash) {
  __shared__ __align__(16) float gs[GRAM_FLOATS];
  __shared__ __align__(16) float wbuf[W][FoldLds<C>::FUSED];
  __shared__ float4 tpb[W][32];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const WaveLds<C> L(wbuf[wave]);
  const int N = un.n_atoms;
  const int nbp = (N + W - 1) / W;
  stage_gram<64 * W>(gs, G);
  __syncthreads();
  for (int b = blockIdx.x; b < nbp; b += gridDim.x) {
    const int i = b * W + wave;
    if (i >= N) continue;
    int s = lane & 31, h = lane >> 5;
    asm volatile("" : "+v"(s), "+v"(h));
    const int qa = un.row_ptr[i], qb = un.row_ptr[i + 1];
    f32x4 T[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) T[b] = zero4();
    const Recv xi = recv_pos(in, i);
    float* zw = stash + (size_t)(blockIdx.x * W + wave) * STASH_TILES * 32 * ZROW;
    for (int q0 = qa; q0 < qb; q0 += 32)
      fwd_tile_tab(in, nullptr, xi, ta, tpb[wave], L.ysm, q0, qa, qb, s, h, T, stash_tile(zw, q0, qa));
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) L.tsm[16 * b + 4 * (lane >> 4) + r][lane & 15] = T[b][r];
    wave_sync_lds();
    float macc[NLM];
    const float* g = gs + lane * GI_LD;
    const float e2 = gram_epilogue(L.tsm, lane, [&](int kk) { return *reinterpret_cast<const float4*>(g + 4 * kk); },
                                   macc);
    if (lane == 0) ei[i] = e2;
    if (qb <= qa) continue;
    wave_sync_lds();  // msm overlays tsm
#pragma unroll
    for (int lm = 0; lm < NLM; ++lm) L.msm[lm][lane] = macc[lm];
    wave_sync_lds();
    for (int q0 = qa; q0 < qb; q0 += 32)
      bwd_tile_tab(in, xi, nullptr, ta, L.msm, L.ybsm, q0, qa, qb, s, h, gout, stash_tile(zw, q0, qa));
  }
}

// ------------------------------------------------------------------ fused (several species)
// Two or three species: one wave per receiver, workgroups taking batches of
// receivers of one species (atoms in species order).  For each sender species
// s in turn the workgroup stages the weights of pair (Z_i, s) in LDS and every
// wave runs the forward tiles of its unit (s, i) and adds h_s T_s^T W3 to its
// A; then E_i and dE/dA; then, species by species again, M_s =
// (dE/dA h_s) W3^T and the backward tiles of (s, i), in reverse order so that
// the last forward species' weights are reused.  The activation stash is
// shared by a receiver's units (its first STASH_TILES tiles in s order).  With
// C = 64, W3 sits in LDS too (read along rows for A, down columns for M);
// with C = 128 it is read from global memory (W3 and its transposed copy).
constexpr int MULTI_MAX_S = 3;

template <int C, bool W3L>
struct MultiLds {
  static constexpr int PW = FoldLds<C>::BWD_ONLY > FoldLds<C>::FWD_ONLY ? FoldLds<C>::BWD_ONLY : FoldLds<C>::FWD_ONLY;
  static constexpr int W3I = W12_FLOATS;  // the interleaved W3 after W1 and W2
  static constexpr int WEIGHTS = W3L ? W12_FLOATS + W3I_FLOATS : W12_FLOATS;
};

// TAB: s2 and ds2/dr of each sender species' pair from the radial tables (only
// W3 is staged); otherwise from the network.
template <int C, int W, bool W3L, bool TAB>
__global__ void __launch_bounds__(64 * W)
k_fold_multi(EdgeIn in, Units un, const int32_t* __restrict__ ord, const int32_t* __restrict__ zstart,
             const float* __restrict__ W1, const float* __restrict__ W2, const float* __restrict__ W3,
             const float* __restrict__ W3T, const float* __restrict__ emb, const float* __restrict__ w_read,
             TabArgs ta, float* __restrict__ ei, float* __restrict__ gout, float* __restrict__ stash) {
  constexpr int NC = 4 * C, CPL = C / 64;
  static_assert(!W3L || C == 64, "the interleaved LDS copy of W3 is laid out for 64 channels");
  __shared__ __align__(16) float wl[MultiLds<C, W3L>::WEIGHTS];
  __shared__ __align__(16) float wbuf[W][MultiLds<C, W3L>::PW];
  __shared__ float4 tpb[W][32];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const WaveLds<C> L(wbuf[wave]);
  const float* w1s = wl + Lds<C>::W1;
  const float* w2s = wl + Lds<C>::W2;
  const int N = un.n_atoms, S = un.S;
  // batches of W receivers of one species, species after species
  int bstart[MULTI_MAX_S + 1];
  bstart[0] = 0;
#pragma unroll
  for (int z = 0; z < MULTI_MAX_S; ++z)
    bstart[z + 1] = bstart[z] + (z < S ? (zstart[z + 1] - zstart[z] + W - 1) / W : 0);
  const int total = bstart[MULTI_MAX_S];
  float* zw = stash + (size_t)(blockIdx.x * W + wave) * STASH_TILES * 32 * ZROW;
  // the network runs the scaled chain (W1 staged as KEXP W1); p is uniform over
  // the workgroup, and a pair already in LDS (the last backward species of one
  // batch is the first forward species of the next) is not staged again
  constexpr bool K = !TAB;
  int loaded = -1;
  auto stage = [&](int p) {
    if ((TAB && !W3L) || p == loaded) return;  // nothing to stage
    __syncthreads();
    if (TAB)
      stage_w3i<64 * W>(wl + MultiLds<C, W3L>::W3I, W3 + (size_t)p * HID * NC);
    else if (W3L) {
      stage_w12<64 * W>(wl, W1, W2, p, KEXP);
      stage_w3i<64 * W>(wl + MultiLds<C, W3L>::W3I, W3 + (size_t)p * HID * NC);
    } else
      stage_w12<64 * W>(wl, W1, W2, p, KEXP);
    __syncthreads();
    loaded = p;
  };
  for (int b = blockIdx.x; b < total; b += gridDim.x) {
    int z = 0;
#pragma unroll
    for (int k = 1; k < MULTI_MAX_S; ++k) z += (k < S && bstart[k] <= b) ? 1 : 0;
    const int zb = z == 0 ? 0 : (z == 1 ? bstart[1] : bstart[2]);
    const int idx = zstart[z] + (b - zb) * W + wave;
    const bool valid = idx < zstart[z + 1];
    const int i = valid ? min(max(ord[idx], 0), N - 1) : 0;
    int s = lane & 31, h = lane >> 5;
    asm volatile("" : "+v"(s), "+v"(h));
    const Recv xi = recv_pos(in, i);
    float acc[CPL][NLM];
#pragma unroll
    for (int q = 0; q < CPL; ++q)
#pragma unroll
      for (int k = 0; k < NLM; ++k) acc[q][k] = 0.f;
    int t = 0;
    for (int sp = 0; sp < S; ++sp) {
      const int p = z * S + sp;
      stage(p);
      const int qa = valid ? un.seg[2 * ((size_t)sp * N + i)] : 0;
      const int qb = valid ? un.seg[2 * ((size_t)sp * N + i) + 1] : 0;
      if (qb <= qa) continue;
      f32x4 T[4];
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) T[bb] = zero4();
      for (int q0 = qa; q0 < qb; q0 += 32, ++t) {
        float* zs = t < STASH_TILES ? zw + (size_t)t * 32 * ZROW : nullptr;
        if (TAB)
          fwd_tile_tab<false>(in, un.perm, xi, tab_pair(ta, p), tpb[wave], L.ysm, q0, qa, qb, s, h, T, zs);
        else
          fwd_tile<K, false>(in, un.perm, xi, w1s, w2s, L.ysm, q0, qa, qb, s, h, T, zs);
      }
      float as[CPL][NLM];
      if (W3L)
        unit_last_layer<C, 0>(T, L.tsm, wl + MultiLds<C, W3L>::W3I, lane, as);
      else
        unit_last_layer<C, NC>(T, L.tsm, W3 + (size_t)p * HID * NC, lane, as);
#pragma unroll
      for (int q = 0; q < CPL; ++q) {
        const float hc = emb[(size_t)sp * C + lane + 64 * q];
#pragma unroll
        for (int k = 0; k < NLM; ++k) acc[q][k] += hc * as[q][k];
      }
    }
    // E_i = sum_c w_c sum_lm A^2; acc becomes dE/dA = 2 w A.  With the scaled
    // chain acc = KEXP A: E_i takes 1 / KEXP^2, and dE/dA is kept as
    // 2 w A / KEXP, which the backward's scaled s2 cancels.
    constexpr float KS = K ? KEXP_INV2 : 1.f;
    float esum = 0.f;
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      const float wc = w_read[lane + 64 * q];
      float sq = 0.f;
#pragma unroll
      for (int k = 0; k < NLM; ++k) {
        sq += acc[q][k] * acc[q][k];
        acc[q][k] *= 2.f * wc * KS;
      }
      esum += wc * sq;
    }
    esum *= KS;
    for (int off = 32; off > 0; off >>= 1) esum += __shfl_xor(esum, off);
    if (valid && lane == 0) ei[i] = esum;
    // backward in reverse species order: the last forward species' weights are
    // still staged
    for (int r = 0; r < S; ++r) {
      const int sp = S - 1 - r;
      const int p = z * S + sp;
      if (r > 0) stage(p);
      const int qa = valid ? un.seg[2 * ((size_t)sp * N + i)] : 0;
      const int qb = valid ? un.seg[2 * ((size_t)sp * N + i) + 1] : 0;
      if (qb <= qa) continue;
      int t = 0;  // the forward's tile count before species sp
      for (int s2 = 0; s2 < sp; ++s2)
        t += (un.seg[2 * ((size_t)s2 * N + i) + 1] - un.seg[2 * ((size_t)s2 * N + i)] + 31) >> 5;
#pragma unroll
      for (int q = 0; q < CPL; ++q) {
        const int c = lane + 64 * q;
        const float hc = emb[(size_t)sp * C + c];
#pragma unroll
        for (int k = 0; k < NLM; ++k) L.ahsm[c][k] = acc[q][k] * hc;
      }
      wave_sync_lds();
      if (W3L)
        unit_M<C, 0>(L.ahsm, wl + MultiLds<C, W3L>::W3I + lane * W3I_LD, lane, L.msm);
      else
        unit_M<C, HID>(L.ahsm, W3T + (size_t)p * NC * HID + lane, lane, L.msm);
      for (int q0 = qa; q0 < qb; q0 += 32, ++t) {
        const float* zs = t < STASH_TILES ? zw + (size_t)t * 32 * ZROW : nullptr;
        if (TAB)
          bwd_tile_tab(in, xi, un.perm, tab_pair(ta, p), L.msm, L.ybsm, q0, qa, qb, s, h, gout, zs);
        else
          bwd_tile<K>(in, xi, un.perm, w1s, w2s, L.msm, L.ybsm, q0, qa, qb, s, h, gout, zs);
      }
    }
  }
}

// W3T[p][j][k] = W3[p][k][j]: the backward reads W3 down its columns.
__global__ void k_transpose_w3(int P, int NC, const float* __restrict__ W3, float* __restrict__ W3T) {
  const int64_t n = (int64_t)P * HID * NC;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < n; t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t p = t / ((int64_t)HID * NC), rem = t % ((int64_t)HID * NC);
    const int k = (int)(rem / NC), j = (int)(rem % NC);
    W3T[(p * NC + j) * HID + k] = W3[t];
  }
}

constexpr int WAVES = 8;

EdgeIn make_in_f(const ConvPlan& p, const eec_graph* g, const double* pos, Box box, double cutoff,
                 const int32_t* species) {
  EdgeIn in;
  in.pos = pos;
  in.Lx = box.L[0];
  in.Ly = box.L[1];
  in.Lz = box.L[2];
  in.rc = cutoff;
  in.inv_rc = 1.0 / cutoff;
  in.inv_rc_f = (float)(1.0 / cutoff);
  in.recv = nullptr;  // the unit kernels know each edge's receiver
  in.col = g->col;
  in.shift = g->shift;
  in.species = species;
  in.n_atoms = g->n_atoms;
  in.n_edges = g->n_edges;
  return in;
}

Units make_units(const ConvPlan& p, const eec_graph* g, const int32_t* species, const char* ws) {
  Units un;
  un.row_ptr = g->row_ptr;
  un.species = species;
  un.perm = p.S > 1 ? (const int32_t*)(ws + p.off_perm) : nullptr;
  un.seg = p.S > 1 ? (const int32_t*)(ws + p.off_seg) : nullptr;
  un.n_atoms = p.N;
  un.S = p.S;
  return un;
}

TabArgs tab_args(const eec_model* m, int log2_pieces, const float* tab, const int32_t* level) {
  TabArgs ta;
  ta.tab = reinterpret_cast<const float2*>(tab);
  ta.level = level;
  ta.n_coarse = 1 << log2_pieces;
  ta.inv_h0 = (double)ta.n_coarse / m->cutoff;
  return ta;
}

int unit_grid(const ConvPlan& p) {
  const int64_t batches = (int64_t)p.P * ((p.N + WAVES - 1) / WAVES);
  return (int)std::max<int64_t>(1, std::min<int64_t>(batches, 256));
}

// One species and at most this many receivers: a workgroup per receiver
// (k_fold_split) instead of a wave per receiver (k_fold_fused).
constexpr int SPLIT_MAX_ATOMS = 768;  // past it a wave per receiver is faster (measured)
bool use_split(const ConvPlan& p) { return p.N <= SPLIT_MAX_ATOMS; }
int split_grid(const ConvPlan& p) { return std::max(1, std::min(p.N, 256)); }

int multi_grid(const ConvPlan& p) {
  return (int)std::max<int64_t>(1, std::min<int64_t>((p.N + WAVES - 1) / WAVES + p.S, 256));
}

}  // namespace

bool fold_multi_supported(const ConvPlan& p) { return p.S >= 2 && p.S <= MULTI_MAX_S; }

void launch_fold_table(hipStream_t s, const ConvPlan& p, const eec_graph* g, const double* pos, Box box,
                       double cutoff, const eec_model* m, int log2_pieces, const float* tab,
                       const int32_t* level, float* ei, float* gout, char* ws) {
  if (p.N == 0) return;
  const float* G = (const float*)(ws + p.off_w3t);
  float* stash = (float*)(ws + p.off_stash);
  const EdgeIn in = make_in_f(p, g, pos, box, cutoff, nullptr);
  const Units un = make_units(p, g, nullptr, ws);
  const TabArgs ta = tab_args(m, log2_pieces, tab, level);
  if (use_split(p)) {
    if (p.C == 64)
      k_fold_split_table<64, WAVES><<<split_grid(p), 64 * WAVES, 0, s>>>(in, un, ta, G, ei, gout, stash);
    else
      k_fold_split_table<128, WAVES><<<split_grid(p), 64 * WAVES, 0, s>>>(in, un, ta, G, ei, gout, stash);
  } else if (p.C == 64) {
    k_fold_table<64, WAVES><<<unit_grid(p), 64 * WAVES, 0, s>>>(in, un, ta, G, ei, gout, stash);
  } else {
    k_fold_table<128, WAVES><<<unit_grid(p), 64 * WAVES, 0, s>>>(in, un, ta, G, ei, gout, stash);
  }
}

size_t fold_stash_bytes(const ConvPlan& p) {
  int waves = 0;
  if (p.S == 1) waves = (use_split(p) ? split_grid(p) : unit_grid(p)) * WAVES;
  else if (fold_multi_supported(p)) waves = multi_grid(p) * WAVES;
  return sizeof(float) * (size_t)waves * STASH_TILES * 32 * ZROW;
}

void launch_fold_multi(hipStream_t s, const ConvPlan& p, const eec_graph* g, const double* pos, Box box,
                       double cutoff, const int32_t* species, const eec_model* m, float* ei, float* gout,
                       char* ws, int log2_pieces, const float* tab, const int32_t* level) {
  if (p.N == 0) return;
  const float* W3T = (const float*)(ws + p.off_w3t);
  float* stash = (float*)(ws + p.off_stash);
  const int32_t* ord = (const int32_t*)(ws + p.off_ord);
  const int32_t* zstart = (const int32_t*)(ws + p.off_zstart);
  const EdgeIn in = make_in_f(p, g, pos, box, cutoff, species);
  const Units un = make_units(p, g, species, ws);
  const TabArgs ta = tab_args(m, log2_pieces, tab, level);
  const bool t = tab != nullptr;
  if (p.C == 64 && t)
    k_fold_multi<64, WAVES, true, true><<<multi_grid(p), 64 * WAVES, 0, s>>>(
        in, un, ord, zstart, m->W1, m->W2, m->W3, W3T, m->emb, m->w_read, ta, ei, gout, stash);
  else if (p.C == 64)
    k_fold_multi<64, WAVES, true, false><<<multi_grid(p), 64 * WAVES, 0, s>>>(
        in, un, ord, zstart, m->W1, m->W2, m->W3, W3T, m->emb, m->w_read, ta, ei, gout, stash);
  else if (t)
    k_fold_multi<128, WAVES, false, true><<<multi_grid(p), 64 * WAVES, 0, s>>>(
        in, un, ord, zstart, m->W1, m->W2, m->W3, W3T, m->emb, m->w_read, ta, ei, gout, stash);
  else
    k_fold_multi<128, WAVES, false, false><<<multi_grid(p), 64 * WAVES, 0, s>>>(
        in, un, ord, zstart, m->W1, m->W2, m->W3, W3T, m->emb, m->w_read, ta, ei, gout, stash);
}

void launch_fold_forward(hipStream_t s, const ConvPlan& p, const eec_graph* g, const double* pos,
                         Box box, double cutoff, const int32_t* species, const eec_model* m,
                         float* A_out, char* ws) {
  if (p.N == 0) return;
  const EdgeIn in = make_in_f(p, g, pos, box, cutoff, species);
  const Units un = make_units(p, g, species, ws);
  if (p.C == 64)
    k_fold_forward<64, WAVES><<<unit_grid(p), 64 * WAVES, 0, s>>>(in, un, m->W1, m->W2, m->W3, m->emb, A_out);
  else
    k_fold_forward<128, WAVES><<<unit_grid(p), 64 * WAVES, 0, s>>>(in, un, m->W1, m->W2, m->W3, m->emb, A_out);
}

void launch_transpose_w3(hipStream_t s, const ConvPlan& p, const eec_model* m, char* ws) {
  float* W3T = (float*)(ws + p.off_w3t);
  const int64_t n = (int64_t)p.P * HID * p.NC;
  k_transpose_w3<<<(int)std::min<int64_t>((n + 255) / 256, 4096), 256, 0, s>>>(p.P, p.NC, m->W3, W3T);
}

bool fold_fused_supported(const ConvPlan& p) { return p.S == 1; }

void launch_gram(hipStream_t s, const ConvPlan& p, const eec_model* m, char* ws) {
  float* G = (float*)(ws + p.off_w3t);
  if (p.C == 64)
    k_gram<64><<<GRAM_BLOCKS, GRAM_T, 0, s>>>(m->W3, m->emb, m->w_read, G);
  else
    k_gram<128><<<GRAM_BLOCKS, GRAM_T, 0, s>>>(m->W3, m->emb, m->w_read, G);
}

void launch_fold_fused(hipStream_t s, const ConvPlan& p, const eec_graph* g, const double* pos, Box box,
                       double cutoff, const int32_t* species, const eec_model* m, float* ei, float* gout,
                       char* ws) {
  if (p.N == 0) return;
  const float* G = (const float*)(ws + p.off_w3t);
  float* stash = (float*)(ws + p.off_stash);
  const EdgeIn in = make_in_f(p, g, pos, box, cutoff, species);
  const Units un = make_units(p, g, species, ws);
  if (use_split(p)) {
    if (p.C == 64)
      k_fold_split<64, WAVES><<<split_grid(p), 64 * WAVES, 0, s>>>(in, un, m->W1, m->W2, G, ei, gout, stash);
    else
      k_fold_split<128, WAVES><<<split_grid(p), 64 * WAVES, 0, s>>>(in, un, m->W1, m->W2, G, ei, gout, stash);
  } else if (p.C == 64) {
    k_fold_fused<64, WAVES><<<unit_grid(p), 64 * WAVES, 0, s>>>(in, un, m->W1, m->W2, G, ei, gout, stash);
  } else {
    k_fold_fused<128, WAVES><<<unit_grid(p), 64 * WAVES, 0, s>>>(in, un, m->W1, m->W2, G, ei, gout, stash);
  }
}

void launch_fold_backward(hipStream_t s, const ConvPlan& p, const eec_graph* g, const double* pos,
                          Box box, double cutoff, const int32_t* species, const eec_model* m,
                          const float* Abar, float* gout, char* ws) {
  if (p.N == 0 || p.E == 0) return;
  const float* W3T = (const float*)(ws + p.off_w3t);
  const EdgeIn in = make_in_f(p, g, pos, box, cutoff, species);
  const Units un = make_units(p, g, species, ws);
  if (p.C == 64)
    k_fold_backward<64, WAVES><<<unit_grid(p), 64 * WAVES, 0, s>>>(in, un, m->W1, m->W2, W3T, m->emb, Abar, gout);
  else
    k_fold_backward<128, WAVES><<<unit_grid(p), 64 * WAVES, 0, s>>>(in, un, m->W1, m->W2, W3T, m->emb, Abar, gout);
}

}  // namespace eec

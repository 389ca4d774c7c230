// FP32 matrix-core kernels of the radial network.
//
//  k_radial   : geometry -> basis (or a given basis) -> z1 = b W1 -> silu ->
//               z2 = s1 W2 -> silu -> R = s2 W3, per 32-edge tile, writing R
//               rows (and harmonics rows) of a chunk of edges.  The chain
//               (E,4,32) -> (E,4,64) -> (E,256) is the radial projection of
//               "deepmd-kit PR #6108", What; it is compute-bound there
//               ("deepmd-kit PR #6108", Why not a fused Triton kernel) and runs
//               here on v_mfma_f32_32x32x2_f32 with weights staged in LDS.
//  k_backward : the matching input-gradient backward per edge tile
//               ("deepmd-kit PR #2", Implementation and scope: finish the
//               reverse chain of one edge cohort before the next), recomputing
//               the forward activations instead of storing them:
//                 Rbar_{l,c} = h_c sum_m Abar_{i,lm,c} Y_lm,
//                 Ybar_lm    = sum_c Abar_{i,lm,c} h_c R_{l,c},
//                 s2bar = Rbar W3^T, z2bar = s2bar silu'(z2), s1bar = z2bar W2^T,
//                 z1bar = s1bar silu'(z1), bbar = z1bar W1^T,
//                 rbar = sum_n bbar_n db_n/dr,
//                 g = rbar u + (I - u u^T) (sum_lm Ybar_lm grad Y_lm) / r.
//
// Work decomposition: edges are taken in pair-grouped order (one weight set per
// tile), in 32-edge tiles, one tile per wave; a workgroup of W waves holds one
// pair's weights in LDS and walks "batches" of W tiles of that pair, grid-stride.
#include <algorithm>

#include "chain.hpp"

namespace eec {
namespace {
using namespace chain;

// ------------------------------------------------------------------ forward
// With `emb` non-NULL the rows written are rho = R h_{Z_j} (the sender embedding
// folded into the streamed chunk, which the message pass then only sums);
// otherwise plain R.
template <int C, int W, bool BASIS_IN>
__global__ void __launch_bounds__(64 * W)
k_radial(EdgeIn in, Sched sc, const float* __restrict__ W1, const float* __restrict__ W2,
         const float* __restrict__ W3, const float* __restrict__ emb, int n_species,
         const float* __restrict__ basis_in, int64_t row_base, float* __restrict__ R_out,
         float* __restrict__ Y_out) {
  constexpr int NC = Lds<C>::NC;
  constexpr bool SCALED = !BASIS_IN;
  __shared__ float lds[Lds<C>::FLOATS];
  __shared__ SchedState st;
  sched_init<W>(sc, st);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int s = lane & 31, h = lane >> 5;
  const float* w1s = lds + Lds<C>::W1;
  const float* w2s = lds + Lds<C>::W2;
  const float* w3s = lds + Lds<C>::W3;
  int loaded = -1;
  const int nb = st.bstart[sc.P];
  for (int b = blockIdx.x; b < nb; b += gridDim.x) {
    int p = 0;
    while (p + 1 < sc.P && st.bstart[p + 1] <= b) ++p;
    if (p != loaded) {
      __syncthreads();
      stage_weights<C, 64 * W>(lds, W1, W2, W3, p, SCALED ? KEXP : 1.f);  // the scaled chain stages KEXP W1
      __syncthreads();
      loaded = p;
    }
    const int tile = (b - st.bstart[p]) * W + wave;
    if (tile >= st.ntile[p]) continue;
    const int64_t q = st.q0[p] + (int64_t)tile * 32 + s;
    const bool valid = q < st.q1[p];
    const int64_t qq = valid ? q : st.q0[p];
    const int64_t e = sc.perm ? (int64_t)sc.perm[qq] : qq;

    float bas[16];
    const Geo g = edge_geo(in, e);
    if (BASIS_IN) {
#pragma unroll
      for (int k = 0; k < 16; ++k) bas[k] = basis_in[e * NB + 16 * h + k];
    } else {
      basis16f<false>(basis_seed(g.r, in.inv_rc, g.inv_r, h), in.inv_rc_f, h, bas, nullptr);
    }
    if (Y_out != nullptr && valid) {
      float Y[16];
      sph16(g.ux, g.uy, g.uz, Y);
      float* yo = Y_out + (e - row_base) * NLM + 8 * h;
#pragma unroll
      for (int k = 0; k < 8; ++k) yo[k] = h ? Y[8 + k] : Y[k];
    }
    f32x16 z[2], a[2];
    layer1(w1s, bas, s, h, z);
    silu_tiles_t<SCALED>(z, a);
    layer2(w2s, a, s, h, z);
    silu_tiles_t<SCALED>(z, a);  // a = s2 (edges on N; as the A operand: edge = s), times KEXP when SCALED

    // output row of the edge held by accumulator register r (edge slot fperm(r) + 4h)
    const int my_row = valid ? (int)(e - row_base) : -1;
    int orow[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) orow[r] = __shfl(my_row, fperm(r) + 4 * h);
    const bool full = __all(valid);
    constexpr int HPL = C / 32;
    float hcv[HPL];
#pragma unroll
    for (int j = 0; j < HPL; ++j)
      hcv[j] = (emb ? emb[(size_t)(p % n_species) * C + 32 * j + s] : 1.f) * (SCALED ? 1.f / KEXP : 1.f);

    // R = s2 W3 with edges on M: D[edge][feature], lane = feature 32 t + s.
    constexpr int LD3 = Lds<C>::LD3;
    const float* w3 = w3s + 4 * h * LD3 + s;  // W3[hid_k0(ks) + 4 h][32 t + s]
#pragma unroll 1
    for (int t = 0; t < NC / 32; ++t, w3 += 32) {
      f32x16 acc = zero16();
#pragma unroll
      for (int ks = 0; ks < 32; ++ks) acc = mfma32(a[ks >> 4][ks & 15], w3[hid_k0(ks) * LD3], acc);
      pipeline_lds_mfma<32, 1, 6>();
      float hc = hcv[0];
#pragma unroll
      for (int j = 1; j < HPL; ++j) hc = (t % HPL) == j ? hcv[j] : hc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] *= hc;
      if (full) {  // no padding slot in the tile: stores without per-row predicates
#pragma unroll
        for (int r = 0; r < 16; ++r) R_out[(size_t)orow[r] * NC + 32 * t + s] = acc[r];
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (orow[r] >= 0) R_out[(size_t)orow[r] * NC + 32 * t + s] = acc[r];
      }
    }
  }
}

// ------------------------------------------------------------------ fused forward
// One wave per (ordered species pair, receiver) unit: the receiver's edges of
// that pair, in 32-edge tiles aligned to the receiver, through geometry ->
// basis -> z1 -> z2 (edges on N) -> rho = (s2 W3) h (edges on M: the lane owns
// one channel column of 16 edges) and the message accumulated in registers:
// A_{i,lm,c} += rho_{e,l,c} Y_{e,lm}, in a fixed order.  Each lane half sums its
// own 16 edge rows of every tile; the halves are added at the end.  The tile's
// harmonics go through a per-wave LDS slot (rows of padding edges are zero).
// No radial row ever leaves the chip.  Output: the unit's partial A (sender
// species s) at A_out + (s * N + i) * 16 * C.


template <int W>
__global__ void __launch_bounds__(64 * W)
k_forward(EdgeIn in, Units un, const float* __restrict__ W1, const float* __restrict__ W2,
          const float* __restrict__ W3, const float* __restrict__ emb, float* __restrict__ A_out) {
  constexpr int C = 64;
  constexpr int LD3 = Lds<C>::LD3;
  __shared__ float lds[Lds<C>::FLOATS];
  __shared__ float ysm[W][32][NLM + 1];  // one padding column against bank conflicts
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int s = lane & 31, h = lane >> 5;
  const float* w1s = lds + Lds<C>::W1;
  const float* w2s = lds + Lds<C>::W2;
  const float* w3s = lds + Lds<C>::W3;
  const int N = un.n_atoms, S = un.S, P = S * S;
  const int nbp = (N + W - 1) / W;  // batches of W receivers per pair
  int loaded = -1;
  for (int b = blockIdx.x; b < P * nbp; b += gridDim.x) {
    const int p = b / nbp;
    if (p != loaded) {
      __syncthreads();
      stage_weights<C, 64 * W>(lds, W1, W2, W3, p);
      __syncthreads();
      loaded = p;
    }
    const int i = (b - p * nbp) * W + wave;
    if (i >= N) continue;
    const int zs = p % S;
    int qa, qb;
    if (S == 1) {
      qa = un.row_ptr[i];
      qb = un.row_ptr[i + 1];
    } else {
      if (min(max(un.species[i], 0), S - 1) != p / S) continue;  // another pair's receiver
      qa = un.seg[2 * ((size_t)zs * N + i)];
      qb = un.seg[2 * ((size_t)zs * N + i) + 1];
    }
    const float* hrow = emb + (size_t)zs * C;
    const float h0 = hrow[s], h1 = hrow[32 + s];  // channel of tiles with t even / odd
    float acc[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) acc[k] = 0.f;

    for (int q0 = qa; q0 < qb; q0 += 32) {
      const int q = q0 + s;
      const bool valid = q < qb;
      const int qq = valid ? q : qa;
      const int64_t e = un.perm ? (int64_t)un.perm[qq] : (int64_t)qq;
      const Geo g = edge_geo(in, e);
      f32x16 z[2], a[2];
      {
        float bas[16];
        basis16f<false>(basis_seed(g.r, in.inv_rc, g.inv_r, h), in.inv_rc_f, h, bas, nullptr);
        layer1(w1s, bas, s, h, z);
      }
      silu_tiles(z, a);
      layer2(w2s, a, s, h, z);
      silu_tiles(z, a);  // a = s2; as the A operand: row = edge slot s
      {
        float Y[16];
        sph16(g.ux, g.uy, g.uz, Y);
#pragma unroll
        for (int k = 0; k < 8; ++k) ysm[wave][s][8 * h + k] = valid ? (h ? Y[8 + k] : Y[k]) : 0.f;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const float* w3 = w3s + 4 * h * LD3 + s;  // W3[hid_k0(ks) + 4 h][32 t + s]
#pragma unroll
      for (int l = 0; l < 4; ++l) {
        // the two 32-channel tiles of degree l: t = 2 l (channel s) and 2 l + 1 (32 + s)
        f32x16 r0 = zero16(), r1 = zero16();
#pragma unroll
        for (int ks = 0; ks < 32; ++ks) {
          const float av = a[ks >> 4][ks & 15];
          r0 = mfma32(av, w3[hid_k0(ks) * LD3 + 64 * l], r0);
          r1 = mfma32(av, w3[hid_k0(ks) * LD3 + 64 * l + 32], r1);
        }
        __builtin_amdgcn_sched_barrier(0);
        constexpr int off[4] = {0, 2, 8, 18};  // acc offset of (l, tile 2l); tile 2l+1 follows
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float* yr = &ysm[wave][fperm(r) + 4 * h][l * l];
          const float p0 = r0[r] * h0, p1 = r1[r] * h1;
#pragma unroll
          for (int m = 0; m < 2 * l + 1; ++m) {
            const float y = yr[m];
            acc[off[l] + m] += p0 * y;
            acc[off[l] + 2 * l + 1 + m] += p1 * y;
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }
    // add the two lane halves' edge subsets; half 0 writes the even tiles, half 1 the odd
#pragma unroll
    for (int k = 0; k < 32; ++k) acc[k] += __shfl_xor(acc[k], 32);
    float* ai = A_out + ((size_t)zs * N + i) * NLM * C + 32 * h + s;
    constexpr int off[4] = {0, 2, 8, 18};
#pragma unroll
    for (int l = 0; l < 4; ++l)
#pragma unroll
      for (int m = 0; m < 2 * l + 1; ++m)
        ai[(l * l + m) * C] = h == 0 ? acc[off[l] + m] : acc[off[l] + 2 * l + 1 + m];
  }
}

// ------------------------------------------------------------------ backward
template <int C, int W>
__global__ void __launch_bounds__(64 * W)
k_backward(EdgeIn in, Sched sc, const float* __restrict__ W1, const float* __restrict__ W2,
           const float* __restrict__ W3, const float* __restrict__ emb, int n_species,
           const float* __restrict__ Abar, float* __restrict__ gout) {
  __shared__ float lds[Lds<C>::FLOATS];
  __shared__ SchedState st;
  sched_init<W>(sc, st);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lane_s = lane & 31, lane_h = lane >> 5;
  const float* w1s = lds + Lds<C>::W1;
  const float* w2s = lds + Lds<C>::W2;
  const float* w3s = lds + Lds<C>::W3;
  int loaded = -1;
  const int nb = st.bstart[sc.P];
  for (int b = blockIdx.x; b < nb; b += gridDim.x) {
    int p = 0;
    while (p + 1 < sc.P && st.bstart[p + 1] <= b) ++p;
    if (p != loaded) {
      __syncthreads();
      stage_weights<C, 64 * W>(lds, W1, W2, W3, p);
      __syncthreads();
      loaded = p;
    }
    const int tile = (b - st.bstart[p]) * W + wave;
    if (tile >= st.ntile[p]) continue;
    // re-derive the lane coordinates every tile: keeps the compiler from
    // hoisting lane-dependent addresses out of the loop into spilled registers
    int s = lane_s, h = lane_h;
    asm volatile("" : "+v"(s), "+v"(h));
    const int64_t q = st.q0[p] + (int64_t)tile * 32 + s;
    const bool valid = q < st.q1[p];
    const int64_t qq = valid ? q : st.q0[p];
    const int64_t e = sc.perm ? (int64_t)sc.perm[qq] : qq;
    const int zj = p % n_species;

    const Geo g = edge_geo(in, e);
    f32x16 z[2], a[2];
    {
      float bas[16];
      basis16f<false>(basis_seed(g.r, in.inv_rc, g.inv_r, h), in.inv_rc_f, h, bas, nullptr);
      layer1(w1s, bas, s, h, z);
    }
    silu_tiles(z, a);
    layer2(w2s, a, s, h, z);
    silu_tiles(z, a);  // a = s2
    float Y[16];
    sph16(g.ux, g.uy, g.uz, Y);

    const float* abar = Abar + (size_t)g.i * NLM * C;
    const float* hrow = emb + (size_t)zj * C;
    f32x16 sb[2];
    sb[0] = zero16();
    sb[1] = zero16();
    float ybp[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) ybp[k] = 0.f;

    constexpr int LD3 = Lds<C>::LD3;
    constexpr int TPL = C / 32;  // 32-feature tiles per degree
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      const float* w3r = w3s + 4 * h * LD3 + s + 32 * TPL * l;  // W3[hid_k0(ks) + 4 h][32 t + s]
      const float* w3c = w3s + s * LD3 + 4 * h + 32 * TPL * l;  // W3[32 m + s][32 t + fperm(ks) + 4 h]
#pragma unroll 1
      for (int tc = 0; tc < TPL; ++tc, w3r += 32, w3c += 32) {
        // R tile (edges on N): register r = feature (l, c = 32 tc + fperm(r) + 4h) of edge s
        f32x16 acc = zero16();
#pragma unroll
        for (int ks = 0; ks < 32; ++ks) acc = mfma32(w3r[hid_k0(ks) * LD3], a[ks >> 4][ks & 15], acc);
        __builtin_amdgcn_sched_barrier(0);
        const int cb = 32 * tc + 4 * h;
        float hv[16], rb[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 v = *reinterpret_cast<const float4*>(hrow + cb + 8 * q4);
          hv[4 * q4 + 0] = v.x; hv[4 * q4 + 1] = v.y; hv[4 * q4 + 2] = v.z; hv[4 * q4 + 3] = v.w;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          acc[r] *= hv[r];  // rho = R h
          rb[r] = 0.f;
        }
#pragma unroll
        for (int lm = l * l; lm < (l + 1) * (l + 1); ++lm) {
          const float* ar = abar + lm * C + cb;
          float av[16];
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const float4 v = *reinterpret_cast<const float4*>(ar + 8 * q4);
            av[4 * q4 + 0] = v.x; av[4 * q4 + 1] = v.y; av[4 * q4 + 2] = v.z; av[4 * q4 + 3] = v.w;
          }
          float yb = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            yb += av[r] * acc[r];
            rb[r] += av[r] * Y[lm];
          }
          ybp[lm] += yb;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) rb[r] *= hv[r];
        __builtin_amdgcn_sched_barrier(0);
        // s2bar += W3[:, tile] Rbar_tile (edges on N)
#pragma unroll
        for (int ks = 0; ks < 16; ++ks)
#pragma unroll
          for (int m = 0; m < 2; ++m) sb[m] = mfma32(w3c[32 * m * LD3 + fperm(ks)], rb[ks], sb[m]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // Ybar (both lane halves hold partial sums over their channels) and its
    // contraction with the harmonic gradients, G = sum_lm Ybar_lm grad Y_lm
    float G[3];
    {
      float yb[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) yb[k] = ybp[k] + __shfl_xor(ybp[k], 32);
      sph16_grad_dot(g.ux, g.uy, g.uz, yb, G);
    }
    __builtin_amdgcn_sched_barrier(0);

    // recompute the basis (with its r-derivative), z1 and z2: nothing of the
    // forward stays live through the loop above
    float bas[16], dbas[16];
    basis16f<true>(basis_seed(g.r, in.inv_rc, g.inv_r, h), in.inv_rc_f, h, bas, dbas);
    f32x16 z1[2], s1[2];
    layer1(w1s, bas, s, h, z1);
    silu_tiles(z1, s1);
    layer2(w2s, s1, s, h, z);  // z = z2
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) sb[m][r] *= silu_d(z[m][r]);  // z2bar
    __builtin_amdgcn_sched_barrier(0);
    // s1bar = z2bar W2^T
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
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) s1b[m][r] *= silu_d(z1[m][r]);  // z1bar
    // bbar = z1bar W1^T; row rho carries basis basis_of_row(rho)
    f32x16 bb = zero16();
    const float* w1c = w1s + basis_of_row(s) * LDH + 4 * h;  // W1[basis_of_row(s)][hid_k0(ks) + 4 h]
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) bb = mfma32(w1c[hid_k0(ks)], s1b[ks >> 4][ks & 15], bb);
    float rbar = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) rbar += bb[r] * dbas[r];
    rbar += __shfl_xor(rbar, 32);

    const float gu = G[0] * g.ux + G[1] * g.uy + G[2] * g.uz;
    if (valid && h == 0) {
      store_grad_row(gout, e, rbar * g.ux + (G[0] - gu * g.ux) * g.inv_r,
                     rbar * g.uy + (G[1] - gu * g.uy) * g.inv_r, rbar * g.uz + (G[2] - gu * g.uz) * g.inv_r);
    }
  }
}

constexpr int WAVES = 8;

EdgeIn make_in(const ConvPlan& p, const eec_graph* g, const double* pos, Box box, double cutoff,
               const int32_t* species, const char* ws) {
  EdgeIn in;
  in.pos = pos;
  in.Lx = box.L[0];
  in.Ly = box.L[1];
  in.Lz = box.L[2];
  in.rc = cutoff;
  in.inv_rc = 1.0 / cutoff;
  in.inv_rc_f = (float)(1.0 / cutoff);
  in.recv = (const int32_t*)(ws + p.off_recv);
  in.col = g->col;
  in.shift = g->shift;
  in.species = species;
  in.n_atoms = g->n_atoms;
  in.n_edges = g->n_edges;
  return in;
}

Sched make_sched(const ConvPlan& p, const char* ws, int64_t e0, int64_t e1) {
  Sched sc;
  sc.P = p.P;
  sc.e0 = e0;
  sc.e1 = e1;
  if (p.S > 1) {
    sc.perm = (const int32_t*)(ws + p.off_perm);
    sc.pair_start = (const int64_t*)(ws + p.off_pair_start);
  } else {
    sc.perm = nullptr;
    sc.pair_start = nullptr;
  }
  return sc;
}

int grid_for(const ConvPlan& p, int64_t e0, int64_t e1) {
  const int64_t tiles = (e1 - e0 + 31) / 32 + p.P;
  const int64_t batches = (tiles + WAVES - 1) / WAVES + p.P;
  return (int)std::max<int64_t>(1, std::min<int64_t>(batches, 256));
}

}  // namespace

void launch_radial(hipStream_t s, const ConvPlan& p, const eec_graph* g, const double* pos, Box box,
                   double cutoff, const int32_t* species, const eec_model* m, const float* basis_in,
                   int64_t e_begin, int64_t e_end, float* R_out, float* Y_out, const char* ws) {
  if (e_end <= e_begin) return;
  const EdgeIn in = make_in(p, g, pos, box, cutoff, species, ws);
  const Sched sc = make_sched(p, ws, e_begin, e_end);
  const int grid = grid_for(p, e_begin, e_end);
  // materialising mode (a given basis) writes R rows at edge index; streaming
  // mode writes rho = R h rows of the chunk [e_begin, e_end) and its harmonics
  const int64_t row_base = basis_in ? 0 : e_begin;
  const float* emb = basis_in ? nullptr : m->emb;
  if (p.C == 64) {
    if (basis_in)
      k_radial<64, WAVES, true><<<grid, 64 * WAVES, 0, s>>>(in, sc, m->W1, m->W2, m->W3, emb, p.S, basis_in, row_base, R_out, Y_out);
    else
      k_radial<64, WAVES, false><<<grid, 64 * WAVES, 0, s>>>(in, sc, m->W1, m->W2, m->W3, emb, p.S, nullptr, row_base, R_out, Y_out);
  } else {
    if (basis_in)
      k_radial<128, WAVES, true><<<grid, 64 * WAVES, 0, s>>>(in, sc, m->W1, m->W2, m->W3, emb, p.S, basis_in, row_base, R_out, Y_out);
    else
      k_radial<128, WAVES, false><<<grid, 64 * WAVES, 0, s>>>(in, sc, m->W1, m->W2, m->W3, emb, p.S, nullptr, row_base, R_out, Y_out);
  }
}

bool fused_forward_supported(const ConvPlan& p) { return p.C == 64; }

void launch_forward(hipStream_t s, const ConvPlan& p, const eec_graph* g, const double* pos, Box box,
                    double cutoff, const int32_t* species, const eec_model* m, float* A_out,
                    const char* ws) {
  if (p.N == 0) return;
  const EdgeIn in = make_in(p, g, pos, box, cutoff, species, ws);
  Units un;
  un.row_ptr = g->row_ptr;
  un.species = species;
  un.perm = p.S > 1 ? (const int32_t*)(ws + p.off_perm) : nullptr;
  un.seg = p.S > 1 ? (const int32_t*)(ws + p.off_seg) : nullptr;
  un.n_atoms = p.N;
  un.S = p.S;
  const int64_t batches = (int64_t)p.P * ((p.N + WAVES - 1) / WAVES);
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(batches, 256));
  k_forward<WAVES><<<grid, 64 * WAVES, 0, s>>>(in, un, m->W1, m->W2, m->W3, m->emb, A_out);
}

void launch_backward(hipStream_t s, const ConvPlan& p, const eec_graph* g, const double* pos, Box box,
                     double cutoff, const int32_t* species, const eec_model* m, const float* Abar,
                     float* gout, const char* ws) {
  if (p.E == 0) return;
  const EdgeIn in = make_in(p, g, pos, box, cutoff, species, ws);
  const Sched sc = make_sched(p, ws, 0, p.E);
  const int grid = grid_for(p, 0, p.E);
  if (p.C == 64)
    k_backward<64, WAVES><<<grid, 64 * WAVES, 0, s>>>(in, sc, m->W1, m->W2, m->W3, m->emb, p.S, Abar, gout);
  else
    k_backward<128, WAVES><<<grid, 64 * WAVES, 0, s>>>(in, sc, m->W1, m->W2, m->W3, m->emb, p.S, Abar, gout);
}

}  // namespace eec

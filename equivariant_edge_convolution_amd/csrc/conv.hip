// Memory-bound kernels of the edge convolution: graph preparation, the
// streaming message and receiver reduction, the energy readout, the force
// scatter (with virial) and the materialised basis.
//
// Every per-atom sum runs in a fixed order with no float atomics: the pages
// reject a per-atom reduction that needs atomics because it breaks
// reproducible gradients ("FastMACE rewrite screens", OPT-T02 stage D) and keep
// deterministic graph sums (OPT4-T02 polar_graph_sums).
#include <algorithm>

#include "eec_device.hpp"
#include "eec_internal.hpp"

namespace eec {
namespace {

inline int blocks_for(int64_t n, int per) {
  return (int)std::max<int64_t>(1, std::min<int64_t>((n + per - 1) / per, 1 << 20));
}

// ------------------------------------------------------------ preparation
// recv[e] = receiver of edge e; zero A rows of atoms without edges.
__global__ void __launch_bounds__(256) k_recv(int32_t n, const int32_t* __restrict__ rp,
                                              int64_t E, int32_t* __restrict__ recv,
                                              float* __restrict__ A, int C) {
  const int lane = threadIdx.x & 63;
  for (int i = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6); i < n;
       i += (int)((gridDim.x * blockDim.x) >> 6)) {
    const int a = max(0, min(rp[i], (int)E)), b = max(a, min(rp[i + 1], (int)E));
    for (int e = a + lane; e < b; e += 64) recv[e] = i;
    if (A != nullptr && a == b)
      for (int k = lane; k < NLM * C; k += 64) A[(size_t)i * NLM * C + k] = 0.f;
  }
}

constexpr int PB = 1024;  // edges per counting block

__device__ __forceinline__ int pair_of(int64_t e, const int32_t* recv, const int32_t* col,
                                       const int32_t* species, int S, int n) {
  const int i = min(max(recv[e], 0), n - 1), j = min(max(col[e], 0), n - 1);
  const int zi = min(max(species[i], 0), S - 1), zj = min(max(species[j], 0), S - 1);
  return zi * S + zj;
}

__global__ void __launch_bounds__(256) k_pair_count(int64_t E, const int32_t* __restrict__ recv,
                                                    const int32_t* __restrict__ col,
                                                    const int32_t* __restrict__ species, int S,
                                                    int n, int64_t nb, int32_t* __restrict__ cnt) {
  __shared__ int32_t c[16];
  const int P = S * S;
  if (threadIdx.x < 16) c[threadIdx.x] = 0;
  __syncthreads();
  const int64_t b = blockIdx.x;
  for (int k = threadIdx.x; k < PB; k += blockDim.x) {
    const int64_t e = b * PB + k;
    if (e < E) atomicAdd(&c[pair_of(e, recv, col, species, S, n)], 1);
  }
  __syncthreads();
  if (threadIdx.x < P) cnt[(int64_t)threadIdx.x * nb + b] = c[threadIdx.x];
}

// Exclusive scan (pair-major, then block) of the block counts; pair_start[p].
__global__ void __launch_bounds__(1024) k_pair_scan(int64_t nb, int P, const int32_t* __restrict__ cnt,
                                                    int64_t* __restrict__ off,
                                                    int64_t* __restrict__ pair_start, int64_t E) {
  __shared__ int64_t part[1024];
  const int t = threadIdx.x;
  const int64_t n = nb * P;
  const int64_t per = (n + 1023) / 1024;
  const int64_t a = std::min<int64_t>(n, t * per), b = std::min<int64_t>(n, a + per);
  int64_t s = 0;
  for (int64_t k = a; k < b; ++k) s += cnt[k];
  part[t] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    int64_t v = (t >= o) ? part[t - o] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int64_t run = part[t] - s;
  for (int64_t k = a; k < b; ++k) {
    off[k] = run;
    if (k % nb == 0) pair_start[k / nb] = run;
    run += cnt[k];
  }
  if (t == 0) pair_start[P] = E;
}

// Stable scatter: perm[pos] = e with edges grouped by pair, CSR order inside a group.
__global__ void __launch_bounds__(256) k_pair_scatter(int64_t E, const int32_t* __restrict__ recv,
                                                      const int32_t* __restrict__ col,
                                                      const int32_t* __restrict__ species, int S,
                                                      int n, int64_t nb,
                                                      const int64_t* __restrict__ off,
                                                      int32_t* __restrict__ perm) {
  __shared__ int32_t pre[16][257];
  const int P = S * S;
  const int t = threadIdx.x;
  const int64_t b = blockIdx.x;
  int pr[4];
  int mycnt[16];
#pragma unroll
  for (int p = 0; p < 16; ++p) mycnt[p] = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t e = b * PB + 4 * t + k;
    pr[k] = (e < E) ? pair_of(e, recv, col, species, S, n) : -1;
    if (pr[k] >= 0) mycnt[pr[k]]++;
  }
  for (int p = 0; p < P; ++p) pre[p][t + 1] = mycnt[p];
  if (t == 0)
    for (int p = 0; p < P; ++p) pre[p][0] = 0;
  __syncthreads();
  // inclusive scan over threads per pair (Hillis-Steele on entries 1..256)
  for (int o = 1; o < 256; o <<= 1) {
    int v[16];
    for (int p = 0; p < P; ++p) v[p] = (t >= o) ? pre[p][t + 1 - o] : 0;
    __syncthreads();
    for (int p = 0; p < P; ++p) pre[p][t + 1] += v[p];
    __syncthreads();
  }
  int seen[16];
#pragma unroll
  for (int p = 0; p < 16; ++p) seen[p] = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int p = pr[k];
    if (p < 0) continue;
    const int64_t e = b * PB + 4 * t + k;
    const int64_t pos = off[(int64_t)p * nb + b] + pre[p][t] + seen[p];
    seen[p]++;
    perm[pos] = (int32_t)e;
  }
}

// Position range, in the pair-grouped order, of the edges of receiver i whose
// sender has species s: inside the group of pair (Z_i, s) the CSR indices
// ascend, so the range is [lower_bound(row_ptr[i]), lower_bound(row_ptr[i+1])).
__global__ void __launch_bounds__(256) k_seg_bounds(int32_t n, int S, const int32_t* __restrict__ rp,
                                                    const int32_t* __restrict__ species,
                                                    const int64_t* __restrict__ pair_start,
                                                    const int32_t* __restrict__ perm,
                                                    int32_t* __restrict__ seg) {
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (t >= (int64_t)n * S) return;
  const int s = (int)(t / n), i = (int)(t % n);
  const int zi = min(max(species[i], 0), S - 1);
  const int p = zi * S + s;
  int64_t lo = pair_start[p], hi = pair_start[p + 1];
  const int64_t g1 = hi;
  const int64_t a = rp[i], b = rp[i + 1];
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if ((int64_t)perm[mid] < a) lo = mid + 1; else hi = mid;
  }
  int64_t lo2 = lo, hi2 = g1;
  while (lo2 < hi2) {
    const int64_t mid = (lo2 + hi2) >> 1;
    if ((int64_t)perm[mid] < b) lo2 = mid + 1; else hi2 = mid;
  }
  seg[2 * t] = (int32_t)lo;
  seg[2 * t + 1] = (int32_t)lo2;
}

// Row-local grouping by sender species: perm lists row i's edges with the
// senders of species 0 first, then 1, ..., each group in CSR order, and
// seg[s][i] is the position range of group s (positions are CSR positions).
// One wave per row: a counting pass, then a placing pass, by ballots.
__global__ void __launch_bounds__(256) k_row_partition(int32_t n, int S, int64_t E, const int32_t* __restrict__ rp,
                                                       const int32_t* __restrict__ col,
                                                       const int32_t* __restrict__ species,
                                                       int32_t* __restrict__ perm, int32_t* __restrict__ seg) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int i = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6); i < n; i += (int)((gridDim.x * blockDim.x) >> 6)) {
    const int a = max(0, min(rp[i], (int)E)), b = max(a, min(rp[i + 1], (int)E));
    int cnt[4] = {0, 0, 0, 0};
    for (int e0 = a; e0 < b; e0 += 64) {
      const int e = e0 + lane;
      const int sp = e < b ? min(max(species[min(max(col[e], 0), n - 1)], 0), S - 1) : -1;
#pragma unroll
      for (int z = 0; z < 4; ++z) cnt[z] += __popcll(__ballot(sp == z));
    }
    int start[4];
    start[0] = a;
#pragma unroll
    for (int z = 1; z < 4; ++z) start[z] = start[z - 1] + cnt[z - 1];
    if (lane < S) {
      int lo = start[0], hi = start[0] + cnt[0];
#pragma unroll
      for (int z = 1; z < 4; ++z)
        if (lane == z) { lo = start[z]; hi = start[z] + cnt[z]; }
      seg[2 * ((size_t)lane * n + i)] = lo;
      seg[2 * ((size_t)lane * n + i) + 1] = hi;
    }
    for (int e0 = a; e0 < b; e0 += 64) {
      const int e = e0 + lane;
      const int sp = e < b ? min(max(species[min(max(col[e], 0), n - 1)], 0), S - 1) : -1;
#pragma unroll
      for (int z = 0; z < 4; ++z) {
        const uint64_t m = __ballot(sp == z);
        if (sp == z) perm[start[z] + __popcll(m & below)] = e;
        start[z] += __popcll(m);
      }
    }
  }
}

// Atoms ordered by species, stably, and the species' offsets in that order
// (zstart [S+1]): one workgroup, each thread a contiguous slice of atoms.
constexpr int SO_T = 1024;
__global__ void __launch_bounds__(SO_T) k_species_order(int32_t n, int S, const int32_t* __restrict__ species,
                                                         int32_t* __restrict__ ord, int32_t* __restrict__ zstart) {
  constexpr int NW = SO_T / 64;
  __shared__ int32_t wsum[4][NW];
  __shared__ int32_t base[5];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int per = (n + SO_T - 1) / SO_T;
  const int a = min(n, t * per), b = min(n, a + per);
  int c[4] = {0, 0, 0, 0};
  for (int k = a; k < b; ++k) c[min(max(species[k], 0), S - 1)]++;
  // exclusive prefix of each species' count over the threads: inclusive scans
  // inside each wave, then the wave totals in order
  int incl[4];
#pragma unroll
  for (int z = 0; z < 4; ++z) {
    int v = c[z];
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(v, o);
      if (lane >= o) v += u;
    }
    incl[z] = v;
    if (lane == 63) wsum[z][wv] = v;
  }
  __syncthreads();
  if (t < 4) {
    int run = 0;
    for (int w = 0; w < NW; ++w) {
      const int x = wsum[t][w];
      wsum[t][w] = run;
      run += x;
    }
    base[t + 1] = run;  // species t's total, made cumulative below
  }
  __syncthreads();
  if (t == 0) {
    base[0] = 0;
    for (int z = 0; z < S; ++z) base[z + 1] += base[z];
    for (int z = 0; z <= S; ++z) zstart[z] = base[z];
  }
  __syncthreads();
  int pos[4];
  for (int z = 0; z < S; ++z) pos[z] = base[z] + wsum[z][wv] + incl[z] - c[z];
  for (int k = a; k < b; ++k) ord[pos[min(max(species[k], 0), S - 1)]++] = k;
}

// ------------------------------------------------------------ message
// One workgroup of 4 waves per receiver; lanes over channels; each wave sums a
// contiguous quarter of the receiver's edges inside the chunk in CSR order
// (four edges per step, all loads first), and the quarters are added in a
// fixed order.  The chunk rows already hold rho = R h_{Z_j}.
template <int C>
__global__ void __launch_bounds__(256) k_message(int64_t e0, int64_t e1, const int32_t* __restrict__ rp,
                                                 const int32_t* __restrict__ recv,
                                                 const float* __restrict__ Rc,
                                                 const float* __restrict__ Yc, float* __restrict__ A) {
  constexpr int CPL = C / 64;  // channels per lane
  constexpr int NC = 4 * C;
  constexpr int U = 4;         // edges in flight per wave
  __shared__ float part[3][NLM * C];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i_first = recv[e0], i_last = recv[e1 - 1];
  for (int i = i_first + blockIdx.x; i <= i_last; i += gridDim.x) {
    const int64_t ra = std::max<int64_t>(rp[i], e0), rb = std::min<int64_t>(rp[i + 1], e1);
    const int64_t len = rb - ra, per = (len + 3) / 4;
    const int wa = (int)(std::min(rb, ra + wave * per) - e0);
    const int wb = (int)(std::min<int64_t>(rb, ra + (wave + 1) * per) - e0);
    float acc[CPL][NLM];
#pragma unroll
    for (int q = 0; q < CPL; ++q)
#pragma unroll
      for (int k = 0; k < NLM; ++k) acc[q][k] = 0.f;
    int el = __builtin_amdgcn_readfirstlane(wa);
    for (; el < wb; el += U) {
      float rv[U][CPL][4];
      float y[U][NLM];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int eu = min(el + u, wb - 1);  // in-range duplicate for the tail; weighted 0 below
        const float* rr = Rc + (size_t)eu * NC;
        const float* yr = Yc + (size_t)eu * NLM;
#pragma unroll
        for (int q = 0; q < CPL; ++q)
#pragma unroll
          for (int l = 0; l < 4; ++l) rv[u][q][l] = rr[l * C + lane + 64 * q];
#pragma unroll
        for (int k = 0; k < NLM; ++k) y[u][k] = yr[k];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (el + u < wb) {
#pragma unroll
          for (int q = 0; q < CPL; ++q) {
            acc[q][0] += rv[u][q][0] * y[u][0];
#pragma unroll
            for (int k = 1; k < 4; ++k) acc[q][k] += rv[u][q][1] * y[u][k];
#pragma unroll
            for (int k = 4; k < 9; ++k) acc[q][k] += rv[u][q][2] * y[u][k];
#pragma unroll
            for (int k = 9; k < 16; ++k) acc[q][k] += rv[u][q][3] * y[u][k];
          }
        }
      }
    }
    if (wave > 0) {
#pragma unroll
      for (int q = 0; q < CPL; ++q)
#pragma unroll
        for (int k = 0; k < NLM; ++k) part[wave - 1][k * C + lane + 64 * q] = acc[q][k];
    }
    __syncthreads();
    if (wave == 0) {
      const bool assign = rp[i] >= e0;
      float* ai = A + (size_t)i * NLM * C;
#pragma unroll
      for (int q = 0; q < CPL; ++q)
#pragma unroll
        for (int k = 0; k < NLM; ++k) {
          const int idx = k * C + lane + 64 * q;
          float v = ((acc[q][k] + part[0][idx]) + part[1][idx]) + part[2][idx];
          ai[idx] = assign ? v : ai[idx] + v;
        }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------ readout
// One wave per atom: A = sum over the partial slabs in slab order, E_i =
// sum_c w_c sum_lm A^2 (fixed lane order and shuffle tree), and dE/dA = 2 w A
// written over slab 0.
template <int C>
__global__ void __launch_bounds__(256) k_readout(int32_t n, int nparts, const float* __restrict__ w,
                                                 float* __restrict__ A, float* __restrict__ ei) {
  constexpr int CPL = C / 64;
  const int i = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (i >= n) return;
  float* ai = A + (size_t)i * NLM * C;
  const size_t slab = (size_t)n * NLM * C;
  float sum = 0.f;
#pragma unroll
  for (int q = 0; q < CPL; ++q) {
    const int c = lane + 64 * q;
    const float wc = w[c];
    float s2 = 0.f;
#pragma unroll
    for (int k = 0; k < NLM; ++k) {
      float a = ai[k * C + c];
      for (int pt = 1; pt < nparts; ++pt) a += ai[pt * slab + k * C + c];
      s2 += a * a;
      ai[k * C + c] = 2.f * wc * a;
    }
    sum += wc * s2;
  }
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane == 0) ei[i] = sum;
}

// ------------------------------------------------------------ totals
// Totals of one workgroup of NTH threads, in binary64 with a fixed order: each
// thread a contiguous slice of atoms, then a tree.  E = sum_i E_i; with VIRIAL,
// W = sum_i vpart_i.
constexpr int TT = 256;   // k_totals
constexpr int TS = 512;   // k_scatter: 16 atoms per workgroup, 32 lanes each
template <bool VIRIAL, int NTH>
__device__ void block_totals(int32_t n, const float* __restrict__ ei, const double* __restrict__ vpart,
                             float* __restrict__ energy, float* __restrict__ virial) {
  constexpr int NT = VIRIAL ? 10 : 1;
  __shared__ double part[NT][NTH];
  const int t = threadIdx.x;
  const int per = (n + NTH - 1) / NTH;
  const int a = std::min(n, t * per), b = std::min(n, a + per);
  double acc[NT];
#pragma unroll
  for (int k = 0; k < NT; ++k) acc[k] = 0.0;
  for (int i = a; i < b; ++i) {
    acc[0] += (double)ei[i];
    if (VIRIAL)
#pragma unroll
      for (int k = 0; k < 9; ++k) acc[1 + k] += vpart[9 * (size_t)i + k];
  }
#pragma unroll
  for (int k = 0; k < NT; ++k) part[k][t] = acc[k];
  __syncthreads();
  for (int o = NTH / 2; o > 0; o >>= 1) {
    if (t < o)
#pragma unroll
      for (int k = 0; k < NT; ++k) part[k][t] += part[k][t + o];
    __syncthreads();
  }
  if (t == 0) energy[0] = (float)part[0][0];
  if (VIRIAL && t < 9) virial[t] = (float)part[1 + t][0];
}

// The totals alone (a cell without atoms: zeros).
template <bool VIRIAL>
__global__ void __launch_bounds__(TT) k_totals(int32_t n, const float* __restrict__ ei,
                                               const double* __restrict__ vpart, float* __restrict__ energy,
                                               float* __restrict__ virial) {
  block_totals<VIRIAL, TT>(n, ei, vpart, energy, virial);
}

// ------------------------------------------------------------ force scatter
// Half a wave per atom: F_i = sum_{e in row i} (g_e - g_rev(e)); lane k of the
// half takes edges k, k + 32, ... of the row (five per lane per pass: a
// diamond row of 158 edges in one pass, every reverse index loaded before the
// rows, every row and reverse row before the sums), then a fixed shuffle tree
// over the 32 lanes.  With VIRIAL, also the atom's share of the virial
// -sum_e d_e g_e^T (in binary64).
constexpr int SLPA = 32;  // lanes per atom
constexpr int SU = 5;     // edges per lane per pass
template <bool VIRIAL>
__device__ __forceinline__ void scatter_atom(bool live, int i, int k, int32_t n, int64_t E,
                                             const int32_t* __restrict__ rp, const int32_t* __restrict__ col,
                                             const int8_t* __restrict__ shift, const int32_t* __restrict__ rev,
                                             const double* __restrict__ pos, double Lx, double Ly, double Lz,
                                             const float* __restrict__ g, float* __restrict__ F,
                                             double* __restrict__ vpart) {
  float fx = 0.f, fy = 0.f, fz = 0.f;
  double v[9];
#pragma unroll
  for (int q = 0; q < 9; ++q) v[q] = 0.0;
  const int a = live ? rp[i] : 0, b = live ? rp[i + 1] : 0;
  for (int e0 = a + k; e0 < b; e0 += SLPA * SU) {
    int er[SU];
#pragma unroll
    for (int u = 0; u < SU; ++u) er[u] = e0 + SLPA * u < b ? min(max(rev[e0 + SLPA * u], 0), (int)E - 1) : 0;
    float3 ge[SU], gr[SU];
#pragma unroll
    for (int u = 0; u < SU; ++u) {
      ge[u] = load_grad_row(g, min(e0 + SLPA * u, b - 1));
      gr[u] = load_grad_row(g, er[u]);
    }
#pragma unroll
    for (int u = 0; u < SU; ++u) {
      const int e = e0 + SLPA * u;
      if (e >= b) break;
      fx += ge[u].x - gr[u].x;
      fy += ge[u].y - gr[u].y;
      fz += ge[u].z - gr[u].z;
      if (VIRIAL) {
        const int j = min(max(col[e], 0), n - 1);
        double d[3];
        edge_vector(pos, i, j, shift + 3 * e, Lx, Ly, Lz, d);
        const double gg[3] = {ge[u].x, ge[u].y, ge[u].z};
#pragma unroll
        for (int p = 0; p < 3; ++p)
#pragma unroll
          for (int q = 0; q < 3; ++q) v[3 * p + q] -= d[p] * gg[q];
      }
    }
  }
#pragma unroll
  for (int off = SLPA / 2; off > 0; off >>= 1) {
    fx += __shfl_xor(fx, off);
    fy += __shfl_xor(fy, off);
    fz += __shfl_xor(fz, off);
    if (VIRIAL)
#pragma unroll
      for (int q = 0; q < 9; ++q) v[q] += __shfl_xor(v[q], off);
  }
  if (live && k == 0) {
    F[3 * i] = fx;
    F[3 * i + 1] = fy;
    F[3 * i + 2] = fz;
    if (VIRIAL)
#pragma unroll
      for (int q = 0; q < 9; ++q) vpart[9 * (size_t)i + q] = v[q];
  }
}

// Forces of every atom, TS / SLPA = 16 atoms per workgroup (the gathered
// reverse-edge rows of consecutive atoms are adjacent rows of their shared
// neighbours: a workgroup's waves reuse each other's cache lines in the CU's
// L1).  The per-atom energies are complete before this kernel starts, so when
// `energy` is given one extra workgroup (the first, so that it runs beside the
// scatter rather than after it) forms their total and the call needs no
// reduction launch for it; the virial total needs the whole scatter and runs
// after it (k_totals).  Workgroups go to the eight XCDs in turn (workgroup b
// to XCD b mod 8), so scatter workgroup v takes atom block (v mod 8) nv / 8 +
// v / 8 (nv, the number of scatter workgroups, a multiple of 8): each XCD
// works through one contiguous range of atoms, and the reverse-edge rows that
// neighbouring atoms gather (adjacent rows of a shared neighbour, one cache
// line) are fetched into its L2 once instead of once per XCD.
template <bool VIRIAL>
__global__ void __launch_bounds__(TS) k_scatter(int32_t n, int64_t E, const int32_t* __restrict__ rp,
                                                const int32_t* __restrict__ col,
                                                const int8_t* __restrict__ shift,
                                                const int32_t* __restrict__ rev,
                                                const double* __restrict__ pos, double Lx, double Ly,
                                                double Lz, const float* __restrict__ g,
                                                float* __restrict__ F, double* __restrict__ vpart,
                                                const float* __restrict__ ei, float* __restrict__ energy) {
  constexpr int APB = TS / SLPA;
  const int first = energy != nullptr ? 1 : 0;
  const int nblk = gridDim.x - first;
  if (first && blockIdx.x == 0) {
    block_totals<false, TS>(n, ei, nullptr, energy, nullptr);
    return;
  }
  const int v = blockIdx.x - first;
  const int xv = (v & 7) * (nblk >> 3) + (v >> 3);
  const int k = threadIdx.x % SLPA;
  // the loop bound is uniform over the workgroup, so every lane reaches the shuffles
  for (int base = xv * APB; base < n; base += nblk * APB) {
    const int i = base + (int)(threadIdx.x / SLPA);
    scatter_atom<VIRIAL>(i < n, min(i, n - 1), k, n, E, rp, col, shift, rev, pos, Lx, Ly, Lz, g, F, vpart);
  }
}

// ------------------------------------------------------------ materialised basis
__global__ void __launch_bounds__(256) k_basis(int64_t E, int32_t n, const int32_t* __restrict__ rp,
                                               const int32_t* __restrict__ col,
                                               const int8_t* __restrict__ shift,
                                               const double* __restrict__ pos, double Lx, double Ly,
                                               double Lz, double rc, float* __restrict__ r_out,
                                               float* __restrict__ basis, float* __restrict__ Y) {
  // two threads per edge: half h computes basis 16 h + 1 .. 16 h + 16
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int64_t e = t >> 1;
  const int h = (int)(t & 1);
  if (e >= E) return;
  // receiver: last row whose start is <= e
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)rp[mid] <= e) lo = mid; else hi = mid;
  }
  const int i = lo, j = min(max(col[e], 0), n - 1);
  double d[3];
  edge_vector(pos, i, j, shift + 3 * e, Lx, Ly, Lz, d);
  const double r = sqrt(norm2_nofma(d));
  if (basis) {
    float b[16];
    basis16<false>(r, rc, 16 * h + 1, b, nullptr);
#pragma unroll
    for (int k = 0; k < 16; ++k) basis[e * NB + 16 * h + k] = b[k];
  }
  if (h == 0) {
    if (r_out) r_out[e] = (float)r;
    if (Y) {
      const double ir = 1.0 / r;
      float y[16];
      sph16((float)(d[0] * ir), (float)(d[1] * ir), (float)(d[2] * ir), y);
#pragma unroll
      for (int k = 0; k < 16; ++k) Y[e * NLM + k] = y[k];
    }
  }
}

}  // namespace

// ---------------------------------------------------------------- host side
ConvPlan conv_plan(int32_t n_atoms, int64_t n_edges, const eec_model* m) {
  ConvPlan p{};
  p.C = m->channels;
  p.NC = 4 * p.C;
  p.S = m->n_species;
  p.P = p.S * p.S;
  p.E = n_edges;
  p.N = n_atoms;
  // Chunk of streamed radial rows: at most 192 MiB of R, so the chunk the
  // message pass reads back (with its harmonics) stays inside the 256 MB
  // last-level cache, and a whole number of 32-edge tiles for each of the
  // radial kernel's 2,048 waves (256 workgroups of 8), so no wave idles
  // through a last round: 196,608 edges at 64 channels (three tiles a wave),
  // 65,536 at 128 (one).  Measured at 4,096 atoms and 64 channels: 128 MiB
  // chunks (two tiles a wave) run the radial kernel at 51 % of the matrix
  // peak and the message pass at 4.9 TB/s, 192 MiB at 53 % and 5.6 TB/s;
  // 256 MiB spills the cache (message pass 4.4 TB/s).  At 128 channels 1.5
  // tiles a wave took the radial kernel from 59 % to 49 %.
  constexpr int64_t TILE_ROUND = 256 * 8 * 32;
  const int64_t fit_rows = (int64_t)(192 << 20) / (4 * p.NC);
  const int64_t chunk_rows = std::max<int64_t>(TILE_ROUND, fit_rows / TILE_ROUND * TILE_ROUND);
  p.chunk = std::max<int64_t>(1, std::min<int64_t>(n_edges, chunk_rows));
  p.n_count_blocks = (n_edges + PB - 1) / PB;
  const int64_t N = std::max(n_atoms, 1), E = std::max<int64_t>(n_edges, 1);
  size_t o = 0;
  p.off_recv = o; o += align256(4 * (size_t)E);
  if (p.S > 1) {
    p.off_perm = o;       o += align256(4 * (size_t)E);
    p.off_pair_start = o; o += align256(8 * (size_t)(p.P + 1));
    p.off_blockcnt = o;   o += align256((4 + 8) * (size_t)p.P * std::max<int64_t>(p.n_count_blocks, 1));
    p.off_seg = o;        o += align256(8 * (size_t)p.S * N);
    p.off_ord = o;        o += align256(4 * (size_t)N);
    p.off_zstart = o;     o += 256;
  }
  p.off_A = o;     o += align256(4 * (size_t)p.S * N * NLM * p.C);  // S partial slabs
  p.off_R = o;     o += align256(4 * (size_t)p.chunk * p.NC);
  p.off_Y = o;     o += align256(4 * (size_t)p.chunk * NLM);
  p.off_g = o;     o += align256(4 * 3 * (size_t)E);  // dE/dd per edge, 12-byte rows
  p.off_ei = o;    o += align256(4 * (size_t)N);
  p.off_vpart = o; o += align256(8 * 9 * (size_t)N);
  p.off_w3t = o;   o += align256(4 * (size_t)p.P * 64 * p.NC);
  p.off_stash = o; o += align256(fold_stash_bytes(p));
  p.bytes = o;
  return p;
}

ConvPlan fold_plan(int32_t n_atoms, int64_t n_edges, const eec_model* m) {
  ConvPlan p = conv_plan(n_atoms, n_edges, m);
  // Only the regions of the folded one-kernel path (one to three species):
  // the row-local species grouping and atom order (S > 1), dE/dd per edge,
  // per-atom energies and virial partials, the Gram matrices or the
  // transposed last layer, and the activation stash.  The other offsets are
  // not carved (0) and no launch of that path reads them.
  const int64_t N = std::max(n_atoms, 1), E = std::max<int64_t>(n_edges, 1);
  p.off_recv = p.off_pair_start = p.off_blockcnt = p.off_A = p.off_R = p.off_Y = 0;
  p.off_perm = p.off_seg = p.off_ord = p.off_zstart = 0;
  size_t o = 0;
  if (p.S > 1) {
    p.off_perm = o;   o += align256(4 * (size_t)E);
    p.off_seg = o;    o += align256(8 * (size_t)p.S * N);
    p.off_ord = o;    o += align256(4 * (size_t)N);
    p.off_zstart = o; o += 256;
  }
  p.off_g = o;     o += align256(4 * 3 * (size_t)E);
  p.off_ei = o;    o += align256(4 * (size_t)N);
  p.off_vpart = o; o += align256(8 * 9 * (size_t)N);
  p.off_w3t = o;   o += align256(4 * (size_t)p.P * 64 * p.NC);
  p.off_stash = o; o += align256(fold_stash_bytes(p));
  p.bytes = o;
  return p;
}

void launch_prepare(hipStream_t s, const ConvPlan& p, const eec_graph* g, const int32_t* species,
                    char* ws, float* zero_rows_of) {
  int32_t* recv = (int32_t*)(ws + p.off_recv);
  if (p.N > 0)
    k_recv<<<blocks_for(p.N, 4), 256, 0, s>>>(p.N, g->row_ptr, p.E, recv, zero_rows_of, p.C);
  if (p.S > 1 && p.E > 0) {
    const int64_t nb = p.n_count_blocks;
    // block counts, then their exclusive offsets, in one region
    int32_t* cnt = (int32_t*)(ws + p.off_blockcnt);
    int64_t* off = (int64_t*)(ws + p.off_blockcnt + ((4 * (size_t)p.P * nb + 7) & ~size_t(7)));
    int64_t* pair_start = (int64_t*)(ws + p.off_pair_start);
    int32_t* perm = (int32_t*)(ws + p.off_perm);
    k_pair_count<<<(int)nb, 256, 0, s>>>(p.E, recv, g->col, species, p.S, p.N, nb, cnt);
    k_pair_scan<<<1, 1024, 0, s>>>(nb, p.P, cnt, off, pair_start, p.E);
    k_pair_scatter<<<(int)nb, 256, 0, s>>>(p.E, recv, g->col, species, p.S, p.N, nb, off, perm);
    if (p.N > 0)
      k_seg_bounds<<<blocks_for((int64_t)p.N * p.S, 256), 256, 0, s>>>(p.N, p.S, g->row_ptr, species,
                                                                       pair_start, perm,
                                                                       (int32_t*)(ws + p.off_seg));
  }
}

void launch_prepare_rows(hipStream_t s, const ConvPlan& p, const eec_graph* g, const int32_t* species, char* ws) {
  if (p.S > 4 || p.S < 2 || p.N == 0) return;
  k_row_partition<<<blocks_for(p.N, 4), 256, 0, s>>>(p.N, p.S, p.E, g->row_ptr, g->col, species,
                                                     (int32_t*)(ws + p.off_perm), (int32_t*)(ws + p.off_seg));
  k_species_order<<<1, SO_T, 0, s>>>(p.N, p.S, species, (int32_t*)(ws + p.off_ord), (int32_t*)(ws + p.off_zstart));
}

void launch_message(hipStream_t s, const ConvPlan& p, const eec_graph* g, const int32_t* species,
                    const eec_model* m, int64_t e0, int64_t e1, const float* R_chunk,
                    const float* Y_chunk, float* A, const char* ws) {
  if (e1 <= e0) return;
  const int32_t* recv = (const int32_t*)(ws + p.off_recv);
  const int grid = (int)std::min<int64_t>(p.N, 2048);
  if (p.C == 64)
    k_message<64><<<grid, 256, 0, s>>>(e0, e1, g->row_ptr, recv, R_chunk, Y_chunk, A);
  else
    k_message<128><<<grid, 256, 0, s>>>(e0, e1, g->row_ptr, recv, R_chunk, Y_chunk, A);
}

void launch_readout(hipStream_t s, const ConvPlan& p, const eec_model* m, float* A, int nparts, float* ei) {
  if (p.N == 0) return;
  if (p.C == 64)
    k_readout<64><<<blocks_for(p.N, 4), 256, 0, s>>>(p.N, nparts, m->w_read, A, ei);
  else
    k_readout<128><<<blocks_for(p.N, 4), 256, 0, s>>>(p.N, nparts, m->w_read, A, ei);
}

void launch_scatter(hipStream_t s, const ConvPlan& p, const eec_graph* g, const double* pos, Box box,
                    const float* gin, float* forces, const float* ei, float* energy, float* virial, char* ws) {
  double* vpart = (double*)(ws + p.off_vpart);
  if (p.N == 0) {
    if (virial)
      k_totals<true><<<1, TT, 0, s>>>(0, ei, vpart, energy, virial);
    else
      k_totals<false><<<1, TT, 0, s>>>(0, ei, vpart, energy, virial);
    return;
  }
  const int grid = (blocks_for(p.N, TS / SLPA) + 7) & ~7;  // a multiple of 8 (k_scatter's XCD mapping)
  if (virial) {
    k_scatter<true><<<grid, TS, 0, s>>>(p.N, p.E, g->row_ptr, g->col, g->shift, g->rev, pos, box.L[0], box.L[1],
                                         box.L[2], gin, forces, vpart, ei, nullptr);
    k_totals<true><<<1, TT, 0, s>>>(p.N, ei, vpart, energy, virial);
  } else {
    k_scatter<false><<<grid + 1, TS, 0, s>>>(p.N, p.E, g->row_ptr, g->col, g->shift, g->rev, pos, box.L[0],
                                              box.L[1], box.L[2], gin, forces, vpart, ei, energy);
  }
}

void launch_basis(hipStream_t s, const eec_graph* g, const double* pos, Box box, double cutoff,
                  float* r, float* basis, float* Y) {
  if (g->n_edges == 0 || g->n_atoms == 0) return;
  k_basis<<<blocks_for(2 * g->n_edges, 256), 256, 0, s>>>(g->n_edges, g->n_atoms, g->row_ptr, g->col,
                                                          g->shift, pos, box.L[0], box.L[1],
                                                          box.L[2], cutoff, r, basis, Y);
}

}  // namespace eec

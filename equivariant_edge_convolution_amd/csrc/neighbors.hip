// Cell-list neighbour builder emitting receiver-sorted CSR with reverse edges.
//
// Edge set: every (i, j, n), n in {-1,0,1}^3, with d = (x_j - x_i) + n L in
// binary64 and (dx*dx + dy*dy) + dz*dz < rc*rc, excluding (i, i, 0).  The list
// is rebuilt beside the force call in an MD loop ("FastMACE rewrite screens",
// OPT2-T04 overlap_rebuild); the pages do not fix an order, so rows are sorted
// by (j, nx, ny, nz), which makes the output independent of thread timing.
//
// Pipeline (one host synchronisation, after the row counts):
//   bin atoms into cells of side >= rc  ->  exclusive scan of cell counts  ->
//   place atoms, with their positions, in cell order  ->  one pass over the 27
//   neighbouring (cell, image) candidates of every receiver (a wave each) that
//   writes the row's (j, n) keys into the receiver's key slots and counts the
//   row  ->  scan of the row counts  ->  [sync: E, flags]  ->  (only when a row
//   outgrew its slots: a second pass writing every row's keys at its CSR
//   offsets)  ->  sort each row  ->  reverse index.
#include <math.h>

#include <algorithm>

#include "eec_device.hpp"
#include "eec_internal.hpp"

namespace eec {

namespace {

constexpr int SORT_LDS = 2048;  // keys a row-sort wave stages in LDS

// counters[c] += 1 for every active lane, one atomic per distinct c in the
// wave; returns the lane's slot (the counter's old value plus its rank among
// the lanes with the same c).  Slots within a cell depend on the order the
// waves arrive in; the rows are sorted afterwards, so the output does not.
__device__ __forceinline__ uint32_t wave_count(uint32_t* __restrict__ counters, int c) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (1ull << lane) - 1ull;
  uint64_t pending = __ballot(1);
  uint32_t slot = 0;
  while (pending != 0ull) {
    const int leader = __ffsll((unsigned long long)pending) - 1;
    const int c0 = __shfl(c, leader);
    const uint64_t same = __ballot(c == c0) & pending;
    uint32_t base = 0;
    if (lane == leader) base = atomicAdd(&counters[c0], (uint32_t)__popcll(same));
    base = __shfl(base, leader);
    if ((same >> lane) & 1ull) slot = base + (uint32_t)__popcll(same & below);
    pending &= ~same;
  }
  return slot;
}

// Clears the cell counts and fills and the 16-byte flags / edge-total word.
__global__ void k_nb_clear(uint32_t* __restrict__ cell_count, uint32_t* __restrict__ cell_fill, int64_t nc,
                           uint32_t* __restrict__ flags) {
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (t < 4) flags[t] = 0u;
  for (int64_t k = t; k < nc; k += (int64_t)gridDim.x * blockDim.x) {
    cell_count[k] = 0u;
    cell_fill[k] = 0u;
  }
}

__global__ void k_nb_bin(int32_t n, const double* __restrict__ pos, double Lx, double Ly, double Lz,
                         int nc0, int nc1, int nc2, const int32_t* __restrict__ species,
                         int32_t n_species, int32_t* __restrict__ cell_of,
                         uint32_t* __restrict__ cell_count, uint32_t* __restrict__ flags) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const double x = pos[3 * i], y = pos[3 * i + 1], z = pos[3 * i + 2];
  const bool ok = isfinite(x) && isfinite(y) && isfinite(z) && x >= 0.0 && y >= 0.0 && z >= 0.0 &&
                  x < Lx && y < Ly && z < Lz;
  int c = 0;
  if (!ok) {
    atomicOr(flags, FLAG_OUT_OF_BOX);
  } else {
    const int cx = min((int)(x * ((double)nc0 / Lx)), nc0 - 1);
    const int cy = min((int)(y * ((double)nc1 / Ly)), nc1 - 1);
    const int cz = min((int)(z * ((double)nc2 / Lz)), nc2 - 1);
    c = (cx * nc1 + cy) * nc2 + cz;
  }
  if (species != nullptr) {
    const int32_t zs = species[i];
    if (zs < 0 || zs >= n_species) atomicOr(flags, FLAG_SPECIES);
  }
  cell_of[i] = c;
  wave_count(cell_count, c);
}

// Exclusive scan of n unsigned counts into out[0..n] (out[n] = total) with one
// workgroup of 1024 threads, each a contiguous slice; also stores the total as
// int64 when asked.  A slice of at most SCAN_REG counts (n up to 32 Ki) is
// loaded with all its loads in flight and kept in registers, instead of one
// load waited on per count.
constexpr int SCAN_REG = 32;
__global__ void __launch_bounds__(1024) k_scan_excl(const uint32_t* __restrict__ in, int64_t n,
                                                    int32_t* __restrict__ out,
                                                    int64_t* __restrict__ total) {
  __shared__ int64_t part[1024];
  const int t = threadIdx.x;
  const int64_t per = (n + 1023) / 1024;
  const int64_t a = std::min<int64_t>(n, t * per), b = std::min<int64_t>(n, a + per);
  const bool reg = per <= SCAN_REG;  // uniform over the workgroup
  uint32_t v[SCAN_REG];
  int64_t s = 0;
  const int m = (int)(b - a);  // at most SCAN_REG when reg
  if (reg) {
    const uint32_t* src = in + a;
#pragma unroll
    for (int u = 0; u < SCAN_REG; ++u) v[u] = u < m ? src[u] : 0u;
#pragma unroll
    for (int u = 0; u < SCAN_REG; ++u) s += v[u];
  } else {
    for (int64_t k = a; k < b; ++k) s += in[k];
  }
  part[t] = s;
  __syncthreads();
  // Hillis-Steele inclusive scan over the 1024 thread sums (fixed order).
  for (int off = 1; off < 1024; off <<= 1) {
    int64_t v = (t >= off) ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int64_t run = part[t] - s;
  if (reg) {
    int32_t* dst = out + a;
#pragma unroll
    for (int u = 0; u < SCAN_REG; ++u)
      if (u < m) {
        dst[u] = (int32_t)run;
        run += v[u];
      }
  } else {
    for (int64_t k = a; k < b; ++k) {
      out[k] = (int32_t)run;
      run += in[k];
    }
  }
  if (t == 1023) {
    out[n] = (int32_t)part[1023];
    if (total) *total = part[1023];
  }
}

// Atom i into the next slot of its cell, and its position into the same slot
// of the cell-ordered copy (read contiguously by the candidate scans).
__global__ void k_cell_place(int32_t n, const double* __restrict__ pos, const int32_t* __restrict__ cell_of,
                             const int32_t* __restrict__ cell_start,
                             uint32_t* __restrict__ cell_fill, int32_t* __restrict__ cell_atoms,
                             double* __restrict__ cell_pos) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int c = cell_of[i];
  const uint32_t slot = wave_count(cell_fill, c);
  const int k = cell_start[c] + slot;
  cell_atoms[k] = i;
#pragma unroll
  for (int q = 0; q < 3; ++q) cell_pos[3 * k + q] = pos[3 * i + q];
}

struct Grid {
  int nc0, nc1, nc2;
  double Lx, Ly, Lz, rc2;
};

// Visit every candidate (j, image) of receiver i; lanes stride over the
// members of each of the 27 neighbouring cells.  f(keep, j, s, r2).
template <class F>
__device__ __forceinline__ void for_candidates(int i, const Grid& gr, const double* __restrict__ pos,
                                               const int32_t* __restrict__ cell_of,
                                               const int32_t* __restrict__ cell_start,
                                               const int32_t* __restrict__ cell_atoms,
                                               const double* __restrict__ cell_pos, int nmax, int lane,
                                               F&& f) {
  // i is the wave's receiver: its cell and the candidate cells' ranges are
  // wave-uniform and come through the scalar unit
  i = __builtin_amdgcn_readfirstlane(i);
  const int ci = __builtin_amdgcn_readfirstlane(cell_of[i]);
  const int cz = ci % gr.nc2, cy = (ci / gr.nc2) % gr.nc1, cx = ci / (gr.nc2 * gr.nc1);
  const double xi[3] = {pos[3 * i], pos[3 * i + 1], pos[3 * i + 2]};
  auto cell = [&](int o, int& c2, int& s, int sh[3]) {
    const int vx = cx + o / 9 - 1, vy = cy + (o / 3) % 3 - 1, vz = cz + o % 3 - 1;
    sh[0] = vx < 0 ? -1 : (vx >= gr.nc0 ? 1 : 0);
    sh[1] = vy < 0 ? -1 : (vy >= gr.nc1 ? 1 : 0);
    sh[2] = vz < 0 ? -1 : (vz >= gr.nc2 ? 1 : 0);
    const int wx = vx - sh[0] * gr.nc0, wy = vy - sh[1] * gr.nc1, wz = vz - sh[2] * gr.nc2;
    c2 = (wx * gr.nc1 + wy) * gr.nc2 + wz;
    s = (sh[0] + 1) * 9 + (sh[1] + 1) * 3 + (sh[2] + 1);
  };
  // The first 64 members of three cells at a time, every load issued before
  // the tests; d = (x_j - x_i) + n L in binary64 as edge_vector forms it.
  constexpr int G = 3;
  uint32_t big = 0;  // bit o: candidate cell o holds more than 64 atoms (wave-uniform)
#pragma unroll
  for (int o0 = 0; o0 < 27; o0 += G) {
    int c2[G], s[G], sh[G][3], a[G], b[G], j[G];
    double xj[G][3];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      cell(o0 + u, c2[u], s[u], sh[u]);
      c2[u] = __builtin_amdgcn_readfirstlane(c2[u]);
      a[u] = cell_start[c2[u]];
      b[u] = cell_start[c2[u] + 1];
      big |= (b[u] - a[u] > 64 ? 1u : 0u) << (o0 + u);
    }
    // loads from a valid slot in every lane (no load under a branch); lanes
    // past the cell's end are masked out below
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int k = min(a[u] + lane < b[u] ? a[u] + lane : a[u], nmax);
      j[u] = cell_atoms[k];
#pragma unroll
      for (int q = 0; q < 3; ++q) xj[u][q] = cell_pos[3 * k + q];
    }
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const bool in_cell = a[u] + lane < b[u];
      if (!in_cell) j[u] = i;
      const double L[3] = {gr.Lx, gr.Ly, gr.Lz};
      double d[3];
      {
#pragma clang fp contract(off)
        for (int q = 0; q < 3; ++q) d[q] = (xj[u][q] - xi[q]) + (double)(int8_t)sh[u][q] * L[q];
      }
      const double r2 = norm2_nofma(d);
      const bool keep = in_cell && (r2 < gr.rc2) && !(j[u] == i && s[u] == 13);
      f(keep, j[u], s[u], in_cell ? r2 : 1.0);
    }
  }
  // members past the first 64 of the cells that have them
  for (uint32_t m = big; m != 0; m &= m - 1) {
    const int o = __builtin_ctz(m);
    int c2, s, shv[3];
    cell(o, c2, s, shv);
    const int ix = shv[0], iy = shv[1], iz = shv[2];
    const int a = cell_start[c2], b = cell_start[c2 + 1];
    for (int base = a + 64; base < b; base += 64) {
      const int k = base + lane;
      bool keep = false;
      int j = 0;
      double r2 = 1.0;
      if (k < b) {
        j = cell_atoms[k];
        const double L[3] = {gr.Lx, gr.Ly, gr.Lz}, shd[3] = {(double)ix, (double)iy, (double)iz};
        double d[3];
        {
#pragma clang fp contract(off)
          for (int q = 0; q < 3; ++q) d[q] = (cell_pos[3 * k + q] - xi[q]) + shd[q] * L[q];
        }
        r2 = norm2_nofma(d);
        keep = (r2 < gr.rc2) && !(j == i && s == 13);
      }
      f(keep, j, s, r2);
    }
  }
}

// Writes the unsorted (j * 27 + s) keys of each row.  SLOTS (the first pass,
// before any row offsets exist): row i's keys go to its NB_SLOT_CAP slots at
// keys + i * NB_SLOT_CAP and its degree to deg[i]; a row longer than its slots
// (the keys past them dropped, the degree whole) raises FLAG_SLOT_OVERFLOW,
// and the host then runs the second form, which writes every row's keys at
// its CSR positions keys + rp[i].
template <bool SLOTS>
__global__ void __launch_bounds__(256) k_nb_fill(int32_t n, Grid gr, const double* __restrict__ pos,
                                                 const int32_t* __restrict__ cell_of,
                                                 const int32_t* __restrict__ cell_start,
                                                 const int32_t* __restrict__ cell_atoms,
                                                 const double* __restrict__ cell_pos,
                                                 const int32_t* __restrict__ rp,
                                                 int32_t* __restrict__ keys, uint32_t* __restrict__ deg,
                                                 uint32_t* __restrict__ flags) {
  const int i = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (i >= n) return;
  const int64_t base0 = SLOTS ? (int64_t)i * NB_SLOT_CAP : (int64_t)rp[i];
  const int64_t end = SLOTS ? base0 + NB_SLOT_CAP : (int64_t)rp[i + 1];
  int64_t base = base0;
  bool coincident = false;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for_candidates(i, gr, pos, cell_of, cell_start, cell_atoms, cell_pos, n - 1, lane,
                 [&](bool keep, int j, int s, double r2) {
                   const uint64_t mask = __ballot(keep);
                   const int64_t at = base + __popcll(mask & below);
                   if (keep && at < end) keys[at] = j * 27 + s;
                   base += __popcll(mask);
                   if (SLOTS) coincident |= keep && (r2 == 0.0);
                 });
  if (SLOTS) {
    const int64_t cnt = base - base0;
    if (coincident) atomicOr(flags, FLAG_GEOMETRY);
    if (lane == 0) {
      deg[i] = (uint32_t)cnt;
      if (cnt > NB_SLOT_CAP) atomicOr(flags, FLAG_SLOT_OVERFLOW);
    }
  }
}

// One 64-thread workgroup per row: rank-sort the row's distinct keys and
// write the sorted senders and image shifts.
// With `slots`, row i's keys are read from slots + i * NB_SLOT_CAP (every row
// then has at most NB_SLOT_CAP keys) and written back there sorted, for the
// reverse search; else they are read from keys + rp[i].
__global__ void __launch_bounds__(64) k_nb_sort(int32_t n, const int32_t* __restrict__ rp,
                                                const int32_t* __restrict__ keys_csr,
                                                int32_t* __restrict__ slots,
                                                int32_t* __restrict__ col, int8_t* __restrict__ shift) {
  __shared__ int32_t sk[SORT_LDS];
  const int i = blockIdx.x;
  const int lane = threadIdx.x;
  if (i >= n) return;
  const int a = rp[i], deg = rp[i + 1] - a;
  const int32_t* row = slots != nullptr ? slots + (int64_t)i * NB_SLOT_CAP : keys_csr + a;  // the row's keys
  auto emit = [&](int r, int32_t key) {
    const int s = key % 27;
    col[a + r] = key / 27;
    shift[3 * (a + r) + 0] = (int8_t)(s / 9 - 1);
    shift[3 * (a + r) + 1] = (int8_t)((s / 3) % 3 - 1);
    shift[3 * (a + r) + 2] = (int8_t)(s % 3 - 1);
  };
  if (deg <= 256) {
    // bitonic sort of up to 256 keys in registers, key x = 4 lane + r: pairs
    // 4 or more apart across lanes (shuffles), closer pairs within a lane
    int32_t v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = 4 * lane + r < deg ? row[4 * lane + r] : INT32_MAX;
    for (int k = 2; k <= 256; k <<= 1) {
      for (int jj = k >> 1; jj > 0; jj >>= 1) {
        if (jj >= 4) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int x = 4 * lane + r;
            const int32_t o = __shfl_xor(v[r], jj >> 2);
            const bool lower = (x & jj) == 0, up = (x & k) == 0;
            v[r] = (lower == up) ? min(v[r], o) : max(v[r], o);
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if ((r & jj) != 0) continue;
            const int r2 = r | jj;
            const bool up = ((4 * lane + r) & k) == 0;
            if ((v[r] > v[r2]) == up) {
              const int32_t t = v[r];
              v[r] = v[r2];
              v[r2] = t;
            }
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * lane + r < deg) emit(4 * lane + r, v[r]);
    if (slots != nullptr) {  // every lane's keys were read before the sort: no other lane reads these
      int32_t* out = slots + (int64_t)i * NB_SLOT_CAP;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * lane + r < deg) out[4 * lane + r] = v[r];
    }
  } else if (deg <= SORT_LDS) {
    // bitonic sort of the keys padded to a power of two (the pads sort last)
    int np2 = 64;
    while (np2 < deg) np2 <<= 1;
    for (int k = lane; k < np2; k += 64) sk[k] = k < deg ? row[k] : INT32_MAX;
    __syncthreads();
    for (int k = 2; k <= np2; k <<= 1) {
      for (int jj = k >> 1; jj > 0; jj >>= 1) {
        for (int x = lane; x < np2; x += 64) {
          const int y = x ^ jj;
          if (y > x) {
            const int32_t kx = sk[x], ky = sk[y];
            const bool up = (x & k) == 0;
            if ((kx > ky) == up) {
              sk[x] = ky;
              sk[y] = kx;
            }
          }
        }
        __syncthreads();
      }
    }
    for (int k = lane; k < deg; k += 64) emit(k, sk[k]);
  } else {
    const int32_t* src = row;
    for (int k = lane; k < deg; k += 64) {
      const int32_t key = src[k];
      int rank = 0;
      for (int q = 0; q < deg; ++q) rank += (src[q] < key) ? 1 : 0;
      emit(rank, key);
    }
  }
}

__device__ __forceinline__ int32_t key_at(const int32_t* __restrict__ col,
                                          const int8_t* __restrict__ shift, int e) {
  return col[e] * 27 + (shift[3 * e] + 1) * 9 + (shift[3 * e + 1] + 1) * 3 + (shift[3 * e + 2] + 1);
}

// One wave per row: rev(e) = index of (j, i, -n) found by binary search in row j.
__global__ void __launch_bounds__(256) k_nb_rev(int32_t n, const int32_t* __restrict__ rp,
                                                const int32_t* __restrict__ col,
                                                const int8_t* __restrict__ shift,
                                                int32_t* __restrict__ rev) {
  const int i = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (i >= n) return;
  for (int e = rp[i] + lane; e < rp[i + 1]; e += 64) {
    const int j = col[e];
    const int s = (shift[3 * e] + 1) * 9 + (shift[3 * e + 1] + 1) * 3 + (shift[3 * e + 2] + 1);
    const int32_t target = i * 27 + (26 - s);
    // first entry of row j with sender i (rows are sorted by sender, then
    // image), then the image among those
    const int end = rp[j + 1];
    int lo = rp[j], hi = end;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (col[mid] < i) lo = mid + 1; else hi = mid;
    }
    while (lo < end && col[lo] == i && key_at(col, shift, lo) < target) ++lo;
    // The reverse edge always exists: d of (j, i, -n) is -d bit for bit and
    // the binary64 cutoff test squares each component, so both directions get
    // the same decision, and the candidate enumeration is symmetric.  The
    // fallback only keeps rev in bounds.
    rev[e] = (lo < end && key_at(col, shift, lo) == target) ? lo : e;
  }
}

// The same from the sorted keys every row left in its slots (rows of at most
// NB_SLOT_CAP = 256 edges): rev(e) = rp[j] + the position of key (i, -n) in
// row j, by a lower-bound search of row j's sorted keys (one load per probe).
// A lane's four edges (256 keys / 64 lanes) are searched together, so their
// probes are in flight at once.
__global__ void __launch_bounds__(256) k_nb_rev_slots(int32_t n, const int32_t* __restrict__ rp,
                                                      const int32_t* __restrict__ slots,
                                                      int32_t* __restrict__ rev) {
  constexpr int U = NB_SLOT_CAP / 64;
  const int i = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (i >= n) return;
  const int a = rp[i], deg = rp[i + 1] - a;
  const int32_t* own = slots + (int64_t)i * NB_SLOT_CAP;
  int32_t target[U];
  int base[U], len[U], start[U];
  const int32_t* rowj[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int k = lane + 64 * u;
    const int32_t key = k < deg ? own[k] : 0;
    const int j = min(max(key / 27, 0), n - 1);
    target[u] = i * 27 + (26 - key % 27);
    rowj[u] = slots + (int64_t)j * NB_SLOT_CAP;
    start[u] = k < deg ? rp[j] : 0;
    len[u] = k < deg ? rp[j + 1] - start[u] : 0;
    base[u] = 0;
  }
  // lower bound of target in rowj[0 .. len): at most 9 halvings for 256 keys
  for (int it = 0; it < 9; ++it) {
    int32_t probe[U];
#pragma unroll
    for (int u = 0; u < U; ++u) probe[u] = len[u] > 0 ? rowj[u][base[u] + (len[u] >> 1)] : 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (len[u] <= 0) continue;
      const int half = len[u] >> 1;
      if (probe[u] < target[u]) {
        base[u] += half + 1;
        len[u] -= half + 1;
      } else {
        len[u] = half;
      }
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int k = lane + 64 * u;
    if (k >= deg) continue;
    const int cnt = rp[min(max(own[k] / 27, 0), n - 1) + 1] - start[u];
    // the reverse edge always exists (see k_nb_rev); the fallback keeps rev in bounds
    rev[a + k] = (base[u] < cnt && rowj[u][base[u]] == target[u]) ? start[u] + base[u] : a + k;
  }
}

__global__ void k_copy_i32(const int32_t* __restrict__ src, int32_t* __restrict__ dst, int64_t n) {
  for (int64_t k = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; k < n;
       k += (int64_t)gridDim.x * blockDim.x)
    dst[k] = src[k];
}

inline int blocks_for(int64_t n, int per) { return (int)std::max<int64_t>(1, (n + per - 1) / per); }

// ---------------------------------------------------------------- skin test
// Largest squared displacement of any atom from the positions its list was
// built from, d = x_i - ref_i in binary64 and (dx*dx + dy*dy) + dz*dz with no
// fused multiply-add, and whether it exceeds half_skin^2.  Non-negative
// binary64 values order like their bit patterns, so the integer maximum of the
// per-block results is the same word in whatever order the blocks finish.
constexpr int SKIN_T = 256;
constexpr int SKIN_MAX_BLOCKS = 1024;

__global__ void k_skin_clear(unsigned long long* __restrict__ max_r2, int32_t* __restrict__ rebuild) {
  if (threadIdx.x == 0) {
    *max_r2 = 0ull;
    *rebuild = 0;
  }
}

__global__ void __launch_bounds__(SKIN_T) k_skin(int32_t n, const double* __restrict__ pos,
                                                 const double* __restrict__ ref, double hs2,
                                                 unsigned long long* __restrict__ max_r2,
                                                 int32_t* __restrict__ rebuild) {
  __shared__ double part[SKIN_T / 64];
  double m = 0.0;
  for (int64_t i = blockIdx.x * (int64_t)SKIN_T + threadIdx.x; i < n; i += (int64_t)gridDim.x * SKIN_T) {
    double d[3];
    {
#pragma clang fp contract(off)
      d[0] = pos[3 * i + 0] - ref[3 * i + 0];
      d[1] = pos[3 * i + 1] - ref[3 * i + 1];
      d[2] = pos[3 * i + 2] - ref[3 * i + 2];
    }
    const double r2 = norm2_nofma(d);
    // a NaN displacement (non-finite input) counts as the largest
    m = (r2 > m || r2 != r2) ? r2 : m;
  }
  for (int o = 32; o > 0; o >>= 1) {
    const double v = __shfl_xor(m, o);
    m = (v > m || v != v) ? v : m;
  }
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < SKIN_T / 64; ++w) m = (part[w] > m || part[w] != part[w]) ? part[w] : m;
    if (m != m) m = __longlong_as_double(0x7ff0000000000000ll);  // NaN -> +inf
    atomicMax(max_r2, (unsigned long long)__double_as_longlong(m));
    if (m > hs2) atomicMax(rebuild, 1);
  }
}

}  // namespace

NbPlan nb_plan(int32_t n_atoms, const double* box, double cutoff) {
  NbPlan p{};
  int64_t nc[3];
  for (int k = 0; k < 3; ++k) {
    double q = floor(box[k] / (cutoff * (1.0 + 1e-9)));
    nc[k] = (q >= 1.0 && q < 1e6) ? (int64_t)q : 1;
  }
  // Keep the grid proportional to the atom count; a coarser grid stays exact.
  const int64_t cap = 2 * (int64_t)std::max(n_atoms, 1) + 64;
  while (nc[0] * nc[1] * nc[2] > cap) {
    int k = (nc[0] >= nc[1] && nc[0] >= nc[2]) ? 0 : (nc[1] >= nc[2] ? 1 : 2);
    nc[k] = std::max<int64_t>(1, nc[k] - 1);
  }
  for (int k = 0; k < 3; ++k) p.nc[k] = (int32_t)nc[k];
  p.n_cells = nc[0] * nc[1] * nc[2];
  const int64_t N = std::max(n_atoms, 0);
  size_t o = 0;
  p.off_cell_count = o; o += align256(sizeof(uint32_t) * p.n_cells);
  p.off_cell_fill = o;  o += align256(sizeof(uint32_t) * p.n_cells);
  p.off_cell_start = o; o += align256(sizeof(int32_t) * (p.n_cells + 1));
  p.off_cell_atoms = o; o += align256(sizeof(int32_t) * std::max<int64_t>(N, 1));
  p.off_cell_of = o;    o += align256(sizeof(int32_t) * std::max<int64_t>(N, 1));
  p.off_cell_pos = o;   o += align256(3 * sizeof(double) * std::max<int64_t>(N, 1));
  p.off_deg = o;        o += align256(sizeof(uint32_t) * (N + 1) + sizeof(int32_t) * (N + 1));
  p.off_scratch = o;    o += 256;
  p.off_slots = o;      o += align256(sizeof(int32_t) * NB_SLOT_CAP * std::max<int64_t>(N, 1));
  p.bytes = o;
  return p;
}

eec_status nb_build(hipStream_t s, const NbPlan& p, int32_t n, const double* pos, const double* box,
                    double cutoff, const int32_t* species, int32_t n_species, int64_t cap,
                    int32_t* row_ptr, int32_t* col, int8_t* shift, int32_t* rev, int64_t* n_edges,
                    char* ws, const char** why) {
  uint32_t* cell_count = (uint32_t*)(ws + p.off_cell_count);
  uint32_t* cell_fill = (uint32_t*)(ws + p.off_cell_fill);
  int32_t* cell_start = (int32_t*)(ws + p.off_cell_start);
  int32_t* cell_atoms = (int32_t*)(ws + p.off_cell_atoms);
  double* cell_pos = (double*)(ws + p.off_cell_pos);
  int32_t* cell_of = (int32_t*)(ws + p.off_cell_of);
  uint32_t* deg = (uint32_t*)(ws + p.off_deg);
  int32_t* rp_tmp = (int32_t*)(ws + p.off_deg + sizeof(uint32_t) * (n + 1));
  uint32_t* flags = (uint32_t*)(ws + p.off_scratch);
  int64_t* total = (int64_t*)(ws + p.off_scratch + 8);

  const int64_t nc = p.n_cells;
  k_nb_clear<<<(int)std::max<int64_t>(1, std::min<int64_t>(blocks_for(nc, 256), 1024)), 256, 0, s>>>(
      cell_count, cell_fill, nc, flags);
  if (n > 0) {
    k_nb_bin<<<blocks_for(n, 256), 256, 0, s>>>(n, pos, box[0], box[1], box[2], p.nc[0], p.nc[1],
                                                 p.nc[2], species, n_species, cell_of, cell_count,
                                                 flags);
  }
  k_scan_excl<<<1, 1024, 0, s>>>(cell_count, nc, cell_start, nullptr);
  Grid gr{p.nc[0], p.nc[1], p.nc[2], box[0], box[1], box[2], cutoff * cutoff};
  // One pass over the candidates into per-atom key slots that also counts the
  // rows; only when a row outgrows its slots does a second pass fill the keys
  // at the CSR positions.
  int32_t* slots = (int32_t*)(ws + p.off_slots);
  if (n > 0) {
    k_cell_place<<<blocks_for(n, 256), 256, 0, s>>>(n, pos, cell_of, cell_start, cell_fill, cell_atoms, cell_pos);
    k_nb_fill<true><<<blocks_for(n, 4), 256, 0, s>>>(n, gr, pos, cell_of, cell_start, cell_atoms, cell_pos,
                                                      nullptr, slots, deg, flags);
  }
  k_scan_excl<<<1, 1024, 0, s>>>(deg, n, rp_tmp, total);
  // The flags and the edge total come back through a 16-byte pinned host word
  // kept per host thread (a copy into pageable memory is staged, and cost as
  // much as the kernels on small cells); allocated on the thread's first build
  // and kept until the process ends (freeing it at thread exit could run after
  // the HIP runtime has shut down).
  struct Readback {
    uint32_t flags;
    uint32_t pad;
    int64_t total;
  };
  static_assert(sizeof(Readback) == 16, "flags word, pad and edge total");
  thread_local Readback* pinned = nullptr;
  if (pinned == nullptr &&
      hipHostMalloc((void**)&pinned, sizeof(Readback), hipHostMallocPortable) != hipSuccess) {
    pinned = nullptr;
    *why = "HIP error while allocating the edge-count readback word";
    return EEC_ERR_HIP;
  }
  if (hipMemcpyAsync(pinned, flags, sizeof(Readback), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess) {
    *why = "HIP error while reading the edge count";
    return EEC_ERR_HIP;
  }
  const Readback host = *pinned;
  if (host.flags & FLAG_OUT_OF_BOX) { *why = "a position is non-finite or outside [0, L)"; return EEC_ERR_OUT_OF_BOX; }
  if (host.flags & FLAG_SPECIES) { *why = "a species index is outside [0, n_species)"; return EEC_ERR_SPECIES; }
  if (host.flags & FLAG_GEOMETRY) { *why = "two atoms (or periodic images) coincide"; return EEC_ERR_GEOMETRY; }
  *n_edges = host.total;
  if (host.total > cap) { *why = "edge_capacity is smaller than the edge count"; return EEC_ERR_CAPACITY; }
  if (host.total > INT32_MAX) { *why = "edge count exceeds int32 indexing"; return EEC_ERR_SHAPE; }

  k_copy_i32<<<blocks_for(n + 1, 256), 256, 0, s>>>(rp_tmp, row_ptr, n + 1);
  if (n > 0 && host.total > 0) {
    if (host.flags & FLAG_SLOT_OVERFLOW) {
      k_nb_fill<false><<<blocks_for(n, 4), 256, 0, s>>>(n, gr, pos, cell_of, cell_start, cell_atoms, cell_pos,
                                                         row_ptr, rev /* keys staged here */, nullptr, nullptr);
      k_nb_sort<<<n, 64, 0, s>>>(n, row_ptr, rev, nullptr, col, shift);
      k_nb_rev<<<blocks_for(n, 4), 256, 0, s>>>(n, row_ptr, col, shift, rev);
    } else {
      k_nb_sort<<<n, 64, 0, s>>>(n, row_ptr, nullptr, slots, col, shift);
      k_nb_rev_slots<<<blocks_for(n, 4), 256, 0, s>>>(n, row_ptr, slots, rev);
    }
  }
  if (hipGetLastError() != hipSuccess) { *why = "kernel launch failed"; return EEC_ERR_HIP; }
  return EEC_OK;
}

void launch_skin_check(hipStream_t s, int32_t n, const double* pos, const double* ref, double half_skin,
                       double* max_r2, int32_t* rebuild) {
  auto* m2 = reinterpret_cast<unsigned long long*>(max_r2);
  k_skin_clear<<<1, 64, 0, s>>>(m2, rebuild);
  if (n > 0) {
    const int blocks = (int)std::min<int64_t>(SKIN_MAX_BLOCKS, ((int64_t)n + SKIN_T - 1) / SKIN_T);
    k_skin<<<blocks, SKIN_T, 0, s>>>(n, pos, ref, half_skin * half_skin, m2, rebuild);
  }
}

}  // namespace eec

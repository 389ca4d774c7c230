// Internal host-side interfaces between the C-ABI layer and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/eec.h"

namespace eec {

// Error bits raised on the device by the neighbour builder.
enum : uint32_t {
  FLAG_OUT_OF_BOX = 1u,
  FLAG_SPECIES = 2u,
  FLAG_GEOMETRY = 4u,
  FLAG_SLOT_OVERFLOW = 8u,  // a row longer than NB_SLOT_CAP (builder-internal)
};

struct Box {
  double L[3];
};

// ---- neighbour list
struct NbPlan {
  int32_t nc[3];
  int64_t n_cells;
  size_t bytes;
  // byte offsets into the workspace
  size_t off_cell_count, off_cell_fill, off_cell_start, off_cell_atoms, off_cell_of, off_cell_pos, off_deg,
      off_scratch, off_slots;
};
// Key slots per atom of the builder's counting fill (N * NB_SLOT_CAP * 4 bytes of workspace).
constexpr int NB_SLOT_CAP = 256;
NbPlan nb_plan(int32_t n_atoms, const double* box, double cutoff);

// Runs the whole builder; returns EEC_OK / error.  Writes *n_edges.
eec_status nb_build(hipStream_t s, const NbPlan& p, int32_t n_atoms, const double* pos,
                    const double* box, double cutoff, const int32_t* species, int32_t n_species,
                    int64_t cap, int32_t* row_ptr, int32_t* col, int8_t* shift, int32_t* rev,
                    int64_t* n_edges, char* ws, const char** why);

// Skin test: *max_r2 = largest squared displacement pos - ref over the atoms,
// *rebuild = (*max_r2 > half_skin^2); both written on the stream, no sync.
void launch_skin_check(hipStream_t s, int32_t n, const double* pos, const double* ref, double half_skin,
                       double* max_r2, int32_t* rebuild);

// ---- edge-convolution workspace plan
struct ConvPlan {
  int C, NC, S, P;
  int64_t E;
  int32_t N;
  int64_t chunk;  // edges per streamed chunk
  size_t bytes;
  size_t off_recv, off_perm, off_pair_start, off_blockcnt, off_seg, off_A, off_R, off_Y, off_g,
      off_vpart, off_ei, off_w3t, off_stash, off_ord, off_zstart;
  int64_t n_count_blocks;
};
ConvPlan conv_plan(int32_t n_atoms, int64_t n_edges, const eec_model* m);
// The smaller layout of the folded one-kernel path (one to three species):
// only the regions that path reads and writes.
ConvPlan fold_plan(int32_t n_atoms, int64_t n_edges, const eec_model* m);

// Graph preparation: receiver of each edge; pair-grouped edge order when S > 1.
void launch_prepare(hipStream_t s, const ConvPlan& p, const eec_graph* g, const int32_t* species,
                    char* ws, float* zero_rows_of /* [N][16][C] or NULL */);

// For 2 <= S <= 4: row-local grouping of the edges by sender species (perm and
// seg in the layout launch_prepare uses, positions being CSR positions), and
// the atoms in species order (stable) with the species' offsets.
void launch_prepare_rows(hipStream_t s, const ConvPlan& p, const eec_graph* g, const int32_t* species, char* ws);

// Radial network over a range of edges.  When `basis_in` is given the basis is
// read from it (materialising entry point); otherwise it is computed from the
// geometry.  Writes R rows (relative to e_begin) and, if Y_out, harmonics rows.
void launch_radial(hipStream_t s, const ConvPlan& p, const eec_graph* g, const double* pos,
                   Box box, double cutoff, const int32_t* species, const eec_model* m,
                   const float* basis_in, int64_t e_begin, int64_t e_end, float* R_out,
                   float* Y_out, const char* ws);

// Streaming message of one chunk [e_begin, e_end) into A (assign or accumulate per row).
void launch_message(hipStream_t s, const ConvPlan& p, const eec_graph* g, const int32_t* species,
                    const eec_model* m, int64_t e_begin, int64_t e_end, const float* R_chunk,
                    const float* Y_chunk, float* A, const char* ws);

// Readout: A_i = sum of `nparts` partial slabs [nparts][N][16][C] (fixed order),
// E_i (into ei) and dE/dA = 2 w A written over slab 0.
void launch_readout(hipStream_t s, const ConvPlan& p, const eec_model* m, float* A, int nparts, float* ei);

// Fused forward (C = 64): radial network + message per (pair, receiver) unit,
// writing the S partial A slabs.  The chunked path (launch_radial +
// launch_message) covers every supported shape.
bool fused_forward_supported(const ConvPlan& p);
void launch_forward(hipStream_t s, const ConvPlan& p, const eec_graph* g, const double* pos, Box box,
                    double cutoff, const int32_t* species, const eec_model* m, float* A_out,
                    const char* ws);

// Backward over all edges: g = dE/dd.
void launch_backward(hipStream_t s, const ConvPlan& p, const eec_graph* g, const double* pos,
                     Box box, double cutoff, const int32_t* species, const eec_model* m,
                     const float* Abar, float* gout, const char* ws);

// Force scatter (and optional virial), the energy total from ei (and the
// virial total).
void launch_scatter(hipStream_t s, const ConvPlan& p, const eec_graph* g, const double* pos, Box box,
                    const float* gin, float* forces, const float* ei, float* energy, float* virial, char* ws);

// Materialised basis / harmonics.
void launch_basis(hipStream_t s, const eec_graph* g, const double* pos, Box box, double cutoff,
                  float* r, float* basis, float* Y);

// Reassociated last layer (the fold): forward per unit into the S partial A
// slabs; backward (reads the transposed last-layer weights launch_transpose_w3
// wrote).
void launch_fold_forward(hipStream_t s, const ConvPlan& p, const eec_graph* g, const double* pos,
                         Box box, double cutoff, const int32_t* species, const eec_model* m,
                         float* A_out, char* ws);
void launch_fold_backward(hipStream_t s, const ConvPlan& p, const eec_graph* g, const double* pos,
                          Box box, double cutoff, const int32_t* species, const eec_model* m,
                          const float* Abar, float* gout, char* ws);

// Bytes of the per-wave activation stash of the one-species fused kernel
// (bounded by its grid, not by the edge count; 0 for several species).
size_t fold_stash_bytes(const ConvPlan& p);

// W3T[p][j][k] = W3[p][k][j] into the workspace (read by the folded backward).
void launch_transpose_w3(hipStream_t s, const ConvPlan& p, const eec_model* m, char* ws);

// One species: the whole folded call per receiver in one kernel (forward tiles,
// T_i, E_i into ei and M_i through the Gram matrices of the quadratic readout,
// backward tiles into gout).  launch_gram writes those matrices (64 KB, in the
// transposed-weights slot of the workspace) first on the stream.
bool fold_fused_supported(const ConvPlan& p);
void launch_gram(hipStream_t s, const ConvPlan& p, const eec_model* m, char* ws);
void launch_fold_fused(hipStream_t s, const ConvPlan& p, const eec_graph* g, const double* pos, Box box,
                       double cutoff, const int32_t* species, const eec_model* m, float* ei, float* gout,
                       char* ws);

// Two or three species: the whole folded call per receiver in one kernel,
// sender species after sender species (needs launch_prepare_rows and
// launch_transpose_w3 first on the stream).  With `tab` (a radial table set of
// 2^log2_pieces coarse pieces, levels `level`), s2 and ds2/dr come from it.
bool fold_multi_supported(const ConvPlan& p);
void launch_fold_multi(hipStream_t s, const ConvPlan& p, const eec_graph* g, const double* pos, Box box,
                       double cutoff, const int32_t* species, const eec_model* m, float* ei, float* gout,
                       char* ws, int log2_pieces = 0, const float* tab = nullptr,
                       const int32_t* level = nullptr);

// Radial tables (one species pair after another): polynomials of degree
// TAB_DEG on the 2^d(c) sub-pieces of each of 2^log2_pieces coarse pieces of
// [0, rc]; coefficients [pair][c][f < TAB_SUB][m = 0..TAB_DEG][unit j % 32][j / 32]
// float32 (slots f >= 2^d(c) unused), levels d [pair][c] int32.
constexpr int TAB_DEG = 10;
constexpr int TAB_NC = TAB_DEG + 1;
constexpr int TAB_DMAX = 4, TAB_SUB = 1 << TAB_DMAX;
constexpr double TAB_TOL = 1e-8;  // binary64 interpolation error that fixes a piece's level
constexpr int TAB_MIN_LOG2 = 2, TAB_MAX_LOG2 = 10;
size_t table_floats(int n_species, int log2_pieces);
size_t table_levels(int n_species, int log2_pieces);
// Builds every pair's table; cert (device, 2 doubles, or NULL) receives the
// largest value and r-derivative errors of the float32 table against binary64,
// relative to the local scale.
void launch_table_build(hipStream_t s, const eec_model* m, int log2_pieces, float* tab, int32_t* level,
                        double* cert);
// One species: the folded call per receiver in one kernel with s2 and ds2/dr
// from the table (needs launch_gram first on the stream, as launch_fold_fused).
void launch_fold_table(hipStream_t s, const ConvPlan& p, const eec_graph* g, const double* pos, Box box,
                       double cutoff, const eec_model* m, int log2_pieces, const float* tab,
                       const int32_t* level, float* ei, float* gout, char* ws);

constexpr size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace eec

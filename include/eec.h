/*
 * eec.h -- C ABI of the MI355X (gfx950) equivariant edge convolution.
 *
 * One hot path of a machine-learned interatomic potential: for every directed
 * edge (i, j, n) inside the cutoff, a radial basis with a polynomial envelope,
 * a dense radial network giving per-degree, per-channel weights R_{l,c}(r), real
 * spherical harmonics Y_lm(u) for l <= 3, the message R Y h_j reduced into the
 * receiving atom, a quadratic invariant energy readout, and the chain-rule
 * backward to the edge vectors, which gives forces.
 *
 * Where the pages state the problem:
 *   - radial basis (E,4,32) feeding a per-degree projection to (E,256):
 *     "deepmd-kit PR #6108", What;
 *   - lmax 3, FP32, and the input-gradient (force) backward over edge cohorts:
 *     "deepmd-kit PR #2", Summary and Implementation and scope;
 *   - positions, species and cell in; energy, forces (and virial) out, through
 *     the normal energy/force/virial call: "deepmd-kit PR #2", Primary capacity;
 *   - deterministic per-atom sums, no float atomics: "FastMACE rewrite screens",
 *     OPT-T02 stage D and OPT4-T02 polar_graph_sums;
 *   - callers' inputs are never overwritten and inputs never alias outputs:
 *     "deepmd-kit PR #2", Implementation and scope.
 *
 * Conventions (all entry points)
 *   - Arrays are row-major and contiguous.  Pointers are DEVICE pointers unless
 *     marked [host].
 *   - The caller owns every buffer.  The library never allocates device memory
 *     (eec_build_neighbors keeps one 16-byte pinned host word per thread),
 *     never writes an input, and rejects output ranges that overlap an input or
 *     another output (EEC_ERR_ALIAS).  Scratch comes from the caller's
 *     `workspace` (device, 256-byte aligned), sized by the *_workspace_bytes
 *     queries.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *     Only eec_build_neighbors synchronises that stream (once).  All other calls
 *     return as soon as their kernels are enqueued.
 *   - The box is orthorhombic and periodic in all three axes with every side
 *     L_k >= cutoff, so image shifts are in {-1, 0, 1}^3.
 *   - Indices are int32 (E <= 2^31 - 1); flattened sizes use int64/size_t.
 *   - Errors: a non-zero eec_status; eec_last_error() returns a thread-local
 *     message for the last failing call on this thread.  On error no output is
 *     written, except where a status says otherwise.
 *   - Calls are reentrant given distinct workspaces; there is no global state
 *     beyond the thread-local error text.
 *   - Results are bitwise reproducible run to run for the same inputs (fixed
 *     summation orders, no float atomics).
 *
 * Model shape supported: n_basis = 32, hidden = 64, lmax = 3,
 * channels C in {64, 128}, 1 <= n_species <= 4.
 */
#ifndef EEC_H
#define EEC_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define EEC_API __attribute__((visibility("default")))
#else
#define EEC_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  EEC_OK = 0,
  EEC_ERR_NULL = 1,        /* a required pointer is NULL                          */
  EEC_ERR_SHAPE = 2,       /* unsupported size or model shape, or bad graph size  */
  EEC_ERR_BOX = 3,         /* a box side <= 0, non-finite, or < cutoff            */
  EEC_ERR_OUT_OF_BOX = 4,  /* a coordinate outside [0, L_k) or non-finite         */
  EEC_ERR_SPECIES = 5,     /* a species index outside [0, n_species)              */
  EEC_ERR_CAPACITY = 6,    /* edge_capacity too small; *n_edges holds the need    */
  EEC_ERR_ALIAS = 7,       /* an output overlaps an input or another output       */
  EEC_ERR_WORKSPACE = 8,   /* workspace NULL, misaligned or smaller than required */
  EEC_ERR_GEOMETRY = 9,    /* two atoms (or images) at distance zero              */
  EEC_ERR_HIP = 10         /* a HIP runtime call failed                           */
} eec_status;

/* Model weights (device, float32), prepared once by the caller and never
 * mutated by the library ("deepmd-kit PR #6108", What: weights frozen at
 * inference).  Pair index p = Z_receiver * n_species + Z_sender.
 *   W1     [S*S][n_basis][hidden]          z1 = b W1
 *   W2     [S*S][hidden][hidden]           z2 = silu(z1) W2
 *   W3     [S*S][hidden][(lmax+1)*C]       R  = silu(z2) W3, column l*C + c
 *   emb    [S][C]                          h_{Z_j, c}
 *   w_read [C]                             E_i = sum_c w_c sum_lm A_{i,lm,c}^2   */
typedef struct {
  int32_t n_species;
  int32_t channels;
  int32_t n_basis;
  int32_t hidden;
  int32_t lmax;
  double cutoff;
  const float *W1;
  const float *W2;
  const float *W3;
  const float *emb;
  const float *w_read;
} eec_model;

/* Receiver-sorted CSR edge list, as produced by eec_build_neighbors (device).
 *   row_ptr [n_atoms + 1]; edges of receiver i are [row_ptr[i], row_ptr[i+1])
 *   col     [n_edges]      sender j
 *   shift   [n_edges][3]   image n in {-1,0,1}^3: d = (x_j - x_i) + n * L
 *   rev     [n_edges]      index of the reverse edge (j, i, -n)
 * The compute entry points trust these invariants (they hold for any output
 * of eec_build_neighbors); they clamp indices so that a malformed graph cannot
 * read outside its arrays, but the results are then meaningless. */
typedef struct {
  int32_t n_atoms;
  int64_t n_edges;
  const int32_t *row_ptr;
  const int32_t *col;
  const int8_t *shift;
  const int32_t *rev;
} eec_graph;

/* ------------------------------------------------------------------------
 * eec_build_neighbors -- periodic cell-list neighbour list as receiver-sorted
 * CSR.  The edge set is every (i, j, n), n in {-1,0,1}^3, with
 *   d = (x_j - x_i) + n*L  (binary64, component-wise, in that order),
 *   r2 = (dx*dx + dy*dy) + dz*dz  (binary64, no fused multiply-add),
 * kept iff r2 < cutoff*cutoff and not (j == i and n == 0).  Rows are ordered by
 * (j, nx, ny, nz) ascending; rev[e] is the index of (j, i, -n).  The list is
 * rebuilt beside the force call in an MD loop ("FastMACE rewrite screens",
 * OPT2-T04 overlap_rebuild).
 *   pos        [n_atoms][3] float64, every coordinate in [0, L_k)
 *   box        [host] [3] float64 side lengths
 *   species    [n_atoms] int32 or NULL; when given, each value is checked to
 *              lie in [0, n_species) (EEC_ERR_SPECIES)
 *   edge_capacity  length of col / rev (and of shift / 3); 0 = size query
 *   n_edges    [host] out: the edge count E.  Written on EEC_OK and on
 *              EEC_ERR_CAPACITY (then it is the capacity required and the CSR
 *              arrays are not written).
 *   workspace  >= eec_neighbors_workspace_bytes(n_atoms, box, cutoff) bytes
 *              (about 1.1 KB per atom: the cell list and 256 key slots per
 *              atom for the counting pass; rows longer than 256 edges take a
 *              second pass over the candidates)
 * Synchronises `stream` once (to read E and the validity flags, through a
 * 16-byte pinned host word that the library allocates on a thread's first
 * call and keeps until the process ends); the CSR arrays are written after that, on `stream`, so
 * work on another stream that reads them must wait for `stream` (an event).  The out-of-box, species and
 * coincident-atom checks are made on the device before any CSR array is
 * written.  A list built with a cutoff larger than the model's (a Verlet skin)
 * serves the compute entry points unchanged: see eec_skin_check. */
EEC_API eec_status eec_build_neighbors(void *stream, int32_t n_atoms, const double *pos,
                               const double *box, double cutoff,
                               const int32_t *species, int32_t n_species,
                               int64_t edge_capacity, int32_t *row_ptr, int32_t *col,
                               int8_t *shift, int32_t *rev, int64_t *n_edges,
                               void *workspace, size_t workspace_bytes);

EEC_API size_t eec_neighbors_workspace_bytes(int32_t n_atoms, const double *box /*[host][3]*/,
                                     double cutoff);

/* ------------------------------------------------------------------------
 * eec_skin_check -- the Verlet-skin test of an MD loop that builds its list
 * with cutoff rc + skin and reuses it while every atom stays within skin / 2
 * of where it was at the build: then no pair closer than rc can be missing
 * from the list, and the listed pairs at rc or beyond add exactly zero to
 * every output of the compute entry points (the envelope and its derivative
 * vanish there, and the radial network has no bias).  The pages rebuild the
 * list beside the force call ("FastMACE rewrite screens", OPT2-T04
 * overlap_rebuild) and try a 0.2 A skin (the research-engine table's skin and
 * edge-bucket row).
 *   pos, ref   [n_atoms][3] float64: current positions, and the positions the
 *              list was built from (the same frame: the list's image shifts
 *              refer to it, so positions must not be wrapped back into the
 *              cell between rebuilds; the displacement is taken without the
 *              minimum image, so an atom wrapped anyway shows a displacement
 *              of about one box side and is flagged)
 *   half_skin  >= 0, the largest displacement allowed (skin / 2)
 *   max_r2     [1] float64 out: max_i (dx*dx + dy*dy) + dz*dz, d = pos_i - ref_i
 *              in binary64 (no fused multiply-add); +inf if a displacement is
 *              not a number; 0 when n_atoms == 0
 *   rebuild    [1] int32 out: 1 if *max_r2 > half_skin * half_skin, else 0
 * Both outputs are device memory, written on `stream` (two small launches, no
 * synchronisation); the caller reads them when it needs them (for instance
 * one step later, so that the loop never waits on the device). */
EEC_API eec_status eec_skin_check(void *stream, int32_t n_atoms, const double *pos,
                          const double *ref, double half_skin, double *max_r2,
                          int32_t *rebuild);

/* ------------------------------------------------------------------------
 * eec_radial_basis -- per-edge geometry, radial basis and harmonics,
 * materialised (per-stage checks; the hot entry points never call it).
 *   r     [E]        edge length (float32 of the binary64 length)
 *   basis [E][32]    b_n = sin(n pi r / rc) / r * env(r / rc), n = 1..32,
 *                    env(x) = 1 - 28 x^6 + 48 x^7 - 21 x^8 for x < 1
 *   Y     [E][16]    real component-normalised harmonics of u = d / r, flat
 *                    index l*l + l + m, m = -l..l, z polar, no Condon-Shortley
 *                    phase (sum_m Y_lm^2 = 2l + 1)
 * Any of r, basis, Y may be NULL (not computed). */
EEC_API eec_status eec_radial_basis(void *stream, const eec_graph *g, const double *pos,
                            const double *box /*[host][3]*/, double cutoff, float *r,
                            float *basis, float *Y);

/* ------------------------------------------------------------------------
 * eec_radial_project -- the radial network on FP32 matrix cores, materialised:
 *   R[e] = silu(silu(basis[e] W1_p) W2_p) W3_p,  p = Z_recv(e) * S + Z_send(e)
 * ("deepmd-kit PR #6108", What: (E,4,32) -> (E,4,64) -> (E,256)).
 *   species [n_atoms] int32; basis [E][32]; R [E][(lmax+1)*C]
 *   workspace >= eec_project_workspace_bytes(g->n_atoms, g->n_edges, m) */
EEC_API eec_status eec_radial_project(void *stream, const eec_graph *g, const int32_t *species,
                              const eec_model *m, const float *basis, float *R,
                              void *workspace, size_t workspace_bytes);

EEC_API size_t eec_project_workspace_bytes(int32_t n_atoms, int64_t n_edges, const eec_model *m);

/* ------------------------------------------------------------------------
 * eec_edge_message -- the streaming forward:
 *   A[i][lm][c] = sum_{e in row i} R_{e,l,c} Y_{e,lm} h_{Z_j,c}
 * computed over edge chunks: the radial kernel writes one chunk of R (never
 * the whole [E][(lmax+1)*C]) and the message kernel reduces it into the
 * receivers in CSR order with no atomics ("FastMACE rewrite screens",
 * OPT6-T01 L2-resident edge chunks and OPT4-T06 streaming forward).
 *   A [n_atoms][16][C] float32
 *   workspace >= eec_workspace_bytes(n_atoms, n_edges, m) */
EEC_API eec_status eec_edge_message(void *stream, const eec_graph *g, const double *pos,
                            const double *box /*[host][3]*/, const int32_t *species,
                            const eec_model *m, float *A, void *workspace,
                            size_t workspace_bytes);

/* ------------------------------------------------------------------------
 * eec_energy_forces -- energy, per-atom energy, forces (and virial) in one call:
 *   E_i = sum_c w_c sum_lm A_{i,lm,c}^2,  E = sum_i E_i (summed in float64),
 *   g_e = dE/dd_e (streaming backward over edge chunks),
 *   F_i = sum_{e in row i} (g_e - g_rev(e))  (fixed order, no atomics),
 *   virial W_ab = -sum_e d_{e,a} g_{e,b}.
 *   energy      [1] float32
 *   atom_energy [n_atoms] float32 or NULL
 *   forces      [n_atoms][3] float32
 *   virial      [9] float32 (row-major 3x3) or NULL
 *   workspace   >= eec_workspace_bytes(n_atoms, n_edges, m) */
EEC_API eec_status eec_energy_forces(void *stream, const eec_graph *g, const double *pos,
                             const double *box /*[host][3]*/, const int32_t *species,
                             const eec_model *m, float *energy, float *atom_energy,
                             float *forces, float *virial, void *workspace,
                             size_t workspace_bytes);

/* ------------------------------------------------------------------------
 * eec_energy_forces_folded -- the same outputs as eec_energy_forces (equal up
 * to float32 rounding), with the linear last radial layer moved past the edge
 * sum: the fold of a frozen linear map applied after a linear reduction
 * ("deepmd-kit PR #6108", What; exact in real arithmetic, "Accuracy").
 *   forward:  T_{i,s}[k][lm] = sum_{e in row i, Z_j = s} silu(z2_e)[k] Y_e[lm],
 *             A_i[lm][c] = sum_s h_{s,c} sum_k T_{i,s}[k][lm] W3_{(Z_i,s)}[k][l C + c];
 *   backward: M_{i,s}[lm][k] = sum_c (dE/dA_i)[lm][c] h_{s,c} W3_{(Z_i,s)}[k][l C + c],
 *             dE/dY_e = M s2_e,  dE/ds2_e = M^T Y_e.
 * The per-edge radial weights R are never formed.  With one to three species
 * the whole call per receiver (forward, readout, backward) runs in one
 * kernel; with one species the quadratic readout is
 * taken through per-degree Gram matrices
 *   G_l[k][k'] = sum_c 2 w_c h_c^2 W3[k][lC+c] W3[k'][lC+c]:
 *   M_i[lm] = G_l(lm) T_i[lm],  E_i = 1/2 sum_lm T_i[lm] . M_i[lm],
 * so A is never formed either.  Arguments as eec_energy_forces; same
 * workspace size. */
EEC_API eec_status eec_energy_forces_folded(void *stream, const eec_graph *g, const double *pos,
                                    const double *box /*[host][3]*/, const int32_t *species,
                                    const eec_model *m, float *energy, float *atom_energy,
                                    float *forces, float *virial, void *workspace,
                                    size_t workspace_bytes);

/* ------------------------------------------------------------------------
 * eec_energy_forces_folded_noalloc -- for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): eec_energy_forces_folded for one to three species with
 * no workspace argument.  Its scratch is a fixed device array inside the
 * library, EEC_NOALLOC_SCRATCH_BYTES (256 MiB) on every GPU the library is
 * loaded on, held until the process ends; the call allocates nothing.
 * Arguments and outputs as eec_energy_forces_folded (the caller still owns
 * every input and output).  The current device must be the stream's device.
 * The scratch holds about 214 MB of activation stash plus 12 bytes per edge
 * and 76 bytes per atom (with S > 1 species 4 more bytes per edge and
 * 4 + 8 S more per atom), so up to about 4.5 million edges: a larger call, or
 * four species, is rejected (EEC_ERR_WORKSPACE, EEC_ERR_SHAPE) before any
 * launch.  Every call on one GPU uses the same scratch, which keeps the last
 * call's contents (nothing in it needs to start cleared): calls that overlap
 * on one GPU (several streams or host threads) race and must be serialised
 * by the caller.  Results are bit for bit those of eec_energy_forces_folded. */
#define EEC_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
EEC_API eec_status eec_energy_forces_folded_noalloc(void *stream, const eec_graph *g, const double *pos,
                                            const double *box /*[host][3]*/, const int32_t *species,
                                            const eec_model *m, float *energy, float *atom_energy,
                                            float *forces, float *virial);

/* ------------------------------------------------------------------------
 * Radial tables -- the radial chain up to the folded last layer,
 * r -> s2(r) = silu(silu(b(r) W1) W2) (hidden width 64, per ordered species
 * pair), as piecewise polynomials of degree 10 on dyadic pieces of
 * [0, cutoff] ("FastMACE rewrite screens", OPT6-T05 radial_tables:
 * per-species-pair degree-10 Chebyshev tables on dyadic pieces, values and
 * r-derivatives certified against binary64, opt-in and float32 only;
 * OPT6-T04: their accuracy premise).  Approximate: results differ from
 * eec_energy_forces_folded by the table error, which the certificate bounds.
 *
 * Pieces: 2^log2_pieces coarse pieces of width h0 = cutoff / 2^log2_pieces;
 * coarse piece c is split into 2^d(c) equal sub-pieces, d(c) in [0, 4] the
 * smallest level at which the binary64 interpolants are within 1e-8 of the
 * network (values and r-derivatives, relative to the local scale) at 16
 * points per sub-piece; the short-range pieces, where the chain is largest
 * and steepest, take the finer levels.
 *
 * eec_radial_table_build -- builds every pair's table in binary64 on the
 * device: each sub-piece interpolated at the 11 Chebyshev points of the
 * first kind, the interpolant stored in float32 in power form in the
 * sub-piece variable t in [-1, 1], r = c h0 + (f + (t + 1) / 2) h0 / 2^d(c):
 *   coef[p][c][f][m][j % 32][j / 32] = a_m of unit j,  s2_j(r) ~ sum_m a_m t^m
 *   (16 sub-piece slots per coarse piece, f < 2^d(c) used, the others written
 *   as zeros), level[p][c] = d(c).
 *   m            the model (W1, W2 and the cutoff are read)
 *   log2_pieces  in [2, 10]; 6 is the default of the binding
 *   coef         device float32, coef_floats >= eec_radial_table_floats(m, log2_pieces)
 *   level        device int32 [eec_radial_table_levels(m, log2_pieces)]
 *   certificate  device double[2] or NULL: the largest error of the stored
 *                table against the binary64 network over 16 points per
 *                sub-piece, [0] for values and [1] for r-derivatives, each
 *                relative to the largest magnitude of that unit's value
 *                (derivative) over the sub-piece; written on the stream.
 * No synchronisation. */
typedef struct {
  int32_t log2_pieces;
  const float *coef;    /* as written by eec_radial_table_build for the same model */
  const int32_t *level;
} eec_radial_table;

EEC_API size_t eec_radial_table_floats(const eec_model *m, int32_t log2_pieces);
EEC_API size_t eec_radial_table_levels(const eec_model *m, int32_t log2_pieces);

EEC_API eec_status eec_radial_table_build(void *stream, const eec_model *m, int32_t log2_pieces,
                                  float *coef, size_t coef_floats, int32_t *level,
                                  double *certificate);

/* eec_energy_forces_tabulated -- the outputs of eec_energy_forces_folded, with
 * s2 and ds2/dr of every edge read from the table of its species pair in
 * `tab` (built for this model) instead of the basis and the first two layers:
 * per edge a Horner evaluation of 64 units and their derivatives replaces two
 * dense layers and their SiLUs in both passes.  Edges at or beyond the cutoff
 * add exactly zero.  Arguments as eec_energy_forces; same workspace size.
 * One to three species (EEC_ERR_SHAPE for four). */
EEC_API eec_status eec_energy_forces_tabulated(void *stream, const eec_graph *g, const double *pos,
                                       const double *box /*[host][3]*/, const int32_t *species,
                                       const eec_model *m, const eec_radial_table *tab,
                                       float *energy, float *atom_energy, float *forces,
                                       float *virial, void *workspace, size_t workspace_bytes);

/* ------------------------------------------------------------------------
 * eec_energy_forces_timed -- eec_energy_forces (variant EEC_VARIANT_DIRECT),
 * eec_energy_forces_folded (EEC_VARIANT_FOLDED) or eec_energy_forces_tabulated
 * (EEC_VARIANT_TABULATED, with `tab`; NULL otherwise), with hipEvent_t handles
 * (created by the caller, e.g. with hipEventCreate) recorded on `stream` around
 * each phase: events[2k] before and events[2k+1] after phase k, for
 *   k = EEC_PHASE_PREPARE   receiver index and pair grouping, and for the
 *                           folded variant the transpose of W3 (folded, one
 *                           species: the Gram matrices instead; two or three
 *                           species: the grouping of each row by sender
 *                           species and the atoms in species order),
 *       EEC_PHASE_FORWARD   radial network + message (one kernel, or the
 *                           radial-row chunks and message passes; folded,
 *                           one to three species, and tabulated: the single
 *                           fused kernel launch, forward, readout and
 *                           backward),
 *       EEC_PHASE_READOUT   per-atom energies and dE/dA (folded, one to
 *                           three species: empty),
 *       EEC_PHASE_BACKWARD  the streaming backward (one kernel launch;
 *                           folded, one to three species: empty),
 *       EEC_PHASE_SCATTER   forces and the energy total in one kernel launch
 *                           (with the virial, a second launch totals both).
 * `events` holds 2 * EEC_N_PHASES handles (a NULL entry skips that record);
 * NULL records nothing.  Results are bit for bit those of the untimed call. */
enum { EEC_PHASE_PREPARE = 0, EEC_PHASE_FORWARD = 1, EEC_PHASE_READOUT = 2,
       EEC_PHASE_BACKWARD = 3, EEC_PHASE_SCATTER = 4, EEC_N_PHASES = 5 };
enum { EEC_VARIANT_DIRECT = 0, EEC_VARIANT_FOLDED = 1, EEC_VARIANT_TABULATED = 2 };

EEC_API eec_status eec_energy_forces_timed(void *stream, const eec_graph *g, const double *pos,
                                   const double *box /*[host][3]*/, const int32_t *species,
                                   const eec_model *m, float *energy, float *atom_energy,
                                   float *forces, float *virial, void *workspace,
                                   size_t workspace_bytes, int32_t variant,
                                   const eec_radial_table *tab, void *const *events);

EEC_API size_t eec_workspace_bytes(int32_t n_atoms, int64_t n_edges, const eec_model *m);

/* Thread-local text of the last error on this thread ("" if none). */
EEC_API const char *eec_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* EEC_H */

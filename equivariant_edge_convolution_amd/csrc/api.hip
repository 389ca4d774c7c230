// C ABI of the edge-convolution library: argument checks, workspace layout and
// the launch sequence of each entry point on the caller's stream.
#include <math.h>

#include <algorithm>
#include <initializer_list>
#include <mutex>
#include <string>

#include "eec_device.hpp"
#include "eec_internal.hpp"

using namespace eec;

namespace {

thread_local std::string g_err;

eec_status fail(eec_status st, const std::string& why) {
  g_err = why;
  return st;
}
eec_status ok() {
  g_err.clear();
  return EEC_OK;
}

struct Span {
  uintptr_t a = 0, b = 0;
  const char* name = "";
};
Span span(const void* p, size_t bytes, const char* name) {
  Span s;
  s.a = (uintptr_t)p;
  s.b = s.a + bytes;
  s.name = name;
  if (p == nullptr || bytes == 0) s.b = s.a;
  return s;
}
bool overlap(const Span& x, const Span& y) { return x.a < y.b && y.a < x.b; }

// Every output must be disjoint from every input and from the other outputs.
eec_status check_alias(std::initializer_list<Span> outs, std::initializer_list<Span> ins) {
  for (auto o = outs.begin(); o != outs.end(); ++o) {
    for (auto i = ins.begin(); i != ins.end(); ++i)
      if (overlap(*o, *i)) return fail(EEC_ERR_ALIAS, std::string(o->name) + " overlaps input " + i->name);
    for (auto o2 = o + 1; o2 != outs.end(); ++o2)
      if (overlap(*o, *o2)) return fail(EEC_ERR_ALIAS, std::string(o->name) + " overlaps " + o2->name);
  }
  return EEC_OK;
}

eec_status check_box(const double* box, double cutoff) {
  if (box == nullptr) return fail(EEC_ERR_NULL, "box is NULL");
  if (!(isfinite(cutoff) && cutoff > 0.0)) return fail(EEC_ERR_SHAPE, "cutoff must be finite and > 0");
  for (int k = 0; k < 3; ++k)
    if (!(isfinite(box[k]) && box[k] > 0.0 && box[k] >= cutoff))
      return fail(EEC_ERR_BOX, "every box side must be finite, > 0 and >= cutoff");
  return EEC_OK;
}

eec_status check_model(const eec_model* m) {
  if (m == nullptr) return fail(EEC_ERR_NULL, "model is NULL");
  if (!m->W1 || !m->W2 || !m->W3 || !m->emb || !m->w_read) return fail(EEC_ERR_NULL, "a model weight pointer is NULL");
  if (m->n_basis != NB || m->hidden != HID || m->lmax != 3)
    return fail(EEC_ERR_SHAPE, "model must have n_basis 32, hidden 64, lmax 3");
  if (m->channels != 64 && m->channels != 128) return fail(EEC_ERR_SHAPE, "channels must be 64 or 128");
  if (m->n_species < 1 || m->n_species > 4) return fail(EEC_ERR_SHAPE, "n_species must be in [1, 4]");
  if (!(isfinite(m->cutoff) && m->cutoff > 0.0)) return fail(EEC_ERR_SHAPE, "model cutoff must be finite and > 0");
  if (((uintptr_t)m->emb & 15) != 0) return fail(EEC_ERR_SHAPE, "emb must be 16-byte aligned");
  return EEC_OK;
}

eec_status check_graph(const eec_graph* g) {
  if (g == nullptr || g->row_ptr == nullptr) return fail(EEC_ERR_NULL, "graph or row_ptr is NULL");
  if (g->n_atoms < 0 || g->n_edges < 0 || g->n_edges > INT32_MAX) return fail(EEC_ERR_SHAPE, "bad graph sizes");
  if (g->n_edges > 0 && (!g->col || !g->shift || !g->rev)) return fail(EEC_ERR_NULL, "graph edge arrays are NULL");
  if (g->n_edges > 0 && g->n_atoms == 0) return fail(EEC_ERR_SHAPE, "edges without atoms");
  return EEC_OK;
}

eec_status check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return EEC_OK;
  if (ws == nullptr) return fail(EEC_ERR_WORKSPACE, "workspace is NULL");
  if (((uintptr_t)ws & 255) != 0) return fail(EEC_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (have < need) return fail(EEC_ERR_WORKSPACE, "workspace is smaller than required");
  return EEC_OK;
}

eec_status launched(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(EEC_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return ok();
}

#define TRY(x)                      \
  do {                              \
    eec_status st_ = (x);           \
    if (st_ != EEC_OK) return st_;  \
  } while (0)

Span graph_span_rp(const eec_graph* g) { return span(g->row_ptr, 4 * (size_t)(g->n_atoms + 1), "row_ptr"); }
Span graph_span_col(const eec_graph* g) { return span(g->col, 4 * (size_t)g->n_edges, "col"); }
Span graph_span_shift(const eec_graph* g) { return span(g->shift, 3 * (size_t)g->n_edges, "shift"); }
Span graph_span_rev(const eec_graph* g) { return span(g->rev, 4 * (size_t)g->n_edges, "rev"); }

Span model_span(const float* p, const eec_model* m, int which) {
  const size_t P = (size_t)m->n_species * m->n_species, C = m->channels;
  switch (which) {
    case 1: return span(p, 4 * P * NB * HID, "W1");
    case 2: return span(p, 4 * P * HID * HID, "W2");
    case 3: return span(p, 4 * P * HID * 4 * C, "W3");
    case 4: return span(p, 4 * (size_t)m->n_species * C, "emb");
    default: return span(p, 4 * C, "w_read");
  }
}

// Scratch of eec_energy_forces_folded_noalloc: a file-scope device array (one
// copy per GPU, held from the library's load until the process ends).  Host
// code never passes the array's name to a kernel or a copy: the name is a
// host-side stand-in, not a device address.  Its address on a device comes
// from hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[EEC_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[MAX_DEVICES] = {};

// The device address of `scratch` on the current device (which must be the
// device of `stream`).
eec_status scratch_on_current_device(hipStream_t stream, char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES)
    return fail(EEC_ERR_HIP, "no current HIP device (or a device index past 63)");
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return fail(EEC_ERR_HIP, "hipStreamGetDevice failed");
    if (sdev != dev) return fail(EEC_ERR_SHAPE, "the stream belongs to a device other than the current one");
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(EEC_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = (char*)ptr;
  }
  *out = g_scratch_ptr[dev];
  return EEC_OK;
}

}  // namespace

extern "C" {

const char* eec_last_error(void) { return g_err.c_str(); }

size_t eec_neighbors_workspace_bytes(int32_t n_atoms, const double* box, double cutoff) {
  if (box == nullptr || n_atoms < 0 || !(cutoff > 0.0)) return 0;
  return nb_plan(n_atoms, box, cutoff).bytes;
}

eec_status eec_build_neighbors(void* stream, int32_t n_atoms, const double* pos, const double* box,
                               double cutoff, const int32_t* species, int32_t n_species,
                               int64_t edge_capacity, int32_t* row_ptr, int32_t* col, int8_t* shift,
                               int32_t* rev, int64_t* n_edges, void* workspace,
                               size_t workspace_bytes) {
  if (n_edges == nullptr || row_ptr == nullptr) return fail(EEC_ERR_NULL, "n_edges or row_ptr is NULL");
  if (n_atoms < 0 || edge_capacity < 0) return fail(EEC_ERR_SHAPE, "negative size");
  if (n_atoms > 0 && pos == nullptr) return fail(EEC_ERR_NULL, "pos is NULL");
  if (species != nullptr && n_species < 1) return fail(EEC_ERR_SHAPE, "n_species must be >= 1");
  if (edge_capacity > 0 && (!col || !shift || !rev)) return fail(EEC_ERR_NULL, "CSR arrays are NULL");
  TRY(check_box(box, cutoff));
  const NbPlan p = nb_plan(n_atoms, box, cutoff);
  TRY(check_ws(workspace, workspace_bytes, p.bytes));
  const size_t cap = (size_t)edge_capacity;
  TRY(check_alias({span(row_ptr, 4 * (size_t)(n_atoms + 1), "row_ptr"), span(col, 4 * cap, "col"),
                   span(shift, 3 * cap, "shift"), span(rev, 4 * cap, "rev"),
                   span(workspace, workspace_bytes, "workspace")},
                  {span(pos, 24 * (size_t)n_atoms, "pos"), span(species, 4 * (size_t)n_atoms, "species")}));
  const char* why = "";
  const eec_status st = nb_build((hipStream_t)stream, p, n_atoms, pos, box, cutoff, species, n_species,
                                 edge_capacity, row_ptr, col, shift, rev, n_edges, (char*)workspace, &why);
  if (st != EEC_OK) return fail(st, why);
  return launched("build_neighbors");
}

eec_status eec_skin_check(void* stream, int32_t n_atoms, const double* pos, const double* ref,
                          double half_skin, double* max_r2, int32_t* rebuild) {
  if (max_r2 == nullptr || rebuild == nullptr) return fail(EEC_ERR_NULL, "max_r2 or rebuild is NULL");
  if (n_atoms < 0) return fail(EEC_ERR_SHAPE, "negative size");
  if (n_atoms > 0 && (pos == nullptr || ref == nullptr)) return fail(EEC_ERR_NULL, "pos or ref is NULL");
  if (!(isfinite(half_skin) && half_skin >= 0.0)) return fail(EEC_ERR_SHAPE, "half_skin must be finite and >= 0");
  if (((uintptr_t)max_r2 & 7) != 0 || ((uintptr_t)rebuild & 3) != 0)
    return fail(EEC_ERR_SHAPE, "max_r2 must be 8-byte and rebuild 4-byte aligned");
  TRY(check_alias({span(max_r2, 8, "max_r2"), span(rebuild, 4, "rebuild")},
                  {span(pos, 24 * (size_t)n_atoms, "pos"), span(ref, 24 * (size_t)n_atoms, "ref")}));
  launch_skin_check((hipStream_t)stream, n_atoms, pos, ref, half_skin, max_r2, rebuild);
  return launched("skin_check");
}

eec_status eec_radial_basis(void* stream, const eec_graph* g, const double* pos, const double* box,
                            double cutoff, float* r, float* basis, float* Y) {
  TRY(check_graph(g));
  TRY(check_box(box, cutoff));
  if (g->n_atoms > 0 && pos == nullptr) return fail(EEC_ERR_NULL, "pos is NULL");
  const size_t E = (size_t)g->n_edges;
  TRY(check_alias({span(r, 4 * E, "r"), span(basis, 4 * E * NB, "basis"), span(Y, 4 * E * NLM, "Y")},
                  {span(pos, 24 * (size_t)g->n_atoms, "pos"), graph_span_rp(g), graph_span_col(g),
                   graph_span_shift(g), graph_span_rev(g)}));
  Box b{{box[0], box[1], box[2]}};
  launch_basis((hipStream_t)stream, g, pos, b, cutoff, r, basis, Y);
  return launched("radial_basis");
}

size_t eec_project_workspace_bytes(int32_t n_atoms, int64_t n_edges, const eec_model* m) {
  if (m == nullptr || n_atoms < 0 || n_edges < 0) return 0;
  return conv_plan(n_atoms, n_edges, m).off_A;
}

eec_status eec_radial_project(void* stream, const eec_graph* g, const int32_t* species,
                              const eec_model* m, const float* basis, float* R, void* workspace,
                              size_t workspace_bytes) {
  TRY(check_graph(g));
  TRY(check_model(m));
  if (g->n_edges > 0 && (!species || !basis || !R)) return fail(EEC_ERR_NULL, "species, basis or R is NULL");
  const ConvPlan p = conv_plan(g->n_atoms, g->n_edges, m);
  TRY(check_ws(workspace, workspace_bytes, p.off_A));
  const size_t E = (size_t)g->n_edges, NC = 4 * (size_t)m->channels;
  TRY(check_alias({span(R, 4 * E * NC, "R"), span(workspace, workspace_bytes, "workspace")},
                  {span(basis, 4 * E * NB, "basis"), span(species, 4 * (size_t)g->n_atoms, "species"),
                   graph_span_rp(g), graph_span_col(g), graph_span_shift(g), graph_span_rev(g),
                   model_span(m->W1, m, 1), model_span(m->W2, m, 2), model_span(m->W3, m, 3),
                   model_span(m->emb, m, 4), model_span(m->w_read, m, 5)}));
  if (E == 0) return ok();
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  launch_prepare(s, p, g, species, ws, nullptr);
  Box b{{1.0, 1.0, 1.0}};
  launch_radial(s, p, g, nullptr, b, m->cutoff, species, m, basis, 0, p.E, R, nullptr, ws);
  return launched("radial_project");
}

size_t eec_workspace_bytes(int32_t n_atoms, int64_t n_edges, const eec_model* m) {
  if (m == nullptr || n_atoms < 0 || n_edges < 0) return 0;
  return conv_plan(n_atoms, n_edges, m).bytes;
}

static eec_status forward_common(hipStream_t s, const ConvPlan& p, const eec_graph* g, const double* pos,
                                 const double* box, const int32_t* species, const eec_model* m, float* A,
                                 char* ws) {
  launch_prepare(s, p, g, species, ws, A);
  Box b{{box[0], box[1], box[2]}};
  float* Rc = (float*)(ws + p.off_R);
  float* Yc = (float*)(ws + p.off_Y);
  for (int64_t e0 = 0; e0 < p.E; e0 += p.chunk) {
    const int64_t e1 = std::min<int64_t>(p.E, e0 + p.chunk);
    launch_radial(s, p, g, pos, b, m->cutoff, species, m, nullptr, e0, e1, Rc, Yc, ws);
    launch_message(s, p, g, species, m, e0, e1, Rc, Yc, A, ws);
  }
  return EEC_OK;
}

eec_status eec_edge_message(void* stream, const eec_graph* g, const double* pos, const double* box,
                            const int32_t* species, const eec_model* m, float* A, void* workspace,
                            size_t workspace_bytes) {
  TRY(check_graph(g));
  TRY(check_model(m));
  TRY(check_box(box, m->cutoff));
  if (g->n_atoms > 0 && (!pos || !species || !A)) return fail(EEC_ERR_NULL, "pos, species or A is NULL");
  const ConvPlan p = conv_plan(g->n_atoms, g->n_edges, m);
  TRY(check_ws(workspace, workspace_bytes, p.bytes));
  const size_t N = (size_t)g->n_atoms;
  TRY(check_alias({span(A, 4 * N * NLM * m->channels, "A"), span(workspace, workspace_bytes, "workspace")},
                  {span(pos, 24 * N, "pos"), span(species, 4 * N, "species"), graph_span_rp(g),
                   graph_span_col(g), graph_span_shift(g), graph_span_rev(g), model_span(m->W1, m, 1),
                   model_span(m->W2, m, 2), model_span(m->W3, m, 3), model_span(m->emb, m, 4),
                   model_span(m->w_read, m, 5)}));
  if (N == 0) return ok();
  forward_common((hipStream_t)stream, p, g, pos, box, species, m, A, (char*)workspace);
  return launched("edge_message");
}

// noalloc: the folded variant (one to three species) in the layout of
// fold_plan, with the static scratch as its workspace (the workspace
// arguments are ignored).
static eec_status energy_forces_impl(void* stream, const eec_graph* g, const double* pos,
                                     const double* box, const int32_t* species, const eec_model* m,
                                     float* energy, float* atom_energy, float* forces, float* virial,
                                     void* workspace, size_t workspace_bytes, int32_t variant,
                                     const eec_radial_table* tab, void* const* events, bool noalloc = false) {
  if (variant != EEC_VARIANT_DIRECT && variant != EEC_VARIANT_FOLDED && variant != EEC_VARIANT_TABULATED)
    return fail(EEC_ERR_SHAPE, "unknown variant");
  TRY(check_graph(g));
  TRY(check_model(m));
  TRY(check_box(box, m->cutoff));
  if (energy == nullptr) return fail(EEC_ERR_NULL, "energy is NULL");
  if (g->n_atoms > 0 && (!pos || !species || !forces)) return fail(EEC_ERR_NULL, "pos, species or forces is NULL");
  const bool tabulated = variant == EEC_VARIANT_TABULATED;
  if (tabulated) {
    if (tab == nullptr || tab->coef == nullptr || tab->level == nullptr)
      return fail(EEC_ERR_NULL, "radial table is NULL");
    if (tab->log2_pieces < TAB_MIN_LOG2 || tab->log2_pieces > TAB_MAX_LOG2)
      return fail(EEC_ERR_SHAPE, "radial table log2_pieces out of range");
    if (m->n_species > 3) return fail(EEC_ERR_SHAPE, "the tabulated variant takes one to three species");
    if (((uintptr_t)tab->coef & 7) != 0) return fail(EEC_ERR_SHAPE, "radial table must be 8-byte aligned");
  }
  if (noalloc) {
    if (variant != EEC_VARIANT_FOLDED || m->n_species > 3)
      return fail(EEC_ERR_SHAPE, "the no-allocation call is the folded variant for one to three species");
    workspace = nullptr;
    workspace_bytes = 0;
  }
  const ConvPlan p = noalloc ? fold_plan(g->n_atoms, g->n_edges, m) : conv_plan(g->n_atoms, g->n_edges, m);
  if (noalloc) {
    if (p.bytes > EEC_NOALLOC_SCRATCH_BYTES)
      return fail(EEC_ERR_WORKSPACE, "the call needs " + std::to_string(p.bytes) +
                                         " bytes of scratch; the static scratch holds " +
                                         std::to_string((size_t)EEC_NOALLOC_SCRATCH_BYTES));
  } else {
    TRY(check_ws(workspace, workspace_bytes, p.bytes));
  }
  const size_t N = (size_t)g->n_atoms;
  const Span tspan = tabulated ? span(tab->coef, 4 * table_floats(m->n_species, tab->log2_pieces), "radial table")
                               : span(nullptr, 0, "radial table");
  const Span lspan = tabulated ? span(tab->level, 4 * table_levels(m->n_species, tab->log2_pieces), "table levels")
                               : span(nullptr, 0, "table levels");
  TRY(check_alias({span(energy, 4, "energy"), span(atom_energy, 4 * N, "atom_energy"),
                   span(forces, 12 * N, "forces"), span(virial, 36, "virial"),
                   span(workspace, workspace_bytes, "workspace")},
                  {span(pos, 24 * N, "pos"), span(species, 4 * N, "species"), graph_span_rp(g),
                   graph_span_col(g), graph_span_shift(g), graph_span_rev(g), model_span(m->W1, m, 1),
                   model_span(m->W2, m, 2), model_span(m->W3, m, 3), model_span(m->emb, m, 4),
                   model_span(m->w_read, m, 5), tspan, lspan}));
  hipStream_t s = (hipStream_t)stream;
  // phase events (the timed entry point): the first failed record is reported
  hipError_t ev_err = hipSuccess;
  auto mark = [&](int k) {
    if (events == nullptr || events[k] == nullptr) return;
    const hipError_t e = hipEventRecord((hipEvent_t)events[k], s);
    if (ev_err == hipSuccess) ev_err = e;
  };
  auto done = [&](const char* what) {
    if (ev_err != hipSuccess) return fail(EEC_ERR_HIP, std::string(what) + ": event record: " + hipGetErrorString(ev_err));
    return launched(what);
  };
  char* ws = (char*)workspace;
  if (noalloc) TRY(scratch_on_current_device(s, &ws));
  float* A = (float*)(ws + p.off_A);
  float* ei = atom_energy ? atom_energy : (float*)(ws + p.off_ei);
  Box b{{box[0], box[1], box[2]}};
  float* Rc = (float*)(ws + p.off_R);
  float* Yc = (float*)(ws + p.off_Y);
  float* gbuf = (float*)(ws + p.off_g);
  const bool folded = variant == EEC_VARIANT_FOLDED;
  if (tabulated) {
    // one kernel per receiver, s2 and ds2/dr from the radial tables
    mark(2 * EEC_PHASE_PREPARE);
    if (p.S == 1) {
      launch_gram(s, p, m, ws);
    } else {
      launch_prepare_rows(s, p, g, species, ws);
      if (p.C != 64) launch_transpose_w3(s, p, m, ws);  // at C = 64 the kernel keeps W3 in LDS
    }
    mark(2 * EEC_PHASE_PREPARE + 1);
    mark(2 * EEC_PHASE_FORWARD);
    if (p.S == 1)
      launch_fold_table(s, p, g, pos, b, m->cutoff, m, tab->log2_pieces, tab->coef, tab->level, ei, gbuf, ws);
    else
      launch_fold_multi(s, p, g, pos, b, m->cutoff, species, m, ei, gbuf, ws, tab->log2_pieces, tab->coef,
                        tab->level);
    mark(2 * EEC_PHASE_FORWARD + 1);
    for (int k : {EEC_PHASE_READOUT, EEC_PHASE_BACKWARD}) {
      mark(2 * k);
      mark(2 * k + 1);
    }
    mark(2 * EEC_PHASE_SCATTER);
    launch_scatter(s, p, g, pos, b, gbuf, forces, ei, energy, virial, ws);
    mark(2 * EEC_PHASE_SCATTER + 1);
    return done("energy_forces_tabulated");
  }
  if (folded && fold_fused_supported(p)) {
    // one kernel per receiver from geometry to dE/dd; no preparation, no A
    mark(2 * EEC_PHASE_PREPARE);
    launch_gram(s, p, m, ws);
    mark(2 * EEC_PHASE_PREPARE + 1);
    mark(2 * EEC_PHASE_FORWARD);
    launch_fold_fused(s, p, g, pos, b, m->cutoff, species, m, ei, gbuf, ws);
    mark(2 * EEC_PHASE_FORWARD + 1);
    for (int k : {EEC_PHASE_READOUT, EEC_PHASE_BACKWARD}) {
      mark(2 * k);
      mark(2 * k + 1);
    }
    mark(2 * EEC_PHASE_SCATTER);
    launch_scatter(s, p, g, pos, b, gbuf, forces, ei, energy, virial, ws);
    mark(2 * EEC_PHASE_SCATTER + 1);
    return done("energy_forces");
  }
  if (folded && fold_multi_supported(p)) {
    // one kernel per call from geometry to dE/dd, sender species after species
    mark(2 * EEC_PHASE_PREPARE);
    launch_prepare_rows(s, p, g, species, ws);
    if (p.C != 64) launch_transpose_w3(s, p, m, ws);  // at C = 64 the kernel keeps W3 in LDS
    mark(2 * EEC_PHASE_PREPARE + 1);
    mark(2 * EEC_PHASE_FORWARD);
    launch_fold_multi(s, p, g, pos, b, m->cutoff, species, m, ei, gbuf, ws);
    mark(2 * EEC_PHASE_FORWARD + 1);
    for (int k : {EEC_PHASE_READOUT, EEC_PHASE_BACKWARD}) {
      mark(2 * k);
      mark(2 * k + 1);
    }
    mark(2 * EEC_PHASE_SCATTER);
    launch_scatter(s, p, g, pos, b, gbuf, forces, ei, energy, virial, ws);
    mark(2 * EEC_PHASE_SCATTER + 1);
    return done("energy_forces");
  }
  mark(2 * EEC_PHASE_PREPARE);
  launch_prepare(s, p, g, species, ws, A);
  if (folded) launch_transpose_w3(s, p, m, ws);
  mark(2 * EEC_PHASE_PREPARE + 1);
  mark(2 * EEC_PHASE_FORWARD);
  int nparts = 1;
  if (folded) {
    launch_fold_forward(s, p, g, pos, b, m->cutoff, species, m, A, ws);  // S partial slabs
    nparts = p.S;
  } else if (fused_forward_supported(p)) {
    launch_forward(s, p, g, pos, b, m->cutoff, species, m, A, ws);  // S partial slabs
    nparts = p.S;
  } else {
    for (int64_t e0 = 0; e0 < p.E; e0 += p.chunk) {
      const int64_t e1 = std::min<int64_t>(p.E, e0 + p.chunk);
      launch_radial(s, p, g, pos, b, m->cutoff, species, m, nullptr, e0, e1, Rc, Yc, ws);
      launch_message(s, p, g, species, m, e0, e1, Rc, Yc, A, ws);
    }
  }
  mark(2 * EEC_PHASE_FORWARD + 1);
  mark(2 * EEC_PHASE_READOUT);
  launch_readout(s, p, m, A, nparts, ei);  // slab 0 of A now holds dE/dA
  mark(2 * EEC_PHASE_READOUT + 1);
  mark(2 * EEC_PHASE_BACKWARD);
  if (folded)
    launch_fold_backward(s, p, g, pos, b, m->cutoff, species, m, A, gbuf, ws);
  else
    launch_backward(s, p, g, pos, b, m->cutoff, species, m, A, gbuf, ws);
  mark(2 * EEC_PHASE_BACKWARD + 1);
  mark(2 * EEC_PHASE_SCATTER);
  launch_scatter(s, p, g, pos, b, gbuf, forces, ei, energy, virial, ws);
  mark(2 * EEC_PHASE_SCATTER + 1);
  return done("energy_forces");
}

eec_status eec_energy_forces(void* stream, const eec_graph* g, const double* pos, const double* box,
                             const int32_t* species, const eec_model* m, float* energy, float* atom_energy,
                             float* forces, float* virial, void* workspace, size_t workspace_bytes) {
  return energy_forces_impl(stream, g, pos, box, species, m, energy, atom_energy, forces, virial, workspace,
                            workspace_bytes, EEC_VARIANT_DIRECT, nullptr, nullptr);
}

eec_status eec_energy_forces_folded(void* stream, const eec_graph* g, const double* pos, const double* box,
                                    const int32_t* species, const eec_model* m, float* energy,
                                    float* atom_energy, float* forces, float* virial, void* workspace,
                                    size_t workspace_bytes) {
  return energy_forces_impl(stream, g, pos, box, species, m, energy, atom_energy, forces, virial, workspace,
                            workspace_bytes, EEC_VARIANT_FOLDED, nullptr, nullptr);
}

eec_status eec_energy_forces_folded_noalloc(void* stream, const eec_graph* g, const double* pos,
                                            const double* box, const int32_t* species, const eec_model* m,
                                            float* energy, float* atom_energy, float* forces, float* virial) {
  return energy_forces_impl(stream, g, pos, box, species, m, energy, atom_energy, forces, virial, nullptr, 0,
                            EEC_VARIANT_FOLDED, nullptr, nullptr, true);
}

eec_status eec_energy_forces_timed(void* stream, const eec_graph* g, const double* pos, const double* box,
                                   const int32_t* species, const eec_model* m, float* energy,
                                   float* atom_energy, float* forces, float* virial, void* workspace,
                                   size_t workspace_bytes, int32_t variant, const eec_radial_table* tab,
                                   void* const* events) {
  return energy_forces_impl(stream, g, pos, box, species, m, energy, atom_energy, forces, virial, workspace,
                            workspace_bytes, variant, tab, events);
}

eec_status eec_energy_forces_tabulated(void* stream, const eec_graph* g, const double* pos, const double* box,
                                       const int32_t* species, const eec_model* m, const eec_radial_table* tab,
                                       float* energy, float* atom_energy, float* forces, float* virial,
                                       void* workspace, size_t workspace_bytes) {
  return energy_forces_impl(stream, g, pos, box, species, m, energy, atom_energy, forces, virial, workspace,
                            workspace_bytes, EEC_VARIANT_TABULATED, tab, nullptr);
}

size_t eec_radial_table_floats(const eec_model* m, int32_t log2_pieces) {
  if (m == nullptr || m->n_species < 1 || m->n_species > 4 || log2_pieces < TAB_MIN_LOG2 ||
      log2_pieces > TAB_MAX_LOG2)
    return 0;
  return table_floats(m->n_species, log2_pieces);
}

size_t eec_radial_table_levels(const eec_model* m, int32_t log2_pieces) {
  if (m == nullptr || m->n_species < 1 || m->n_species > 4 || log2_pieces < TAB_MIN_LOG2 ||
      log2_pieces > TAB_MAX_LOG2)
    return 0;
  return table_levels(m->n_species, log2_pieces);
}

eec_status eec_radial_table_build(void* stream, const eec_model* m, int32_t log2_pieces, float* coef,
                                  size_t coef_floats, int32_t* level, double* certificate) {
  TRY(check_model(m));
  if (log2_pieces < TAB_MIN_LOG2 || log2_pieces > TAB_MAX_LOG2)
    return fail(EEC_ERR_SHAPE, "log2_pieces out of range");
  if (coef == nullptr || level == nullptr) return fail(EEC_ERR_NULL, "coef or level is NULL");
  const size_t need = table_floats(m->n_species, log2_pieces);
  if (coef_floats < need) return fail(EEC_ERR_SHAPE, "coef is smaller than eec_radial_table_floats");
  if (((uintptr_t)coef & 7) != 0 || ((uintptr_t)certificate & 7) != 0)
    return fail(EEC_ERR_SHAPE, "coef and certificate must be 8-byte aligned");
  if (((uintptr_t)level & 3) != 0) return fail(EEC_ERR_SHAPE, "level must be 4-byte aligned");
  TRY(check_alias({span(coef, 4 * need, "coef"), span(level, 4 * table_levels(m->n_species, log2_pieces), "level"),
                   span(certificate, 16, "certificate")},
                  {model_span(m->W1, m, 1), model_span(m->W2, m, 2)}));
  launch_table_build((hipStream_t)stream, m, log2_pieces, coef, level, certificate);
  return launched("radial_table_build");
}

}  // extern "C"

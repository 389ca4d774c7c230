"""Thin ctypes binding of ``libeec.so`` (the C ABI declared in include/eec.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  PyTorch provides device memory and the current
stream.  The functions keep the C names without the ``eec_`` prefix.

The library must have been built in-tree (``python -m
equivariant_edge_convolution_amd.build``); without it the first call raises,
so nothing can silently fall back to another implementation.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libeec.so")

# status codes of include/eec.h
STATUS = {
    0: "EEC_OK", 1: "EEC_ERR_NULL", 2: "EEC_ERR_SHAPE", 3: "EEC_ERR_BOX", 4: "EEC_ERR_OUT_OF_BOX",
    5: "EEC_ERR_SPECIES", 6: "EEC_ERR_CAPACITY", 7: "EEC_ERR_ALIAS", 8: "EEC_ERR_WORKSPACE",
    9: "EEC_ERR_GEOMETRY", 10: "EEC_ERR_HIP",
}
EEC_ERR_CAPACITY = 6

# every entry point include/eec.h declares
SYMBOLS = (
    "eec_build_neighbors", "eec_neighbors_workspace_bytes", "eec_skin_check", "eec_radial_basis",
    "eec_radial_project", "eec_project_workspace_bytes", "eec_edge_message",
    "eec_energy_forces", "eec_energy_forces_folded", "eec_energy_forces_folded_noalloc",
    "eec_energy_forces_timed", "eec_workspace_bytes",
    "eec_radial_table_floats", "eec_radial_table_levels", "eec_radial_table_build", "eec_energy_forces_tabulated", "eec_last_error",
)
PHASES = ("prepare", "forward", "readout", "backward", "scatter")
VARIANTS = {"direct": 0, "folded": 1, "tabulated": 2}


class EECError(RuntimeError):
    def __init__(self, status: int, what: str, msg: str):
        super().__init__(f"{what}: {STATUS.get(status, status)}: {msg}")
        self.status = status
        self.name = STATUS.get(status, str(status))


class _Model(ctypes.Structure):
    _fields_ = [
        ("n_species", ctypes.c_int32), ("channels", ctypes.c_int32), ("n_basis", ctypes.c_int32),
        ("hidden", ctypes.c_int32), ("lmax", ctypes.c_int32), ("cutoff", ctypes.c_double),
        ("W1", ctypes.c_void_p), ("W2", ctypes.c_void_p), ("W3", ctypes.c_void_p),
        ("emb", ctypes.c_void_p), ("w_read", ctypes.c_void_p),
    ]


class _Graph(ctypes.Structure):
    _fields_ = [
        ("n_atoms", ctypes.c_int32), ("n_edges", ctypes.c_int64), ("row_ptr", ctypes.c_void_p),
        ("col", ctypes.c_void_p), ("shift", ctypes.c_void_p), ("rev", ctypes.c_void_p),
    ]


class _Table(ctypes.Structure):
    _fields_ = [("log2_pieces", ctypes.c_int32), ("coef", ctypes.c_void_p), ("level", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libeec.so once and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m equivariant_edge_convolution_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, dbl, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_size_t
    P = ctypes.POINTER
    L.eec_last_error.restype = ctypes.c_char_p
    L.eec_last_error.argtypes = []
    L.eec_neighbors_workspace_bytes.restype = sz
    L.eec_neighbors_workspace_bytes.argtypes = [i32, P(dbl), dbl]
    L.eec_build_neighbors.restype = ctypes.c_int
    L.eec_build_neighbors.argtypes = [vp, i32, vp, P(dbl), dbl, vp, i32, i64, vp, vp, vp, vp, P(i64), vp, sz]
    L.eec_skin_check.restype = ctypes.c_int
    L.eec_skin_check.argtypes = [vp, i32, vp, vp, dbl, vp, vp]
    L.eec_radial_basis.restype = ctypes.c_int
    L.eec_radial_basis.argtypes = [vp, P(_Graph), vp, P(dbl), dbl, vp, vp, vp]
    L.eec_project_workspace_bytes.restype = sz
    L.eec_project_workspace_bytes.argtypes = [i32, i64, P(_Model)]
    L.eec_radial_project.restype = ctypes.c_int
    L.eec_radial_project.argtypes = [vp, P(_Graph), vp, P(_Model), vp, vp, vp, sz]
    L.eec_workspace_bytes.restype = sz
    L.eec_workspace_bytes.argtypes = [i32, i64, P(_Model)]
    L.eec_edge_message.restype = ctypes.c_int
    L.eec_edge_message.argtypes = [vp, P(_Graph), vp, P(dbl), vp, P(_Model), vp, vp, sz]
    L.eec_energy_forces.restype = ctypes.c_int
    L.eec_energy_forces.argtypes = [vp, P(_Graph), vp, P(dbl), vp, P(_Model), vp, vp, vp, vp, vp, sz]
    L.eec_energy_forces_folded.restype = ctypes.c_int
    L.eec_energy_forces_folded.argtypes = [vp, P(_Graph), vp, P(dbl), vp, P(_Model), vp, vp, vp, vp, vp, sz]
    L.eec_energy_forces_folded_noalloc.restype = ctypes.c_int
    L.eec_energy_forces_folded_noalloc.argtypes = [vp, P(_Graph), vp, P(dbl), vp, P(_Model), vp, vp, vp, vp]
    L.eec_energy_forces_timed.restype = ctypes.c_int
    L.eec_energy_forces_timed.argtypes = [vp, P(_Graph), vp, P(dbl), vp, P(_Model), vp, vp, vp, vp, vp, sz,
                                          i32, P(_Table), P(vp)]
    L.eec_energy_forces_tabulated.restype = ctypes.c_int
    L.eec_energy_forces_tabulated.argtypes = [vp, P(_Graph), vp, P(dbl), vp, P(_Model), P(_Table), vp, vp, vp,
                                              vp, vp, sz]
    L.eec_radial_table_floats.restype = sz
    L.eec_radial_table_floats.argtypes = [P(_Model), i32]
    L.eec_radial_table_build.restype = ctypes.c_int
    L.eec_radial_table_levels.restype = sz
    L.eec_radial_table_levels.argtypes = [P(_Model), i32]
    L.eec_radial_table_build.argtypes = [vp, P(_Model), i32, vp, sz, vp, vp]
    _lib = L
    return L


def _check(status: int, what: str):
    if status != 0:
        raise EECError(status, what, lib().eec_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _box(box) -> ctypes.Array:
    b = np.asarray(box, dtype=np.float64).reshape(3)
    return (ctypes.c_double * 3)(*b.tolist())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


@dataclass
class Model:
    """Model weights resident on the device (float32, contiguous)."""

    n_species: int
    channels: int
    cutoff: float
    W1: torch.Tensor
    W2: torch.Tensor
    W3: torch.Tensor
    emb: torch.Tensor
    w_read: torch.Tensor

    @classmethod
    def from_arrays(cls, m, device="cuda") -> "Model":
        f = lambda a: torch.as_tensor(np.ascontiguousarray(a, dtype=np.float32)).to(device)
        return cls(int(m.n_species), int(m.channels), float(m.cutoff), f(m.W1), f(m.W2), f(m.W3),
                   f(m.emb), f(m.w_read))

    def struct(self) -> _Model:
        return _Model(self.n_species, self.channels, 32, 64, 3, self.cutoff,
                      self.W1.data_ptr(), self.W2.data_ptr(), self.W3.data_ptr(),
                      self.emb.data_ptr(), self.w_read.data_ptr())


@dataclass
class Graph:
    """Receiver-sorted CSR on the device."""

    n_atoms: int
    n_edges: int
    row_ptr: torch.Tensor
    col: torch.Tensor
    shift: torch.Tensor
    rev: torch.Tensor

    @classmethod
    def from_arrays(cls, row_ptr, col, shift, rev, device="cuda") -> "Graph":
        t = lambda a, dt: torch.as_tensor(np.ascontiguousarray(a, dtype=dt)).to(device)
        return cls(len(row_ptr) - 1, len(col), t(row_ptr, np.int32), t(col, np.int32),
                   t(shift, np.int8).reshape(-1, 3), t(rev, np.int32))

    def struct(self) -> _Graph:
        return _Graph(self.n_atoms, self.n_edges, self.row_ptr.data_ptr(),
                      self.col.data_ptr() if self.n_edges else None,
                      self.shift.data_ptr() if self.n_edges else None,
                      self.rev.data_ptr() if self.n_edges else None)


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def neighbors_workspace_bytes(n_atoms: int, box, cutoff: float) -> int:
    return int(lib().eec_neighbors_workspace_bytes(int(n_atoms), _box(box), float(cutoff)))


def workspace_bytes(n_atoms: int, n_edges: int, model: Model) -> int:
    m = model.struct()
    return int(lib().eec_workspace_bytes(int(n_atoms), int(n_edges), ctypes.byref(m)))


def project_workspace_bytes(n_atoms: int, n_edges: int, model: Model) -> int:
    m = model.struct()
    return int(lib().eec_project_workspace_bytes(int(n_atoms), int(n_edges), ctypes.byref(m)))


def build_neighbors(pos: torch.Tensor, box, cutoff: float, species: torch.Tensor | None = None,
                    n_species: int = 0, edge_capacity: int | None = None) -> Graph:
    """eec_build_neighbors; retries once with the exact capacity it reports."""
    dev = pos.device
    n = int(pos.shape[0])
    ws = _workspace(neighbors_workspace_bytes(n, box, cutoff), dev)
    cap = int(edge_capacity) if edge_capacity is not None else 200 * max(n, 1)
    for _ in range(2):
        row_ptr = torch.empty(n + 1, dtype=torch.int32, device=dev)
        col = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
        shift = torch.empty((max(cap, 1), 3), dtype=torch.int8, device=dev)
        rev = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
        ne = ctypes.c_int64(0)
        st = lib().eec_build_neighbors(_stream(dev), n, _ptr(pos), _box(box), float(cutoff),
                                       _ptr(species), int(n_species), cap, _ptr(row_ptr), _ptr(col),
                                       _ptr(shift), _ptr(rev), ctypes.byref(ne), _ptr(ws), ws.numel())
        if st == EEC_ERR_CAPACITY and edge_capacity is None:
            cap = int(ne.value)
            continue
        _check(st, "build_neighbors")
        E = int(ne.value)
        return Graph(n, E, row_ptr, col[:E], shift[:E], rev[:E])
    raise EECError(EEC_ERR_CAPACITY, "build_neighbors", "capacity retry failed")


class NeighborList:
    """Preallocated CSR buffers (``edge_capacity`` edges) and workspace for
    repeated eec_build_neighbors calls on one cell, e.g. the rebuilds of an MD
    loop, which may run on a side stream (the current stream at ``build``)."""

    def __init__(self, n_atoms: int, box, cutoff: float, edge_capacity: int, device,
                 species: torch.Tensor | None = None, n_species: int = 0):
        self.n, self.box, self.cutoff = int(n_atoms), box, float(cutoff)
        self.cap = int(edge_capacity)
        self.species, self.n_species = species, int(n_species)
        self.row_ptr = torch.empty(self.n + 1, dtype=torch.int32, device=device)
        self.col = torch.empty(max(self.cap, 1), dtype=torch.int32, device=device)
        self.shift = torch.empty((max(self.cap, 1), 3), dtype=torch.int8, device=device)
        self.rev = torch.empty(max(self.cap, 1), dtype=torch.int32, device=device)
        self.workspace = _workspace(neighbors_workspace_bytes(self.n, box, cutoff), device)

    def build(self, pos: torch.Tensor) -> Graph:
        """Build into the buffers on the current stream; returns a Graph view
        of them (its arrays are complete once that stream reaches this point)."""
        ne = ctypes.c_int64(0)
        st = lib().eec_build_neighbors(_stream(pos.device), self.n, _ptr(pos), _box(self.box), self.cutoff,
                                       _ptr(self.species), self.n_species, self.cap, _ptr(self.row_ptr),
                                       _ptr(self.col), _ptr(self.shift), _ptr(self.rev), ctypes.byref(ne),
                                       _ptr(self.workspace), self.workspace.numel())
        _check(st, "build_neighbors")
        E = int(ne.value)
        return Graph(self.n, E, self.row_ptr, self.col[:E], self.shift[:E], self.rev[:E])


def skin_check(pos: torch.Tensor, ref: torch.Tensor, half_skin: float, out=None):
    """eec_skin_check on the current stream: (max_r2 [1] float64, rebuild [1]
    int32), device tensors, nothing synchronised."""
    dev = pos.device
    m2, flag = out if out is not None else (torch.empty(1, dtype=torch.float64, device=dev),
                                            torch.empty(1, dtype=torch.int32, device=dev))
    _check(lib().eec_skin_check(_stream(dev), int(pos.shape[0]), _ptr(pos), _ptr(ref), float(half_skin),
                                _ptr(m2), _ptr(flag)), "skin_check")
    return m2, flag


def radial_basis(graph: Graph, pos: torch.Tensor, box, cutoff: float):
    dev = pos.device
    E = graph.n_edges
    r = torch.empty(E, dtype=torch.float32, device=dev)
    basis = torch.empty((E, 32), dtype=torch.float32, device=dev)
    Y = torch.empty((E, 16), dtype=torch.float32, device=dev)
    g = graph.struct()
    _check(lib().eec_radial_basis(_stream(dev), ctypes.byref(g), _ptr(pos), _box(box), float(cutoff),
                                  _ptr(r), _ptr(basis), _ptr(Y)), "radial_basis")
    return r, basis, Y


def radial_project(graph: Graph, species: torch.Tensor, model: Model, basis: torch.Tensor):
    dev = basis.device
    E = graph.n_edges
    R = torch.empty((E, 4 * model.channels), dtype=torch.float32, device=dev)
    ws = _workspace(project_workspace_bytes(graph.n_atoms, E, model), dev)
    g, m = graph.struct(), model.struct()
    _check(lib().eec_radial_project(_stream(dev), ctypes.byref(g), _ptr(species), ctypes.byref(m),
                                    _ptr(basis), _ptr(R), _ptr(ws), ws.numel()), "radial_project")
    return R


def edge_message(graph: Graph, pos: torch.Tensor, box, species: torch.Tensor, model: Model,
                 workspace: torch.Tensor | None = None, out: torch.Tensor | None = None):
    dev = pos.device
    n = graph.n_atoms
    A = out if out is not None else torch.empty((n, 16, model.channels), dtype=torch.float32, device=dev)
    ws = workspace if workspace is not None else _workspace(workspace_bytes(n, graph.n_edges, model), dev)
    g, m = graph.struct(), model.struct()
    _check(lib().eec_edge_message(_stream(dev), ctypes.byref(g), _ptr(pos), _box(box), _ptr(species),
                                  ctypes.byref(m), _ptr(A), _ptr(ws), ws.numel()), "edge_message")
    return A


class RadialTable:
    """eec_radial_table_build: the model's radial tables (device float32) and
    their certificate (device float64 [2]: value and r-derivative error
    relative to the local scale)."""

    def __init__(self, model: "Model", log2_pieces: int = 6):
        m = model.struct()
        n = int(lib().eec_radial_table_floats(ctypes.byref(m), int(log2_pieces)))
        nl = int(lib().eec_radial_table_levels(ctypes.byref(m), int(log2_pieces)))
        if n == 0 or nl == 0:
            raise EECError(2, "radial_table_build", "log2_pieces out of range")
        dev = model.W1.device
        self.log2_pieces = int(log2_pieces)
        self.coef = torch.empty(n, dtype=torch.float32, device=dev)
        self.level = torch.empty(nl, dtype=torch.int32, device=dev)
        self.certificate = torch.empty(2, dtype=torch.float64, device=dev)
        _check(lib().eec_radial_table_build(_stream(dev), ctypes.byref(m), self.log2_pieces, _ptr(self.coef), n,
                                            _ptr(self.level), _ptr(self.certificate)), "radial_table_build")

    def struct(self) -> _Table:
        return _Table(self.log2_pieces, self.coef.data_ptr(), self.level.data_ptr())


class EnergyForces:
    """Preallocated outputs + workspace for repeated eec_energy_forces calls."""

    def __init__(self, graph: Graph, model: Model, device, atom_energy=True, virial=False,
                 variant: str = "direct", edge_capacity: int | None = None, table: RadialTable | None = None):
        n = graph.n_atoms
        if (variant == "tabulated") != (table is not None):
            raise ValueError("the tabulated variant takes a RadialTable, the others none")
        self.table = table
        self._t = table.struct() if table is not None else None
        self.variant = VARIANTS[variant]
        self.graph, self.model = graph, model
        self.energy = torch.empty(1, dtype=torch.float32, device=device)
        self.atom_energy = torch.empty(n, dtype=torch.float32, device=device) if atom_energy else None
        self.forces = torch.empty((n, 3), dtype=torch.float32, device=device)
        self.virial = torch.empty((3, 3), dtype=torch.float32, device=device) if virial else None
        self.cap = max(graph.n_edges, 0 if edge_capacity is None else int(edge_capacity))
        self.workspace = _workspace(workspace_bytes(n, self.cap, model), device)
        self._g = graph.struct()
        self._m = model.struct()

    def __call__(self, pos: torch.Tensor, box, species: torch.Tensor, events=None, graph: Graph | None = None):
        """One eec_energy_forces call on the current stream; with ``events`` (a
        sequence of 2 * len(PHASES) hipEvent_t handles) the instrumented entry
        point records them around each phase.  ``graph`` replaces the bound
        list (same atoms, at most ``edge_capacity`` edges), e.g. after a rebuild."""
        if graph is not None:
            if graph.n_atoms != self.graph.n_atoms or graph.n_edges > self.cap:
                raise ValueError("graph does not fit this EnergyForces (atoms or edge capacity)")
            self.graph, self._g = graph, graph.struct()
        s = _stream(pos.device)
        args = (s, ctypes.byref(self._g), _ptr(pos), _box(box), _ptr(species), ctypes.byref(self._m),
                _ptr(self.energy), _ptr(self.atom_energy), _ptr(self.forces), _ptr(self.virial),
                _ptr(self.workspace), self.workspace.numel())
        tab = ctypes.byref(self._t) if self._t is not None else None
        if events is None:
            if self.variant == 2:
                _check(lib().eec_energy_forces_tabulated(*args[:6], tab, *args[6:]), "energy_forces_tabulated")
            else:
                fn = lib().eec_energy_forces if self.variant == 0 else lib().eec_energy_forces_folded
                _check(fn(*args), "energy_forces")
        else:
            arr = (ctypes.c_void_p * len(events))(*events)
            _check(lib().eec_energy_forces_timed(*args, self.variant, tab, arr), "energy_forces_timed")
        return self


def energy_forces(graph: Graph, pos: torch.Tensor, box, species: torch.Tensor, model: Model,
                  virial: bool = False, variant: str = "direct", table: RadialTable | None = None):
    """eec_energy_forces (variant "direct"), eec_energy_forces_folded ("folded")
    or eec_energy_forces_tabulated ("tabulated", with ``table``)."""
    ef = EnergyForces(graph, model, pos.device, atom_energy=True, virial=virial, variant=variant, table=table)
    ef(pos, box, species)
    out = dict(energy=ef.energy, atom_energy=ef.atom_energy, forces=ef.forces)
    if virial:
        out["virial"] = ef.virial
    return out


def energy_forces_folded_noalloc(graph: Graph, pos: torch.Tensor, box, species: torch.Tensor, model: Model,
                                 virial: bool = False, out: dict | None = None):
    """eec_energy_forces_folded_noalloc: the folded call with the library's
    static device scratch instead of a workspace.  `out` (energy, atom_energy,
    forces and optionally virial tensors, e.g. from an earlier call) is
    written in place; otherwise the outputs are allocated here (by torch, on
    the caller's side of the boundary)."""
    dev = pos.device
    n = graph.n_atoms
    if out is None:
        out = dict(energy=torch.empty(1, dtype=torch.float32, device=dev),
                   atom_energy=torch.empty(n, dtype=torch.float32, device=dev),
                   forces=torch.empty((n, 3), dtype=torch.float32, device=dev))
        if virial:
            out["virial"] = torch.empty((3, 3), dtype=torch.float32, device=dev)
    g, m = graph.struct(), model.struct()
    _check(lib().eec_energy_forces_folded_noalloc(_stream(dev), ctypes.byref(g), _ptr(pos), _box(box),
                                                  _ptr(species), ctypes.byref(m), _ptr(out["energy"]),
                                                  _ptr(out.get("atom_energy")), _ptr(out["forces"]),
                                                  _ptr(out.get("virial"))), "energy_forces_folded_noalloc")
    return out


class HipEvents:
    """hipEvent_t handles from the HIP runtime, for timing phases on the stream
    the library launches on (torch's own events only see torch's launches)."""

    def __init__(self, n: int):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.handles = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self._hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.handles.append(h.value)

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        if self._hip.hipEventElapsedTime(ctypes.byref(ms), self.handles[a], self.handles[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def close(self):
        for h in self.handles:
            self._hip.hipEventDestroy(h)
        self.handles = []

"""The C ABI library loads, exports every symbol include/eec.h declares, and
its host-side checks reject bad arguments before touching a GPU (CPU only)."""
import ctypes
import os
import re

import numpy as np
import pytest

from equivariant_edge_convolution_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "eec.h")


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"EEC_API\s+[\w\s\*]+?\b(eec_\w+)\s*\(", txt)))


def test_header_declares_expected_entry_points():
    assert set(_declared()) == set(B.SYMBOLS)


def test_library_exports_every_declared_symbol():
    L = B.lib()
    for name in _declared():
        assert hasattr(L, name), name


def _model_struct(channels=64, n_species=1, n_basis=32, fake_ptr=256):
    return B._Model(n_species, channels, n_basis, 64, 3, 6.0, fake_ptr, fake_ptr, fake_ptr, fake_ptr, fake_ptr)


def test_workspace_queries_are_host_only_and_monotone():
    L = B.lib()
    m = _model_struct()
    a = L.eec_workspace_bytes(64, 10112, ctypes.byref(m))
    b = L.eec_workspace_bytes(4096, 647168, ctypes.byref(m))
    assert 0 < a < b
    assert b % 256 == 0
    # the streamed radial chunk is bounded: the whole [E, 256] float tensor never fits the workspace
    assert b < 647168 * 256 * 4
    assert L.eec_project_workspace_bytes(64, 10112, ctypes.byref(m)) <= a
    box = (ctypes.c_double * 3)(28.536, 28.536, 28.536)
    assert L.eec_neighbors_workspace_bytes(4096, box, 6.0) > 0
    m128 = _model_struct(channels=128)
    big = L.eec_workspace_bytes(32768, 5177344, ctypes.byref(m128))
    assert big < 5177344 * 512 * 4 / 8


def test_host_side_errors():
    L = B.lib()
    box_small = (ctypes.c_double * 3)(5.0, 7.0, 7.0)
    ne = ctypes.c_int64(-1)
    st = L.eec_build_neighbors(None, 4, ctypes.c_void_p(256), box_small, 6.0, None, 0, 0,
                               ctypes.c_void_p(4096), None, None, None, ctypes.byref(ne), None, 0)
    assert B.STATUS[st] == "EEC_ERR_BOX"
    assert b"cutoff" in L.eec_last_error()
    box = (ctypes.c_double * 3)(7.2, 7.2, 7.2)
    st = L.eec_build_neighbors(None, 4, ctypes.c_void_p(256), box, 6.0, None, 0, 0,
                               ctypes.c_void_p(4096), None, None, None, None, None, 0)
    assert B.STATUS[st] == "EEC_ERR_NULL"
    st = L.eec_build_neighbors(None, 4, ctypes.c_void_p(256), box, 6.0, None, 0, 0,
                               ctypes.c_void_p(4096), None, None, None, ctypes.byref(ne), None, 0)
    assert B.STATUS[st] == "EEC_ERR_WORKSPACE"
    # unsupported model shapes
    g = B._Graph(4, 0, 4096, None, None, None)
    for bad in (_model_struct(channels=96), _model_struct(n_species=5), _model_struct(n_basis=16)):
        st = L.eec_energy_forces(None, ctypes.byref(g), ctypes.c_void_p(256), box, ctypes.c_void_p(512),
                                 ctypes.byref(bad), ctypes.c_void_p(1024), None, ctypes.c_void_p(2048),
                                 None, ctypes.c_void_p(8192), 1 << 20)
        assert B.STATUS[st] == "EEC_ERR_SHAPE"
    # edge counts past the int32 index range (E <= 2^31 - 1) and negative sizes
    good = _model_struct()
    for n_atoms, n_edges in ((4, 1 << 31), (-1, 0), (4, -1)):
        gbig = B._Graph(n_atoms, n_edges, 4096, 4096, 4096, 4096)
        st = L.eec_energy_forces(None, ctypes.byref(gbig), ctypes.c_void_p(256), box, ctypes.c_void_p(512),
                                 ctypes.byref(good), ctypes.c_void_p(1024), None, ctypes.c_void_p(2048),
                                 None, ctypes.c_void_p(8192), 1 << 20)
        assert B.STATUS[st] == "EEC_ERR_SHAPE", (n_atoms, n_edges)
    # outputs overlapping inputs
    m = _model_struct(fake_ptr=1 << 20)
    st = L.eec_energy_forces(None, ctypes.byref(g), ctypes.c_void_p(1 << 16), box, ctypes.c_void_p(1 << 24),
                             ctypes.byref(m), ctypes.c_void_p(1 << 16), None, ctypes.c_void_p(1 << 26),
                             None, ctypes.c_void_p(1 << 28), 1 << 24)
    assert B.STATUS[st] == "EEC_ERR_ALIAS"
    # workspace too small
    need = L.eec_workspace_bytes(4, 0, ctypes.byref(m))
    st = L.eec_energy_forces(None, ctypes.byref(g), ctypes.c_void_p(1 << 16), box, ctypes.c_void_p(1 << 24),
                             ctypes.byref(m), ctypes.c_void_p(1 << 25), None, ctypes.c_void_p(1 << 26),
                             None, ctypes.c_void_p(1 << 28), need - 256)
    assert B.STATUS[st] == "EEC_ERR_WORKSPACE"
    st = L.eec_energy_forces(None, ctypes.byref(g), ctypes.c_void_p(1 << 16), box, ctypes.c_void_p(1 << 24),
                             ctypes.byref(m), ctypes.c_void_p(1 << 25), None, ctypes.c_void_p(1 << 26),
                             None, ctypes.c_void_p((1 << 28) + 64), need)
    assert B.STATUS[st] == "EEC_ERR_WORKSPACE"  # misaligned


def test_skin_check_host_side_errors():
    # every case is rejected before anything is launched
    L = B.lib()
    vp = ctypes.c_void_p
    st = L.eec_skin_check(None, 4, vp(1 << 16), vp(1 << 17), 0.1, None, vp(1 << 20))
    assert B.STATUS[st] == "EEC_ERR_NULL"
    st = L.eec_skin_check(None, 4, None, vp(1 << 17), 0.1, vp(1 << 19), vp(1 << 20))
    assert B.STATUS[st] == "EEC_ERR_NULL"
    st = L.eec_skin_check(None, -1, vp(1 << 16), vp(1 << 17), 0.1, vp(1 << 19), vp(1 << 20))
    assert B.STATUS[st] == "EEC_ERR_SHAPE"
    for half in (float("nan"), float("inf"), -0.5):
        st = L.eec_skin_check(None, 4, vp(1 << 16), vp(1 << 17), half, vp(1 << 19), vp(1 << 20))
        assert B.STATUS[st] == "EEC_ERR_SHAPE", half
    st = L.eec_skin_check(None, 4, vp(1 << 16), vp(1 << 17), 0.1, vp((1 << 19) + 4), vp(1 << 20))
    assert B.STATUS[st] == "EEC_ERR_SHAPE"  # misaligned max_r2
    st = L.eec_skin_check(None, 4, vp(1 << 16), vp(1 << 17), 0.1, vp((1 << 16) + 8), vp(1 << 20))
    assert B.STATUS[st] == "EEC_ERR_ALIAS"  # max_r2 inside pos
    st = L.eec_skin_check(None, 4, vp(1 << 16), vp(1 << 17), 0.1, vp(1 << 19), vp(1 << 19))
    assert B.STATUS[st] == "EEC_ERR_ALIAS"  # the two outputs overlap


def test_radial_table_host_side_errors():
    L = B.lib()
    vp = ctypes.c_void_p
    m = _model_struct(fake_ptr=1 << 20)
    assert L.eec_radial_table_floats(ctypes.byref(m), 1) == 0  # log2_pieces out of range
    assert L.eec_radial_table_levels(ctypes.byref(m), 11) == 0
    n = L.eec_radial_table_floats(ctypes.byref(m), 6)
    assert n == 64 * 16 * 11 * 64 and L.eec_radial_table_levels(ctypes.byref(m), 6) == 64
    st = L.eec_radial_table_build(None, ctypes.byref(m), 1, vp(1 << 24), n, vp(1 << 26), None)
    assert B.STATUS[st] == "EEC_ERR_SHAPE"
    st = L.eec_radial_table_build(None, ctypes.byref(m), 6, None, n, vp(1 << 26), None)
    assert B.STATUS[st] == "EEC_ERR_NULL"
    st = L.eec_radial_table_build(None, ctypes.byref(m), 6, vp(1 << 24), n - 1, vp(1 << 26), None)
    assert B.STATUS[st] == "EEC_ERR_SHAPE"  # too small
    st = L.eec_radial_table_build(None, ctypes.byref(m), 6, vp(1 << 20), n, vp(1 << 26), None)
    assert B.STATUS[st] == "EEC_ERR_ALIAS"  # coef over the weights
    # the tabulated call: a NULL table, and several species
    g = B._Graph(4, 0, 4096, None, None, None)
    box = (ctypes.c_double * 3)(7.2, 7.2, 7.2)
    args = (None, ctypes.byref(g), vp(1 << 16), box, vp(1 << 17), ctypes.byref(m))
    outs = (vp(1 << 25), None, vp(1 << 26), None, vp(1 << 28), 1 << 24)
    assert B.STATUS[L.eec_energy_forces_tabulated(*args, None, *outs)] == "EEC_ERR_NULL"
    m3 = _model_struct(n_species=4, fake_ptr=1 << 20)
    t = B._Table(6, 1 << 29, 1 << 30)
    args3 = (None, ctypes.byref(g), vp(1 << 16), box, vp(1 << 17), ctypes.byref(m3))
    assert B.STATUS[L.eec_energy_forces_tabulated(*args3, ctypes.byref(t), *outs)] == "EEC_ERR_SHAPE"


def test_noalloc_host_side_rejections():
    # the no-allocation call rejects four species and a call whose folded
    # layout exceeds the static scratch, on the host, before any HIP call
    L = B.lib()
    box = (ctypes.c_double * 3)(60.0, 60.0, 60.0)
    fake = dict(pos=ctypes.c_void_p(1 << 40), species=ctypes.c_void_p(1 << 41), energy=ctypes.c_void_p(1 << 42),
                forces=ctypes.c_void_p(1 << 43))
    args = lambda g, m: (None, ctypes.byref(g), fake["pos"], box, fake["species"], ctypes.byref(m), fake["energy"],
                         None, fake["forces"], None)
    g = B._Graph(32768, 5177344, 1 << 44, 1 << 45, 1 << 46, 1 << 47)  # 12 B/edge of dE/dd alone: 62 MB
    st = L.eec_energy_forces_folded_noalloc(*args(g, _model_struct(n_species=4, fake_ptr=1 << 48)))
    assert B.STATUS[st] == "EEC_ERR_SHAPE"
    st = L.eec_energy_forces_folded_noalloc(*args(g, _model_struct(channels=128, fake_ptr=1 << 48)))
    assert B.STATUS[st] == "EEC_ERR_WORKSPACE"
    assert b"static scratch" in L.eec_last_error()
    g = B._Graph(4096, 60_000_000, 1 << 44, 1 << 45, 1 << 46, 1 << 47)
    st = L.eec_energy_forces_folded_noalloc(*args(g, _model_struct(fake_ptr=1 << 48)))
    assert B.STATUS[st] == "EEC_ERR_WORKSPACE"

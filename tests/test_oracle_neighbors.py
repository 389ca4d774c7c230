"""Pins of the oracle's neighbour list (CPU only)."""
import json
import os

import numpy as np
import pytest

import eec_inputs as I
from oracle import neighbors as N

RC = 6.0
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_edge_counts.json")


def _same(a, b):
    for k in ("row_ptr", "col", "shift", "rev"):
        assert np.array_equal(getattr(a, k), getattr(b, k)), k


@pytest.mark.parametrize("name", ["D64", "D512", "RS2", "RS3", "PV2", "PV3"])
def test_bruteforce_equals_celllist(name):
    cfg = I.make_config(name)
    _same(N.neighbors_bruteforce(cfg.pos, cfg.box, RC), N.neighbors_celllist(cfg.pos, cfg.box, RC))


def test_bruteforce_equals_celllist_sampled_rows_perovskite():
    # the 10^3 perovskite has edges within 1e-4 A of the cutoff: the bitwise rule decides
    cfg = I.make_config("PV")
    cl = N.neighbors_celllist(cfg.pos, cfg.box, RC)
    rows = np.random.default_rng(3).choice(cfg.n_atoms, 60, replace=False)
    rows.sort()
    recv, keys = N.neighbors_bruteforce(cfg.pos, cfg.box, RC, rows=rows)
    for i in rows:
        a, b = cl.row_ptr[i], cl.row_ptr[i + 1]
        ck = cl.col[a:b].astype(np.int64) * 27 + ((cl.shift[a:b].astype(np.int64) + 1) @ np.array([9, 3, 1]))
        assert np.array_equal(ck, keys[recv == i])


def test_near_cutoff_edges_exist_in_perovskite():
    cfg = I.make_config("PV")
    cl = N.neighbors_celllist(cfg.pos, cfg.box, RC)
    r = np.linalg.norm(N.edge_vectors(cfg.pos, cfg.box, cl), axis=1)
    assert r.max() > RC - 1e-3


def test_one_cell_per_axis_and_repeated_images():
    # D64 (L = 7.134 < 2 rc) has one cell per axis; the same sender then appears
    # with several image shifts in one row, each a separate edge
    cfg = I.make_config("D64")
    assert np.all(N.cell_grid(cfg.box, RC) == 1)
    cl = N.neighbors_celllist(cfg.pos, cfg.box, RC)
    recv = cl.receivers()
    pair = recv.astype(np.int64) * cfg.n_atoms + cl.col
    assert len(np.unique(pair)) < cl.n_edges


@pytest.mark.parametrize("lattice,reps,expect", [
    ("diamond", 2, {0: 158}), ("diamond", 4, {0: 158}),
    ("rocksalt", 2, {0: 32, 1: 32}),
])
def test_perfect_lattice_shell_counts(lattice, reps, expect):
    pos, spec, box = I.lattice_sites(lattice, reps)
    cl = N.neighbors_celllist(pos, box, RC)
    deg = np.diff(cl.row_ptr)
    for s, k in expect.items():
        assert np.all(deg[spec == s] == k)


def test_perfect_perovskite_site_counts():
    pos, spec, box = I.lattice_sites("perovskite", 3)
    cl = N.neighbors_celllist(pos, box, RC)
    deg = np.diff(cl.row_ptr)
    assert np.all(deg[spec == 0] == 62)
    assert np.all(deg[spec == 1] == 86)
    assert np.all(deg[spec == 2] == 74)


@pytest.mark.parametrize("name", ["D64", "RS2", "PV3"])
def test_reverse_edges(name):
    cfg = I.make_config(name)
    cl = N.neighbors_celllist(cfg.pos, cfg.box, RC)
    e = np.arange(cl.n_edges)
    assert np.array_equal(cl.rev[cl.rev], e)
    d = N.edge_vectors(cfg.pos, cfg.box, cl)
    assert np.array_equal(d[cl.rev], -d)  # bitwise
    recv = cl.receivers()
    assert np.array_equal(cl.col[cl.rev], recv)
    assert np.array_equal(np.bincount(cl.col, minlength=cfg.n_atoms), np.diff(cl.row_ptr))


def test_rows_sorted_and_within_cutoff():
    cfg = I.make_config("PV2")
    cl = N.neighbors_celllist(cfg.pos, cfg.box, RC)
    d = N.edge_vectors(cfg.pos, cfg.box, cl)
    r2 = (d[:, 0] * d[:, 0] + d[:, 1] * d[:, 1]) + d[:, 2] * d[:, 2]
    assert np.all(r2 < RC * RC)
    key = cl.col.astype(np.int64) * 27 + (cl.shift.astype(np.int64) + 1) @ np.array([9, 3, 1])
    for i in range(cfg.n_atoms):
        a, b = cl.row_ptr[i], cl.row_ptr[i + 1]
        assert np.all(np.diff(key[a:b]) > 0)


@pytest.mark.parametrize("reps", [2, 4, 5, 8])
def test_pages_printed_diamond_edge_counts(reps):
    with open(GOLDEN) as f:
        g = json.load(f)
    pos, spec, box = I.lattice_sites("diamond", reps)
    n = len(pos)
    pos = I.wrap(pos + np.random.default_rng(0).normal(0.0, I.NOISE, pos.shape), box)
    cl = N.neighbors_celllist(pos, box, RC)
    assert cl.n_edges == 158 * n
    assert g["counts"][str(n)] - cl.n_edges == 2


def test_errors():
    cfg = I.make_config("D64")
    with pytest.raises(ValueError):
        N.neighbors_celllist(cfg.pos, np.array([5.0, 7.134, 7.134]), RC)
    p = cfg.pos.copy()
    p[3, 1] = cfg.box[1]
    with pytest.raises(ValueError):
        N.neighbors_celllist(p, cfg.box, RC)

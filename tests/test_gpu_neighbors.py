"""Neighbour CSR on the GPU: bit-exact against the oracle; error statuses."""
import numpy as np
import pytest
import torch

import eec_inputs as I
from equivariant_edge_convolution_amd import binding as B
from oracle import neighbors as N

from gpu_util import DEV, device_inputs, graph_for, np_, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["D64", "RS2", "RS3", "PV2", "PV3", "D512", "RS", "PV", "D4096", "D32k"])
def test_csr_bit_exact(name):
    say(f"[neighbors] {name}")
    cfg = I.make_config(name)
    pos, species, _ = device_inputs(cfg)
    g = graph_for(cfg, pos, species)
    ref = N.neighbors_celllist(cfg.pos, cfg.box, cfg.model.cutoff)
    assert g.n_edges == ref.n_edges
    assert np.array_equal(np_(g.row_ptr), ref.row_ptr)
    assert np.array_equal(np_(g.col), ref.col)
    assert np.array_equal(np_(g.shift), ref.shift)
    assert np.array_equal(np_(g.rev), ref.rev)


@pytest.mark.parametrize("n_atoms", [150, 600])
def test_csr_bit_exact_dense_rows(n_atoms):
    # random atoms in a 6.1 A box with rc = 6.0: rows of about 600 (sorted in
    # LDS) and 2,400 keys (past the LDS sort: the rank sort), every image kept
    say(f"[neighbors] dense rows, {n_atoms} atoms")
    box = np.full(3, 6.1)
    cfg = I.make_cluster(np.random.default_rng(n_atoms).uniform(0.0, 6.1, (n_atoms, 3)), box)
    pos = torch.as_tensor(cfg.pos).to(DEV)
    g = B.build_neighbors(pos, box, 6.0)
    ref = N.neighbors_celllist(cfg.pos, box, 6.0)
    deg = np.diff(ref.row_ptr)
    assert deg.max() > (2048 if n_atoms == 600 else 256)
    assert g.n_edges == ref.n_edges
    assert np.array_equal(np_(g.row_ptr), ref.row_ptr)
    assert np.array_equal(np_(g.col), ref.col)
    assert np.array_equal(np_(g.shift), ref.shift)
    assert np.array_equal(np_(g.rev), ref.rev)


def test_csr_bit_exact_more_than_32k_atoms():
    # 40,000 random atoms in a 100 A box (about 36 edges a row): more row counts
    # than the scan keeps in registers (32 per thread of 1,024), so the scan
    # takes its slice-by-slice path
    say("[neighbors] 40,000 atoms")
    box = np.full(3, 100.0)
    cfg = I.make_cluster(np.random.default_rng(40000).uniform(0.0, 100.0, (40000, 3)), box)
    pos = torch.as_tensor(cfg.pos).to(DEV)
    g = B.build_neighbors(pos, box, 6.0)
    ref = N.neighbors_celllist(cfg.pos, box, 6.0)
    assert ref.n_edges > 1_000_000
    assert g.n_edges == ref.n_edges
    assert np.array_equal(np_(g.row_ptr), ref.row_ptr)
    assert np.array_equal(np_(g.col), ref.col)
    assert np.array_equal(np_(g.shift), ref.shift)
    assert np.array_equal(np_(g.rev), ref.rev)


def test_repeat_is_identical():
    cfg = I.make_config("PV3")
    pos, species, _ = device_inputs(cfg)
    a = graph_for(cfg, pos, species)
    b = graph_for(cfg, pos, species)
    for k in ("row_ptr", "col", "shift", "rev"):
        assert torch.equal(getattr(a, k), getattr(b, k))


def test_capacity_query_and_small_capacity():
    cfg = I.make_config("D64")
    pos, species, _ = device_inputs(cfg)
    with pytest.raises(B.EECError) as ei:
        B.build_neighbors(pos, cfg.box, 6.0, species, 1, edge_capacity=100)
    assert ei.value.name == "EEC_ERR_CAPACITY"
    g = B.build_neighbors(pos, cfg.box, 6.0, species, 1)  # queries, then retries with the exact count
    assert g.n_edges == 158 * 64


def test_device_side_input_errors():
    cfg = I.make_config("D64")
    pos, species, _ = device_inputs(cfg)
    bad = pos.clone()
    bad[5, 2] = float(cfg.box[2])  # == L: outside [0, L)
    with pytest.raises(B.EECError) as ei:
        B.build_neighbors(bad, cfg.box, 6.0)
    assert ei.value.name == "EEC_ERR_OUT_OF_BOX"
    bad = pos.clone()
    bad[7, 0] = float("nan")
    with pytest.raises(B.EECError) as ei:
        B.build_neighbors(bad, cfg.box, 6.0)
    assert ei.value.name == "EEC_ERR_OUT_OF_BOX"
    sp = species.clone()
    sp[3] = 1
    with pytest.raises(B.EECError) as ei:
        B.build_neighbors(pos, cfg.box, 6.0, sp, 1)
    assert ei.value.name == "EEC_ERR_SPECIES"
    dup = pos.clone()
    dup[9] = dup[8]
    with pytest.raises(B.EECError) as ei:
        B.build_neighbors(dup, cfg.box, 6.0)
    assert ei.value.name == "EEC_ERR_GEOMETRY"


def test_empty_and_isolated():
    box = np.full(3, 30.0)
    g = B.build_neighbors(torch.zeros((0, 3), dtype=torch.float64, device=DEV), box, 6.0)
    assert g.n_edges == 0 and g.n_atoms == 0
    pos = torch.tensor([[1.0, 1.0, 1.0], [15.0, 15.0, 15.0], [16.0, 15.5, 15.0]], dtype=torch.float64, device=DEV)
    g = B.build_neighbors(pos, box, 6.0)
    assert g.n_edges == 2
    assert np.array_equal(np_(g.row_ptr), [0, 0, 1, 2])
    assert np.array_equal(np_(g.rev), [1, 0])

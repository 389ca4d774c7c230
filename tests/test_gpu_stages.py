"""Per-stage parity: materialised geometry / basis / harmonics and the radial
network on the matrix cores, against the oracle."""
import numpy as np
import pytest
import torch

import eec_inputs as I
from equivariant_edge_convolution_amd import binding as B
from oracle import model as M
from oracle import neighbors as N

from gpu_util import device_inputs, graph_for, np_, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["D64", "PV3"])
def test_basis_and_harmonics(name):
    say(f"[stages] basis {name}")
    cfg = I.make_config(name)
    pos, species, _ = device_inputs(cfg)
    g = graph_for(cfg, pos, species)
    r, b, Y = B.radial_basis(g, pos, cfg.box, cfg.model.cutoff)
    csr = N.neighbors_celllist(cfg.pos, cfg.box, cfg.model.cutoff)
    r0, b0, Y0 = M.stage_basis(cfg.pos, cfg.box, csr, cfg.model.cutoff)
    # r: one float32 rounding of the binary64 length
    assert np.all(np.abs(np_(r) - r0) <= 6e-8 * r0)
    # basis: binary64 recurrence rounded once to float32
    assert np.abs(np_(b) - b0).max() <= 1e-6 * np.abs(b0).max()
    # harmonics: float32 polynomials of a float32 unit vector (values up to ~3)
    assert np.abs(np_(Y) - Y0).max() <= 3e-6


@pytest.mark.parametrize("name", ["D64", "RS3", "PV3", "D64c128"])
def test_radial_projection(name):
    say(f"[stages] project {name}")
    cfg = I.make_config(name)
    pos, species, model = device_inputs(cfg)
    g = graph_for(cfg, pos, species)
    csr = N.neighbors_celllist(cfg.pos, cfg.box, cfg.model.cutoff)
    # both sides take the oracle's basis rounded to float32 (the CSR is the
    # same bit for bit), so the projection alone is compared
    b32 = M.stage_basis(cfg.pos, cfg.box, csr, cfg.model.cutoff)[1].astype(np.float32)
    R = np_(B.radial_project(g, species, model, torch.as_tensor(b32).to(pos.device)))
    R0 = M.stage_project(b32.astype(np.float64), csr, cfg.species, cfg.model)
    # three float32 layers with K <= 64: relative error a few 1e-6 of the output scale
    assert np.all(np.isfinite(R))
    assert np.abs(R - R0).max() <= 2e-5 * np.abs(R0).max()

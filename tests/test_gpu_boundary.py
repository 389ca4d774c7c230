"""The C ABI's contract on the device: callers' inputs are never written,
overlapping outputs are rejected, degenerate cells work, streams and
workspaces behave as documented."""
import ctypes

import numpy as np
import pytest
import torch

import eec_inputs as I
from equivariant_edge_convolution_amd import binding as B
from oracle import model as M

from gpu_util import DEV, device_inputs, graph_for, np_, rms, say

pytestmark = pytest.mark.gpu


def _snapshot(ts):
    torch.cuda.synchronize()
    return [t.detach().clone() for t in ts]


def _same(a, b):
    torch.cuda.synchronize()
    return all(torch.equal(x, y) for x, y in zip(a, b))


def _ef(g, pos, box, species, model, variant, **kw):
    """energy_forces of a variant; the tabulated one with a table built here."""
    table = B.RadialTable(model, 5) if variant == "tabulated" else None
    return B.energy_forces(g, pos, box, species, model, variant=variant, table=table, **kw), table


VARIANTS = ["direct", "folded", "tabulated"]


@pytest.mark.parametrize("variant", VARIANTS)
def test_inputs_are_never_written(variant):
    say(f"[boundary] inputs untouched {variant}")
    cfg = I.make_config("PV3")
    pos, species, model = device_inputs(cfg)
    g = graph_for(cfg, pos, species)
    table = B.RadialTable(model, 5) if variant == "tabulated" else None
    ins = [pos, species, g.row_ptr, g.col, g.shift, g.rev, model.W1, model.W2, model.W3, model.emb, model.w_read]
    if table is not None:
        ins += [table.coef, table.level]
    before = _snapshot(ins)
    B.energy_forces(g, pos, cfg.box, species, model, virial=True, variant=variant, table=table)
    B.edge_message(g, pos, cfg.box, species, model)
    _, basis, _ = B.radial_basis(g, pos, cfg.box, cfg.model.cutoff)
    b_before = _snapshot([basis])
    B.radial_project(g, species, model, basis)
    assert _same(ins, before)
    assert _same([basis], b_before)
    p0 = _snapshot([pos, species])
    graph_for(cfg, pos, species)
    assert _same([pos, species], p0)


def test_overlapping_output_is_rejected():
    cfg = I.make_config("D64")
    pos, species, model = device_inputs(cfg)
    g = graph_for(cfg, pos, species)
    L = B.lib()
    gs, ms = g.struct(), model.struct()
    ws = torch.empty(B.workspace_bytes(g.n_atoms, g.n_edges, model), dtype=torch.uint8, device=DEV)
    energy = torch.empty(1, dtype=torch.float32, device=DEV)
    box = B._box(cfg.box)
    # forces written over the positions
    st = L.eec_energy_forces(None, ctypes.byref(gs), B._ptr(pos), box, B._ptr(species), ctypes.byref(ms),
                             B._ptr(energy), None, B._ptr(pos), None, B._ptr(ws), ws.numel())
    assert B.STATUS[st] == "EEC_ERR_ALIAS"
    # workspace overlapping the weights
    st = L.eec_energy_forces(None, ctypes.byref(gs), B._ptr(pos), box, B._ptr(species), ctypes.byref(ms),
                             B._ptr(energy), None, B._ptr(torch.empty((64, 3), device=DEV)), None,
                             B._ptr(model.W3), ws.numel())
    assert B.STATUS[st] in ("EEC_ERR_ALIAS", "EEC_ERR_WORKSPACE")
    # energy inside the forces
    F = torch.empty((64, 3), dtype=torch.float32, device=DEV)
    st = L.eec_energy_forces(None, ctypes.byref(gs), B._ptr(pos), box, B._ptr(species), ctypes.byref(ms),
                             B._ptr(F), None, B._ptr(F), None, B._ptr(ws), ws.numel())
    assert B.STATUS[st] == "EEC_ERR_ALIAS"


@pytest.mark.parametrize("variant", VARIANTS)
def test_empty_and_edgeless_cells(variant):
    model = B.Model.from_arrays(I.draw_model(1, 64), DEV)
    box = np.full(3, 30.0)
    # no atoms
    pos = torch.zeros((0, 3), dtype=torch.float64, device=DEV)
    sp = torch.zeros(0, dtype=torch.int32, device=DEV)
    g = B.build_neighbors(pos, box, 6.0)
    out, _ = _ef(g, pos, box, sp, model, variant)
    assert float(out["energy"].cpu()[0]) == 0.0
    # atoms, no edges
    pos = torch.tensor([[1.0, 1.0, 1.0], [15.0, 15.0, 15.0], [25.0, 3.0, 9.0]], dtype=torch.float64, device=DEV)
    sp = torch.zeros(3, dtype=torch.int32, device=DEV)
    g = B.build_neighbors(pos, box, 6.0)
    assert g.n_edges == 0
    out, _ = _ef(g, pos, box, sp, model, variant, virial=True)
    assert float(out["energy"].cpu()[0]) == 0.0
    assert np.all(np_(out["forces"]) == 0.0) and np.all(np_(out["atom_energy"]) == 0.0)
    assert np.all(np_(out["virial"]) == 0.0)


@pytest.mark.parametrize("variant", VARIANTS)
def test_isolated_atom_among_others(variant):
    # a trimer plus one far atom: the lone atom has zero energy and force
    box = np.full(3, 40.0)
    xyz = np.array([[5.0, 5.0, 5.0], [6.4, 5.3, 5.1], [5.6, 6.5, 4.2], [30.0, 30.0, 30.0]])
    cfg = I.make_cluster(xyz, box, channels=64, seed=3)
    pos, species, model = device_inputs(cfg)
    g = graph_for(cfg, pos, species)
    assert g.n_edges == 6
    out, _ = _ef(g, pos, cfg.box, species, model, variant)
    ref = M.energy_forces(cfg.pos, cfg.species, cfg.box, cfg.model)
    F = np_(out["forces"])
    assert np.all(F[3] == 0.0) and float(np_(out["atom_energy"])[3]) == 0.0
    assert np.abs(F - ref["F"]).max() <= 1e-4 * rms(ref["F"])
    assert abs(float(np_(out["energy"])[0]) - ref["E"]) <= 1e-5 * abs(ref["E"])


def test_side_stream_and_workspace_reuse():
    cfg = I.make_config("RS3")
    pos, species, model = device_inputs(cfg)
    g = graph_for(cfg, pos, species)
    ef = B.EnergyForces(g, model, pos.device, variant="folded")
    ef(pos, cfg.box, species)
    E, F = ef.energy.clone(), ef.forces.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ef(pos, cfg.box, species)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(ef.energy, E) and torch.equal(ef.forces, F)
    # the same workspace serves a smaller graph next
    cfg2 = I.make_config("RS2")
    pos2, species2, _ = device_inputs(cfg2)
    g2 = graph_for(cfg2, pos2, species2)
    assert B.workspace_bytes(g2.n_atoms, g2.n_edges, model) <= ef.workspace.numel()
    ef2 = B.EnergyForces(g2, model, pos.device, variant="folded")
    ef2.workspace = ef.workspace
    ef2(pos2, cfg2.box, species2)
    ref = M.energy_forces(cfg2.pos, cfg2.species, cfg2.box, cfg2.model)
    assert abs(float(np_(ef2.energy)[0]) - ref["E"]) <= 1e-5 * abs(ref["E"])


def test_message_and_energy_entry_points_agree():
    # the streamed message A, read out on the host, gives the energy the
    # energy entry points report
    cfg = I.make_config("D512")
    pos, species, model = device_inputs(cfg)
    g = graph_for(cfg, pos, species)
    A = np_(B.edge_message(g, pos, cfg.box, species, model)).astype(np.float64)
    E_from_A = float(((A**2).sum(axis=1) @ cfg.model.w_read.astype(np.float64)).sum())
    for variant in ("direct", "folded"):
        E = float(np_(B.energy_forces(g, pos, cfg.box, species, model, variant=variant)["energy"])[0])
        assert abs(E - E_from_A) <= 1e-5 * abs(E_from_A)

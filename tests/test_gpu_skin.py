"""Verlet skin on the GPU: the skin test against the oracle bit for bit; a
list built with cutoff rc + skin bit for bit the oracle's; the energy/force
entry points on such a list, at positions moved up to half the skin, against
the oracle on the exact list of the moved positions (energy within 1e-5
relative, forces max|dF| <= 1e-4 RMS(F)); and the MD loop's rebuild on a side
stream bit for bit equal to the same rebuild on the call's stream ("FastMACE
rewrite screens", OPT2-T04 overlap_rebuild: exact)."""
import os
import sys

import numpy as np
import pytest
import torch

import eec_inputs as I
from equivariant_edge_convolution_amd import binding as B
from oracle import model as M
from oracle import neighbors as NB

from gpu_util import DEV, device_inputs, np_, rms, say

pytestmark = pytest.mark.gpu

SKIN = 0.4


def _check(pos, ref, half):
    p = torch.as_tensor(np.ascontiguousarray(pos, np.float64)).to(DEV)
    r = torch.as_tensor(np.ascontiguousarray(ref, np.float64)).to(DEV)
    m2, flag = B.skin_check(p, r, half)
    return float(np_(m2)[0]), int(np_(flag)[0])


def _skin_cases():
    rng = np.random.default_rng(11)
    cases = [("empty", np.zeros((0, 3)), np.zeros((0, 3)), 0.1)]
    ref = np.zeros((3, 3))
    pos = np.array([[0.375, 0.5, 0.0], [-0.25, 0.0, 0.125], [0.0, 0.0, 0.0]])
    cases.append(("dyadic", pos, ref, 0.625))
    cases.append(("dyadic_below", pos, ref, 0.6))
    edge = np.array([[0.625, 0.0, 0.0]])
    cases.append(("at_threshold", edge, np.zeros((1, 3)), 0.625))
    cases.append(("past_threshold", np.array([[np.nextafter(0.625, 1.0), 0.0, 0.0]]), np.zeros((1, 3)), 0.625))
    cfg = I.make_config("D512")
    d = rng.normal(0.0, 0.03, cfg.pos.shape)
    moved = cfg.pos + d
    m2 = NB.max_displacement2(moved, cfg.pos)
    for k, h in enumerate([0.05, float(np.sqrt(m2)), np.nextafter(float(np.sqrt(m2)), 0.0), 0.5]):
        cases.append((f"D512_{k}", moved, cfg.pos, h))
    wrapped = cfg.pos.copy()
    wrapped[7] = I.wrap(wrapped[7:8] - np.array([[wrapped[7, 0] + 1e-3, 0.0, 0.0]]), cfg.box)[0]
    cases.append(("wrapped_atom", wrapped, cfg.pos, 0.1))
    nan = cfg.pos.copy()
    nan[100, 1] = np.nan
    cases.append(("nan", nan, cfg.pos, 0.1))
    big_ref = rng.uniform(0.0, 50.0, (300_001, 3))
    big = big_ref + rng.normal(0.0, 0.01, big_ref.shape)
    cases.append(("grid_stride", big, big_ref, 0.06))
    return cases


@pytest.mark.parametrize("case", _skin_cases(), ids=lambda c: c[0])
def test_skin_check_bitwise(case):
    name, pos, ref, half = case
    say(f"[skin_check] {name} n={len(pos)} half={half!r}")
    m2, flag = _check(pos, ref, half)
    assert m2 == NB.max_displacement2(pos, ref) or (np.isinf(m2) and np.isinf(NB.max_displacement2(pos, ref)))
    assert flag == int(NB.needs_rebuild(pos, ref, half))


def test_skin_check_rejects_bad_arguments():
    p = torch.zeros((4, 3), dtype=torch.float64, device=DEV)
    with pytest.raises(B.EECError):
        B.skin_check(p, p, -1.0)
    with pytest.raises(B.EECError):
        B.skin_check(p, p, float("nan"))
    with pytest.raises(B.EECError):  # output aliasing an input
        B.skin_check(p, p, 0.1, out=(p.view(-1)[:1], torch.empty(1, dtype=torch.int32, device=DEV)))


@pytest.mark.parametrize("name", ["D512", "PV2"])
def test_skin_list_bitwise(name):
    say(f"[skin_list] {name}")
    cfg = I.make_config(name)
    pos, species, _ = device_inputs(cfg)
    g = B.build_neighbors(pos, cfg.box, cfg.model.cutoff + SKIN, species, cfg.model.n_species)
    ref = NB.neighbors_celllist(cfg.pos, cfg.box, cfg.model.cutoff + SKIN)
    assert g.n_edges == ref.n_edges
    np.testing.assert_array_equal(np_(g.row_ptr), ref.row_ptr)
    np.testing.assert_array_equal(np_(g.col), ref.col)
    np.testing.assert_array_equal(np_(g.shift), ref.shift)
    np.testing.assert_array_equal(np_(g.rev), ref.rev)


_MOVED_REF = {}


@pytest.mark.parametrize("variant", ["direct", "folded"])
@pytest.mark.parametrize("name", ["D512", "PV2", "D64c128", "D1728"])
def test_energy_forces_on_skin_list(name, variant):
    say(f"[skin_energy_forces] {name} {variant}")
    cfg = I.make_config(name)
    pos0, species, model = device_inputs(cfg)
    g = B.build_neighbors(pos0, cfg.box, cfg.model.cutoff + SKIN, species, cfg.model.n_species)
    rng = np.random.default_rng(3)
    d = rng.normal(size=cfg.pos.shape)
    d *= (0.5 * SKIN) * rng.uniform(0.5, 1.0, (len(d), 1)) / np.linalg.norm(d, axis=1, keepdims=True)
    moved = cfg.pos + d  # the list's frame, not wrapped
    assert not NB.needs_rebuild(moved, cfg.pos, 0.5 * SKIN)
    pos = torch.as_tensor(moved).to(DEV)
    got = {k: np_(v) for k, v in B.energy_forces(g, pos, cfg.box, species, model, variant=variant).items()}
    if name not in _MOVED_REF:
        _MOVED_REF[name] = M.energy_forces(I.wrap(moved, cfg.box), cfg.species, cfg.box, cfg.model)
    ref = _MOVED_REF[name]
    assert ref["csr"].n_edges < g.n_edges
    assert abs(float(got["energy"][0]) - ref["E"]) <= 1e-5 * abs(ref["E"])
    assert np.abs(got["atom_energy"] - ref["Ei"]).max() <= 1e-5 * np.abs(ref["Ei"]).max()
    assert np.abs(got["forces"] - ref["F"]).max() <= 1e-4 * rms(ref["F"])


def test_md_side_stream_rebuild_bitwise():
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench

    cfg = I.make_config("D512")
    model = B.Model.from_arrays(cfg.model, DEV)
    steps, skin = 40, 0.2
    say("[md] serial")
    a = bench.md_loop(B, torch, cfg, model, torch.device(DEV), steps, skin, "serial", record=True)
    say(f"[md] side (serial rebuilt {a['rebuilds']} times)")
    b = bench.md_loop(B, torch, cfg, model, torch.device(DEV), steps, skin, "side", record=True)
    assert a["rebuilds"] >= 2 and a["rebuilds"] == b["rebuilds"]
    assert a["E"] == b["E"]
    for fa, fb in zip(a["F"], b["F"]):
        np.testing.assert_array_equal(fa, fb)
    # every call used a valid list: no atom past half the skin of its list
    assert a["max_r2"].max() <= (0.5 * skin) ** 2
    np.testing.assert_array_equal(a["max_r2"], b["max_r2"])
    # the last step against the oracle at the same positions (exact list)
    t = steps - 1
    x = I.md_positions(cfg.pos, I.md_velocities(cfg.n_atoms), t)
    say("[md] oracle at the last step")
    ref = M.energy_forces(I.wrap(x, cfg.box), cfg.species, cfg.box, cfg.model)
    assert abs(a["E"][t] - ref["E"]) <= 1e-5 * abs(ref["E"])
    assert np.abs(a["F"][t] - ref["F"]).max() <= 1e-4 * rms(ref["F"])
    say("[md] every step rebuilt")
    c = bench.md_loop(B, torch, cfg, model, torch.device(DEV), steps, skin, "every", record=True)
    assert c["rebuilds"] == steps
    assert abs(c["E"][t] - ref["E"]) <= 1e-5 * abs(ref["E"])
    assert np.abs(c["F"][t] - ref["F"]).max() <= 1e-4 * rms(ref["F"])

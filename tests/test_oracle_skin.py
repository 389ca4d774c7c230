"""Pins of the oracle's Verlet-skin test and of the skin list (CPU only).

The skin test reuses a list built with cutoff rc + skin while every atom stays
within skin / 2 of where it was at the build ("FastMACE rewrite screens",
OPT2-T04 overlap_rebuild; the research-engine table's 0.2 A skin row).  Pinned
here: the displacement by closed forms and special cases, the half-skin
guarantee by brute force over every image pair, its sharpness by an explicit
head-on pair, and that the listed pairs at rc or beyond add exactly nothing
(energy, forces and virial of a skin list equal those of the exact list).
"""
import math

import numpy as np
import pytest

import eec_inputs as I
from oracle import model as M
from oracle import neighbors as NB


def test_displacement_closed_form():
    ref = np.zeros((3, 3))
    pos = np.array([[0.375, 0.5, 0.0], [-0.25, 0.0, 0.125], [0.0, 0.0, 0.0]])
    # dyadic values: every product and sum is exact
    assert NB.max_displacement2(pos, ref) == 0.140625 + 0.25
    assert NB.max_displacement2(pos[1:], ref[1:]) == 0.0625 + 0.015625
    assert NB.max_displacement2(np.zeros((0, 3)), np.zeros((0, 3))) == 0.0


def test_threshold_is_strict():
    ref = np.zeros((1, 3))
    pos = np.array([[0.625, 0.0, 0.0]])
    assert not NB.needs_rebuild(pos, ref, 0.625)  # exactly half the skin: still valid
    pos[0, 0] = np.nextafter(0.625, 1.0)
    assert NB.needs_rebuild(pos, ref, 0.625)


def test_wrapped_atom_and_nan_are_flagged():
    box = np.array([10.0, 10.0, 10.0])
    ref = np.array([[0.01, 5.0, 5.0], [5.0, 5.0, 5.0]])
    pos = ref.copy()
    pos[0, 0] = I.wrap(np.array([[0.01 - 0.02, 5.0, 5.0]]), box)[0, 0]  # crossed x = 0, wrapped to ~L
    assert NB.max_displacement2(pos, ref) > 99.0
    assert NB.needs_rebuild(pos, ref, 0.1)
    pos = ref.copy()
    pos[1, 2] = np.nan
    assert NB.max_displacement2(pos, ref) == math.inf
    assert NB.needs_rebuild(pos, ref, 0.1)


def _pairs_within(pos, box, rc):
    """Every (i, j, n) with |x_j - x_i + n L| < rc, n in {-1,0,1}^3, by brute
    force over all image pairs (positions need not lie in the cell)."""
    n = len(pos)
    out = set()
    for s, sh in enumerate(NB.SHIFTS):
        d = (pos[None, :, :] - pos[:, None, :]) + sh.astype(np.float64) * box
        r2 = (d[..., 0] * d[..., 0] + d[..., 1] * d[..., 1]) + d[..., 2] * d[..., 2]
        ii, jj = np.nonzero(r2 < rc * rc)
        for i, j in zip(ii.tolist(), jj.tolist()):
            if not (i == j and tuple(sh) == (0, 0, 0)):
                out.add((i, j, s))
    return out


def _csr_keys(csr):
    recv = csr.receivers()
    s = (csr.shift[:, 0].astype(np.int64) + 1) * 9 + (csr.shift[:, 1] + 1) * 3 + (csr.shift[:, 2] + 1)
    return set(zip(recv.tolist(), csr.col.tolist(), s.tolist()))


@pytest.mark.parametrize("name", ["D64", "RS2"])
def test_half_skin_guarantee_bruteforce(name):
    cfg = I.make_config(name)
    rc, skin = 6.0, 0.4
    csr = NB.neighbors_bruteforce(cfg.pos, cfg.box, rc + skin)
    listed = _csr_keys(csr)
    rng = np.random.default_rng(5)
    for trial in range(3):
        d = rng.normal(size=cfg.pos.shape)
        d *= (0.5 * skin) * rng.uniform(0.0, 1.0, (len(d), 1)) / np.linalg.norm(d, axis=1, keepdims=True)
        d[0] *= (0.5 * skin) / np.linalg.norm(d[0]) * (1.0 - 1e-12)  # one atom at the limit
        pos = cfg.pos + d  # not wrapped: the list's frame
        assert not NB.needs_rebuild(pos, cfg.pos, 0.5 * skin)
        inside = _pairs_within(pos, cfg.box, rc)
        assert inside, "no pairs"
        assert inside <= listed, f"{len(inside - listed)} pairs inside rc missing from the skin list"


def test_half_skin_is_sharp():
    # two atoms head-on, just outside rc + skin: not listed; each moves a bit
    # more than half the skin towards the other and they come inside rc
    rc, skin = 6.0, 0.4
    box = np.array([40.0, 40.0, 40.0])
    ref = np.array([[10.0, 20.0, 20.0], [10.0 + rc + skin + 1e-3, 20.0, 20.0]])
    assert NB.neighbors_bruteforce(ref, box, rc + skin).n_edges == 0
    step = 0.5 * skin + 1e-3
    pos = ref + np.array([[step, 0.0, 0.0], [-step, 0.0, 0.0]])
    assert _pairs_within(pos, box, rc)
    assert NB.needs_rebuild(pos, ref, 0.5 * skin)


@pytest.mark.parametrize("name", ["D64", "PV2"])
def test_skin_edges_add_nothing(name):
    # the same positions through the exact list and a list with a 0.4 A skin:
    # the extra pairs lie at r >= rc, where the envelope and its slope vanish
    cfg = I.make_config(name)
    model = cfg.model
    exact = M.energy_forces(cfg.pos, cfg.species, cfg.box, model, want_virial=True)
    skin_csr = NB.neighbors_celllist(cfg.pos, cfg.box, 6.4)
    assert skin_csr.n_edges > exact["csr"].n_edges
    sk = M.energy_forces(cfg.pos, cfg.species, cfg.box, model, csr=skin_csr, want_virial=True)
    assert abs(sk["E"] - exact["E"]) <= 1e-12 * abs(exact["E"])
    np.testing.assert_allclose(sk["Ei"], exact["Ei"], rtol=0, atol=1e-12 * np.abs(exact["Ei"]).max())
    fs = np.abs(exact["F"]).max()
    np.testing.assert_allclose(sk["F"], exact["F"], rtol=0, atol=1e-12 * fs)
    np.testing.assert_allclose(sk["virial"], exact["virial"], rtol=0, atol=1e-12 * np.abs(exact["virial"]).max())
    # and every extra edge's own contribution is exactly zero
    r = np.linalg.norm(sk["d"], axis=1)
    far = r >= 6.0
    assert far.any()
    assert np.all(sk["g"][far] == 0.0)

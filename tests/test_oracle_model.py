"""Pins of the oracle's edge convolution, readout, backward and folded forms (CPU only)."""
import math

import numpy as np
import pytest
from numpy.polynomial import legendre

import eec_inputs as I
from oracle import model as M
from oracle import neighbors as N
from oracle import sph

RC = 6.0


def _fd(f, x, h):
    return (f(x + h) - f(x - h)) / (2 * h)


# ------------------------------------------------------------- radial basis
def test_envelope_boundary_conditions():
    # value 1 and slope 0 at x = 0; value, slope and curvature 0 at x = 1
    assert M.envelope(np.array([0.0]))[0] == 1.0
    x1 = np.array([1.0 - 1e-12])
    assert abs(M.envelope(x1)[0]) < 1e-20
    assert abs(M.envelope_d(x1)[0]) < 1e-20
    # a triple zero at x = 1 (value, slope, curvature): u(1 - t) / t^3 tends to a constant (56)
    t = np.array([1e-3, 3e-4, 1e-4])  # small enough for the limit, large enough for binary64
    ratio = M.envelope(1.0 - t) / t**3
    assert np.allclose(ratio, 56.0, rtol=1e-2)
    xs = np.linspace(0.05, 0.95, 19)
    assert np.allclose(M.envelope_d(xs), _fd(M.envelope, xs, 1e-6), atol=1e-8)
    assert np.all(M.envelope(np.array([1.0, 1.3])) == 0.0)


def test_basis_sine_orthogonality():
    # recover sin(n pi r / rc) = b_n r / env and integrate: (rc/2) delta_nm
    xg, wg = legendre.leggauss(96)
    r = (xg + 1) * (RC / 2) * 0.999999 + 1e-9
    w = wg * (RC / 2) * 0.999999
    b = M.radial_basis(r, RC)
    s = b * r[:, None] / M.envelope(r / RC)[:, None]
    G = (s * w[:, None]).T @ s
    assert np.allclose(G, np.eye(32) * RC / 2, atol=1e-4)


def test_basis_node_counts():
    # b_n has exactly n - 1 sign changes inside (0, rc): fixes the first index n = 1
    r = np.linspace(1e-3, 0.99 * RC, 20001)  # last interior zero of b_32 is at 31/32 rc
    b = M.radial_basis(r, RC)
    changes = (np.diff(np.sign(b), axis=0) != 0).sum(axis=0)
    assert np.array_equal(changes, np.arange(32))


def test_basis_derivative_against_finite_differences():
    r = np.linspace(0.8, 5.99, 57)
    _, db = M.radial_basis(r, RC, deriv=True)
    h = 1e-6
    fd = (M.radial_basis(r + h, RC) - M.radial_basis(r - h, RC)) / (2 * h)
    assert np.allclose(db, fd, atol=1e-7)


def test_special_weight_network_closed_form():
    # W1 = e_{n0} e_a^T, W2 = e_a e_b^T: R = silu(silu(b_{n0})) * W3[b, :]
    # (catches a transposed square W2, a misplaced SiLU, an off-by-one basis index)
    n0, a, bcol = 6, 9, 41
    W1 = np.zeros((32, 64))
    W1[n0, a] = 1.0
    W2 = np.zeros((64, 64))
    W2[a, bcol] = 1.0
    W3 = np.random.default_rng(0).normal(size=(64, 256))
    r = np.array([1.7, 2.9, 4.4, 5.8])
    b = M.radial_basis(r, RC)
    R = M.radial_mlp(b, W1, W2, W3)[-1]

    def silu(t):
        return t / (1.0 + math.exp(-t))

    for q in range(len(r)):
        assert np.allclose(R[q], silu(silu(b[q, n0])) * W3[bcol], rtol=1e-14, atol=1e-300)


# -------------------------------------------------------------- assembly
def _dimer(r, channels=64, seed=0):
    box = np.full(3, 20.0)
    pos = np.array([[5.0, 6.0, 7.0], [5.0, 6.0, 7.0]])
    dirn = np.array([0.36, -0.48, 0.8])
    pos[1] = pos[0] + r * dirn
    return I.make_cluster(pos, box, channels=channels, seed=seed)


def _dimer_closed_form(cfg, r, absolute=False):
    # E = 2 sum_{l,c} (2l+1) w_c h_c^2 R_{l,c}(r)^2  (sum_m Y_lm^2 = 2l+1)
    m = cfg.model
    b = M.radial_basis(np.array([r]), RC)
    R = M.radial_mlp(b, m.W1[0].astype(np.float64), m.W2[0].astype(np.float64),
                     m.W3[0].astype(np.float64))[-1].reshape(4, m.channels)
    w = m.w_read.astype(np.float64)
    if absolute:
        w = np.abs(w)
    h = m.emb[0].astype(np.float64)
    return 2.0 * sum((2 * l + 1) * (w * h * h * R[l] ** 2).sum() for l in range(4))


@pytest.mark.parametrize("r", [1.9, 3.3, 5.6])
def test_dimer_energy_and_force_closed_form(r):
    cfg = _dimer(r)
    out = M.energy_forces(cfg.pos, cfg.species, cfg.box, cfg.model)
    assert out["csr"].n_edges == 2
    dv = cfg.pos[1] - cfg.pos[0]
    r = math.sqrt((dv[0] * dv[0] + dv[1] * dv[1]) + dv[2] * dv[2])  # the bond the positions hold
    Ec = _dimer_closed_form(cfg, r)
    assert abs(out["E"] - Ec) <= 1e-13 * _dimer_closed_form(cfg, r, absolute=True)
    # F_0 = +dE/dr u along d = x_1 - x_0
    h = 1e-5
    dEdr = (_dimer_closed_form(cfg, r + h) - _dimer_closed_form(cfg, r - h)) / (2 * h)
    u = (cfg.pos[1] - cfg.pos[0]) / r
    assert np.allclose(out["F"][0], dEdr * u, atol=1e-7 * max(1.0, abs(dEdr)))
    assert np.allclose(out["F"][1], -dEdr * u, atol=1e-7 * max(1.0, abs(dEdr)))


@pytest.mark.parametrize("name", ["D64", "PV2"])
def test_addition_theorem_double_sum(name):
    # E_i = sum_c w_c sum_l (2l+1) sum_{j,k in row i} rho_j rho_k P_l(u_j . u_k)
    cfg = I.make_config(name)
    m = cfg.model
    csr = N.neighbors_celllist(cfg.pos, cfg.box, RC)
    d = N.edge_vectors(cfg.pos, cfg.box, csr)
    fw = M.forward_edges(d, csr, cfg.species, m)
    r, u = M.geometry(d)
    R = M.stage_project(M.radial_basis(r, RC), csr, cfg.species, m).reshape(-1, 4, m.channels)
    rho = R * m.emb.astype(np.float64)[cfg.species[csr.col]][:, None, :]
    w = m.w_read.astype(np.float64)
    for i in [0, 3, len(cfg.pos) - 1]:
        a, b = csr.row_ptr[i], csr.row_ptr[i + 1]
        cosm = u[a:b] @ u[a:b].T
        Ei = 0.0
        for l in range(4):
            coef = np.zeros(l + 1)
            coef[l] = 1.0
            P = legendre.legval(cosm, coef)
            Ei += (2 * l + 1) * np.einsum("jc,kc,jk,c->", rho[a:b, l], rho[a:b, l], P, w)
        assert abs(fw["Ei"][i] - Ei) <= 1e-11 * abs(Ei) + 1e-12


def test_perfect_crystal_site_symmetry():
    L = sph.l_of_index()
    # diamond (T_d): l = 1, 2 vanish, forces vanish
    pos, spec, box = I.lattice_sites("diamond", 2)
    model = I.draw_model(1, 64)
    out = M.energy_forces(pos, spec, box, model)
    A = out["A"]
    scale = np.abs(A).max()
    assert np.abs(A[:, (L == 1) | (L == 2)]).max() < 1e-12 * scale
    assert np.abs(out["F"]).max() < 1e-10 * np.abs(out["g"]).max()
    assert np.ptp(out["Ei"]) < 1e-12 * np.abs(out["Ei"]).max()
    # rocksalt (O_h): every l >= 1 vanishes
    pos, spec, box = I.lattice_sites("rocksalt", 2)
    out = M.energy_forces(pos, spec, box, I.draw_model(2, 64))
    A = out["A"]
    assert np.abs(A[:, L >= 1]).max() < 1e-12 * np.abs(A).max()
    # perovskite: A and B sites O_h (l >= 1 vanish); O sites D_4h (l = 1, 3 vanish)
    pos, spec, box = I.lattice_sites("perovskite", 2)
    out = M.energy_forces(pos, spec, box, I.draw_model(3, 64))
    A = out["A"]
    sc = np.abs(A).max()
    assert np.abs(A[spec <= 1][:, L >= 1]).max() < 1e-12 * sc
    assert np.abs(A[spec == 2][:, (L == 1) | (L == 3)]).max() < 1e-12 * sc
    assert np.abs(A[spec == 2][:, L == 2]).max() > 1e-6 * sc
    for s in range(3):
        assert np.ptp(out["Ei"][spec == s]) < 1e-11 * np.abs(out["Ei"]).max()


# ------------------------------------------------------------ invariances
@pytest.mark.parametrize("name", ["D64", "RS2", "PV2"])
def test_rotation_invariance_and_force_equivariance(name):
    cfg = I.make_config(name)
    m = cfg.model
    csr = N.neighbors_celllist(cfg.pos, cfg.box, RC)
    d = N.edge_vectors(cfg.pos, cfg.box, csr)
    fw = M.forward_edges(d, csr, cfg.species, m)
    F = M.forces_from_g(M.backward_edges(d, csr, cfg.species, m, fw["A"]), csr)
    for seed in (11, 12):
        Q = I.random_rotation(seed)
        dq = d @ Q.T
        fq = M.forward_edges(dq, csr, cfg.species, m)
        assert abs(fq["E"] - fw["E"]) <= 1e-10 * abs(fw["E"])
        Fq = M.forces_from_g(M.backward_edges(dq, csr, cfg.species, m, fq["A"]), csr)
        assert np.abs(Fq - F @ Q.T).max() <= 1e-10 * np.abs(F).max()


@pytest.mark.parametrize("name", ["D64", "PV2"])
def test_translation_invariance(name):
    cfg = I.make_config(name)
    E0 = M.energy_forces(cfg.pos, cfg.species, cfg.box, cfg.model)["E"]
    t = np.array([1.234, -2.5, 0.77])
    pos = I.wrap(cfg.pos + t[None, :], cfg.box)
    E1 = M.energy_forces(pos, cfg.species, cfg.box, cfg.model)["E"]
    assert abs(E1 - E0) <= 1e-10 * abs(E0)


# ----------------------------------------------------------------- forces
@pytest.mark.parametrize("name,ncomp", [("D64", 12), ("RS2", 8), ("PV2", 8)])
def test_forces_against_central_differences(name, ncomp):
    cfg = I.make_config(name)
    out = M.energy_forces(cfg.pos, cfg.species, cfg.box, cfg.model)
    F, csr = out["F"], out["csr"]
    rms = math.sqrt((F**2).mean())
    rng = np.random.default_rng(7)
    h = 1e-5
    for _ in range(ncomp):
        i, k = int(rng.integers(cfg.n_atoms)), int(rng.integers(3))
        p = cfg.pos.copy()
        p[i, k] += h
        Ep = M.energy_fixed_csr(p, cfg.species, cfg.box, cfg.model, csr)
        p[i, k] -= 2 * h
        Em = M.energy_fixed_csr(p, cfg.species, cfg.box, cfg.model, csr)
        assert abs(-(Ep - Em) / (2 * h) - F[i, k]) <= 1e-6 * rms


@pytest.mark.parametrize("name", ["D64", "RS2", "PV3"])
def test_total_force_zero(name):
    cfg = I.make_config(name)
    F = M.energy_forces(cfg.pos, cfg.species, cfg.box, cfg.model)["F"]
    assert np.abs(F.sum(0)).max() <= 1e-12 * np.abs(F).sum()


def test_virial_against_strain_derivative():
    # dE/deps_ab under d_e -> (I + eps) d_e equals -W_ab with W = -sum_e d_e g_e^T
    cfg = I.make_config("PV2")
    out = M.energy_forces(cfg.pos, cfg.species, cfg.box, cfg.model, want_virial=True)
    csr, d = out["csr"], out["d"]
    W = out["virial"]
    h = 1e-6
    for a in range(3):
        for b in range(3):
            eps = np.zeros((3, 3))
            eps[a, b] = h
            Ep = M.forward_edges(d @ (np.eye(3) + eps).T, csr, cfg.species, cfg.model)["E"]
            Em = M.forward_edges(d @ (np.eye(3) - eps).T, csr, cfg.species, cfg.model)["E"]
            assert abs((Ep - Em) / (2 * h) + W[a, b]) <= 1e-6 * np.abs(W).max()
    assert np.allclose(W, W.T, atol=1e-9 * np.abs(W).max())


# ------------------------------------------------------------ folded forms
@pytest.mark.parametrize("name", ["D64", "RS2", "PV2"])
def test_folded_and_reassociated_last_layer(name):
    cfg = I.make_config(name)
    m = cfg.model
    csr = N.neighbors_celllist(cfg.pos, cfg.box, RC)
    d = N.edge_vectors(cfg.pos, cfg.box, csr)
    A = M.forward_edges(d, csr, cfg.species, m)["A"]
    sc = np.abs(A).max()
    assert np.abs(M.message_h_folded(d, csr, cfg.species, m) - A).max() <= 1e-12 * sc
    assert np.abs(M.message_reassociated(d, csr, cfg.species, m) - A).max() <= 1e-12 * sc
    yd, sd = M.backward_direct_terms(d, csr, cfg.species, m, A)
    yr, sr = M.backward_reassociated_terms(d, csr, cfg.species, m, A)
    assert np.abs(yr - yd).max() <= 1e-12 * np.abs(yd).max()
    assert np.abs(sr - sd).max() <= 1e-12 * np.abs(sd).max()


@pytest.mark.parametrize("name", ["D64", "D64c128"])
def test_gram_readout(name):
    # E_i and dE/dA pulled back to T through per-degree Gram matrices, with no A:
    # equal to the unfolded chain's E_i and its Ybar, s2bar
    cfg = I.make_config(name)
    m = cfg.model
    csr = N.neighbors_celllist(cfg.pos, cfg.box, RC)
    d = N.edge_vectors(cfg.pos, cfg.box, csr)
    out = M.forward_edges(d, csr, cfg.species, m)
    Ei, Mg = M.gram_readout(d, csr, cfg.species, m)
    assert np.abs(Ei - out["Ei"]).max() <= 1e-12 * np.abs(out["Ei"]).max()
    yd, sd = M.backward_direct_terms(d, csr, cfg.species, m, out["A"])
    st = M._edge_stage(d, M.pair_index(cfg.species, csr, 1), m, m.cutoff)
    Me = Mg[csr.receivers()]
    yg = np.einsum("emk,ek->em", Me, st["s2"])
    sg = np.einsum("emk,em->ek", Me, st["Y"])
    assert np.abs(yg - yd).max() <= 1e-12 * np.abs(yd).max()
    assert np.abs(sg - sd).max() <= 1e-12 * np.abs(sd).max()


def test_edge_direction_reading_only_flips_odd_degrees():
    # reversing every edge vector flips odd-l A and leaves E unchanged
    cfg = I.make_config("D64")
    csr = N.neighbors_celllist(cfg.pos, cfg.box, RC)
    d = N.edge_vectors(cfg.pos, cfg.box, csr)
    f1 = M.forward_edges(d, csr, cfg.species, cfg.model)
    f2 = M.forward_edges(-d, csr, cfg.species, cfg.model)
    L = sph.l_of_index()
    sign = np.where(L % 2 == 1, -1.0, 1.0)
    assert np.allclose(f2["A"], f1["A"] * sign[None, :, None], atol=1e-12 * np.abs(f1["A"]).max())
    assert abs(f1["E"] - f2["E"]) <= 1e-12 * abs(f1["E"])


# ------------------------------------------------------------- conditioning
@pytest.mark.parametrize("r", [1.9, 4.4])
def test_conditioning_closed_forms(r):
    # kappa_E's numerator sum_i sum_c |w_c| sum_lm A^2 is the dimer closed form
    # with |w|; kappa_F of a dimer is exactly sqrt 3: g_rev = -g_e, so |F_0| =
    # 2|g| = the row's sum of |g_e| + |g_rev|, and RMS(F) over the six force
    # components is |F_0| / sqrt 3
    cfg = _dimer(r)
    out = M.energy_forces(cfg.pos, cfg.species, cfg.box, cfg.model)
    dv = cfg.pos[1] - cfg.pos[0]
    rr = math.sqrt((dv[0] * dv[0] + dv[1] * dv[1]) + dv[2] * dv[2])
    kE, kF, rms = M.conditioning(out, cfg.model, out["csr"])
    want = _dimer_closed_form(cfg, rr, absolute=True) / abs(_dimer_closed_form(cfg, rr))
    assert want > 1.0
    assert abs(kE - want) <= 1e-10 * want
    assert abs(kF - math.sqrt(3.0)) <= 1e-12
    assert abs(rms - float(np.linalg.norm(out["F"][0])) / math.sqrt(3.0)) <= 1e-12 * rms
    # with every readout weight of one sign the energy cannot cancel: kappa_E = 1
    pos_w = I.make_cluster(cfg.pos, cfg.box)
    pos_w.model.w_read[:] = np.abs(pos_w.model.w_read)
    out = M.energy_forces(pos_w.pos, pos_w.species, pos_w.box, pos_w.model)
    assert abs(M.conditioning(out, pos_w.model, out["csr"])[0] - 1.0) <= 1e-12

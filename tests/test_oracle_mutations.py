"""Planted mistakes in the oracle must fail a pin (CPU only).

Each case patches one plausible slip into the oracle (a dropped term, a wrong
sign, index or coefficient, a transposed operand), re-runs the pin test that
should catch it, and expects that test to fail.  This checks the pins, not the
GPU path: nothing here touches the HIP library.
"""
import math

import numpy as np
import pytest

import eec_inputs as I
from oracle import model as M
from oracle import sph

import test_oracle_model as TM
import test_oracle_sph as TS


def _fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_envelope_coefficient_slip(monkeypatch):
    orig = M.envelope

    def bad(x):
        x = np.asarray(x, np.float64)
        return np.where(x < 1.0, 1.0 - 28.0 * x**6 + 47.0 * x**7 - 21.0 * x**8, 0.0)

    monkeypatch.setattr(M, "envelope", bad)
    _fails(TM.test_envelope_boundary_conditions)
    monkeypatch.setattr(M, "envelope", orig)


def test_basis_index_off_by_one(monkeypatch):
    orig = M.radial_basis

    def bad(r, rc, n_basis=32, deriv=False):
        out = orig(r, rc, n_basis + 1, deriv)
        return tuple(o[:, 1:] for o in out) if deriv else out[:, 1:]

    monkeypatch.setattr(M, "radial_basis", bad)
    TM.test_basis_sine_orthogonality()  # a shifted sine family is still orthogonal
    _fails(TM.test_basis_node_counts)


def test_basis_derivative_dropped_term(monkeypatch):
    orig = M.radial_basis

    def bad(r, rc, n_basis=32, deriv=False):
        if not deriv:
            return orig(r, rc, n_basis)
        b, db = orig(r, rc, n_basis, True)
        x = np.asarray(r) / rc
        s_over_r = b / M.envelope(x)[:, None]
        return b, db - s_over_r * (M.envelope_d(x) / rc)[:, None]  # drop the envelope-slope term

    monkeypatch.setattr(M, "radial_basis", bad)
    _fails(TM.test_basis_derivative_against_finite_differences)


def test_transposed_square_layer(monkeypatch):
    orig = M.radial_mlp

    def bad(b, W1, W2, W3):
        return orig(b, W1, np.ascontiguousarray(W2.T), W3)

    monkeypatch.setattr(M, "radial_mlp", bad)
    _fails(TM.test_special_weight_network_closed_form)


def test_silu_after_last_layer(monkeypatch):
    orig = M.radial_mlp

    def bad(b, W1, W2, W3):
        z1, s1, z2, s2, R = orig(b, W1, W2, W3)
        return z1, s1, z2, s2, M.silu(R)

    monkeypatch.setattr(M, "radial_mlp", bad)
    _fails(TM.test_special_weight_network_closed_form)


def test_harmonic_normalisation_slip(monkeypatch):
    orig = sph.real_sph

    def bad(u, lmax=3, grad=False):
        out = orig(u, lmax, grad)
        Y = (out[0] if grad else out).copy()
        Y[:, sph.lm_index(2, 2)] *= math.sqrt(2.0)  # a doubled m != 0 factor
        return (Y, out[1]) if grad else Y

    monkeypatch.setattr(sph, "real_sph", bad)
    _fails(TS.test_addition_theorem)
    _fails(TS.test_y00_and_component_normalisation)


def test_harmonic_sign_convention_slip(monkeypatch):
    # a Condon-Shortley sign on odd m leaves every invariant unchanged; the
    # explicit polynomial table fixes the convention the GPU path shares
    orig = sph.real_sph

    def bad(u, lmax=3, grad=False):
        out = orig(u, lmax, grad)
        Y = (out[0] if grad else out).copy()
        for l in range(lmax + 1):
            for m in (-1, 1, -3, 3):
                if abs(m) <= l:
                    Y[:, sph.lm_index(l, m)] *= -1.0
        return (Y, out[1]) if grad else Y

    monkeypatch.setattr(sph, "real_sph", bad)
    TS.test_addition_theorem()  # convention-free: still passes
    _fails(TS.test_convention_against_explicit_polynomials)


def test_receiver_embedding_instead_of_sender(monkeypatch):
    orig = M.forward_edges

    def bad(d, csr, species, model, keep_edges=False):
        # h of the receiver (wrong) in place of the sender's
        swapped = I.Model(model.n_species, model.channels, model.W1, model.W2, model.W3,
                          model.emb, model.w_read, model.cutoff)
        out = orig(d, csr, species, swapped, keep_edges)
        recv = csr.receivers()
        h = model.emb.astype(np.float64)
        msg, _ = M.edge_messages(d, M.pair_index(species, csr, model.n_species), h[species[recv]], model)
        A = np.zeros_like(out["A"])
        np.add.at(A, recv, msg)
        out["A"] = A
        out["Ei"] = (A**2).sum(axis=1) @ model.w_read.astype(np.float64)
        return out

    monkeypatch.setattr(M, "forward_edges", bad)
    _fails(TM.test_addition_theorem_double_sum, "PV2")


def test_missing_tangential_projection(monkeypatch):
    orig = M.edge_backward

    def bad(d, pairs, hj, Ab, model):
        g = orig(d, pairs, hj, Ab, model)
        # add back the radial component of the angular gradient (projection dropped)
        st = M._edge_stage(d, pairs, model, model.cutoff, want_grad=True)
        R = st["R"].reshape(len(d), 4, model.channels)
        Ybar = (Ab * (R * hj[:, None, :])[:, M.LIDX, :]).sum(axis=2)
        G = np.einsum("ek,ekx->ex", Ybar, st["dY"])
        u, r = st["u"], st["r"]
        return g + ((G * u).sum(axis=1, keepdims=True) * u) / r[:, None]

    monkeypatch.setattr(M, "edge_backward", bad)
    _fails(TM.test_forces_against_central_differences, "PV2", 8)


def test_force_sign_slip(monkeypatch):
    orig = M.forces_from_g
    monkeypatch.setattr(M, "forces_from_g", lambda g, csr: -orig(g, csr))
    _fails(TM.test_forces_against_central_differences, "D64", 4)


def test_virial_transposed_and_signed(monkeypatch):
    monkeypatch.setattr(M, "virial_from_g", lambda d, g: d.T @ g)
    _fails(TM.test_virial_against_strain_derivative)


def test_fold_with_receiver_species_weights(monkeypatch):
    # the reassociated form indexing W3 by (Z_j, Z_i) instead of (Z_i, Z_j)
    orig = M.message_reassociated

    def bad(d, csr, species, model):
        S = model.n_species
        W3 = model.W3.reshape(S, S, *model.W3.shape[1:]).transpose(1, 0, 2, 3).reshape(model.W3.shape)
        swapped = I.Model(S, model.channels, model.W1, model.W2, np.ascontiguousarray(W3),
                          model.emb, model.w_read, model.cutoff)
        return orig(d, csr, species, swapped)

    monkeypatch.setattr(M, "message_reassociated", bad)
    _fails(TM.test_folded_and_reassociated_last_layer, "RS2")


def test_gram_without_the_factor_two(monkeypatch):
    # the Gram matrices built from w h^2 instead of 2 w h^2 (the derivative's factor)
    orig = M.gram_readout

    def bad(d, csr, species, model):
        Ei, Mg = orig(d, csr, species, model)
        return Ei, 0.5 * Mg

    monkeypatch.setattr(M, "gram_readout", bad)
    _fails(TM.test_gram_readout, "D64")


def test_gram_with_the_wrong_degree_block(monkeypatch):
    # every harmonic paired with the l = 1 block of W3
    orig_lidx = M.LIDX

    def bad(d, csr, species, model):
        monkeypatch.setattr(M, "LIDX", np.where(orig_lidx == 0, 0, 1))
        try:
            return M.__dict__["_gram_orig"](d, csr, species, model)
        finally:
            monkeypatch.setattr(M, "LIDX", orig_lidx)

    monkeypatch.setattr(M, "_gram_orig", M.gram_readout, raising=False)
    monkeypatch.setattr(M, "gram_readout", bad)
    _fails(TM.test_gram_readout, "D64")


def test_envelope_not_cut_off_beyond_rc(monkeypatch):
    # the polynomial continued past x = 1 instead of zero there: skin edges leak
    import test_oracle_skin as TK

    def bad(x):
        x = np.asarray(x, np.float64)
        return 1.0 - 28.0 * x**6 + 48.0 * x**7 - 21.0 * x**8

    monkeypatch.setattr(M, "envelope", bad)
    _fails(TK.test_skin_edges_add_nothing, "D64")


def test_skin_displacement_by_minimum_image(monkeypatch):
    # minimum image would hide an atom wrapped back into the cell
    import test_oracle_skin as TK
    from oracle import neighbors as NB

    def bad(pos, ref):
        d = np.asarray(pos, np.float64) - np.asarray(ref, np.float64)
        d -= 10.0 * np.rint(d / 10.0)
        r2 = (d[:, 0] * d[:, 0] + d[:, 1] * d[:, 1]) + d[:, 2] * d[:, 2]
        return float(r2.max()) if len(r2) else 0.0

    monkeypatch.setattr(NB, "max_displacement2", bad)
    _fails(TK.test_wrapped_atom_and_nan_are_flagged)

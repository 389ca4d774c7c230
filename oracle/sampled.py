"""Exact per-atom energies and forces for a sample of atoms of a large cell.

TEST INFRASTRUCTURE ONLY (oracle; never used by the product path).

Same definitions as ``model`` (the edge convolution of the pages; see that
module's header for the citations), restricted to the rows they depend on:
E_i needs row i; F_i = sum_{e in row i} (g_e - g_rev(e)) needs g on row i and
on the reverse edges, which live in the rows of i's senders j, and g on a row
needs that row's complete A.  So A is formed for the sampled atoms and all of
their senders, nothing is approximated, and the cost scales with the sample.
Parity pins: inherited from ``model`` (the restriction only selects rows; the
test suite checks it equals the full oracle on a small cell).
"""
from __future__ import annotations

import numpy as np

from . import model as M
from .neighbors import CSR


def _rows(rp, atoms):
    return np.concatenate([np.arange(rp[i], rp[i + 1]) for i in atoms] + [np.zeros(0, np.int64)])


def sampled_energy_forces(pos, species, box, model, csr: CSR, atoms, forces_for=None):
    """E_i for ``atoms`` and F_i for ``forces_for`` (default: the same atoms)."""
    pos = np.asarray(pos, np.float64)
    box = np.asarray(box, np.float64)
    rp = csr.row_ptr.astype(np.int64)
    S = np.unique(np.asarray(atoms, np.int64))
    FS = S if forces_for is None else np.unique(np.asarray(forces_for, np.int64))
    eF = _rows(rp, FS)
    T = np.union1d(np.union1d(S, FS), csr.col[eF].astype(np.int64))
    C = model.channels
    h = np.asarray(model.emb, np.float64)
    w = np.asarray(model.w_read, np.float64)
    recv_all = csr.receivers()

    def dvec(edges):
        i = recv_all[edges]
        j = csr.col[edges]
        return (pos[j] - pos[i]) + csr.shift[edges].astype(np.float64) * box[None, :]

    def pairs_of(edges):
        return species[recv_all[edges]].astype(np.int64) * model.n_species + species[csr.col[edges]]

    # complete A rows for every atom in T
    A = {}
    for blk in np.array_split(T, max(1, len(T) // 256)):
        eT = _rows(rp, blk)
        msg, _ = M.edge_messages(dvec(eT), pairs_of(eT), h[species[csr.col[eT]]], model)
        loc = np.searchsorted(blk, recv_all[eT])
        Ablk = np.zeros((len(blk), 16, C))
        np.add.at(Ablk, loc, msg)
        for k, i in enumerate(blk):
            A[int(i)] = Ablk[k]
    Ei = np.array([float(((A[int(i)] ** 2).sum(axis=0) * w).sum()) for i in S])
    # g on rows of FS and on their reverse edges
    eg = np.union1d(eF, csr.rev[eF].astype(np.int64))
    Ab = np.stack([2.0 * w[None, :] * A[int(i)] for i in recv_all[eg]]) if len(eg) else np.zeros((0, 16, C))
    g = M.edge_backward(dvec(eg), pairs_of(eg), h[species[csr.col[eg]]], Ab, model)
    gmap = dict(zip(eg.tolist(), range(len(eg))))
    F = np.zeros((len(FS), 3))
    for k, i in enumerate(FS):
        for e in range(rp[i], rp[i + 1]):
            F[k] += g[gmap[e]] - g[gmap[int(csr.rev[e])]]
    return dict(atoms=S, Ei=Ei, force_atoms=FS, F=F)

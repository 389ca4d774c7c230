"""Seeded synthetic inputs for the equivariant edge convolution.

This module only *draws* inputs: lattice sites, Gaussian position noise, and
random model weights.  It holds none of the method's arithmetic (no distances,
no basis, no network), so both the float64 oracle and the HIP path can take
their inputs from here without sharing any computation.

Workloads stand in for the crystal frames the pages measure on (a perturbed
carbon diamond frame at N = 64 / 512 / 4096 atoms with seed 0 and 0.02 A
noise, "deepmd-kit PR #2", Summary and "Multi-model and N4096 update"; the
ionic NaCl / NaNbO3 roles of "FastMACE rewrite screens").  No dataset or
trained weights exist here, so every value is synthetic:

* lattice: conventional cubic cell, supercell order (ix, iy, iz) cell-major
  then basis site;
* noise: N(0, 0.02^2) per Cartesian component, then wrapped into [0, L);
* weights per ordered species pair p = Z_recv * S + Z_send, drawn in float64
  and rounded to float32: W1 [32, 64] ~ N(0, 1/32), W2 [64, 64] ~ N(0, 1/64),
  W3 [64, 4C] ~ N(0, 1/64) (draw order: p ascending, then W1, W2, W3);
* species embedding h [S, C] ~ N(0, 1); readout w [C] ~ N(0, 1/C).

Independent streams come from ``numpy.random.SeedSequence(seed).spawn(4)``:
positions, radial weights, embeddings, readout.
"""
from __future__ import annotations

import dataclasses
import numpy as np

N_BASIS = 32
HIDDEN = 64
LMAX = 3
N_LM = (LMAX + 1) ** 2
CUTOFF = 6.0
NOISE = 0.02

# Fractional basis sites and species of each conventional cubic cell.
_FCC = [(0.0, 0.0, 0.0), (0.0, 0.5, 0.5), (0.5, 0.0, 0.5), (0.5, 0.5, 0.0)]
LATTICES = {
    "diamond": dict(
        a=3.567,
        sites=_FCC + [(x + 0.25, y + 0.25, z + 0.25) for (x, y, z) in _FCC],
        species=[0] * 8,
        n_species=1,
    ),
    "rocksalt": dict(
        a=5.64,
        sites=_FCC + [(x + 0.5, y, z) for (x, y, z) in _FCC],
        species=[0] * 4 + [1] * 4,
        n_species=2,
    ),
    "perovskite": dict(
        a=3.95,
        sites=[(0.0, 0.0, 0.0), (0.5, 0.5, 0.5), (0.5, 0.5, 0.0), (0.5, 0.0, 0.5), (0.0, 0.5, 0.5)],
        species=[0, 1, 2, 2, 2],
        n_species=3,
    ),
}

# name -> (lattice, repetitions per axis, channels)
CONFIGS = {
    "D64": ("diamond", 2, 64),
    "D512": ("diamond", 4, 64),
    "D4096": ("diamond", 8, 64),
    "RS": ("rocksalt", 8, 64),
    "PV": ("perovskite", 10, 64),
    "D32k": ("diamond", 16, 128),
    # small cases for tests (several tiles, ragged tails, multi-species)
    "RS2": ("rocksalt", 2, 64),
    "RS3": ("rocksalt", 3, 64),
    "PV2": ("perovskite", 2, 64),
    "PV3": ("perovskite", 3, 64),
    "D64c128": ("diamond", 2, 128),
    "D512c128": ("diamond", 4, 128),
    "D1728": ("diamond", 6, 64),
    "D1728c128": ("diamond", 6, 128),
}


@dataclasses.dataclass
class Model:
    """Random-init weights of the synthetic radial-MLP model (float32)."""

    n_species: int
    channels: int
    W1: np.ndarray  # [S*S, 32, 64]
    W2: np.ndarray  # [S*S, 64, 64]
    W3: np.ndarray  # [S*S, 64, 4*C], column l*C + c
    emb: np.ndarray  # [S, C]
    w_read: np.ndarray  # [C]
    cutoff: float = CUTOFF


@dataclasses.dataclass
class Config:
    name: str
    pos: np.ndarray  # [N, 3] float64, inside [0, L)
    species: np.ndarray  # [N] int32
    box: np.ndarray  # [3] float64
    model: Model

    @property
    def n_atoms(self) -> int:
        return int(self.pos.shape[0])


def lattice_sites(lattice: str, reps: int):
    """Perfect-crystal positions (float64) and species, cell-major order."""
    lat = LATTICES[lattice]
    a = lat["a"]
    frac = np.asarray(lat["sites"], dtype=np.float64)
    spec = np.asarray(lat["species"], dtype=np.int32)
    cells = np.array(
        [(ix, iy, iz) for ix in range(reps) for iy in range(reps) for iz in range(reps)],
        dtype=np.float64,
    )
    pos = (cells[:, None, :] + frac[None, :, :]).reshape(-1, 3) * a
    species = np.tile(spec, len(cells))
    box = np.full(3, reps * a, dtype=np.float64)
    return wrap(pos, box), species, box


def wrap(pos: np.ndarray, box: np.ndarray) -> np.ndarray:
    """Map positions into [0, L) per axis (a value that lands on L maps to 0)."""
    out = np.mod(pos, box)
    out[out >= box] = 0.0
    return out


def draw_model(n_species: int, channels: int, seed: int = 0) -> Model:
    ss = np.random.SeedSequence(seed).spawn(4)
    rng_w = np.random.default_rng(ss[1])
    P = n_species * n_species
    W1 = np.empty((P, N_BASIS, HIDDEN), np.float32)
    W2 = np.empty((P, HIDDEN, HIDDEN), np.float32)
    W3 = np.empty((P, HIDDEN, (LMAX + 1) * channels), np.float32)
    for p in range(P):
        W1[p] = rng_w.normal(0.0, np.sqrt(1.0 / N_BASIS), (N_BASIS, HIDDEN)).astype(np.float32)
        W2[p] = rng_w.normal(0.0, np.sqrt(1.0 / HIDDEN), (HIDDEN, HIDDEN)).astype(np.float32)
        W3[p] = rng_w.normal(0.0, np.sqrt(1.0 / HIDDEN), (HIDDEN, (LMAX + 1) * channels)).astype(np.float32)
    emb = np.random.default_rng(ss[2]).normal(0.0, 1.0, (n_species, channels)).astype(np.float32)
    w_read = np.random.default_rng(ss[3]).normal(0.0, np.sqrt(1.0 / channels), channels).astype(np.float32)
    return Model(n_species, channels, W1, W2, W3, emb, w_read)


def make_config(name: str, seed: int = 0, noise: float = NOISE) -> Config:
    lattice, reps, channels = CONFIGS[name]
    pos, species, box = lattice_sites(lattice, reps)
    ss = np.random.SeedSequence(seed).spawn(4)
    if noise > 0:
        pos = pos + np.random.default_rng(ss[0]).normal(0.0, noise, pos.shape)
    pos = wrap(pos, box)
    model = draw_model(LATTICES[lattice]["n_species"], channels, seed)
    return Config(name, np.ascontiguousarray(pos), species.astype(np.int32), box, model)


def make_cluster(pos, box, species=None, n_species: int = 1, channels: int = 64, seed: int = 0) -> Config:
    """Explicit positions (e.g. a dimer or trimer in a large box) with seeded weights."""
    pos = np.asarray(pos, dtype=np.float64).reshape(-1, 3)
    box = np.asarray(box, dtype=np.float64).reshape(3)
    if species is None:
        species = np.zeros(len(pos), np.int32)
    return Config("cluster", wrap(pos, box), np.asarray(species, np.int32), box,
                  draw_model(n_species, channels, seed))


def random_rotation(seed: int) -> np.ndarray:
    """Uniform random proper rotation (QR of a Gaussian matrix, sign-fixed)."""
    g = np.random.default_rng(seed).normal(size=(3, 3))
    q, r = np.linalg.qr(g)
    q = q * np.sign(np.diag(r))[None, :]
    if np.linalg.det(q) < 0:
        q[:, 0] = -q[:, 0]
    return q


# ---------------------------------------------------------------- MD motion
# A synthetic trajectory for exercising a Verlet-skin neighbour list: every
# atom moves along its own seeded straight line and back, its offset from the
# start following a triangle wave (amplitude period / 4 steps of its
# velocity), so the structure stays close to the lattice for any number of
# steps while the list still has to be rebuilt every few steps.
MD_SIGMA = 0.003  # A per step, per component
MD_PERIOD = 40  # steps


def md_velocities(n_atoms: int, seed: int = 0, sigma: float = MD_SIGMA) -> np.ndarray:
    return np.random.default_rng(np.random.SeedSequence(seed).spawn(5)[4]).normal(0.0, sigma, (n_atoms, 3))


def md_phase(step: int, period: int = MD_PERIOD) -> float:
    """Triangle wave: 0 at step 0, slope +1 then -1, extremes +-period / 4."""
    q = period / 4.0
    return q - abs(((step + q) % period) - 2.0 * q)


def md_positions(pos0: np.ndarray, vel: np.ndarray, step: int, period: int = MD_PERIOD) -> np.ndarray:
    """Unwrapped positions at `step` (the frame of pos0; not mapped into the cell)."""
    return pos0 + vel * md_phase(step, period)

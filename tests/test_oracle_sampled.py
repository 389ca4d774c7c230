"""The sampled oracle used at full size equals the full oracle (CPU only)."""
import numpy as np

import eec_inputs as I
from oracle import model as M
from oracle import neighbors as N
from oracle.sampled import sampled_energy_forces


def test_sampled_oracle_matches_full_oracle():
    # the restriction selects rows only: equal to the full oracle on a small cell
    cfg = I.make_config("PV3")
    csr = N.neighbors_celllist(cfg.pos, cfg.box, cfg.model.cutoff)
    full = M.energy_forces(cfg.pos, cfg.species, cfg.box, cfg.model, csr)
    atoms = np.array([0, 7, 50, 134])
    s = sampled_energy_forces(cfg.pos, cfg.species, cfg.box, cfg.model, csr, atoms)
    assert np.allclose(s["Ei"], full["Ei"][atoms], rtol=1e-12, atol=1e-14)
    assert np.allclose(s["F"], full["F"][atoms], rtol=1e-10, atol=1e-12)
    s2 = sampled_energy_forces(cfg.pos, cfg.species, cfg.box, cfg.model, csr, atoms, forces_for=[3])
    assert np.allclose(s2["F"][0], full["F"][3], rtol=1e-10, atol=1e-12)

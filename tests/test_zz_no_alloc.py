"""The no-allocation folded call (eec_energy_forces_folded_noalloc, scratch in
a static device array inside the library) against the workspace entry point
it mirrors (eec_energy_forces_folded), through the C ABI.

Two no-allocation calls in a row, the second on a smaller cell, so the second
call reuses scratch that holds the first call's larger contents.  Outputs
meet the parity bars against the workspace call (energy 1e-5 relative,
per-atom energy 1e-5 of the largest, forces max|dF| <= 1e-4 RMS(F), virial
1e-4 of the largest), and in fact equal it bit for bit: the same kernels run
on the same inputs in a fixed order."""
import numpy as np
import pytest

import eec_inputs as I
from equivariant_edge_convolution_amd import binding as B

from gpu_util import device_inputs, graph_for, np_, rms, say

pytestmark = pytest.mark.gpu

KEYS = ("energy", "atom_energy", "forces", "virial")


def _inputs(name):
    cfg = I.make_config(name)
    pos, species, model = device_inputs(cfg)
    return cfg, pos, species, model, graph_for(cfg, pos, species)


def _bars(got, ref):
    for k in KEYS:
        assert np.all(np.isfinite(got[k])), k
    assert abs(float(got["energy"][0]) - float(ref["energy"][0])) <= 1e-5 * abs(float(ref["energy"][0]))
    assert np.abs(got["atom_energy"] - ref["atom_energy"]).max() <= 1e-5 * np.abs(ref["atom_energy"]).max()
    assert np.abs(got["forces"] - ref["forces"]).max() <= 1e-4 * rms(ref["forces"])
    assert np.abs(got["virial"] - ref["virial"]).max() <= 1e-4 * np.abs(ref["virial"]).max()
    for k in KEYS:
        np.testing.assert_array_equal(got[k], ref[k])


@pytest.mark.parametrize("big,small", [("D4096", "D512"), ("PV3", "RS2")])
def test_noalloc_matches_folded_on_two_calls(big, small):
    cells = [_inputs(big), _inputs(small)]
    assert cells[1][4].n_edges < cells[0][4].n_edges
    refs = []
    for name, (cfg, pos, species, model, g) in zip((big, small), cells):
        say(f"[noalloc] workspace call {name}")
        out = B.energy_forces(g, pos, cfg.box, species, model, virial=True, variant="folded")
        refs.append({k: np_(v) for k, v in out.items()})
    got = []
    for name, (cfg, pos, species, model, g) in zip((big, small), cells):
        say(f"[noalloc] no-allocation call {name}")
        out = B.energy_forces_folded_noalloc(g, pos, cfg.box, species, model, virial=True)
        got.append({k: np_(v) for k, v in out.items()})
    for name, a, b in zip((big, small), got, refs):
        say(f"[noalloc] compare {name}")
        _bars(a, b)

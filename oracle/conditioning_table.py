"""Conditioning of the energy and the forces on the five benchmark workloads.

TEST INFRASTRUCTURE ONLY (oracle; never used by the product path).

Writes ``oracle/conditioning.json``: for each workload the float64 oracle's
full energy/force call and ``model.conditioning`` of it,

    kappa_E = sum_i sum_c |w_c| sum_lm A_{i,lm,c}^2 / |E|
    kappa_F = max_i sum_{e in row i} (|g_e| + |g_rev(e)|) / RMS(F)

(the float32 energy error is about eps * kappa_E relative, the float32 force
error about eps_g * kappa_F * RMS(F) / sqrt(row length)), with RMS(F), E and
the edge count.  The values are deterministic (seeded inputs); the benchmark
reports them beside its timing.  Run from the repository root:

    python -m oracle.conditioning_table [names...]
"""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import eec_inputs as I  # noqa: E402

from . import model as M  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "conditioning.json")
WORKLOADS = ("D64", "D512", "D4096", "RS", "PV", "D32k")


def table(names=WORKLOADS) -> dict:
    out = {}
    for name in names:
        cfg = I.make_config(name)
        t0 = time.perf_counter()
        ref = M.energy_forces(cfg.pos, cfg.species, cfg.box, cfg.model)
        kE, kF, rms = M.conditioning(ref, cfg.model, ref["csr"])
        out[name] = {"kappa_E": kE, "kappa_F": kF, "rms_F": rms, "E": ref["E"],
                     "n_edges": int(ref["csr"].n_edges), "oracle_s": time.perf_counter() - t0}
        print(name, out[name], flush=True)
    return out


def main(argv) -> int:
    names = tuple(argv) or WORKLOADS
    try:
        with open(OUT) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    rec.update(table(names))
    with open(OUT, "w") as f:
        json.dump({k: rec[k] for k in sorted(rec)}, f, indent=1)
        f.write("\n")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))

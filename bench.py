#!/usr/bin/env python3
"""Throughput of one energy + force call (forward + force backward, FP32) on
one MI355X, in edges per second.

Default workload: the 4096-atom carbon diamond (8 x 8 x 8 conventional cells,
a = 3.567 A, 0.02 A seeded noise, cutoff 6.0 A, E = 647,168 directed edges),
one species, 64 channels.  Inputs are synthetic and seeded (eec_inputs); the
neighbour list is built once before timing (it is timed separately and
reported as context).  Each timed step is one full energy/force call with
every input already resident in device memory: radial network + message +
readout + streaming backward + force scatter.

Before the timed calls the headline variant runs untimed for at least
--preload-ms of wall time (reported as "preload"), so that the clock has
settled under load whatever --warmup asks for; then --warmup untimed calls,
then --steps timed calls between two device synchronisations.

The headline variant (--variant, default "folded") is eec_energy_forces_folded:
the linear last radial layer applied once per receiver instead of once per
edge (same outputs up to float32 rounding).  The other variants ("direct",
eec_energy_forces: the radial weights R of every edge on matrix cores;
"tabulated": certified radial tables) are timed in the same run and reported
under "variants".

Also reported:
  roofline      the dominant kernel (one species, folded: the fused
                forward+backward kernel; otherwise the streaming backward),
                its launch duration measured with hipEvents recorded by the
                library on the stream it launches on; its algorithmic flops
                (dominant_kernel; recomputation excluded) over that duration,
                against the FP32 matrix peak; `traffic` the HBM bytes per
                launch from the recorded counter runs (recorded_traffic), or
                null when the kernel has changed since they were taken;
  call_ms       per-call device time (first to last kernel of a call, from the
                hipEvents of a second pass of --steps calls): P50, P90, mean;
  cpu_baseline  the float64 oracle on a bounded sample of the same workload
                (its first receivers: their forward and force backward), median
                of three runs on the host cores, with the CPU model and the
                BLAS threads in use, and one-thread runs on the 64-atom cell
                and a sample of the 512-atom cell;
  conditioning  kappa_E and kappa_F of the workload (oracle/conditioning.json);
  neighbors_ms  the neighbour build on its own (warm, preallocated buffers,
                its host synchronisation included; the first, cold build as
                neighbors_first_ms), and with_neighbours: a build followed by
                the call, per step.

--mode suite times every workload (64, 512, 4096-atom diamond, rocksalt,
perovskite, 32768-atom diamond at 128 channels) in ABBA order (each workload
visited twice, the second pass in reverse), one JSON line per workload with
per-call P50/P90 over both visits.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# BLAS / OpenMP threads of the CPU baseline: the cores this process may run on,
# fixed before NumPy is first imported (a count the environment already sets
# is kept).
HOST_CORES = len(os.sched_getaffinity(0))
for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_v, str(HOST_CORES))

METRIC = "edges/s fwd+force bwd, fp32, 4096-atom diamond (E≈6.5e5); % of roofline"
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
# Algorithmic flops of the backward kernel (recomputation excluded).
# direct: network input gradient 45,056 + Rbar 2,304 + Ybar 2,048 per edge.
# folded: per edge Ybar = M s2 (2,048) + s2bar = M^T Y (2,048) + W2^T (8,192)
#         + W1^T (4,096); per (receiver, sender species) unit M = Abar h W3^T
#         (2 * 16 * 64 * 64 = 131,072).
BWD_FLOP_PER_EDGE = {"direct": 45056 + 2304 + 2048, "folded": 2048 + 2048 + 8192 + 4096}
BWD_FLOP_PER_UNIT = {"direct": 0, "folded": 2 * 16 * 64 * 64}
# The one-species fused kernel (forward and backward in one launch): per edge
# the forward W1 (4,096) + W2 (8,192) + T = s2 Y^T (2,048) and the backward
# (BWD_FLOP_PER_EDGE["folded"]); per receiver M = G T through the readout's
# Gram matrices (2 * 16 * 64 * 64) and E_i = T . M / 2 (2 * 16 * 64).
FOLD_FWD_FLOP_PER_EDGE = 4096 + 8192 + 2048
FUSED_FLOP_PER_UNIT = 2 * 16 * 64 * 64 + 2 * 16 * 64
# Several species (k_fold_multi): per (receiver, sender species) unit the
# forward's A += h T^T W3 (2 * 16 * 64 * 64) and the backward's M.
FOLD_FWD_FLOP_PER_UNIT = 2 * 16 * 64 * 64
# Radial tables (k_fold_table): per edge the Horner evaluation of 64 units and
# their t-derivatives (degree 10: 2 * 64 * 10 multiply-adds), T = s2^T Y,
# Ybar = M s2, s2bar = M^T Y and rbar = s2bar . ds2/dr; per receiver as the
# fused kernel.
TAB_FLOP_PER_EDGE = 2 * (2 * 64 * 10) + 2048 + 2048 + 2048 + 2 * 64


def dominant_kernel(variant: str, n_species: int, n_edges: int, n_units: int, n_atoms: int = 1 << 30):
    """(kernel, phase whose events bracket exactly that launch, algorithmic flops per launch)."""
    if variant == "tabulated":
        return "k_fold_table", "forward", TAB_FLOP_PER_EDGE * n_edges + FUSED_FLOP_PER_UNIT * n_units
    if variant == "folded" and n_species == 1:
        flop = (FOLD_FWD_FLOP_PER_EDGE + BWD_FLOP_PER_EDGE["folded"]) * n_edges + FUSED_FLOP_PER_UNIT * n_units
        # up to 768 receivers the library gives each a workgroup (k_fold_split)
        return ("k_fold_split" if n_atoms <= 768 else "k_fold_fused"), "forward", flop
    if variant == "folded" and n_species <= 3:
        # per (receiver, sender species) unit: A += h T^T W3 and M = (dE/dA h) W3^T
        flop = ((FOLD_FWD_FLOP_PER_EDGE + BWD_FLOP_PER_EDGE["folded"]) * n_edges
                + (FOLD_FWD_FLOP_PER_UNIT + BWD_FLOP_PER_UNIT["folded"]) * n_units)
        return "k_fold_multi", "forward", flop
    flop = BWD_FLOP_PER_EDGE[variant] * n_edges + BWD_FLOP_PER_UNIT[variant] * n_units
    return ("k_backward" if variant == "direct" else "k_fold_backward"), "backward", flop


WORKLOADS = {
    "D4096": "diamond 8x8x8 conventional cells, 4096 atoms, a=3.567 A, rc=6.0 A, 0.02 A noise, seed 0, C=64",
    "D512": "diamond 4x4x4 conventional cells, 512 atoms, rc=6.0 A, C=64",
    "D64": "diamond 2x2x2 conventional cells, 64 atoms, rc=6.0 A, C=64",
    "RS": "rocksalt 8x8x8 cells, 4096 atoms, 2 species, a=5.64 A, rc=6.0 A, C=64",
    "PV": "cubic perovskite 10x10x10 cells, 5000 atoms, 3 species, a=3.95 A, rc=6.0 A, C=64",
    "D32k": "diamond 16x16x16 conventional cells, 32768 atoms, rc=6.0 A, C=128",
}
SUITE = ("D64", "D512", "D4096", "RS", "PV", "D32k")


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
CONDITIONING_FILE = os.path.join(ROOT, "oracle", "conditioning.json")


def code_text(text: str) -> str:
    """The code of a C++ source without its comments and blank space: what
    the counters depend on (a comment edit leaves a traffic record valid)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    lines = (" ".join(line.split("//", 1)[0].split()) for line in text.splitlines())
    return "\n".join(line for line in lines if line)


def sources_digest() -> str:
    """SHA-256 over the code of the kernel sources (csrc/*.hip, csrc/*.hpp,
    by name; comments and blank space excluded)."""
    import hashlib
    src = os.path.join(ROOT, "equivariant_edge_convolution_amd", "csrc")
    h = hashlib.sha256()
    for fn in sorted(os.listdir(src)):
        if fn.endswith((".hip", ".hpp")):
            h.update(fn.encode())
            with open(os.path.join(src, fn), encoding="utf-8") as f:
                h.update(code_text(f.read()).encode())
    return h.hexdigest()


def recorded_traffic(kernel: str, config_name: str):
    """HBM bytes per launch of `kernel` from the FETCH_SIZE / WRITE_SIZE
    counter runs recorded in profiles/hbm_traffic.json, scaled by the copy
    calibration there; None unless the record is for this workload and the
    kernel sources are still the ones that were counted."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("workload") != config_name or rec.get("sources_sha256") != sources_digest():
        return None
    return float(rec["bytes_per_launch"])


def conditioning(config_name: str):
    """kappa_E, kappa_F and RMS(F) of the workload from the oracle's table
    (oracle/conditioning_table.py), or None when it has no entry."""
    try:
        with open(CONDITIONING_FILE) as f:
            rec = json.load(f).get(config_name)
    except (OSError, ValueError):
        return None
    if not rec:
        return None
    return {k: rec[k] for k in ("kappa_E", "kappa_F", "rms_F")}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_threads() -> int:
    """Threads of the BLAS library NumPy loaded (what the oracle's products use)."""
    try:
        from threadpoolctl import threadpool_info
        n = [d["num_threads"] for d in threadpool_info() if d.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:  # threadpoolctl missing or unable to introspect
        return int(os.environ.get("OMP_NUM_THREADS", HOST_CORES))


def oracle_sample(cfg, n_rows: int):
    """Seconds of the oracle's forward (basis, network, harmonics, message) and
    force backward over the first n_rows receivers of a workload, and their
    edge count."""
    import numpy as np

    from oracle import model as M
    from oracle import neighbors as N

    csr = N.neighbors_celllist(cfg.pos, cfg.box, cfg.model.cutoff)
    rp = csr.row_ptr.astype(np.int64)
    n_rows = min(n_rows, cfg.n_atoms)
    e1 = int(rp[n_rows])
    recv = csr.receivers()[:e1]
    edges = np.arange(e1)
    d = (cfg.pos[csr.col[edges]] - cfg.pos[recv]) + csr.shift[edges].astype(np.float64) * cfg.box[None, :]
    pairs = cfg.species[recv].astype(np.int64) * cfg.model.n_species + cfg.species[csr.col[edges]]
    h = np.asarray(cfg.model.emb, np.float64)
    hj = h[cfg.species[csr.col[edges]]]
    w = np.asarray(cfg.model.w_read, np.float64)
    t0 = time.perf_counter()
    msg, _ = M.edge_messages(d, pairs, hj, cfg.model)
    A = np.zeros((n_rows, 16, cfg.model.channels))
    np.add.at(A, recv, msg)
    Abar = 2.0 * w[None, None, :] * A
    M.edge_backward(d, pairs, hj, Abar[recv], cfg.model)
    return time.perf_counter() - t0, e1


def cpu_baseline(cfg, n_rows: int = 1024, repeats: int = 3):
    """The oracle (as it stands) on the first n_rows receivers of the workload:
    the median of `repeats` runs with the BLAS threads set at start-up, and
    one-thread runs on the 64-atom diamond and the first 128 receivers of the
    512-atom diamond."""
    import numpy as np

    import eec_inputs as I

    runs = [oracle_sample(cfg, n_rows) for _ in range(repeats)]
    dt = float(np.median([r[0] for r in runs]))
    e1 = runs[0][1]
    one = {}
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1):
            for name, rows in (("D64", 64), ("D512", 128)):
                t, e = oracle_sample(I.make_config(name), rows)
                one[name] = {"value": e / t, "unit": "edges/s", "edges": e, "receivers": rows, "s": t}
    except ImportError:
        one = None
    return {"value": e1 / dt, "unit": "edges/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"first {min(n_rows, cfg.n_atoms)} receivers of the workload ({e1} edges): float64 "
                      f"forward (basis, network, harmonics, message) and force backward; median of "
                      f"{repeats} runs, {dt:.2f} s each",
            "runs_s": [r[0] for r in runs], "cpu_model": cpu_model(), "host_cores": HOST_CORES,
            "one_thread": one}


def copy_calibration(args, torch, dev) -> int:
    """A plain device-to-device copy of 256 MiB: 256 MiB read and 256 MiB
    written per launch, to scale the profiler's FETCH_SIZE / WRITE_SIZE."""
    n = 256 << 20
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / max(args.steps, 1)
    print(json.dumps({"mode": "copy", "bytes_read": n, "bytes_written": n, "ms": dt * 1e3,
                      "GBps": 2 * n / dt / 1e9}), flush=True)
    return 0


def message_mode(args, B, torch, cfg, g, pos, species, model, dev) -> int:
    """Time eec_edge_message: radial rows streamed chunk by chunk into the
    message pass (profile it to read the message kernel's own duration)."""
    ws = torch.empty(B.workspace_bytes(g.n_atoms, g.n_edges, model), dtype=torch.uint8, device=dev)
    A = torch.empty((g.n_atoms, 16, model.channels), dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        B.edge_message(g, pos, cfg.box, species, model, workspace=ws, out=A)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        B.edge_message(g, pos, cfg.box, species, model, workspace=ws, out=A)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / max(args.steps, 1)
    print(json.dumps({"mode": "edge_message", "config": args.config, "n_edges": g.n_edges,
                      "ms_per_call": ms, "edges_per_s": g.n_edges / (ms * 1e-3)}), flush=True)
    return 0


def md_loop(B, torch, cfg, model, dev, steps: int, skin: float, scheme: str, variant: str = "folded",
            warmup: int = 0, record: bool = False) -> dict:
    """An MD-like loop over the synthetic trajectory of eec_inputs (atoms on
    seeded straight lines and back): per step one energy/force call, with the
    neighbour list kept by one of three schemes
      "every"   rebuilt at the model cutoff before every call;
      "serial"  built with cutoff rc + skin and reused; when the skin test
                (eec_skin_check) of the previous step found an atom past the
                trigger, rebuilt on the call's stream after the step's call;
      "side"    the same decisions, the rebuild on a second stream beside the
                step's call, the next call waiting for it (an event).
    The skin test of step t is read by the host at step t + 1 (it ran before
    the call of step t), so the loop never drains the stream for it; to keep
    every list valid with that lag the trigger is skin / 2 - 2 max_i |v_i|
    (v_i the per-step motion).  Positions stay in the frame of the list they
    are used with (wrapped into the cell at each rebuild only).  The last
    `steps` of warmup + steps are timed; with `record`, each step's energy,
    forces and largest squared displacement are returned too."""
    import numpy as np

    import eec_inputs as I

    rc, n, S = cfg.model.cutoff, cfg.n_atoms, cfg.model.n_species
    species = torch.as_tensor(cfg.species).to(dev)
    x0 = torch.as_tensor(cfg.pos).to(dev)
    vel_np = I.md_velocities(n)
    vel = torch.as_tensor(vel_np).to(dev)
    Lt = torch.as_tensor(np.asarray(cfg.box, np.float64)).to(dev)
    vmax = float(np.sqrt((vel_np * vel_np).sum(axis=1)).max())
    every = scheme == "every"
    lc = rc if every else rc + skin
    trig = 0.5 * skin - 2.0 * vmax
    if not every and trig <= 0.0:
        raise ValueError(f"skin {skin} too small for a per-step motion of up to {vmax:.4f} A")

    def u(t):
        return x0 + vel * I.md_phase(t)

    def wrapped(x):
        w = torch.remainder(x, Lt)
        return torch.where(w >= Lt, w - Lt, w)

    g0 = B.build_neighbors(x0, cfg.box, lc, species, S)
    cap = int(1.25 * g0.n_edges) + 1024
    lists = [B.NeighborList(n, cfg.box, lc, cap, dev, species, S) for _ in range(2)]
    table = B.RadialTable(model, 6) if variant == "tabulated" else None
    ef = B.EnergyForces(g0, model, dev, atom_energy=False, variant=variant, edge_capacity=cap, table=table)
    main = torch.cuda.current_stream(dev)
    side = torch.cuda.Stream(device=dev) if scheme == "side" else None
    total = warmup + steps
    m2 = torch.zeros(total, dtype=torch.float64, device=dev)
    flag = torch.zeros(total, dtype=torch.int32, device=dev)
    flag_h = torch.zeros(total, dtype=torch.int32, pin_memory=True)
    checked = [None] * total
    rec_E, rec_F = [], []
    ref = x0
    off = torch.zeros_like(x0)
    cur, nxt = lists[0].build(x0), 1
    valid_from, rebuilds, edges = 0, 0, 0
    t0 = None
    for t in range(total):
        if t == warmup:
            torch.cuda.synchronize()
            t0, rebuilds, edges = time.perf_counter(), 0, 0
        ut = u(t)
        if every:
            pos_t = wrapped(ut)
            cur = lists[nxt].build(pos_t)
            nxt ^= 1
            rebuilds += 1
        else:
            pos_t = ut - off
            B.skin_check(pos_t, ref, trig, out=(m2[t:t + 1], flag[t:t + 1]))
            flag_h[t:t + 1].copy_(flag[t:t + 1], non_blocking=True)
            checked[t] = torch.cuda.Event()
            checked[t].record(main)
        rebuild = False
        if not every and t - 1 >= valid_from:
            checked[t - 1].synchronize()
            rebuild = bool(flag_h[t - 1])
        if rebuild:
            w = wrapped(ut)
            if side is not None:
                ready = torch.cuda.Event()
                ready.record(main)
        ef(pos_t, cfg.box, species, graph=cur)
        edges += cur.n_edges
        if record:
            rec_E.append(ef.energy.clone())
            rec_F.append(ef.forces.clone())
        if rebuild:
            if side is not None:
                with torch.cuda.stream(side):
                    side.wait_event(ready)
                    cur = lists[nxt].build(w)
                    built = torch.cuda.Event()
                    built.record(side)
                main.wait_event(built)
            else:
                cur = lists[nxt].build(w)
            nxt ^= 1
            ref, off = w, ut - w
            valid_from = t + 1
            rebuilds += 1
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    out = {"scheme": scheme, "skin": 0.0 if every else skin, "list_cutoff": lc, "ms_per_step": dt * 1e3 / steps,
           "rebuilds": rebuilds, "mean_edges": edges / steps, "trigger": None if every else trig,
           "max_step_motion": vmax}
    if record:
        out["E"] = [float(e.cpu()[0]) for e in rec_E]
        out["F"] = [f.cpu().numpy() for f in rec_F]
        out["max_r2"] = m2.cpu().numpy()
    return out


def md_mode(args, B, torch, cfg, model, dev) -> int:
    """Time the MD-like loop (md_loop) under its three list schemes."""
    res = {}
    for scheme in ("every", "serial", "side"):
        r = md_loop(B, torch, cfg, model, dev, args.steps, args.skin, scheme, args.variant, warmup=args.warmup)
        res[scheme] = r
        print(json.dumps({"mode": "md", "config": args.config, **r}), flush=True)
    call = res["serial"]
    print(json.dumps({"mode": "md_summary", "config": args.config, "variant": args.variant,
                      "skin": args.skin, "steps": args.steps, "warmup": args.warmup,
                      "ms_per_step": {k: v["ms_per_step"] for k, v in res.items()},
                      "steps_per_rebuild": args.steps / max(call["rebuilds"], 1),
                      "side_over_serial": res["side"]["ms_per_step"] / call["ms_per_step"]}), flush=True)
    return 0


class Workload:
    """One workload on the device: inputs, model, neighbour list and the
    number of (receiver, sender species) units with at least one edge."""

    def __init__(self, B, torch, name: str, dev):
        import numpy as np

        import eec_inputs as I

        self.name = name
        self.cfg = cfg = I.make_config(name)
        self.pos = torch.as_tensor(cfg.pos).to(dev)
        self.species = torch.as_tensor(cfg.species).to(dev)
        self.model = B.Model.from_arrays(cfg.model, dev)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        self.g = B.build_neighbors(self.pos, cfg.box, cfg.model.cutoff, self.species, cfg.model.n_species)
        torch.cuda.synchronize()
        self.nb_first_ms = (time.perf_counter() - t0) * 1e3
        self.E = self.g.n_edges
        rp = self.g.row_ptr.cpu().numpy()
        if cfg.model.n_species == 1:
            self.n_units = int(np.count_nonzero(np.diff(rp)))
        else:
            col = self.g.col.cpu().numpy()
            recv = np.repeat(np.arange(self.g.n_atoms), np.diff(rp))
            self.n_units = len(np.unique(recv.astype(np.int64) * cfg.model.n_species + cfg.species[col]))
        self.table = None

    def radial_table(self, B):
        if self.table is None:
            self.table = B.RadialTable(self.model, 6)
        return self.table

    def energy_forces(self, B, variant: str, dev):
        return B.EnergyForces(self.g, self.model, dev, atom_energy=True, variant=variant,
                              table=self.radial_table(B) if variant == "tabulated" else None)

    def dominant(self, variant: str):
        c = self.cfg
        return dominant_kernel(variant, c.model.n_species, self.E, self.n_units, c.n_atoms)


def preload(torch, ef, w, min_ms: float) -> dict:
    """Untimed calls until at least min_ms of wall time has passed (the clock
    settles under sustained load), then a device synchronisation."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(8):
            ef(w.pos, w.cfg.box, w.species)
        n += 8
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= min_ms:
            break
    return {"ms": (time.perf_counter() - t0) * 1e3, "calls": n}


def timed(B, torch, w, ef, variant: str, steps: int, warmup: int) -> dict:
    """Timed region: `steps` calls between two device synchronisations, with
    hipEvents around the dominant kernel's launch only.  Then the same number
    of calls with every phase recorded (phases_ms and the per-call device time
    call_ms, first to last kernel of a call; not part of the timed figure)."""
    import numpy as np

    nph = len(B.PHASES)
    _, dom_phase, _ = w.dominant(variant)
    dp = B.PHASES.index(dom_phase)
    steps = max(steps, 1)
    ev = B.HipEvents(2 * nph * steps)
    for _ in range(warmup):
        ef(w.pos, w.cfg.box, w.species)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        handles = [None] * (2 * nph)
        handles[2 * dp], handles[2 * dp + 1] = ev.handles[2 * k], ev.handles[2 * k + 1]
        ef(w.pos, w.cfg.box, w.species, events=handles)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    dom = [ev.elapsed_ms(2 * k, 2 * k + 1) for k in range(steps)]
    for k in range(steps):
        ef(w.pos, w.cfg.box, w.species, events=ev.handles[2 * nph * k: 2 * nph * (k + 1)])
    torch.cuda.synchronize()
    phase_ms = {}
    for p, name in enumerate(B.PHASES):
        phase_ms[name] = float(np.mean([ev.elapsed_ms(2 * nph * k + 2 * p, 2 * nph * k + 2 * p + 1)
                                        for k in range(steps)]))
    calls = [ev.elapsed_ms(2 * nph * k, 2 * nph * k + 2 * nph - 1) for k in range(steps)]
    ev.close()
    return {"ms_per_step": dt * 1e3 / steps, "phases_ms": phase_ms, "energy": float(ef.energy.cpu()[0]),
            "dom_ms": float(np.mean(dom)), "dom_p50_ms": float(np.median(dom)), "call_samples": calls}


def pct(x, q):
    import numpy as np
    return float(np.percentile(np.asarray(x, np.float64), q))


def roofline(w, variant: str, launch_ms: float) -> dict:
    kernel, _, flop = w.dominant(variant)
    achieved = flop / (launch_ms * 1e-3) / 1e12
    return {"bound": "mfma", "kernel": kernel, "achieved": achieved, "peak": PEAK_FP32_MFMA_TFLOPS,
            "unit": "TFLOP/s", "frac": achieved / PEAK_FP32_MFMA_TFLOPS,
            "traffic": recorded_traffic(kernel, w.name), "flop_per_launch": flop, "launch_ms": launch_ms}


def suite_mode(args, B, torch, dev) -> int:
    """Every workload, ABBA order, the headline variant: per workload the
    per-call device time (P50, P90) over both visits and the dominant kernel's
    roofline fraction."""
    import numpy as np

    order = list(SUITE) + list(reversed(SUITE))
    res = {n: {"calls": [], "ms": [], "dom": []} for n in SUITE}
    loaded = {}
    for name in order:
        if name not in loaded:
            w = Workload(B, torch, name, dev)
            loaded[name] = (w, w.energy_forces(B, args.variant, dev))
        w, ef = loaded[name]
        pre = preload(torch, ef, w, args.preload_ms)
        r = timed(B, torch, w, ef, args.variant, args.steps, args.warmup)
        res[name]["calls"] += r["call_samples"]
        res[name]["ms"].append(r["ms_per_step"])
        res[name]["dom"].append(r["dom_ms"])
        res[name]["preload"] = pre
        res[name]["phases_ms"] = r["phases_ms"]
        print(json.dumps({"mode": "suite_visit", "config": name, "ms_per_step": r["ms_per_step"],
                          "dom_ms": r["dom_ms"]}), flush=True)
    for name in SUITE:
        w, _ = loaded[name]
        rr = res[name]
        ms = float(np.mean(rr["ms"]))
        dom = float(np.mean(rr["dom"]))
        print(json.dumps({"mode": "suite", "config": name, "workload": WORKLOADS[name], "variant": args.variant,
                          "n_atoms": w.cfg.n_atoms, "n_edges": w.E, "ms_per_step": ms, "edges_per_s": w.E / (ms * 1e-3),
                          "call_ms": {"p50": pct(rr["calls"], 50), "p90": pct(rr["calls"], 90),
                                      "n": len(rr["calls"])},
                          "phases_ms": rr["phases_ms"], "roofline": roofline(w, args.variant, dom),
                          "conditioning": conditioning(name), "preload": rr["preload"]}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200, help="untimed calls after the pre-load")
    ap.add_argument("--preload-ms", type=float, default=1000.0,
                    help="untimed calls of the headline variant for at least this much wall time before "
                         "the warm-up (the clock needs sustained load to settle); reported as `preload`")
    ap.add_argument("--config", default="D4096", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-variant", action="store_true",
                    help="time only --variant (for profiler runs that should see one kernel family)")
    ap.add_argument("--variant", default="folded", choices=["direct", "folded", "tabulated"],
                    help="direct: the radial weights R of every edge (eec_energy_forces); folded: the "
                         "last radial layer moved past the edge sum (eec_energy_forces_folded); "
                         "tabulated: s2 and ds2/dr from certified radial tables "
                         "(eec_energy_forces_tabulated, approximate, one to three species)")
    ap.add_argument("--mode", default="energy_forces",
                    choices=["energy_forces", "suite", "edge_message", "copy", "md"],
                    help="energy_forces: the headline call; suite: every workload in ABBA order; "
                         "edge_message: the chunked streaming forward (radial rows + message pass), for "
                         "profiling its kernels; copy: a plain 256 MiB device copy, the calibration of the "
                         "HBM byte counters; md: an MD-like loop with a Verlet-skin neighbour list, rebuilt "
                         "serially or on a side stream, against a rebuild before every call")
    ap.add_argument("--skin", type=float, default=0.2, help="Verlet skin of --mode md, A")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the single-GPU figure is the workload's throughput)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import eec_inputs as I
    from equivariant_edge_convolution_amd import binding as B

    dev = torch.device("cuda:0")
    if args.mode == "copy":
        return copy_calibration(args, torch, dev)
    if args.mode == "suite":
        return suite_mode(args, B, torch, dev)
    cfg = I.make_config(args.config)
    if args.mode == "md":
        return md_mode(args, B, torch, cfg, B.Model.from_arrays(cfg.model, dev), dev)

    w = Workload(B, torch, args.config, dev)
    if args.mode == "edge_message":
        return message_mode(args, B, torch, cfg, w.g, w.pos, w.species, w.model, dev)
    E = w.E
    ef = w.energy_forces(B, args.variant, dev)
    pre = preload(torch, ef, w, args.preload_ms)
    head = timed(B, torch, w, ef, args.variant, args.steps, args.warmup)
    others = [v for v in ("folded", "direct", "tabulated") if v != args.variant
              and (v != "tabulated" or cfg.model.n_species <= 3)]
    other_res = {}
    if not args.no_other_variant:
        for other in others:
            ef_o = w.energy_forces(B, other, dev)
            other_res[other] = timed(B, torch, w, ef_o, other, max(args.steps // 2, 1), max(args.warmup // 2, 1))

    # the neighbour build timed on its own (warm, into preallocated buffers,
    # host synchronisation included), and build + call per step
    nl = B.NeighborList(cfg.n_atoms, cfg.box, cfg.model.cutoff, E + 1024, dev, w.species, cfg.model.n_species)
    for _ in range(5):
        nl.build(w.pos)
    nb_times = []
    for _ in range(20):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        nl.build(w.pos)
        torch.cuda.synchronize()
        nb_times.append((time.perf_counter() - t0) * 1e3)
    nb_warm_ms = float(np.median(nb_times))
    n_with = max(args.steps // 4, 10)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n_with):
        ef(w.pos, cfg.box, w.species, graph=nl.build(w.pos))
    torch.cuda.synchronize()
    with_ms = (time.perf_counter() - t0) * 1e3 / n_with

    ms_per_step = head["ms_per_step"]
    calls = head["call_samples"]
    out = {
        "metric": METRIC,
        "value": E / (ms_per_step * 1e-3),
        "unit": "edges/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": WORKLOADS[args.config], "name": args.config, "n_atoms": cfg.n_atoms,
                   "n_edges": E, "channels": cfg.model.channels, "n_species": cfg.model.n_species},
        "roofline": roofline(w, args.variant, head["dom_ms"]),
        "variant": args.variant,
        "preload": pre,
        "call_ms": {"p50": pct(calls, 50), "p90": pct(calls, 90), "mean": float(np.mean(calls)), "n": len(calls),
                    "kernel_p50": head["dom_p50_ms"]},
        "variants": {
            other: {"ms_per_step": r["ms_per_step"], "value": E / (r["ms_per_step"] * 1e-3),
                    "phases_ms": r["phases_ms"], "energy": r["energy"],
                    "call_ms": {"p50": pct(r["call_samples"], 50), "p90": pct(r["call_samples"], 90)},
                    "roofline_kernel": w.dominant(other)[0], "kernel_ms": r["dom_ms"],
                    "roofline_frac": roofline(w, other, r["dom_ms"])["frac"],
                    **({"table_certificate": [float(x) for x in w.table.certificate.cpu()], "approximate": True}
                       if other == "tabulated" else {})}
            for other, r in other_res.items()},
        "phases_ms": head["phases_ms"],
        "neighbors_ms": nb_warm_ms,
        "neighbors_first_ms": w.nb_first_ms,
        "with_neighbours": {"ms_per_step": with_ms, "value": E / (with_ms * 1e-3), "steps": n_with},
        "energy": head["energy"],
        "conditioning": conditioning(args.config),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

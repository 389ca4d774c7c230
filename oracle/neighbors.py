"""Periodic neighbour list of an orthorhombic cell, as receiver-sorted CSR.

TEST INFRASTRUCTURE ONLY (float64 oracle; never used by the product path).

Follows the edge set every page on the subject convolves over: all directed
pairs (i, j) of atoms closer than the cutoff, periodic images included
("deepmd-kit PR #2", Summary: the N64 diamond frame with E ~ 10,114 edges;
"FastMACE rewrite screens", OPT2-T04 overlap_rebuild and the skin/edge-bucket
row of the research-engine table: the list is rebuilt in the MD loop beside the
force call).  The pages fix neither the tie rule, the order, nor the image
convention; the plain reading used here is:

* box orthorhombic, periodic, every side L_k >= rc, so image shifts
  n in {-1, 0, 1}^3 suffice;
* d = (x_j - x_i) + n * L per component in IEEE binary64, in that order;
  r2 = (dx*dx + dy*dy) + dz*dz with no fused multiply-add;
* keep (i, j, n) iff r2 < rc*rc (strict) and not (j == i and n == 0);
  several images of the same j are separate edges;
* rows ordered by receiver i; inside a row by (j, nx, ny, nz) ascending;
* rev(e) = index of (j, i, -n); it exists because d_rev == -d_e bitwise.

Pins: brute force == cell list exactly; perfect-lattice shell counts;
rev(rev(e)) == e; d_rev == -d bitwise; in-degree == out-degree; the pages'
printed diamond edge counts (tests/golden/pages_edge_counts.json).
"""
from __future__ import annotations

import dataclasses
import math
import numpy as np

# shift index s = (nx+1)*9 + (ny+1)*3 + (nz+1); ascending s == lexicographic (nx, ny, nz)
SHIFTS = np.array([(a, b, c) for a in (-1, 0, 1) for b in (-1, 0, 1) for c in (-1, 0, 1)], dtype=np.int64)


@dataclasses.dataclass
class CSR:
    row_ptr: np.ndarray  # [N+1] int32
    col: np.ndarray  # [E] int32 (sender j)
    shift: np.ndarray  # [E, 3] int8 (image n)
    rev: np.ndarray  # [E] int32

    @property
    def n_edges(self) -> int:
        return int(self.col.shape[0])

    def receivers(self) -> np.ndarray:
        n = self.row_ptr.shape[0] - 1
        return np.repeat(np.arange(n, dtype=np.int64), np.diff(self.row_ptr.astype(np.int64)))


def check_box(pos: np.ndarray, box: np.ndarray, rc: float) -> None:
    """Raise on the conditions the library reports as errors."""
    box = np.asarray(box, np.float64)
    if box.shape != (3,) or not np.all(np.isfinite(box)) or np.any(box <= 0) or np.any(box < rc):
        raise ValueError("box must be orthorhombic with every side >= cutoff")
    if not np.all(np.isfinite(pos)):
        raise ValueError("non-finite position")
    if np.any(pos < 0) or np.any(pos >= box[None, :]):
        raise ValueError("position outside [0, L)")


def _edge_disp(pos, box, i, j, s):
    """d = (x_j - x_i) + n*L, component-wise binary64 in exactly this order."""
    return (pos[j] - pos[i]) + SHIFTS[s].astype(np.float64) * box[None, :]


def _r2(d):
    return (d[:, 0] * d[:, 0] + d[:, 1] * d[:, 1]) + d[:, 2] * d[:, 2]


def _finish(n_atoms: int, recv: np.ndarray, keys: np.ndarray) -> CSR:
    """Sort candidate edges by (i, j, shift) and attach the reverse-edge index."""
    order = np.lexsort((keys, recv))
    recv = recv[order]
    keys = keys[order]
    col = (keys // 27).astype(np.int64)
    s = (keys % 27).astype(np.int64)
    counts = np.bincount(recv, minlength=n_atoms)
    row_ptr = np.zeros(n_atoms + 1, np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    # global key (i, j, s) is strictly increasing along the CSR
    gkey = (recv * n_atoms + col) * 27 + s
    rev_s = 26 - s  # index of -n
    rkey = (col * n_atoms + recv) * 27 + rev_s
    rev = np.searchsorted(gkey, rkey)
    if np.any(rev >= len(gkey)) or np.any(gkey[np.minimum(rev, len(gkey) - 1)] != rkey):
        raise AssertionError("reverse edge missing")
    return CSR(row_ptr.astype(np.int32), col.astype(np.int32), SHIFTS[s].astype(np.int8), rev.astype(np.int32))


def neighbors_bruteforce(pos: np.ndarray, box: np.ndarray, rc: float, rows=None) -> CSR:
    """O(N^2 * 27) definition: test every (i, j, n).

    ``rows`` restricts the receivers (for spot checks on large cells); the
    result then only holds those rows and has no valid ``rev``.
    """
    pos = np.asarray(pos, np.float64)
    box = np.asarray(box, np.float64)
    check_box(pos, box, rc)
    n = len(pos)
    rc2 = rc * rc
    recv_all, key_all = [], []
    jj = np.repeat(np.arange(n), 27)
    ss = np.tile(np.arange(27), n)
    for i in (range(n) if rows is None else rows):
        d = _edge_disp(pos, box, np.full(len(jj), i), jj, ss)
        keep = _r2(d) < rc2
        keep &= ~((jj == i) & (ss == 13))
        recv_all.append(np.full(int(keep.sum()), i, np.int64))
        key_all.append(jj[keep] * 27 + ss[keep])
    recv = np.concatenate(recv_all) if recv_all else np.zeros(0, np.int64)
    keys = np.concatenate(key_all) if key_all else np.zeros(0, np.int64)
    if rows is not None:
        order = np.lexsort((keys, recv))
        return recv[order], keys[order]
    return _finish(n, recv, keys)


def cell_grid(box: np.ndarray, rc: float) -> np.ndarray:
    """Cells per axis: the largest count whose side still exceeds rc by a margin."""
    return np.maximum(1, np.floor(np.asarray(box) / (rc * (1.0 + 1e-9))).astype(np.int64))


def neighbors_celllist(pos: np.ndarray, box: np.ndarray, rc: float) -> CSR:
    """Cell list: bin atoms into cells of side >= rc, test the 27 neighbour
    (cell, image) pairs of each atom's cell.  Same edge set as brute force."""
    pos = np.asarray(pos, np.float64)
    box = np.asarray(box, np.float64)
    check_box(pos, box, rc)
    n = len(pos)
    rc2 = rc * rc
    nc = cell_grid(box, rc)
    cidx = np.minimum((pos * (nc / box)[None, :]).astype(np.int64), nc - 1)
    flat = (cidx[:, 0] * nc[1] + cidx[:, 1]) * nc[2] + cidx[:, 2]
    order = np.argsort(flat, kind="stable")
    start = np.searchsorted(flat[order], np.arange(nc.prod() + 1))
    recv_all, key_all = [], []
    for c0 in range(nc[0]):
        for c1 in range(nc[1]):
            for c2 in range(nc[2]):
                home = (c0 * nc[1] + c1) * nc[2] + c2
                ia = order[start[home]:start[home + 1]]
                if len(ia) == 0:
                    continue
                for o in SHIFTS:
                    v = np.array([c0, c1, c2]) + o
                    img = np.floor_divide(v, nc)  # image shift n
                    w = v - img * nc
                    other = (w[0] * nc[1] + w[1]) * nc[2] + w[2]
                    ja = order[start[other]:start[other + 1]]
                    if len(ja) == 0:
                        continue
                    s = int((img[0] + 1) * 9 + (img[1] + 1) * 3 + (img[2] + 1))
                    I = np.repeat(ia, len(ja))
                    J = np.tile(ja, len(ia))
                    d = (pos[J] - pos[I]) + img.astype(np.float64)[None, :] * box[None, :]
                    keep = _r2(d) < rc2
                    if s == 13:
                        keep &= I != J
                    recv_all.append(I[keep])
                    key_all.append(J[keep] * 27 + s)
    recv = np.concatenate(recv_all) if recv_all else np.zeros(0, np.int64)
    keys = np.concatenate(key_all) if key_all else np.zeros(0, np.int64)
    return _finish(n, recv.astype(np.int64), keys.astype(np.int64))


def edge_vectors(pos: np.ndarray, box: np.ndarray, csr: CSR) -> np.ndarray:
    """d_e = (x_j - x_i) + n*L in binary64 (same operation order as the test)."""
    recv = csr.receivers()
    return (pos[csr.col] - pos[recv]) + csr.shift.astype(np.float64) * np.asarray(box)[None, :]


def max_displacement2(pos: np.ndarray, ref: np.ndarray) -> float:
    """Largest squared displacement of any atom since the list was built:
    max_i (dx*dx + dy*dy) + dz*dz with d = pos_i - ref_i in binary64, no fused
    multiply-add, no minimum image (the list's image shifts refer to the frame
    of ``ref``, so an atom wrapped back into the cell must show as moved);
    +inf if any displacement is not a number; 0.0 for no atoms.

    Verlet skin of an MD loop that reuses its list between rebuilds ("FastMACE
    rewrite screens", OPT2-T04 overlap_rebuild; the research-engine table's
    row on a 0.2 A skin)."""
    pos = np.asarray(pos, np.float64)
    ref = np.asarray(ref, np.float64)
    if pos.shape[0] == 0:
        return 0.0
    d = pos - ref
    r2 = (d[:, 0] * d[:, 0] + d[:, 1] * d[:, 1]) + d[:, 2] * d[:, 2]
    if np.any(np.isnan(r2)):
        return math.inf
    return float(r2.max())


def needs_rebuild(pos: np.ndarray, ref: np.ndarray, half_skin: float) -> bool:
    """True iff some atom moved farther than half the skin: a list built with
    cutoff rc + skin at ``ref`` then may miss a pair closer than rc (two atoms
    approaching each other head-on close the gap by twice the displacement)."""
    hs = float(half_skin)
    return max_displacement2(pos, ref) > hs * hs

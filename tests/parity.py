"""GPU <-> oracle comparison helpers (test infrastructure).

Several results of the method are equally correct where a rounding decision
sits exactly on a tie, so code parity is judged as follows, using only the
oracle's own pre-rounding values:

* at most ``max_frac`` of the codes may differ;
* in every row, the first differing code must sit on a tie of the oracle:
  the code's own pre-rounding value (w/s, or (w+M)/S) within ``tau`` code
  units of a half-integer (weight tie), or the group's zero point (affine) /
  the sub-block's scale or min code (two-level grid) within ``tau`` of a
  half-integer (grid tie);
* later differences in that row are the tie's cascade (the compensation
  carries the other choice forward) and are accepted;
* every difference is one code step (|dq| = 1).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

import oracle as O


def rel_fro(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def near_half(x, tau) -> np.ndarray:
    x = np.asarray(x, np.float64)
    return np.abs(x - np.floor(x) - 0.5) < tau


@dataclass
class CodeReport:
    n: int
    mismatches: int
    rows_with_mismatch: int
    unclassified: list
    max_step: int

    @property
    def frac(self):
        return self.mismatches / max(self.n, 1)


def classify_codes(q_gpu_p: np.ndarray, orc: "O.SweepResult", grid: str, group: int,
                   tau: float = 1e-3, search_tau: float = 1e-9) -> CodeReport:
    """q_gpu_p: GPU codes in processing order (rows x d).  With the weighted
    grid search, a group whose best and next-best candidate errors lie within
    ``search_tau`` (relative) of each other is a grid tie too."""
    qo = orc.q.astype(np.int64)
    qg = q_gpu_p.astype(np.int64)
    diff = qg != qo
    unclassified = []
    search_rows = []
    rows = np.nonzero(diff.any(axis=1))[0]
    for r in rows:
        j0 = int(np.argmax(diff[r]))
        tie = bool(near_half(orc.ratio[r, j0], tau))
        if grid == "affine":
            g = j0 // group
            tie = tie or bool(near_half(orc.zratio[r, g], tau))
            if orc.sgap is not None and orc.sgap[r, g] < search_tau:
                # the weighted search's two best scales are equally good: either
                # choice is the method's result, and codes may then differ by
                # more than one step in that row
                tie = True
                search_rows.append(int(r))
        else:
            sb = j0 // O.Q4K_SUPER
            subs = slice(sb * 8, sb * 8 + 8)
            tie = tie or bool(near_half(orc.zratio[r, subs], tau).any()) \
                or bool(near_half(orc.mratio[r, subs], tau).any())
            if orc.sgap is not None and (orc.sgap[r, subs] < search_tau).any():
                tie = True
                search_rows.append(int(r))
        if not tie:
            unclassified.append((int(r), j0, float(orc.ratio[r, j0]), int(qo[r, j0]),
                                 int(qg[r, j0])))
    keep = np.ones(qo.shape[0], bool)
    keep[search_rows] = False
    step = int(np.abs(qg - qo)[keep].max()) if diff[keep].any() else 0
    return CodeReport(n=qo.size, mismatches=int(diff.sum()), rows_with_mismatch=len(rows),
                      unclassified=unclassified, max_step=step)


def cascade_mask(q_gpu_p: np.ndarray, orc: "O.SweepResult", span: int) -> np.ndarray:
    """Groups (rows x d/span) at or after the first differing code of their
    row: there both sides follow different, equally valid, tie decisions, so
    their grids are compared only for validity, not for equality."""
    diff = q_gpu_p.astype(np.int64) != orc.q.astype(np.int64)
    r, d = diff.shape
    first = np.where(diff.any(axis=1), np.argmax(diff, axis=1), d)
    g = np.arange(d // span)[None, :]
    return g >= (first // span)[:, None]


def assert_codes(rep: CodeReport, max_frac: float = 1e-3):
    assert rep.frac <= max_frac, f"{rep.mismatches}/{rep.n} codes differ"
    assert not rep.unclassified, f"mismatches not at a tie: {rep.unclassified[:5]}"
    assert rep.max_step <= 1, f"a code differs by {rep.max_step} steps"

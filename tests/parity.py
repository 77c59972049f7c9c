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


def assert_codes(rep: CodeReport, max_frac: float = 1e-3, max_step: int = 1):
    assert rep.frac <= max_frac, f"{rep.mismatches}/{rep.n} codes differ"
    assert not rep.unclassified, f"mismatches not at a tie: {rep.unclassified[:5]}"
    assert rep.max_step <= max_step, f"a code differs by {rep.max_step} steps"


# --------------------------------------------------------------------------
# Tie-forced replay.  The oracle sweeps the same weights again and, wherever
# its own pre-rounding value sits within tau of a rounding boundary and the
# GPU took the other side, adopts the GPU's decision (either one satisfies
# the method).  Both sides then follow the same decisions, so every code,
# zero point and grid code must agree exactly afterwards; a difference that
# is not at a tie is a bug, wherever in the row it happens.
# --------------------------------------------------------------------------
def _other_side(pre):
    """+1 where rint(pre) rounded down, -1 where it rounded up."""
    pre = np.asarray(pre, np.float64)
    return np.where(np.rint(pre) == np.floor(pre), 1.0, -1.0)


@dataclass
class ReplayReport:
    n: int                       # codes compared
    forced: dict                 # decision name -> GPU decisions adopted at a tie
    bad: list                    # (name, col, row, pre, oracle, gpu): differs off a tie
    sweep: "O.SweepResult"       # the oracle's sweep with those decisions adopted
    search_ties: int = 0         # two-level search ties adopted for a whole super-block

    @property
    def forced_total(self) -> int:
        return int(sum(self.forced.values()))


class _Adopt:
    def __init__(self, spec: "O.GridSpec", q_p, grid: dict, tau, tau_half, search_tau):
        self.spec = spec
        self.q = np.asarray(q_p).astype(np.float32)
        self.g = {k: np.asarray(v) for k, v in grid.items()}
        self.tau, self.tau_half, self.search_tau = tau, tau_half, search_tau
        rows, d = self.q.shape
        self.stie = np.zeros((rows, max(d // O.Q4K_SUPER, 1)), bool)
        self.forced = {}
        self.bad = []
        self.search_ties = 0

    def _count(self, name, k):
        if k:
            self.forced[name] = self.forced.get(name, 0) + int(k)

    def _report(self, name, j, mask, pre, val, g):
        for idx in zip(*np.nonzero(mask)):
            r = int(idx[0])
            self.bad.append((name, j, r, float(np.asarray(pre)[idx]), float(np.asarray(val)[idx]),
                             float(np.asarray(g)[idx])))

    def _integer(self, name, j, pre, val, g, wholesale=None):
        val = np.asarray(val, np.float32).copy()
        g = np.asarray(g, np.float32)
        mism = g != val
        if wholesale is not None:         # two-level search tie: take the GPU's
            take = mism & wholesale
            val[take] = g[take]
            self._count(name + " (search tie)", take.sum())
            mism &= ~wholesale
        if not mism.any():
            return val
        with np.errstate(invalid="ignore"):
            tie = near_half(pre, self.tau) & (g == val + _other_side(pre))
        ok = mism & tie
        val[ok] = g[ok]
        self._count(name, ok.sum())
        self._report(name, j, mism & ~tie, pre, val, g)
        return val

    def _half(self, name, j, pre, val, g, wholesale):
        val = np.asarray(val, np.float16).copy()
        g = np.asarray(g, np.float16)
        mism = g != val
        take = mism & wholesale
        val[take] = g[take]
        self._count(name + " (search tie)", take.sum())
        mism &= ~wholesale
        if not mism.any():
            return val
        x = np.asarray(pre, np.float64)
        v64, g64 = val.astype(np.float64), g.astype(np.float64)
        adjacent = np.nextafter(val, g) == g
        between = (x - v64) * (x - g64) <= 0
        mid = 0.5 * (v64 + g64)
        tie = adjacent & between & (np.abs(x - mid) <= self.tau_half * np.abs(x))
        ok = mism & tie
        val[ok] = g[ok]
        self._count(name, ok.sum())
        self._report(name, j, mism & ~tie, pre, val, g)
        return val

    def __call__(self, name, j, pre, val):
        sp = self.spec
        if name == "code":
            whole = self.stie[:, j // O.Q4K_SUPER] if sp.grid == "q4k" else None
            return self._integer("code", j, pre, val, self.q[:, j], whole)
        if name == "zero":
            return self._integer("zero", j, pre, val, self.g["zero"][:, j // sp.group])
        if name in ("D", "Dm"):
            sb = j // O.Q4K_SUPER
            return self._half(name, j, pre, val, self.g[name][:, sb], self.stie[:, sb])
        if name in ("sc", "mc"):
            sb = j // O.Q4K_SUPER
            b0 = j // O.Q4K_SUB
            g = self.g[name][:, b0:b0 + O.Q4K_SUPER // O.Q4K_SUB]
            whole = np.repeat(self.stie[:, sb:sb + 1], g.shape[1], axis=1)
            return self._integer(name, j, pre, val, g, whole)
        if name == "search":
            return self._search(j, pre, val)
        raise ValueError(name)

    def _search(self, j, pre, best):
        best = np.array(best)
        if self.spec.grid == "affine":
            E, cand = pre
            g = self.g["scale"][:, j // self.spec.group].astype(np.float64)
            r = np.arange(E.shape[1])
            s_or = cand[best, r].astype(np.float64)
            for i in np.nonzero(np.abs(g - s_or) > 1e-3 * s_or)[0]:
                close = np.nonzero(np.abs(cand[:, i] - g[i]) <= 1e-3 * g[i])[0]
                e0 = E[best[i], i]
                k = [c for c in close if E[c, i] - e0 <= self.search_tau * max(e0, 1e-300)]
                if k:
                    best[i] = k[0]
                    self._count("search", 1)
                else:
                    self.bad.append(("search", j, int(i), float(e0), float(s_or[i]), float(g[i])))
            return best
        # two-level grid: a sub-block's (scale, min) is not an output, so a
        # row's super-block whose choice is a tie is taken from the GPU whole
        E = pre[0]
        Es = np.sort(E, axis=0)
        with np.errstate(divide="ignore", invalid="ignore"):
            gap = np.where(Es[0] > 0, (Es[1] - Es[0]) / Es[0], np.where(Es[1] > 0, np.inf, 0.0))
        tie_rows = (gap < self.search_tau).any(axis=1)
        self.stie[:, j // O.Q4K_SUPER] |= tie_rows
        self.search_ties += int(tie_rows.sum())
        return best


def replay_ties(Wp, U, spec: "O.GridSpec", q_p, grid: dict, importance=None,
                tau: float = 1e-3, tau_half: float = 1e-4,
                search_tau: float = 1e-9) -> ReplayReport:
    """Tie-forced replay of the plain (unblocked) oracle sweep.

    Wp: weights in processing order (dead columns zeroed), U: the oracle's
    factor, q_p: the GPU's codes in processing order, grid: the GPU's grid in
    processing order ({"scale", "zero"} for the affine grid; {"D", "Dm",
    "sc", "mc"} for the two-level grid).  A GPU decision is adopted where the
    oracle's pre-rounding value lies within ``tau`` (code units) of a
    half-integer and the GPU's is the other rounding; an fp16 super-scale or
    super-min where the oracle's value lies within ``tau_half`` (relative) of
    the midpoint between the two adjacent fp16 values; a weighted-search
    choice where the two candidates' errors lie within ``search_tau``
    (relative)."""
    ad = _Adopt(spec, q_p, grid, tau, tau_half, search_tau)
    sw = O.gptq_sweep(Wp, U, spec, None, importance=importance, decide=ad)
    return ReplayReport(n=int(np.asarray(q_p).size), forced=ad.forced, bad=ad.bad, sweep=sw,
                        search_ties=ad.search_ties)


def replay_layer(W, o: "O.LayerResult", q_gpu, grid: dict, *, grid_kind: str, bits: int,
                 group: int, diag=None, search: bool = False, **kw) -> ReplayReport:
    """replay_ties for a whole layer: W and q_gpu in original column order,
    o the oracle's LayerResult for the same rows, grid in processing order."""
    Wd = np.array(W, np.float64)
    Wd[:, o.dead] = 0.0
    spec = O.GridSpec(grid=grid_kind, bits=bits,
                      group=(O.Q4K_SUPER if grid_kind == "q4k" else group), search=search)
    imp = np.asarray(diag, np.float64)[o.perm] if search else None
    return replay_ties(Wd[:, o.perm], o.U, spec, np.asarray(q_gpu)[:, o.perm], grid,
                       importance=imp, **kw)


def assert_replay(rep: ReplayReport, q_gpu_p, grid: dict, grid_kind: str,
                  max_frac: float = 1e-3, max_search_rows: int | None = None):
    """After the replay: no difference off a tie, few ties, and the GPU's
    codes and grid equal to the replayed oracle's everywhere (scales within
    1e-3 relative: they carry the float32 rounding of the compensation)."""
    assert not rep.bad, f"GPU decisions off a tie: {rep.bad[:5]}"
    plain = {k: v for k, v in rep.forced.items() if "search" not in k}
    assert sum(plain.values()) <= max_frac * rep.n, f"too many ties adopted: {rep.forced}"
    if max_search_rows is not None:
        assert rep.search_ties + rep.forced.get("search", 0) <= max_search_rows, rep.forced
    sw = rep.sweep
    np.testing.assert_array_equal(np.asarray(q_gpu_p).astype(np.float32), sw.q,
                                  err_msg="codes differ after the tie-forced replay")
    if grid_kind == "affine":
        np.testing.assert_array_equal(np.asarray(grid["zero"]).astype(np.float32), sw.zero)
        rel = np.abs(np.asarray(grid["scale"], np.float64) - sw.scale) / sw.scale
        assert rel.max() <= 1e-3, f"scale rel err {rel.max():.2e}"
    else:
        for k in ("D", "Dm", "sc", "mc"):
            np.testing.assert_array_equal(np.asarray(grid[k]), getattr(sw, k), err_msg=k)

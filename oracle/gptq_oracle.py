"""Float64 CPU oracle for GPTQ layer quantization.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this module.  The product path (the HIP
library and its Python binding) never imports, links or calls it, and it
shares no code with that path.

Written from the text of these pages (cited by title and section):

* "GPTQ" (robocikowo.com, technologie-ai/gptq), sections "Jak dziala",
  "Komponenty", "Hiperparametry", "Implementacja", "Zlozonosc obliczeniowa".
* "Add gguf q4_k quantization" (pytorch/ao pull request 2001), its summary and
  the review thread on super-block scales and separate scale/min tensors.
* "GPTQ implementation with tensor subclasses" (pytorch/ao issue 577),
  section "Background" (collect the layer's inputs, update its weight, use the
  updated weight for the layer's outputs).
* "Hugging Face AutoGPTQ and Transformers Integration", section
  "The Quantization Algorithm" (one weight at a time, remaining weights
  updated through the Hessian).

The method is defined by an algorithm, not by a closed form, so the oracle
takes its steps in the pages' order, plainly:

1. H = 2 X X^T accumulated over token chunks ("Komponenty").
2. Columns with H_ii = 0 carry no signal: H_ii := 1 and their weights are 0
   (reading: the pages are silent on this).
3. Act-order: columns processed by decreasing diag(H), the activation energy
   ("Hiperparametry": order by activation importance); ties keep the lower
   original index first.
4. Damping: a value percdamp * mean(diag H) added to the diagonal
   ("Hiperparametry": value added to the Hessian diagonal for stability).
5. U = upper Cholesky factor of the inverse of the damped H, so U^T U = H^-1
   ("Komponenty": Cholesky decomposition of the inverse Hessian).
6. Column-by-column quantization in that fixed order; after each column the
   not-yet-quantized columns absorb the error through the inverse Hessian
   (Optimal Brain Surgeon rule, "Jak dziala" / "Komponenty").  Group grid
   parameters are chosen at each group's first column from the then-current,
   compensated weights ("Jak dziala": a scale per group).
7. The blocked ("lazy") form of step 6, which reaches the same result
   ("Komponenty": block updates).

Precision: every float computation is float64, except the grid decisions
(scale, zero point, code), which are taken in float32 -- the precision in
which the GPU kernels take them -- so that both sides decide integers in the
same precision; the compensation itself stays float64.  Rounding is
round-half-to-even throughout (np.rint, and numpy's float16 conversion).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

f32 = np.float32


class NotSPD(ArithmeticError):
    """The damped Hessian is not symmetric positive definite."""


# --------------------------------------------------------------------------
# Step 1. Hessian of the layer inputs ("GPTQ", section "Komponenty").
# --------------------------------------------------------------------------
def hessian(chunks) -> np.ndarray:
    """H = 2 * sum_c X_c X_c^T over token chunks X_c (d x n_c), in float64.

    The matrix is the unnormalized 2 X X^T of the page; no averaging over
    tokens (the result of the whole method is invariant to a positive scale
    of H, see the pins)."""
    G = None
    for Xc in chunks:
        Xc = np.asarray(Xc, dtype=np.float64)
        P = Xc @ Xc.T
        G = P if G is None else G + P
    return 2.0 * G


def hessian_diag(chunks) -> np.ndarray:
    """diag(H) = 2 * sum_t x_it^2, the activation energy of each feature."""
    s = None
    for Xc in chunks:
        Xc = np.asarray(Xc, dtype=np.float64)
        p = np.einsum("it,it->i", Xc, Xc)
        s = p if s is None else s + p
    return 2.0 * s


# --------------------------------------------------------------------------
# Steps 2-4. Dead columns, act-order, damping ("Hiperparametry").
# --------------------------------------------------------------------------
def dead_columns(diag: np.ndarray) -> np.ndarray:
    return np.asarray(diag) == 0


def act_order_perm(diag: np.ndarray) -> np.ndarray:
    """Processing order: decreasing activation energy, stable on ties."""
    return np.argsort(-np.asarray(diag, dtype=np.float64), kind="stable")


def damped_processing_hessian(H: np.ndarray, diag: np.ndarray, perm: np.ndarray,
                              percdamp: float) -> np.ndarray:
    """H_p = P (H with dead fix) P^T + delta I, delta = percdamp * mean(diag).

    ``diag`` is the activation energy (diag of H) used for the dead test, the
    order and the damping base."""
    H = np.array(H, dtype=np.float64)
    dead = dead_columns(diag)
    H[dead, dead] = 1.0
    dg = np.array(diag, dtype=np.float64)
    dg[dead] = 1.0
    delta = percdamp * np.mean(dg)
    Hp = H[np.ix_(perm, perm)]
    Hp[np.diag_indices_from(Hp)] += delta
    return Hp


# --------------------------------------------------------------------------
# Step 5. Cholesky factor of the inverse Hessian ("Komponenty").
# --------------------------------------------------------------------------
def inverse_cholesky_upper(Hp: np.ndarray) -> np.ndarray:
    """U upper triangular, positive diagonal, U^T U = Hp^-1.

    Literal route: invert, then take the Cholesky factor of the inverse.
    Raises NotSPD when Hp is not positive definite."""
    try:
        np.linalg.cholesky(Hp)           # Hp itself must be SPD
        Hinv = np.linalg.inv(Hp)
        L = np.linalg.cholesky(Hinv)     # Hinv = L L^T, L lower
    except np.linalg.LinAlgError as exc:
        raise NotSPD(str(exc)) from exc
    return np.triu(L.T)


def inverse_cholesky_upper_ul(Hp: np.ndarray) -> np.ndarray:
    """Same U by the reversed route: Hp = R R^T with R upper, U = R^-1.

    R is the Cholesky factor of Hp taken from the last index backwards
    (R = J chol(J Hp J) J, J the exchange matrix); U = R^-1 is then upper with
    U^T U = (R R^T)^-1.  The upper Cholesky factor of Hp^-1 is unique, so this
    equals the literal route."""
    try:
        Lr = np.linalg.cholesky(Hp[::-1, ::-1])
    except np.linalg.LinAlgError as exc:
        raise NotSPD(str(exc)) from exc
    R = Lr[::-1, ::-1]
    d = Hp.shape[0]
    U = np.linalg.solve(R, np.eye(d))
    return np.triu(U)


def unit_upper_factor(Hp: np.ndarray) -> np.ndarray:
    """T unit upper triangular with Hp = T D T^T, D diagonal and positive.

    The same reversed factor as above without its inverse: Hp = R R^T with R
    upper (R = J chol(J Hp J) J), then T = R diag(R)^-1 (column k of R divided
    by R_kk) and D = diag(R)^2.  Since U = R^-1, T = U^-1 diag(U): the
    compensation of "Komponenty" written with the factor of the Hessian
    itself rather than of its inverse.  Raises NotSPD like the routes above."""
    try:
        Lr = np.linalg.cholesky(Hp[::-1, ::-1])
    except np.linalg.LinAlgError as exc:
        raise NotSPD(str(exc)) from exc
    R = Lr[::-1, ::-1]
    return np.triu(R / np.diag(R)[None, :])


# --------------------------------------------------------------------------
# Grids.  Decisions in float32 (the kernel's precision), see module header.
# --------------------------------------------------------------------------
def _keep(name, pre, val):
    """Default decision rule: the oracle's own rounding."""
    return val


def affine_params(v: np.ndarray, bits: int, decide=_keep):
    """Asymmetric min-max grid of one group for each row.

    v: (rows, g) current weights of the group.  The range always contains 0
    so that the zero point is an integer code in [0, maxq]; an all-zero group
    uses the range [-1, 1].  Returns float32 (scale, zero, zero before rounding).

    ``decide(name, pre, val)`` returns the integer decision taken from the
    pre-rounding value ``pre`` (here "zero"); the default keeps the oracle's
    rounding ``val``.  Where ``pre`` sits on a tie, either rounding satisfies
    the method, and a caller may adopt the other one."""
    maxq = f32(2 ** bits - 1)
    v = np.asarray(v, dtype=f32)
    xmin = np.minimum(v.min(axis=1), f32(0))
    xmax = np.maximum(v.max(axis=1), f32(0))
    flat = xmin == xmax
    xmin = np.where(flat, f32(-1), xmin)
    xmax = np.where(flat, f32(1), xmax)
    s = (xmax - xmin) / maxq
    zr = -xmin / s
    z = np.clip(np.rint(zr), f32(0), maxq)
    z = decide("zero", zr, z)
    return s.astype(f32), z.astype(f32), zr.astype(f32)


# Importance-weighted grid choice (the search the gguf discussion describes:
# "Add gguf q4_k quantization", review thread -- scales and offsets chosen to
# minimize a weighted squared error, which covers rounding and clamping
# error, the weights being per-channel importances from the activations).
# Reading: the candidates share the min-max zero point and shrink the
# min-max scale by f_k = 1 - k/32, k = 0..15, clipping both ends of the range
# in proportion; the importance of column i is its activation energy
# diag(H)_i; the first candidate of least weighted error is taken.
SEARCH_SHRINK = np.array([1.0 - k / 32.0 for k in range(16)], dtype=f32)


def affine_params_weighted(v: np.ndarray, h: np.ndarray, bits: int, decide=_keep):
    """Affine grid of one group for each row by importance-weighted search.

    v: (rows, g) current weights of the group, h: (g,) importances.  For each
    candidate scale s_k = f_k s0 (float32, s0 and z0 from affine_params):
    q = clamp(rint(v / s_k) + z0, 0, maxq) and w^ = s_k (q - z0) in float32,
    E_k = sum_i h_i (v_i - w^_i)^2 in float64.  Returns float32 (scale, zero,
    zero before rounding) and, for each row, the relative gap between the
    least and the next-least E_k (0 when the choice is a tie).  ``decide`` as
    in affine_params ("zero", then "search" with pre = (E, candidate scales))."""
    s0, z0, zr = affine_params(v, bits, decide)
    maxq = f32(2 ** bits - 1)
    v = np.asarray(v, dtype=f32)
    h = np.asarray(h, dtype=np.float64)
    E = np.empty((len(SEARCH_SHRINK), v.shape[0]))
    cand = np.empty((len(SEARCH_SHRINK), v.shape[0]), f32)
    for k, f in enumerate(SEARCH_SHRINK):
        s = (f * s0).astype(f32)
        cand[k] = s
        q = np.clip(np.rint(v / s[:, None]) + z0[:, None], f32(0), maxq)
        what = (s[:, None] * (q - z0[:, None])).astype(f32)
        d = (v - what).astype(np.float64)
        E[k] = (h[None, :] * (d * d)).sum(axis=1)
    best = np.argmin(E, axis=0)                    # first least error
    best = decide("search", (E, cand), best)
    s = (SEARCH_SHRINK[best] * s0).astype(f32)
    Es = np.sort(E, axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        gap = np.where(Es[0] > 0, (Es[1] - Es[0]) / Es[0], np.where(Es[1] > 0, np.inf, 0.0))
    return s, z0, zr, gap


def affine_quantize(w: np.ndarray, s: np.ndarray, z: np.ndarray, bits: int, decide=_keep):
    """Code and dequantized value of one column: q = clamp(rint(w/s)+z), w^ = s(q-z).
    ``decide`` as in affine_params ("code", pre = w/s)."""
    maxq = f32(2 ** bits - 1)
    w = np.asarray(w, dtype=f32)
    ratio = w / s
    q = np.clip(np.rint(ratio) + z, f32(0), maxq)
    q = decide("code", ratio, q)
    return q.astype(f32), (s * (q - z)).astype(f32)


Q4K_SUB = 32      # weights per sub-block (scale and min code each)
Q4K_SUPER = 256   # weights per super-block (fp16 super-scale and super-min)


def kquant_sub_bits(bits: int) -> int:
    """Width of the sub-block scale and min codes of the two-level grid with
    `bits`-bit weights.  "Add gguf q4_k quantization", review thread: 4-bit
    sub-block scales and mins for the 2-bit type, 6-bit for the 3-, 4- and
    5-bit types, 8-bit for the 6-bit type."""
    widths = {2: 4, 3: 6, 4: 6, 5: 6, 6: 8}
    if bits not in widths:
        raise ValueError("the two-level grid has 2..6-bit codes")
    return widths[bits]


def q4k_params(v: np.ndarray, bits: int = 4, decide=_keep):
    """Two-level grid of one super-block of 256 weights for each row.

    From "Add gguf q4_k quantization": w = q * block_scale + block_min with
    sub-block scale and min codes under a super-block scale, chosen by a
    plain min-max rule rather than gguf's search.  Reading used here (the
    page gives the form, not the constants' derivation), with
    maxq = 2^bits - 1 and kmax = 2^kquant_sub_bits(bits) - 1 (63 for the
    4-bit codes of Q4_K):

    per sub-block b of 32: mn = min(v_b, 0), mx = max(v_b, 0),
        s_b = (mx - mn)/maxq, m_b = -mn (>= 0);
    D  = fp16(max_b s_b / kmax), Dm = fp16(max_b m_b / kmax);
    sc_b = clamp(rint(s_b / D), 1, kmax) if s_b > 0 and D > 0 else 0;
    mc_b = clamp(rint(m_b / Dm), 0, kmax) if Dm > 0 else 0;
    effective S_b = D sc_b, M_b = Dm mc_b.

    Returns D, Dm (float16), sc, mc (uint8, (rows, 8)), S, M (float32, (rows, 8)).
    ``decide`` as in affine_params, for "D" and "Dm" (pre: the float32 value
    rounded to fp16) and then "sc" and "mc" (pre: s_b/D and m_b/Dm)."""
    maxq = f32(2 ** bits - 1)
    v = np.asarray(v, dtype=f32)
    rows = v.shape[0]
    vb = v.reshape(rows, Q4K_SUPER // Q4K_SUB, Q4K_SUB)
    mn = np.minimum(vb.min(axis=2), f32(0))
    mx = np.maximum(vb.max(axis=2), f32(0))
    s_b = (mx - mn) / maxq
    m_b = -mn
    return _q4k_second_level(s_b, m_b, bits, decide)


def _q4k_second_level(s_b, m_b, bits, decide):
    """Super-block level of the two-level grid from the sub-block (scale, min)
    pairs s_b, m_b (rows, 8): fp16 D and Dm, then the sub-block codes."""
    kmax = f32(2 ** kquant_sub_bits(bits) - 1)
    xd = s_b.max(axis=1) / kmax
    xm = m_b.max(axis=1) / kmax
    D = decide("D", xd, xd.astype(np.float16))
    Dm = decide("Dm", xm, xm.astype(np.float16))
    Df = D.astype(f32)[:, None]
    Dmf = Dm.astype(f32)[:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        rs = s_b / Df
        rm = m_b / Dmf
        sc = np.where((s_b > 0) & (Df > 0), np.clip(np.rint(rs), 1, kmax), 0)
        mc = np.where(Dmf > 0, np.clip(np.rint(rm), 0, kmax), 0)
    sc = decide("sc", rs, sc.astype(f32))
    mc = decide("mc", rm, mc.astype(f32))
    S = (Df * sc).astype(f32)
    M = (Dmf * mc).astype(f32)
    return D, Dm, sc.astype(np.uint8), mc.astype(np.uint8), S, M


def q4k_params_weighted(v: np.ndarray, h: np.ndarray, bits: int = 4, decide=_keep):
    """Two-level grid of one super-block for each row by importance-weighted
    search of each sub-block's scale and min, then the same second level as
    q4k_params.

    Reading (as for the affine search): for sub-block b with min-max values
    s_b0 = (mx - mn)/maxq and m_b0 = -mn, the candidates are
    (s, m) = (f_k s_b0, f_k m_b0), f_k = 1 - k/32, k = 0..15, both float32;
    q = clamp(rint((v + m)/s), 0, maxq) and w^ = s q - m in float32;
    E_k = sum_i h_i (v_i - w^_i)^2 in float64; the first least E_k gives the
    sub-block's (s_b, m_b), from which D, Dm, sc, mc follow as in q4k_params.
    Returns those six arrays and the relative gap of each sub-block's choice
    (rows, 8).  ``decide`` as in q4k_params, with first "search" (pre = (E,
    candidate scales, candidate mins), each (16, rows, 8))."""
    maxq = f32(2 ** bits - 1)
    v = np.asarray(v, dtype=f32)
    h = np.asarray(h, dtype=np.float64)
    rows = v.shape[0]
    nb = Q4K_SUPER // Q4K_SUB
    vb = v.reshape(rows, nb, Q4K_SUB)
    hb = h.reshape(nb, Q4K_SUB)
    mn = np.minimum(vb.min(axis=2), f32(0))
    mx = np.maximum(vb.max(axis=2), f32(0))
    s0 = (mx - mn) / maxq
    m0 = -mn
    E = np.empty((len(SEARCH_SHRINK), rows, nb))
    cs = np.empty((len(SEARCH_SHRINK), rows, nb), f32)
    cm = np.empty((len(SEARCH_SHRINK), rows, nb), f32)
    for k, f in enumerate(SEARCH_SHRINK):
        s = (f * s0).astype(f32)
        m = (f * m0).astype(f32)
        cs[k], cm[k] = s, m
        with np.errstate(divide="ignore", invalid="ignore"):
            q = np.where(s[..., None] > 0,
                         np.clip(np.rint((vb + m[..., None]) / s[..., None]), f32(0), maxq),
                         f32(0)).astype(f32)
        what = ((s[..., None] * q).astype(f32) - m[..., None]).astype(f32)
        d = (vb - what).astype(np.float64)
        E[k] = (hb[None, :, :] * (d * d)).sum(axis=2)
    best = np.argmin(E, axis=0)
    best = decide("search", (E, cs, cm), best)
    s_b = (SEARCH_SHRINK[best] * s0).astype(f32)
    m_b = (SEARCH_SHRINK[best] * m0).astype(f32)
    Es = np.sort(E, axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        gap = np.where(Es[0] > 0, (Es[1] - Es[0]) / Es[0], np.where(Es[1] > 0, np.inf, 0.0))
    D, Dm, sc, mc, S, M = _q4k_second_level(s_b, m_b, bits, decide)
    return D, Dm, sc, mc, S, M, s_b, m_b, gap


def q4k_quantize(w: np.ndarray, S: np.ndarray, M: np.ndarray, bits: int = 4, decide=_keep):
    """q = clamp(rint((w + M)/S), 0, 2^bits - 1) (0 when S = 0), w^ = S q - M.
    ``decide`` as in affine_params ("code", pre = (w + M)/S)."""
    w = np.asarray(w, dtype=f32)
    maxq = f32(2 ** bits - 1)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (w + M) / S
        q = np.where(S > 0, np.clip(np.rint(ratio), 0, maxq), 0).astype(f32)
    q = decide("code", ratio, q)
    return q, (S * q - M).astype(f32)


# --------------------------------------------------------------------------
# Step 6/7. The column sweep with OBS compensation.
# --------------------------------------------------------------------------
@dataclass
class GridSpec:
    grid: str = "affine"   # "affine" or "q4k"
    bits: int = 4
    group: int = 128       # affine: weights per scale; q4k: 256
    search: bool = False   # importance-weighted grid choice

    @property
    def span(self) -> int:
        return Q4K_SUPER if self.grid == "q4k" else self.group


@dataclass
class SweepResult:
    q: np.ndarray          # codes (rows, d), processing order, float (integer-valued)
    what: np.ndarray       # dequantized weights (rows, d), processing order, float32
    scale: np.ndarray      # affine: (rows, d/g); q4k: effective S_b (rows, d/32)
    zero: np.ndarray       # affine: (rows, d/g); q4k: effective M_b (rows, d/32)
    ratio: np.ndarray      # pre-rounding value of each code, float32 (rows, d)
    zratio: np.ndarray     # affine: pre-rounding zero point (rows, d/g); q4k: s_b/D
    mratio: np.ndarray     # q4k: m_b/Dm (rows, d/32); affine: unused
    sgap: np.ndarray | None = None  # weighted search: relative gap of each choice
                                    # (affine: per group; q4k: per sub-block)
    D: np.ndarray | None = None
    Dm: np.ndarray | None = None
    sc: np.ndarray | None = None
    mc: np.ndarray | None = None


class _GroupState:
    """Grid parameters of the group (super-block) currently being quantized.

    ``decide(name, j, pre, val)``, when given, is consulted for every integer
    or fp16 decision taken at column j (see affine_params); None keeps the
    oracle's own rounding everywhere."""

    def __init__(self, spec: GridSpec, rows: int, d: int, importance=None, decide=None):
        self.spec = spec
        self.importance = importance
        self.decide = decide
        ng = d // spec.span
        self.sgap = np.full((rows, ng), np.inf)
        if spec.grid == "affine":
            self.scale = np.zeros((rows, ng), f32)
            self.zero = np.zeros((rows, ng), f32)
            self.zratio = np.zeros((rows, ng), f32)
            self.mratio = np.zeros((rows, 0), f32)
        else:
            nsub = d // Q4K_SUB
            self.scale = np.zeros((rows, nsub), f32)
            self.zero = np.zeros((rows, nsub), f32)
            self.zratio = np.zeros((rows, nsub), f32)
            self.mratio = np.zeros((rows, nsub), f32)
            self.D = np.zeros((rows, ng), np.float16)
            self.Dm = np.zeros((rows, ng), np.float16)
            self.sc = np.zeros((rows, nsub), np.uint8)
            self.mc = np.zeros((rows, nsub), np.uint8)
            self.subgap = np.full((rows, nsub), np.inf)

    def _at(self, j: int):
        if self.decide is None:
            return _keep
        return lambda name, pre, val: self.decide(name, j, pre, val)

    def choose(self, j: int, v: np.ndarray):
        """Choose the grid of the group starting at column j from current weights v."""
        sp = self.spec
        gi = j // sp.span
        dec = self._at(j)
        if sp.grid == "affine" and sp.search:
            h = self.importance[j:j + v.shape[1]]
            s, z, zr, gap = affine_params_weighted(v, h, sp.bits, dec)
            self.scale[:, gi], self.zero[:, gi], self.zratio[:, gi] = s, z, zr
            self.sgap[:, gi] = gap
        elif sp.grid == "affine":
            s, z, zr = affine_params(v, sp.bits, dec)
            self.scale[:, gi], self.zero[:, gi], self.zratio[:, gi] = s, z, zr
        else:
            b0 = j // Q4K_SUB
            nb = Q4K_SUPER // Q4K_SUB
            if sp.search:
                h = self.importance[j:j + v.shape[1]]
                D, Dm, sc, mc, S, M, s_b, m_b, gap = q4k_params_weighted(v, h, sp.bits, dec)
                self.subgap[:, b0:b0 + nb] = gap
            else:
                D, Dm, sc, mc, S, M = q4k_params(v, sp.bits, dec)
                vb = np.asarray(v, f32).reshape(v.shape[0], nb, Q4K_SUB)
                mn = np.minimum(vb.min(axis=2), f32(0))
                mx = np.maximum(vb.max(axis=2), f32(0))
                s_b = (mx - mn) / f32(2 ** sp.bits - 1)
                m_b = -mn
            self.D[:, gi], self.Dm[:, gi] = D, Dm
            self.sc[:, b0:b0 + nb], self.mc[:, b0:b0 + nb] = sc, mc
            self.scale[:, b0:b0 + nb], self.zero[:, b0:b0 + nb] = S, M
            with np.errstate(divide="ignore", invalid="ignore"):
                self.zratio[:, b0:b0 + nb] = s_b / D.astype(f32)[:, None]
                self.mratio[:, b0:b0 + nb] = m_b / Dm.astype(f32)[:, None]

    def quantize(self, j: int, w: np.ndarray):
        sp = self.spec
        if sp.grid == "affine":
            gi = j // sp.group
            s, z = self.scale[:, gi], self.zero[:, gi]
            q, what = affine_quantize(w, s, z, sp.bits, self._at(j))
            ratio = np.asarray(w, f32) / s
        else:
            b = j // Q4K_SUB
            S, M = self.scale[:, b], self.zero[:, b]
            q, what = q4k_quantize(w, S, M, sp.bits, self._at(j))
            with np.errstate(divide="ignore", invalid="ignore"):
                ratio = (np.asarray(w, f32) + M) / S
        return q, what, ratio


def _check_shapes(W, U, spec: GridSpec, block: int | None):
    r, d = W.shape
    if U.shape != (d, d):
        raise ValueError("U must be d x d")
    if d % spec.span:
        raise ValueError("cols must be a multiple of the group size")
    if block is not None and not (spec.span % block == 0 or block % spec.span == 0):
        raise ValueError("group and block sizes must divide one another")


def gptq_sweep(Wp: np.ndarray, U: np.ndarray, spec: GridSpec,
               block: int | None = None, importance=None, decide=None) -> SweepResult:
    """Quantize Wp (rows x d, processing order) column by column.

    block=None is the plain definition: after column j every later column k
    takes W[:, k] -= e_j U[j, k] at once, with e_j = (w_j - w^_j)/U[j, j].
    block=B is the lazy blocked form: inside a block of B columns the update
    reaches only the block's own later columns, and the accumulated errors
    reach everything after the block in one product Err @ U[block, after].

    ``decide(name, j, pre, val)`` may replace a rounding decision taken on a
    tie by the other, equally valid one (see affine_params); None keeps the
    oracle's own."""
    _check_shapes(Wp, U, spec, block)
    W = np.array(Wp, dtype=np.float64)
    U = np.asarray(U, dtype=np.float64)
    r, d = W.shape
    Q = np.zeros((r, d), f32)
    What = np.zeros((r, d), f32)
    ratio = np.zeros((r, d), f32)
    if spec.search and importance is None:
        raise ValueError("the weighted grid search needs the columns' importances")
    gs = _GroupState(spec, r, d, importance, decide)
    B = d if block is None else block
    for i1 in range(0, d, B):
        i2 = min(i1 + B, d)
        hi = d if block is None else i2          # reach of the eager update
        Err = np.zeros((r, i2 - i1))
        for j in range(i1, i2):
            if j % spec.span == 0:
                gs.choose(j, W[:, j:j + spec.span].astype(f32))
            w = W[:, j]
            q, what, rat = gs.quantize(j, w.astype(f32))
            e = (w - what.astype(np.float64)) / U[j, j]
            W[:, j + 1:hi] -= np.outer(e, U[j, j + 1:hi])
            Err[:, j - i1] = e
            Q[:, j], What[:, j], ratio[:, j] = q, what, rat
            W[:, j] = what
        if block is not None and i2 < d:
            W[:, i2:] -= Err @ U[i1:i2, i2:]
    sgap = None
    if spec.search:   # per group (affine) or per sub-block (two-level grid)
        sgap = gs.sgap if spec.grid == "affine" else gs.subgap
    res = SweepResult(q=Q, what=What, scale=gs.scale, zero=gs.zero, ratio=ratio,
                      zratio=gs.zratio, mratio=gs.mratio, sgap=sgap)
    if spec.grid == "q4k":
        res.D, res.Dm, res.sc, res.mc = gs.D, gs.Dm, gs.sc, gs.mc
    return res


def rtn(Wp: np.ndarray, spec: GridSpec) -> SweepResult:
    """Round-to-nearest on the same grid rule and grouping, no compensation."""
    d = Wp.shape[1]
    return gptq_sweep(Wp, np.eye(d), spec)   # U = I: every update is zero


# --------------------------------------------------------------------------
# Whole layer.
# --------------------------------------------------------------------------
@dataclass
class LayerResult:
    perm: np.ndarray       # processing position -> original column
    dead: np.ndarray       # bool per original column
    U: np.ndarray          # float64, processing order
    sweep: SweepResult     # processing order
    q: np.ndarray          # codes, original column order
    what: np.ndarray       # dequantized weights, original column order
    g_idx: np.ndarray      # group of each original column


def quantize_layer(W: np.ndarray, H: np.ndarray, diag: np.ndarray, *, bits: int,
                   group: int, block: int | None, act_order: bool,
                   percdamp: float, grid: str = "affine", route: str = "literal",
                   rows: np.ndarray | None = None, search: bool = False) -> LayerResult:
    """GPTQ on one linear layer (W rows x d, H d x d, diag = activation energy).

    ``rows`` restricts the sweep to a subset of W's rows (rows are independent
    given U); W is then only those rows.  ``search`` chooses each group's
    (affine) or sub-block's (two-level) grid by the importance-weighted
    search, the importance of a column being its activation energy diag[i]."""
    W = np.asarray(W, dtype=np.float64)
    d = W.shape[1]
    diag = np.asarray(diag, dtype=np.float64)
    dead = dead_columns(diag)
    perm = act_order_perm(diag) if act_order else np.arange(d)
    Hp = damped_processing_hessian(H, diag, perm, percdamp)
    U = inverse_cholesky_upper(Hp) if route == "literal" else inverse_cholesky_upper_ul(Hp)
    Wd = W.copy()
    Wd[:, dead] = 0.0
    spec = GridSpec(grid=grid, bits=bits, group=(Q4K_SUPER if grid == "q4k" else group),
                    search=search)
    sw = gptq_sweep(Wd[:, perm], U, spec, block, importance=diag[perm] if search else None)
    q = np.empty_like(sw.q)
    what = np.empty_like(sw.what)
    q[:, perm] = sw.q
    what[:, perm] = sw.what
    gsz = Q4K_SUB if grid == "q4k" else group
    g_idx = np.empty(d, np.int64)
    g_idx[perm] = np.arange(d) // gsz
    return LayerResult(perm=perm, dead=dead, U=U, sweep=sw, q=q, what=what, g_idx=g_idx)


def reconstruction_error(W: np.ndarray, What: np.ndarray, H: np.ndarray) -> float:
    """||(W - W^) X||_F^2 = 1/2 tr(dW H dW^T) for H = 2 X X^T (undamped)."""
    dW = np.asarray(W, np.float64) - np.asarray(What, np.float64)
    return 0.5 * float(np.sum((dW @ np.asarray(H, np.float64)) * dW))


# --------------------------------------------------------------------------
# Storage: codes as a bit stream ("Zlozonosc obliczeniowa": about 4.x bits per
# weight once packed with the per-group parameters).
# --------------------------------------------------------------------------
def pack(codes: np.ndarray, bits: int) -> np.ndarray:
    """Rows of b-bit codes -> rows of uint32 words, least significant bit first.

    Code k of a row occupies stream bits [k*b, (k+1)*b); stream bit t is bit
    (t mod 32) of word t // 32."""
    codes = np.asarray(codes, dtype=np.int64)
    r, n = codes.shape
    if (n * bits) % 32:
        raise ValueError("cols*bits must be a multiple of 32")
    if codes.min(initial=0) < 0 or codes.max(initial=0) >= (1 << bits):
        raise ValueError("code out of range")
    nw = n * bits // 32
    out = np.zeros((r, nw), dtype=np.uint64)
    for k in range(n):
        for b in range(bits):
            t = k * bits + b
            bit = (codes[:, k] >> b) & 1
            out[:, t // 32] |= (bit.astype(np.uint64) << np.uint64(t % 32))
    return out.astype(np.uint32)


def unpack(words: np.ndarray, bits: int, n: int) -> np.ndarray:
    words = np.asarray(words, dtype=np.uint64)
    r = words.shape[0]
    out = np.zeros((r, n), dtype=np.int64)
    for k in range(n):
        for b in range(bits):
            t = k * bits + b
            bit = (words[:, t // 32] >> np.uint64(t % 32)) & np.uint64(1)
            out[:, k] |= bit.astype(np.int64) << b
    return out

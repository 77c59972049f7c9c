"""Seeded synthetic layer inputs (weights W and calibration activations X).

This module only draws random numbers and rounds them to the storage dtype;
it holds none of the quantization method's arithmetic.  It is the single
piece of code shared by the float64 oracle side (tests, CPU baseline) and the
HIP side (tests, bench), so both see bit-identical inputs.

Every element is a pure function of (seed, stream, row, token chunk):

* W row ``i``           -> Philox key (seed, STREAM_W, i, 0)
* X row ``i``, chunk c  -> Philox key (seed, STREAM_X, i, c), chunks of
  ``TOKEN_CHUNK`` tokens (the SiLU gate draws its second factor from
  STREAM_X_GATE); a chunk can be regenerated row by row, and a token prefix
  of a chunk needs only that many draws, so a test can rebuild any single
  feature row of a 131072-token X without the rest.
* outlier channels      -> Philox key (seed, STREAM_OUTLIER, 0, 0)

Values are drawn as float32 standard normals; bf16 storage is obtained by
round-to-nearest-even on the float32 bit pattern, and the very same bf16 bits
go to the GPU and (widened exactly) to the oracle.

The workloads stand in for calibration runs of 7B-70B LLM linears (the pages
measure on whole OPT/BLOOM/Llama models with real calibration text, which is
not available here): Gaussian activations, Gaussian activations with a few
outlier channels scaled up, and SiLU-gated products with heavy tails.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

TOKEN_CHUNK = 8192
STREAM_W, STREAM_X, STREAM_OUTLIER, STREAM_X_GATE = 0, 1, 2, 3
STREAM_STORED, STREAM_ACT16 = 4, 5
BASE_SEED = 20261203


@dataclass(frozen=True)
class LayerConfig:
    """One synthetic linear layer plus its quantization settings."""

    name: str
    rows: int            # output features (rows of W)
    cols: int            # input features d (cols of W, rows of X)
    tokens: int          # calibration tokens n (cols of X)
    x_dtype: str         # "f32" or "bf16"
    w_dtype: str         # "f32" or "bf16"
    w_sigma: float
    x_kind: str          # "gauss" or "silu_gated"
    outlier_frac: float  # fraction of channels scaled by outlier_scale
    outlier_scale: float
    bits: int
    group: int           # affine: weights per scale; q4k: superblock (256)
    block: int           # lazy-update block size B
    act_order: bool
    percdamp: float
    grid: str            # "affine" or "q4k"
    seed: int

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)


def _cfg(idx, name, rows, cols, tokens, x_dtype, w_dtype, w_sigma, x_kind,
         outlier_frac, outlier_scale, bits, group, block, act_order, grid):
    return LayerConfig(name=name, rows=rows, cols=cols, tokens=tokens,
                       x_dtype=x_dtype, w_dtype=w_dtype, w_sigma=w_sigma,
                       x_kind=x_kind, outlier_frac=outlier_frac,
                       outlier_scale=outlier_scale, bits=bits, group=group,
                       block=block, act_order=act_order, percdamp=0.01,
                       grid=grid, seed=BASE_SEED + idx)


# The five workloads, named by what they are.
CONFIGS = {
    "tiny_64x128_int4_g32": _cfg(
        0, "tiny_64x128_int4_g32", 64, 128, 512, "f32", "f32", 0.02, "gauss",
        0.0, 1.0, 4, 32, 32, False, "affine"),
    "q_proj_4096x4096_int4_g128": _cfg(
        1, "q_proj_4096x4096_int4_g128", 4096, 4096, 65536, "bf16", "bf16",
        0.02, "gauss", 0.01, 20.0, 4, 128, 128, False, "affine"),
    "down_proj_4096x11008_int4_g128_actorder": _cfg(
        2, "down_proj_4096x11008_int4_g128_actorder", 4096, 11008, 131072,
        "bf16", "bf16", 0.015, "silu_gated", 0.0, 1.0, 4, 128, 128, True,
        "affine"),
    "up_proj_28672x8192_int3_g128_actorder": _cfg(
        3, "up_proj_28672x8192_int3_g128_actorder", 28672, 8192, 65536,
        "bf16", "bf16", 0.01, "gauss", 0.005, 30.0, 3, 128, 128, True,
        "affine"),
    "q4k_14336x4096": _cfg(
        4, "q4k_14336x4096", 14336, 4096, 65536, "bf16", "bf16", 0.02,
        "gauss", 0.0, 1.0, 4, 256, 128, False, "q4k"),
}
HEADLINE = "down_proj_4096x11008_int4_g128_actorder"


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _rng(seed: int, stream: int, row: int, chunk: int) -> np.random.Generator:
    key = np.array([(seed << 8) | stream, (row << 24) | chunk], dtype=np.uint64)
    return np.random.Generator(np.random.Philox(key=key))


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    b = (u >> 16) & np.uint32(1)
    b += np.uint32(0x7FFF)
    b += u
    b >>= 16
    return b.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def round_bf16(a: np.ndarray) -> np.ndarray:
    return bf16_to_f32(bf16_bits(a))


# ----------------------------------------------------------------- weights
def weight_rows(cfg: LayerConfig, rows=None) -> np.ndarray:
    """Rows of W (float32 values; bf16-exact when w_dtype is bf16)."""
    rows = np.arange(cfg.rows) if rows is None else np.asarray(rows)
    out = np.empty((len(rows), cfg.cols), dtype=np.float32)
    sig = np.float32(cfg.w_sigma)

    def one(k):
        v = _rng(cfg.seed, STREAM_W, int(rows[k]), 0).standard_normal(
            cfg.cols, dtype=np.float32) * sig
        out[k] = round_bf16(v) if cfg.w_dtype == "bf16" else v

    if len(rows) > 256:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, range(len(rows))))
    else:
        for k in range(len(rows)):
            one(k)
    return out


def weight(cfg: LayerConfig) -> np.ndarray:
    return weight_rows(cfg)


# ------------------------------------------------------------- activations
def outlier_channels(cfg: LayerConfig) -> np.ndarray:
    k = int(round(cfg.outlier_frac * cfg.cols))
    if k == 0:
        return np.zeros(0, dtype=np.int64)
    g = _rng(cfg.seed, STREAM_OUTLIER, 0, 0)
    return np.sort(g.choice(cfg.cols, size=k, replace=False))


def _row_scales(cfg: LayerConfig) -> np.ndarray:
    s = np.ones(cfg.cols, dtype=np.float32)
    s[outlier_channels(cfg)] = np.float32(cfg.outlier_scale)
    return s


def _x_row_chunk(cfg: LayerConfig, row: int, chunk: int, scale: np.float32,
                 upto: int = TOKEN_CHUNK) -> np.ndarray:
    """The first ``upto`` tokens of feature ``row`` in chunk ``chunk`` (float32,
    pre-rounding); a prefix of the chunk's values, whatever ``upto`` is."""
    g = _rng(cfg.seed, STREAM_X, row, chunk)
    if cfg.x_kind == "gauss":
        v = g.standard_normal(upto, dtype=np.float32)
    elif cfg.x_kind == "silu_gated":
        a = g.standard_normal(upto, dtype=np.float32)
        b = _rng(cfg.seed, STREAM_X_GATE, row, chunk).standard_normal(upto, dtype=np.float32)
        with np.errstate(over="ignore"):
            v = (a / (np.float32(1) + np.exp(-a))) * b
    else:
        raise ValueError(cfg.x_kind)
    if scale != 1:
        v = v * scale
    return v


def x_rows(cfg: LayerConfig, rows, tok0: int = 0, ntok: int | None = None) -> np.ndarray:
    """Feature rows of X over tokens [tok0, tok0+ntok) as float32 values."""
    ntok = cfg.tokens - tok0 if ntok is None else ntok
    assert 0 <= tok0 and tok0 + ntok <= cfg.tokens
    rows = np.asarray(rows)
    scales = _row_scales(cfg)
    out = np.empty((len(rows), ntok), dtype=np.float32)
    c0, c1 = tok0 // TOKEN_CHUNK, (tok0 + ntok + TOKEN_CHUNK - 1) // TOKEN_CHUNK

    def one(k):
        r = int(rows[k])
        for c in range(c0, c1):
            lo = max(tok0, c * TOKEN_CHUNK)
            hi = min(tok0 + ntok, (c + 1) * TOKEN_CHUNK)
            v = _x_row_chunk(cfg, r, c, scales[r], hi - c * TOKEN_CHUNK)[lo - c * TOKEN_CHUNK:]
            out[k, lo - tok0: hi - tok0] = round_bf16(v) if cfg.x_dtype == "bf16" else v

    if len(rows) * (c1 - c0) > 64:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, range(len(rows))))
    else:
        for k in range(len(rows)):
            one(k)
    return out


def x_chunk(cfg: LayerConfig, tok0: int, ntok: int) -> np.ndarray:
    """All d feature rows of X over tokens [tok0, tok0+ntok) as float32 values."""
    return x_rows(cfg, np.arange(cfg.cols), tok0, ntok)


def x_chunk_storage(cfg: LayerConfig, tok0: int, ntok: int) -> np.ndarray:
    """Same chunk in its storage dtype: uint16 bf16 bits, or float32."""
    v = x_chunk(cfg, tok0, ntok)
    return bf16_bits(v) if cfg.x_dtype == "bf16" else v


def token_chunks(cfg: LayerConfig, chunk_tokens: int):
    """(tok0, ntok) pairs that tile [0, tokens)."""
    return [(t, min(chunk_tokens, cfg.tokens - t)) for t in range(0, cfg.tokens, chunk_tokens)]


# ------------------------------------------------- stored 4-bit layers (W4A16)
@dataclass(frozen=True)
class StoredLayer:
    """A quantized layer as stored: codes, group index, scales, zero points."""

    codes: np.ndarray   # (rows, cols) uint8 in [0, 16)
    g_idx: np.ndarray   # (cols,) int32, group of each original column
    scale: np.ndarray   # (rows, cols // group) float32 > 0
    zero: np.ndarray    # (rows, cols // group) uint8 in [0, 16)
    group: int


def stored_int4_layer(rows: int, cols: int, group: int, act_order: bool, seed: int,
                      w_sigma: float = 0.02) -> StoredLayer:
    """Seeded stand-in for a 4-bit layer as it leaves quantization.

    Codes and zero points are uniform over [0, 16).  Scales are spread around
    the step of a min-max grid over a group of N(0, w_sigma^2) weights (about
    0.35 w_sigma), log-normally.  With act_order the columns of each group are
    a random subset of the row (a random processing order cut into groups of
    ``group``); without it group g is columns [g*group, (g+1)*group)."""
    assert cols % group == 0
    ng = cols // group
    g = _rng(seed, STREAM_STORED, 0, 0)
    codes = g.integers(0, 16, size=(rows, cols), dtype=np.uint8)
    zero = g.integers(0, 16, size=(rows, ng), dtype=np.uint8)
    scale = (np.float32(0.35 * w_sigma)
             * np.exp(np.float32(0.25) * g.standard_normal((rows, ng), dtype=np.float32)))
    order = g.permutation(cols) if act_order else np.arange(cols)
    g_idx = np.empty(cols, dtype=np.int32)
    g_idx[order] = np.arange(cols, dtype=np.int32) // group
    return StoredLayer(codes=codes, g_idx=g_idx, scale=scale.astype(np.float32),
                       zero=zero, group=group)


def activations_f16(batch: int, cols: int, seed: int, outlier_frac: float = 0.01,
                    outlier_scale: float = 20.0) -> np.ndarray:
    """(batch, cols) float16 bit patterns: N(0, 1) activations with a fraction
    of channels scaled up, rounded to float16 (nearest, ties to even)."""
    g = _rng(seed, STREAM_ACT16, 0, 0)
    v = g.standard_normal((batch, cols), dtype=np.float32)
    k = int(round(outlier_frac * cols))
    if k:
        v[:, g.choice(cols, size=k, replace=False)] *= np.float32(outlier_scale)
    return v.astype(np.float16).view(np.uint16)

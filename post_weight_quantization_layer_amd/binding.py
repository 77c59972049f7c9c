"""ctypes binding of libgptq_mi355x.so (argument marshalling only).

Every function here has the name of the C entry point it wraps and does no
arithmetic of its own: tensors are turned into device pointers, the current
torch stream into a hipStream_t, and a non-OK status into an exception.
The library must be built (``python -m post_weight_quantization_layer_amd.build``);
there is no fallback of any kind when it is missing.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgptq_mi355x.so")

GPTQ_OK, GPTQ_ERR_INVALID_ARG, GPTQ_ERR_NOT_SPD, GPTQ_ERR_DEVICE, GPTQ_ERR_WORKSPACE = range(5)
GPTQ_DT_F32, GPTQ_DT_BF16 = 0, 1
GPTQ_GRID_AFFINE, GPTQ_GRID_Q4K = 0, 1

EXPORTED = (
    "gptq_last_error", "gptq_workspace_bytes", "gptq_hessian_accumulate",
    "gptq_prepare_hinv", "gptq_quantize_layer", "gptq_pack",
    "gptq_profile_enable", "gptq_profile_reset", "gptq_profile_query",
    "gptq_w4a16_layer_bytes", "gptq_w4a16_prepare", "gptq_w4a16_workspace_bytes",
    "gptq_w4a16_gemm", "gptq_linear_forward_ws_bytes", "gptq_linear_forward",
    "gptq_silu_mul", "gptq_w4a16_gemm_noalloc",
)


class GptqError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"status {status}: {msg}")
        self.status = status


class NotSPDError(GptqError):
    pass


class gptq_params(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("group", ctypes.c_int32),
                ("block", ctypes.c_int32), ("act_order", ctypes.c_int32),
                ("percdamp", ctypes.c_float), ("grid", ctypes.c_int32),
                ("search", ctypes.c_int32), ("route", ctypes.c_int32)]


ROUTES = {"inverse": 0, "hessian": 1}


def make_params(bits: int, group: int, block: int, act_order: bool, percdamp: float,
                grid: str | int = "affine", search: bool = False,
                route: str | int = "inverse") -> gptq_params:
    g = grid if isinstance(grid, int) else {"affine": GPTQ_GRID_AFFINE, "q4k": GPTQ_GRID_Q4K}[grid]
    rt = route if isinstance(route, int) else ROUTES[route]
    return gptq_params(int(bits), int(group), int(block), int(bool(act_order)), float(percdamp), g,
                       int(bool(search)), rt)


class gptq_w4a16_layer(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("group", ctypes.c_int32), ("permuted", ctypes.c_int32),
                ("rows_pad", ctypes.c_int64), ("k_pad", ctypes.c_int64),
                ("mem", ctypes.c_void_p), ("mem_bytes", ctypes.c_size_t)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the native library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m post_weight_quantization_layer_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    L.gptq_last_error.restype = ctypes.c_char_p
    L.gptq_last_error.argtypes = []
    L.gptq_workspace_bytes.restype = SZ
    L.gptq_workspace_bytes.argtypes = [I64, I64, ctypes.POINTER(gptq_params)]
    L.gptq_hessian_accumulate.restype = I32
    L.gptq_hessian_accumulate.argtypes = [P, P, I64, P, I32, I64, I64, P, SZ, P]
    L.gptq_prepare_hinv.restype = I32
    L.gptq_prepare_hinv.argtypes = [P, P, I64, ctypes.POINTER(gptq_params), P, P, P, P, SZ, P]
    L.gptq_quantize_layer.restype = I32
    L.gptq_quantize_layer.argtypes = [P, I64, I64, P, P, P, P, ctypes.POINTER(gptq_params),
                                      P, P, P, P, P, P, P, P, P, SZ, P]
    L.gptq_pack.restype = I32
    L.gptq_pack.argtypes = [P, I64, I64, I32, P, P]
    L.gptq_profile_enable.restype = None
    L.gptq_profile_enable.argtypes = [ctypes.c_int]
    L.gptq_profile_reset.restype = None
    L.gptq_profile_reset.argtypes = []
    L.gptq_profile_query.restype = I32
    L.gptq_profile_query.argtypes = [ctypes.c_char_p, ctypes.POINTER(I64),
                                     ctypes.POINTER(ctypes.c_double)]
    L.gptq_w4a16_layer_bytes.restype = SZ
    L.gptq_w4a16_layer_bytes.argtypes = [I64, I64, I32]
    L.gptq_w4a16_prepare.restype = I32
    L.gptq_w4a16_prepare.argtypes = [P, P, P, P, I64, I64, I32, P, SZ,
                                     ctypes.POINTER(gptq_w4a16_layer), P]
    L.gptq_w4a16_workspace_bytes.restype = SZ
    L.gptq_w4a16_workspace_bytes.argtypes = [ctypes.POINTER(gptq_w4a16_layer), I64]
    L.gptq_w4a16_gemm.restype = I32
    L.gptq_w4a16_gemm.argtypes = [ctypes.POINTER(gptq_w4a16_layer), P, I64, P, P, SZ, P]
    L.gptq_w4a16_gemm_noalloc.restype = I32
    L.gptq_w4a16_gemm_noalloc.argtypes = [ctypes.POINTER(gptq_w4a16_layer), P, I64, P, P]
    L.gptq_linear_forward_ws_bytes.restype = SZ
    L.gptq_linear_forward_ws_bytes.argtypes = [I64, I64, I64]
    L.gptq_linear_forward.restype = I32
    L.gptq_linear_forward.argtypes = [P, I64, I64, P, I64, I64, P, I64, P, SZ, P]
    L.gptq_silu_mul.restype = I32
    L.gptq_silu_mul.argtypes = [P, P, I64, I64, I64, P, I64, P]
    _lib = L
    return L


def _check(status: int):
    if status != GPTQ_OK:
        msg = lib().gptq_last_error().decode()
        if status == GPTQ_ERR_NOT_SPD:
            raise NotSPDError(status, msg)
        raise GptqError(status, msg)


def _ptr(t) -> int | None:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def gptq_last_error() -> str:
    return lib().gptq_last_error().decode()


def gptq_workspace_bytes(rows: int, cols: int, params: gptq_params) -> int:
    n = lib().gptq_workspace_bytes(rows, cols, ctypes.byref(params))
    if n == 0:
        raise GptqError(GPTQ_ERR_INVALID_ARG, gptq_last_error())
    return n


def gptq_hessian_accumulate(H, hdiag, X, n_tok: int | None = None, ld_x: int | None = None,
                            ws=None, stream=None):
    """H (d x d fp32), hdiag (d fp64), X (d x n) bf16 or fp32 (device tensors);
    ws: optional uint8 device scratch."""
    import torch
    d = H.shape[0]
    if X.dtype == torch.bfloat16:
        dt = GPTQ_DT_BF16
    elif X.dtype == torch.float32:
        dt = GPTQ_DT_F32
    else:
        raise TypeError("X must be bfloat16 or float32")
    n = X.shape[1] if n_tok is None else n_tok
    ld = X.stride(0) if ld_x is None else ld_x
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().gptq_hessian_accumulate(_ptr(H), _ptr(hdiag), d, _ptr(X), dt, n, ld, _ptr(ws),
                                         nbytes, _stream(stream)))


def gptq_prepare_hinv(H, hdiag, params: gptq_params, U, perm, dead, ws, stream=None):
    _check(lib().gptq_prepare_hinv(_ptr(H), _ptr(hdiag), H.shape[0], ctypes.byref(params),
                                   _ptr(U), _ptr(perm), _ptr(dead), _ptr(ws), ws.numel(),
                                   _stream(stream)))


def gptq_quantize_layer(W, U, perm, dead, params: gptq_params, q, g_idx, scale=None, zero=None,
                        q4k_super_scale=None, q4k_super_min=None, q4k_sub_scale=None,
                        q4k_sub_min=None, ws=None, stream=None, hdiag=None):
    rows, cols = W.shape
    _check(lib().gptq_quantize_layer(
        _ptr(W), rows, cols, _ptr(U), _ptr(perm), _ptr(dead), _ptr(hdiag), ctypes.byref(params),
        _ptr(q),
        _ptr(g_idx), _ptr(scale), _ptr(zero), _ptr(q4k_super_scale), _ptr(q4k_super_min),
        _ptr(q4k_sub_scale), _ptr(q4k_sub_min), _ptr(ws), 0 if ws is None else ws.numel(),
        _stream(stream)))


def gptq_pack(codes, bits: int, packed, rows: int | None = None, cols: int | None = None,
              stream=None):
    r = codes.shape[0] if rows is None else rows
    c = codes.shape[1] if cols is None else cols
    _check(lib().gptq_pack(_ptr(codes), r, c, bits, _ptr(packed), _stream(stream)))


def gptq_w4a16_layer_bytes(rows: int, cols: int, group: int) -> int:
    n = lib().gptq_w4a16_layer_bytes(rows, cols, group)
    if n == 0:
        raise GptqError(GPTQ_ERR_INVALID_ARG, "invalid W4A16 layer shape or group")
    return n


def gptq_w4a16_prepare(packed, g_idx, scale, zero_packed, rows: int, cols: int, group: int,
                       mem, stream=None) -> gptq_w4a16_layer:
    """Synchronous.  ``mem`` must stay alive as long as the returned layer is used."""
    layer = gptq_w4a16_layer()
    _check(lib().gptq_w4a16_prepare(_ptr(packed), _ptr(g_idx), _ptr(scale), _ptr(zero_packed),
                                    rows, cols, group, _ptr(mem),
                                    mem.numel() * mem.element_size(), ctypes.byref(layer),
                                    _stream(stream)))
    return layer


def gptq_w4a16_workspace_bytes(layer: gptq_w4a16_layer, batch: int) -> int:
    return lib().gptq_w4a16_workspace_bytes(ctypes.byref(layer), batch)


def gptq_w4a16_gemm_noalloc(layer: gptq_w4a16_layer, x, y, batch: int | None = None,
                            stream=None):
    """As gptq_w4a16_gemm, with the library's static device scratch (no workspace)."""
    b = x.shape[0] if batch is None else batch
    _check(lib().gptq_w4a16_gemm_noalloc(ctypes.byref(layer), _ptr(x), b, _ptr(y),
                                         _stream(stream)))


def gptq_w4a16_gemm(layer: gptq_w4a16_layer, x, y, ws=None, batch: int | None = None,
                    stream=None):
    """x (batch x cols) and y (batch x rows) float16 device tensors."""
    b = x.shape[0] if batch is None else batch
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().gptq_w4a16_gemm(ctypes.byref(layer), _ptr(x), b, _ptr(y), _ptr(ws), nbytes,
                                 _stream(stream)))


def gptq_linear_forward_ws_bytes(rows: int, cols: int, n_tok: int) -> int:
    return lib().gptq_linear_forward_ws_bytes(rows, cols, n_tok)


def gptq_linear_forward(W, X, Y, ws, n_tok: int | None = None, ld_x: int | None = None,
                        ld_y: int | None = None, stream=None):
    """W rows x cols float32, X cols x n bf16, Y rows x n bf16 (device tensors)."""
    rows, cols = W.shape
    n = X.shape[1] if n_tok is None else n_tok
    _check(lib().gptq_linear_forward(
        _ptr(W), rows, cols, _ptr(X), n, X.stride(0) if ld_x is None else ld_x, _ptr(Y),
        Y.stride(0) if ld_y is None else ld_y, _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))


def gptq_silu_mul(G, U, A, n_tok: int | None = None, stream=None):
    rows = G.shape[0]
    n = G.shape[1] if n_tok is None else n_tok
    _check(lib().gptq_silu_mul(_ptr(G), _ptr(U), rows, n, G.stride(0), _ptr(A), A.stride(0),
                               _stream(stream)))


def gptq_profile_enable(on: bool = True):
    lib().gptq_profile_enable(1 if on else 0)


def gptq_profile_reset():
    lib().gptq_profile_reset()


def gptq_profile_query(name: str) -> tuple[int, float]:
    n = ctypes.c_int64(0)
    ms = ctypes.c_double(0.0)
    _check(lib().gptq_profile_query(name.encode(), ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value

"""ctypes face of the CPU oracle (``moe_oracle.cpp``).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this module; the product package never
does.  The oracle shares no code with the HIP library.

All functions take and return numpy arrays on the host.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

FMT_FP8_B128 = 0
FMT_MX = 1
FMT_BF16 = 2

_lib = None


def build() -> str:
    """Compile the oracle with the host compiler (g++, OpenMP)."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["g++", "-O2", "-std=c++17", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, _SRC]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32 = ctypes.c_int32
    i64 = ctypes.c_int64
    lib.oracle_e4m3_decode.argtypes = [P, i64, P]
    lib.oracle_e2m1_decode.argtypes = [P, i64, P]
    lib.oracle_e4m3_encode.argtypes = [P, i64, P]
    lib.oracle_e8m0_decode.argtypes = [P, i64, P]
    lib.oracle_route_sort.argtypes = [P, i32, i32, i32, i32, P, P, P, P]
    lib.oracle_route_sort.restype = ctypes.c_int
    lib.oracle_router_topk.argtypes = [P, i32, i32, i32, i32, P, P]
    lib.oracle_router_topk.restype = ctypes.c_int
    lib.oracle_quant_rows_bf16.argtypes = [P, i32, i32, i32, P, P]
    lib.oracle_quant_rows_bf16.restype = ctypes.c_int
    lib.oracle_quant_rows_bf16_static.argtypes = [P, i32, i32, i32, P, i32, P]
    lib.oracle_quant_rows_bf16_static.restype = ctypes.c_int
    lib.oracle_quant_rows_f32.argtypes = [P, i32, i32, i32, P, P]
    lib.oracle_quant_rows_f32.restype = ctypes.c_int
    lib.oracle_grouped_gemm.argtypes = [i32, P, P, P, i32, P, i32, P, P, i32, i32, P]
    lib.oracle_grouped_gemm.restype = ctypes.c_int
    lib.oracle_forward.argtypes = [i32, i32, i32, i32, P, P, P, P, P, P, P, i32, i32, i32, i32,
                                   ctypes.c_float, P, i32, P, P, P, P, P, P, i32]
    lib.oracle_forward.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class OracleError(RuntimeError):
    pass


def _check(rc):
    if rc != 0:
        raise OracleError(f"oracle returned {rc}")


def e4m3_decode(codes) -> np.ndarray:
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().oracle_e4m3_decode(_ptr(c), c.size, _ptr(out))
    return out


def e2m1_decode(nibbles) -> np.ndarray:
    c = _c(nibbles, np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().oracle_e2m1_decode(_ptr(c), c.size, _ptr(out))
    return out


def e8m0_decode(b) -> np.ndarray:
    c = _c(b, np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().oracle_e8m0_decode(_ptr(c), c.size, _ptr(out))
    return out


def e4m3_encode(x) -> np.ndarray:
    f = _c(x, np.float32)
    out = np.empty(f.shape, np.uint8)
    _load().oracle_e4m3_encode(_ptr(f), f.size, _ptr(out))
    return out


def route_sort(ids, E: int, expert_begin: int = 0):
    """ids: int32 [T, k].  Returns (sorted_slot[S], expert_offsets[E+1], slot_pos[S], invalid)."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    S = T * k
    sorted_slot = np.empty(S, np.int32)
    slot_pos = np.empty(S, np.int32)
    offsets = np.empty(E + 1, np.int32)
    inv = np.zeros(1, np.int32)
    _check(_load().oracle_route_sort(_ptr(ids), T, k, E, expert_begin, _ptr(sorted_slot),
                                     _ptr(offsets), _ptr(slot_pos), _ptr(inv)))
    return sorted_slot, offsets, slot_pos, int(inv[0])


def router_topk(logits, k: int, renormalize: bool = True):
    """logits: float32 [T, E].  Returns (ids int32 [T, k], weights float32 [T, k]):
    softmax, the k largest (lower id first among equal logits), renormalised."""
    lg = _c(logits, np.float32)
    T, E = lg.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    _check(_load().oracle_router_topk(_ptr(lg), T, E, k, 1 if renormalize else 0, _ptr(ids), _ptr(w)))
    return ids, w


def _scale_shape(fmt, rows, H):
    if fmt == FMT_FP8_B128:
        return (rows, H // 128), np.float32
    return (rows, H // 32), np.uint8


def quant_rows_bf16(x_bits, fmt: int):
    """x_bits: uint16 [rows, H] (bf16 bit patterns).  Returns (codes u8, scales)."""
    x = _c(x_bits, np.uint16)
    rows, H = x.shape
    codes = np.empty((rows, H), np.uint8)
    shp, dt = _scale_shape(fmt, rows, H)
    scales = np.empty(shp, dt)
    _check(_load().oracle_quant_rows_bf16(_ptr(x), rows, H, fmt, _ptr(codes), _ptr(scales)))
    return codes, scales


def quant_rows_bf16_static(x_bits, fmt: int, scales, row_stride=None):
    """Static per-block quantization: x_bits uint16 [rows, H] (bf16 bit
    patterns) with the caller's block scales (FP8: float32, MX: uint8 UE8M0
    bytes).  ``scales`` is [rows, H/B] (row_stride None: H/B) or one row [H/B]
    for every token (row_stride 0).  Returns the codes u8 [rows, H]."""
    x = _c(x_bits, np.uint16)
    rows, H = x.shape
    nb = H // (128 if fmt == FMT_FP8_B128 else 32)
    sc = _c(scales, np.float32 if fmt == FMT_FP8_B128 else np.uint8)
    if row_stride is None:
        row_stride = 0 if sc.ndim == 1 else nb
    codes = np.empty((rows, H), np.uint8)
    _check(_load().oracle_quant_rows_bf16_static(_ptr(x), rows, H, fmt, _ptr(sc), int(row_stride), _ptr(codes)))
    return codes


def quant_rows_f32(x, fmt: int):
    x = _c(x, np.float32)
    rows, H = x.shape
    codes = np.empty((rows, H), np.uint8)
    shp, dt = _scale_shape(fmt, rows, H)
    scales = np.empty(shp, dt)
    _check(_load().oracle_quant_rows_f32(_ptr(x), rows, H, fmt, _ptr(codes), _ptr(scales)))
    return codes, scales


def grouped_gemm(fmt, a_codes, a_scales, offsets, b_codes, b_scales, N, K, row_index=None, row_div=1):
    """C[r, n] over expert-sorted rows, fp64.  Rows = offsets[E].  BF16: A and B
    are bf16 bit patterns (uint16) and the scales are None."""
    bf = fmt == FMT_BF16
    a_codes = _c(a_codes, np.uint16 if bf else np.uint8)
    a_scales = None if bf else _c(a_scales, np.float32 if fmt == FMT_FP8_B128 else np.uint8)
    offsets = _c(offsets, np.int32)
    b_codes = _c(b_codes, np.uint16 if bf else np.uint8)
    b_scales = None if bf else _c(b_scales, np.float32 if fmt == FMT_FP8_B128 else np.uint8)
    E = offsets.size - 1
    ri = None if row_index is None else _c(row_index, np.int32)
    out = np.zeros((int(offsets[E]), N), np.float64)
    _check(_load().oracle_grouped_gemm(fmt, _ptr(a_codes), _ptr(a_scales), _ptr(ri), row_div, _ptr(offsets),
                                       E, _ptr(b_codes), _ptr(b_scales), N, K, _ptr(out)))
    return out


def forward(fmt, w13, w13_scale, w2, w2_scale, x_bits, ids, wts, swiglu_limit=None, expert_begin=0,
            tokens=None, debug=False, act_scales=None, act_scales_row_stride=None):
    """The experts forward on the host.

    Weights in the nt layout (see ``moe_oracle.cpp``); BF16: bf16 bit patterns
    (uint16) [E, 2I, H] and [E, H, I], scales None.  Returns the bf16 bit
    patterns uint16 [T, H] (rows of tokens not listed in ``tokens`` stay 0) and,
    when ``debug`` is set, a dict of per-slot intermediates.  ``act_scales``
    (static activation scheme): the layer input's precomputed block scales, as
    in quant_rows_bf16_static; None quantizes dynamically.
    """
    bf = fmt == FMT_BF16
    w13 = _c(w13, np.uint16 if bf else np.uint8)
    w2 = _c(w2, np.uint16 if bf else np.uint8)
    sdt = np.float32 if fmt == FMT_FP8_B128 else np.uint8
    w13_scale = None if bf else _c(w13_scale, sdt)
    w2_scale = None if bf else _c(w2_scale, sdt)
    x = _c(x_bits, np.uint16)
    ids = _c(ids, np.int32)
    wts = _c(wts, np.float32)
    T, H = x.shape
    k = ids.shape[1]
    E = w13.shape[0]
    I = w13.shape[1] // 2
    S = T * k
    out = np.zeros((T, H), np.uint16)
    tok = None if tokens is None else _c(tokens, np.int32)
    dbg = {}
    if debug:
        dbg["gu"] = np.full((S, 2 * I), np.nan, np.float32)
        dbg["h_codes"] = np.zeros((S, I), np.uint8)
        shp, dt = _scale_shape(fmt, S, I)
        dbg["h_scales"] = np.zeros(shp, dt)
        dbg["y"] = np.full((S, H), np.nan, np.float32)
    has = 0 if swiglu_limit is None else 1
    lim = 0.0 if swiglu_limit is None else float(swiglu_limit)
    asc = None
    stride = 0
    if act_scales is not None:
        asc = _c(act_scales, np.float32 if fmt == FMT_FP8_B128 else np.uint8)
        nb = H // (128 if fmt == FMT_FP8_B128 else 32)
        stride = act_scales_row_stride if act_scales_row_stride is not None else (0 if asc.ndim == 1 else nb)
    _check(_load().oracle_forward(fmt, E, H, I, _ptr(w13), _ptr(w13_scale), _ptr(w2), _ptr(w2_scale), _ptr(x),
                                  _ptr(ids), _ptr(wts), T, k, expert_begin, has, lim, _ptr(tok),
                                  0 if tok is None else tok.size, _ptr(out),
                                  _ptr(dbg.get("gu")), _ptr(dbg.get("h_codes")), _ptr(dbg.get("h_scales")),
                                  _ptr(dbg.get("y")), _ptr(asc), int(stride)))
    return (out, dbg) if debug else out

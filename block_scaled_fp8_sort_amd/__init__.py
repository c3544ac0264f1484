"""MI355X (gfx950) fine-grained-quantized MoE experts forward.

Thin Python face of the C ABI in ``include/moe.h`` (``libmoe.so``, built by
``block_scaled_fp8_sort_amd.build``).  This module only marshals arguments:
torch supplies device memory and the current HIP stream, and every step of the
forward runs in the library's HIP kernels.  There is no CPU fallback: importing
works without the library, but every call raises if it is missing.

Errors follow the pages' guards: a non-bf16 input raises ValueError, a
non-int8 FP4 weight raises NotImplementedError, tensors on another device raise
RuntimeError.  Both activation schemes are served: dynamic (per-block amax) and
static (the caller's precomputed per-block scales).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "FMT_FP8_B128", "FMT_MXFP8A_MXFP4W", "FMT_BF16", "EPI_STORE_F32", "EPI_SWIGLU_QUANT", "EPI_WEIGHTED_SCATTER",
    "MoeError", "library_path", "load_library", "route_sort", "route_topk", "quant_act", "quant_act_static",
    "prepare_weights",
    "grouped_gemm", "experts_forward", "experts_forward_from_logits", "experts_forward_noalloc",
    "forward_workspace_bytes", "NOALLOC_SCRATCH_BYTES", "Weights",
    "TILE_COUNTERS_INTS", "probe_mfma_rate", "PROBE_KINDS",
]

FMT_FP8_B128 = 0
FMT_MXFP8A_MXFP4W = 1
FMT_BF16 = 2
LAYOUT_NT = 0
LAYOUT_NN = 1
EPI_STORE_F32 = 0
EPI_SWIGLU_QUANT = 1
EPI_WEIGHTED_SCATTER = 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmoe.so")
_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_F32 = ctypes.c_float
_SZ = ctypes.c_size_t


class MoeWeights(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int), ("E", _I32), ("H", _I32), ("I", _I32), ("w13", _P), ("w13_scale", _P),
                ("w2", _P), ("w2_scale", _P)]


class MoeGemmArgs(ctypes.Structure):
    _fields_ = [("weights", ctypes.POINTER(MoeWeights)), ("which", _I32), ("max_rows", _I32),
                ("a_codes", _P), ("a_scales", _P), ("a_rows", _I32), ("a_row_index", _P), ("a_row_divisor", _I32),
                ("expert_offsets", _P), ("epilogue", ctypes.c_int),
                ("c_f32", _P), ("h_codes", _P), ("h_scales", _P), ("has_swiglu_limit", _I32),
                ("swiglu_limit", _F32), ("slot_out", _P), ("top_k_weights", _P), ("slot_of_row", _P),
                ("tile_counters", _P), ("a_scales_sorted", _P)]


class MoeDebug(ctypes.Structure):
    _fields_ = [("sorted_slot", _P), ("expert_offsets", _P), ("act_codes", _P), ("act_scales", _P),
                ("h_codes", _P), ("h_scales", _P)]


class MoeOptions(ctypes.Structure):
    _fields_ = [("has_swiglu_limit", _I32), ("swiglu_limit", _F32), ("expert_begin", _I32),
                ("static_activation_scales", _I32), ("invalid_count", _P), ("debug", ctypes.POINTER(MoeDebug)),
                ("act_scales", _P), ("act_scales_row_stride", _I32)]


class MoeError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name}: {detail}")
        self.status = status


_EXC = {3: ValueError, 4: NotImplementedError, 7: RuntimeError}


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libmoe.so (raises if it was not built: there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m block_scaled_fp8_sort_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_last_error.argtypes = []
    lib.moe_route_sort_workspace.restype = _SZ
    lib.moe_route_sort_workspace.argtypes = [_I32, _I32, _I32]
    lib.moe_route_sort.restype = ctypes.c_int
    lib.moe_route_sort.argtypes = [_P, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _SZ, _P]
    lib.moe_route_topk_workspace.restype = _SZ
    lib.moe_route_topk_workspace.argtypes = [_I32, _I32, _I32]
    lib.moe_route_topk.restype = ctypes.c_int
    lib.moe_route_topk.argtypes = [_P, _I32, _I32, _I32, _I32, _P, _P, _I32, _I32, _P, _P, _P, _P, _P, _SZ, _P]
    lib.moe_quant_act.restype = ctypes.c_int
    lib.moe_quant_act.argtypes = [_P, _I32, _I32, ctypes.c_int, _P, _P, _P]
    lib.moe_quant_act_static.restype = ctypes.c_int
    lib.moe_quant_act_static.argtypes = [_P, _I32, _I32, ctypes.c_int, _P, _I32, _P, _P, _P]
    lib.moe_prepared_weights_size.restype = _SZ
    lib.moe_prepared_weights_size.argtypes = [ctypes.c_int, _I32, _I32, _I32]
    lib.moe_prepare_weights.restype = ctypes.c_int
    lib.moe_prepare_weights.argtypes = [ctypes.c_int, ctypes.c_int, _I32, _I32, _I32, _P, _P, _P, _P, _P, _SZ,
                                        ctypes.POINTER(MoeWeights), _P]
    lib.moe_grouped_gemm.restype = ctypes.c_int
    lib.moe_grouped_gemm.argtypes = [ctypes.POINTER(MoeGemmArgs), _P]
    lib.moe_forward_sorts_scales.restype = _I32
    lib.moe_forward_sorts_scales.argtypes = [_I32, _I32, ctypes.c_int]
    lib.moe_experts_forward_workspace.restype = _SZ
    lib.moe_experts_forward_workspace.argtypes = [_I32, _I32, ctypes.POINTER(MoeWeights)]
    lib.moe_experts_forward.restype = ctypes.c_int
    lib.moe_experts_forward.argtypes = [ctypes.POINTER(MoeWeights), _P, _P, _P, _I32, _I32,
                                        ctypes.POINTER(MoeOptions), _P, _P, _SZ, _P]
    lib.moe_experts_forward_noalloc.restype = ctypes.c_int
    lib.moe_experts_forward_noalloc.argtypes = [ctypes.POINTER(MoeWeights), _P, _P, _P, _I32, _I32,
                                                ctypes.POINTER(MoeOptions), _P, _P]
    lib.moe_clock_stamp.restype = ctypes.c_int
    lib.moe_clock_stamp.argtypes = [ctypes.c_void_p, _I32, ctypes.c_void_p]
    lib.moe_probe_mfma_rate.restype = ctypes.c_int
    lib.moe_probe_mfma_rate.argtypes = [_I32, _I32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
                                        _P]
    lib.moe_experts_forward_from_logits.restype = ctypes.c_int
    lib.moe_experts_forward_from_logits.argtypes = [ctypes.POINTER(MoeWeights), _P, _P, _I32, _I32, _I32, _I32,
                                                    ctypes.POINTER(MoeOptions), _P, _P, _P, _P, _SZ, _P]
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        lib = load_library()
        name = lib.moe_status_string(status).decode()
        detail = lib.moe_last_error().decode()
        exc = _EXC.get(status)
        if exc is not None:
            raise exc(f"{name}: {detail}")
        raise MoeError(status, name, detail)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(device: torch.device):
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype, device=None):
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise RuntimeError(f"{name} is on {t.device}, expected {device} (one device per process)")


def _shape(t: torch.Tensor, name: str, shape: tuple):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_forward_shapes(hidden_states, top_k_index, top_k_weights, weights, out):
    """The shapes the C call takes on trust (it sees bare pointers and uses
    weights.H): refuse any mismatch before the library is called."""
    if hidden_states.dim() != 2:
        raise ValueError(f"hidden_states must be [T, H], got shape {tuple(hidden_states.shape)}")
    T, H = hidden_states.shape
    if H != weights.H:
        raise ValueError(f"hidden_states has H={H} but the weights have H={weights.H}")
    if top_k_index.dim() != 2 or top_k_index.shape[0] != T:
        raise ValueError(f"top_k_index must be [T={T}, k], got shape {tuple(top_k_index.shape)}")
    if top_k_weights is not None:
        _shape(top_k_weights, "top_k_weights", top_k_index.shape)
    if out is not None:
        _shape(out, "out", (T, weights.H))


def _scale_dtype(fmt: int):
    return torch.float32 if fmt == FMT_FP8_B128 else torch.uint8


def _scale_cols(fmt: int, n: int) -> int:
    return n // 128 if fmt == FMT_FP8_B128 else n // 32


def _scale_shape(fmt: int, K: int, rows: int):
    """Shape of K-block-major scales: [K/128, rows] fp32, or [K/128, rows, 4] bytes (MX)."""
    return (K // 128, rows) if fmt == FMT_FP8_B128 else (K // 128, rows, 4)


# ------------------------------------------------------------------ route sort
def route_sort(top_k_index: torch.Tensor, num_experts: int, expert_begin: int = 0, with_slot_pos: bool = True):
    """Stable sort of the flat (token, slot) pairs by local expert id.

    Returns (sorted_slot int32 [T*k], expert_offsets int32 [E+1], slot_pos int32
    [T*k] or None, invalid_count int32 [1]); all stay on the device.
    """
    lib = load_library()
    dev = top_k_index.device
    _need(top_k_index, "top_k_index", torch.int32)
    T, k = top_k_index.shape
    S = T * k
    sorted_slot = torch.empty(S, dtype=torch.int32, device=dev)
    offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
    slot_pos = torch.empty(S, dtype=torch.int32, device=dev) if with_slot_pos else None
    invalid = torch.zeros(1, dtype=torch.int32, device=dev)
    ws_bytes = lib.moe_route_sort_workspace(T, k, num_experts)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    _check(lib.moe_route_sort(_ptr(top_k_index), T, k, num_experts, expert_begin, _ptr(sorted_slot), _ptr(offsets),
                              _ptr(slot_pos), _ptr(invalid), _ptr(ws), ws_bytes, _stream(dev)))
    return sorted_slot, offsets, slot_pos, invalid


# ------------------------------------------------------- router + route sort
def route_topk(router_logits: torch.Tensor, k: int, renormalize: bool = True, num_experts: Optional[int] = None,
               expert_begin: int = 0, sort: bool = True, with_slot_pos: bool = True):
    """Router top-k (softmax over the logits, the k largest, optionally
    renormalised) and the route sort of its ids, in one call (one launch up to
    16 tokens of at most 128 experts).

    router_logits fp32 [T, n_experts].  Returns (top_k_index int32 [T, k],
    top_k_weights fp32 [T, k], sorted_slot, expert_offsets, slot_pos,
    invalid_count); the last four are None when ``sort`` is False.  The sort
    covers ``num_experts`` local experts from ``expert_begin`` (default: all).
    """
    lib = load_library()
    dev = router_logits.device
    _need(router_logits, "router_logits", torch.float32)
    T, n = router_logits.shape
    E = n if num_experts is None else num_experts
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    sorted_slot = offsets = slot_pos = invalid = ws = None
    ws_bytes = 0
    if sort:
        sorted_slot = torch.empty(T * k, dtype=torch.int32, device=dev)
        offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        slot_pos = torch.empty(T * k, dtype=torch.int32, device=dev) if with_slot_pos else None
        invalid = torch.zeros(1, dtype=torch.int32, device=dev)
        ws_bytes = lib.moe_route_topk_workspace(T, k, E)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    _check(lib.moe_route_topk(_ptr(router_logits), T, n, k, 1 if renormalize else 0, _ptr(ids), _ptr(w), E,
                              expert_begin, _ptr(sorted_slot), _ptr(offsets), _ptr(slot_pos), _ptr(invalid), _ptr(ws),
                              ws_bytes, _stream(dev)))
    return ids, w, sorted_slot, offsets, slot_pos, invalid


# -------------------------------------------------------------- quantization
def quant_act(x: torch.Tensor, fmt: int = FMT_FP8_B128):
    """Dynamic per-block quantization of bf16 rows.

    Returns K-block-major codes uint8 [H/128, rows, 128] and scales [H/128, rows]
    (fp32, FP8_B128) or [H/128, rows, 4] (uint8 UE8M0, MX).
    """
    lib = load_library()
    _need(x, "x", torch.bfloat16)
    rows, H = x.shape
    codes = torch.empty((H // 128, rows, 128), dtype=torch.uint8, device=x.device)
    scales = torch.empty(_scale_shape(fmt, H, rows), dtype=_scale_dtype(fmt), device=x.device)
    _check(lib.moe_quant_act(_ptr(x), rows, H, fmt, _ptr(codes), _ptr(scales), _stream(x.device)))
    return codes, scales


def _static_scales(act_scales: torch.Tensor, fmt: int, rows: int, H: int, device):
    """Checks a static scale tensor ([rows, H/B] per token, or [H/B] for every
    token) and returns its row stride in elements."""
    if fmt not in (FMT_FP8_B128, FMT_MXFP8A_MXFP4W):
        raise NotImplementedError("static activation scales need a quantized format (FP8_B128 or MX)")
    nb = H // 128 if fmt == FMT_FP8_B128 else H // 32
    dt = torch.float32 if fmt == FMT_FP8_B128 else torch.uint8
    _need(act_scales, "act_scales", dt, device)
    if act_scales.dim() == 1:
        _shape(act_scales, "act_scales", (nb,))
        return 0
    _shape(act_scales, "act_scales", (rows, nb))
    return nb


def quant_act_static(x: torch.Tensor, act_scales: torch.Tensor, fmt: int = FMT_FP8_B128):
    """Static per-block quantization of bf16 rows with the caller's block scales
    (act_scales: fp32 [rows, H/128] for FP8_B128 or uint8 UE8M0 [rows, H/32]
    for MX; a 1-D [H/B] tensor serves every row).  Returns (codes, scales) as
    quant_act does."""
    lib = load_library()
    _need(x, "x", torch.bfloat16)
    rows, H = x.shape
    stride = _static_scales(act_scales, fmt, rows, H, x.device)
    codes = torch.empty((H // 128, rows, 128), dtype=torch.uint8, device=x.device)
    scales = torch.empty(_scale_shape(fmt, H, rows), dtype=_scale_dtype(fmt), device=x.device)
    _check(lib.moe_quant_act_static(_ptr(x), rows, H, fmt, _ptr(act_scales), stride, _ptr(codes), _ptr(scales),
                                    _stream(x.device)))
    return codes, scales


# ------------------------------------------------------------------- weights
class Weights:
    """Prepared expert weights: the C descriptor plus the tensors it points at."""

    def __init__(self, desc: MoeWeights, keep: tuple):
        self.desc = desc
        self._keep = keep

    @property
    def fmt(self):
        return self.desc.fmt

    @property
    def E(self):
        return self.desc.E

    @property
    def H(self):
        return self.desc.H

    @property
    def I(self):
        return self.desc.I


def prepare_weights(gate_up: torch.Tensor, gate_up_scale: torch.Tensor, down: torch.Tensor,
                    down_scale: torch.Tensor, fmt: int = FMT_FP8_B128, transposed: bool = False) -> Weights:
    """One-shot weight preparation into the library's tiled layout.

    FP8_B128: gate_up uint8 [E, 2I, H] (or [E, H, 2I] when transposed), fp32 scales
    per 128x128 block; down uint8 [E, H, I].  MX: int8/uint8 packed e2m1
    [E, 2I, H/2] and [E, H, I/2] with uint8 UE8M0 scales per 1x32 (nt only).
    BF16: bfloat16 [E, 2I, H] and [E, H, I] (or [E, H, 2I] and [E, I, H] when
    transposed), no scales (pass None).
    """
    lib = load_library()
    dev = gate_up.device
    if fmt == FMT_MXFP8A_MXFP4W and gate_up.dtype not in (torch.int8, torch.uint8):
        raise NotImplementedError(f"MXFP4 experts need FP4-packed int8 weights, got {gate_up.dtype}")
    for name, t in (("gate_up", gate_up), ("down", down)):
        if fmt == FMT_BF16:
            if t.dtype != torch.bfloat16:
                raise ValueError(f"{name} must be bfloat16 for the bf16 experts, got {t.dtype}")
        elif t.dtype not in (torch.uint8, torch.int8, torch.float8_e4m3fn):
            raise ValueError(f"{name} must hold 8-bit codes, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if gate_up.dim() != 3 or down.dim() != 3:
        raise ValueError("gate_up and down must be 3-D [E, rows, cols]")
    E = gate_up.shape[0]
    if fmt in (FMT_BF16, FMT_FP8_B128):
        H, I2 = (gate_up.shape[1], gate_up.shape[2]) if transposed else (gate_up.shape[2], gate_up.shape[1])
    else:
        if transposed:
            raise ValueError("MX weights are accepted in the nt layout only")
        H, I2 = gate_up.shape[2] * 2, gate_up.shape[1]
    I = I2 // 2
    if I2 % 2:
        raise ValueError(f"gate_up has {I2} gate+up rows, which is odd")
    # every array the C call reads, at the shape it assumes for (fmt, layout, E, H, I)
    if fmt == FMT_FP8_B128:
        _shape(down, "down", (E, I, H) if transposed else (E, H, I))
        for name, t in (("gate_up_scale", gate_up_scale), ("down_scale", down_scale)):
            if t is None or t.dtype != torch.float32 or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous float32 tensor")
        _shape(gate_up_scale, "gate_up_scale",
               (E, H // 128, I2 // 128) if transposed else (E, I2 // 128, H // 128))
        _shape(down_scale, "down_scale", (E, I // 128, H // 128) if transposed else (E, H // 128, I // 128))
    elif fmt == FMT_MXFP8A_MXFP4W:
        _shape(down, "down", (E, H, I // 2))
        for name, t in (("gate_up_scale", gate_up_scale), ("down_scale", down_scale)):
            if t is None or t.dtype not in (torch.uint8, torch.int8) or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous uint8 tensor of UE8M0 bytes")
        _shape(gate_up_scale, "gate_up_scale", (E, I2, H // 32))
        _shape(down_scale, "down_scale", (E, H, I // 32))
    else:
        _shape(down, "down", (E, I, H) if transposed else (E, H, I))
    read = [("gate_up", gate_up), ("down", down)]
    if fmt != FMT_BF16:
        read += [("gate_up_scale", gate_up_scale), ("down_scale", down_scale)]
    for name, t in read:
        if t.device != dev:
            raise RuntimeError(f"{name} is on {t.device}, expected {dev} (one device per process)")
    desc = MoeWeights()
    nbytes = lib.moe_prepared_weights_size(fmt, E, H, I)
    prepared = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _check(lib.moe_prepare_weights(fmt, LAYOUT_NN if transposed else LAYOUT_NT, E, H, I, _ptr(gate_up),
                                   _ptr(gate_up_scale), _ptr(down), _ptr(down_scale), _ptr(prepared), nbytes,
                                   ctypes.byref(desc), _stream(dev)))
    return Weights(desc, (prepared,))


# -------------------------------------------------------------- grouped GEMM
TILE_COUNTERS_INTS = 256  # MOE_TILE_COUNTERS_BYTES / 4


def grouped_gemm(weights: Weights, which: int, a_codes, a_scales, a_rows: int, expert_offsets, epilogue: int,
                 max_rows: int, a_row_index=None, a_row_divisor: int = 1, c_f32=None, h_codes=None, h_scales=None,
                 swiglu_limit: Optional[float] = None, slot_out=None, top_k_weights=None, slot_of_row=None,
                 tile_counters="new", a_scales_sorted=None):
    """Enqueue one grouped GEMM (see moe_grouped_gemm); outputs are caller tensors.

    a_scales_sorted: optional copy of the activation scales by sorted row (as
    the forward builds for large batches, see forward_sorts_scales), read by the
    256-row tiled paths instead of a_scales at the gathered rows.

    which = 0 multiplies by the gate_up weight, 1 by the down weight.  A is
    K-block-major with a_rows rows per plane.  tile_counters: "new" (default)
    allocates zeroed counters for dynamic tile dispensing, as the fused forward
    uses; a caller's int32 tensor of TILE_COUNTERS_INTS zeros may be reused
    across launches that do not overlap (each launch leaves it zero); None takes
    tiles in the fixed round-robin order.
    """
    lib = load_library()
    a = MoeGemmArgs()
    a.weights = ctypes.pointer(weights.desc)
    a.which = which
    a.max_rows = max_rows
    a.a_codes, a.a_scales, a.a_rows = _ptr(a_codes), _ptr(a_scales), a_rows
    a.a_row_index, a.a_row_divisor = _ptr(a_row_index), a_row_divisor
    a.expert_offsets = _ptr(expert_offsets)
    a.epilogue = epilogue
    a.c_f32, a.h_codes, a.h_scales = _ptr(c_f32), _ptr(h_codes), _ptr(h_scales)
    a.has_swiglu_limit = 0 if swiglu_limit is None else 1
    a.swiglu_limit = 0.0 if swiglu_limit is None else float(swiglu_limit)
    a.slot_out, a.top_k_weights, a.slot_of_row = _ptr(slot_out), _ptr(top_k_weights), _ptr(slot_of_row)
    if isinstance(tile_counters, str):
        tile_counters = torch.zeros(TILE_COUNTERS_INTS, dtype=torch.int32, device=a_codes.device)
    elif tile_counters is not None:
        _need(tile_counters, "tile_counters", torch.int32)
        if tile_counters.numel() < TILE_COUNTERS_INTS:
            raise ValueError(f"tile_counters needs {TILE_COUNTERS_INTS} int32")
    a.tile_counters = _ptr(tile_counters)
    a.a_scales_sorted = _ptr(a_scales_sorted)
    _check(lib.moe_grouped_gemm(ctypes.byref(a), _stream(a_codes.device)))


# ------------------------------------------------------------ fused forward
def forward_sorts_scales(T: int, k: int, fmt: int) -> bool:
    """Whether the forward hands its gate_up GEMM a copy of the activation
    scales by sorted row (moe_forward_sorts_scales)."""
    return bool(load_library().moe_forward_sorts_scales(T, k, fmt))


NOALLOC_SCRATCH_BYTES = 64 << 20  # MOE_NOALLOC_SCRATCH_BYTES

_ws_cache: dict = {}


def _pow2_tokens(T: int) -> int:
    # sized for the next power of two, as the pages size their buffers: a batch
    # that grows reallocates a few times, for at most twice the memory
    return 1 << (T - 1).bit_length() if T > 0 else 0


def forward_workspace_bytes(T: int, k: int, weights: Weights) -> int:
    return load_library().moe_experts_forward_workspace(T, k, ctypes.byref(weights.desc))


def _workspace(T: int, k: int, weights: Weights, device) -> torch.Tensor:
    # one cached workspace per (device, stream, layer shape): two forwards on
    # different streams must not share scratch while both run, and forwards on
    # one stream run one after the other
    need = forward_workspace_bytes(_pow2_tokens(T), k, weights)
    key = (device, _stream(device), weights.E, weights.H, weights.I, weights.fmt, k)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def _options(swiglu_limit, expert_begin, invalid_count, act_scales=None, act_stride=0):
    opt = MoeOptions()
    opt.has_swiglu_limit = 0 if swiglu_limit is None else 1
    opt.swiglu_limit = 0.0 if swiglu_limit is None else float(swiglu_limit)
    opt.expert_begin = expert_begin
    opt.static_activation_scales = 0 if act_scales is None else 1
    opt.invalid_count = _ptr(invalid_count)
    opt.act_scales = _ptr(act_scales)
    opt.act_scales_row_stride = act_stride
    return opt


def _scheme(activation_scheme: str, act_scales, weights, T, H, device):
    """Static scales (and their row stride) for the forward, or (None, 0)."""
    if activation_scheme not in ("dynamic", "static"):
        raise ValueError(f"activation_scheme must be 'dynamic' or 'static', got {activation_scheme!r}")
    if activation_scheme == "dynamic":
        if act_scales is not None:
            raise ValueError("act_scales are the static scheme's; pass activation_scheme='static'")
        return None, 0
    if act_scales is None:
        raise ValueError("activation_scheme='static' needs the precomputed per-block act_scales")
    return act_scales, _static_scales(act_scales, weights.fmt, T, H, device)


def experts_forward_from_logits(hidden_states: torch.Tensor, router_logits: torch.Tensor, k: int,
                                weights: Weights, renormalize: bool = True, swiglu_limit: Optional[float] = None,
                                expert_begin: int = 0, out: Optional[torch.Tensor] = None,
                                top_k_index: Optional[torch.Tensor] = None,
                                top_k_weights: Optional[torch.Tensor] = None,
                                workspace: Optional[torch.Tensor] = None,
                                invalid_count: Optional[torch.Tensor] = None,
                                activation_scheme: str = "dynamic", act_scales: Optional[torch.Tensor] = None):
    """The experts forward from the router's logits (see route_topk): returns
    (out bf16 [T, H], top_k_index int32 [T, k], top_k_weights fp32 [T, k])."""
    lib = load_library()
    if hidden_states.dtype != torch.bfloat16:
        raise ValueError(f"the experts forward requires bfloat16 hidden states, got {hidden_states.dtype}")
    dev = hidden_states.device
    _need(hidden_states, "hidden_states", torch.bfloat16, dev)
    _need(router_logits, "router_logits", torch.float32, dev)
    if hidden_states.dim() != 2 or router_logits.dim() != 2:
        raise ValueError("hidden_states and router_logits must be 2-D")
    T, H = hidden_states.shape
    n = router_logits.shape[1]
    if router_logits.shape[0] != T:
        raise ValueError(f"router_logits has {router_logits.shape[0]} rows for {T} tokens")
    if out is None:
        out = torch.empty((T, weights.H), dtype=torch.bfloat16, device=dev)
    if top_k_index is None:
        top_k_index = torch.empty((T, k), dtype=torch.int32, device=dev)
    if top_k_weights is None:
        top_k_weights = torch.empty((T, k), dtype=torch.float32, device=dev)
    _need(top_k_index, "top_k_index", torch.int32, dev)
    _need(top_k_weights, "top_k_weights", torch.float32, dev)
    _need(out, "out", torch.bfloat16, dev)
    _shape(top_k_index, "top_k_index", (T, k))
    _check_forward_shapes(hidden_states, top_k_index, top_k_weights, weights, out)
    asc, astride = _scheme(activation_scheme, act_scales, weights, T, H, dev)
    if T > 0 and workspace is None:
        workspace = _workspace(T, k, weights, dev)
    opt = _options(swiglu_limit, expert_begin, invalid_count, asc, astride)
    _check(lib.moe_experts_forward_from_logits(ctypes.byref(weights.desc), _ptr(hidden_states), _ptr(router_logits), T,
                                               n, k, 1 if renormalize else 0, ctypes.byref(opt), _ptr(top_k_index),
                                               _ptr(top_k_weights), _ptr(out), _ptr(workspace),
                                               0 if workspace is None else workspace.numel(), _stream(dev)))
    return out, top_k_index, top_k_weights


def experts_forward(hidden_states: torch.Tensor, top_k_index: torch.Tensor, top_k_weights: torch.Tensor,
                    weights: Weights, swiglu_limit: Optional[float] = None, expert_begin: int = 0,
                    activation_scheme: str = "dynamic", out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, invalid_count: Optional[torch.Tensor] = None,
                    debug: Optional[dict] = None, act_scales: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The fused experts forward: out[t] = sum_j w[t, j] * expert_{id[t, j]}(hidden_states[t]).

    hidden_states bf16 [T, H]; top_k_index int32 [T, k] (global ids, -1 skips the
    slot); top_k_weights fp32 [T, k].  Returns bf16 [T, H].
    activation_scheme "dynamic" quantizes hidden_states per block from its own
    amax; "static" uses act_scales, the precomputed block scales (fp32
    [T, H/128] for FP8_B128, uint8 UE8M0 [T, H/32] for MX, or one [H/B] row
    for every token).
    """
    lib = load_library()
    if hidden_states.dtype != torch.bfloat16:
        raise ValueError(f"the experts forward requires bfloat16 hidden states, got {hidden_states.dtype}")
    dev = hidden_states.device
    _need(hidden_states, "hidden_states", torch.bfloat16, dev)
    _need(top_k_index, "top_k_index", torch.int32, dev)
    _need(top_k_weights, "top_k_weights", torch.float32, dev)
    _check_forward_shapes(hidden_states, top_k_index, top_k_weights, weights, out)
    T, H = hidden_states.shape
    k = top_k_index.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, dev)
    asc, astride = _scheme(activation_scheme, act_scales, weights, T, H, dev)
    if T == 0:
        return out
    if workspace is None:
        workspace = _workspace(T, k, weights, dev)
    opt = _options(swiglu_limit, expert_begin, invalid_count, asc, astride)
    dbg = None
    if debug is not None:
        S = T * k
        debug["sorted_slot"] = torch.empty(S, dtype=torch.int32, device=dev)
        debug["expert_offsets"] = torch.empty(weights.E + 1, dtype=torch.int32, device=dev)
        debug["act_codes"] = torch.empty((H // 128, T, 128), dtype=torch.uint8, device=dev)
        debug["act_scales"] = torch.empty(_scale_shape(weights.fmt, H, T), dtype=_scale_dtype(weights.fmt),
                                          device=dev)
        if weights.fmt != FMT_BF16:
            I = weights.I
            debug["h_codes"] = torch.empty((I // 128, S, 128), dtype=torch.uint8, device=dev)
            debug["h_scales"] = torch.empty(_scale_shape(weights.fmt, I, S), dtype=_scale_dtype(weights.fmt),
                                            device=dev)
        dbg = MoeDebug(_ptr(debug["sorted_slot"]), _ptr(debug["expert_offsets"]), _ptr(debug["act_codes"]),
                       _ptr(debug["act_scales"]), _ptr(debug.get("h_codes")), _ptr(debug.get("h_scales")))
        opt.debug = ctypes.pointer(dbg)
    _check(lib.moe_experts_forward(ctypes.byref(weights.desc), _ptr(hidden_states), _ptr(top_k_index),
                                   _ptr(top_k_weights), T, k, ctypes.byref(opt), _ptr(out), _ptr(workspace),
                                   workspace.numel(), _stream(dev)))
    return out


def experts_forward_noalloc(hidden_states: torch.Tensor, top_k_index: torch.Tensor, top_k_weights: torch.Tensor,
                            weights: Weights, swiglu_limit: Optional[float] = None, expert_begin: int = 0,
                            out: Optional[torch.Tensor] = None, invalid_count: Optional[torch.Tensor] = None,
                            activation_scheme: str = "dynamic",
                            act_scales: Optional[torch.Tensor] = None) -> torch.Tensor:
    """experts_forward through moe_experts_forward_noalloc: the library's own
    per-GPU scratch (NOALLOC_SCRATCH_BYTES) replaces the workspace, so the C call
    allocates nothing (pass ``out`` to allocate nothing here either).  Calls
    that overlap on one GPU share that scratch and must not run concurrently."""
    lib = load_library()
    if hidden_states.dtype != torch.bfloat16:
        raise ValueError(f"the experts forward requires bfloat16 hidden states, got {hidden_states.dtype}")
    dev = hidden_states.device
    _need(hidden_states, "hidden_states", torch.bfloat16, dev)
    _need(top_k_index, "top_k_index", torch.int32, dev)
    _need(top_k_weights, "top_k_weights", torch.float32, dev)
    _check_forward_shapes(hidden_states, top_k_index, top_k_weights, weights, out)
    T, H = hidden_states.shape
    k = top_k_index.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, dev)
    asc, astride = _scheme(activation_scheme, act_scales, weights, T, H, dev)
    opt = _options(swiglu_limit, expert_begin, invalid_count, asc, astride)
    _check(lib.moe_experts_forward_noalloc(ctypes.byref(weights.desc), _ptr(hidden_states), _ptr(top_k_index),
                                           _ptr(top_k_weights), T, k, ctypes.byref(opt), _ptr(out), _stream(dev)))
    return out


# The MFMA forms moe_probe_mfma_rate measures, by kind.
PROBE_KINDS = {
    0: "e4m3 x e4m3 16x16x128",
    1: "e2m1 x e4m3 16x16x128, UE8M0 scales (the MX GEMM's form)",
    2: "e2m1 x e2m1 16x16x128, UE8M0 scales",
    3: "bf16 16x16x32",
    4: "e4m3 x e4m3 16x16x128 + fp32 promotion (the FP8 GEMM's form)",
}


def clock_stamp(n: int = 1024, device: Optional[torch.device] = None) -> torch.Tensor:
    """Enqueue one set of clock stamps (moe_clock_stamp) on the current stream:
    an int64 device tensor [n, 3] of (compute unit: XCD id * 256 + its SE / array
    / CU ids, that unit's shader-clock counter, 100 MHz real-time counter), one
    row per one-wave workgroup.  Two stamps bracket the work enqueued between
    them (shader_clock_ghz)."""
    lib = load_library()
    dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    out = torch.empty((int(n), 3), dtype=torch.int64, device=dev)
    _check(lib.moe_clock_stamp(out.data_ptr(), int(n), _stream(dev)))
    return out


def shader_clock_ghz(before: torch.Tensor, after: torch.Tensor) -> dict:
    """Mean shader clock per XCD (GHz) between two clock_stamp results: for each
    compute unit stamped in both, its shader-clock ticks over the 100 MHz
    real-time ticks (the counters of different units are not aligned); per
    XCD, the mean over its units.  Synchronizes with the device."""
    a, b = before.cpu(), after.cpu()

    def first(t):
        d = {}
        for u, clk, real in t.tolist():
            d.setdefault(int(u), (clk, real))
        return d

    fa, fb = first(a), first(b)
    per_xcd = {}
    for u in sorted(set(fa) & set(fb)):
        dt, dr = fb[u][0] - fa[u][0], fb[u][1] - fa[u][1]
        if dr > 0:
            per_xcd.setdefault(u // 256, []).append(dt / dr * 0.1)
    return {x: sum(v) / len(v) for x, v in per_xcd.items()}


def probe_mfma_rate(kind: int, iters: int = 20000, device: Optional[torch.device] = None):
    """The matrix cores' issue rate for one MFMA form (moe_probe_mfma_rate): random
    operands in registers, 8 waves on every CU.  Returns (TFLOP/s, mean shader
    clock in GHz).  A measurement utility; blocks until the probe has run."""
    lib = load_library()
    dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    tf, ghz = ctypes.c_double(), ctypes.c_double()
    _check(lib.moe_probe_mfma_rate(int(kind), int(iters), ctypes.byref(tf), ctypes.byref(ghz), _stream(dev)))
    return tf.value, ghz.value

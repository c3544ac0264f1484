"""The C-ABI library on the host: it loads, exports every function include/moe.h
declares, and refuses bad calls before touching the GPU (no GPU here)."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import block_scaled_fp8_sort_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

OK, NULL, SHAPE, DTYPE, UNSUP, WS = 0, 1, 2, 3, 4, 5


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.library_path()):
        import block_scaled_fp8_sort_amd.build as b
        b.build()
    return moe.load_library()


def test_library_exports_every_declared_function(lib):
    names = _declared_functions()
    assert "moe_experts_forward" in names and "moe_grouped_gemm" in names
    assert len(names) == 18
    for n in names:
        assert hasattr(lib, n), n


def test_forward_sorts_scales(lib):
    # the forward copies the activation scales by sorted row exactly where it
    # takes the multi-workgroup sort (16384 slots and more), quantized formats only
    assert lib.moe_forward_sorts_scales(2048, 8, 0) == 1
    assert lib.moe_forward_sorts_scales(2047, 8, 0) == 0
    assert lib.moe_forward_sorts_scales(16384, 8, 1) == 1
    assert lib.moe_forward_sorts_scales(4096, 8, 2) == 0  # bf16: no scales
    assert lib.moe_forward_sorts_scales(0, 8, 0) == 0
    assert lib.moe_forward_sorts_scales(4096, 8, 9) == 0
    assert lib.moe_forward_sorts_scales(4096, 0, 0) == 0
    assert moe.forward_sorts_scales(8192, 8, moe.FMT_FP8_B128) and not moe.forward_sorts_scales(64, 8, 0)


def test_status_strings(lib):
    assert lib.moe_status_string(0) == b"MOE_OK"
    assert lib.moe_status_string(5) == b"MOE_ERR_WORKSPACE"


def test_route_sort_refusals(lib):
    p = ctypes.c_void_p(16)  # never dereferenced: the calls fail validation first
    assert lib.moe_route_sort(p, 4, 0, 8, 0, p, p, None, None, None, 0, None) == SHAPE
    assert lib.moe_route_sort(p, 4, 65, 8, 0, p, p, None, None, None, 0, None) == SHAPE
    assert lib.moe_route_sort(p, 4, 2, 0, 0, p, p, None, None, None, 0, None) == SHAPE
    assert lib.moe_route_sort(p, 4, 2, 513, 0, p, p, None, None, None, 0, None) == SHAPE
    assert lib.moe_route_sort(p, -1, 2, 8, 0, p, p, None, None, None, 0, None) == SHAPE
    assert lib.moe_route_sort(p, 4, 2, 8, -1, p, p, None, None, None, 0, None) == SHAPE  # -1 must stay skipped
    assert lib.moe_route_sort(None, 4, 2, 8, 0, p, p, None, None, None, 0, None) == NULL
    assert lib.moe_route_sort(p, 4, 2, 8, 0, p, None, None, None, None, 0, None) == NULL
    assert lib.moe_route_sort(p, 4, 2, 8, 0, p, ctypes.c_void_p(32), None, None, None, 0, None) == UNSUP
    assert b"alias" in lib.moe_last_error()
    # an empty batch passes validation even though its (empty) arrays share an address


def test_route_sort_workspace(lib):
    # one workgroup below 16384 slots (no workspace); above, per-chunk
    # histograms of E + 2 rows over at most 2048 chunks of at least 256 slots,
    # and the E + 2 row totals
    assert lib.moe_route_sort_workspace(64, 8, 128) == 0
    assert lib.moe_route_sort_workspace(16383, 1, 8) == 0
    assert lib.moe_route_sort_workspace(2048, 8, 256) == 4 * 258 * (64 + 1)  # 64 chunks of 256 slots
    assert lib.moe_route_sort_workspace(8192, 8, 256) == 4 * 258 * (256 + 1)
    assert lib.moe_route_sort_workspace(65536, 8, 256) == 4 * 258 * (2048 + 1)  # 2048 chunks of 256
    for T, k, E in [(16384, 8, 256), (40000, 8, 512), (1 << 26, 16, 512)]:
        ws = lib.moe_route_sort_workspace(T, k, E)
        assert 0 < ws <= 4 * (E + 2) * (2048 + 1)
    assert lib.moe_route_sort_workspace(-1, 8, 8) == 0
    p = ctypes.c_void_p(16)
    assert lib.moe_route_sort(p, 2048, 8, 256, 0, ctypes.c_void_p(64), p, None, None, None, 0, None) == WS
    assert lib.moe_route_sort(p, 2048, 8, 256, 0, ctypes.c_void_p(64), p, None, None, p, 100, None) == WS


def test_route_topk_refusals(lib):
    p = ctypes.c_void_p(16)
    q, r, u = ctypes.c_void_p(48), ctypes.c_void_p(80), ctypes.c_void_p(112)

    def call(T=4, n=8, k=2, ids=q, w=r, E=8, ss=u, off=ctypes.c_void_p(144), ws=None, ws_bytes=0, logits=p, begin=0):
        return lib.moe_route_topk(logits, T, n, k, 1, ids, w, E, begin, ss, off, None, None, ws, ws_bytes, None)

    assert call(begin=-1) == SHAPE

    assert call(k=9) == SHAPE  # k > n_experts
    assert call(k=0) == SHAPE
    assert call(n=0) == SHAPE
    assert call(n=513, k=2) == SHAPE
    assert call(T=-1) == SHAPE
    assert call(E=0) == SHAPE
    assert call(logits=None) == NULL
    assert call(ids=None) == NULL
    assert call(off=None) == NULL  # sorted_slot without expert_offsets
    assert call(ss=None) == NULL  # the sort needs sorted_slot when T > 0
    assert call(ids=p) == UNSUP  # top_k_index aliases the logits
    assert b"alias" in lib.moe_last_error()
    assert call(w=q) == UNSUP
    assert call(ss=q) == UNSUP
    assert call(T=2048, n=256, k=8, E=256) == WS  # multi-workgroup sort needs its histograms
    assert call(T=0, ss=None, off=None, ids=None, w=None, logits=None) == OK  # router alone, nothing to do
    assert lib.moe_route_topk_workspace(2048, 8, 256) == lib.moe_route_sort_workspace(2048, 8, 256)


def test_forward_from_logits_refusals(lib):
    p = ctypes.c_void_p(16)
    w = _weights()

    def fwd(T=8, n=8, k=2, logits=ctypes.c_void_p(24), ids=ctypes.c_void_p(48), wts=ctypes.c_void_p(80),
            out=ctypes.c_void_p(112), ws=ctypes.c_void_p(64), ws_bytes=1 << 40):
        return lib.moe_experts_forward_from_logits(ctypes.byref(w), p, logits, T, n, k, 1, None, ids, wts, out, ws,
                                                   ws_bytes, None)

    assert fwd(k=9) == SHAPE
    assert fwd(n=0) == SHAPE
    assert fwd(n=600) == SHAPE
    assert fwd(T=0) == OK
    assert fwd(logits=None) == NULL
    assert fwd(ids=None) == NULL
    assert fwd(ids=ctypes.c_void_p(24)) == UNSUP  # top_k_index aliases the logits
    assert fwd(wts=ctypes.c_void_p(48)) == UNSUP  # the two routing outputs alias
    assert fwd(out=ctypes.c_void_p(80)) == UNSUP
    assert fwd(ws=None) == WS


def test_quant_refusals(lib):
    p = ctypes.c_void_p(16)
    q = ctypes.c_void_p(48)
    assert lib.moe_quant_act(p, 4, 100, 0, q, q, None) == SHAPE
    assert lib.moe_quant_act(p, 4, 128, 7, q, q, None) == UNSUP
    assert lib.moe_quant_act(None, 4, 128, 0, q, q, None) == NULL
    assert lib.moe_quant_act(p, 0, 128, 0, q, q, None) == OK  # nothing to do, nothing enqueued


def _weights(E=4, H=256, I=128, fmt=0):
    w = moe.MoeWeights()
    w.fmt, w.E, w.H, w.I = fmt, E, H, I
    w.w13 = w.w13_scale = w.w2 = w.w2_scale = 64
    return w


def test_forward_refusals(lib):
    p = ctypes.c_void_p(16)
    w = _weights()
    opt = moe.MoeOptions()

    def fwd(w=w, T=8, k=2, opt=None, out=ctypes.c_void_p(32), ws=ctypes.c_void_p(64), ws_bytes=1 << 40):
        return lib.moe_experts_forward(ctypes.byref(w), p, p, p, T, k, None if opt is None else ctypes.byref(opt),
                                       out, ws, ws_bytes, None)

    assert fwd(T=0) == OK
    assert fwd(k=0) == SHAPE
    # quantized formats: the rows of a 128-wide K plane are addressed with
    # 32-bit offsets, so T*k*128 must stay below 2^31
    assert fwd(T=1 << 21, k=8) == SHAPE
    assert b"2^31" in lib.moe_last_error()
    assert fwd(T=(1 << 21) - 1, k=8, ws=None) == WS  # one slot under the bound gets past the shape checks
    assert fwd(w=_weights(H=200)) == SHAPE
    assert fwd(w=_weights(I=64)) == SHAPE
    assert fwd(w=_weights(E=0)) == SHAPE
    assert fwd(w=_weights(fmt=9)) == UNSUP
    opt.expert_begin = -1
    assert fwd(opt=opt) == SHAPE
    opt.expert_begin = 0
    # the static activation scheme: needs its scales, a quantized format and a
    # row stride of 0 or at least one row of block scales
    opt.static_activation_scales = 1
    assert fwd(opt=opt) == NULL
    assert b"act_scales" in lib.moe_last_error()
    opt.act_scales = 48
    opt.act_scales_row_stride = 1  # H = 256: two FP8 block scales per row
    assert fwd(opt=opt) == SHAPE
    opt.act_scales_row_stride = -2
    assert fwd(opt=opt) == SHAPE
    opt.act_scales_row_stride = 2
    assert fwd(opt=opt, ws=None) == WS  # past every static check
    opt.act_scales_row_stride = 0
    assert fwd(opt=opt, ws=None) == WS
    assert fwd(w=_weights(fmt=2), opt=opt) == UNSUP  # bf16 experts quantize nothing
    assert b"static" in lib.moe_last_error()
    assert fwd(opt=opt, out=ctypes.c_void_p(48)) == UNSUP  # out aliases act_scales
    opt.static_activation_scales = 0
    opt.act_scales = None
    opt.has_swiglu_limit, opt.swiglu_limit = 1, float("nan")
    assert fwd(opt=opt) == SHAPE
    opt.swiglu_limit = -2.0
    assert fwd(opt=opt) == SHAPE
    opt.swiglu_limit = float("inf")
    assert fwd(opt=opt) == SHAPE
    assert fwd(ws=None) == WS
    need = lib.moe_experts_forward_workspace(8, 2, ctypes.byref(w))
    assert need > 0
    assert fwd(ws_bytes=need - 1) == WS
    assert fwd(out=p) == UNSUP  # out aliases hidden_states

    def fwd3(x, ids, wts, out):
        return lib.moe_experts_forward(ctypes.byref(w), ctypes.c_void_p(x), ctypes.c_void_p(ids),
                                       ctypes.c_void_p(wts), 8, 2, None, ctypes.c_void_p(out), ctypes.c_void_p(64),
                                       1 << 40, None)

    assert fwd3(16, 24, 40, 24) == UNSUP  # out aliases top_k_index (the combine reads it while writing out)
    assert fwd3(16, 24, 40, 40) == UNSUP  # out aliases top_k_weights
    assert b"alias" in lib.moe_last_error()
    bad = _weights()
    bad.w2 = None
    assert fwd(w=bad) == NULL


def test_gemm_refusals(lib):
    w = _weights()
    a = moe.MoeGemmArgs()
    a.weights = ctypes.pointer(w)
    a.which, a.max_rows, a.a_rows = 0, 64, 64
    a.a_codes, a.a_scales, a.expert_offsets = 16, 24, 32
    a.epilogue = moe.EPI_STORE_F32
    assert lib.moe_grouped_gemm(ctypes.byref(a), None) == NULL  # c_f32 missing
    for alias in (16, 24, 32):  # an output may not alias an input of the launch
        a.c_f32 = alias
        assert lib.moe_grouped_gemm(ctypes.byref(a), None) == UNSUP
    a.c_f32 = 40
    a.which = 2
    assert lib.moe_grouped_gemm(ctypes.byref(a), None) == UNSUP
    a.which = 0
    a.a_rows = 10  # fewer A rows than max_rows without a row index
    assert lib.moe_grouped_gemm(ctypes.byref(a), None) == SHAPE
    a.a_rows = 64
    a.epilogue = moe.EPI_SWIGLU_QUANT
    a.h_codes, a.h_scales = 48, 56
    a.which = 1
    assert lib.moe_grouped_gemm(ctypes.byref(a), None) == UNSUP  # SwiGLU only on gate_up
    a.which = 0
    a.has_swiglu_limit, a.swiglu_limit = 1, 0.0
    assert lib.moe_grouped_gemm(ctypes.byref(a), None) == SHAPE
    a.epilogue = 9
    assert lib.moe_grouped_gemm(ctypes.byref(a), None) == UNSUP
    a.epilogue = moe.EPI_STORE_F32
    a.tile_counters = 4100  # the dispensers are 64-bit counters
    assert lib.moe_grouped_gemm(ctypes.byref(a), None) == SHAPE
    a.tile_counters = None
    a.max_rows = 0
    assert lib.moe_grouped_gemm(ctypes.byref(a), None) == OK  # nothing to do
    bad = _weights(H=100)
    a.weights = ctypes.pointer(bad)
    assert lib.moe_grouped_gemm(ctypes.byref(a), None) == SHAPE


def test_prepare_weights_refusals_and_sizes(lib):
    desc = moe.MoeWeights()
    p = ctypes.c_void_p(4096)
    assert lib.moe_prepare_weights(0, 0, 4, 256, 128, p, p, p, p, None, 0, ctypes.byref(desc), None) == NULL
    assert lib.moe_prepare_weights(0, 0, 4, 256, 128, p, p, p, p, p, 10, ctypes.byref(desc), None) == WS
    assert lib.moe_prepare_weights(1, 1, 4, 256, 128, p, p, p, p, p, 1 << 30, ctypes.byref(desc), None) == UNSUP
    assert lib.moe_prepare_weights(0, 0, 4, 200, 128, p, p, p, p, p, 1 << 30, ctypes.byref(desc), None) == SHAPE
    # FP8: tiled gate_up 4*256*256, its scales 4*2*2 floats, tiled down (H=256 -> one 256-row tile) 4*256*128,
    # its scales 4*2*1 floats, each rounded up to 256 bytes
    assert lib.moe_prepared_weights_size(0, 4, 256, 128) == 4 * 256 * 256 + 256 + 4 * 256 * 128 + 256
    # H = 384 pads the down weight to two 256-row tiles
    assert lib.moe_prepared_weights_size(0, 1, 384, 128) == 256 * 384 + 256 + 2 * 256 * 128 + 256
    assert lib.moe_prepared_weights_size(0, 4, 250, 128) == 0


def test_python_face_raises_like_the_pages():
    x = torch.zeros((4, 256), dtype=torch.float32)
    ids = torch.zeros((4, 2), dtype=torch.int32)
    w = torch.ones((4, 2), dtype=torch.float32)
    with pytest.raises(ValueError, match="bfloat16"):
        moe.experts_forward(x, ids, w, weights=None)
    with pytest.raises(NotImplementedError, match="int8"):
        moe.prepare_weights(torch.zeros(2, 4, dtype=torch.float16), None, None, None, fmt=moe.FMT_MXFP8A_MXFP4W)


def _fake_weights(E=4, H=256, I=128, fmt=0):
    return moe.Weights(_weights(E, H, I, fmt), ())


def test_python_forward_shape_refusals():
    """Shapes the C call takes on trust (bare pointers, sizes from the weight
    descriptor) are refused in Python before the library is called: a mismatch
    would otherwise become an out-of-bounds device access."""
    wt = _fake_weights()  # H = 256
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    ids = torch.zeros((4, 2), dtype=torch.int32)
    w = torch.ones((4, 2), dtype=torch.float32)
    cases = [
        (dict(hidden_states=torch.zeros((4, 384), dtype=torch.bfloat16)), "H=384"),
        (dict(hidden_states=torch.zeros((4, 2, 128), dtype=torch.bfloat16)), r"\[T, H\]"),
        (dict(top_k_index=torch.zeros((5, 2), dtype=torch.int32)), "top_k_index"),
        (dict(top_k_index=torch.zeros(8, dtype=torch.int32)), "top_k_index"),
        (dict(top_k_weights=torch.ones((4, 3), dtype=torch.float32)), "top_k_weights"),
        (dict(out=torch.empty((4, 128), dtype=torch.bfloat16)), "out"),
    ]
    for over, msg in cases:
        a = dict(hidden_states=x, top_k_index=ids, top_k_weights=w)
        a.update(over)
        with pytest.raises(ValueError, match=msg):
            moe.experts_forward(a["hidden_states"], a["top_k_index"], a["top_k_weights"], wt, out=a.get("out"))
    with pytest.raises(ValueError, match="out"):
        moe.experts_forward(x, ids, w, wt, out=torch.empty((4, 256), dtype=torch.float32))
    logits = torch.zeros((4, 8), dtype=torch.float32)
    with pytest.raises(ValueError, match="rows"):
        moe.experts_forward_from_logits(x, torch.zeros((5, 8)), 2, wt)
    with pytest.raises(ValueError, match="H=384"):
        moe.experts_forward_from_logits(torch.zeros((4, 384), dtype=torch.bfloat16), logits, 2, wt)
    with pytest.raises(ValueError, match="top_k_index"):
        moe.experts_forward_from_logits(x, logits, 2, wt, top_k_index=torch.zeros((4, 3), dtype=torch.int32))
    with pytest.raises(ValueError, match="out"):
        moe.experts_forward_from_logits(x, logits, 2, wt, out=torch.empty((4, 512), dtype=torch.bfloat16))


def test_python_static_scheme_refusals():
    wt = _fake_weights()  # FP8, H = 256: two block scales per token
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    ids = torch.zeros((4, 2), dtype=torch.int32)
    w = torch.ones((4, 2), dtype=torch.float32)
    with pytest.raises(ValueError, match="act_scales"):
        moe.experts_forward(x, ids, w, wt, activation_scheme="static")
    with pytest.raises(ValueError, match="static"):
        moe.experts_forward(x, ids, w, wt, act_scales=torch.ones((4, 2)))
    with pytest.raises(ValueError, match="activation_scheme"):
        moe.experts_forward(x, ids, w, wt, activation_scheme="per_tensor")
    with pytest.raises(ValueError, match="act_scales"):
        moe.experts_forward(x, ids, w, wt, activation_scheme="static", act_scales=torch.ones((4, 3)))
    with pytest.raises(ValueError, match="act_scales"):
        moe.experts_forward(x, ids, w, wt, activation_scheme="static", act_scales=torch.ones(2, dtype=torch.float64))
    with pytest.raises(NotImplementedError, match="quantized"):
        moe.experts_forward(x, ids, w, _fake_weights(fmt=2), activation_scheme="static", act_scales=torch.ones(2))
    with pytest.raises(ValueError, match="act_scales"):  # MX: one UE8M0 byte per 32 columns
        moe.quant_act_static(x, torch.ones((4, 2), dtype=torch.uint8), fmt=moe.FMT_MXFP8A_MXFP4W)


def test_quant_static_refusals(lib):
    p = ctypes.c_void_p(16)
    q = lambda **kw: lib.moe_quant_act_static(kw.get("x", p), kw.get("rows", 4), kw.get("H", 256), kw.get("fmt", 0),
                                              kw.get("sc", ctypes.c_void_p(24)), kw.get("stride", 2),
                                              kw.get("codes", ctypes.c_void_p(32)), kw.get("scales", ctypes.c_void_p(40)),
                                              None)
    assert q(rows=0) == OK
    assert q(fmt=2) == UNSUP
    assert q(fmt=7) == UNSUP
    assert q(H=200) == SHAPE
    assert q(stride=1) == SHAPE
    assert q(stride=-1) == SHAPE
    assert q(fmt=1, stride=4) == SHAPE  # MX: 8 block scales per row of 256
    assert q(sc=None) == NULL
    assert q(codes=ctypes.c_void_p(24)) == UNSUP  # codes alias the input scales
    assert q(scales=p) == UNSUP  # scales alias x


def test_python_prepare_weights_shape_refusals():
    E, H, I = 2, 384, 128
    u8 = lambda *s: torch.zeros(s, dtype=torch.uint8)
    f32 = lambda *s: torch.ones(s, dtype=torch.float32)
    good = dict(gate_up=u8(E, 2 * I, H), gate_up_scale=f32(E, 2 * I // 128, H // 128), down=u8(E, H, I),
                down_scale=f32(E, H // 128, I // 128))
    bad = [
        ("down", u8(E, H, 2 * I)), ("down", u8(E + 1, H, I)), ("gate_up_scale", f32(E, H // 128, 2 * I // 128)),
        ("down_scale", f32(E, I // 128, H // 128)), ("gate_up_scale", torch.ones((E, 2, 2), dtype=torch.float64)),
        ("gate_up", u8(E, 2 * I + 1, H)),
    ]
    for name, t in bad:
        a = dict(good)
        a[name] = t
        with pytest.raises(ValueError):
            moe.prepare_weights(a["gate_up"], a["gate_up_scale"], a["down"], a["down_scale"], fmt=moe.FMT_FP8_B128)
    # MX: packed codes [E, 2I, H/2] and [E, H, I/2], UE8M0 bytes [E, 2I, H/32] and [E, H, I/32]
    mx = dict(gate_up=u8(E, 2 * I, H // 2), gate_up_scale=u8(E, 2 * I, H // 32), down=u8(E, H, I // 2),
              down_scale=u8(E, H, I // 32))
    for name, t in (("down", u8(E, H, I)), ("down_scale", u8(E, H, I // 128)), ("gate_up_scale", u8(E, 2 * I, H // 128)),
                    ("down_scale", f32(E, H, I // 32))):
        a = dict(mx)
        a[name] = t
        with pytest.raises(ValueError):
            moe.prepare_weights(a["gate_up"], a["gate_up_scale"], a["down"], a["down_scale"],
                                fmt=moe.FMT_MXFP8A_MXFP4W)
    with pytest.raises(ValueError, match="nt"):
        moe.prepare_weights(mx["gate_up"], mx["gate_up_scale"], mx["down"], mx["down_scale"],
                            fmt=moe.FMT_MXFP8A_MXFP4W, transposed=True)


def test_workspace_sized_for_next_power_of_two():
    path = os.path.join(ROOT, "tests", "golden", "pow2_buffer_tokens.txt")
    rows = [tuple(int(v) for v in l.split()) for l in open(path) if l.strip() and not l.startswith("#")]
    for n, sized in rows:
        assert moe._pow2_tokens(n) == sized
        assert sized < 2 * n or n == 1


def test_bf16_format_on_the_host(lib):
    # prepared size: the two bf16 weights tiled, each rounded up to 256 bytes; the
    # down weight's rows (H) padded to whole 256-row tiles
    assert lib.moe_prepared_weights_size(2, 4, 256, 128) == 4 * 256 * 256 * 2 + 4 * 256 * 128 * 2
    assert lib.moe_prepared_weights_size(2, 3, 384, 128) == 3 * 256 * 384 * 2 + 3 * 512 * 128 * 2
    desc = moe.MoeWeights()
    p = ctypes.c_void_p(4096)
    # the nn layout is refused for MX only; bf16 scale pointers may be NULL (with
    # no GPU here, both bf16 layouts get as far as the device check)
    assert lib.moe_prepare_weights(1, 1, 4, 256, 128, p, p, p, p, p, 1 << 30, ctypes.byref(desc), None) == UNSUP
    for layout in (0, 1):
        assert lib.moe_prepare_weights(2, layout, 4, 256, 128, p, None, p, None, p, 1 << 30, ctypes.byref(desc),
                                       None) not in (UNSUP, NULL)
    assert lib.moe_prepare_weights(0, 0, 4, 256, 128, p, None, p, None, p, 1 << 30, ctypes.byref(desc), None) == NULL
    # the forward's workspace holds no activation codes for bf16 but h in bf16
    w8, wb = _weights(fmt=0), _weights(fmt=2)
    assert lib.moe_experts_forward_workspace(64, 2, ctypes.byref(wb)) > 0
    assert lib.moe_experts_forward_workspace(64, 2, ctypes.byref(wb)) != lib.moe_experts_forward_workspace(
        64, 2, ctypes.byref(w8))
    # a bf16 GEMM needs no scales: with a_scales NULL it fails only on the missing output
    a = moe.MoeGemmArgs()
    wb.w13_scale = wb.w2_scale = None
    a.weights = ctypes.pointer(wb)
    a.which, a.max_rows, a.a_rows = 0, 64, 64
    a.a_codes = a.expert_offsets = 16
    a.epilogue = moe.EPI_STORE_F32
    assert lib.moe_grouped_gemm(ctypes.byref(a), None) == NULL
    assert b"c_f32" in lib.moe_last_error()
    w8.w13_scale = None
    a.weights = ctypes.pointer(w8)
    assert lib.moe_grouped_gemm(ctypes.byref(a), None) == NULL
    assert b"scale" in lib.moe_last_error()


def test_noalloc_forward_host_refusals(lib):
    """The forward without allocation refuses, on the host, anything its scratch
    cannot hold (and the usual bad arguments) before touching the GPU."""
    p = ctypes.c_void_p(16)
    big = _weights(E=8, H=4096, I=14336)
    assert lib.moe_experts_forward_workspace(4096, 2, ctypes.byref(big)) > moe.NOALLOC_SCRATCH_BYTES
    assert lib.moe_experts_forward_noalloc(ctypes.byref(big), p, p, p, 4096, 2, None, ctypes.c_void_p(32), None) == WS
    assert b"no-allocation" in lib.moe_last_error()
    small = _weights()
    assert lib.moe_experts_forward_noalloc(ctypes.byref(small), p, p, p, 0, 2, None, ctypes.c_void_p(32), None) == OK
    assert lib.moe_experts_forward_noalloc(ctypes.byref(small), p, p, p, 8, 0, None, ctypes.c_void_p(32), None) == SHAPE
    assert lib.moe_experts_forward_noalloc(ctypes.byref(_weights(H=100)), p, p, p, 8, 2, None, ctypes.c_void_p(32),
                                           None) == SHAPE


def test_mfma_probe_host_refusals(lib):
    """The matrix-core rate probe refuses bad arguments on the host, before
    touching the GPU (its kinds are the MFMA forms the GEMMs use)."""
    d = ctypes.c_double()
    assert lib.moe_probe_mfma_rate(0, 100, None, ctypes.byref(d), None) == NULL
    assert lib.moe_probe_mfma_rate(5, 100, ctypes.byref(d), ctypes.byref(d), None) == UNSUP
    assert lib.moe_probe_mfma_rate(-1, 100, ctypes.byref(d), ctypes.byref(d), None) == UNSUP
    assert lib.moe_probe_mfma_rate(0, 0, ctypes.byref(d), ctypes.byref(d), None) == SHAPE
    assert lib.moe_probe_mfma_rate(0, (1 << 24) + 1, ctypes.byref(d), ctypes.byref(d), None) == SHAPE
    assert sorted(moe.PROBE_KINDS) == [0, 1, 2, 3, 4]


def test_clock_stamp_host_refusals(lib):
    """The clock stamps refuse a NULL output and a stamp count outside
    [1, 4096] on the host, before touching the GPU."""
    dummy = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails first
    assert lib.moe_clock_stamp(None, 64, None) == NULL
    assert lib.moe_clock_stamp(dummy, 0, None) == SHAPE
    assert lib.moe_clock_stamp(dummy, 4097, None) == SHAPE
    assert lib.moe_clock_stamp(dummy, -1, None) == SHAPE

"""The forward without allocation (moe_experts_forward_noalloc), called through
the C ABI: the same kernels as moe_experts_forward on the library's own per-GPU
scratch, so the same output bit for bit.  Two calls in a row, the second with a
smaller batch (the scratch keeps the first call's contents, which must not
leak into the second), on two layers; and a forward too large for the scratch
is refused on the host before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import block_scaled_fp8_sort_amd as moe
import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _opt(limit):
    opt = moe.MoeOptions()
    opt.has_swiglu_limit = 0 if limit is None else 1
    opt.swiglu_limit = 0.0 if limit is None else float(limit)
    return opt


def _noalloc(lib, w, x, ids, wts, limit):
    """One call of the C entry point on torch's current stream; returns (status, out)."""
    T, k = ids.shape
    out = torch.full((T, w.H), float("nan"), dtype=torch.bfloat16, device=DEV)
    opt = _opt(limit)
    st = lib.moe_experts_forward_noalloc(ctypes.byref(w.desc), x.data_ptr(), ids.data_ptr(), wts.data_ptr(), T, k,
                                         ctypes.byref(opt), out.data_ptr(),
                                         torch.cuda.current_stream(DEV).cuda_stream)
    return st, out


CASES = [
    W.WORKLOADS["qwen3_moe_decode"],
    W.Workload("noalloc_mx_clamp", T=300, H=384, I=256, E=7, k=4, fmt=W.FMT_MX, routing="zipf", zipf_s=1.1,
               skip=0.1, swiglu_limit=7.0, seed=15),
]


@pytest.mark.parametrize("wl", CASES, ids=[w.name for w in CASES])
def test_noalloc_forward_equals_the_workspace_forward(wl):
    print(f"noalloc forward {wl.name}", flush=True)
    lib = moe.load_library()
    inp = W.inputs(wl, DEV)
    w = moe.prepare_weights(inp["w13"], inp["s13"], inp["w2"], inp["s2"], fmt=wl.fmt)
    assert moe.forward_workspace_bytes(wl.T, wl.k, w) <= moe.NOALLOC_SCRATCH_BYTES
    for T in (wl.T, wl.T * 3 // 8):  # the second call smaller than the first
        x = inp["x"][:T].contiguous()
        ids = inp["ids"][:T].contiguous()
        wts = inp["w"][:T].contiguous()
        ref = moe.experts_forward(x, ids, wts, w, swiglu_limit=wl.swiglu_limit).clone()
        st, out = _noalloc(lib, w, x, ids, wts, wl.swiglu_limit)
        torch.cuda.synchronize()
        assert st == 0, lib.moe_last_error().decode()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"T={T}"
        # the Python face of the same entry point
        again = moe.experts_forward_noalloc(x, ids, wts, w, swiglu_limit=wl.swiglu_limit)
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int16), ref.view(torch.int16)), f"T={T} (binding)"


def test_noalloc_refuses_a_forward_larger_than_its_scratch():
    lib = moe.load_library()
    wd = moe.MoeWeights()
    wd.fmt, wd.E, wd.H, wd.I = 0, 8, 4096, 14336
    wd.w13 = wd.w13_scale = wd.w2 = wd.w2_scale = 64  # never dereferenced: refused on the host
    p = ctypes.c_void_p(16)
    assert lib.moe_experts_forward_workspace(4096, 2, ctypes.byref(wd)) > moe.NOALLOC_SCRATCH_BYTES
    st = lib.moe_experts_forward_noalloc(ctypes.byref(wd), p, p, p, 4096, 2, None, ctypes.c_void_p(32),
                                         torch.cuda.current_stream(DEV).cuda_stream)
    assert st == 5 and b"no-allocation" in lib.moe_last_error()

"""GPU parity of the router row: softmax top-k fused with the route sort, and the
experts forward started from router logits, called through the C ABI and
checked against the CPU oracle.

Bit-exact: the chosen ids and their order, sorted_slot, expert_offsets,
slot_pos and the invalid count.  Routing weights: within the relative bound the
library states, (n_experts + 4 + 2 (max - min logit of the token)) * 2^-24 (one
rounding of l - max, exp to about 1 ulp, fp32 sums over at most n_experts
terms, one division).  Forward outputs: the forward's own bar, max|err| <=
1e-2 * max|ref| and relative L2 <= 5e-3, and bit-identical to the forward given
the same routing.
"""
import sys

import numpy as np
import pytest
import torch

import block_scaled_fp8_sort_amd as moe
import oracle
import workloads as W
from parity_checks import assert_forward_parity, flip_explainer

pytestmark = pytest.mark.gpu

FP8, MX = W.FMT_FP8_B128, W.FMT_MX
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t):
    return W.to_numpy(t)


def assert_weights_close(got, ref, logits, n_experts):
    spread = logits.max(axis=1) - logits.min(axis=1)
    tol = (n_experts + 4 + 2 * spread.astype(np.float64))[:, None] * 2.0 ** -24
    rel = np.abs(got.astype(np.float64) - ref.astype(np.float64)) / np.abs(ref.astype(np.float64))
    worst = float(np.max(rel / tol)) if rel.size else 0.0
    say(f"  weights: worst relative error / bound = {worst:.3f}")
    assert np.all(rel <= tol), f"weights off by {np.max(rel)} (bound {np.min(tol)})"


# T, n_experts, k, renormalize, ties, local experts (E, expert_begin) or None = all
ROUTER_CASES = [
    (1, 1, 1, True, False, None),
    (16, 128, 8, True, True, None),         # small decode: router inside the sort's workgroup
    (11, 100, 6, False, False, None),
    (64, 128, 8, True, False, None),        # decode: router launch, then the one-workgroup sort
    (64, 128, 8, False, True, None),
    (4096, 8, 2, True, False, None),        # T * n_experts = 32768: still one workgroup
    (700, 100, 3, True, True, None),        # 70000 logits: router launch of its own, one-workgroup sort
    (8192, 256, 8, True, False, None),      # multi-workgroup sort
    (16384, 256, 8, False, True, None),
    (333, 5, 5, True, False, None),         # k = n_experts
    (50, 512, 64, True, True, None),        # the largest n_experts and k
    (1000, 60, 6, True, False, None),       # 64 lanes per token, partly idle
    (3000, 7, 7, False, True, None),
    (513, 256, 8, True, False, (64, 96)),   # one GPU's share of 64 experts
    (9000, 64, 4, True, True, (16, 40)),    # the share, with the multi-workgroup sort
]


@pytest.mark.parametrize("T,n,k,renorm,ties,local", ROUTER_CASES)
def test_route_topk_bit_exact(T, n, k, renorm, ties, local):
    say(f"route_topk T={T} n_experts={n} k={k} renorm={renorm} ties={ties} local={local}")
    lg = W.router_logits(T, n, seed=T + n + k, device=DEV, ties=ties)
    E, begin = local if local else (n, 0)
    ids, w, ss, off, sp, inv = moe.route_topk(lg, k, renorm, num_experts=E, expert_begin=begin)
    torch.cuda.synchronize()
    lg_h = host(lg)
    o_ids, o_w = oracle.router_topk(lg_h, k, renorm)
    assert np.array_equal(host(ids), o_ids)
    assert_weights_close(host(w), o_w, lg_h, n)
    o_ss, o_off, o_sp, o_inv = oracle.route_sort(o_ids, E, expert_begin=begin)
    assert np.array_equal(host(off), o_off)
    assert np.array_equal(host(ss), o_ss)
    assert np.array_equal(host(sp), o_sp)
    assert int(host(inv)[0]) == o_inv


def test_route_topk_router_alone_and_empty():
    lg = W.router_logits(2000, 96, seed=5, device=DEV)
    ids, w, ss, off, sp, inv = moe.route_topk(lg, 6, sort=False)
    torch.cuda.synchronize()
    assert ss is None and off is None
    o_ids, o_w = oracle.router_topk(host(lg), 6)
    assert np.array_equal(host(ids), o_ids)
    assert_weights_close(host(w), o_w, host(lg), 96)
    ids, w, ss, off, sp, inv = moe.route_topk(lg[:0], 6)
    torch.cuda.synchronize()
    assert ids.shape == (0, 6) and list(host(off)) == [0] * 97


def _workload(name, fmt, T, H, I, E, k, limit=None, seed=0):
    return W.Workload(name, T=T, H=H, I=I, E=E, k=k, fmt=fmt, routing="uniform", swiglu_limit=limit, seed=seed)


FWD_CASES = [
    _workload("logits_small_decode_fp8", FP8, T=16, H=512, I=256, E=16, k=4, seed=30),  # router+sort+quant in one launch
    _workload("logits_decode_fp8", FP8, T=24, H=512, I=256, E=16, k=4, seed=31),       # router launch, fused sort+quant
    _workload("logits_ragged_fp8", FP8, T=300, H=384, I=256, E=6, k=3, seed=32),
    # 70000 logits: the router runs as a launch of its own
    _workload("logits_router_launch", FP8, T=700, H=512, I=256, E=100, k=3, seed=33),
    _workload("logits_router_launch_i128", FP8, T=700, H=512, I=128, E=100, k=3, seed=33),
    _workload("logits_mx_clamp", MX, T=200, H=256, I=256, E=8, k=2, limit=7.0, seed=34),
]


@pytest.mark.parametrize("wl", FWD_CASES, ids=[w.name for w in FWD_CASES])
def test_forward_from_logits_parity(wl):
    say(f"forward from logits {wl.name}")
    inp = W.inputs(wl, DEV)
    lg = W.router_logits(wl.T, wl.E, seed=wl.seed, device=DEV)
    w = moe.prepare_weights(inp["w13"], inp["s13"], inp["w2"], inp["s2"], fmt=wl.fmt)
    out, ids, wts = moe.experts_forward_from_logits(inp["x"], lg, wl.k, w, swiglu_limit=wl.swiglu_limit)
    out = out.clone()
    torch.cuda.synchronize()
    lg_h = host(lg)
    o_ids, o_w = oracle.router_topk(lg_h, wl.k)
    assert np.array_equal(host(ids), o_ids)
    assert_weights_close(host(wts), o_w, lg_h, wl.E)
    # the same kernels as the forward given this routing: identical bits
    dbg = {}
    same = moe.experts_forward(inp["x"], ids, wts, w, swiglu_limit=wl.swiglu_limit, debug=dbg)
    torch.cuda.synchronize()
    assert np.array_equal(host(out).view(np.uint16), host(same).view(np.uint16))
    n = {k_: host(v) for k_, v in inp.items()}
    ref = oracle.forward(wl.fmt, n["w13"], n["s13"], n["w2"], n["s2"], n["x"], o_ids, o_w,
                         swiglu_limit=wl.swiglu_limit)
    got = host(out)
    # the explanation path runs on the router's own choice (the same ids and
    # weights the GPU used, equal to the oracle's ids, weights to 1 fp32 rounding)
    n_gpu = dict(n, ids=host(ids), w=host(wts))
    assert_forward_parity(wl.name, got, ref,
                          flip_explainer(wl.fmt, wl.T, wl.k, wl.H, wl.I, n_gpu, got, dbg, swiglu_limit=wl.swiglu_limit))


def test_forward_from_logits_full_decode_sampled():
    """The decode-sized layer (64 tokens, hidden 2048, intermediate 768, 128
    experts, top-8) from its logits, in the launch configuration the benchmark
    times; the oracle recomputes a seeded sample of tokens."""
    wl = W.WORKLOADS["qwen3_moe_decode"]
    inp = W.inputs(wl, DEV)
    lg = W.router_logits(wl.T, wl.E, seed=wl.seed, device=DEV)
    w = moe.prepare_weights(inp["w13"], inp["s13"], inp["w2"], inp["s2"], fmt=wl.fmt)
    out, ids, wts = moe.experts_forward_from_logits(inp["x"], lg, wl.k, w)
    torch.cuda.synchronize()
    o_ids, o_w = oracle.router_topk(host(lg), wl.k)
    assert np.array_equal(host(ids), o_ids)
    tokens = W.sample_tokens(wl.T, 48, wl.seed)
    n = {k_: host(v) for k_, v in inp.items()}
    ref = oracle.forward(wl.fmt, n["w13"], n["s13"], n["w2"], n["s2"], n["x"], o_ids, o_w, tokens=tokens)
    g = torch.from_numpy(host(out)[tokens].view(np.int16)).view(torch.bfloat16).double().numpy()
    r = torch.from_numpy(ref[tokens].view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.max(np.abs(g - r)) <= 1e-2 * np.max(np.abs(r))
    assert np.linalg.norm(g - r) / np.linalg.norm(r) <= 5e-3


def test_forward_from_logits_graph_replay():
    """Captured in a HIP graph, the forward from logits replays bit-exactly."""
    wl = FWD_CASES[0]
    inp = W.inputs(wl, DEV)
    lg = W.router_logits(wl.T, wl.E, seed=wl.seed, device=DEV)
    w = moe.prepare_weights(inp["w13"], inp["s13"], inp["w2"], inp["s2"], fmt=wl.fmt)
    ref, _, _ = moe.experts_forward_from_logits(inp["x"], lg, wl.k, w)
    ref = ref.clone()
    torch.cuda.synchronize()
    out = torch.empty_like(ref)
    ids = torch.empty((wl.T, wl.k), dtype=torch.int32, device=DEV)
    wts = torch.empty((wl.T, wl.k), dtype=torch.float32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moe.experts_forward_from_logits(inp["x"], lg, wl.k, w, out=out, top_k_index=ids, top_k_weights=wts)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.experts_forward_from_logits(inp["x"], lg, wl.k, w, out=out, top_k_index=ids, top_k_weights=wts)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        ids.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out).view(np.uint16), host(ref).view(np.uint16)), f"replay {rep}"


# ------------------------------------------------ one GPU's share under EP
EP_CASES = [
    _workload("ep_fp8_tiled", FP8, T=333, H=512, I=256, E=12, k=4, seed=41),
    _workload("ep_fp8_few_rows", FP8, T=40, H=512, I=256, E=32, k=4, seed=42),
    _workload("ep_mx_clamp", MX, T=250, H=256, I=256, E=8, k=3, limit=7.0, seed=43),
    # 16800 slots: the whole batch takes the multi-workgroup sort (with a nonzero
    # expert_begin in the expert-group test), the token slices the one-workgroup sort
    _workload("ep_fp8_multiblock_sort", FP8, T=4200, H=256, I=128, E=16, k=4, seed=44),
]


@pytest.mark.parametrize("wl", EP_CASES, ids=[w.name for w in EP_CASES])
@pytest.mark.parametrize("world", [2, 3])
def test_ep_equal_token_slices_gather_to_the_full_batch(wl, world):
    """The Mega MoE EP implementation hands each rank an equal slice of the
    batch, pads the last slice with skipped slots and all-gathers the outputs
    ("deepgemm_megamoe EP implementation for DeepGEMM Mega MoE", "How it runs").
    Each slice is one call here; tokens are independent, so the gathered
    slices equal the whole-batch forward on every real token, and padded rows
    are exact zeros."""
    inp = W.inputs(wl, DEV)
    w = moe.prepare_weights(inp["w13"], inp["s13"], inp["w2"], inp["s2"], fmt=wl.fmt)
    full = moe.experts_forward(inp["x"], inp["ids"], inp["w"], w, swiglu_limit=wl.swiglu_limit).clone()
    per = -(-wl.T // world)
    pad = per * world - wl.T
    x = torch.cat([inp["x"], torch.zeros((pad, wl.H), dtype=torch.bfloat16, device=DEV)])
    ids = torch.cat([inp["ids"], torch.full((pad, wl.k), -1, dtype=torch.int32, device=DEV)])
    wts = torch.cat([inp["w"], torch.full((pad, wl.k), float("nan"), dtype=torch.float32, device=DEV)])
    outs = [moe.experts_forward(x[r * per:(r + 1) * per].contiguous(), ids[r * per:(r + 1) * per].contiguous(),
                                wts[r * per:(r + 1) * per].contiguous(), w, swiglu_limit=wl.swiglu_limit).clone()
            for r in range(world)]
    gathered = torch.cat(outs)
    torch.cuda.synchronize()
    g, f = host(gathered).view(np.uint16), host(full).view(np.uint16)
    ref = oracle.forward(wl.fmt, *(host(inp[n]) for n in ("w13", "s13", "w2", "s2", "x", "ids", "w")),
                         swiglu_limit=wl.swiglu_limit)
    ga = torch.from_numpy(g[:wl.T].view(np.int16)).view(torch.bfloat16).double().numpy()
    ra = torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.max(np.abs(ga - ra)) <= 1e-2 * np.max(np.abs(ra))
    assert np.linalg.norm(ga - ra) / np.linalg.norm(ra) <= 5e-3
    assert not np.any(g[wl.T:]), "padded slots must give exact zeros"
    # a slice that runs the same GEMM path as the whole batch gives the same bits
    if (per * wl.k <= 8 * wl.E) == (wl.T * wl.k <= 8 * wl.E):
        assert np.array_equal(g[:wl.T], f)


@pytest.mark.parametrize("wl", EP_CASES, ids=[w.name for w in EP_CASES])
def test_ep_expert_groups_sum_to_the_full_layer(wl):
    """Expert parallelism without moving tokens ("all_reduce" in the pages' EP
    table): each rank holds E / G experts (expert_begin), runs them over the
    whole batch with global ids, and the partial outputs are summed.  Ids of
    other ranks' experts are skipped there and counted as out of range."""
    G = 4 if wl.E % 4 == 0 else 2
    inp = W.inputs(wl, DEV)
    n = {k_: host(v) for k_, v in inp.items()}
    Eg = wl.E // G
    parts = []
    for r in range(G):
        sl = slice(r * Eg, (r + 1) * Eg)
        w = moe.prepare_weights(inp["w13"][sl].contiguous(), inp["s13"][sl].contiguous(), inp["w2"][sl].contiguous(),
                                inp["s2"][sl].contiguous(), fmt=wl.fmt)
        inv = torch.zeros(1, dtype=torch.int32, device=DEV)
        out = moe.experts_forward(inp["x"], inp["ids"], inp["w"], w, swiglu_limit=wl.swiglu_limit, expert_begin=r * Eg,
                                  invalid_count=inv)
        torch.cuda.synchronize()
        ids = n["ids"]
        assert int(host(inv)[0]) == int(((ids >= 0) & ((ids < r * Eg) | (ids >= (r + 1) * Eg))).sum())
        # this rank's partial against the oracle run on the same share
        ref_r = oracle.forward(wl.fmt, n["w13"][sl], n["s13"][sl], n["w2"][sl], n["s2"][sl], n["x"], ids, n["w"],
                               swiglu_limit=wl.swiglu_limit, expert_begin=r * Eg)
        p = torch.from_numpy(host(out).view(np.int16)).view(torch.bfloat16).double().numpy()
        rr = torch.from_numpy(ref_r.view(np.int16)).view(torch.bfloat16).double().numpy()
        assert np.max(np.abs(p - rr)) <= 1e-2 * np.max(np.abs(rr))
        parts.append(p)
    full = oracle.forward(wl.fmt, n["w13"], n["s13"], n["w2"], n["s2"], n["x"], n["ids"], n["w"],
                          swiglu_limit=wl.swiglu_limit)
    fr = torch.from_numpy(full.view(np.int16)).view(torch.bfloat16).double().numpy()
    total = np.sum(parts, axis=0)
    assert np.max(np.abs(total - fr)) <= 1e-2 * np.max(np.abs(fr))
    assert np.linalg.norm(total - fr) / np.linalg.norm(fr) <= 5e-3

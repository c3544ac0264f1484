"""GPU parity of the unquantized bf16 experts (the pages' grouped_mm fallback),
called through the C ABI, against the CPU oracle.

Bit-exact: the route sort (shared with the quantized path).  Tolerances: the
grouped GEMM alone within 2e-5 of max|C| (bf16 products are exact in fp32; the
MFMA and the oracle sum K of them in different orders, fp32 against fp64);
forward outputs within the forward's bar, max|err| <= 1e-2 * max|ref| and
relative L2 <= 5e-3 (h is rounded to bf16 on both sides from differently
rounded fp32 / fp64 values, so a few h elements may differ by one bf16 ulp).
"""
import sys

import numpy as np
import pytest
import torch

import block_scaled_fp8_sort_amd as moe
import oracle
import workloads as W

pytestmark = pytest.mark.gpu

BF16 = W.FMT_BF16
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t):
    return W.to_numpy(t)


def bits_to_f64(b):
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).double().numpy()


def assert_out_close(got_bits, ref_bits, what=""):
    g, r = bits_to_f64(got_bits), bits_to_f64(ref_bits)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    max_ref = np.max(np.abs(r))
    max_err = np.max(np.abs(g - r))
    rel_l2 = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)
    say(f"  {what}: max|err| / max|ref| = {max_err / max(max_ref, 1e-30):.2e}, rel L2 = {rel_l2:.2e}")
    assert max_err <= 1e-2 * max_ref
    assert rel_l2 <= 5e-3


def _rand_ids(rng, T, k, E, p_skip):
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    ids[rng.random((T, k)) < p_skip] = -1
    return ids


@pytest.mark.parametrize("which", [0, 1])
@pytest.mark.parametrize("E,H,I,T,k", [(3, 256, 128, 40, 2), (5, 640, 384, 700, 3), (2, 384, 1024, 300, 1),
                                       (16, 512, 256, 24, 4)])
def test_bf16_grouped_gemm_store_f32(which, E, H, I, T, k):
    say(f"bf16 gemm store f32 which={which} E={E} H={H} I={I} T={T} k={k}")
    seed = H + I + T + which
    rng = np.random.default_rng(seed)
    w13 = W.bf16_weights(E, 2 * I, H, seed, "w13", DEV)
    w2 = W.bf16_weights(E, H, I, seed, "w2", DEV)
    w = moe.prepare_weights(w13, None, w2, None, fmt=moe.FMT_BF16)
    N, K = (2 * I, H) if which == 0 else (H, I)
    x = W.hidden_states(T, K, seed, DEV)
    ids = torch.from_numpy(_rand_ids(rng, T, k, E, 0.1)).to(DEV)
    ss, off, _, _ = moe.route_sort(ids, E)
    S = T * k
    c = torch.full((S, N), float("nan"), dtype=torch.float32, device=DEV)
    moe.grouped_gemm(w, which, x, None, T, off, moe.EPI_STORE_F32, S, a_row_index=ss, a_row_divisor=k, c_f32=c)
    torch.cuda.synchronize()
    offs = host(off)
    b = host(w13) if which == 0 else host(w2)
    ref = oracle.grouped_gemm(BF16, host(x), None, offs, b, None, N, K, row_index=host(ss), row_div=k)
    got = host(c)[: offs[-1]].astype(np.float64)
    assert np.all(np.isnan(host(c)[offs[-1]:]))  # rows past the valid ones are never written
    scale = np.max(np.abs(ref))
    err = np.max(np.abs(got - ref))
    say(f"  max err / max ref = {err / scale:.2e}")
    assert err <= 2e-5 * scale + 1e-30


def _wl(name, T, H, I, E, k, routing="uniform", skip=0.0, limit=None, seed=0):
    return W.Workload(name, T=T, H=H, I=I, E=E, k=k, fmt=BF16, routing=routing, zipf_s=1.1, skip=skip,
                      swiglu_limit=limit, seed=seed)


SMALL = [
    _wl("bf16_tiny", T=64, H=256, I=128, E=8, k=2, seed=50),
    _wl("bf16_ragged_zipf", T=300, H=512, I=384, E=6, k=3, routing="zipf", skip=0.1, seed=51),
    _wl("bf16_clamp", T=517, H=384, I=256, E=12, k=4, routing="zipf", skip=0.05, limit=0.05, seed=52),
    _wl("bf16_few_rows", T=16, H=640, I=384, E=32, k=8, routing="zipf", skip=0.1, seed=53),
    _wl("bf16_e512", T=600, H=256, I=128, E=512, k=6, routing="zipf", skip=0.05, seed=54),
    _wl("bf16_k64", T=20, H=256, I=128, E=128, k=64, routing="zipf", skip=0.1, seed=58),
]


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_bf16_forward_parity(wl):
    say(f"bf16 forward {wl.name}")
    inp = W.inputs(wl, DEV)
    w = moe.prepare_weights(inp["w13"], None, inp["w2"], None, fmt=BF16)
    dbg = {}
    out = moe.experts_forward(inp["x"], inp["ids"], inp["w"], w, swiglu_limit=wl.swiglu_limit, debug=dbg)
    torch.cuda.synchronize()
    n = {k_: host(v) for k_, v in inp.items()}
    o_ss, o_off, _, _ = oracle.route_sort(n["ids"], wl.E)
    assert np.array_equal(host(dbg["sorted_slot"]), o_ss)
    assert np.array_equal(host(dbg["expert_offsets"]), o_off)
    ref = oracle.forward(BF16, n["w13"], None, n["w2"], None, n["x"], n["ids"], n["w"], swiglu_limit=wl.swiglu_limit)
    assert_out_close(host(out), ref, wl.name)


def test_bf16_forward_every_tile_height():
    """Experts whose last m-tile runs at each height the tiled kernel picks
    (64, 128, 256, and 192 on the gate_up GEMM for an expert whose only m-tile
    has 129-192 rows), at both ends of each range."""
    counts = [1, 64, 65, 128, 129, 150, 192, 193, 255, 256, 256 + 129, 256 + 192, 512 + 170, 256 + 64]
    wl = _wl("bf16_tile_heights", T=sum(counts), H=256, I=256, E=len(counts), k=1, seed=59)
    say(f"bf16 forward {wl.name}")
    inp = W.inputs(wl, DEV)
    ids = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts)])
    inp["ids"] = torch.from_numpy(np.random.default_rng(59).permutation(ids).reshape(-1, 1)).to(DEV)
    w = moe.prepare_weights(inp["w13"], None, inp["w2"], None, fmt=BF16)
    dbg = {}
    out = moe.experts_forward(inp["x"], inp["ids"], inp["w"], w, debug=dbg)
    torch.cuda.synchronize()
    n = {k_: host(v) for k_, v in inp.items()}
    assert np.array_equal(host(dbg["expert_offsets"]), np.concatenate([[0], np.cumsum(counts)]))
    ref = oracle.forward(BF16, n["w13"], None, n["w2"], None, n["x"], n["ids"], n["w"])
    assert_out_close(host(out), ref, wl.name)


def test_bf16_forward_invariants():
    wl = SMALL[1]
    inp = W.inputs(wl, DEV)
    w = moe.prepare_weights(inp["w13"], None, inp["w2"], None, fmt=BF16)
    a = moe.experts_forward(inp["x"], inp["ids"], inp["w"], w).clone()
    b = moe.experts_forward(inp["x"], inp["ids"], inp["w"], w).clone()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "not deterministic"
    perm = torch.randperm(wl.T, generator=torch.Generator().manual_seed(5)).to(DEV)
    c = moe.experts_forward(inp["x"][perm].contiguous(), inp["ids"][perm].contiguous(), inp["w"][perm].contiguous(),
                            w)
    assert torch.equal(c.view(torch.int16), a[perm].view(torch.int16)), "token permutation changed results"
    z = moe.experts_forward(inp["x"], torch.full_like(inp["ids"], -1), torch.full_like(inp["w"], float("nan")), w)
    torch.cuda.synchronize()
    assert torch.count_nonzero(z.view(torch.int16)).item() == 0


def test_bf16_prepare_nn_layout_matches_nt():
    """bf16 weights given transposed ([E, H, 2I] and [E, I, H]) prepare to the
    same bytes as the nt layout, so the forward is bit-identical."""
    wl = _wl("bf16_nn", T=96, H=384, I=256, E=3, k=2, seed=59)
    inp = W.inputs(wl, DEV)
    w_nt = moe.prepare_weights(inp["w13"], None, inp["w2"], None, fmt=BF16)
    w_nn = moe.prepare_weights(inp["w13"].transpose(1, 2).contiguous(), None, inp["w2"].transpose(1, 2).contiguous(),
                               None, fmt=BF16, transposed=True)
    torch.cuda.synchronize()
    assert torch.equal(w_nt._keep[0], w_nn._keep[0])
    a = moe.experts_forward(inp["x"], inp["ids"], inp["w"], w_nt).clone()
    b = moe.experts_forward(inp["x"], inp["ids"], inp["w"], w_nn)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_bf16_forward_from_logits():
    wl = _wl("bf16_logits", T=96, H=512, I=256, E=16, k=4, seed=55)
    inp = W.inputs(wl, DEV)
    lg = W.router_logits(wl.T, wl.E, seed=wl.seed, device=DEV)
    w = moe.prepare_weights(inp["w13"], None, inp["w2"], None, fmt=BF16)
    out, ids, wts = moe.experts_forward_from_logits(inp["x"], lg, wl.k, w)
    torch.cuda.synchronize()
    o_ids, o_w = oracle.router_topk(host(lg), wl.k)
    assert np.array_equal(host(ids), o_ids)
    n = {k_: host(v) for k_, v in inp.items()}
    ref = oracle.forward(BF16, n["w13"], None, n["w2"], None, n["x"], o_ids, o_w)
    assert_out_close(host(out), ref, wl.name)


def test_bf16_forward_full_size_sampled():
    """The Mixtral-shaped layer in bf16 (4096 tokens, hidden 4096, intermediate
    14336, 8 experts, top-2), whole on the GPU in the launch configuration the
    benchmark times; the oracle recomputes a seeded sample of tokens."""
    wl = W.WORKLOADS["mixtral_8x7b_bf16"]
    say(f"bf16 forward full {wl.name}: generating inputs")
    inp = W.inputs(wl, DEV)
    w = moe.prepare_weights(inp["w13"], None, inp["w2"], None, fmt=BF16)
    out = moe.experts_forward(inp["x"], inp["ids"], inp["w"], w)
    torch.cuda.synchronize()
    tokens = W.sample_tokens(wl.T, 48, wl.seed)
    say(f"bf16 forward full {wl.name}: oracle on {tokens.size} tokens")
    n = {k_: host(v) for k_, v in inp.items()}
    ref = oracle.forward(BF16, n["w13"], None, n["w2"], None, n["x"], n["ids"], n["w"], tokens=tokens)
    assert_out_close(host(out)[tokens], ref[tokens], wl.name)


def test_bf16_forward_edge_cases():
    """Empty batch, a single token, k = E = 1, and a batch large enough for the
    multi-workgroup sort (T * k >= 16384 slots)."""
    wl = SMALL[0]
    inp = W.inputs(wl, DEV)
    w = moe.prepare_weights(inp["w13"], None, inp["w2"], None, fmt=BF16)
    out = moe.experts_forward(inp["x"][:0], inp["ids"][:0], inp["w"][:0], w)
    assert out.shape == (0, wl.H)
    one = moe.experts_forward(inp["x"][-1:].contiguous(), inp["ids"][-1:].contiguous(), inp["w"][-1:].contiguous(), w)
    torch.cuda.synchronize()
    n = {k_: host(v) for k_, v in inp.items()}
    ref = oracle.forward(BF16, n["w13"], None, n["w2"], None, n["x"][-1:], n["ids"][-1:], n["w"][-1:])
    assert_out_close(host(one), ref, "single token")
    for case in (_wl("bf16_k1_e1", T=130, H=256, I=128, E=1, k=1, seed=56),
                 _wl("bf16_multiblock_sort", T=2100, H=256, I=128, E=64, k=8, routing="zipf", skip=0.05, seed=57)):
        say(f"bf16 forward {case.name}")
        inp = W.inputs(case, DEV)
        w = moe.prepare_weights(inp["w13"], None, inp["w2"], None, fmt=BF16)
        out = moe.experts_forward(inp["x"], inp["ids"], inp["w"], w)
        torch.cuda.synchronize()
        n = {k_: host(v) for k_, v in inp.items()}
        ref = oracle.forward(BF16, n["w13"], None, n["w2"], None, n["x"], n["ids"], n["w"])
        assert_out_close(host(out), ref, case.name)


def test_bf16_forward_graph_replay():
    """Captured in a HIP graph, the bf16 forward replays bit-exactly, with eager
    work and synchronizations between the replays."""
    wl = SMALL[1]
    inp = W.inputs(wl, DEV)
    w = moe.prepare_weights(inp["w13"], None, inp["w2"], None, fmt=BF16)
    ref = moe.experts_forward(inp["x"], inp["ids"], inp["w"], w).clone()
    torch.cuda.synchronize()
    out = torch.empty_like(ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moe.experts_forward(inp["x"], inp["ids"], inp["w"], w, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.experts_forward(inp["x"], inp["ids"], inp["w"], w, out=out)
    torch.cuda.synchronize()
    for rep in range(3):
        junk = moe.experts_forward(inp["x"], inp["ids"], inp["w"], w)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out).view(np.uint16), host(ref).view(np.uint16)), f"replay {rep}"
        assert np.array_equal(host(junk).view(np.uint16), host(ref).view(np.uint16))

"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Bit-exact: the route sort (sorted_slot, expert_offsets, slot_pos, invalid
count) and the activation codes and scales.  Tolerance (bf16 outputs):
max|err| <= 1e-2 * max|ref| and relative L2 <= 5e-3.  Sizes: the tiny layer and
mid-size cases that span several tiles with ragged tails run whole through the
oracle; the full-size layers run whole on the GPU and are checked on a seeded
sample of tokens.
"""
import sys

import numpy as np
import pytest
import torch

import block_scaled_fp8_sort_amd as moe
import oracle
import workloads as W
from parity_checks import (assert_forward_parity, bits_to_f64, check_down_half, check_h_codes, flip_explainer,
                           host, rowmajor_codes, rowmajor_scales, say)

pytestmark = pytest.mark.gpu

FP8, MX = W.FMT_FP8_B128, W.FMT_MX
DEV = "cuda:0"


def assert_out_close(got_bits, ref_bits, what=""):
    """The forward's tolerance with no exception path (outputs without debug data)."""
    g, r = bits_to_f64(got_bits), bits_to_f64(ref_bits)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    max_ref = np.max(np.abs(r))
    max_err = np.max(np.abs(g - r))
    rel_l2 = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)
    say(f"  {what}: max|err| / max|ref| = {max_err / max(max_ref, 1e-30):.2e}, rel L2 = {rel_l2:.2e}")
    assert max_err <= 1e-2 * max_ref, f"{what}: max|err| {max_err} > 1e-2 * {max_ref}"
    assert rel_l2 <= 5e-3, f"{what}: rel L2 {rel_l2}"


# ---------------------------------------------------------------- route sort
def _rand_ids(rng, T, k, E, p_skip, p_bad, lo=0):
    ids = rng.integers(lo, lo + E, size=(T, k)).astype(np.int32)
    u = rng.random((T, k))
    ids[u < p_skip] = -1
    bad = u > 1 - p_bad
    ids[bad] = rng.choice(np.array([lo + E, lo + E + 3, -5, lo - 1, 1 << 30], np.int32), size=int(bad.sum()))
    return ids


SORT_CASES = [
    (1, 1, 1, 0.0, 0.0), (7, 2, 3, 0.2, 0.1), (64, 2, 8, 0.0, 0.0), (64, 8, 128, 0.05, 0.0),
    (4096, 2, 8, 0.0, 0.0), (8192, 8, 256, 0.05, 0.01), (16384, 8, 256, 0.05, 0.0), (1000, 3, 512, 0.3, 0.05),
    (333, 64, 5, 0.1, 0.1),
    # around and above the size where the sort switches to several workgroups
    (16383, 1, 7, 0.1, 0.0), (2048, 8, 256, 0.05, 0.01), (20000, 1, 1, 0.3, 0.1), (40000, 8, 512, 0.05, 0.02),
    # past 2048 chunks of 256 slots: longer chunks (320 and 448 slots), a chunk
    # count that is not a multiple of the four waves of a workgroup
    (70000, 8, 256, 0.05, 0.01), (100000, 9, 512, 0.1, 0.01),
]


@pytest.mark.parametrize("T,k,E,p_skip,p_bad", SORT_CASES)
def test_route_sort_bit_exact(T, k, E, p_skip, p_bad):
    say(f"route_sort T={T} k={k} E={E}")
    rng = np.random.default_rng(T + 7 * k + 13 * E)
    ids = _rand_ids(rng, T, k, E, p_skip, p_bad, lo=3)
    ss, off, sp, inv = moe.route_sort(torch.from_numpy(ids).to(DEV), E, expert_begin=3)
    torch.cuda.synchronize()
    o_ss, o_off, o_sp, o_inv = oracle.route_sort(ids, E, expert_begin=3)
    assert np.array_equal(host(off), o_off)
    assert np.array_equal(host(ss), o_ss)
    assert np.array_equal(host(sp), o_sp)
    assert int(host(inv)[0]) == o_inv


def test_route_sort_degenerate():
    for ids in (np.full((50, 4), -1, np.int32), np.full((50, 4), 2, np.int32), np.zeros((0, 4), np.int32),
                np.full((5000, 8), -1, np.int32), np.full((5000, 8), 1, np.int32)):
        ss, off, sp, inv = moe.route_sort(torch.from_numpy(ids).to(DEV), 3)
        torch.cuda.synchronize()
        o = oracle.route_sort(ids, 3)
        assert np.array_equal(host(off), o[1])
        assert np.array_equal(host(ss), o[0])


# -------------------------------------------------------------- quantization
def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16)


@pytest.mark.parametrize("fmt", [FP8, MX])
def test_quant_act_bit_exact_random(fmt):
    say(f"quant_act random fmt={fmt}")
    rng = np.random.default_rng(5 + fmt)
    rows, H = 2048, 1024
    x = rng.standard_normal((rows, H)) * np.exp(rng.uniform(-12, 12, size=(rows, 1)))
    x[::17, :128] = 0.0                                  # zero blocks -> floor scale
    x[5::23, 64] = 3e4                                   # outliers
    x[7::29] *= 1e-6                                     # tiny rows (below the floor)
    xb = _bf16(x)
    codes, scales = moe.quant_act(xb.to(DEV), fmt)
    torch.cuda.synchronize()
    o_codes, o_scales = oracle.quant_rows_bf16(xb.view(torch.int16).numpy().view(np.uint16), fmt)
    g_codes = rowmajor_codes(codes)
    mism = np.argwhere(g_codes != o_codes)
    assert mism.size == 0, f"{len(mism)} code mismatches, first at {mism[:5]}"
    assert np.array_equal(rowmajor_scales(scales).view(np.uint8), o_scales.view(np.uint8))


@pytest.mark.parametrize("fmt", [FP8, MX])
def test_quant_act_all_bf16_values(fmt):
    """Every finite bf16 with |x| <= 448 (both signs), in blocks whose scale is 1,
    then the same values under a random non-power-of-two scale."""
    say(f"quant_act all-bf16 fmt={fmt}")
    B = 128 if fmt == FP8 else 32
    bits = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    vals = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    keep = np.isfinite(vals) & (np.abs(vals) <= 448)
    v = vals[keep]
    per = B - 1
    n_rows = (v.size + per - 1) // per
    v = np.concatenate([v, np.zeros(n_rows * per - v.size, np.float32)]).reshape(n_rows, per)
    rng = np.random.default_rng(9)
    for mult in (1.0, float(np.float32(rng.uniform(1.01, 1.99))) * 2.0 ** -7):
        block = np.concatenate([np.full((n_rows, 1), 448.0, np.float32), v], axis=1) * np.float32(mult)
        # pack the blocks into rows of 128 (one FP8 block or four MX blocks per row)
        flat = block.reshape(-1)
        pad = (-flat.size) % 128
        flat = np.concatenate([flat, np.zeros(pad, np.float32)]).reshape(-1, 128)
        xb = _bf16(flat)
        codes, scales = moe.quant_act(xb.to(DEV), fmt)
        torch.cuda.synchronize()
        o_codes, o_scales = oracle.quant_rows_bf16(xb.view(torch.int16).numpy().view(np.uint16), fmt)
        assert np.array_equal(rowmajor_codes(codes), o_codes)
        assert np.array_equal(rowmajor_scales(scales).view(np.uint8), o_scales.view(np.uint8))


# -------------------------------------------------------------- grouped GEMM
@pytest.mark.parametrize("fmt", [FP8, MX])
@pytest.mark.parametrize("which", [0, 1])
@pytest.mark.parametrize("E,H,I,T,k", [
    (3, 256, 128, 40, 2), (5, 640, 384, 700, 3), (2, 384, 1024, 300, 1),
    # at most 12 rows per expert on average: the FP8 path streams weights
    # through registers one K block ahead; K / 128 = 5, 3, 16, 4, 2
    (12, 640, 384, 10, 3), (16, 2048, 512, 24, 4), (20, 256, 256, 30, 2),
])
def test_grouped_gemm_store_f32(fmt, which, E, H, I, T, k):
    """Either weight of a prepared layer times gathered rows, against the oracle's
    grouped GEMM (which = 0: N = 2I over K = H; which = 1: N = H over K = I)."""
    say(f"gemm store f32 fmt={fmt} which={which} E={E} H={H} I={I} T={T} k={k}")
    seed = H + I + T + which
    rng = np.random.default_rng(seed)
    gen = W.fp8_weights if fmt == FP8 else W.fp4_weights
    w13, s13 = gen(E, 2 * I, H, seed, "w13", DEV)
    w2, s2 = gen(E, H, I, seed, "w2", DEV)
    w = moe.prepare_weights(w13, s13, w2, s2, fmt=fmt)
    N, K = (2 * I, H) if which == 0 else (H, I)
    x = W.hidden_states(T, K, seed, DEV)
    ids = torch.from_numpy(_rand_ids(rng, T, k, E, 0.1, 0.0)).to(DEV)
    a, asc = moe.quant_act(x, fmt)
    ss, off, _, _ = moe.route_sort(ids, E)
    S = T * k
    c = torch.full((S, N), float("nan"), dtype=torch.float32, device=DEV)
    moe.grouped_gemm(w, which, a, asc, T, off, moe.EPI_STORE_F32, S, a_row_index=ss, a_row_divisor=k, c_f32=c)
    torch.cuda.synchronize()
    offs = host(off)
    b, bs = (host(w13), host(s13)) if which == 0 else (host(w2), host(s2))
    ref = oracle.grouped_gemm(fmt, rowmajor_codes(a), rowmajor_scales(asc), offs, b, bs, N, K, row_index=host(ss),
                              row_div=k)
    got = host(c)[: offs[-1]].astype(np.float64)
    assert np.all(np.isnan(host(c)[offs[-1]:]))  # rows past the valid ones are never written
    err = np.abs(got - ref)
    scale = np.max(np.abs(ref))
    say(f"  max err / max ref = {np.max(err) / scale:.2e}")
    # fp8 products are exact, but the MFMA's internal sum of a 128-long block is
    # not a sequential fp32 sum: measured ~2e-5 of max|ref| against fp64
    assert np.max(err) <= 1e-4 * scale + 1e-30


@pytest.mark.parametrize("fmt", [FP8, MX])
def test_grouped_gemm_sorted_scales_bit_identical(fmt):
    """The scales laid out by sorted row (a_scales_sorted, as the forward builds
    them for large batches) give the same bits as the scales gathered by
    a_row_index, on the 256-row tiled path, and match the oracle."""
    E, H, I, T, k = 6, 384, 256, 900, 4
    seed = 77 + fmt
    rng = np.random.default_rng(seed)
    gen = W.fp8_weights if fmt == FP8 else W.fp4_weights
    w13, s13 = gen(E, 2 * I, H, seed, "w13", DEV)
    w2, s2 = gen(E, H, I, seed, "w2", DEV)
    w = moe.prepare_weights(w13, s13, w2, s2, fmt=fmt)
    x = W.hidden_states(T, H, seed, DEV)
    ids = torch.from_numpy(_rand_ids(rng, T, k, E, 0.1, 0.0)).to(DEV)
    a, asc = moe.quant_act(x, fmt)
    ss, off, _, _ = moe.route_sort(ids, E)
    S = T * k
    sorted_sc = asc[:, ss.long() // k].contiguous()
    outs = []
    for srt in (None, sorted_sc):
        c = torch.full((S, 2 * I), float("nan"), dtype=torch.float32, device=DEV)
        moe.grouped_gemm(w, 0, a, asc, T, off, moe.EPI_STORE_F32, S, a_row_index=ss, a_row_divisor=k, c_f32=c,
                         a_scales_sorted=srt)
        outs.append(c)
    torch.cuda.synchronize()
    offs = host(off)
    g0, g1 = host(outs[0])[: offs[-1]], host(outs[1])[: offs[-1]]
    assert np.array_equal(g0.view(np.uint32), g1.view(np.uint32))
    ref = oracle.grouped_gemm(fmt, rowmajor_codes(a), rowmajor_scales(asc), offs, host(w13), host(s13), 2 * I, H,
                              row_index=host(ss), row_div=k)
    assert np.max(np.abs(g1.astype(np.float64) - ref)) <= 1e-4 * np.max(np.abs(ref))


def _gemm_vs_oracle(fmt, which, E, H, I, ids_np, k, seed):
    gen = W.fp8_weights if fmt == FP8 else W.fp4_weights
    w13, s13 = gen(E, 2 * I, H, seed, "w13", DEV)
    w2, s2 = gen(E, H, I, seed, "w2", DEV)
    w = moe.prepare_weights(w13, s13, w2, s2, fmt=fmt)
    N, K = (2 * I, H) if which == 0 else (H, I)
    T = ids_np.shape[0]
    x = W.hidden_states(T, K, seed, DEV)
    a, asc = moe.quant_act(x, fmt)
    ss, off, _, _ = moe.route_sort(torch.from_numpy(ids_np).to(DEV), E)
    S = T * k
    c = torch.full((S, N), float("nan"), dtype=torch.float32, device=DEV)
    moe.grouped_gemm(w, which, a, asc, T, off, moe.EPI_STORE_F32, S, a_row_index=ss, a_row_divisor=k, c_f32=c)
    torch.cuda.synchronize()
    offs = host(off)
    b, bs = (host(w13), host(s13)) if which == 0 else (host(w2), host(s2))
    del w, w13, w2
    ref = oracle.grouped_gemm(fmt, rowmajor_codes(a), rowmajor_scales(asc), offs, b, bs, N, K, row_index=host(ss),
                              row_div=k)
    got = host(c)[: offs[-1]].astype(np.float64)
    assert np.all(np.isnan(host(c)[offs[-1]:]))
    scale = np.max(np.abs(ref))
    err = np.max(np.abs(got - ref))
    say(f"  max err / max ref = {err / scale:.2e}")
    assert err <= 1e-4 * scale + 1e-30


@pytest.mark.parametrize("which", [0, 1])
def test_grouped_gemm_few_rows_one_heavy_expert(which):
    """Few rows per expert on average, but one expert with 40 rows (three
    16-row tiles) and several experts with none."""
    say(f"gemm heavy expert which={which}")
    T, k, E = 40, 2, 16
    ids = np.full((T, k), -1, np.int32)
    ids[:20, :] = 3                 # expert 3: 40 slots
    ids[20:, 0] = np.arange(20) % 5 + 9
    _gemm_vs_oracle(FP8, which, E, 512, 384, ids, k, seed=77)


@pytest.mark.parametrize("H", [512, 640])
def test_grouped_gemm_half_width_tail_tiles(H):
    """The unpaired GEMM runs an expert's short remainder tile (at most 128 rows
    past its full 256-row tiles) as two 128-row halves of each n-tile: rows
    counts with remainders of 1, 40, 64, 65, 100 and 128 rows (both half
    heights), an expert with no remainder and one with fewer than 256 rows;
    H = 640 leaves the second half of the last n-tile past N."""
    say(f"gemm half-width tail tiles H={H}")
    counts = [256 + 40, 512 + 100, 256 + 128, 300, 256 + 1, 512, 200, 256 + 64, 256 + 65]
    ids = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts)])
    ids = np.random.default_rng(90).permutation(ids).reshape(-1, 1)
    _gemm_vs_oracle(FP8, 1, len(counts), H, 256, ids, 1, seed=90)


# rows per expert whose last m-tile takes each height the tiled GEMMs choose
# from at both ends of its range, alone and past one or two full 256-row
# m-tiles: 64, 128, 256, and on the gate_up GEMM 192 for an expert whose only
# m-tile has 129-192 rows
TILE_HEIGHT_COUNTS = [1, 64, 65, 128, 129, 150, 192, 193, 255, 256, 256 + 129, 256 + 192, 512 + 170, 256 + 64]


def _ids_with_counts(counts, seed):
    ids = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts)])
    return np.random.default_rng(seed).permutation(ids).reshape(-1, 1)


@pytest.mark.parametrize("fmt", [FP8, MX])
@pytest.mark.parametrize("which", [0, 1])
def test_grouped_gemm_every_tile_height(fmt, which):
    """Both GEMMs (paired and unpaired) on experts whose last m-tile runs at
    each height, 64 to 256 rows (the paired one's 192-row tiles included)."""
    say(f"gemm every tile height fmt={fmt} which={which}")
    counts = TILE_HEIGHT_COUNTS
    _gemm_vs_oracle(fmt, which, len(counts), 384, 256, _ids_with_counts(counts, 95 + which), 1, seed=95)


@pytest.mark.parametrize("fmt", [FP8, MX])
def test_grouped_gemm_tile_order_and_counters(fmt):
    """The fixed round-robin tile order (no counters) and the dynamic dispensers
    give the same result bit for bit (each output tile is computed by one
    workgroup in the same way), and a launch leaves its counters zero, so they
    can be reused."""
    say(f"gemm tile order fmt={fmt}")
    E, H, I, T, k = 6, 512, 384, 900, 3
    rng = np.random.default_rng(41)
    gen = W.fp8_weights if fmt == FP8 else W.fp4_weights
    w13, s13 = gen(E, 2 * I, H, 41, "w13", DEV)
    w2, s2 = gen(E, H, I, 41, "w2", DEV)
    w = moe.prepare_weights(w13, s13, w2, s2, fmt=fmt)
    x = W.hidden_states(T, H, 41, DEV)
    ids = torch.from_numpy(_rand_ids(rng, T, k, E, 0.1, 0.0)).to(DEV)
    a, asc = moe.quant_act(x, fmt)
    ss, off, _, _ = moe.route_sort(ids, E)
    S = T * k
    counters = torch.zeros(moe.TILE_COUNTERS_INTS, dtype=torch.int32, device=DEV)
    outs = []
    for tc in (None, counters, counters):  # static, dynamic, dynamic reusing the counters
        c = torch.full((S, 2 * I), float("nan"), dtype=torch.float32, device=DEV)
        moe.grouped_gemm(w, 0, a, asc, T, off, moe.EPI_STORE_F32, S, a_row_index=ss, a_row_divisor=k, c_f32=c,
                         tile_counters=tc)
        torch.cuda.synchronize()
        outs.append(host(c))
        assert int(host(counters).astype(np.int64).sum()) == 0
    n = host(off)[-1]
    for o in outs[1:]:
        assert np.array_equal(o[:n].view(np.uint32), outs[0][:n].view(np.uint32))


def test_grouped_gemm_few_rows_many_tiles():
    """More tiles than a workgroup fetches row data for at once (16 per
    workgroup on 256 CUs needs over 4096 tiles): 80 experts x 64 paired
    n-tiles."""
    say("gemm many tiles")
    rng = np.random.default_rng(5)
    T, k, E = 64, 4, 80
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    _gemm_vs_oracle(FP8, 0, E, 256, 8192, ids, k, seed=78)


# ------------------------------------------------------------- the forward
def _prepare(inp, fmt):
    return moe.prepare_weights(inp["w13"], inp["s13"], inp["w2"], inp["s2"], fmt=fmt)


def _forward_case(wl, inp, tokens=None, debug=False, limit="workload"):
    lim = wl.swiglu_limit if limit == "workload" else limit
    w = _prepare(inp, wl.fmt)
    dbg = {} if debug else None
    inv = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = moe.experts_forward(inp["x"], inp["ids"], inp["w"], w, swiglu_limit=lim, invalid_count=inv, debug=dbg)
    torch.cuda.synchronize()
    n = {k_: host(v) for k_, v in inp.items()}
    ref = oracle.forward(wl.fmt, n["w13"], n["s13"], n["w2"], n["s2"], n["x"], n["ids"], n["w"], swiglu_limit=lim,
                         tokens=tokens)
    return host(out), ref, dbg, n, int(host(inv)[0])


def _small_workload(name, fmt, T, H, I, E, k, routing="uniform", skip=0.0, limit=None, seed=0):
    return W.Workload(name, T=T, H=H, I=I, E=E, k=k, fmt=fmt, routing=routing, zipf_s=1.1, skip=skip,
                      swiglu_limit=limit, seed=seed)


SMALL = [
    W.WORKLOADS["tiny"],
    _small_workload("ragged_fp8", FP8, T=300, H=512, I=384, E=6, k=3, routing="zipf", skip=0.1, seed=11),
    _small_workload("ragged_fp8_clamp", FP8, T=517, H=384, I=256, E=12, k=4, routing="zipf", skip=0.05,
                    limit=0.05, seed=12),
    _small_workload("k1_one_expert", FP8, T=129, H=256, I=128, E=1, k=1, seed=13),
    # decode-like: at most 12 rows per expert on average
    _small_workload("decode_fp8", FP8, T=24, H=512, I=256, E=16, k=4, seed=17),
    _small_workload("decode_fp8_ragged_clamp", FP8, T=16, H=640, I=384, E=32, k=8, routing="zipf", skip=0.1,
                    limit=0.05, seed=18),
    _small_workload("mx_tiny", MX, T=64, H=256, I=128, E=8, k=2, seed=14),
    _small_workload("mx_ragged_clamp", MX, T=300, H=384, I=256, E=7, k=4, routing="zipf", skip=0.1, limit=7.0,
                    seed=15),
    _small_workload("mx_tight_clamp", MX, T=200, H=512, I=384, E=5, k=3, routing="zipf", skip=0.05, limit=0.05,
                    seed=16),
    # the largest expert count the tile tables hold (512), on both FP8 paths and MX
    _small_workload("e512_fp8_few_rows", FP8, T=160, H=256, I=128, E=512, k=8, routing="zipf", skip=0.05, seed=19),
    _small_workload("e512_fp8_tiled", FP8, T=1500, H=256, I=256, E=512, k=6, routing="zipf", skip=0.05, seed=20),
    _small_workload("e512_mx", MX, T=1200, H=256, I=128, E=512, k=4, routing="zipf", skip=0.05, limit=7.0, seed=22),
    # more than 8 slots per token (the combine's wide path), up to the largest k
    _small_workload("k16_fp8", FP8, T=96, H=256, I=128, E=32, k=16, routing="zipf", skip=0.1, seed=24),
    _small_workload("k64_fp8", FP8, T=20, H=256, I=128, E=128, k=64, routing="zipf", skip=0.1, seed=25),
    # both sides of the switch between the FP8 GEMMs: 12 slots per expert on
    # average streams weights through registers (skewed, so some experts span
    # several 16-row tiles), 13 takes the LDS-tiled kernel
    _small_workload("switch_12_rows_fp8", FP8, T=96, H=512, I=256, E=32, k=4, routing="zipf", skip=0.05, seed=41),
    _small_workload("switch_13_rows_fp8", FP8, T=104, H=512, I=256, E=32, k=4, routing="zipf", skip=0.05, seed=42),
    _small_workload("k24_mx", MX, T=40, H=256, I=128, E=48, k=24, routing="zipf", skip=0.1, limit=7.0, seed=26),
    # the down GEMM's half-width tail tiles: experts of 303-339 rows (remainders
    # of 47 to 83 past one 256-row tile: both half heights), H = 640 (a partial
    # last n-tile)
    _small_workload("tail_halves_fp8", FP8, T=640, H=640, I=256, E=4, k=2, seed=29),
    # 16384 slots and more: the multi-workgroup sort; the activation scales are
    # then copied by sorted row (sorted_slot / k) for the gate_up GEMM
    _small_workload("multiblock_fp8", FP8, T=2100, H=384, I=256, E=64, k=8, routing="zipf", skip=0.05, seed=27),
    _small_workload("multiblock_fp8_i128", FP8, T=2100, H=384, I=128, E=64, k=8, routing="zipf", skip=0.05,
                    seed=27),
    _small_workload("multiblock_mx", MX, T=4100, H=256, I=128, E=24, k=4, routing="zipf", skip=0.05, limit=7.0,
                    seed=28),
]


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_forward_parity_small(wl):
    say(f"forward {wl.name}")
    inp = W.inputs(wl, DEV)
    got, ref, dbg, n, inv = _forward_case(wl, inp, debug=True)
    o_ss, o_off, _, o_inv = oracle.route_sort(n["ids"], wl.E)
    assert np.array_equal(host(dbg["sorted_slot"]), o_ss)
    assert np.array_equal(host(dbg["expert_offsets"]), o_off)
    assert inv == o_inv
    o_codes, o_scales = oracle.quant_rows_bf16(n["x"], wl.fmt)
    assert np.array_equal(rowmajor_codes(dbg["act_codes"]), o_codes)
    assert np.array_equal(rowmajor_scales(dbg["act_scales"]).view(np.uint8), o_scales.view(np.uint8))
    assert_forward_parity(wl.name, got, ref,
                          flip_explainer(wl.fmt, wl.T, wl.k, wl.H, wl.I, n, got, dbg, swiglu_limit=wl.swiglu_limit))


@pytest.mark.parametrize("fmt", [FP8, MX])
def test_forward_every_tile_height(fmt):
    """The forward (SwiGLU and h quantization, the weighted scatter, the
    combine) over experts whose last m-tile runs at each height, 64 to 256
    rows."""
    counts = TILE_HEIGHT_COUNTS
    wl = _small_workload(f"tile_heights_{fmt}", fmt, T=sum(counts), H=256, I=256, E=len(counts), k=1,
                         limit=7.0 if fmt == MX else None, seed=96)
    say(f"forward every tile height {wl.name}")
    inp = W.inputs(wl, DEV)
    inp["ids"] = torch.from_numpy(_ids_with_counts(counts, 96)).to(DEV)
    got, ref, dbg, n, inv = _forward_case(wl, inp, debug=True)
    assert np.array_equal(host(dbg["expert_offsets"]), np.concatenate([[0], np.cumsum(counts)]))
    assert inv == 0
    assert_forward_parity(wl.name, got, ref,
                          flip_explainer(wl.fmt, wl.T, wl.k, wl.H, wl.I, n, got, dbg, swiglu_limit=wl.swiglu_limit))


H_CASES = ["tiny", "ragged_fp8_clamp", "decode_fp8_ragged_clamp", "multiblock_fp8_i128", "mx_ragged_clamp",
           "e512_fp8_tiled"]


@pytest.mark.parametrize("name", H_CASES)
def test_forward_down_half_from_the_gpus_own_h(name):
    """The down projection, routing weight and combine, checked on their own
    (parity_checks.check_down_half): the oracle's grouped GEMM on the GPU's own
    quantized h, the weighted per-token sum in fp64, and the GPU's output within
    the rounding the GPU path does after h.  A wrong h scale, a misplaced h row
    or a wrong weight would be far outside that bound.  The GPU's h codes
    against the oracle's: neighbouring e4m3 values at most (they follow fp32
    sums in another order)."""
    wl = W.WORKLOADS.get(name) or next(w for w in SMALL if w.name == name)
    say(f"down half from GPU h: {name}")
    inp = W.inputs(wl, DEV)
    w = _prepare(inp, wl.fmt)
    dbg = {}
    out = moe.experts_forward(inp["x"], inp["ids"], inp["w"], w, swiglu_limit=wl.swiglu_limit, debug=dbg)
    torch.cuda.synchronize()
    n = {k_: host(v) for k_, v in inp.items()}
    hq, hs, slots = check_down_half(wl.fmt, wl.T, wl.k, wl.H, wl.I, n, host(out), dbg)
    _, odbg = oracle.forward(wl.fmt, n["w13"], n["s13"], n["w2"], n["s2"], n["x"], n["ids"], n["w"],
                             swiglu_limit=wl.swiglu_limit, debug=True)
    check_h_codes(wl.fmt, hq, hs, slots, odbg["h_codes"], odbg["h_scales"], wl.I, odbg["gu"], wl.swiglu_limit)

DUP_CASES = [
    _small_workload("dup_garbage_fp8", FP8, T=200, H=384, I=256, E=10, k=4, seed=40),
    _small_workload("dup_garbage_decode_fp8", FP8, T=12, H=512, I=256, E=16, k=4, seed=41),
    _small_workload("dup_garbage_mx", MX, T=150, H=256, I=128, E=6, k=3, limit=7.0, seed=42),
    _small_workload("dup_garbage_multiblock", FP8, T=2100, H=256, I=256, E=24, k=8, seed=43),
]


@pytest.mark.parametrize("wl", DUP_CASES, ids=[w.name for w in DUP_CASES])
@pytest.mark.parametrize("begin", [0, 7])
def test_forward_duplicate_and_out_of_range_ids(wl, begin):
    """The same expert twice in one token counts twice (two independent slots),
    and ids outside [begin, begin + E) other than -1 (-5, 1 << 30, begin + E,
    begin + E + 3, and begin - 1 when begin > 0) are skipped and counted."""
    say(f"forward duplicate / garbage ids {wl.name} begin={begin}")
    inp = W.inputs(wl, DEV)
    ids = host(inp["ids"]).astype(np.int64)
    ids = np.where(ids >= 0, ids + begin, ids)
    ids[::3, 1] = ids[::3, 0]
    ids[1::7, 2 % wl.k] = -5
    ids[2::11, 0] = 1 << 30
    ids[3::13, wl.k - 1] = begin + wl.E
    ids[4::17, 1] = begin + wl.E + 3
    if begin > 0:
        ids[5::19, 0] = begin - 1
    ids = ids.astype(np.int32)
    assert np.any((ids[:, 0] == ids[:, 1]) & (ids[:, 0] >= begin))
    inp["ids"] = torch.from_numpy(ids).to(DEV)
    w = _prepare(inp, wl.fmt)
    inv = torch.zeros(1, dtype=torch.int32, device=DEV)
    dbg = {}
    out = moe.experts_forward(inp["x"], inp["ids"], inp["w"], w, swiglu_limit=wl.swiglu_limit, expert_begin=begin,
                              invalid_count=inv, debug=dbg)
    torch.cuda.synchronize()
    n = {k_: host(v) for k_, v in inp.items()}
    ref = oracle.forward(wl.fmt, n["w13"], n["s13"], n["w2"], n["s2"], n["x"], ids, n["w"],
                         swiglu_limit=wl.swiglu_limit, expert_begin=begin)
    o_ss, o_off, _, o_inv = oracle.route_sort(ids, wl.E, expert_begin=begin)
    assert int(host(inv)[0]) == o_inv > 0
    assert np.array_equal(host(dbg["sorted_slot"]), o_ss) and np.array_equal(host(dbg["expert_offsets"]), o_off)
    got = host(out)
    assert_forward_parity(f"{wl.name} begin={begin}", got, ref,
                          flip_explainer(wl.fmt, wl.T, wl.k, wl.H, wl.I, n, got, dbg, swiglu_limit=wl.swiglu_limit,
                                         expert_begin=begin))


def test_forward_invariants_tiny():
    wl = W.WORKLOADS["tiny"]
    inp = W.inputs(wl, DEV)
    w = _prepare(inp, wl.fmt)
    a = moe.experts_forward(inp["x"], inp["ids"], inp["w"], w).clone()
    b = moe.experts_forward(inp["x"], inp["ids"], inp["w"], w).clone()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "not deterministic"
    perm = torch.randperm(wl.T, generator=torch.Generator().manual_seed(3)).to(DEV)
    c = moe.experts_forward(inp["x"][perm].contiguous(), inp["ids"][perm].contiguous(), inp["w"][perm].contiguous(),
                            w)
    assert torch.equal(c.view(torch.int16), a[perm].view(torch.int16)), "token permutation changed results"
    # a NaN-poisoned workspace changes nothing
    ws = torch.full((moe.forward_workspace_bytes(wl.T, wl.k, w),), 0xFF, dtype=torch.uint8, device=DEV)
    d = moe.experts_forward(inp["x"], inp["ids"], inp["w"], w, workspace=ws)
    assert torch.equal(d.view(torch.int16), a.view(torch.int16))
    # skipped slots with NaN weights contribute exactly nothing
    ids = inp["ids"].clone()
    wts = inp["w"].clone()
    ids[:, 1] = -1
    wts[:, 1] = float("nan")
    e = moe.experts_forward(inp["x"], ids, wts, w)
    ids2 = inp["ids"][:, :1].contiguous()
    f = moe.experts_forward(inp["x"], ids2, inp["w"][:, :1].contiguous(), w)
    torch.cuda.synchronize()
    assert torch.equal(e.view(torch.int16), f.view(torch.int16))
    # every slot skipped -> exact zeros
    z = moe.experts_forward(inp["x"], torch.full_like(inp["ids"], -1), torch.full_like(inp["w"], float("nan")), w)
    torch.cuda.synchronize()
    assert torch.count_nonzero(z.view(torch.int16)).item() == 0


@pytest.mark.parametrize("name", ["multiblock_fp8", "multiblock_mx"])
def test_forward_poisoned_workspace_large_batch(name):
    """With the multi-workgroup sort the forward also builds the activation
    scales by sorted row in its workspace; a workspace filled with 0xFF (NaN
    patterns) beforehand changes no output bit, so every scale the gate_up GEMM
    reads was written first."""
    wl = next(w for w in SMALL if w.name == name)
    assert moe.forward_sorts_scales(wl.T, wl.k, wl.fmt)
    inp = W.inputs(wl, DEV)
    w = _prepare(inp, wl.fmt)
    a = moe.experts_forward(inp["x"], inp["ids"], inp["w"], w, swiglu_limit=wl.swiglu_limit).clone()
    ws = torch.full((moe.forward_workspace_bytes(wl.T, wl.k, w),), 0xFF, dtype=torch.uint8, device=DEV)
    b = moe.experts_forward(inp["x"], inp["ids"], inp["w"], w, swiglu_limit=wl.swiglu_limit, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_forward_empty_and_single_token():
    wl = W.WORKLOADS["tiny"]
    inp = W.inputs(wl, DEV)
    w = _prepare(inp, wl.fmt)
    out = moe.experts_forward(inp["x"][:0], inp["ids"][:0], inp["w"][:0], w)
    assert out.shape == (0, wl.H)
    one = moe.experts_forward(inp["x"][-1:].contiguous(), inp["ids"][-1:].contiguous(), inp["w"][-1:].contiguous(), w)
    torch.cuda.synchronize()
    n = {k_: host(v) for k_, v in inp.items()}
    ref = oracle.forward(wl.fmt, n["w13"], n["s13"], n["w2"], n["s2"], n["x"][-1:], n["ids"][-1:], n["w"][-1:])
    assert_out_close(host(one), ref, "single token")


@pytest.mark.parametrize("wl", [SMALL[1], SMALL[5], SMALL[7]], ids=[SMALL[1].name, SMALL[5].name, SMALL[7].name])
def test_forward_graph_replay(wl):
    """The forward allocates nothing and records no memset, so it can be captured
    in a HIP graph: every replay, with the program's own eager work and
    synchronizations in between, reproduces the eager result bit for bit."""
    say(f"graph replay {wl.name}")
    inp = W.inputs(wl, DEV)
    w = _prepare(inp, wl.fmt)
    lim = wl.swiglu_limit
    ref = moe.experts_forward(inp["x"], inp["ids"], inp["w"], w, swiglu_limit=lim)  # also caches the workspace
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moe.experts_forward(inp["x"], inp["ids"], inp["w"], w, swiglu_limit=lim)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = moe.experts_forward(inp["x"], inp["ids"], inp["w"], w, swiglu_limit=lim)
    torch.cuda.synchronize()
    ref_bits = host(ref).view(np.uint16)
    for rep in range(4):
        junk = moe.experts_forward(inp["x"], inp["ids"], inp["w"], w, swiglu_limit=lim)  # eager work between replays
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out).view(np.uint16), ref_bits), f"replay {rep}"
        assert np.array_equal(host(junk).view(np.uint16), ref_bits)


def test_prepare_weights_nn_layout_matches_nt():
    wl = _small_workload("nn", FP8, T=96, H=384, I=256, E=3, k=2, seed=21)
    inp = W.inputs(wl, DEV)
    w_nt = _prepare(inp, FP8)
    gate_up_nn = inp["w13"].transpose(1, 2).contiguous()
    s13_nn = inp["s13"].transpose(1, 2).contiguous()
    down_nn = inp["w2"].transpose(1, 2).contiguous()
    s2_nn = inp["s2"].transpose(1, 2).contiguous()
    w_nn = moe.prepare_weights(gate_up_nn, s13_nn, down_nn, s2_nn, fmt=FP8, transposed=True)
    a = moe.experts_forward(inp["x"], inp["ids"], inp["w"], w_nt).clone()
    b = moe.experts_forward(inp["x"], inp["ids"], inp["w"], w_nn)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


FULL = ["qwen3_moe_decode", "mixtral_8x7b", "deepseek_v3", "megamoe_fp8xfp4"]


@pytest.mark.parametrize("name", FULL)
def test_forward_parity_full_size_sampled(name):
    """The full layer on the GPU (the launch configuration the benchmark times);
    the oracle recomputes a seeded sample of tokens."""
    wl = W.WORKLOADS[name]
    say(f"forward full {name}: generating inputs")
    inp = W.inputs(wl, DEV)
    tokens = W.sample_tokens(wl.T, 48, wl.seed)
    say(f"forward full {name}: running GPU + oracle on {tokens.size} tokens")
    got, ref, _, n, _ = _forward_case(wl, inp, tokens=tokens)
    assert_out_close(got[tokens], ref[tokens], name)

"""GPU: a seeded sweep of random small and mid-size layers against the CPU oracle.

Each case draws its shape (T, H, I, E, k), format, routing, skipped slots,
clamp and expert_begin from a fixed seed, so the sweep reaches combinations
the hand-picked cases do not (both FP8 GEMM paths and their switch-over, the
half-width tail tiles, the tile dispensers' stealing on small grids, MX and
bf16 experts), and a set of extreme shapes (up to 512 experts, top-64, half
the slots skipped).  Checked: the route sort bit-exact; the activation codes
and scales bit-exact (quantized formats); the forward within the parity bar
(max|err| <= 1e-2 max|ref|, relative L2 <= 5e-3), a breach accepted only with
the h-flip explanation of parity_checks.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp8_sort_amd as moe
import oracle
import workloads as W
from parity_checks import (assert_forward_parity, bits_to_f64, flip_explainer, host, rowmajor_codes,
                           rowmajor_scales, say)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
FMTS = [W.FMT_FP8_B128, W.FMT_MX, W.FMT_BF16]
FMT_NAME = {W.FMT_FP8_B128: "fp8", W.FMT_MX: "mx", W.FMT_BF16: "bf16"}


def _cases(n=36, seed=2024, large=False):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        fmt = FMTS[i % 3]
        if large:  # hundreds of rows per expert: full m-tiles, remainders, several rounds
            E = int(rng.choice([2, 3, 5, 8, 16]))
            k = int(rng.integers(1, min(4, E) + 1))
            T = int(rng.integers(400, 1500))
        else:  # few rows per expert (the register-streaming FP8 GEMM) to a few hundred
            E = int(rng.choice([1, 2, 3, 5, 8, 13, 24, 40, 64, 128]))
            k = int(rng.integers(1, min(8, E) + 1))
            T = int(rng.choice([1, 3, int(rng.integers(4, 64)), int(rng.integers(64, 400))]))
        H = int(rng.choice([256, 384, 512, 640, 768]))
        I = int(rng.choice([128, 256, 384]))
        routing = "zipf" if rng.random() < 0.5 else "uniform"
        skip = float(rng.choice([0.0, 0.1]))
        limit = None if rng.random() < 0.5 else (7.0 if fmt == W.FMT_MX else float(rng.choice([0.05, 7.0])))
        begin = int(rng.choice([0, 0, 3]))
        tag = "L" if large else "r"
        out.append((f"{tag}{i:02d}_{FMT_NAME[fmt]}_T{T}_H{H}_I{I}_E{E}_k{k}_b{begin}",
                    W.Workload(f"sweep{tag}{i}", T=T, H=H, I=I, E=E, k=k, fmt=fmt, routing=routing, zipf_s=1.1,
                               skip=skip, swiglu_limit=limit, seed=(300 if large else 100) + i), begin))
    return out


def _wide_cases(n=40, seed=777):
    """Extreme shapes: up to 512 experts, top-64, hidden up to 2048 and
    intermediate up to 1024 (one to sixteen and one to eight 128-wide blocks),
    half the slots skipped, ids offset by 100; the oracle's work capped."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        i = len(out)
        fmt = FMTS[i % 3]
        E = int(rng.choice([1, 2, 4, 7, 16, 33, 64, 128, 256, 512]))
        k = int(rng.integers(1, min(64, E) + 1)) if rng.random() < 0.3 else int(rng.integers(1, min(8, E) + 1))
        T = int(rng.choice([1, 2, int(rng.integers(3, 32)), int(rng.integers(32, 512)), int(rng.integers(512, 4000))]))
        H = 128 * int(rng.integers(1, 17))
        I = 128 * int(rng.integers(1, 9))
        if T * k * H * I > 4e9:
            continue
        routing = "zipf" if rng.random() < 0.5 else "uniform"
        skip = float(rng.choice([0.0, 0.1, 0.5]))
        limit = None if rng.random() < 0.5 else (7.0 if fmt == W.FMT_MX else float(rng.choice([0.05, 1.0, 7.0])))
        begin = int(rng.choice([0, 0, 3, 100]))
        out.append((f"w{i:02d}_{FMT_NAME[fmt]}_T{T}_H{H}_I{I}_E{E}_k{k}_b{begin}_s{skip}",
                    W.Workload(f"wide{i}", T=T, H=H, I=I, E=E, k=k, fmt=fmt, routing=routing, zipf_s=1.1,
                               skip=skip, swiglu_limit=limit, seed=5000 + i), begin))
    return out


CASES = _cases() + _cases(n=15, seed=2025, large=True) + _wide_cases()

# Two 3-token FP8 layers of a wider sweep (seed 9090) whose outputs pass the
# bars only through the h-flip explanation: one of 1152 h codes (r54) and five
# of 2304 (r96) round to the neighbouring e4m3 value, which moves the few
# outputs by 6.6e-3 and 6.1e-3 in relative L2.
FLIP_CASES = [c for c in _cases(n=150, seed=9090)
              if c[0] in ("r54_fp8_T3_H640_I384_E40_k1_b0", "r96_fp8_T3_H640_I384_E2_k2_b3")]
assert len(FLIP_CASES) == 2
CASES = CASES + FLIP_CASES


@pytest.mark.parametrize("name,wl,begin", CASES, ids=[c[0] for c in CASES])
def test_random_layer_parity(name, wl, begin):
    say(f"sweep {name}")
    inp = W.inputs(wl, DEV)
    ids = host(inp["ids"]).astype(np.int64)
    ids = np.where(ids >= 0, ids + begin, ids)
    if wl.T * wl.k >= 8:  # a few ids outside [begin, begin + E): skipped and counted
        rng = np.random.default_rng(wl.seed)
        flat = ids.reshape(-1)
        pick = rng.choice(flat.size, size=max(1, flat.size // 50), replace=False)
        flat[pick] = rng.choice(np.array([begin + wl.E, -7, 1 << 30] + ([begin - 1] if begin else []), np.int64),
                                size=pick.size)
    ids = ids.astype(np.int32)
    inp["ids"] = torch.from_numpy(ids).to(DEV)
    if wl.fmt == W.FMT_BF16:
        w = moe.prepare_weights(inp["w13"], None, inp["w2"], None, fmt=wl.fmt)
    else:
        w = moe.prepare_weights(inp["w13"], inp["s13"], inp["w2"], inp["s2"], fmt=wl.fmt)
    inv = torch.zeros(1, dtype=torch.int32, device=DEV)
    dbg = {}
    out = moe.experts_forward(inp["x"], inp["ids"], inp["w"], w, swiglu_limit=wl.swiglu_limit, expert_begin=begin,
                              invalid_count=inv, debug=dbg)
    torch.cuda.synchronize()
    n = {k_: host(v) for k_, v in inp.items()}
    o_ss, o_off, _, o_inv = oracle.route_sort(ids, wl.E, expert_begin=begin)
    assert np.array_equal(host(dbg["sorted_slot"]), o_ss)
    assert np.array_equal(host(dbg["expert_offsets"]), o_off)
    assert int(host(inv)[0]) == o_inv
    got = host(out)
    if wl.fmt == W.FMT_BF16:
        ref = oracle.forward(wl.fmt, n["w13"], None, n["w2"], None, n["x"], ids, n["w"],
                             swiglu_limit=wl.swiglu_limit, expert_begin=begin)
        g, r = bits_to_f64(got), bits_to_f64(ref)
        assert np.all(np.isfinite(g))
        max_ref = max(np.max(np.abs(r)), 1e-30)
        rel_l2 = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)
        say(f"  {name}: max|err| / max|ref| = {np.max(np.abs(g - r)) / max_ref:.2e}, rel L2 = {rel_l2:.2e}")
        assert np.max(np.abs(g - r)) <= 1e-2 * max_ref and rel_l2 <= 5e-3
        return
    o_codes, o_scales = oracle.quant_rows_bf16(n["x"], wl.fmt)
    assert np.array_equal(rowmajor_codes(dbg["act_codes"]), o_codes)
    assert np.array_equal(rowmajor_scales(dbg["act_scales"]).view(np.uint8), o_scales.view(np.uint8))
    ref = oracle.forward(wl.fmt, n["w13"], n["s13"], n["w2"], n["s2"], n["x"], ids, n["w"],
                         swiglu_limit=wl.swiglu_limit, expert_begin=begin)
    if not np.any(bits_to_f64(ref)):  # every slot skipped: exact zeros
        assert not np.any(got.view(np.uint16) & 0x7FFF)
        return
    n["ids"] = ids
    assert_forward_parity(name, got, ref,
                          flip_explainer(wl.fmt, wl.T, wl.k, wl.H, wl.I, n, got, dbg, swiglu_limit=wl.swiglu_limit,
                                         expert_begin=begin))

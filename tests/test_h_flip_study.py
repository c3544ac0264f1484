"""How far legitimate h-code rounding flips move the forward's output (CPU).

The GPU computes the gate/up products from fp32 accumulators; the oracle sums
in fp64.  The standalone grouped GEMM agrees with fp64 to about 2e-5 of a
row's max|C|, and h = silu(g) u is then quantized to e4m3, an integer decided by
floating point: a code may round to its neighbour, which near the top of e4m3's
range is 1/14 of the block maximum away.  This study perturbs the oracle's own
gate/up values by noise of that size, re-quantizes h with the oracle's rule and
redoes the down projection and the combine in fp64: the flips alone move the
output by about as much as the forward's max-norm bar (1e-2 of max|ref|) on a
64-expert, top-8 layer with one 128-wide h block per row, while the relative L2
stays well under its 5e-3 bar.  The GPU parity tests therefore accept a
max-norm breach only when the flips are shown to be all there is
(tests/parity_checks.py)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W


def test_fp32_level_gate_up_noise_alone_reaches_the_max_norm_bar():
    wl = W.Workload("flip_study", T=2100, H=384, I=128, E=64, k=8, fmt=W.FMT_FP8_B128, routing="zipf",
                    zipf_s=1.1, skip=0.05, seed=27)
    inp = W.inputs(wl, "cpu")
    n = {k: W.to_numpy(v) for k, v in inp.items()}
    ref, d = oracle.forward(wl.fmt, n["w13"], n["s13"], n["w2"], n["s2"], n["x"], n["ids"], n["w"], debug=True)
    ss, off, _, _ = oracle.route_sort(n["ids"], wl.E)
    nv = int(off[-1])
    gu = d["gu"][ss[:nv]].astype(np.float64)
    I = wl.I
    rng = np.random.default_rng(0)
    row_max = np.max(np.abs(gu), axis=1, keepdims=True)
    g = gu[:, :I] + 2e-5 * row_max * rng.standard_normal((nv, I))
    u = gu[:, I:] + 2e-5 * row_max * rng.standard_normal((nv, I))
    h = (g / (1 + np.exp(-g)) * u).astype(np.float32)
    hq, hs = oracle.quant_rows_f32(h, wl.fmt)
    y = oracle.grouped_gemm(wl.fmt, hq, hs, off, n["w2"], n["s2"], wl.H, I)
    acc = np.zeros((wl.T, wl.H))
    wts = n["w"].reshape(-1).astype(np.float64)
    np.add.at(acc, ss[:nv] // wl.k, wts[ss[:nv]][:, None] * y)
    out = torch.from_numpy(acc).float().to(torch.bfloat16).double().numpy()
    r = torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy()
    flips = float(np.mean(hq != d["h_codes"][ss[:nv]]))
    max_rel = float(np.max(np.abs(out - r)) / np.max(np.abs(r)))
    rel_l2 = float(np.linalg.norm(out - r) / np.linalg.norm(r))
    print(f"h codes flipped: {100 * flips:.2f}%, max|err| / max|ref| = {max_rel:.2e}, rel L2 = {rel_l2:.2e}")
    assert 1e-3 < flips < 2e-2
    assert max_rel > 0.8e-2  # as large as the bar itself, from flips alone
    assert rel_l2 < 4e-3


def _study_layer():
    wl = W.Workload("flip_check", T=600, H=384, I=256, E=16, k=4, fmt=W.FMT_FP8_B128, routing="zipf",
                    zipf_s=1.1, skip=0.05, seed=29)
    inp = W.inputs(wl, "cpu")
    n = {k: W.to_numpy(v) for k, v in inp.items()}
    _, d = oracle.forward(wl.fmt, n["w13"], n["s13"], n["w2"], n["s2"], n["x"], n["ids"], n["w"], debug=True)
    ss, off, _, _ = oracle.route_sort(n["ids"], wl.E)
    nv = int(off[-1])
    return wl, d, ss[:nv]


def _requantized_h(wl, d, slots, noise, seed):
    """h from the oracle's gate/up sums moved by uniform noise of `noise` times
    their largest magnitude, quantized with the oracle's rule (by sorted row)."""
    gu = d["gu"][slots].astype(np.float64)
    I = wl.I
    rng = np.random.default_rng(seed)
    gu = gu + noise * np.max(np.abs(gu)) * rng.uniform(-1, 1, gu.shape)
    g, u = gu[:, :I], gu[:, I:]
    h = (g / (1 + np.exp(-g)) * u).astype(np.float32)
    return oracle.quant_rows_f32(h, wl.fmt)


def test_h_check_accepts_gate_up_error_within_the_gemm_bound():
    """The h-code check of the GPU parity tests (parity_checks.check_h_codes)
    accepts every h the gate/up GEMM's own tolerance allows: sums moved by up
    to 1e-4 of the largest |g|, |u|, requantized."""
    from parity_checks import check_h_codes
    wl, d, slots = _study_layer()
    hq, hs = _requantized_h(wl, d, slots, 1e-4, 1)
    assert np.mean(hq != d["h_codes"][slots]) > 1e-3  # the noise does flip codes
    check_h_codes(wl.fmt, hq, hs, slots, d["h_codes"], d["h_scales"], wl.I, d["gu"])


def test_h_check_rejects_misplaced_or_wrong_h():
    """... and rejects what a bug would leave: two sorted rows' h swapped, one
    large code three e4m3 steps off, or h computed from sums moved by ten times
    the GEMM's tolerance."""
    from parity_checks import check_h_codes
    wl, d, slots = _study_layer()
    hq, hs = _requantized_h(wl, d, slots, 0.0, 1)
    check_h_codes(wl.fmt, hq, hs, slots, d["h_codes"], d["h_scales"], wl.I, d["gu"])  # exact h passes
    bad = hq.copy()
    bad[[3, 7]] = bad[[7, 3]]
    with pytest.raises(AssertionError):
        check_h_codes(wl.fmt, bad, hs, slots, d["h_codes"], d["h_scales"], wl.I, d["gu"])
    bad = hq.copy()
    r, c = np.unravel_index(np.argmax(np.where(hq & 0x7F < 0x70, hq & 0x7F, 0)), hq.shape)
    bad[r, c] = hq[r, c] + 3  # three steps up in magnitude, same sign
    with pytest.raises(AssertionError):
        check_h_codes(wl.fmt, bad, hs, slots, d["h_codes"], d["h_scales"], wl.I, d["gu"])
    hq10, hs10 = _requantized_h(wl, d, slots, 1e-3, 2)
    with pytest.raises(AssertionError):
        check_h_codes(wl.fmt, hq10, hs10, slots, d["h_codes"], d["h_scales"], wl.I, d["gu"])


"""Pins of the CPU oracle against things other than itself.

Each test ties one part of the oracle to a spec table (tests/golden), a library
routine (torch's float8 cast, torch.sort, torch float64 matmul), a closed form,
an invariant the pages fix, or brute force on tiny inputs.  A plausible mistake
anywhere in the oracle (a dropped term, a wrong sign or index, a transposed
operand, swapped gate/up halves, a skipped slot that leaks) fails at least one.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FP8, MX, BF16 = oracle.FMT_FP8_B128, oracle.FMT_MX, oracle.FMT_BF16


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b = line.split()
            rows.append((int(a, 0), float(b)))
    return rows


def _same(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(
        np.where(np.isnan(a), 0, a), np.where(np.isnan(b), 0, b)) and np.array_equal(
        np.signbit(np.where(np.isnan(a), 0, a)), np.signbit(np.where(np.isnan(b), 0, b)))


# ------------------------------------------------------------------ codecs --

def test_e4m3_decode_spec_points():
    pts = _golden("e4m3_points.txt")
    codes = np.array([c for c, _ in pts], np.uint8)
    assert _same(oracle.e4m3_decode(codes), [v for _, v in pts])


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert _same(oracle.e4m3_decode(codes), ref)


def test_e2m1_decode_spec_table():
    pts = _golden("e2m1_values.txt")
    nib = np.array([c for c, _ in pts], np.uint8)
    assert _same(oracle.e2m1_decode(nib), [v for _, v in pts])


def test_e8m0_decode_spec_points():
    pts = _golden("e8m0_points.txt")
    b = np.array([c for c, _ in pts], np.uint8)
    got = oracle.e8m0_decode(b)
    ref = np.array([v for _, v in pts])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.allclose(got[ok], ref[ok], rtol=1e-15, atol=0)


def _e4m3_values():
    return torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_encode_matches_torch_cast_dense_sweep():
    # every 97th fp32 bit pattern with |x| <= 448, both signs
    bits = np.arange(0, 0x43E00000 + 1, 97, dtype=np.uint32)
    pos = bits.view(np.float32)
    x = np.concatenate([pos, -pos])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_encode(x)
    assert np.array_equal(got, ref)


def test_e4m3_encode_ties_and_neighbours():
    v = _e4m3_values()
    mids = (v[1:] + v[:-1]) / 2  # exact in fp32: e4m3 values have 4 significant bits
    mids32 = mids.astype(np.float32)
    assert np.array_equal(mids32.astype(np.float64), mids)
    cand = [mids32, np.nextafter(mids32, np.float32(np.inf)), np.nextafter(mids32, np.float32(0)),
            v.astype(np.float32)]
    x = np.concatenate(cand + [-c for c in cand])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(x), ref)
    # ties go to the even mantissa code
    codes = oracle.e4m3_encode(mids32)
    assert np.all(codes % 2 == 0)


def test_e4m3_encode_saturates_and_keeps_sign():
    x = np.array([448.0, 449.0, 463.99, 464.0, 500.0, 1e30, 3.4e38], np.float32)
    assert np.all(oracle.e4m3_encode(x) == 0x7E)
    assert np.all(oracle.e4m3_encode(-x) == 0xFE)
    z = np.array([0.0, -0.0, 1e-30, -1e-30, 2.0 ** -11, -(2.0 ** -11)], np.float32)
    assert list(oracle.e4m3_encode(z)) == [0x00, 0x80, 0x00, 0x80, 0x00, 0x80]
    # 2^-10 is the tie between 0 and the smallest subnormal 2^-9: goes to 0 (even)
    assert list(oracle.e4m3_encode(np.array([2.0 ** -10, 2.0 ** -10 * 1.0001], np.float32))) == [0x00, 0x01]


# -------------------------------------------------------------- route sort --

def _rand_ids(rng, T, k, E, p_skip=0.1, p_bad=0.02, lo=0):
    ids = rng.integers(lo, lo + E, size=(T, k)).astype(np.int32)
    u = rng.random((T, k))
    ids[u < p_skip] = -1
    bad = u > 1 - p_bad
    ids[bad] = rng.choice(np.array([lo + E, lo + E + 7, -2, -100, lo - 1], np.int32), size=bad.sum())
    return ids


@pytest.mark.parametrize("T,k,E", [(1, 1, 1), (7, 2, 3), (64, 2, 8), (64, 8, 128), (333, 8, 256), (1000, 3, 5)])
def test_route_sort_matches_torch_stable_sort(T, k, E):
    rng = np.random.default_rng(T * 1000 + k * 10 + E)
    ids = _rand_ids(rng, T, k, E)
    ss, off, sp, inv = oracle.route_sort(ids, E)
    flat = torch.from_numpy(ids.reshape(-1).astype(np.int64))
    key = torch.where((flat >= 0) & (flat < E), flat, torch.full_like(flat, E))
    _, perm = torch.sort(key, stable=True)
    assert np.array_equal(ss, perm.numpy().astype(np.int32))
    cnt = np.bincount(key.numpy(), minlength=E + 1)
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(cnt)[:E]]).astype(np.int32))
    assert np.array_equal(sp[ss], np.arange(T * k))
    assert inv == int(((flat != -1) & ((flat < 0) | (flat >= E))).sum())


def test_route_sort_brute_force_tiny():
    ids = np.array([[2, -1], [0, 2], [1, 0], [-1, 5]], np.int32)
    ss, off, sp, inv = oracle.route_sort(ids, 3)
    # flat slots: 0:2 1:-1 2:0 3:2 4:1 5:0 6:-1 7:5(out of range)
    assert list(ss) == [2, 5, 4, 0, 3, 1, 6, 7]
    assert list(off) == [0, 2, 3, 5]
    assert inv == 1
    assert list(sp) == [3, 5, 0, 4, 2, 1, 6, 7]


def test_route_sort_expert_begin_is_a_shift():
    rng = np.random.default_rng(5)
    ids = _rand_ids(rng, 100, 4, 16, lo=0)
    a = oracle.route_sort(ids, 16, 0)
    shifted = np.where(ids == -1, -1, ids + 32).astype(np.int32)
    b = oracle.route_sort(shifted, 16, 32)
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(x, y)
    # -1 stays a plain skip, never counted as invalid
    assert b[3] == a[3]


def test_route_sort_degenerate():
    ss, off, sp, inv = oracle.route_sort(np.full((5, 2), -1, np.int32), 4)
    assert list(off) == [0, 0, 0, 0, 0] and list(ss) == list(range(10)) and inv == 0
    ss, off, sp, inv = oracle.route_sort(np.full((5, 2), 3, np.int32), 4)
    assert list(off) == [0, 0, 0, 0, 10] and list(ss) == list(range(10))
    ss, off, sp, inv = oracle.route_sort(np.zeros((0, 2), np.int32), 4)
    assert list(off) == [0] * 5 and ss.size == 0


# ------------------------------------------------------------------ router --

@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (50, 8, 2), (64, 128, 8), (40, 256, 8), (9, 512, 64), (30, 5, 5)])
@pytest.mark.parametrize("renorm", [True, False])
def test_router_matches_torch_softmax_topk(T, E, k, renorm):
    # distinct logits (N(0,1) draws): the selection is unique, so torch.topk of
    # the float64 softmax fixes ids and their order; weights are that softmax
    # (renormalised over the k), rounded once to fp32
    rng = np.random.default_rng(T * 7 + E * 3 + k)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = oracle.router_topk(lg, k, renorm)
    p = torch.softmax(torch.from_numpy(lg).double(), dim=-1)
    pv, pi = torch.topk(p, k, dim=-1)
    if renorm:
        pv = pv / pv.sum(dim=-1, keepdim=True)
    assert np.array_equal(ids, pi.numpy().astype(np.int32))
    np.testing.assert_allclose(w, pv.float().numpy(), rtol=2.0 ** -23, atol=0)


def test_router_ties_take_the_lower_id():
    # many equal logits: torch's stable descending sort and a brute force both
    # put the lower id first among equals
    rng = np.random.default_rng(11)
    lg = rng.integers(0, 4, size=(64, 32)).astype(np.float32)
    lg[:, 5] = -0.0
    lg[:, 6] = 0.0  # -0 and +0 are equal logits
    ids, _ = oracle.router_topk(lg, 6)
    _, perm = torch.sort(torch.from_numpy(lg), dim=-1, descending=True, stable=True)
    assert np.array_equal(ids, perm[:, :6].numpy().astype(np.int32))
    for t in range(4):
        brute = sorted(range(32), key=lambda e: (-float(lg[t, e]), e))[:6]
        assert list(ids[t]) == brute


def test_router_closed_forms():
    # all logits equal: ids 0..k-1, weights exactly 1/k (renormalised) or 1/E
    lg = np.full((3, 16), 0.75, np.float32)
    ids, w = oracle.router_topk(lg, 4)
    assert (ids == np.arange(4)).all() and (w == np.float32(0.25)).all()
    ids, w = oracle.router_topk(lg, 4, renormalize=False)
    assert (w == np.float32(1.0 / 16)).all()
    # two experts, top-1: renormalised weight 1; otherwise the logistic
    # function of the logit gap
    lg = np.array([[2.0, -1.0], [0.5, 3.0]], np.float32)
    ids, w = oracle.router_topk(lg, 1)
    assert list(ids[:, 0]) == [0, 1] and (w == 1.0).all()
    ids, w = oracle.router_topk(lg, 1, renormalize=False)
    assert w[0, 0] == np.float32(1.0 / (1.0 + math.exp(-3.0)))
    assert w[1, 0] == np.float32(1.0 / (1.0 + math.exp(-2.5)))
    # k = E with renormalisation: the whole softmax, sorted
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((5, 7)).astype(np.float32)
    ids, w = oracle.router_topk(lg, 7)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=4e-7)
    assert (np.diff(w, axis=1) <= 0).all()


def test_router_shift_invariance_large_logits():
    # adding a constant to every logit of a token changes nothing; the shifted
    # logits are exact in fp32 (multiples of 1/64, |l| < 4, shift 1000), and
    # exp(1000) would overflow, so the row maximum must be taken out first
    rng = np.random.default_rng(3)
    lg = (rng.integers(-256, 256, size=(20, 64)) / 64.0).astype(np.float32)
    a = oracle.router_topk(lg, 6)
    for c in (1000.0, -1000.0):
        sh = (lg + np.float32(c)).astype(np.float32)
        assert np.array_equal(sh - np.float32(c), lg)
        b = oracle.router_topk(sh, 6)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.isfinite(a[1]).all()


def test_router_rejects_bad_arguments():
    with pytest.raises(oracle.OracleError):
        oracle.router_topk(np.zeros((2, 4), np.float32), 5)
    ids, w = oracle.router_topk(np.zeros((0, 4), np.float32), 2)
    assert ids.shape == (0, 2) and w.shape == (0, 2)


# ---------------------------------------------------- activation quantization --

def _bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _e4m3_codes_with_max(rng, n):
    """n e4m3 codes (finite, with value exactly representable in bf16) whose max |value| is 448."""
    c = rng.integers(0, 0x7F, size=n).astype(np.uint8)
    c |= (rng.random(n) < 0.5).astype(np.uint8) << 7
    c[rng.integers(0, n)] = 0x7E | (c[0] & 0x80)
    return c


@pytest.mark.parametrize("fmt", [FP8, MX])
@pytest.mark.parametrize("p", [-20, -3, 0, 5, 40])
def test_quant_reproduces_scaled_codes(fmt, p):
    """A block equal to 2^p * c (max|c| = 448) gives back the codes c and the scale 2^p exactly."""
    rng = np.random.default_rng(100 + p + 7 * fmt)
    B = 128 if fmt == FP8 else 32
    rows, H = 3, 4 * B
    c = np.stack([_e4m3_codes_with_max(rng, B) for _ in range(rows * H // B)]).reshape(rows, H)
    vals = torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy() * 2.0 ** p
    x = _bf16_bits(vals)
    assert np.array_equal(torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double().numpy(), vals)
    codes, sc = oracle.quant_rows_bf16(x, fmt)
    # the codes of 0 and -0 both mean zero; compare values
    got = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    want = torch.from_numpy(c).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(got, want)
    if fmt == FP8:
        assert np.all(sc == np.float32(2.0 ** p))
    else:
        assert np.all(sc == 127 + p)


@pytest.mark.parametrize("fmt", [FP8, MX])
def test_quant_zero_block_and_floor(fmt):
    B = 128 if fmt == FP8 else 32
    x = np.zeros((2, 2 * B), np.float32)
    x[1, B + 3] = 1e-6  # below the 1e-4 floor
    codes, sc = oracle.quant_rows_f32(x, fmt)
    r = np.float32(np.float32(1e-4) / np.float32(448.0))
    if fmt == FP8:
        assert np.all(sc == r)
        # 1e-6 / (1e-4/448) = 4.48 -> nearest e4m3 is 4.5 (code 0x49)
        assert codes[1, B + 3] == 0x49
    else:
        # ceil(log2(2.232e-7)) = -22 -> byte 105; 1e-6 * 2^22 = 4.194 -> nearest e4m3 is 4.0 (0x48)
        assert np.all(sc == 105)
        assert codes[1, B + 3] == 0x48
    codes[1, B + 3] = 0
    assert np.all(codes == 0)


@pytest.mark.parametrize("fmt", [FP8, MX])
def test_quant_single_nonzero(fmt):
    B = 128 if fmt == FP8 else 32
    x = np.zeros((4, B), np.float32)
    vals = [3.0, -0.37, 1e-4, 65504.0]
    for r, v in enumerate(vals):
        x[r, 11] = v
    codes, sc = oracle.quant_rows_f32(x, fmt)
    for r, v in enumerate(vals):
        if fmt == FP8:
            assert codes[r, 11] == (0xFE if v < 0 else 0x7E)
        else:
            e = int(sc[r, 0]) - 127
            assert 2.0 ** (e - 1) < abs(v) / 448 <= 2.0 ** e
            q = abs(v) * 2.0 ** -e
            assert 224 < q <= 448
            want = torch.tensor([q * np.sign(v)], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)
            assert codes[r, 11] == int(want[0])


@pytest.mark.parametrize("fmt", [FP8, MX])
def test_quant_power_of_two_scaling_invariance(fmt):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((16, 256)).astype(np.float32)
    c0, s0 = oracle.quant_rows_f32(x, fmt)
    for p in (-5, 1, 9):
        c1, s1 = oracle.quant_rows_f32(x * np.float32(2.0 ** p), fmt)
        assert np.array_equal(c0, c1)
        if fmt == FP8:
            assert np.array_equal(s1, s0 * np.float32(2.0 ** p))
        else:
            assert np.array_equal(s1.astype(int), s0.astype(int) + p)


def test_quant_codes_equal_torch_division_and_cast():
    """Given the block scales, FP8-format codes are torch's float8 cast of torch's fp32 division x / s."""
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((512, 1024)) * np.exp(rng.standard_normal((512, 1)))).astype(np.float32)
    # Half the blocks hold values right at e4m3 rounding midpoints times the block
    # scale (and one fp32 ulp either side): there x / s and x * (1 / s) can round
    # to different codes, so the division itself is pinned.
    v = _e4m3_values()
    mids = ((v[1:] + v[:-1]) / 2)[8:]
    blocks = x.reshape(-1, 128)
    for b in range(0, blocks.shape[0], 2):
        s0 = np.float32(np.exp(rng.uniform(-8, 8)))
        blocks[b, 0] = np.float32(448.0) * s0
        m = rng.choice(mids, size=127).astype(np.float32) * s0
        step = rng.integers(-1, 2, size=127)
        m = np.where(step > 0, np.nextafter(m, np.float32(np.inf)), np.where(step < 0, np.nextafter(m, np.float32(0)), m))
        blocks[b, 1:] = m * np.where(rng.random(127) < 0.5, -1, 1).astype(np.float32)
    x = blocks.reshape(512, 1024)
    codes, sc = oracle.quant_rows_f32(x, FP8)
    xt = torch.from_numpy(x).view(512, 8, 128)
    st = torch.from_numpy(sc).view(512, 8, 1)
    q = torch.div(xt, st).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).view(512, 1024)
    assert np.array_equal(codes, q.numpy())
    # the scale itself: fp32 max(amax, 1e-4) / 448
    amax = xt.abs().amax(dim=2)
    assert np.array_equal(sc, (torch.clamp(amax, min=np.float32(1e-4)) / 448.0).numpy())


@pytest.mark.parametrize("fmt", [FP8, MX])
def test_quant_error_bound_and_bf16_entry(fmt):
    rng = np.random.default_rng(11)
    xf = (rng.standard_normal((32, 512)) * np.exp(rng.standard_normal((32, 1)) * 3)).astype(np.float32)
    xb = _bf16_bits(xf)
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).float().numpy()
    codes, sc = oracle.quant_rows_bf16(xb, fmt)
    c2, s2 = oracle.quant_rows_f32(x, fmt)
    assert np.array_equal(codes, c2) and np.array_equal(sc, s2)
    B = 128 if fmt == FP8 else 32
    s = sc.astype(np.float64) if fmt == FP8 else 2.0 ** (sc.astype(np.float64) - 127)
    s_full = np.repeat(s, B, axis=1)
    q = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    xs = x.astype(np.float64) / s_full
    assert np.all(np.abs(xs) <= 448 * (1 + 2 ** -23))
    # half an e4m3 ulp at |x/s| (normal range: 2^(floor(log2|v|)-3); subnormal: 2^-9), plus fp32 division slack
    mag = np.maximum(np.abs(xs), 2.0 ** -6)
    half_ulp = 0.5 * 2.0 ** (np.floor(np.log2(mag)) - 3)
    assert np.all(np.abs(xs - q) <= half_ulp * (1 + 1e-6) + np.abs(xs) * 2 ** -23)
    # amax element of each block lands within half an ulp of 448
    blk = np.abs(xs).reshape(32, -1, B).max(axis=2)
    if fmt == FP8:
        assert np.allclose(blk, 448, rtol=1e-6)
    else:
        assert np.all((blk > 224) & (blk <= 448))


# ------------------------------------------------- static activation scales --
# The static scheme hands the layer its activation scales precomputed, per
# block (the same blocks and scale types as the dynamic rule); only the amax
# pass goes away, the encoding is unchanged.


def _torch_static_codes(x_bits, fmt, scales):
    """Independent encoding with torch: FP8, torch's fp32 division by the block
    scale, clamped to +-448 and cast to float8_e4m3fn; MX, exact scaling by
    2^-(b-127) in float64 and the same clamp and cast."""
    x = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(torch.bfloat16)
    rows, H = x.shape
    B = 128 if fmt == FP8 else 32
    xb = x.float().view(rows, H // B, B)
    if fmt == FP8:
        q = torch.div(xb, torch.from_numpy(np.ascontiguousarray(scales, np.float32)).view(rows, H // B, 1))
    else:
        e = torch.from_numpy(np.ascontiguousarray(scales).astype(np.int64) - 127).view(rows, H // B, 1)
        q = xb.double() * torch.exp2(-e.double())
    return q.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).view(rows, H).numpy()


@pytest.mark.parametrize("fmt", [FP8, MX])
def test_static_scales_equal_to_dynamic_give_the_dynamic_codes(fmt):
    """Static scales that happen to equal the dynamic ones give bit-identical codes."""
    rng = np.random.default_rng(31 + fmt)
    x = (rng.standard_normal((64, 512)) * np.exp(rng.uniform(-10, 10, size=(64, 1)))).astype(np.float32)
    x[::7, :128] = 0.0
    x[3::11] *= 1e-7
    xb = _bf16_bits(x)
    codes, sc = oracle.quant_rows_bf16(xb, fmt)
    assert np.array_equal(oracle.quant_rows_bf16_static(xb, fmt, sc), codes)


@pytest.mark.parametrize("fmt", [FP8, MX])
@pytest.mark.parametrize("p", [-30, -4, 0, 3, 60])
def test_static_power_of_two_scale_reproduces_codes(fmt, p):
    """x = c * 2^p for e4m3 codes c, with the static scale 2^p: the codes are c
    (as values), whatever the block's amax (no code needs to reach 448)."""
    rng = np.random.default_rng(40 + p + 5 * fmt)
    B = 128 if fmt == FP8 else 32
    rows, H = 4, 2 * 128
    c = rng.integers(0, 0x77, size=(rows, H)).astype(np.uint8)  # magnitudes up to 240
    c |= (rng.random((rows, H)) < 0.5).astype(np.uint8) << 7
    vals = torch.from_numpy(c).view(torch.float8_e4m3fn).double().numpy() * 2.0 ** p
    xb = _bf16_bits(vals)
    assert np.array_equal(_bits_to_f64(xb), vals)
    sc = np.full((rows, H // B), np.float32(2.0 ** p), np.float32) if fmt == FP8 else \
        np.full((rows, H // B), 127 + p, np.uint8)
    codes = oracle.quant_rows_bf16_static(xb, fmt, sc)
    got = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(got, torch.from_numpy(c).view(torch.float8_e4m3fn).double().numpy())


@pytest.mark.parametrize("fmt", [FP8, MX])
def test_static_values_past_448_s_saturate(fmt):
    """|x| >= 448 s gives the largest code of x's sign (0x7E / 0xFE), and so does
    anything that rounds up past 448 (464 s would be the next binade's first
    value); just below the midpoint 448 s < |x| < 464 s stays 448 too."""
    B = 128 if fmt == FP8 else 32
    s32 = np.float32(0.75) if fmt == FP8 else None
    s = 0.75 if fmt == FP8 else 2.0 ** -3
    vals = np.array([448.0, 449.0, 460.0, 464.0, 500.0, 1e4, 3e38 / 1e30, 1e30], np.float64) * s
    x = np.zeros((2, 128), np.float64)
    x[0, :vals.size] = vals
    x[1, :vals.size] = -vals
    xb = _bf16_bits(x)
    xv = _bits_to_f64(xb)
    assert np.all(np.abs(xv[:, :vals.size]) >= 440 * s)  # bf16 rounding keeps them at or past 448 s (within bf16)
    sc = np.full((2, 128 // B), s32, np.float32) if fmt == FP8 else np.full((2, 128 // B), 124, np.uint8)
    codes = oracle.quant_rows_bf16_static(xb, fmt, sc)
    big = np.abs(xv[0, :vals.size]) >= 448 * s
    assert np.all(codes[0, :vals.size][big] == 0x7E) and np.all(codes[1, :vals.size][big] == 0xFE)
    assert np.array_equal(codes, _torch_static_codes(xb, fmt, sc))


@pytest.mark.parametrize("fmt", [FP8, MX])
def test_static_codes_equal_torch_division_and_cast(fmt):
    """Arbitrary (non-power-of-two, FP8) static scales, values well past and
    well under them, and values at e4m3 rounding midpoints of x / s (one fp32
    ulp either side): torch's fp32 division and float8 cast give the same codes
    (this pins a division, not a product with 1 / s)."""
    rng = np.random.default_rng(77 + fmt)
    B = 128 if fmt == FP8 else 32
    rows, H = 256, 512
    if fmt == FP8:
        sc = np.exp(rng.uniform(-12, 6, size=(rows, H // B))).astype(np.float32)
        s_full = np.repeat(sc.astype(np.float64), B, axis=1)
    else:
        sc = rng.integers(100, 140, size=(rows, H // B)).astype(np.uint8)
        s_full = np.repeat(2.0 ** (sc.astype(np.float64) - 127), B, axis=1)
    x = rng.standard_normal((rows, H)) * s_full * np.exp(rng.uniform(-4, 7, size=(rows, 1)))
    if fmt == FP8:
        # half the rows: per block a bf16 value x0 and a midpoint m0 between
        # neighbouring e4m3 values, the block scale s = fp32(x0 / m0), and the
        # block's entries x0 * 2^-j, so that every x / s lies within an fp32 ulp
        # of an e4m3 rounding midpoint
        v = _e4m3_values()
        mids = ((v[1:] + v[:-1]) / 2)[16:]
        for r in range(rows // 2):
            for b in range(H // B):
                x0 = float(_bits_to_f64(_bf16_bits([rng.uniform(0.5, 4.0)]))[0])
                m0 = float(rng.choice(mids[mids > 16]))
                sc[r, b] = np.float32(x0 / m0)
                j = rng.integers(0, 4, size=B)
                x[r, b * B:(b + 1) * B] = x0 * 2.0 ** -j * np.where(rng.random(B) < 0.5, -1, 1)
    xb = _bf16_bits(x)
    codes = oracle.quant_rows_bf16_static(xb, fmt, sc)
    assert np.array_equal(codes, _torch_static_codes(xb, fmt, sc))
    if fmt == FP8:
        # the midpoint rows do hold quotients whose reciprocal product rounds
        # differently (else this test could not tell the two apart)
        xs = _bits_to_f64(xb)[: rows // 2].astype(np.float32)
        s_rep = np.repeat(sc[: rows // 2], B, axis=1)
        by_recip = torch.from_numpy((xs * (np.float32(1) / s_rep)).astype(np.float32)).clamp(-448, 448)
        c_recip = by_recip.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.count_nonzero(c_recip != codes[: rows // 2]) > 0


@pytest.mark.parametrize("fmt", [FP8, MX])
def test_static_one_row_broadcasts(fmt):
    """Row stride 0: one row of block scales serves every token, the same as
    repeating it per token."""
    rng = np.random.default_rng(90 + fmt)
    B = 128 if fmt == FP8 else 32
    xb = _bf16_bits(rng.standard_normal((9, 384)))
    row = np.exp(rng.uniform(-3, 0, size=384 // B)).astype(np.float32) if fmt == FP8 else \
        rng.integers(120, 127, size=384 // B).astype(np.uint8)
    a = oracle.quant_rows_bf16_static(xb, fmt, row, row_stride=0)
    b = oracle.quant_rows_bf16_static(xb, fmt, np.tile(row, (9, 1)))
    assert np.array_equal(a, b)
    with pytest.raises(oracle.OracleError):
        oracle.quant_rows_bf16_static(xb, fmt, np.tile(row, (9, 1)), row_stride=1)  # shorter than a row


# ----------------------------------------------------------- grouped GEMM --

def _fp8_decode_t(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64)


def _dequant_w_fp8(codes, scales):
    E, N, K = codes.shape
    s = torch.from_numpy(scales).double().repeat_interleave(128, 1).repeat_interleave(128, 2)
    return _fp8_decode_t(codes) * s


_E2M1 = {c: v for c, v in _golden("e2m1_values.txt")}


def _dequant_w_mx(packed, scales):
    lut = np.array([_E2M1[i] for i in range(16)])
    lo = lut[packed & 0xF]
    hi = lut[packed >> 4]
    vals = np.stack([lo, hi], axis=-1).reshape(packed.shape[0], packed.shape[1], -1)
    s = 2.0 ** (scales.astype(np.float64) - 127)
    return torch.from_numpy(vals * np.repeat(s, 32, axis=2))


def _dequant_act(codes, scales, fmt):
    q = _fp8_decode_t(codes)
    if fmt == FP8:
        s = torch.from_numpy(scales).double().repeat_interleave(128, 1)
    else:
        s = torch.from_numpy(2.0 ** (scales.astype(np.float64) - 127)).repeat_interleave(32, 1)
    return q * s


@pytest.mark.parametrize("fmt", [FP8, MX])
def test_grouped_gemm_matches_torch_matmul(fmt):
    rng = np.random.default_rng(3 + fmt)
    E, N, K, T, k = 3, 256, 384, 20, 2
    if fmt == FP8:
        b, bs = W.fp8_weights(E, N, K, seed=9, tag="g")
    else:
        b, bs = W.fp4_weights(E, N, K, seed=9, tag="g")
    b, bs = b.numpy(), bs.numpy()
    x = rng.standard_normal((T, K)).astype(np.float32)
    a, asc = oracle.quant_rows_f32(x, fmt)
    ids = _rand_ids(rng, T, k, E, p_skip=0.2, p_bad=0.0)
    ss, off, _, _ = oracle.route_sort(ids, E)
    got = oracle.grouped_gemm(fmt, a, asc, off, b, bs, N, K, row_index=ss, row_div=k)
    A = _dequant_act(a, asc, fmt)
    Bd = _dequant_w_fp8(b, bs) if fmt == FP8 else _dequant_w_mx(b, bs)
    for e in range(E):
        rows = ss[off[e]:off[e + 1]] // k
        ref = A[torch.from_numpy(rows.astype(np.int64))] @ Bd[e].T
        np.testing.assert_allclose(got[off[e]:off[e + 1]], ref.numpy(), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- forward --

def _small_inputs(fmt, T=24, H=256, I=256, E=4, k=3, seed=0, skip=0.15, device="cpu"):
    x = W.hidden_states(T, H, seed, device)
    ids, w = W.routing(T, E, k, "uniform", seed, skip=skip)
    if fmt == FP8:
        w13, s13 = W.fp8_weights(E, 2 * I, H, seed, "w13")
        w2, s2 = W.fp8_weights(E, H, I, seed, "w2")
    else:
        w13, s13 = W.fp4_weights(E, 2 * I, H, seed, "w13")
        w2, s2 = W.fp4_weights(E, H, I, seed, "w2")
    return {n: W.to_numpy(t) for n, t in dict(x=x, ids=ids, w=w, w13=w13, s13=s13, w2=w2, s2=s2).items()}


def _run(fmt, d, limit=None, **kw):
    return oracle.forward(fmt, d["w13"], d["s13"], d["w2"], d["s2"], d["x"], d["ids"], d["w"], swiglu_limit=limit,
                          **kw)


def _bits_to_f64(b):
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).double().numpy()


def _brute_force(fmt, d, limit=None, act=None):
    """Every expert for every token with torch float64 matmuls, then the routed
    ones are picked.  act: (codes, scales) of the layer input, else the oracle's
    dynamic quantization."""
    T, H = d["x"].shape
    E = d["w13"].shape[0]
    I = d["w13"].shape[1] // 2
    k = d["ids"].shape[1]
    a, asc = oracle.quant_rows_bf16(d["x"], fmt) if act is None else act
    A = _dequant_act(a, asc, fmt)
    if fmt == FP8:
        W13, W2 = _dequant_w_fp8(d["w13"], d["s13"]), _dequant_w_fp8(d["w2"], d["s2"])
    else:
        W13, W2 = _dequant_w_mx(d["w13"], d["s13"]), _dequant_w_mx(d["w2"], d["s2"])
    GU = torch.einsum("th,enh->etn", A, W13)  # [E, T, 2I]
    g, u = GU[..., :I], GU[..., I:]
    if limit is not None:
        g = torch.clamp(g, max=limit)
        u = torch.clamp(u, -limit, limit)
    h = (torch.nn.functional.silu(g) * u).float().numpy()  # [E, T, I] fp32
    out = np.zeros((T, H), np.float64)
    hq_all = {}
    for e in range(E):
        hq, hs = oracle.quant_rows_f32(h[e], fmt)
        hq_all[e] = (hq, hs)
        Y = (_dequant_act(hq, hs, fmt) @ W2[e].T).numpy()  # [T, H]
        hq_all[e] = (hq, hs, Y)
    for t in range(T):
        for j in range(k):
            e = d["ids"][t, j]
            if 0 <= e < E:
                out[t] += float(d["w"][t, j]) * hq_all[e][2][t]
    bits = torch.from_numpy(out).float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return bits, GU.numpy()


@pytest.mark.parametrize("fmt,limit", [(FP8, None), (FP8, 0.05), (MX, None), (MX, 0.05)])
def test_forward_matches_dense_brute_force(fmt, limit):
    d = _small_inputs(fmt)
    out, dbg = _run(fmt, d, limit=limit, debug=True)
    ref, GU = _brute_force(fmt, d, limit)
    # both sides are fp64 sums in different orders, rounded to bf16: equal, or one bf16 ulp apart
    o, r = _bits_to_f64(out), _bits_to_f64(ref)
    assert np.all(np.abs(o - r) <= np.abs(r) * 2 ** -7 + 1e-30)
    assert np.mean(out == ref) > 0.99
    # the L1 debug output is the per-slot gate_up product
    ids = d["ids"]
    T, k = ids.shape
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            if 0 <= e < d["w13"].shape[0]:
                np.testing.assert_allclose(dbg["gu"][t * k + j], GU[e, t], rtol=1e-6, atol=1e-9)
            else:
                assert np.all(np.isnan(dbg["gu"][t * k + j]))


@pytest.mark.parametrize("fmt", [FP8, MX])
def test_forward_static_scales(fmt):
    """Static activation scales: equal to the dynamic ones, the forward is the
    dynamic forward bit for bit; other scales (per token, and one broadcast row)
    match a dense brute force whose activation codes come from torch's division
    and float8 cast (h stays dynamic)."""
    d = _small_inputs(fmt)
    _, dyn_sc = oracle.quant_rows_bf16(d["x"], fmt)
    assert np.array_equal(_run(fmt, d, act_scales=dyn_sc), _run(fmt, d))
    rng = np.random.default_rng(5 + fmt)
    T, H = d["x"].shape
    B = 128 if fmt == FP8 else 32
    if fmt == FP8:
        per_tok = (dyn_sc * np.exp(rng.uniform(-0.7, 0.7, size=dyn_sc.shape))).astype(np.float32)
        row = np.full(H // B, np.float32(3.1 / 448), np.float32)  # saturates the largest activations
    else:
        per_tok = (dyn_sc.astype(np.int64) + rng.integers(-1, 2, size=dyn_sc.shape)).astype(np.uint8)
        row = np.full(H // B, 125, np.uint8)
    for sc, stride in ((per_tok, None), (row, 0)):
        out = _run(fmt, d, act_scales=sc, act_scales_row_stride=stride)
        full = sc if sc.ndim == 2 else np.tile(sc, (T, 1))
        ref, _ = _brute_force(fmt, d, None, act=(_torch_static_codes(d["x"], fmt, full), full))
        o, r = _bits_to_f64(out), _bits_to_f64(ref)
        assert np.all(np.abs(o - r) <= np.abs(r) * 2 ** -7 + 1e-30)
        assert np.mean(out == ref) > 0.99


def test_forward_textbook_reduction_k1_e1():
    """k = 1, E = 1, weight 1: a plain quantized SwiGLU MLP y = W2 q(silu(W1 x) * (W3 x))."""
    d = _small_inputs(FP8, T=16, E=1, k=1, skip=0.0)
    d["w"] = np.ones_like(d["w"])
    out = _run(FP8, d)
    a, asc = oracle.quant_rows_bf16(d["x"], FP8)
    A = _dequant_act(a, asc, FP8)
    W13 = _dequant_w_fp8(d["w13"], d["s13"])[0]
    I = W13.shape[0] // 2
    W1, W3 = W13[:I], W13[I:]
    h = (torch.nn.functional.silu(A @ W1.T) * (A @ W3.T)).float().numpy()
    hq, hs = oracle.quant_rows_f32(h, FP8)
    y = _dequant_act(hq, hs, FP8) @ _dequant_w_fp8(d["w2"], d["s2"])[0].T
    ref = y.float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.mean(out == ref) > 0.99
    assert np.allclose(_bits_to_f64(out), _bits_to_f64(ref), rtol=2 ** -7, atol=0)


def test_forward_gate_is_the_first_half():
    """Gate rows [0, I) go through silu: a strongly negative gate silences the slot, a negative up does not."""
    d = _small_inputs(FP8, T=8, E=1, k=1, skip=0.0)
    I = d["w13"].shape[1] // 2
    x = np.abs(_bits_to_f64(d["x"])).astype(np.float32)
    d["x"] = _bf16_bits(x)
    pos = np.full_like(d["w13"][:, :I], 0x38)  # +1.0
    neg = np.full_like(d["w13"][:, :I], 0xB8)  # -1.0
    ones = np.ones_like(d["s13"])
    d1 = dict(d, w13=np.concatenate([neg, pos], axis=1), s13=ones)  # g << 0: silu(g) ~ 0
    d2 = dict(d, w13=np.concatenate([pos, neg], axis=1), s13=ones)  # g >> 0, u << 0
    o1, o2 = _bits_to_f64(_run(FP8, d1)), _bits_to_f64(_run(FP8, d2))
    assert np.max(np.abs(o1)) < 1e-6 * np.max(np.abs(o2))
    assert np.max(np.abs(o2)) > 0


@pytest.mark.parametrize("fmt", [FP8, MX])
def test_forward_all_skipped_is_zero_even_with_nan_weights(fmt):
    d = _small_inputs(fmt, T=6)
    d["ids"] = np.full_like(d["ids"], -1)
    d["w"] = np.full_like(d["w"], np.nan)
    out = _run(fmt, d)
    assert np.all(out == 0)


@pytest.mark.parametrize("fmt", [FP8, MX])
def test_forward_skip_equals_dropping_the_slot(fmt):
    d = _small_inputs(fmt, T=10, k=3, skip=0.0)
    ids = d["ids"].copy()
    ids[:, 1] = -1
    wts = d["w"].copy()
    wts[:, 1] = np.nan  # never read
    a = _run(fmt, dict(d, ids=ids, w=wts))
    b = _run(fmt, dict(d, ids=np.ascontiguousarray(d["ids"][:, [0, 2]]), w=np.ascontiguousarray(d["w"][:, [0, 2]])))
    assert np.array_equal(a, b)
    # an id outside the local range behaves like -1
    ids_bad = ids.copy()
    ids_bad[:, 1] = 4 + 9
    c = _run(fmt, dict(d, ids=ids_bad, w=wts))
    assert np.array_equal(a, c)


@pytest.mark.parametrize("fmt", [FP8, MX])
def test_forward_weight_scaling_and_token_permutation(fmt):
    d = _small_inputs(fmt, T=20)
    base = _run(fmt, d)
    twice = _run(fmt, dict(d, w=(d["w"] * 2).astype(np.float32)))
    assert np.array_equal(_bits_to_f64(twice), 2 * _bits_to_f64(base))
    perm = np.random.default_rng(1).permutation(20)
    dp = dict(d, x=d["x"][perm], ids=d["ids"][perm], w=d["w"][perm])
    assert np.array_equal(_run(fmt, dp), base[perm])


@pytest.mark.parametrize("fmt", [FP8, MX])
def test_forward_expert_begin_shift_and_subset(fmt):
    d = _small_inputs(fmt, T=12)
    base = _run(fmt, d)
    ids = np.where(d["ids"] >= 0, d["ids"] + 64, -1).astype(np.int32)
    assert np.array_equal(_run(fmt, dict(d, ids=ids), expert_begin=64), base)
    sub = np.array([0, 5, 11], np.int32)
    part = _run(fmt, d, tokens=sub)
    assert np.array_equal(part[sub], base[sub])
    rest = np.setdiff1d(np.arange(12), sub)
    assert np.all(part[rest] == 0)


@pytest.mark.parametrize("fmt", [FP8, MX])
def test_forward_loose_limit_equals_no_limit(fmt):
    d = _small_inputs(fmt, T=8)
    base, dbg = _run(fmt, d, debug=True)
    big = float(np.nanmax(np.abs(dbg["gu"]))) * 1.01
    assert np.array_equal(_run(fmt, d, limit=big), base)
    assert np.array_equal(_run(fmt, d, limit=1e30), base)


def test_forward_duplicate_expert_in_one_token_counts_twice():
    d = _small_inputs(FP8, T=6, k=2, skip=0.0)
    ids = np.stack([d["ids"][:, 0], d["ids"][:, 0]], axis=1).astype(np.int32)
    w = np.stack([d["w"][:, 0], d["w"][:, 0]], axis=1).astype(np.float32)
    two = _bits_to_f64(_run(FP8, dict(d, ids=ids, w=w)))
    one = _bits_to_f64(_run(FP8, dict(d, ids=ids[:, :1].copy(), w=(w[:, :1] * 2).copy())))
    assert np.array_equal(two, one)


def test_forward_tiny_workload_runs_fast():
    import time
    wl = W.WORKLOADS["tiny"]
    n = {k: W.to_numpy(v) for k, v in W.inputs(wl).items()}
    t0 = time.time()
    out = oracle.forward(wl.fmt, n["w13"], n["s13"], n["w2"], n["s2"], n["x"], n["ids"], n["w"])
    assert time.time() - t0 < 5
    assert np.isfinite(_bits_to_f64(out)).all() and np.any(out != 0)


def test_forward_rejects_bad_arguments():
    d = _small_inputs(FP8, T=4)
    with pytest.raises(oracle.OracleError):
        _run(FP8, d, limit=float("nan"))
    with pytest.raises(oracle.OracleError):
        _run(FP8, d, limit=-1.0)
    with pytest.raises(oracle.OracleError):
        oracle.quant_rows_f32(np.zeros((2, 100), np.float32), FP8)


# ------------------------------------------------------- bf16 experts --

def _bf16_t(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double()


def _bf16_inputs(T=24, H=256, I=256, E=4, k=3, seed=0, skip=0.15):
    x = W.hidden_states(T, H, seed)
    ids, w = W.routing(T, E, k, "uniform", seed, skip=skip)
    w13 = W.bf16_weights(E, 2 * I, H, seed, "w13")
    w2 = W.bf16_weights(E, H, I, seed, "w2")
    return {n: W.to_numpy(t) for n, t in dict(x=x, ids=ids, w=w, w13=w13, w2=w2).items()}


def test_bf16_grouped_gemm_matches_torch_matmul():
    rng = np.random.default_rng(8)
    E, N, K, T, k = 3, 256, 384, 20, 2
    b = W.to_numpy(W.bf16_weights(E, N, K, seed=9, tag="g"))
    a = W.to_numpy(W.hidden_states(T, K, 4))
    ids = _rand_ids(rng, T, k, E, p_skip=0.2, p_bad=0.0)
    ss, off, _, _ = oracle.route_sort(ids, E)
    got = oracle.grouped_gemm(BF16, a, None, off, b, None, N, K, row_index=ss, row_div=k)
    A, B = _bf16_t(a), _bf16_t(b)
    for e in range(E):
        rows = torch.from_numpy((ss[off[e]:off[e + 1]] // k).astype(np.int64))
        np.testing.assert_allclose(got[off[e]:off[e + 1]], (A[rows] @ B[e].T).numpy(), rtol=1e-12, atol=1e-12)


def _bf16_brute_force(d, limit=None):
    """Every expert for every token with torch float64 matmuls (h rounded to
    bf16 through fp32), then the routed ones picked and weighted."""
    X, W13, W2 = _bf16_t(d["x"]), _bf16_t(d["w13"]), _bf16_t(d["w2"])
    E, I = W13.shape[0], W13.shape[1] // 2
    T, k = d["ids"].shape
    GU = torch.einsum("th,enh->etn", X, W13)
    g, u = GU[..., :I], GU[..., I:]
    if limit is not None:
        g = torch.clamp(g, max=limit)
        u = torch.clamp(u, -limit, limit)
    h = (torch.nn.functional.silu(g) * u).float().to(torch.bfloat16).double()
    Y = torch.einsum("eti,ehi->eth", h, W2).numpy()
    out = np.zeros((T, X.shape[1]), np.float64)
    for t in range(T):
        for j in range(k):
            e = d["ids"][t, j]
            if 0 <= e < E:
                out[t] += float(d["w"][t, j]) * Y[e, t]
    return torch.from_numpy(out).float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("limit", [None, 0.05])
def test_bf16_forward_matches_dense_brute_force(limit):
    d = _bf16_inputs()
    out = oracle.forward(BF16, d["w13"], None, d["w2"], None, d["x"], d["ids"], d["w"], swiglu_limit=limit)
    ref = _bf16_brute_force(d, limit)
    o, r = _bits_to_f64(out), _bits_to_f64(ref)
    assert np.all(np.abs(o - r) <= np.abs(r) * 2 ** -7 + 1e-30)
    assert np.mean(out == ref) > 0.99
    assert np.any(o != 0)


def test_bf16_forward_textbook_swiglu_mlp():
    """k = 1, E = 1, weight 1: y = W2 bf16(silu(W1 x) * (W3 x)) with
    torch.nn.functional.silu and float64 matmuls."""
    d = _bf16_inputs(T=16, E=1, k=1, skip=0.0)
    d["w"] = np.ones_like(d["w"])
    out = oracle.forward(BF16, d["w13"], None, d["w2"], None, d["x"], d["ids"], d["w"])
    X, W13, W2 = _bf16_t(d["x"]), _bf16_t(d["w13"])[0], _bf16_t(d["w2"])[0]
    I = W13.shape[0] // 2
    h = (torch.nn.functional.silu(X @ W13[:I].T) * (X @ W13[I:].T)).float().to(torch.bfloat16).double()
    ref = (h @ W2.T).float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.mean(out == ref) > 0.99
    assert np.allclose(_bits_to_f64(out), _bits_to_f64(ref), rtol=2 ** -7, atol=0)


def test_bf16_forward_skips_and_weights():
    d = _bf16_inputs(seed=3)
    base = oracle.forward(BF16, d["w13"], None, d["w2"], None, d["x"], d["ids"], d["w"])
    # every slot skipped, NaN weights: exact zeros
    ids = np.full_like(d["ids"], -1)
    z = oracle.forward(BF16, d["w13"], None, d["w2"], None, d["x"], ids, np.full_like(d["w"], np.nan))
    assert not np.any(z)
    # all weights doubled: outputs doubled exactly
    two = oracle.forward(BF16, d["w13"], None, d["w2"], None, d["x"], d["ids"], 2 * d["w"])
    assert np.array_equal(_bits_to_f64(two), 2 * _bits_to_f64(base))
    # the gate is the first half of gate_up: swapping the halves changes the result
    sw = np.concatenate([d["w13"][:, 256:], d["w13"][:, :256]], axis=1)
    other = oracle.forward(BF16, sw, None, d["w2"], None, d["x"], d["ids"], d["w"])
    assert not np.array_equal(other, base)

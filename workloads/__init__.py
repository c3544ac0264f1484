"""Seeded synthetic inputs for the MoE experts forward.

This module generates inputs only: hidden states, top-k routing (the experts
forward takes the router's outputs as inputs), router logits (the input of the
router step in front of it) and offline-quantized expert weights.  It holds none of the forward's arithmetic:
weights are quantized with torch's own float8 cast (FP8) or a nearest-grid
lookup (FP4), which stands for the checkpoint's offline quantization.  Both the
HIP path and the CPU oracle receive the same arrays from here.

Shapes and distributions follow the layers the pages name (Mixtral,
Qwen3-MoE, DeepSeek-V3, and the DeepSeek-V4-style FP8 x FP4 Mega MoE layer):
no checkpoint is available, so random weights of those shapes stand in.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np
import torch

FMT_FP8_B128 = 0
FMT_MX = 1
FMT_BF16 = 2


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int          # tokens
    H: int          # hidden size
    I: int          # expert intermediate size
    E: int          # experts on this GPU
    k: int          # slots per token (top-k)
    fmt: int        # FMT_FP8_B128, FMT_MX or FMT_BF16
    routing: str    # "uniform" (softmax top-k of N(0,1) logits) or "zipf"
    zipf_s: float = 0.0
    skip: float = 0.0               # probability that a slot is set to -1
    swiglu_limit: Optional[float] = None
    seed: int = 0

    @property
    def S(self):
        return self.T * self.k


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny", T=64, H=256, I=128, E=8, k=2, fmt=FMT_FP8_B128, routing="uniform", seed=0),
        Workload("mixtral_8x7b", T=4096, H=4096, I=14336, E=8, k=2, fmt=FMT_FP8_B128, routing="uniform",
                 seed=1),
        Workload("qwen3_moe_decode", T=64, H=2048, I=768, E=128, k=8, fmt=FMT_FP8_B128, routing="uniform",
                 seed=2),
        Workload("deepseek_v3", T=8192, H=7168, I=2048, E=256, k=8, fmt=FMT_FP8_B128, routing="zipf",
                 zipf_s=1.1, skip=0.05, seed=3),
        Workload("megamoe_fp8xfp4", T=16384, H=7168, I=2048, E=256, k=8, fmt=FMT_MX, routing="zipf",
                 zipf_s=1.1, skip=0.05, swiglu_limit=7.0, seed=4),
        # the unquantized bf16 experts (the pages' grouped_mm fallback) on the Mixtral-shaped layer
        Workload("mixtral_8x7b_bf16", T=4096, H=4096, I=14336, E=8, k=2, fmt=FMT_BF16, routing="uniform",
                 seed=1),
    ]
}


def _seed(seed: int, tag: str) -> int:
    h = hashlib.sha256(f"{seed}:{tag}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, seed, tag):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, tag))
    return g


def hidden_states(T: int, H: int, seed: int, device="cpu") -> torch.Tensor:
    """bf16 [T, H], entries N(0, 1) rounded to bf16."""
    g = _gen(device, seed, "x")
    return torch.randn((T, H), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def router_logits(T: int, E: int, seed: int, device="cpu", ties: bool = False) -> torch.Tensor:
    """fp32 [T, E] router logits, N(0, 1); with ``ties`` drawn from the eight
    integers -4..3 instead, so that many logits of a token are equal."""
    g = _gen(device, seed, "logits")
    if ties:
        return torch.randint(-4, 4, (T, E), generator=g, device=device).to(torch.float32)
    return torch.randn((T, E), generator=g, device=device, dtype=torch.float32)


def routing(T: int, E: int, k: int, kind: str, seed: int, zipf_s: float = 0.0, skip: float = 0.0,
            device="cpu"):
    """Top-k routing: (ids int32 [T, k], weights fp32 [T, k]).

    uniform: logits N(0,1) over E experts, softmax, top-k, weights renormalised
    to sum 1.  zipf: expert popularity p_r ~ r^-s (r = 1..E) mapped to ids by a
    seeded permutation; k distinct experts per token drawn without replacement
    in proportion to p (Gumbel top-k); weights are the softmax of N(0,1) logits
    over the chosen k.  Then each slot becomes -1 with probability `skip`; its
    weight is kept (routing weights are unmasked).
    """
    g = _gen(device, seed, "route")
    if kind == "uniform":
        logits = torch.randn((T, E), generator=g, device=device, dtype=torch.float32)
        probs = torch.softmax(logits, dim=-1)
        w, ids = torch.topk(probs, k, dim=-1)
        w = w / w.sum(dim=-1, keepdim=True)
    elif kind == "zipf":
        ranks = torch.arange(1, E + 1, device=device, dtype=torch.float64)
        logp = -zipf_s * torch.log(ranks)
        perm = torch.randperm(E, generator=g, device=device)
        logp_by_id = torch.empty_like(logp)
        logp_by_id[perm] = logp
        u = torch.rand((T, E), generator=g, device=device, dtype=torch.float64).clamp_min(1e-300)
        gumbel = -torch.log(-torch.log(u))
        _, ids = torch.topk(logp_by_id[None, :] + gumbel, k, dim=-1)
        lw = torch.randn((T, k), generator=g, device=device, dtype=torch.float32)
        w = torch.softmax(lw, dim=-1)
    else:
        raise ValueError(kind)
    ids = ids.to(torch.int32)
    if skip > 0:
        drop = torch.rand((T, k), generator=g, device=device) < skip
        ids = torch.where(drop, torch.full_like(ids, -1), ids)
    return ids.contiguous(), w.to(torch.float32).contiguous()


def fp8_weights(E: int, N: int, K: int, seed: int, tag: str, device="cpu", std: float = 0.02):
    """Offline-quantized FP8 weights: (codes u8 [E, N, K], scales fp32 [E, N/128, K/128]).

    Each expert's N(0, std) matrix is scaled per 128x128 block by amax/448 and
    cast with torch's float8_e4m3fn conversion (the checkpoint's quantizer).
    """
    g = _gen(device, seed, tag)
    codes = torch.empty((E, N, K), dtype=torch.uint8, device=device)
    scales = torch.empty((E, N // 128, K // 128), dtype=torch.float32, device=device)
    for e in range(E):
        w = torch.randn((N, K), generator=g, device=device, dtype=torch.float32) * std
        blk = w.view(N // 128, 128, K // 128, 128)
        amax = blk.abs().amax(dim=(1, 3)).clamp_min(1e-12)
        s = amax / 448.0
        q = (blk / s[:, None, :, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
        codes[e] = q.view(N, K).view(torch.uint8)
        scales[e] = s
    return codes, scales


_E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def fp4_weights(E: int, N: int, K: int, seed: int, tag: str, device="cpu", std: float = 0.02):
    """Offline-quantized MXFP4 weights: (packed u8 [E, N, K/2], scales u8 [E, N, K/32]).

    Per 1x32 block along K: scale 2^ceil(log2(amax/6)) stored as the byte e+127;
    each value goes to the nearest e2m1 magnitude (sign separate), and two
    nibbles are packed per byte with the even k in the low nibble.
    """
    g = _gen(device, seed, tag)
    grid = torch.tensor(_E2M1_GRID, device=device, dtype=torch.float32)
    mids = (grid[1:] + grid[:-1]) / 2
    packed = torch.empty((E, N, K // 2), dtype=torch.uint8, device=device)
    scales = torch.empty((E, N, K // 32), dtype=torch.uint8, device=device)
    for e in range(E):
        w = torch.randn((N, K), generator=g, device=device, dtype=torch.float32) * std
        blk = w.view(N, K // 32, 32)
        amax = blk.abs().amax(dim=2).clamp_min(1e-30)
        ex = torch.ceil(torch.log2(amax / 6.0)).clamp(-127, 127)
        v = blk / torch.exp2(ex)[:, :, None]
        mag = torch.bucketize(v.abs().clamp(max=6.0), mids)  # index into the grid, 0..7
        nib = (mag | ((v < 0).to(torch.int64) << 3)).to(torch.uint8).view(N, K)
        packed[e] = nib[:, 0::2] | (nib[:, 1::2] << 4)
        scales[e] = (ex + 127).to(torch.uint8)
    return packed, scales


def bf16_weights(E: int, N: int, K: int, seed: int, tag: str, device="cpu", std: float = 0.02):
    """Unquantized bf16 weights [E, N, K]: N(0, std) rounded to bf16."""
    g = _gen(device, seed, tag)
    return (torch.randn((E, N, K), generator=g, device=device, dtype=torch.float32) * std).to(torch.bfloat16)


def expert_weights(wl: Workload, device="cpu"):
    """(w13, w13_scale, w2, w2_scale) in the nt layout: gate_up [E, 2I, H], down [E, H, I].
    The bf16 format has no scales (empty tensors stand in for them)."""
    if wl.fmt == FMT_BF16:
        none = torch.empty(0, dtype=torch.float32, device=device)
        return (bf16_weights(wl.E, 2 * wl.I, wl.H, wl.seed, "w13", device), none,
                bf16_weights(wl.E, wl.H, wl.I, wl.seed, "w2", device), none)
    if wl.fmt == FMT_FP8_B128:
        w13, s13 = fp8_weights(wl.E, 2 * wl.I, wl.H, wl.seed, "w13", device)
        w2, s2 = fp8_weights(wl.E, wl.H, wl.I, wl.seed, "w2", device)
    else:
        w13, s13 = fp4_weights(wl.E, 2 * wl.I, wl.H, wl.seed, "w13", device)
        w2, s2 = fp4_weights(wl.E, wl.H, wl.I, wl.seed, "w2", device)
    return w13, s13, w2, s2


def inputs(wl: Workload, device="cpu"):
    """Everything one forward of the workload needs, as torch tensors on `device`."""
    x = hidden_states(wl.T, wl.H, wl.seed, device)
    ids, w = routing(wl.T, wl.E, wl.k, wl.routing, wl.seed, wl.zipf_s, wl.skip, device)
    w13, s13, w2, s2 = expert_weights(wl, device)
    return dict(x=x, ids=ids, w=w, w13=w13, s13=s13, w2=w2, s2=s2)


def sample_tokens(T: int, n: int, seed: int) -> np.ndarray:
    """A seeded, sorted sample of n distinct token indices (always includes the last token)."""
    rng = np.random.default_rng(_seed(seed, "sample"))
    n = min(n, T)
    pick = rng.choice(T, size=n, replace=False)
    pick[-1] = T - 1 if (T - 1) not in pick else pick[-1]
    return np.sort(np.unique(pick)).astype(np.int32)


def to_numpy(t: torch.Tensor) -> np.ndarray:
    """Host copy; bf16 tensors come back as their uint16 bit patterns."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
        return t.cpu().numpy().view(np.uint16)
    return t.cpu().numpy()

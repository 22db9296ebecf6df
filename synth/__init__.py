"""Seeded synthetic inputs shaped like the pages' DeepSeek-V3 / MoE / MOSS layers.

Shared by the tests, the bench and the smoke check.  This module draws random
numbers and formats them (float32 -> bf16 bit patterns with round-to-nearest-
even, i.e. plain input formatting); it performs none of the method's
arithmetic: no scale rule, no E4M3 encoding, no GEMM.

Every tensor comes from its own torch generator seeded with
``seed * 1000 + stream``; the same call on the same device gives the same
bytes.  CPU and GPU generators give different streams, so a check that needs
the same bytes on both sides generates once and copies.

Recipes (the readings are listed in the design notes):
  linear_tiny   X fp32 [256, 512] N(0,1), 4 channels x50; W fp32 [256, 512]
                N(0, 0.02); dY fp32 [256, 256] N(0, 1e-3).
  linear_dsv3   X bf16 [8192, 7168] N(0,1) with 1% of channels (72) replaced by
                Student-t(3) draws; W bf16 [2048, 7168] N(0, 0.02);
                dY bf16 [8192, 2048] N(0, 1e-3).
  moe           X bf16 [16384, 7168] N(0,1); top-8 of 32 experts by
                Gumbel-top-k on weights (rank)^-1.1; probs = normalised
                weights of the chosen experts; W1 bf16 [32, 4096, 7168],
                W2 bf16 [32, 7168, 2048] N(0, 0.02).
  moe_grad      dO bf16 [16384, 7168] N(0, 1e-3): the gradient of the MoE
                layer's output, for the expert backward.
  wgrad_codes   row-wise E4M3 codes [T, C] drawn directly (sign uniform,
                exponent field 15 - floor(3|z|) clipped at 0, mantissa
                uniform, NaN pattern excluded) with per-1x128-tile scale bytes
                127 + U{-20..4}.
  token_scaled  bf16 [T, C] N(0,1) times 2^u per row, u ~ U{lo..hi} (tokens whose
                magnitudes differ by up to 2^24, the range of the Wgrad workload's
                tile scales).
  moss          W bf16 [8192, 28672] N(0, 0.02) times a per-row factor
                10^U(-2, 1); A bf16 [4096, 8192] N(0, 1).
"""
import numpy as np
import torch


def _gen(seed, stream, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000 + int(stream))
    return g


def normal(shape, std, seed, stream, device="cpu", dtype=torch.float32):
    """N(0, std) draws (std is a standard deviation), cast to dtype (bf16: RNE)."""
    g = _gen(seed, stream, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def student_t3(shape, seed, stream, device="cpu"):
    """Student-t with 3 degrees of freedom: Z / sqrt(chi2_3 / 3), float32."""
    g = _gen(seed, stream, device)
    z = torch.randn(shape, generator=g, device=device)
    c = torch.randn(shape + (3,), generator=g, device=device).pow_(2).sum(-1)
    return z / torch.sqrt(c / 3.0)


def channel_pick(n_channels, n_pick, seed, stream):
    g = _gen(seed, stream, "cpu")
    return torch.randperm(n_channels, generator=g)[:n_pick].sort().values


def linear_tiny(seed=0, device="cpu"):
    """Tiny Linear: X [256,512] fp32 with 4 outlier channels x50, W [256,512], dY [256,256]."""
    X = normal((256, 512), 1.0, seed, 1, device)
    ch = channel_pick(512, 4, seed, 2).to(device)
    X[:, ch] *= 50.0
    W = normal((256, 512), 0.02, seed, 3, device)
    dY = normal((256, 256), 1e-3, seed, 4, device)
    return X, W, dY


def linear_dsv3(seed=0, device="cpu", T=8192, Cin=7168, Cout=2048):
    """DeepSeek-V3-shaped Linear: bf16 X [T,Cin] (1% Student-t channels), W [Cout,Cin], dY [T,Cout]."""
    X = normal((T, Cin), 1.0, seed, 11, device)
    n_heavy = int(round(0.01 * Cin))
    ch = channel_pick(Cin, n_heavy, seed, 12).to(device)
    X[:, ch] = student_t3((T, n_heavy), seed, 13, device)
    X = X.to(torch.bfloat16)
    W = normal((Cout, Cin), 0.02, seed, 14, device, torch.bfloat16)
    dY = normal((T, Cout), 1e-3, seed, 15, device, torch.bfloat16)
    return X, W, dY


def routing(T=16384, E=32, topk=8, s=1.1, seed=0):
    """Top-k routing by Gumbel-top-k on expert weights (rank)^-s.

    Returns topk_idx int32 [T, topk] (slots in descending key order, experts
    distinct within a token) and probs float32 [T, topk] (chosen weights
    normalised per token)."""
    rng = np.random.default_rng([seed, 21])
    w = (np.arange(1, E + 1, dtype=np.float64)) ** (-s)
    keys = np.log(w)[None, :] + rng.gumbel(size=(T, E))
    idx = np.argsort(-keys, axis=1, kind="stable")[:, :topk].astype(np.int32)
    pw = w[idx]
    probs = (pw / pw.sum(axis=1, keepdims=True)).astype(np.float32)
    return idx, probs


def moe(seed=0, device="cpu", T=16384, H=7168, F=2048, E=32, topk=8, weights=True):
    """MoE expert-MLP inputs: X bf16 [T,H], topk_idx, probs, W1 [E,2F,H], W2 [E,H,F] (bf16)."""
    X = normal((T, H), 1.0, seed, 31, device, torch.bfloat16)
    idx, probs = routing(T, E, topk, 1.1, seed)
    W1 = W2 = None
    if weights:
        W1 = normal((E, 2 * F, H), 0.02, seed, 32, device, torch.bfloat16)
        W2 = normal((E, H, F), 0.02, seed, 33, device, torch.bfloat16)
    return X, idx, probs, W1, W2


def moe_grad(seed=0, device="cpu", T=16384, H=7168):
    """Gradient of the MoE layer output: dO bf16 [T, H] N(0, 1e-3)."""
    return normal((T, H), 1e-3, seed, 34, device, torch.bfloat16)


def wgrad_codes(T, C, seed=0, stream=41, device="cpu"):
    """Row-wise E4M3 codes [T, C] (uint8) and 1x128 scale bytes [T, C/128] drawn directly."""
    g = _gen(seed, stream, device)
    z = torch.randn((T, C), generator=g, device=device).abs_()
    E = (15 - torch.floor(z * 3.0)).clamp_(min=0).to(torch.int32)
    m = torch.randint(0, 8, (T, C), generator=g, device=device, dtype=torch.int32)
    m = torch.where((E == 15) & (m == 7), torch.full_like(m, 6), m)
    sign = torch.randint(0, 2, (T, C), generator=g, device=device, dtype=torch.int32)
    q = ((sign << 7) | (E << 3) | m).to(torch.uint8)
    s = (torch.randint(-20, 5, (T, C // 128), generator=g, device=device, dtype=torch.int32)
         + 127).to(torch.uint8)
    return q, s


def token_scaled(T, C, lo=-20, hi=4, seed=0, stream=51, device="cpu"):
    """bf16 [T, C]: N(0, 1) rows, row t times 2^u_t with u_t ~ U{lo..hi}."""
    g = _gen(seed, stream, device)
    x = torch.randn((T, C), generator=g, device=device)
    u = torch.randint(lo, hi + 1, (T, 1), generator=g, device=device).float()
    return (x * torch.exp2(u)).to(torch.bfloat16)


def moss(seed=0, device="cpu", R=8192, C=28672, M=4096):
    """MOSS inputs: W bf16 [R, C] = N(0,0.02) * 10^U(-2,1) per row; A bf16 [M, R] N(0,1)."""
    W = normal((R, C), 0.02, seed, 51, device)
    g = _gen(seed, 52, device)
    f = torch.pow(10.0, torch.rand((R, 1), generator=g, device=device) * 3.0 - 2.0)
    W = (W * f).to(torch.bfloat16)
    A = normal((M, R), 1.0, seed, 53, device, torch.bfloat16)
    return W, A


def bf16_bits(t):
    """bf16 tensor -> numpy uint16 bit patterns (CPU copy)."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)

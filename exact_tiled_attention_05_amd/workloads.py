"""Seeded synthetic workloads for the attention forward pass.

This module only draws random numbers and shapes them; it holds none of the attention
arithmetic, so both the GPU path's tests/bench and the CPU oracle can take their inputs from it.

Recipe (shared by every workload):
  * a CPU ``torch.Generator`` seeded with the workload's seed;
  * Q, then K, then V drawn in that order as float32 standard normals of shape [B, H, N, d];
  * workload-specific shaping (below), applied in float32;
  * a cast to the compute dtype (bf16 or fp32). The cast tensors are what the GPU receives, and
    the oracle upcasts exactly those tensors to float64.

The five workloads are the shapes the pages discuss: a single small head, a mid-size batch at
d = 64, the Llama-3-8B layer shape (32 heads at N = 8192, d = 128, causal) that the
"FlashAttention-2 -- Deeper Math" page uses for its occupancy argument (Fix 4) and that
"Flash Attention" ("The problem, quantified") uses for its traffic count, a large-score stress
case, and a 32K-token causal case. A sixth gives that Llama layer its grouped K/V heads (32 query
heads over 8 K/V heads, "Understanding FlashAttention Pt 1", §4.1) in the tokens-outermost
[B][N][heads][d] layout of that section; K and V are then drawn with H_kv heads. A seventh is that
layer decoding: one new query token per sequence (Nq = 1) against N = 32768 cached keys, for a
batch of 8 sequences ("FlashAttention-2 -- Deeper Math", "What FA-2 does not fix"); Q is then drawn
with Nq rows. The two "_bwd" workloads are the Llama layer (with and without grouped K/V heads)
run backward ("Understanding FlashAttention Pt 1", §3.6): the same Q, K, V recipe and seeds as the
forward workloads, plus an upstream gradient dO drawn like Q from its own seed. Four more exercise
the score variants and the largest head dim ("Understanding FlashAttention Pt 1", §0.2, §3.5, §4.2;
"Flash Attention": head dims up to 256): a d = 256 layer (16 heads, N = 8192, causal); the
grouped Llama layer with a causal sliding window of 4096 keys (each query sees itself and the 4095
keys before it); the Llama layer with ALiBi slopes 2^(-8 (h + 1) / H); and a non-causal layer with
an additive bf16 bias of its own seed, N(0, 1), one [N, N] matrix per head.
"""
import math

import torch

# name -> shape and recipe. "causal" lists the mask settings the workload is run with.
WORKLOADS = {
    "single_head_fp32": dict(B=1, H=1, N=256, d=64, dtype="fp32", causal=(False, True), seed=0),
    "b4h16_n1k_d64": dict(B=4, H=16, N=1024, d=64, dtype="bf16", causal=(False,), seed=1),
    "llama3_8b_n8k_causal": dict(B=1, H=32, N=8192, d=128, dtype="bf16", causal=(True,), seed=2),
    "outlier_b16h32_n2k": dict(B=16, H=32, N=2048, d=128, dtype="bf16", causal=(False,), seed=3,
                               q_mult=8.0, outlier_frac=0.01, outlier_mult=4.0),
    "long_n32k_causal": dict(B=1, H=32, N=32768, d=128, dtype="bf16", causal=(True,), seed=4,
                             sample_rows=64),
    "llama3_8b_gqa_n8k_causal": dict(B=1, H=32, H_kv=8, N=8192, d=128, dtype="bf16",
                                     causal=(True,), seed=5, layout="bnhd", sample_rows=64),
    "llama3_8b_gqa_decode_b8_n32k": dict(B=8, H=32, H_kv=8, Nq=1, N=32768, d=128, dtype="bf16",
                                         causal=(True,), seed=6, layout="bnhd"),
    "d256_h16_n8k_causal": dict(B=1, H=16, N=8192, d=256, dtype="bf16", causal=(True,), seed=7,
                                sample_rows=64),
    "llama3_8b_gqa_n8k_swa4k": dict(B=1, H=32, H_kv=8, N=8192, d=128, dtype="bf16", causal=(True,),
                                    seed=5, layout="bnhd", window=(4095, -1), sample_rows=64),
    "llama3_8b_n8k_causal_alibi": dict(B=1, H=32, N=8192, d=128, dtype="bf16", causal=(True,),
                                       seed=2, alibi=True, sample_rows=64),
    "b1h16_n4k_bias": dict(B=1, H=16, N=4096, d=128, dtype="bf16", causal=(False,), seed=8,
                           bias_seed=18, sample_rows=64),
    "llama3_8b_n8k_causal_bwd": dict(B=1, H=32, N=8192, d=128, dtype="bf16", causal=(True,),
                                     seed=2, grad_seed=12, backward=True),
    "llama3_8b_gqa_n8k_causal_bwd": dict(B=1, H=32, H_kv=8, N=8192, d=128, dtype="bf16",
                                         causal=(True,), seed=5, grad_seed=15, layout="bnhd",
                                         backward=True),
}

_TORCH_DTYPE = {"bf16": torch.bfloat16, "fp32": torch.float32}


def softmax_scale(d):
    """The conventional 1/sqrt(d), rounded once to float32 (the value both sides use)."""
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))


def outlier_rows(N, count, seed):
    """Indices of the key rows to enlarge in the large-score stress workload.

    ``count`` distinct rows drawn with a seeded permutation; the last key (N-1) is always one of
    them, so a late-arriving maximum is guaranteed whatever the key tile size, and at least one
    more lands in the last tenth of the keys.
    """
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(N, generator=g)
    chosen = [int(x) for x in perm[: max(count, 2)]]
    if N - 1 not in chosen:
        chosen[0] = N - 1
    tail0 = N - max(1, N // 10)
    if not any(tail0 <= c < N - 1 for c in chosen) and N >= 3:
        chosen[1] = tail0 if tail0 != N - 1 else N - 2
    return sorted(set(chosen))


def make_inputs(B, H, N, d, dtype="bf16", seed=0, q_mult=1.0, outlier_frac=0.0,
                outlier_mult=4.0, H_kv=None, Nq=None, **_ignored):
    """Return (q, k, v) CPU tensors in the compute dtype: q [B, H, Nq, d], k and v
    [B, H_kv, N, d] (H_kv defaults to H, Nq to N)."""
    H_kv = H if H_kv is None else H_kv
    Nq = N if Nq is None else Nq
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, H, Nq, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, H_kv, N, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, H_kv, N, d), generator=g, dtype=torch.float32)
    if q_mult != 1.0:
        q.mul_(q_mult)
    if outlier_frac > 0.0:
        count = max(1, int(math.floor(outlier_frac * N)))
        for b in range(B):
            for h in range(H_kv):
                idx = outlier_rows(N, count, seed * 1000003 + b * 4099 + h)
                k[b, h, idx] *= outlier_mult
    t = _TORCH_DTYPE[dtype]
    return q.to(t).contiguous(), k.to(t).contiguous(), v.to(t).contiguous()


def to_layout(x, layout):
    """A [B, heads, N, d] tensor as a contiguous tensor in the given layout ("bhnd" or "bnhd")."""
    if layout == "bhnd":
        return x.contiguous()
    if layout == "bnhd":
        return x.permute(0, 2, 1, 3).contiguous()
    raise ValueError("layout must be 'bhnd' or 'bnhd'")


def sampled_rows(N, count, seed):
    """Query rows checked against the oracle when the full output is too large to check.

    Always includes the first and the last row; the rest are distinct rows drawn uniformly
    with a seeded permutation. Returned sorted.
    """
    if count >= N:
        return torch.arange(N)
    g = torch.Generator().manual_seed(seed)
    rest = torch.randperm(N - 2, generator=g)[: count - 2] + 1
    return torch.sort(torch.cat([torch.tensor([0, N - 1]), rest])).values


def workload_inputs(name):
    """(q, k, v, scale) for a named workload."""
    w = WORKLOADS[name]
    q, k, v = make_inputs(**w)
    return q, k, v, softmax_scale(w["d"])


def alibi_slopes(H):
    """The geometric ALiBi slopes 2^(-8 (h + 1) / H), h = 0 .. H-1, as float32 values."""
    return torch.tensor([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=torch.float32)


def workload_bias(name):
    """The additive bias [1, H, N, N] (bf16, N(0, 1)) of a bias workload."""
    w = WORKLOADS[name]
    g = torch.Generator().manual_seed(w["bias_seed"])
    return torch.randn((1, w["H"], w["N"], w["N"]), generator=g).to(torch.bfloat16)


def visible_pairs(N, causal, window=None):
    """Number of (query, key) pairs a row-wise mask leaves visible in one [N, N] head: query i sees
    keys max(0, i - left) .. min(N - 1, i + right), capped at i when causal."""
    i = torch.arange(N, dtype=torch.int64)
    lo = torch.zeros_like(i)
    hi = torch.full_like(i, N - 1)
    if window is not None:
        if window[0] >= 0:
            lo = torch.clamp(i - window[0], min=0)
        if window[1] >= 0:
            hi = torch.clamp(i + window[1], max=N - 1)
    if causal:
        hi = torch.minimum(hi, i)
    return int((hi - lo + 1).clamp(min=0).sum())


def metric_flops_masked(B, H, N, d, causal, window=None):
    """4*d FLOPs per visible (query, key) pair: the two products restricted to what the mask
    keeps. Equals metric_flops up to the diagonal's N/2 pairs when there is no window."""
    return 4.0 * B * H * d * visible_pairs(N, causal, window)


def workload_grad(name):
    """The upstream gradient dO [B, H, N, d] of a backward workload (drawn like Q)."""
    w = WORKLOADS[name]
    return make_inputs(w["B"], w["H"], w["N"], w["d"], dtype=w["dtype"], seed=w["grad_seed"])[0]


def metric_flops(B, H, N, d, causal):
    """The throughput metric's FLOP count: 4*B*H*N^2*d, halved when causal."""
    f = 4.0 * B * H * N * N * d
    return f / 2.0 if causal else f


def metric_flops_bwd(B, H, N, d, causal):
    """FLOP count of the backward pass: the five N x N x d products of the gradient formulas
    (S = QK^T, dP = dO V^T, dV = P^T dO, dQ = dS K, dK = dS^T Q), 10*B*H*N^2*d, halved when
    causal -- 2.5 times the forward's."""
    f = 10.0 * B * H * N * N * d
    return f / 2.0 if causal else f

"""GPU parity of the backward pass (fa_bwd) against the CPU oracle's attention_backward.

End to end: the GPU forward produces O and the logsumexp, the GPU backward turns a seeded dO into
dQ, dK, dV, and the float64 oracle computes the gradients of the same bf16 inputs from the
definition ("Understanding FlashAttention Pt 1", §3.6).

Bound (elementwise, derived from the kernel's arithmetic, unit roundoff u = 2^-8 of bf16): the only
reduced-precision steps are P and dS rounded to bf16 as matrix-core operands (relative u each),
the outputs rounded to bf16 (relative u), and D = rowsum(dO * O) taken from the forward's bf16 O,
whose error is within 2u (P|V|) (its own P rounding and output rounding); everything else is fp32.
Hence
    |dV err| <= u (P^T |dO|) + u |dV|
    |dK err| <= scale sum_i (u |dS_ij| + 3u P_ij w_i) |Q_i| + u |dK|,   w_i = sum_r |dO_ir| (P|V|)_ir
    |dQ err| <= scale sum_j (u |dS_ij| + 3u P_ij w_i) |K_j| + u |dQ|
(summed over the query heads of a K/V head for dK, dV). The test allows twice that, for the fp32
sums and the logsumexp's own rounding. Being worst-case, that bound is loose (a correct kernel
uses a few percent of it), so each gradient tensor must also have a relative Frobenius error of
at most 4u: its elements are sums of terms that each carry at most one bf16 rounding, plus the
output rounding, and with the random-sign data here those add like a random walk -- a CPU
emulation of exactly these rounding steps gives 0.6u -- while one element off by 5% of the
tensor's largest entry already exceeds 4u at these sizes.
"""
import itertools

import numpy as np
import pytest
import torch

import exact_tiled_attention_05_amd as fa
from exact_tiled_attention_05_amd.workloads import make_inputs, softmax_scale, to_layout
from oracle import attention_backward_head, attention_head, kv_head_of

from gpu_util import log

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
U = 2.0 ** -8


def _as64(t):
    return t.float().numpy().astype(np.float64)


def gpu_fwd_bwd(q, k, v, do, scale, causal, layout="bhnd", workspace=None):
    """[B, H, N, d] / [B, H_kv, N, d] CPU bf16 -> (dq, dk, dv) float64 in [B, heads, N, d] order,
    via the GPU forward (o, lse) and the GPU backward in ``layout``."""
    qd, kd, vd, dod = (to_layout(x, layout).to(DEV) for x in (q, k, v, do))
    o, lse = fa.forward(qd, kd, vd, scale=scale, causal=causal, layout=layout)
    dq, dk, dv = fa.backward(qd, kd, vd, o, lse, dod, scale=scale, causal=causal, layout=layout,
                             workspace=workspace)
    torch.cuda.synchronize()
    out = []
    for t in (dq, dk, dv):
        if layout == "bnhd":
            t = t.permute(0, 2, 1, 3)
        out.append(t.float().cpu().numpy().astype(np.float64))
    return out


def reference(q, k, v, do, scale, causal, heads=None):
    """Oracle gradients and the elementwise bounds above for query heads ``heads`` (default all)
    and the K/V heads they use (dK, dV summed over those query heads only)."""
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    heads = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    ref = {"dq": {}, "dk": {}, "dv": {}}
    bnd = {"dq": {}, "dk": {}, "dv": {}}
    for (b, h) in heads:
        j = kv_head_of(h, H, H_kv)
        qh, kh, vh, doh = _as64(q[b, h]), _as64(k[b, j]), _as64(v[b, j]), _as64(do[b, h])
        gq, gk, gv = attention_backward_head(qh, kh, vh, doh, scale, causal)
        _, _, _, p = attention_head(qh, kh, vh, scale, causal, return_sp=True)
        dp = doh @ vh.T
        ds = p * (dp - (p * dp).sum(axis=1)[:, None])
        w = (np.abs(doh) * (p @ np.abs(vh))).sum(axis=1)
        coef = U * np.abs(ds) + 3 * U * p * w[:, None]
        ref["dq"][(b, h)] = gq
        bnd["dq"][(b, h)] = scale * (coef @ np.abs(kh)) + U * np.abs(gq)
        for name, g, bb in (("dk", gk, scale * (coef.T @ np.abs(qh))),
                            ("dv", gv, U * (p.T @ np.abs(doh)))):
            ref[name][(b, j)] = ref[name].get((b, j), 0.0) + g
            bnd[name][(b, j)] = bnd[name].get((b, j), 0.0) + bb
    for name in ("dk", "dv"):
        for key in bnd[name]:
            bnd[name][key] = bnd[name][key] + U * np.abs(ref[name][key])
    return ref, bnd


def check(got, ref, bnd, tag):
    """got: (dq, dk, dv) arrays; ref/bnd from reference()."""
    for name, g in zip(("dq", "dk", "dv"), got):
        num = den = 0.0
        count = 0
        worst = 0.0
        for key, r in ref[name].items():
            e = np.abs(g[key] - r)
            worst = max(worst, float((e / (2 * bnd[name][key] + 1e-6)).max()))
            num += float((e ** 2).sum())
            den += float((r ** 2).sum())
            count += r.size
        rel = (num / max(den, 1e-300)) ** 0.5
        log("  %s %s: rel Frobenius error %.3g, worst |err| / allowed %.3g" % (tag, name, rel, worst))
        assert np.isfinite(g).all(), name
        assert worst <= 1.0, (name, worst)
        # (the absolute floor only matters where the exact gradient is 0, e.g. dQ with one key)
        assert num ** 0.5 <= 4 * U * den ** 0.5 + 1e-6 * count ** 0.5, (name, rel)


def _cases():
    shapes = [(1, 2, 2), (17, 4, 2), (64, 4, 1), (100, 2, 2), (130, 4, 2), (257, 4, 1), (200, 8, 8),
              (64, 2, 2), (129, 6, 3)]
    cyc = itertools.cycle(itertools.product((128, 64), ("bhnd", "bnhd")))
    out = []
    for (N, H, H_kv) in shapes:
        for causal in (False, True):
            d, layout = next(cyc)
            out.append((N, H, H_kv, d, causal, layout))
    return out


@pytest.mark.parametrize("N,H,H_kv,d,causal,layout", _cases())
def test_backward_ragged_shapes(N, H, H_kv, d, causal, layout):
    log("bwd case N=%d H=%d H_kv=%d d=%d causal=%s layout=%s" % (N, H, H_kv, d, causal, layout))
    q, k, v = make_inputs(2, H, N, d, H_kv=H_kv, seed=N * 7 + H)
    do = make_inputs(2, H, N, d, seed=N * 7 + H + 1)[0]
    scale = softmax_scale(d)
    got = gpu_fwd_bwd(q, k, v, do, scale, causal, layout)
    ref, bnd = reference(q, k, v, do, scale, causal)
    check(got, ref, bnd, "N=%d" % N)


@pytest.mark.parametrize("N,H,H_kv,causal,layout", [(513, 2, 2, False, "bhnd"),
                                                   (1000, 4, 2, True, "bnhd"),
                                                   (777, 4, 1, True, "bnhd"),
                                                   (1300, 2, 2, True, "bhnd")])
def test_backward_several_key_blocks(N, H, H_kv, causal, layout):
    # d = 128 over several 256-key blocks of the dK/dV kernel (one wave per 64 keys): ragged last
    # blocks, waves whose keys all lie past N, grouped heads split over workgroups, both layouts.
    log("bwd several key blocks N=%d H=%d H_kv=%d causal=%s %s" % (N, H, H_kv, causal, layout))
    q, k, v = make_inputs(1, H, N, 128, H_kv=H_kv, seed=N + 5)
    do = make_inputs(1, H, N, 128, seed=N + 6)[0]
    scale = softmax_scale(128)
    got = gpu_fwd_bwd(q, k, v, do, scale, causal, layout)
    ref, bnd = reference(q, k, v, do, scale, causal)
    check(got, ref, bnd, "N=%d" % N)


def test_backward_large_scores():
    # Scaled-up queries and enlarged keys: P is nearly one-hot in many rows.
    q, k, v = make_inputs(1, 4, 1024, 128, seed=31, q_mult=8.0, outlier_frac=0.01, outlier_mult=4.0)
    do = make_inputs(1, 4, 1024, 128, seed=32)[0]
    for causal in (False, True):
        got = gpu_fwd_bwd(q, k, v, do, softmax_scale(128), causal)
        ref, bnd = reference(q, k, v, do, softmax_scale(128), causal)
        check(got, ref, bnd, "outliers causal=%s" % causal)


def test_backward_llama_layer_full_size():
    # B=1, H=32, N=8192, d=128, causal: the whole layer runs; two heads are checked densely.
    q, k, v = make_inputs(1, 32, 8192, 128, seed=2)
    do = make_inputs(1, 32, 8192, 128, seed=12)[0]
    scale = softmax_scale(128)
    got = gpu_fwd_bwd(q, k, v, do, scale, True)
    for g in got:
        assert np.isfinite(g).all()
    heads = [(0, 0), (0, 31)]
    ref, bnd = reference(q, k, v, do, scale, True, heads)
    check(got, ref, bnd, "llama N=8192")


def test_backward_grouped_llama_full_size():
    # 32 query heads over 8 K/V heads, [B][N][H][d]: K/V head 3 and its 4 query heads densely.
    q, k, v = make_inputs(1, 32, 8192, 128, H_kv=8, seed=5)
    do = make_inputs(1, 32, 8192, 128, seed=15)[0]
    scale = softmax_scale(128)
    got = gpu_fwd_bwd(q, k, v, do, scale, True, "bnhd")
    heads = [(0, h) for h in range(12, 16)]
    ref, bnd = reference(q, k, v, do, scale, True, heads)
    check(got, ref, bnd, "gqa N=8192")


def test_backward_scale_zero():
    # Uniform weights over the visible keys: dQ = dK = 0 and dV_j = sum_{i >= j} dO_i / (i + 1).
    q, k, v = make_inputs(1, 2, 300, 64, seed=9)
    do = make_inputs(1, 2, 300, 64, seed=10)[0]
    dq, dk, dv = gpu_fwd_bwd(q, k, v, do, 0.0, True)
    assert np.all(dq == 0.0) and np.all(dk == 0.0)
    dd = _as64(do)
    ref = np.flip(np.cumsum(np.flip(dd / np.arange(1, 301)[None, None, :, None], axis=2), axis=2), axis=2)
    assert np.abs(dv - ref).max() <= 2 * U * np.abs(ref).max() + 1e-3


def test_backward_deterministic_and_workspace_reuse():
    q, k, v = make_inputs(2, 8, 1000, 128, H_kv=2, seed=21)
    do = make_inputs(2, 8, 1000, 128, seed=22)[0]
    ws = torch.empty(fa.fa_bwd_workspace_bytes(2, 8, 2, 1000, 128), dtype=torch.uint8, device=DEV)
    a = gpu_fwd_bwd(q, k, v, do, 0.1, True, "bnhd", workspace=ws)
    small = make_inputs(1, 2, 77, 64, seed=23)
    gpu_fwd_bwd(*small, make_inputs(1, 2, 77, 64, seed=24)[0], 0.1, False, workspace=ws)
    b = gpu_fwd_bwd(q, k, v, do, 0.1, True, "bnhd", workspace=ws)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_backward_over_2g_elements_per_tensor():
    # B=520, 32 query heads over 8 K/V heads, N=1024, d=128, causal, [B][N][H][d]: 2.2e9 elements
    # per Q-sized tensor, so batch offsets need 64-bit arithmetic in every kernel. Inputs are drawn
    # on the GPU; three batches are checked densely (every query head of one K/V group each).
    B, H, H_kv, N, d = 520, 32, 8, 1024, 128
    dev = DEV
    log("bwd over 2^31 elements: B=%d H=%d H_kv=%d N=%d d=%d bnhd" % (B, H, H_kv, N, d))
    g = torch.Generator(device=dev).manual_seed(993)
    mk = lambda h: torch.randn((B, N, h, d), generator=g, device=dev).to(torch.bfloat16)
    q, k, v, do = mk(H), mk(H_kv), mk(H_kv), mk(H)
    assert q.numel() > 2 ** 31
    scale = softmax_scale(d)
    o, lse = fa.forward(q, k, v, scale=scale, causal=True, layout="bnhd")
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, scale=scale, causal=True, layout="bnhd")
    torch.cuda.synchronize()
    for b, j in [(0, 0), (B - 1, H_kv - 1), (263, 5)]:
        cpu = lambda t: t[b:b + 1].permute(0, 2, 1, 3).contiguous().cpu()
        qs, ks, vs, dos = cpu(q), cpu(k), cpu(v), cpu(do)
        heads = [(0, h) for h in range(H) if kv_head_of(h, H, H_kv) == j]
        ref, bnd = reference(qs, ks, vs, dos, scale, True, heads)
        got = [cpu(t).float().numpy().astype(np.float64) for t in (dq, dk, dv)]
        check(got, ref, bnd, "b=%d kv head %d" % (b, j))
    del q, k, v, do, o, lse, dq, dk, dv
    torch.cuda.empty_cache()

"""GPU parity of the score variants and d = 256 (fa_fwd_ext; fa_fwd / fa_fwd_gqa at d = 256)
against the CPU oracle's attention_ext.

Sliding windows of several shapes (one key, left-only, right-only, two-sided, wider than N), ALiBi
slopes, additive bf16 bias (shared over batch or over heads, random values, a -inf mask, a row
with every key masked), their combinations, head dims 64/128/256, grouped heads, both layouts and
ragged lengths; the Llama layer with a 1024-key causal window and a d = 256 layer at N = 8192 on
sampled rows. Bounds as for the forward: |O - O_ref| <= 2e-2, |LSE - LSE_ref| <= 1e-3.
"""
import itertools

import numpy as np
import pytest
import torch

import exact_tiled_attention_05_amd as fa
from exact_tiled_attention_05_amd.workloads import make_inputs, sampled_rows, softmax_scale, to_layout
from oracle import attention_ext

from gpu_util import TOL_LSE, TOL_O_BF16, log

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _as64(t):
    return t.float().numpy().astype(np.float64)


def alibi(H):
    """The geometric slopes 2^(-8 (h + 1) / H) (any positive slopes would do for parity)."""
    return np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=np.float32)


def gpu_ext(q, k, v, scale, causal, layout="bhnd", window=(-1, -1), slopes=None, bias=None):
    qd, kd, vd = (to_layout(x, layout).to(DEV) for x in (q, k, v))
    sl = None if slopes is None else torch.tensor(slopes, device=DEV)
    bi = None
    if bias is not None:  # rows padded to a multiple of 8 elements on the device (the contract)
        n = bias.shape[-1]
        pad = torch.zeros(tuple(bias.shape[:-1]) + ((n + 7) // 8 * 8,), dtype=torch.bfloat16,
                          device=DEV)
        pad[..., :n] = bias.to(DEV)
        bi = pad[..., :n]
    o, lse = fa.forward_ext(qd, kd, vd, scale=scale, causal=causal, layout=layout, window=window,
                            alibi_slopes=sl, bias=bi)
    torch.cuda.synchronize()
    if layout == "bnhd":
        o = o.permute(0, 2, 1, 3)
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check(q, k, v, scale, causal, layout="bhnd", window=(-1, -1), slopes=None, bias=None,
          rows=None, tag=""):
    log("ext case %s: q %s k %s causal=%s layout=%s window=%s alibi=%s bias=%s" % (
        tag, tuple(q.shape), tuple(k.shape), causal, layout, window, slopes is not None,
        None if bias is None else tuple(bias.shape)))
    o, lse = gpu_ext(q, k, v, scale, causal, layout, window, slopes, bias)
    win = None if window == (-1, -1) else window
    ro, rl = attention_ext(_as64(q), _as64(k), _as64(v), scale, causal, win,
                           None if slopes is None else [float(x) for x in slopes],
                           None if bias is None else _as64(bias), rows)
    if rows is not None:
        o, lse = o[:, :, rows], lse[:, :, rows]
    eo = float(np.abs(o - ro).max())
    el = float(np.abs(lse - rl).max())
    log("  max|dO| %.3g  max|dLSE| %.3g" % (eo, el))
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    assert eo <= TOL_O_BF16, eo
    assert el <= TOL_LSE, el


_WINDOWS = [(0, 0), (16, -1), (100, 50), (-1, 0), (5, 5), (300, 300), (-1, 31), (63, 0)]


def _window_cases():
    shapes = [(77, 4, 2), (300, 2, 2), (1000, 4, 1), (129, 8, 8)]
    cyc = itertools.cycle(itertools.product((128, 64, 256), ("bhnd", "bnhd")))
    out = []
    for (N, H, H_kv), w in itertools.product(shapes, _WINDOWS):
        for causal in (False, True):
            if (N + w[0] + causal) % 3:  # a deterministic third of the combinations
                continue
            d, layout = next(cyc)
            out.append((N, H, H_kv, d, causal, layout, w))
    return out


@pytest.mark.parametrize("N,H,H_kv,d,causal,layout,window", _window_cases())
def test_sliding_window(N, H, H_kv, d, causal, layout, window):
    q, k, v = make_inputs(2, H, N, d, H_kv=H_kv, seed=N + 3 * d + window[0])
    check(q, k, v, softmax_scale(d), causal, layout, window, tag="window")


@pytest.mark.parametrize("N,d,causal,window", [(300, 128, True, (-1, -1)), (500, 64, False, (-1, -1)),
                                               (1000, 128, True, (256, -1)), (257, 256, False, (40, 40)),
                                               (333, 64, True, (-1, -1)), (700, 256, True, (100, -1)),
                                               (129, 128, True, (0, 0))])
def test_alibi(N, d, causal, window):
    H = 8
    q, k, v = make_inputs(2, H, N, d, H_kv=4, seed=N + d)
    check(q, k, v, softmax_scale(d), causal, "bnhd", window, alibi(H), tag="alibi")


@pytest.mark.parametrize("B,N,H,H_kv,layout,window", [
    (1, 4096, 4, 4, "bhnd", (4095, -1)), (2, 4097, 4, 2, "bnhd", (1000, 7)),
    (1, 5000, 2, 1, "bnhd", (63, -1)), (1, 4160, 2, 2, "bhnd", (0, -1)),
    (1, 4500, 2, 2, "bnhd", (300, 0)), (1, 4096, 2, 2, "bhnd", (10000, -1))])
def test_window_long_causal(B, N, H, H_kv, layout, window):
    """A causal sliding window at d = 128 and N >= 4096 (on the wide-row kernel): windows of one
    key, of less and more than a workgroup's rows, and wider than N, with and without a right bound
    (which the causal rule makes moot); ragged lengths, grouped heads, both layouts; sampled rows
    plus the first and last 70 rows."""
    q, k, v = make_inputs(B, H, N, 128, H_kv=H_kv, seed=N + window[0])
    rows = np.unique(np.concatenate([sampled_rows(N, 96, seed=N + 1).numpy(),
                                     np.arange(0, 70), np.arange(N - 70, N)]))
    check(q, k, v, softmax_scale(128), True, layout, window, rows=rows, tag="window long causal")


@pytest.mark.parametrize("B,N,H,H_kv,layout,slope_mult,scale_mult", [
    (1, 4096, 4, 4, "bhnd", 1.0, 1.0), (2, 4097, 4, 2, "bnhd", 1.0, 1.0),
    (1, 5000, 2, 1, "bnhd", 64.0, 1.0), (1, 4160, 2, 2, "bhnd", 0.25, 0.05),
    (1, 8192, 4, 1, "bnhd", 1.0, 1.0), (1, 4096, 2, 1, "bhnd", 1.0, 1e-5),
    (1, 32768, 2, 2, "bhnd", 1.0, 1.0)])
def test_alibi_long_causal(B, N, H, H_kv, layout, slope_mult, scale_mult):
    """Causal ALiBi at d = 128 and N >= 4096 (on the wide-row kernel, walking the keys from the
    diagonal down): ragged lengths, grouped heads, both layouts, slopes up to 64x the geometric
    ones (a strongly local softmax), a small scale, a scale below 1e-6 (left to the 4-wave
    kernel) and N = 32768 (rows far from key 0, where the ALiBi term is large), on sampled rows
    plus the first and last 70 rows."""
    q, k, v = make_inputs(B, H, N, 128, H_kv=H_kv, seed=N + H)
    rows = np.unique(np.concatenate([sampled_rows(N, 96, seed=N).numpy(),
                                     np.arange(0, 70), np.arange(N - 70, N)]))
    slopes = (alibi(H) * np.float32(slope_mult)).astype(np.float32)
    check(q, k, v, softmax_scale(128) * scale_mult, True, layout, (-1, -1), slopes, rows=rows,
          tag="alibi long causal")


def _bias(shape, seed, kind):
    g = torch.Generator().manual_seed(seed)
    b = torch.randn(shape, generator=g)
    if kind == "mask":  # about 30% of the entries -inf, the diagonal always kept
        drop = torch.rand(shape, generator=g) < 0.3
        eye = torch.eye(shape[-1], dtype=torch.bool).expand(shape)
        b = torch.where(drop & ~eye, torch.full_like(b, float("-inf")), torch.zeros_like(b))
    return b.to(torch.bfloat16)


@pytest.mark.parametrize("N,d,causal,bshape,kind", [
    (300, 128, False, "1H", "randn"), (300, 128, True, "B1", "randn"), (77, 64, False, "BH", "mask"),
    (513, 128, True, "1H", "mask"), (200, 256, False, "B1", "randn")])
def test_bias(N, d, causal, bshape, kind):
    B, H = 2, 4
    shape = (B if bshape[0] == "B" else 1, H if bshape[1] == "H" else 1, N, N)
    q, k, v = make_inputs(B, H, N, d, seed=N + d + 7)
    check(q, k, v, softmax_scale(d), causal, "bhnd", (-1, -1), None, _bias(shape, N, kind),
          tag="bias")


def test_everything_together():
    B, H, N, d = 2, 8, 700, 128
    q, k, v = make_inputs(B, H, N, d, H_kv=2, seed=71)
    check(q, k, v, softmax_scale(d), True, "bnhd", (200, -1), alibi(H), _bias((1, H, N, N), 72, "randn"),
          tag="window+alibi+bias")


def test_fully_masked_row_gives_zero_and_minus_inf():
    B, H, N, d = 1, 2, 100, 64
    q, k, v = make_inputs(B, H, N, d, seed=73)
    bias = torch.zeros((1, 1, N, N), dtype=torch.bfloat16)
    bias[0, 0, 17, :] = float("-inf")
    o, lse = gpu_ext(q, k, v, 0.125, False, bias=bias)
    assert np.all(o[:, :, 17] == 0.0) and np.all(lse[:, :, 17] == -np.inf)
    rows = np.array([r for r in range(N) if r != 17])
    ro, rl = attention_ext(_as64(q), _as64(k), _as64(v), 0.125, False, None, None, _as64(bias), rows)
    assert np.abs(o[:, :, rows] - ro).max() <= TOL_O_BF16
    assert np.abs(lse[:, :, rows] - rl).max() <= TOL_LSE


@pytest.mark.parametrize("N,causal,layout,H_kv", [(1000, True, "bhnd", 8), (333, False, "bnhd", 2),
                                                  (64, True, "bnhd", 1)])
def test_head_dim_256_through_forward(N, causal, layout, H_kv):
    B, H, d = 2, 8, 256
    q, k, v = make_inputs(B, H, N, d, H_kv=H_kv, seed=N + 11)
    qd, kd, vd = (to_layout(x, layout).to(DEV) for x in (q, k, v))
    o, lse = fa.forward(qd, kd, vd, causal=causal, layout=layout)
    torch.cuda.synchronize()
    if layout == "bnhd":
        o = o.permute(0, 2, 1, 3)
    o = o.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    ro, rl = attention_ext(_as64(q), _as64(k), _as64(v), softmax_scale(d), causal)
    assert np.abs(o - ro).max() <= TOL_O_BF16
    assert np.abs(lse - rl).max() <= TOL_LSE


def test_llama_layer_with_causal_window_sampled_rows():
    B, H, N, d = 1, 32, 8192, 128
    q, k, v = make_inputs(B, H, N, d, H_kv=8, seed=5)
    rows = sampled_rows(N, 64, seed=81).numpy()
    check(q, k, v, softmax_scale(d), True, "bnhd", (1023, -1), alibi(H), rows=rows,
          tag="llama window 1024 + alibi")


def test_head_dim_256_layer_sampled_rows():
    B, H, N, d = 1, 16, 8192, 256
    q, k, v = make_inputs(B, H, N, d, seed=82)
    rows = sampled_rows(N, 64, seed=83).numpy()
    check(q, k, v, softmax_scale(d), True, "bhnd", rows=rows, tag="d256 N=8192")


def test_deterministic():
    q, k, v = make_inputs(1, 4, 600, 128, seed=84)
    bias = _bias((1, 4, 600, 600), 85, "randn")
    a = gpu_ext(q, k, v, 0.1, True, window=(100, -1), slopes=alibi(4), bias=bias)
    b = gpu_ext(q, k, v, 0.1, True, window=(100, -1), slopes=alibi(4), bias=bias)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("name", ["d256_h16_n8k_causal", "llama3_8b_gqa_n8k_swa4k",
                                  "llama3_8b_n8k_causal_alibi", "b1h16_n4k_bias"])
def test_bench_workloads_sampled_rows(name):
    # the inputs and the call the bench times, checked on 64 sampled rows per head
    from exact_tiled_attention_05_amd import workloads as W
    w = W.WORKLOADS[name]
    q, k, v, scale = W.workload_inputs(name)
    slopes = W.alibi_slopes(w["H"]).numpy() if w.get("alibi") else None
    bias = W.workload_bias(name) if w.get("bias_seed") else None
    rows = sampled_rows(w["N"], w["sample_rows"], seed=w["seed"]).numpy()
    check(q, k, v, scale, w["causal"][-1], w.get("layout", "bhnd"), tuple(w.get("window", (-1, -1))),
          slopes, bias, rows=rows, tag=name)


def test_variants_over_2g_elements_per_tensor():
    # B=20, 32 query heads over 8 K/V heads, N=32768, d=128, [B][N][H][d] (2.7e9 elements per Q),
    # causal 4096-key window and ALiBi: the variant kernel's 64-bit offsets. Sampled rows of four
    # heads checked.
    from oracle import attention_head, kv_head_of
    B, H, H_kv, N, d = 20, 32, 8, 32768, 128
    log("ext over 2^31 elements: B=%d H=%d H_kv=%d N=%d d=%d bnhd window (4095, -1) alibi" % (B, H, H_kv, N, d))
    g = torch.Generator(device=DEV).manual_seed(995)
    mk = lambda h: torch.randn((B, N, h, d), generator=g, device=DEV).to(torch.bfloat16)
    q, k, v = mk(H), mk(H_kv), mk(H_kv)
    assert q.numel() > 2 ** 31
    scale = softmax_scale(d)
    sl = alibi(H)
    o, lse = fa.forward_ext(q, k, v, scale=scale, causal=True, layout="bnhd", window=(4095, -1),
                            alibi_slopes=torch.tensor(sl, device=DEV))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 4095, 4096, N - 1], sampled_rows(N, 28, seed=996).numpy()]))
    for b, h in [(0, 0), (B - 1, H - 1), (9, 14), (17, 3)]:
        j = kv_head_of(h, H, H_kv)
        ro, rl = attention_head(_as64(q[b, :, h].cpu()), _as64(k[b, :, j].cpu()), _as64(v[b, :, j].cpu()),
                                scale, True, rows=rows, window=(4095, -1), alibi_slope=float(sl[h]))
        go = o[b, :, h].float().cpu().numpy().astype(np.float64)[rows]
        gl = lse[b, h].cpu().numpy().astype(np.float64)[rows]
        eo, el = float(np.abs(go - ro).max()), float(np.abs(gl - rl).max())
        log("  b=%d h=%d: max|dO| %.3g  max|dLSE| %.3g" % (b, h, eo, el))
        assert eo <= TOL_O_BF16 and el <= TOL_LSE
    del q, k, v, o, lse
    torch.cuda.empty_cache()

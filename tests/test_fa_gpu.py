"""GPU parity: the HIP path (through the C-ABI) against the CPU float64 oracle on the same seeded
inputs. Bounds: max |O - O_oracle| <= 2e-2 (bf16) / 1e-5 (fp32), max |LSE - LSE_oracle| <= 1e-3.

Full-size workloads run on the GPU at their real shape, in the launch configuration the bench
times; the oracle checks every row where it finishes in seconds and sampled rows otherwise, and
properties that hold at any size are checked on every row.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from exact_tiled_attention_05_amd import workloads as W  # noqa: E402
import exact_tiled_attention_05_amd as fa  # noqa: E402

from gpu_util import (TOL_LSE, TOL_O_BF16, TOL_O_F32, compare, log, oracle_rows,  # noqa: E402
                      run_gpu)


def _tol(dtype):
    return TOL_O_BF16 if dtype == "bf16" else TOL_O_F32


def _check(name, q, k, v, scale, causal, rows=None, heads=None, tol_o=None):
    log(f"[gpu] {name}: shape={tuple(q.shape)} dtype={q.dtype} causal={causal}")
    o, lse = run_gpu(q, k, v, scale, causal)
    assert np.isfinite(o).all() and np.isfinite(lse).all(), f"{name}: non-finite output"
    ref = oracle_rows(q, k, v, scale, causal, rows=rows, heads=heads)
    eo, el = compare(o, lse, ref)
    log(f"[gpu] {name}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    tol = tol_o if tol_o is not None else (TOL_O_BF16 if q.dtype == torch.bfloat16 else TOL_O_F32)
    assert eo <= tol, f"{name}: O error {eo} > {tol}"
    assert el <= TOL_LSE, f"{name}: LSE error {el} > {TOL_LSE}"
    return o, lse, eo, el


# --------------------------------------------------------------------------------------------
# The five workloads.
# --------------------------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_single_head_fp32(causal):
    q, k, v, sc = W.workload_inputs("single_head_fp32")
    _, _, eo, el = _check(f"single_head_fp32 causal={causal}", q, k, v, sc, causal)
    assert el <= 1e-5  # the fp32 path keeps LSE far inside the common bound


def test_b4h16_n1k_d64():
    q, k, v, sc = W.workload_inputs("b4h16_n1k_d64")
    _check("b4h16_n1k_d64", q, k, v, sc, False)


def _boundary_rows(N, extra):
    rows = set(int(r) for r in extra)
    for t in (32, 64, 128, 256):
        for base in range(0, N, max(t, N // 8)):
            for r in (base - 1, base, base + 1):
                if 0 <= r < N:
                    rows.add(r)
    return np.array(sorted(rows))


def test_llama3_n8k_causal():
    name = "llama3_8b_n8k_causal"
    q, k, v, sc = W.workload_inputs(name)
    N = q.shape[2]
    rows = _boundary_rows(N, W.sampled_rows(N, 64, seed=102).numpy())
    log(f"[gpu] {name}: every head on {len(rows)} rows")
    o, lse, _, _ = _check(name, q, k, v, sc, True, rows=rows)
    # two heads in full
    ref = oracle_rows(q, k, v, sc, True, heads=[(0, 0), (0, 31)], workers=2)
    eo, el = compare(o, lse, ref)
    log(f"[gpu] {name}: heads 0 and 31 in full: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O_BF16 and el <= TOL_LSE
    _properties(q, k, v, sc, True, o, lse)


def test_outlier_b16h32_n2k_full():
    name = "outlier_b16h32_n2k"
    q, k, v, sc = W.workload_inputs(name)
    o, lse, _, _ = _check(name, q, k, v, sc, False)  # every row of every head
    _properties(q, k, v, sc, False, o, lse)


def test_long_n32k_causal():
    name = "long_n32k_causal"
    q, k, v, sc = W.workload_inputs(name)
    N = q.shape[2]
    rows = W.sampled_rows(N, W.WORKLOADS[name]["sample_rows"], seed=104).numpy()
    o, lse, _, _ = _check(name, q, k, v, sc, True, rows=rows)
    _properties(q, k, v, sc, True, o, lse)


def _properties(q, k, v, scale, causal, o, lse):
    """Checks valid at any size, on every row: O lies within the range of V per column; LSE is at
    least the score of any visible key (the diagonal when causal, key 0 otherwise) and at most
    scale*|q_i|*max_j|k_j| + ln(#visible)."""
    B, H, N, d = q.shape
    for b in range(B):
        for h in range(H):
            qh = q[b, h].double()
            kh = k[b, h].double()
            vh = v[b, h].double()
            vmin = vh.min(dim=0).values.numpy()
            vmax = vh.max(dim=0).values.numpy()
            assert (o[b, h] >= vmin - 2e-2).all() and (o[b, h] <= vmax + 2e-2).all()
            if causal:
                lo = scale * (qh * kh).sum(dim=1)
                vis = torch.arange(1, N + 1, dtype=torch.float64)
            else:
                lo = scale * (qh @ kh[0])
                vis = torch.full((N,), float(N), dtype=torch.float64)
            hi = scale * qh.norm(dim=1) * kh.norm(dim=1).max() + torch.log(vis)
            assert (lse[b, h] >= lo.numpy() - TOL_LSE).all()
            assert (lse[b, h] <= hi.numpy() + TOL_LSE).all()


# --------------------------------------------------------------------------------------------
# Ragged shapes, both head dims, both masks, both precisions.
# --------------------------------------------------------------------------------------------

@pytest.mark.parametrize("N", [1, 4, 31, 77, 300, 1000])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_bf16(N, d, causal):
    q, k, v = W.make_inputs(2, 3, N, d, "bf16", seed=1000 + N + d)
    _check(f"ragged bf16 N={N} d={d}", q, k, v, W.softmax_scale(d), causal)


@pytest.mark.parametrize("N", [4096, 4097, 4351, 5000, 8191])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_wide_rows(N, causal):
    """d = 128 with N >= 4096 runs the wide-row kernel (256-row workgroups, 64-key tiles, waves
    that go idle past their blocks' diagonal): lengths that end inside a tile, a workgroup and a
    wave's block, every head on every boundary row and on sampled rows."""
    q, k, v = W.make_inputs(1, 3, N, 128, "bf16", seed=N + causal)
    rows = _boundary_rows(N, W.sampled_rows(N, 48, seed=N).numpy())
    _check("wide N=%d" % N, q, k, v, W.softmax_scale(128), causal, rows=rows)


@pytest.mark.parametrize("N", [1, 77, 300])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_f32(N, d, causal):
    q, k, v = W.make_inputs(2, 3, N, d, "fp32", seed=2000 + N + d)
    _check(f"ragged fp32 N={N} d={d}", q, k, v, W.softmax_scale(d), causal)


# --------------------------------------------------------------------------------------------
# Pins repeated on the GPU: the pages' worked example and closed forms.
# --------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_worked_example(dtype, golden_dir):
    """Handbook §2.5 row s = [2, 1, 4, 3] with 2-D values, zero-padded to d = 64."""
    with open(os.path.join(golden_dir, "worked_example.json")) as f:
        g = json.load(f)
    t = torch.bfloat16 if dtype == "bf16" else torch.float32
    N, d = 4, 64
    q = torch.zeros(1, 1, N, d)
    k = torch.zeros(1, 1, N, d)
    v = torch.zeros(1, 1, N, d)
    q[0, 0, :, 0] = 1.0
    k[0, 0, :, 0] = torch.tensor(g["scores"])
    v[0, 0, :, :2] = torch.tensor(g["values"])
    log(f"[gpu] worked example {dtype}")
    o, lse = run_gpu(q.to(t), k.to(t), v.to(t), 1.0, False)
    pr = g["printed"]
    tol = _tol(dtype)
    for i in range(N):  # every query row is the same row
        np.testing.assert_allclose(o[0, 0, i, :2], pr["O"]["value"], rtol=0, atol=tol + 0.5e-8)
        assert np.abs(o[0, 0, i, 2:]).max() == 0.0
        assert abs(lse[0, 0, i] - (4.0 + math.log(pr["ell"]["value"]))) <= TOL_LSE


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("causal", [False, True])
def test_closed_forms(dtype, causal):
    """Identical keys: O is the mean of the visible values and LSE = s + ln(#visible);
    scale = 0: the same with s = 0; constant V: O = V."""
    t = torch.bfloat16 if dtype == "bf16" else torch.float32
    tol = _tol(dtype)
    B, H, N, d = 1, 2, 200, 64
    q, k, v = W.make_inputs(B, H, N, d, "fp32", seed=77)
    k[:] = k[:, :, :1]
    q, k, v = q.to(t), k.to(t), v.to(t)
    sc = 0.125
    log(f"[gpu] closed forms {dtype} causal={causal}")
    o, lse = run_gpu(q, k, v, sc, causal)
    v64 = v.double()
    cnt = torch.arange(1, N + 1, dtype=torch.float64)
    mean = (v64.cumsum(dim=2) / cnt[None, None, :, None]) if causal else \
        v64.mean(dim=2, keepdim=True).expand_as(v64)
    s = sc * (q.double() * k.double()).sum(-1)
    nvis = cnt if causal else torch.full((N,), float(N), dtype=torch.float64)
    assert np.abs(o - mean.numpy()).max() <= tol
    assert np.abs(lse - (s + torch.log(nvis)).numpy()).max() <= (1e-5 if dtype == "fp32" else TOL_LSE)
    q2, k2, _ = W.make_inputs(B, H, N, d, "fp32", seed=78)
    o0, lse0 = run_gpu(q2.to(t), k2.to(t), v, 0.0, causal)
    assert np.abs(o0 - mean.numpy()).max() <= tol
    assert np.abs(lse0 - torch.log(nvis).numpy()).max() <= 1e-5
    vc = torch.linspace(-2, 2, d).expand(B, H, N, d).contiguous().to(t)
    oc, _ = run_gpu(q2.to(t), k2.to(t), vc, sc, causal)
    assert np.abs(oc - vc.double().numpy()).max() <= tol


def test_shift_invariance_f32():
    """Adding u to every key leaves O unchanged and moves LSE_i by scale * q_i . u."""
    B, H, N, d = 1, 2, 300, 64
    q, k, v = W.make_inputs(B, H, N, d, "fp32", seed=99)
    u = torch.randn(d, generator=torch.Generator().manual_seed(5))
    sc = 0.125
    log("[gpu] shift invariance fp32")
    for causal in (False, True):
        o1, l1 = run_gpu(q, k, v, sc, causal)
        o2, l2 = run_gpu(q, (k + u).contiguous(), v, sc, causal)
        assert np.abs(o2 - o1).max() <= 1e-5
        shift = sc * (q.double() @ u.double()).numpy()
        assert np.abs(l2 - (l1 + shift)).max() <= 1e-4


def test_deterministic():
    """No atomics and no cross-workgroup reductions: outputs are bitwise identical run to run."""
    q, k, v, sc = W.workload_inputs("b4h16_n1k_d64")
    dev = torch.device("cuda:0")
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    log("[gpu] determinism")
    for causal in (False, True):
        o1, l1 = fa.forward(qd, kd, vd, scale=sc, causal=causal)
        o1, l1 = o1.clone(), l1.clone()
        o2, l2 = fa.forward(qd, kd, vd, scale=sc, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_stream_and_buffers():
    """Runs on a caller-provided stream into caller-provided buffers, and leaves memory beyond
    the outputs untouched."""
    q, k, v = W.make_inputs(1, 2, 333, 128, "bf16", seed=3)
    dev = torch.device("cuda:0")
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    big = torch.full((2 * 333 * 128 + 64,), 7.0, dtype=torch.bfloat16, device=dev)
    out = big[: 2 * 333 * 128].view(1, 2, 333, 128)
    lbig = torch.full((2 * 333 + 16,), 5.0, dtype=torch.float32, device=dev)
    lse = lbig[: 2 * 333].view(1, 2, 333)
    s = torch.cuda.Stream()
    log("[gpu] stream and buffers")
    with torch.cuda.stream(s):
        fa.forward(qd, kd, vd, causal=True, out=out, lse=lse)
    s.synchronize()
    assert (big[2 * 333 * 128:] == 7.0).all() and (lbig[2 * 333:] == 5.0).all()
    ref = oracle_rows(q, k, v, W.softmax_scale(128), True)
    eo, el = compare(out.float().cpu().numpy().astype(np.float64),
                     lse.cpu().numpy().astype(np.float64), ref)
    assert eo <= TOL_O_BF16 and el <= TOL_LSE


def test_error_codes_on_device_tensors():
    """Bad arguments are refused before any launch and leave the outputs untouched."""
    dev = torch.device("cuda:0")
    q = torch.randn(1, 1, 64, 64, device=dev).to(torch.bfloat16)
    o = torch.zeros_like(q)
    lse = torch.zeros(1, 1, 64, device=dev)
    p, po, pl = q.data_ptr(), o.data_ptr(), lse.data_ptr()
    log("[gpu] error codes")
    cases = [
        ((p + 2, p, p, po, pl, 1, 1, 64, 64, 0.1, 0), fa.FA_ERR_ALIGNMENT),
        ((p, p, p, po, pl, 1, 1, 64, 96, 0.1, 0), fa.FA_ERR_UNSUPPORTED),
        ((p, p, p, po, pl, 1, 1, 0, 64, 0.1, 0), fa.FA_ERR_INVALID_ARG),
        ((p, p, p, po, pl, 1, 1, 64, 64, -0.1, 0), fa.FA_ERR_INVALID_ARG),
        ((p, p, p, po, pl, 1, 1, 64, 64, float("nan"), 0), fa.FA_ERR_INVALID_ARG),
        ((p, p, p, po, pl, 1, 1, 64, 64, 0.1, 2), fa.FA_ERR_INVALID_ARG),
        ((p, p, p, p, pl, 1, 1, 64, 64, 0.1, 0), fa.FA_ERR_INVALID_ARG),  # o aliases q
        ((p, p, p, po, po, 1, 1, 64, 64, 0.1, 0), fa.FA_ERR_INVALID_ARG),  # lse inside o
    ]
    for args, code in cases:
        assert fa.fa_fwd(*args, None) == code, args
    torch.cuda.synchronize()
    assert (o == 0).all() and (lse == 0).all()


# --------------------------------------------------------------------------------------------
# Tensors past 2^31 elements: every element offset needs 64-bit arithmetic.
# --------------------------------------------------------------------------------------------

def _big_inputs(B, H, H_kv, N, d, layout, seed):
    """Seeded N(0, 1) bf16 Q, K, V drawn on the GPU (tensors this large would take minutes on the
    host), in ``layout``."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(seed)
    shape = (lambda h: (B, h, N, d)) if layout == "bhnd" else (lambda h: (B, N, h, d))
    return tuple(torch.randn(shape(h), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
                 for h in (H, H_kv, H_kv))


def _head(x, b, h, layout):
    """One (b, h) slice [N, d] of a device tensor, as a CPU float64 array."""
    t = x[b, h] if layout == "bhnd" else x[b, :, h]
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("layout", ["bhnd", "bnhd"])
def test_over_2g_elements_per_tensor(layout):
    # B=20, H=32, N=32768, d=128: 2.7e9 elements (5 GiB) per tensor, causal; grouped 32/8 heads in
    # [B][N][H][d]. Heads in the first and last batch are checked on sampled rows.
    from oracle import attention_head, kv_head_of
    B, H, N, d = 20, 32, 32768, 128
    H_kv = H if layout == "bhnd" else 8
    log(f"[gpu] over 2^31 elements: B={B} H={H} H_kv={H_kv} N={N} d={d} layout={layout}")
    q, k, v = _big_inputs(B, H, H_kv, N, d, layout, seed=991)
    assert q.numel() > 2 ** 31
    scale = W.softmax_scale(d)
    o, lse = fa.forward(q, k, v, scale=scale, causal=True, layout=layout)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, N - 1], W.sampled_rows(N, 29, seed=992).numpy()]))
    worst_o = worst_l = 0.0
    for b, h in [(0, 0), (B - 1, H - 1), (B - 1, 5), (11, 17)]:
        j = kv_head_of(h, H, H_kv)
        qh, kh, vh = _head(q, b, h, layout), _head(k, b, j, layout), _head(v, b, j, layout)
        ro, rl = attention_head(qh, kh, vh, scale, True, rows=rows)
        go = _head(o, b, h, layout)[rows]
        gl = lse[b, h].cpu().numpy().astype(np.float64)[rows]
        worst_o = max(worst_o, float(np.abs(go - ro).max()))
        worst_l = max(worst_l, float(np.abs(gl - rl).max()))
    log(f"[gpu] over 2^31 elements ({layout}): max|dO|={worst_o:.3e} max|dLSE|={worst_l:.3e}")
    assert worst_o <= TOL_O_BF16 and worst_l <= TOL_LSE
    del q, k, v, o, lse
    torch.cuda.empty_cache()

"""GPU parity for grouped K/V heads and the [B][N][H][d] layout ("Understanding FlashAttention
Pt 1", §4.1) through fa_fwd_gqa / fa_fwd_gqa_f32, against the CPU float64 oracle
(oracle.attention_gqa's head assignment). Same bounds as the MHA tests. Two exact checks hold at
any size: the [B][N][H][d] result equals the [B][H][N][d] result bit for bit, and grouped heads
equal multi-head attention with each K/V head repeated for its query heads, bit for bit (the
kernel does the same arithmetic on the same values either way).
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from exact_tiled_attention_05_amd import workloads as W  # noqa: E402
import exact_tiled_attention_05_amd as fa  # noqa: E402
from oracle import kv_head_of  # noqa: E402

from gpu_util import (TOL_LSE, TOL_O_BF16, TOL_O_F32, compare, log, oracle_rows_gqa,  # noqa: E402
                      run_gpu, run_gpu_layout)


def _rand(B, H, H_kv, N, d, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, H, N, d), generator=g)
    k = torch.randn((B, H_kv, N, d), generator=g)
    v = torch.randn((B, H_kv, N, d), generator=g)
    return q.to(dtype), k.to(dtype), v.to(dtype)


def _check(name, q, k, v, scale, causal, layout, rows=None, heads=None):
    log(f"[gpu] {name}: q={tuple(q.shape)} kv={tuple(k.shape)} {q.dtype} causal={causal} layout={layout}")
    o, lse = run_gpu_layout(q, k, v, scale, causal, layout)
    assert np.isfinite(o).all() and np.isfinite(lse).all(), f"{name}: non-finite output"
    ref = oracle_rows_gqa(q, k, v, scale, causal, rows=rows, heads=heads)
    eo, el = compare(o, lse, ref)
    log(f"[gpu] {name}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    tol = TOL_O_BF16 if q.dtype == torch.bfloat16 else TOL_O_F32
    assert eo <= tol, f"{name}: O error {eo} > {tol}"
    assert el <= TOL_LSE, f"{name}: LSE error {el} > {TOL_LSE}"
    return o, lse


def _boundary_rows(N, extra):
    rows = set(int(r) for r in extra)
    for t in (32, 64, 128, 256):
        for base in range(0, N, max(t, N // 8)):
            for r in (base - 1, base, base + 1):
                if 0 <= r < N:
                    rows.add(r)
    return np.array(sorted(rows))


def test_llama3_gqa_n8k_causal():
    """The Llama-3-8B layer with its 8 K/V heads, tokens outermost, at full size."""
    name = "llama3_8b_gqa_n8k_causal"
    w = W.WORKLOADS[name]
    q, k, v, sc = W.workload_inputs(name)
    N = q.shape[2]
    rows = _boundary_rows(N, W.sampled_rows(N, w["sample_rows"], seed=105).numpy())
    log(f"[gpu] {name}: every head on {len(rows)} rows")
    o, lse = _check(name, q, k, v, sc, True, w["layout"], rows=rows)
    ref = oracle_rows_gqa(q, k, v, sc, True, heads=[(0, 3), (0, 28)], workers=2)
    eo, el = compare(o, lse, ref)
    log(f"[gpu] {name}: heads 3 and 28 in full: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O_BF16 and el <= TOL_LSE
    # on every row: O within the range of its K/V head's V, LSE at least the diagonal score
    H, H_kv = q.shape[1], k.shape[1]
    for h in range(H):
        j = kv_head_of(h, H, H_kv)
        vh = v[0, j].double()
        assert (o[0, h] >= vh.min(dim=0).values.numpy() - 2e-2).all()
        assert (o[0, h] <= vh.max(dim=0).values.numpy() + 2e-2).all()
        diag = sc * (q[0, h].double() * k[0, j].double()).sum(dim=1)
        assert (lse[0, h] >= diag.numpy() - TOL_LSE).all()


def test_llama3_gqa_equals_expanded_mha_bitwise():
    """Grouped heads through fa_fwd_gqa ([B][N][H][d]) == fa_fwd on K/V repeated per query head."""
    name = "llama3_8b_gqa_n8k_causal"
    w = W.WORKLOADS[name]
    q, k, v, sc = W.workload_inputs(name)
    o1, l1 = run_gpu_layout(q, k, v, sc, True, w["layout"])
    G = q.shape[1] // k.shape[1]
    ke, ve = (x.repeat_interleave(G, dim=1).contiguous() for x in (k, v))
    o2, l2 = run_gpu(q, ke, ve, sc, True)
    log(f"[gpu] {name}: grouped vs expanded: max|dO|={np.abs(o1 - o2).max():.3e}")
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_layouts_bitwise_equal(d, causal):
    q, k, v = _rand(2, 8, 2, 1000, d, torch.bfloat16, 11)
    sc = W.softmax_scale(d)
    a = run_gpu_layout(q, k, v, sc, causal, "bhnd")
    b = run_gpu_layout(q, k, v, sc, causal, "bnhd")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("layout", ["bhnd", "bnhd"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("heads", [(6, 2), (4, 1), (3, 3)], ids=["gqa6x2", "mqa4", "mha3"])
@pytest.mark.parametrize("N", [77, 300])
def test_ragged_gqa(N, heads, d, causal, layout):
    H, H_kv = heads
    q, k, v = _rand(2, H, H_kv, N, d, torch.bfloat16, 100 + N + H + d)
    _check(f"ragged_gqa N={N} H={H} H_kv={H_kv} d={d}", q, k, v, W.softmax_scale(d), causal, layout)


@pytest.mark.parametrize("layout", ["bhnd", "bnhd"])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_f32(causal, layout):
    q, k, v = _rand(1, 4, 2, 100, 64, torch.float32, 7)
    _check("gqa_f32", q, k, v, 0.125, causal, layout)


def test_gqa_error_codes_on_device_tensors():
    dev = torch.device("cuda:0")
    q = torch.zeros(1, 4, 64, 64, dtype=torch.bfloat16, device=dev)
    k = torch.zeros(1, 3, 64, 64, dtype=torch.bfloat16, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty(1, 4, 64, device=dev)
    rc = fa.fa_fwd_gqa(q.data_ptr(), k.data_ptr(), k.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       1, 4, 3, 64, 64, 0.125, 0, fa.FA_LAYOUT_BHND,
                       torch.cuda.current_stream().cuda_stream)
    assert rc == fa.FA_ERR_INVALID_ARG

"""Race check of the LDS pipelines: the fast library against its race-check build, bit for bit.

libfa_race.so is libfa.so compiled with FA_RACE_CHECK=1: every K/V (or Q/dO) tile load into LDS
completes for the whole work-group before any wave goes on, staged stores wait at a barrier, and
LDS starts filled with NaN. The arithmetic and its order are the same, so outputs must be
identical bit for bit. A read of a tile before it has landed, or a load overwriting a tile a wave
still reads, makes the fast build differ; a read of LDS that no load wrote gives NaN.

Cases: every kernel with a cross-wave LDS pipeline -- the wide-row forward (the causal Llama
layer's shape with fewer heads, N = 32768, a ragged non-causal N), the 4-wave forward of the
variants (the outlier recipe's shape, a sliding window with grouped heads, ALiBi, an additive bias,
d = 256), the 8-wave forward (d = 64 and d = 128 small grids) and both backward kernels. The
split-KV decode kernel keeps one LDS tile per wave (no cross-wave sharing) and is not part of it.
"""
import os
import zlib

import pytest
import torch

import exact_tiled_attention_05_amd as fa
from exact_tiled_attention_05_amd.workloads import make_inputs, softmax_scale, to_layout

from gpu_util import log

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def race_lib():
    path = fa.race_check_library_path()
    if not os.path.exists(path):
        raise RuntimeError("libfa_race.so is not built: python -m exact_tiled_attention_05_amd.build --all")
    return fa.load_library(path)


def _bits_equal(a, b):
    assert a.shape == b.shape and a.dtype == b.dtype
    ia = a.contiguous().view(torch.int16 if a.element_size() == 2 else torch.int32)
    ib = b.contiguous().view(torch.int16 if b.element_size() == 2 else torch.int32)
    return bool(torch.equal(ia, ib))


def _both(race_lib, fn):
    """fn() with libfa.so, then with libfa_race.so; tuples of output tensors."""
    fast = fn()
    torch.cuda.synchronize()
    with fa.using_library(race_lib):
        slow = fn()
    torch.cuda.synchronize()
    return fast, slow


def _check(name, fast, slow):
    for i, (a, b) in enumerate(zip(fast, slow)):
        assert torch.isfinite(b.float()).all(), "%s: output %d of the race-check build not finite" % (name, i)
        if not _bits_equal(a, b):
            diff = (a.float() - b.float()).abs()
            raise AssertionError("%s: output %d differs from the race-check build at %d elements "
                                 "(max |diff| %g)" % (name, i, int((diff != 0).sum()), float(diff.max())))


FWD_CASES = [
    # name, dict(B, H, H_kv, N, d, causal, layout, extra make_inputs args)
    ("wide_llama_n8k_causal", dict(B=1, H=8, H_kv=8, N=8192, d=128, causal=True, layout="bhnd")),
    ("wide_gqa_n8k_causal_bnhd", dict(B=1, H=8, H_kv=2, N=8192, d=128, causal=True, layout="bnhd")),
    ("wide_n32k_causal", dict(B=1, H=16, H_kv=16, N=32768, d=128, causal=True, layout="bhnd")),
    ("wide_ragged_noncausal", dict(B=2, H=3, H_kv=3, N=4097 + 63, d=128, causal=False,
                                   layout="bhnd")),
    ("ext_outlier_n2k", dict(B=2, H=32, H_kv=32, N=2048, d=128, causal=False, layout="bhnd",
                             q_mult=8.0, outlier_frac=0.01, outlier_mult=4.0)),
    ("ext_causal_n2k_ragged", dict(B=1, H=32, H_kv=8, N=2000, d=128, causal=True, layout="bnhd")),
    ("ext_d256_causal", dict(B=1, H=4, H_kv=4, N=4096, d=256, causal=True, layout="bhnd")),
    ("base_d64_b4h16_n1k", dict(B=4, H=16, H_kv=16, N=1024, d=64, causal=False, layout="bhnd")),
    ("base_d128_small_causal", dict(B=1, H=4, H_kv=4, N=1000, d=128, causal=False, layout="bhnd")),
]


@pytest.mark.parametrize("name,w", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_forward_matches_race_check_build(race_lib, name, w):
    log("race check %s %s" % (name, w))
    w = dict(w)
    layout = w.pop("layout")
    causal = w.pop("causal")
    q, k, v = make_inputs(dtype="bf16", seed=zlib.crc32(name.encode()) % 1000, **w)
    qd, kd, vd = (to_layout(x, layout).to(DEV) for x in (q, k, v))
    sc = softmax_scale(w["d"])
    fast, slow = _both(race_lib, lambda: fa.forward(qd, kd, vd, scale=sc, causal=causal,
                                                     layout=layout))
    _check(name, fast, slow)


def test_variants_match_race_check_build(race_lib):
    """Sliding window with grouped heads and causal ALiBi (both on the wide-row kernel at N = 8192,
    ALiBi walking the key tiles from the diagonal down), and an additive bias (its own LDS tiles,
    loaded ahead of the K/V tiles they belong to)."""
    B, H, H_kv, N, d = 1, 8, 2, 8192, 128
    q, k, v = make_inputs(B=B, H=H, H_kv=H_kv, N=N, d=d, dtype="bf16", seed=5)
    qd, kd, vd = (to_layout(x, "bnhd").to(DEV) for x in (q, k, v))
    sc = softmax_scale(d)
    log("race check window (4095, -1) causal bnhd")
    _check("window", *_both(race_lib, lambda: fa.forward_ext(qd, kd, vd, scale=sc, causal=True,
                                                               layout="bnhd", window=(4095, -1))))
    slopes = torch.tensor([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], device=DEV)
    log("race check alibi causal")
    _check("alibi", *_both(race_lib, lambda: fa.forward_ext(qd, kd, vd, scale=sc, causal=True,
                                                              layout="bnhd", alibi_slopes=slopes)))
    B, H, N = 1, 4, 4096
    q, k, v = make_inputs(B=B, H=H, N=N, d=d, dtype="bf16", seed=8)
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    g = torch.Generator().manual_seed(18)
    bias = torch.randn(B, H, N, N, generator=g).to(torch.bfloat16).to(DEV)
    for causal in (False, True):
        log("race check bias causal=%s" % causal)
        _check("bias causal=%s" % causal,
               *_both(race_lib, lambda: fa.forward_ext(qd, kd, vd, scale=sc, causal=causal,
                                                       bias=bias)))
    # window and bias together at a ragged length
    N = 3000
    q, k, v = make_inputs(B=1, H=4, N=N, d=d, dtype="bf16", seed=9)
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    pad = torch.zeros(1, 4, N, (N + 7) // 8 * 8, dtype=torch.bfloat16, device=DEV)
    pad[..., :N] = torch.randn(1, 4, N, N, generator=g).to(torch.bfloat16).to(DEV)
    log("race check window + bias ragged")
    _check("window+bias", *_both(race_lib, lambda: fa.forward_ext(
        qd, kd, vd, scale=sc, causal=False, window=(700, 300), bias=pad[..., :N])))


BWD_CASES = [
    ("bwd_llama_n4k_causal", dict(B=1, H=4, H_kv=4, N=4096, d=128, causal=True, layout="bhnd")),
    ("bwd_gqa_n4k_causal_bnhd", dict(B=1, H=8, H_kv=2, N=4096, d=128, causal=True,
                                     layout="bnhd")),
    ("bwd_d64_ragged", dict(B=2, H=4, H_kv=4, N=1000, d=64, causal=False, layout="bhnd")),
]


@pytest.mark.parametrize("name,w", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_backward_matches_race_check_build(race_lib, name, w):
    log("race check %s %s" % (name, w))
    w = dict(w)
    layout = w.pop("layout")
    causal = w.pop("causal")
    q, k, v = make_inputs(dtype="bf16", seed=zlib.crc32(name.encode()) % 1000, **w)
    g = torch.Generator().manual_seed(12)
    do = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    qd, kd, vd, dod = (to_layout(x, layout).to(DEV) for x in (q, k, v, do))
    sc = softmax_scale(w["d"])
    o, lse = fa.forward(qd, kd, vd, scale=sc, causal=causal, layout=layout)
    torch.cuda.synchronize()
    fast, slow = _both(race_lib, lambda: fa.backward(qd, kd, vd, o, lse, dod, scale=sc,
                                                     causal=causal, layout=layout))
    _check(name, fast, slow)

"""A CPU model of the bf16 forward kernels' rounding, run on the outlier recipe over several seeds.

Why: the bf16 kernels keep a lazy reference maximum (the reference moves only when a score exceeds
it by more than a slack, in log2 units) and feed P to the PV product rounded to bf16. Both are exact
in real arithmetic ("Understanding FlashAttention Pt 1", §2.2: any reference point gives the same
softmax), so what they change is rounding. This model takes the kernels' rounding steps -- fp32
scores from bf16 operands, the lazy reference checked once per 32 keys for a block of 32 query rows,
p = 2^(s c - ref) in fp32, l summed from the fp32 p, P rounded to bf16 for the product, the output
divided by l and rounded to bf16 -- and checks, against the float64 oracle, that the slack the
kernels use keeps max |dO| inside the 2e-2 bf16 tolerance with room to spare on outlier rows
(queries x 8, 1% of the keys x 4).
"""
import numpy as np
import pytest
import torch

from exact_tiled_attention_05_amd.workloads import make_inputs, softmax_scale
from oracle import attention_head

ROW_BLOCK = 32   # query rows that take the rescale decision together (one MFMA block)
KEY_STEP = 32    # keys per check of the reference
KERNEL_SLACK = 2.0
LOG2E = 1.4426950408889634


def _bf16(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).float().numpy()


def kernel_rounding_model(q, k, v, scale, slack):
    """Non-causal forward of one head with the kernels' rounding steps; returns bf16 O as float64."""
    n, dv = q.shape[0], v.shape[1]
    s = q.astype(np.float32) @ k.astype(np.float32).T          # MFMA: bf16 in, fp32 out
    c = np.float32(scale * LOG2E)
    x_all = (s * c).astype(np.float32)                         # scores in log2 units
    g = n // ROW_BLOCK
    m = np.full((g, ROW_BLOCK), -np.inf, np.float32)
    ref = np.zeros((g, ROW_BLOCK), np.float32)
    ell = np.zeros((g, ROW_BLOCK), np.float32)
    acc = np.zeros((g, ROW_BLOCK, dv), np.float32)
    x_all = x_all.reshape(g, ROW_BLOCK, n)
    for k0 in range(0, n, KEY_STEP):
        x = x_all[:, :, k0:k0 + KEY_STEP]
        top = x.max(axis=2)
        # the block moves its reference when any of its rows exceeds it by more than the slack
        # (every row while the block has seen no score yet)
        thr = np.where(np.isfinite(m), ref + np.float32(slack), -np.inf)
        move = np.any(top > thr, axis=1)
        if move.any():
            mn = np.maximum(m, top)
            alpha = np.where(np.isfinite(m), np.exp2(m - mn), 0.0).astype(np.float32)
            alpha = np.where(move[:, None], alpha, np.float32(1.0))
            ell = (ell * alpha).astype(np.float32)
            acc = (acc * alpha[:, :, None]).astype(np.float32)
            m = np.where(move[:, None], mn, m)
            ref = np.where(np.isfinite(m), m, np.float32(0.0)).astype(np.float32)
        p = np.exp2(x - ref[:, :, None]).astype(np.float32)
        ell = (ell + p.sum(axis=2, dtype=np.float32)).astype(np.float32)
        pb = _bf16(p)
        pv = pb.reshape(-1, pb.shape[2]) @ v[k0:k0 + KEY_STEP].astype(np.float32)
        acc = (acc + pv.reshape(acc.shape)).astype(np.float32)
    o = (acc / ell[:, :, None]).reshape(n, dv)
    return _bf16(o).astype(np.float64)


def _worst_error(seed, slack, heads=6):
    q, k, v = make_inputs(B=1, H=heads, N=2048, d=128, dtype="bf16", seed=seed, q_mult=8.0,
                          outlier_frac=0.01, outlier_mult=4.0)
    sc = softmax_scale(128)
    worst = 0.0
    for h in range(heads):
        qh, kh, vh = (x[0, h].float().numpy().astype(np.float64) for x in (q, k, v))
        o_ref, _ = attention_head(qh, kh, vh, sc, False)
        o = kernel_rounding_model(qh, kh, vh, sc, slack)
        worst = max(worst, float(np.abs(o - o_ref).max()))
    return worst


def test_model_with_zero_slack_is_plain_bf16_rounding():
    """With the reference always at the exact running max the model only adds the bf16 rounding
    of P and of O to the oracle: well inside the tolerance on ordinary inputs."""
    q, k, v = make_inputs(B=1, H=1, N=256, d=64, dtype="bf16", seed=11)
    qh, kh, vh = (x[0, 0].float().numpy().astype(np.float64) for x in (q, k, v))
    sc = softmax_scale(64)
    o_ref, _ = attention_head(qh, kh, vh, sc, False)
    assert np.abs(kernel_rounding_model(qh, kh, vh, sc, 0.0) - o_ref).max() < 1e-2


@pytest.mark.parametrize("seed", [3, 21, 22, 23])
def test_kernel_slack_keeps_outlier_rows_in_tolerance(seed):
    worst = _worst_error(seed, KERNEL_SLACK)
    assert worst <= 0.018, "slack %g: max |dO| = %.5f" % (KERNEL_SLACK, worst)

"""The pages' streaming recurrences (oracle/online.py) reach the dense oracle's max, sum, output
and logsumexp for every way of cutting the keys into blocks -- on the CPU, in float64."""
import json
import math
import os

import numpy as np
import pytest

from oracle import attention_head, blockwise_row, online_normalizer, tiled_attention

RNG = np.random.default_rng(7)


def test_worked_example_blockwise_states(golden_dir):
    """Handbook §2.5, two blocks [2, 1] and [4, 3]: the printed intermediate states."""
    with open(os.path.join(golden_dir, "worked_example.json")) as f:
        g = json.load(f)
    s = np.array(g["scores"])
    v = np.array(g["values"])
    pr = g["printed"]
    bounds = [tuple(b) for b in pr["block_split"]]
    m, ell, a, o, states = blockwise_row(s, v, bounds)
    tol8 = 0.5e-8 + 1e-12
    m1, ell1, a1 = states[0]
    assert m1 == pr["m_1"]
    assert abs(ell1 - pr["ell_1"]["value"]) < tol8
    np.testing.assert_allclose(a1, [1.0, math.exp(-1.0)], rtol=0, atol=1e-15)
    assert m == 4.0
    assert abs(ell - pr["ell"]["value"]) < tol8
    np.testing.assert_allclose(a, pr["a_2"]["value"], rtol=0, atol=tol8)
    np.testing.assert_allclose(o, pr["O"]["value"], rtol=0, atol=tol8)
    mm, ll = online_normalizer([s[0:2], s[2:4]])
    assert mm == 4.0 and abs(ll - pr["ell"]["value"]) < tol8


def _splits(n):
    """Every uniform block size 1..n (last block short when it does not divide n) plus a few
    irregular splits."""
    out = []
    for b in range(1, n + 1):
        out.append([(s, min(s + b, n)) for s in range(0, n, b)])
    cuts = sorted(set(RNG.choice(np.arange(1, n), size=min(4, n - 1), replace=False).tolist()))
    edges = [0] + cuts + [n]
    out.append(list(zip(edges[:-1], edges[1:])))
    return out


@pytest.mark.parametrize("n", [1, 2, 5, 16, 23])
def test_online_normalizer_equals_dense(n):
    """Block summaries merged by Chapter 26 Eq 26.2 over any split give the dense max and sum
    (to 1e-12 relative)."""
    s = RNG.standard_normal(n) * 5
    s_masked = s.copy()
    s_masked[n // 2 + 1:] = -np.inf  # a causal-style row: future keys are -inf
    for row in (s, s_masked):
        m_ref = row.max()
        ell_ref = np.exp(row - m_ref).sum()
        for split in _splits(n):
            m, ell = online_normalizer([row[a:b] for a, b in split])
            assert m == m_ref
            assert abs(ell - ell_ref) <= 1e-12 * ell_ref


@pytest.mark.parametrize("n", [1, 3, 8, 19])
def test_blockwise_row_equals_dense(n):
    d, dv = 4, 3
    q = RNG.standard_normal((n, d))
    k = RNG.standard_normal((n, d))
    v = RNG.standard_normal((n, dv))
    sc = 0.9
    for causal in (False, True):
        o_ref, lse_ref, s, _ = attention_head(q, k, v, sc, causal, return_sp=True)
        for i in range(n):
            for split in _splits(n):
                m, ell, a, o, _ = blockwise_row(s[i], v, split)
                np.testing.assert_allclose(o, o_ref[i], rtol=0, atol=1e-12)
                assert abs(m + math.log(ell) - lse_ref[i]) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_tiled_equals_dense_all_block_sizes(causal):
    """FA-2 form (queries outermost, one division at the end, LSE stored, causal tiles skipped /
    unmasked / masked by their coordinates) equals the dense oracle for all tile sizes, including
    tiles that do not divide N and query tiles different from key tiles (Exercise 26.4)."""
    n, d = 19, 6
    q = RNG.standard_normal((n, d)) * 2
    k = RNG.standard_normal((n, d)) * 2
    v = RNG.standard_normal((n, d))
    o_ref, lse_ref = attention_head(q, k, v, 0.5, causal)
    for bq in range(1, n + 2):
        for bk in range(1, n + 2):
            o, lse = tiled_attention(q, k, v, 0.5, causal, bq, bk)
            np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_tiled_toy_card_shape():
    """tokentrails card toy: 8 tokens, d = 4, 4 x 4 tiles, checked against ordinary attention."""
    q = RNG.standard_normal((8, 4))
    k = RNG.standard_normal((8, 4))
    v = RNG.standard_normal((8, 4))
    for causal in (False, True):
        o, lse = tiled_attention(q, k, v, 0.5, causal, 4, 4)
        o_ref, lse_ref = attention_head(q, k, v, 0.5, causal)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-13)


def test_tiled_late_large_maximum():
    """A maximum that arrives in the last key tile forces a large rescale of earlier state."""
    n, d = 64, 8
    q = RNG.standard_normal((n, d)) * 8
    k = RNG.standard_normal((n, d))
    k[-1] *= 4
    k[-3] *= 4
    v = RNG.standard_normal((n, d))
    sc = 1 / math.sqrt(d)
    o_ref, lse_ref = attention_head(q, k, v, sc, False)
    for bk in (1, 7, 16, 64):
        o, lse = tiled_attention(q, k, v, sc, False, 16, bk)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)

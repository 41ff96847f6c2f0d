"""Pins for the grouped-K/V-head oracle (oracle.attention_gqa, oracle.kv_head_of), on the CPU.

"Understanding FlashAttention Pt 1", §4.1: the query heads divide evenly over the K/V heads and
each query head attends with its assigned K/V head. The pins tie the oracle to a closed form
whose value depends on which K/V head a query head uses, to brute force in scalar Python, and to
the MHA and MQA special cases; planted wrong head assignments must fail them.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import attention_gqa, kv_head_of

RNG = np.random.default_rng(4242)


def _brute_gqa(q, k, v, scale, causal):
    """Scalar-Python attention with grouped K/V heads. Group of query head h: floor(h*H_kv/H)."""
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    o = np.zeros((B, H, N, v.shape[3]))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            j = (h * H_kv) // H
            for i in range(N):
                keys = range(i + 1) if causal else range(N)
                s = [scale * math.fsum(q[b, h, i, t] * k[b, j, n, t] for t in range(d)) for n in keys]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                tot = math.fsum(e)
                for c in range(v.shape[3]):
                    o[b, h, i, c] = math.fsum(e[n] * v[b, j, n, c] for n in range(len(e))) / tot
                lse[b, h, i] = m + math.log(tot)
    return o, lse


def pin_identical_keys_per_group(fn, causal):
    """Every key row of K/V head j equals one vector: all weights are equal, so O for a query of
    group j is the mean of head j's visible V rows and LSE = s + ln(#visible). V differs between
    K/V heads, so a query head attending with any other K/V head gives a different mean."""
    B, H, H_kv, N, d = 2, 6, 3, 5, 4
    q = RNG.standard_normal((B, H, N, d))
    k = np.repeat(RNG.standard_normal((B, H_kv, 1, d)), N, axis=2)
    v = RNG.standard_normal((B, H_kv, N, d)) + 3.0 * np.arange(H_kv)[None, :, None, None]
    o, lse = fn(q, k, v, 0.7, causal)
    for b in range(B):
        for h in range(H):
            j = h // (H // H_kv)
            for i in range(N):
                n = i + 1 if causal else N
                np.testing.assert_allclose(o[b, h, i], v[b, j, :n].mean(axis=0), atol=1e-12)
                s = 0.7 * float(q[b, h, i] @ k[b, j, 0])
                np.testing.assert_allclose(lse[b, h, i], s + math.log(n), atol=1e-12)


def pin_brute_force(fn):
    for (B, H, H_kv, N, d) in [(1, 4, 2, 3, 2), (2, 6, 3, 4, 3), (1, 3, 1, 5, 2), (1, 2, 2, 4, 2)]:
        q = RNG.standard_normal((B, H, N, d))
        k = RNG.standard_normal((B, H_kv, N, d))
        v = RNG.standard_normal((B, H_kv, N, d))
        for causal in (False, True):
            o, lse = fn(q, k, v, 0.9, causal)
            ob, lb = _brute_gqa(q, k, v, 0.9, causal)
            np.testing.assert_allclose(o, ob, atol=1e-12)
            np.testing.assert_allclose(lse, lb, atol=1e-12)


def pin_mqa_shared_head(fn):
    """One K/V head (MQA): query heads with the same queries give the same output."""
    q1 = RNG.standard_normal((1, 1, 6, 4))
    q = np.repeat(q1, 5, axis=1)
    k = RNG.standard_normal((1, 1, 6, 4))
    v = RNG.standard_normal((1, 1, 6, 4))
    o, lse = fn(q, k, v, 0.5, True)
    for h in range(1, 5):
        np.testing.assert_array_equal(o[0, h], o[0, 0])
        np.testing.assert_array_equal(lse[0, h], lse[0, 0])


def _all_pins(fn):
    pin_identical_keys_per_group(fn, False)
    pin_identical_keys_per_group(fn, True)
    pin_brute_force(fn)
    pin_mqa_shared_head(fn)


def test_gqa_oracle_passes_pins():
    _all_pins(attention_gqa)


def test_gqa_with_one_head_per_group_is_mha():
    q, k, v = (RNG.standard_normal((2, 3, 7, 4)) for _ in range(3))
    for causal in (False, True):
        o1, l1 = attention_gqa(q, k, v, 0.8, causal)
        o2, l2 = oracle.attention(q, k, v, 0.8, causal)
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)


def test_gqa_rows_subset():
    q = RNG.standard_normal((1, 4, 9, 3))
    k, v = RNG.standard_normal((1, 2, 9, 3)), RNG.standard_normal((1, 2, 9, 3))
    rows = np.array([0, 4, 8])
    o, lse = attention_gqa(q, k, v, 0.6, True)
    o2, l2 = attention_gqa(q, k, v, 0.6, True, rows)
    np.testing.assert_allclose(o2, o[:, :, rows], atol=1e-14)
    np.testing.assert_allclose(l2, lse[:, :, rows], atol=1e-14)


def test_kv_head_of_rejects_uneven_groups():
    assert [kv_head_of(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    assert [kv_head_of(h, 4, 1) for h in range(4)] == [0, 0, 0, 0]
    for bad in [(6, 4), (3, 0), (2, 3)]:
        with pytest.raises(ValueError):
            kv_head_of(0, *bad)


def _mutant(assign):
    """attention_gqa with a different (wrong) query-head -> K/V-head assignment."""
    def fn(q, k, v, scale, causal):
        B, H = q.shape[0], q.shape[1]
        H_kv = k.shape[1]
        o = np.empty((B, H, q.shape[2], v.shape[3]))
        lse = np.empty((B, H, q.shape[2]))
        for b in range(B):
            for h in range(H):
                j = assign(h, H, H_kv)
                o[b, h], lse[b, h] = oracle.attention_head(q[b, h], k[b, j], v[b, j], scale, causal)
        return o, lse
    return fn


@pytest.mark.parametrize("name,assign", [
    ("interleaved", lambda h, H, H_kv: h % H_kv),
    ("always_first", lambda h, H, H_kv: 0),
    ("reversed_groups", lambda h, H, H_kv: H_kv - 1 - h // (H // H_kv)),
])
def test_wrong_head_assignments_fail_a_pin(name, assign):
    with pytest.raises(AssertionError):
        _all_pins(_mutant(assign))


def test_correct_assignment_in_mutant_factory_passes():
    _all_pins(_mutant(lambda h, H, H_kv: h // (H // H_kv)))

"""Pins for the oracle's score modifiers: sliding window, ALiBi, additive bias (CPU).

"Understanding FlashAttention Pt 1" writes the scores as S = QK^T / sqrt(d) + B with B an optional
additive mask or bias (§0.2, §1.1) and names local/sliding-window attention and ALiBi-style bias
among the variants a tiled kernel executes (§3.5, §4.2) without fixing their formulas. Readings
(also in the design notes): a window (left, right) keeps keys i - left <= j <= i + right (negative:
unbounded), on top of the causal rule; ALiBi adds -m |i - j| with one slope m per query head; B is
added to the scaled scores. Each is pinned by brute force in scalar Python, by closed forms, and by
the cases that reduce to plain attention; plausible mistakes (a window bound off by one, the ALiBi
sign flipped, the bias added before scaling) must fail a pin.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import attention_ext, attention_head

RNG = np.random.default_rng(9090)


def _brute(q, k, v, scale, causal, window, slope, bias):
    N, dv = k.shape[0], v.shape[1]
    o = np.zeros((q.shape[0], dv))
    lse = np.zeros(q.shape[0])
    for i in range(q.shape[0]):
        s = []
        for j in range(N):
            ok = (not causal or j <= i)
            if window is not None:
                if window[0] >= 0 and j < i - window[0]:
                    ok = False
                if window[1] >= 0 and j > i + window[1]:
                    ok = False
            if not ok:
                continue
            x = scale * math.fsum(q[i, t] * k[j, t] for t in range(q.shape[1]))
            if bias is not None:
                x += bias[i, j]
            if slope is not None:
                x -= slope * abs(i - j)
            s.append((j, x))
        m = max(x for _, x in s)
        w = [(j, math.exp(x - m)) for j, x in s]
        tot = math.fsum(e for _, e in w)
        for c in range(dv):
            o[i, c] = math.fsum(e * v[j, c] for j, e in w) / tot
        lse[i] = m + math.log(tot)
    return o, lse


def pin_brute_force(fn):
    N, d = 9, 3
    q, k, v = (RNG.standard_normal((N, d)) for _ in range(3))
    bias = RNG.standard_normal((N, N))
    cases = [((2, 1), None, None), ((0, 0), None, None), ((3, -1), 0.3, None), ((-1, 2), None, bias),
             ((4, 4), 0.7, bias), (None, 0.5, None), (None, None, bias), ((1, 5), None, None)]
    for causal in (False, True):
        for window, slope, b in cases:
            o, lse = fn(q, k, v, 0.8, causal, window, slope, b)
            ob, lb = _brute(q, k, v, 0.8, causal, window, slope, b)
            np.testing.assert_allclose(o, ob, atol=1e-12)
            np.testing.assert_allclose(lse, lb, atol=1e-12)


def pin_closed_forms(fn):
    N, d = 8, 4
    q, k, v = (RNG.standard_normal((N, d)) for _ in range(3))
    # a window of one key (causal, left 0): each query sees only itself
    o, lse = fn(q, k, v, 0.6, True, (0, 0), None, None)
    np.testing.assert_allclose(o, v, atol=1e-12)
    np.testing.assert_allclose(lse, 0.6 * (q * k).sum(axis=1), atol=1e-12)
    # identical keys: uniform weights over the window -> mean of V over it
    kk = np.repeat(RNG.standard_normal((1, d)), N, axis=0)
    o, _ = fn(q, kk, v, 0.6, False, (2, 1), None, None)
    for i in range(N):
        np.testing.assert_allclose(o[i], v[max(0, i - 2):min(N, i + 2)].mean(axis=0), atol=1e-12)
    # identical keys, causal ALiBi: weights e^{-m t}, t = i - j: O_i = sum_t e^{-m t} V_{i-t} / Z,
    # LSE_i = s + ln Z with Z = (1 - e^{-m (i+1)}) / (1 - e^{-m})
    m = 0.4
    o, lse = fn(q, kk, v, 0.6, True, None, m, None)
    for i in range(N):
        w = np.exp(-m * (i - np.arange(i + 1)))
        np.testing.assert_allclose(o[i], (w[:, None] * v[:i + 1]).sum(axis=0) / w.sum(), atol=1e-12)
        z = (1 - math.exp(-m * (i + 1))) / (1 - math.exp(-m))
        np.testing.assert_allclose(lse[i], 0.6 * float(q[i] @ kk[0]) + math.log(z), atol=1e-12)
    # a constant bias c leaves O and shifts LSE by c
    o0, l0 = fn(q, k, v, 0.6, True, None, None, None)
    o1, l1 = fn(q, k, v, 0.6, True, None, None, np.full((N, N), 2.5))
    np.testing.assert_allclose(o1, o0, atol=1e-12)
    np.testing.assert_allclose(l1, l0 + 2.5, atol=1e-12)


def pin_reductions(fn):
    N, d = 10, 3
    q, k, v = (RNG.standard_normal((N, d)) for _ in range(3))
    for causal in (False, True):
        ref = attention_head(q, k, v, 0.9, causal)
        for window, slope, b in [((-1, -1), None, None), ((N, N), None, None), (None, 0.0, None),
                                 (None, None, np.zeros((N, N)))]:
            o, lse = fn(q, k, v, 0.9, causal, window, slope, b)
            np.testing.assert_allclose(o, ref[0], atol=1e-12)
            np.testing.assert_allclose(lse, ref[1], atol=1e-12)
    # a -inf bias above the diagonal is the causal mask; a window (N, 0) is too
    mask = np.where(np.arange(N)[None, :] > np.arange(N)[:, None], -np.inf, 0.0)
    ref = attention_head(q, k, v, 0.9, True)
    for window, b in [(None, mask), ((N, 0), None)]:
        o, lse = fn(q, k, v, 0.9, False, window, None, b)
        np.testing.assert_allclose(o, ref[0], atol=1e-12)
        np.testing.assert_allclose(lse, ref[1], atol=1e-12)


def _oracle(q, k, v, scale, causal, window, slope, bias):
    return attention_head(q, k, v, scale, causal, window=window, alibi_slope=slope, bias=bias)


def _all(fn):
    pin_brute_force(fn)
    pin_closed_forms(fn)
    pin_reductions(fn)


def test_variant_oracle_passes_pins():
    _all(_oracle)


def test_batched_form_matches_heads_and_broadcasts_bias():
    B, H, H_kv, N, d = 2, 4, 2, 7, 3
    q = RNG.standard_normal((B, H, N, d))
    k = RNG.standard_normal((B, H_kv, N, d))
    v = RNG.standard_normal((B, H_kv, N, d))
    slopes = [0.1, 0.2, 0.3, 0.4]
    bias = RNG.standard_normal((1, H, N, N))
    o, lse = attention_ext(q, k, v, 0.5, True, (3, -1), slopes, bias)
    for b in range(B):
        for h in range(H):
            j = oracle.kv_head_of(h, H, H_kv)
            ro, rl = attention_head(q[b, h], k[b, j], v[b, j], 0.5, True, window=(3, -1),
                                    alibi_slope=slopes[h], bias=bias[0, h])
            np.testing.assert_array_equal(o[b, h], ro)
            np.testing.assert_array_equal(lse[b, h], rl)


def _mutant(kind):
    def fn(q, k, v, scale, causal, window, slope, bias):
        N = k.shape[0]
        i = np.arange(q.shape[0])[:, None]
        j = np.arange(N)[None, :]
        s = (q @ k.T) * scale
        if bias is not None:
            s = (q @ k.T + bias) * scale if kind == "bias_before_scale" else s + bias
        if slope is not None:
            s = s + slope * np.abs(i - j) if kind == "alibi_sign" else s - slope * np.abs(i - j)
        vis = np.ones(s.shape, bool)
        if causal:
            vis &= j <= i
        if window is not None:
            if window[0] >= 0:
                vis &= (j > i - window[0]) if kind == "window_off_by_one" else (j >= i - window[0])
            if window[1] >= 0:
                vis &= j <= i + window[1]
        s = np.where(vis, s, -np.inf)
        m = s.max(axis=1)
        e = np.exp(s - m[:, None])
        return (e / e.sum(axis=1)[:, None]) @ v, m + np.log(e.sum(axis=1))
    return fn


@pytest.mark.parametrize("kind", ["alibi_sign", "window_off_by_one", "bias_before_scale"])
def test_mutants_fail_a_pin(kind):
    with pytest.raises(AssertionError):
        _all(_mutant(kind))


def test_mutant_harness_is_sound():
    # the mutant template without a mutation passes, so the failures above are the mutations
    _all(_mutant("none"))

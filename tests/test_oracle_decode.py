"""Pins for the decoding oracle (oracle.attention_decode), on the CPU.

Few queries against a longer key/value sequence ("FlashAttention-2 -- Deeper Math", "What FA-2 does
not fix"); the queries are the last N_q tokens, so with a causal mask query i sees keys
j <= N_kv - N_q + i. The pins: a closed form whose value depends on exactly which keys a query sees,
brute force in scalar Python, the N_q = N_kv case (ordinary self-attention, pinned elsewhere), and
the method the GPU uses -- split the keys, keep per split (O_s, LSE_s), merge with the blockwise
recurrence of "Understanding FlashAttention Pt 1", §2.4 -- which must reproduce the dense result.
A wrong query alignment must fail them.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import attention_decode, attention_head, kv_head_of

RNG = np.random.default_rng(777)


def pin_identical_keys(fn):
    """All keys of a K/V head equal: weights are uniform over the visible keys, so
    O_i = mean(V[0 .. last visible]) and LSE_i = s + ln(#visible)."""
    B, H, H_kv, Nq, Nkv, d = 1, 4, 2, 3, 9, 4
    q = RNG.standard_normal((B, H, Nq, d))
    k = np.repeat(RNG.standard_normal((B, H_kv, 1, d)), Nkv, axis=2)
    v = RNG.standard_normal((B, H_kv, Nkv, d))
    for causal in (False, True):
        o, lse = fn(q, k, v, 0.6, causal)
        for h in range(H):
            j = h // (H // H_kv)
            for i in range(Nq):
                n = (Nkv - Nq + i + 1) if causal else Nkv
                np.testing.assert_allclose(o[0, h, i], v[0, j, :n].mean(axis=0), atol=1e-12)
                s = 0.6 * float(q[0, h, i] @ k[0, j, 0])
                np.testing.assert_allclose(lse[0, h, i], s + math.log(n), atol=1e-12)


def _brute(q, k, v, scale, causal):
    B, H, Nq, d = q.shape
    H_kv, Nkv = k.shape[1], k.shape[2]
    o = np.zeros((B, H, Nq, v.shape[3]))
    lse = np.zeros((B, H, Nq))
    for b in range(B):
        for h in range(H):
            j = (h * H_kv) // H
            for i in range(Nq):
                last = Nkv - Nq + i if causal else Nkv - 1
                s = [scale * math.fsum(q[b, h, i, t] * k[b, j, n, t] for t in range(d))
                     for n in range(last + 1)]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                tot = math.fsum(e)
                for c in range(v.shape[3]):
                    o[b, h, i, c] = math.fsum(e[n] * v[b, j, n, c] for n in range(len(e))) / tot
                lse[b, h, i] = m + math.log(tot)
    return o, lse


def pin_brute_force(fn):
    for (B, H, H_kv, Nq, Nkv, d) in [(1, 2, 1, 1, 7, 3), (2, 4, 2, 2, 5, 2), (1, 3, 3, 3, 3, 2)]:
        q = RNG.standard_normal((B, H, Nq, d))
        k = RNG.standard_normal((B, H_kv, Nkv, d))
        v = RNG.standard_normal((B, H_kv, Nkv, d))
        for causal in (False, True):
            o, lse = fn(q, k, v, 0.8, causal)
            ob, lb = _brute(q, k, v, 0.8, causal)
            np.testing.assert_allclose(o, ob, atol=1e-12)
            np.testing.assert_allclose(lse, lb, atol=1e-12)


def _all_pins(fn):
    pin_identical_keys(fn)
    pin_brute_force(fn)


def test_decode_oracle_passes_pins():
    _all_pins(attention_decode)


def test_square_case_is_self_attention():
    q, k, v = (RNG.standard_normal((1, 2, 6, 3)) for _ in range(3))
    for causal in (False, True):
        o1, l1 = attention_decode(q, k, v, 0.5, causal)
        o2, l2 = oracle.attention(q, k, v, 0.5, causal)
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)


def _split_merge(q, k, v, scale, causal, bounds):
    """The GPU's method, written with the oracle as the per-split step: per key split s a partial
    (O_s, LSE_s) over the split's visible keys (O_s = 0, LSE_s = -inf if none), merged with
    LSE = M + ln sum_s e^{LSE_s - M}, O = sum_s e^{LSE_s - LSE} O_s."""
    B, H, Nq, d = q.shape
    H_kv, Nkv = k.shape[1], k.shape[2]
    o = np.zeros((B, H, Nq, v.shape[3]))
    lse = np.zeros((B, H, Nq))
    for b in range(B):
        for h in range(H):
            j = kv_head_of(h, H, H_kv)
            for i in range(Nq):
                last = Nkv - Nq + i if causal else Nkv - 1
                parts = []
                for lo, hi in zip(bounds[:-1], bounds[1:]):
                    top = min(hi, last + 1)
                    if top <= lo:
                        parts.append((np.zeros(v.shape[3]), -np.inf))
                        continue
                    po, pl = attention_head(q[b, h, i:i + 1], k[b, j, lo:top], v[b, j, lo:top], scale)
                    parts.append((po[0], pl[0]))
                M = max(p[1] for p in parts)
                w = np.array([0.0 if p[1] == -np.inf else math.exp(p[1] - M) for p in parts])
                lse[b, h, i] = M + math.log(w.sum())
                o[b, h, i] = sum(wi * p[0] for wi, p in zip(w, parts)) / w.sum()
    return o, lse


@pytest.mark.parametrize("bounds", [[0, 50], [0, 13, 50], [0, 7, 20, 21, 44, 50], list(range(0, 51, 5))])
def test_split_and_merge_reproduces_dense(bounds):
    q = RNG.standard_normal((1, 4, 3, 5))
    k = RNG.standard_normal((1, 2, 50, 5)) * 2.0
    v = RNG.standard_normal((1, 2, 50, 5))
    for causal in (False, True):
        o, lse = attention_decode(q, k, v, 0.7, causal)
        o2, l2 = _split_merge(q, k, v, 0.7, causal, bounds)
        np.testing.assert_allclose(o2, o, atol=1e-12)
        np.testing.assert_allclose(l2, lse, atol=1e-12)


def test_causal_needs_queries_within_keys():
    q = RNG.standard_normal((1, 1, 5, 2))
    k = RNG.standard_normal((1, 1, 4, 2))
    with pytest.raises(ValueError):
        attention_decode(q, k, k, 1.0, True)
    attention_decode(q, k, k, 1.0, False)  # without a mask any N_q is fine


def _mutant_offset(offset_fn):
    def fn(q, k, v, scale, causal):
        B, H, Nq = q.shape[:3]
        H_kv, Nkv = k.shape[1], k.shape[2]
        o = np.empty((B, H, Nq, v.shape[3]))
        lse = np.empty((B, H, Nq))
        for b in range(B):
            for h in range(H):
                j = kv_head_of(h, H, H_kv)
                o[b, h], lse[b, h] = attention_head(q[b, h], k[b, j], v[b, j], scale, causal,
                                                    query_offset=offset_fn(Nq, Nkv))
        return o, lse
    return fn


@pytest.mark.parametrize("name,off", [("top_left", lambda nq, nkv: 0),
                                      ("off_by_one", lambda nq, nkv: nkv - nq - 1)])
def test_wrong_alignment_fails_a_pin(name, off):
    with pytest.raises(AssertionError):
        _all_pins(_mutant_offset(off))

"""Pins for the CPU float64 oracle (oracle/attention.py), all on the CPU.

Each pin ties the oracle to something other than itself: values printed on the pages, closed
forms, invariants that hold for any input, brute force in scalar Python, and float64 library
routines. ``test_mutants_are_caught`` plants plausible mistakes in copies of the oracle and shows
that every one of them fails at least one pin.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention, attention_head

RNG = np.random.default_rng(20240601)


def _rand(n, d, dv=None, scale=1.0):
    dv = d if dv is None else dv
    return (RNG.standard_normal((n, d)) * scale, RNG.standard_normal((n, d)) * scale,
            RNG.standard_normal((n, dv)))


def _golden(golden_dir):
    with open(os.path.join(golden_dir, "worked_example.json")) as f:
        return json.load(f)


# ---------------------------------------------------------------------------------------------
# Pin functions. Each takes an attention_head-like callable fn(q, k, v, scale, causal, ...) and
# raises AssertionError (or any exception) when the callable is wrong.
# ---------------------------------------------------------------------------------------------

def pin_worked_example(fn, g):
    """Handbook §2.5: one already-scaled row s = [2, 1, 4, 3] and 2-D values."""
    s = np.array(g["scores"])
    v = np.array(g["values"])
    q = np.array([[1.0, 0.0]])
    k = np.stack([s, np.zeros_like(s)], axis=1)  # q . k_j = s_j
    o, lse = fn(q, k, v, 1.0, False)
    pr = g["printed"]
    tol8 = 0.5e-8 + 1e-12
    np.testing.assert_allclose(o[0], pr["O"]["value"], rtol=0, atol=tol8)
    # LSE = m + ln(l) with the printed l (its 8-digit rounding moves ln l by < 4e-9).
    assert abs(lse[0] - (4.0 + math.log(pr["ell"]["value"]))) < 4e-9
    # the printed unnormalised weights e^(s - m), m = 4
    w = np.exp(s - lse[0]) * pr["ell"]["value"]
    np.testing.assert_allclose(w, pr["weights"]["value"], rtol=0, atol=0.5e-6 + 1e-8)


def pin_overflow(fn, g):
    """Handbook §2.2: x = [1000, 999] must not overflow; weights are [1, e^-1] / (1 + e^-1)."""
    ex = g["overflow_example"]
    q = np.array([[1.0]])
    k = np.array([[ex["x"][0]], [ex["x"][1]]])
    v = np.array([[1.0, 0.0], [0.0, 1.0]])  # O equals the weight vector
    o, lse = fn(q, k, v, 1.0, False)
    e1 = math.exp(-1.0)
    assert abs(e1 - ex["e_minus_1_printed"]["value"]) < 0.5e-3
    np.testing.assert_allclose(o[0], [1.0 / (1.0 + e1), e1 / (1.0 + e1)], rtol=0, atol=1e-15)
    assert abs(lse[0] - (1000.0 + math.log1p(e1))) < 1e-12


def pin_identical_keys(fn):
    """All keys equal: every visible score of a row is the same, so P is uniform over them."""
    n, d = 13, 5
    q, k, v = _rand(n, d)
    k[:] = k[3]
    sc = 0.37
    o, lse = fn(q, k, v, sc, False)
    s = sc * (q @ k[0])
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, s + math.log(n), rtol=0, atol=1e-13)
    o, lse = fn(q, k, v, sc, True)
    for i in range(n):
        np.testing.assert_allclose(o[i], v[: i + 1].mean(axis=0), rtol=0, atol=1e-13)
        assert abs(lse[i] - (s[i] + math.log(i + 1))) < 1e-13


def pin_zero_scale(fn):
    """scale = 0: every visible score is 0, O is the mean of the visible values, LSE = ln(#visible)."""
    n, d = 11, 4
    q, k, v = _rand(n, d)
    o, lse = fn(q, k, v, 0.0, False)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, math.log(n), rtol=0, atol=1e-13)
    o, lse = fn(q, k, v, 0.0, True)
    for i in range(n):
        np.testing.assert_allclose(o[i], v[: i + 1].mean(axis=0), rtol=0, atol=1e-13)
        assert abs(lse[i] - math.log(i + 1)) < 1e-13


def pin_constant_values(fn):
    """V rows all equal to c: O = c for any scores."""
    n, d = 9, 6
    q, k, v = _rand(n, d, scale=3.0)
    v[:] = np.linspace(-2, 2, d)
    for causal in (False, True):
        o, _ = fn(q, k, v, 0.5, causal)
        np.testing.assert_allclose(o, v, rtol=0, atol=1e-13)


def pin_causal_first_row_and_single_key(fn):
    """Causal row 0 sees only key 0; N = 1 sees only itself: O = V_0, LSE = scale q.k_0."""
    n, d = 7, 3
    q, k, v = _rand(n, d)
    sc = 0.8
    o, lse = fn(q, k, v, sc, True)
    np.testing.assert_allclose(o[0], v[0], rtol=0, atol=1e-15)
    assert abs(lse[0] - sc * (q[0] @ k[0])) < 1e-14
    for causal in (False, True):
        o, lse = fn(q[:1], k[:1], v[:1], sc, causal)
        np.testing.assert_allclose(o[0], v[0], rtol=0, atol=1e-15)
        assert abs(lse[0] - sc * (q[0] @ k[0])) < 1e-14


def pin_two_keys(fn):
    """N = 2, no mask: O = sigmoid(s1 - s2) v1 + sigmoid(s2 - s1) v2, LSE = log(e^s1 + e^s2)."""
    q, k, v = _rand(2, 4)
    sc = 0.9
    o, lse = fn(q, k, v, sc, False)
    for i in range(2):
        s1, s2 = sc * (q[i] @ k[0]), sc * (q[i] @ k[1])
        sig = 1.0 / (1.0 + math.exp(-(s1 - s2)))
        np.testing.assert_allclose(o[i], sig * v[0] + (1.0 - sig) * v[1], rtol=0, atol=1e-14)
        hi = max(s1, s2)
        assert abs(lse[i] - (hi + math.log(math.exp(s1 - hi) + math.exp(s2 - hi)))) < 1e-14


def _brute(q, k, v, scale, causal):
    """Scalar Python: scores one at a time, math.exp and math.fsum, no numpy arithmetic."""
    q, k, v = q.tolist(), k.tolist(), v.tolist()
    n_q, n_k, dv = len(q), len(k), len(v[0])
    out, lse = [], []
    for i in range(n_q):
        vis = [j for j in range(n_k) if (not causal) or j <= i]
        s = [scale * math.fsum(q[i][t] * k[j][t] for t in range(len(q[i]))) for j in vis]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        ell = math.fsum(e)
        out.append([math.fsum(e[a] * v[j][c] for a, j in enumerate(vis)) / ell for c in range(dv)])
        lse.append(m + math.log(ell))
    return np.array(out), np.array(lse)


def pin_brute_force(fn):
    """Toy shape of the tokentrails card (8 tokens, d = 4) and a few others, both masks."""
    for n, d, dv in ((8, 4, 4), (5, 3, 2), (1, 4, 4), (8, 4, 7)):
        q, k, v = _rand(n, d, dv, scale=1.5)
        for causal in (False, True):
            o, lse = fn(q, k, v, 0.5, causal)
            ob, lb = _brute(q, k, v, 0.5, causal)
            np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-12)


def pin_torch_float64(fn):
    """float64 CPU torch: softmax, logsumexp and scaled_dot_product_attention."""
    n, d = 37, 16
    q, k, v = _rand(n, d, scale=2.0)
    sc = 1.0 / math.sqrt(d)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    for causal in (False, True):
        o, lse = fn(q, k, v, sc, causal)
        s = sc * (tq @ tk.T)
        if causal:
            s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
        np.testing.assert_allclose(o, (torch.softmax(s, dim=-1) @ tv).numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)
        sdpa = torch.nn.functional.scaled_dot_product_attention(
            tq[None, None], tk[None, None], tv[None, None], is_causal=causal, scale=sc)[0, 0]
        np.testing.assert_allclose(o, sdpa.numpy(), rtol=0, atol=1e-12)


PINS_NO_GOLDEN = [pin_identical_keys, pin_zero_scale, pin_constant_values,
                  pin_causal_first_row_and_single_key, pin_two_keys, pin_brute_force,
                  pin_torch_float64]


# ---------------------------------------------------------------------------------------------
# The oracle passes every pin.
# ---------------------------------------------------------------------------------------------

def test_worked_example(golden_dir):
    pin_worked_example(attention_head, _golden(golden_dir))


def test_overflow_example(golden_dir):
    pin_overflow(attention_head, _golden(golden_dir))


@pytest.mark.parametrize("pin", PINS_NO_GOLDEN, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(attention_head)


@pytest.mark.parametrize("causal", [False, True])
def test_invariants(causal):
    """Rows of P sum to 1, P >= 0 and is 0 where masked, O lies between the min and max of the
    visible values per column, and max S <= LSE <= max S + ln(#visible)."""
    n, d = 64, 8
    q, k, v = _rand(n, d, scale=2.0)
    o, lse, s, p = attention_head(q, k, v, 0.7, causal, return_sp=True)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert (p >= 0).all()
    if causal:
        assert (p[np.triu_indices(n, 1)] == 0).all()
    for i in range(n):
        vis = np.arange(n) if not causal else np.arange(i + 1)
        assert (o[i] >= v[vis].min(axis=0) - 1e-12).all() and (o[i] <= v[vis].max(axis=0) + 1e-12).all()
        smax = s[i, vis].max()
        assert smax - 1e-12 <= lse[i] <= smax + math.log(len(vis)) + 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_shift_invariance(causal):
    """Adding u to every key row leaves O unchanged and moves LSE_i by scale * q_i . u."""
    n, d = 40, 8
    q, k, v = _rand(n, d)
    u = RNG.standard_normal(d)
    sc = 0.6
    o1, l1 = attention_head(q, k, v, sc, causal)
    o2, l2 = attention_head(q, k + u, v, sc, causal)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l1 + sc * (q @ u), rtol=0, atol=1e-12)


def test_permutation_equivariance():
    """Without a mask, permuting keys with their values changes nothing; permuting queries
    permutes the output rows."""
    n, d = 30, 8
    q, k, v = _rand(n, d)
    o, lse = attention_head(q, k, v, 0.5, False)
    pk = RNG.permutation(n)
    o2, l2 = attention_head(q, k[pk], v[pk], 0.5, False)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, lse, rtol=0, atol=1e-12)
    pq = RNG.permutation(n)
    o3, l3 = attention_head(q[pq], k, v, 0.5, False)
    np.testing.assert_allclose(o3, o[pq], rtol=0, atol=1e-12)
    np.testing.assert_allclose(l3, lse[pq], rtol=0, atol=1e-12)


def test_rows_subset_matches_full():
    """Evaluating a subset of query rows gives exactly those rows of the full result."""
    n, d = 50, 8
    q, k, v = _rand(n, d)
    rows = np.array([0, 7, 8, 31, 49])
    for causal in (False, True):
        o, lse = attention_head(q, k, v, 0.4, causal)
        o2, l2 = attention_head(q, k, v, 0.4, causal, rows=rows)
        np.testing.assert_array_equal(o2, o[rows])
        np.testing.assert_array_equal(l2, lse[rows])


def test_batched_wrapper_matches_heads():
    B, H, n, d = 2, 3, 17, 8
    q = RNG.standard_normal((B, H, n, d))
    k = RNG.standard_normal((B, H, n, d))
    v = RNG.standard_normal((B, H, n, d))
    o, lse = attention(q, k, v, 0.3, True)
    for b in range(B):
        for h in range(H):
            oh, lh = attention_head(q[b, h], k[b, h], v[b, h], 0.3, True)
            np.testing.assert_array_equal(o[b, h], oh)
            np.testing.assert_array_equal(lse[b, h], lh)
    rows = np.tile(np.array([0, 5, 16]), (B, H, 1))
    o2, l2 = attention(q, k, v, 0.3, True, rows=rows)
    np.testing.assert_array_equal(o2, o[:, :, [0, 5, 16]])
    np.testing.assert_array_equal(l2, lse[:, :, [0, 5, 16]])


def test_bf16_inputs_are_upcast_exactly():
    """The oracle sees exactly the bf16 values the GPU receives (upcast is exact)."""
    t = torch.randn(8, 4).to(torch.bfloat16)
    a = t.float().numpy().astype(np.float64)
    assert np.array_equal(a.astype(np.float32), t.float().numpy())


# ---------------------------------------------------------------------------------------------
# Mutants: plausible mistakes, each of which must fail at least one pin.
# ---------------------------------------------------------------------------------------------

def _mk(variant):
    def fn(q, k, v, scale, causal=False, rows=None, return_sp=False):
        q = np.asarray(q, dtype=np.float64)
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        n = q.shape[0]
        sc = 1.0 if variant == "no_scale" else scale
        s = sc * (q @ k.T)
        if causal:
            i = np.arange(n)[:, None]
            j = np.arange(k.shape[0])[None, :]
            vis = {"strict_mask": j < i, "flipped_mask": j >= i}.get(variant, j <= i)
            s = np.where(vis, s, -np.inf)
        if variant == "no_max":
            m = np.zeros(n)
        else:
            m = s.max(axis=1)
        e = np.exp(s - m[:, None])
        axis = 0 if variant == "wrong_axis" else 1
        ell = e.sum(axis=axis)
        if variant == "normalise_by_max":
            ell = e.max(axis=1)
        p = e / (ell[:, None] if axis == 1 else ell[None, :])
        o = (p.T @ v) if variant == "transposed_p" else (p @ v)
        if variant == "lse_log2":
            lse = m + np.log2(ell)
        elif variant == "lse_no_log":
            lse = m + ell
        elif variant == "lse_no_max":
            lse = np.log(ell)
        else:
            lse = m + np.log(ell)
        if variant == "v_off_by_one":
            o = p @ np.roll(v, 1, axis=0)
        return o, lse
    return fn


MUTANTS = ["no_scale", "strict_mask", "flipped_mask", "no_max", "wrong_axis", "normalise_by_max",
           "transposed_p", "lse_log2", "lse_no_log", "lse_no_max", "v_off_by_one"]


@pytest.mark.parametrize("variant", MUTANTS)
def test_mutants_are_caught(variant, golden_dir):
    g = _golden(golden_dir)
    fn = _mk(variant)
    pins = [lambda f: pin_worked_example(f, g), lambda f: pin_overflow(f, g)] + PINS_NO_GOLDEN
    failed = 0
    for pin in pins:
        try:
            with np.errstate(all="ignore"):
                pin(fn)
        except Exception:
            failed += 1
    assert failed >= 1, f"mutant {variant} passed every pin"


def test_unmutated_copy_passes(golden_dir):
    """The mutant factory with no mutation is a correct attention and passes every pin, so the
    mutant results above come from the planted mistakes alone."""
    g = _golden(golden_dir)
    fn = _mk("none")
    pin_worked_example(fn, g)
    pin_overflow(fn, g)
    for pin in PINS_NO_GOLDEN:
        pin(fn)

"""Pins for the backward oracle (oracle.attention_backward_head / attention_backward), on the CPU.

The oracle writes out the gradient formulas of "Understanding FlashAttention Pt 1", §3.6. They are
pinned here to things that do not use those formulas:
  * central finite differences of sum(dO * O) through the forward oracle (itself pinned to the
    pages' worked example, closed forms and brute force), per head, with and without the causal
    mask, and through the grouped-head forward for shared K/V heads;
  * torch autograd (float64, CPU) through a forward written with torch's own softmax;
  * closed forms: scale 0 (uniform weights: dQ = dK = 0, dV_j = sum over the queries that see key
    j of dO_i / (number of keys query i sees)) and a single key (O = V: dV = dO, dQ = dK = 0);
  * the row identity of §3.6, sum_r dO_ir O_ir = sum_j P_ij dP_ij, checked on the forward oracle.
Plausible mistakes (the D term dropped, its sign flipped, the scale left out, dS used untransposed
for dK, D taken over columns) must each fail a pin.
"""
import numpy as np
import pytest
import torch

from oracle import attention_backward, attention_backward_head, attention_gqa, attention_head

RNG = np.random.default_rng(4242)


def _loss(q, k, v, do, scale, causal):
    o, _ = attention_head(q, k, v, scale, causal)
    return float((o * do).sum())


def _fd_grads(q, k, v, do, scale, causal, h=1e-5):
    grads = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        x = args[which]
        g = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(*args, do, scale, causal)
            x[idx] = old - h
            lm = _loss(*args, do, scale, causal)
            x[idx] = old
            g[idx] = (lp - lm) / (2 * h)
        grads.append(g)
    return grads


def pin_finite_differences(fn):
    for (N, d, dv) in [(5, 3, 3), (6, 4, 2), (1, 3, 3)]:
        q, k = RNG.standard_normal((N, d)), RNG.standard_normal((N, d))
        v, do = RNG.standard_normal((N, dv)), RNG.standard_normal((N, dv))
        for causal in (False, True):
            for scale in (0.7, 1.3):
                got = fn(q, k, v, do, scale, causal)
                ref = _fd_grads(q, k, v, do, scale, causal)
                for g, r in zip(got, ref):
                    np.testing.assert_allclose(g, r, atol=2e-8)


def pin_autograd(fn):
    N, d = 9, 5
    q, k, v, do = (RNG.standard_normal((N, d)) for _ in range(4))
    for causal in (False, True):
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        s = 0.4 * tq @ tk.T
        if causal:
            s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
        o = torch.softmax(s, dim=1) @ tv
        (o * torch.tensor(do)).sum().backward()
        got = fn(q, k, v, do, 0.4, causal)
        for g, t in zip(got, (tq, tk, tv)):
            np.testing.assert_allclose(g, t.grad.numpy(), atol=1e-12)


def pin_closed_forms(fn):
    N, d = 7, 3
    q, k, v, do = (RNG.standard_normal((N, d)) for _ in range(4))
    for causal in (False, True):
        dq, dk, dv = fn(q, k, v, do, 0.0, causal)
        np.testing.assert_allclose(dq, 0.0, atol=1e-15)
        np.testing.assert_allclose(dk, 0.0, atol=1e-15)
        ref = np.zeros_like(v)
        for i in range(N):
            n = i + 1 if causal else N
            ref[:n] += do[i] / n
        np.testing.assert_allclose(dv, ref, atol=1e-14)
    q1, k1, v1, do1 = (RNG.standard_normal((1, d)) for _ in range(4))
    dq, dk, dv = fn(q1, k1, v1, do1, 0.9, False)
    np.testing.assert_allclose(dv, do1, atol=1e-15)
    np.testing.assert_allclose(dq, 0.0, atol=1e-15)
    np.testing.assert_allclose(dk, 0.0, atol=1e-15)


def _all_pins(fn):
    pin_closed_forms(fn)
    pin_autograd(fn)
    pin_finite_differences(fn)


def test_backward_oracle_passes_pins():
    _all_pins(attention_backward_head)


def test_row_identity_of_the_pages():
    # sum_r dO_ir O_ir = sum_j P_ij dP_ij, with O and P from the forward oracle
    N, d = 8, 4
    q, k, v, do = (RNG.standard_normal((N, d)) for _ in range(4))
    for causal in (False, True):
        o, _, _, p = attention_head(q, k, v, 0.5, causal, return_sp=True)
        np.testing.assert_allclose((do * o).sum(axis=1), (p * (do @ v.T)).sum(axis=1), atol=1e-13)


def test_grouped_heads_by_finite_differences():
    # Shared K/V heads: dK and dV of a K/V head sum over its query heads. Finite differences of
    # sum(dO * O) through the grouped-head forward oracle.
    B, H, H_kv, N, d = 1, 4, 2, 4, 3
    q = RNG.standard_normal((B, H, N, d))
    k = RNG.standard_normal((B, H_kv, N, d))
    v = RNG.standard_normal((B, H_kv, N, d))
    do = RNG.standard_normal((B, H, N, d))
    for causal in (False, True):
        dq, dk, dv = attention_backward(q, k, v, do, 0.8, causal)

        def loss(q_, k_, v_):
            o, _ = attention_gqa(q_, k_, v_, 0.8, causal)
            return float((o * do).sum())

        for x, g in ((q, dq), (k, dk), (v, dv)):
            for idx in np.ndindex(*x.shape):
                old = x[idx]
                x[idx] = old + 1e-5
                lp = loss(q, k, v)
                x[idx] = old - 1e-5
                lm = loss(q, k, v)
                x[idx] = old
                assert abs((lp - lm) / 2e-5 - g[idx]) < 2e-8


def _mutant(kind):
    def fn(q, k, v, do, scale, causal):
        from oracle import dense_scores
        s = dense_scores(q, k, scale, causal, np.arange(q.shape[0]))
        e = np.exp(s - s.max(axis=1)[:, None])
        p = e / e.sum(axis=1)[:, None]
        dv = p.T @ do
        dp = do @ v.T
        dr = (p * dp).sum(axis=0 if kind == "d_over_columns" else 1)
        if kind == "no_d":
            ds = p * dp
        elif kind == "d_sign":
            ds = p * (dp + dr[:, None])
        else:
            ds = p * (dp - dr[:, None])
        sc = 1.0 if kind == "no_scale" else scale
        dq = sc * (ds @ k)
        dk = scale * ((ds if kind == "untransposed" else ds.T) @ q)
        return dq, dk, dv
    return fn


@pytest.mark.parametrize("kind", ["no_d", "d_sign", "no_scale", "untransposed", "d_over_columns"])
def test_mutants_fail_a_pin(kind):
    with pytest.raises(AssertionError):
        _all_pins(_mutant(kind))

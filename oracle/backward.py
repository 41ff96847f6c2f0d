"""Dense CPU float64 attention backward: the gradients the tiled GPU backward must reproduce.

TEST INFRASTRUCTURE ONLY -- imported by tests, the smoke check and the bench's cpu_baseline leg,
never by the product path.

For one (batch, head) with S = scale * Q K^T (future keys -> -inf when causal), P = softmax_rows(S),
O = P V and an upstream gradient dO, the gradients of sum(dO * O) are ("Understanding FlashAttention
Pt 1", §3.6, written there for scale = 1/sqrt(d); "Online Softmax & FlashAttention", §26.4):

    dV = P^T dO
    dP = dO V^T
    D_i = sum_j P_ij dP_ij                (= sum_r dO_ir O_ir, the identity of the same section)
    dS = P * (dP - D[:, None])            (masked entries have P = 0, so they contribute nothing)
    dQ = scale * dS K
    dK = scale * dS^T Q

P is materialised from the dense softmax, not rebuilt from a saved logsumexp: the plain definition,
which the tiled kernels reach (FA-2 page, Fix 2: P_ij = exp(S_ij - L_i)) up to rounding.

Grouped K/V heads ("Understanding FlashAttention Pt 1", §4.1): a K/V head used by several query
heads receives the sum of their dK and dV (the chain rule through the shared tensor).
"""
import numpy as np

from .attention import dense_scores, kv_head_of


def attention_backward_head(q, k, v, do, scale, causal=False):
    """Gradients (dQ [N, d], dK [N, d], dV [N, dv]) of sum(dO * O) for one head, in float64.

    q: [N, d], k: [N, d], v: [N, dv], do: [N, dv]; any float dtype (upcast to float64).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    s = dense_scores(q, k, scale, causal, np.arange(q.shape[0]))
    m = s.max(axis=1)
    if not np.all(np.isfinite(m)):
        raise ValueError("a query row has no visible key; its softmax is undefined")
    e = np.exp(s - m[:, None])
    p = e / e.sum(axis=1)[:, None]
    dv = p.T @ do
    dp = do @ v.T
    d_row = (p * dp).sum(axis=1)
    ds = p * (dp - d_row[:, None])
    dq = float(scale) * (ds @ k)
    dk = float(scale) * (ds.T @ q)
    return dq, dk, dv


def attention_backward(q, k, v, do, scale, causal=False):
    """Batched gradients over [B, H, N, d] Q and dO with [B, H_kv, N, d] K and V (H a multiple of
    H_kv; H_kv = H is ordinary multi-head attention). Query head h uses K/V head
    kv_head_of(h, H, H_kv); each K/V head's dK and dV sum over the query heads that use it.
    Returns (dQ [B, H, N, d], dK [B, H_kv, N, d], dV [B, H_kv, N, dv]) in float64.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    do = np.asarray(do)
    B, H = q.shape[0], q.shape[1]
    H_kv = k.shape[1]
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            j = kv_head_of(h, H, H_kv)
            gq, gk, gv = attention_backward_head(q[b, h], k[b, j], v[b, j], do[b, h], scale, causal)
            dq[b, h] = gq
            dk[b, j] += gk
            dv[b, j] += gv
    return dq, dk, dv

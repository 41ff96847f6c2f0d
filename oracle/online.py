"""The pages' streaming recurrences in float64 -- a TEST MODEL, pinned to the dense oracle.

TEST INFRASTRUCTURE ONLY. The GPU is compared against ``oracle.attention``; this module exists so
that the tests can show, on the CPU, that the blockwise recurrence the kernel implements reaches
the dense max, sum and output for every way of cutting the keys into blocks.

online_normalizer -- (m, l) of a row that arrives in blocks: each block is reduced to its own
    (max, sum of exponentials) pair, and pairs are merged by moving both sums to the larger max;
    the merge is associative, so the pairs are combined as a balanced tree
    ("Online Softmax & FlashAttention", §26.1, Eq 26.2; handbook §2.3).
blockwise_row     -- the (m, l, a) merge for one query row: m' = max(m, max s), alpha = e^(m-m'),
    p = e^(s-m'), l' = alpha l + sum p, a' = alpha a + p^T V_b, o = a / l at the end
    ("Understanding FlashAttention Pt 1", §2.4).
tiled_attention   -- the forward pass with query blocks outermost and key blocks innermost, an
    unnormalised accumulator divided once after the last key block and the logsumexp stored per
    row ("FlashAttention-2 -- Deeper Math", Fixes 1-3), with causal tiles classified from their
    block coordinates: skipped above the diagonal, unmasked below it, masked per element only
    where they cross it (same page, "Causal masking: skip the blocks").
"""
import numpy as np


def _block_summary(s):
    """(max, sum of e^(s - max)) of one block; (-inf, 0) when no score in it is visible."""
    s = np.asarray(s, dtype=np.float64)
    if s.size == 0 or s.max() == -np.inf:
        return -np.inf, 0.0
    top = s.max()
    return top, float(np.exp(s - top).sum())


def _merge(x, y):
    """Combine two (max, sum) summaries: both sums rescaled to the larger max (Eq 26.2)."""
    (mx, lx), (my, ly) = x, y
    top = max(mx, my)
    if top == -np.inf:
        return -np.inf, 0.0
    return top, lx * np.exp(mx - top) + ly * np.exp(my - top)


def online_normalizer(blocks):
    """Return (m, l) of one score row given as a sequence of 1-D blocks.

    Every block is summarised on its own, then neighbouring summaries are merged level by level
    until one is left; the result equals the dense max and sum of e^(s - max) over the whole row.
    """
    level = [_block_summary(b) for b in blocks]
    if not level:
        return -np.inf, 0.0
    while len(level) > 1:
        nxt = [_merge(level[i], level[i + 1]) for i in range(0, len(level) - 1, 2)]
        if len(level) % 2:
            nxt.append(level[-1])
        level = nxt
    return level[0]


def blockwise_row(s, v, bounds):
    """Fold one query row through the (m, l, a) recurrence block by block.

    s: [N] scores of the row (already scaled, -inf where masked); v: [N, dv];
    bounds: list of (start, stop) key ranges covering 0..N in order.
    Returns (m, l, a, o) after the last block, plus the list of per-block states for inspection.
    """
    s = np.asarray(s, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    m = -np.inf
    ell = 0.0
    a = np.zeros(v.shape[1])
    states = []
    for start, stop in bounds:
        sb = s[start:stop]
        m_new = max(m, sb.max()) if sb.size else m
        ref = m_new if np.isfinite(m_new) else 0.0  # no visible score yet: any finite reference
        alpha = np.exp(m - ref) if np.isfinite(m) else 0.0
        p = np.exp(sb - ref)
        ell = alpha * ell + p.sum()
        a = alpha * a + p @ v[start:stop]
        m = m_new
        states.append((m, ell, a.copy()))
    return m, ell, a, a / ell, states


def tiled_attention(q, k, v, scale, causal, block_q, block_k):
    """Tiled forward pass of one head; returns (O, LSE) in float64.

    q: [N, d], k: [N, d], v: [N, dv]; block_q / block_k are the query and key tile sizes
    (any positive integers; the last tile of each axis may be short).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_q, n_k = q.shape[0], k.shape[0]
    out = np.zeros((n_q, v.shape[1]))
    lse = np.zeros(n_q)
    for q0 in range(0, n_q, block_q):
        q1 = min(q0 + block_q, n_q)
        qi = q[q0:q1]
        rows = np.arange(q0, q1)
        m = np.full(q1 - q0, -np.inf)
        ell = np.zeros(q1 - q0)
        acc = np.zeros((q1 - q0, v.shape[1]))
        for k0 in range(0, n_k, block_k):
            k1 = min(k0 + block_k, n_k)
            if causal and k0 > q1 - 1:
                break  # every key of this tile and of all later tiles is in the future
            s = scale * (qi @ k[k0:k1].T)
            if causal and k1 - 1 > q0:  # the tile crosses the diagonal: mask per element
                keys = np.arange(k0, k1)
                s = np.where(keys[None, :] <= rows[:, None], s, -np.inf)
            m_new = np.maximum(m, s.max(axis=1))
            ref = np.where(np.isfinite(m_new), m_new, 0.0)
            alpha = np.where(np.isfinite(m), np.exp(m - ref), 0.0)
            p = np.exp(s - ref[:, None])
            ell = alpha * ell + p.sum(axis=1)
            acc = alpha[:, None] * acc + p @ v[k0:k1]
            m = m_new
        out[q0:q1] = acc / ell[:, None]
        lse[q0:q1] = m + np.log(ell)
    return out, lse

"""Dense CPU float64 attention: the definition the tiled GPU kernel must reproduce.

TEST INFRASTRUCTURE ONLY -- imported by tests, the smoke check and the bench's cpu_baseline leg,
never by the product path.

What is computed (per batch b and head h, each an independent [N, d] problem):

    S   = scale * Q K^T                        ("Understanding FlashAttention Pt 1", §0.2 and §1.2;
                                                "Online Softmax & FlashAttention", Listing 26.2)
    S[i, j] = -inf  for j > i  when causal      (same chapter, Listing 26.2's mask; handbook §3.5)
    m   = max_j S[i, j]                         (stable softmax: handbook §2.2, chapter Eq 26.1)
    E   = exp(S - m),  l = sum_j E[i, j]
    P   = E / l,  O = P V
    LSE = m + ln(l)                             ("FlashAttention-2 -- Deeper Math", Fix 2)

S and P are materialised on purpose: this is the "standard attention" the pages contrast the
tiled kernel with, and the tiled kernel is exact with respect to it up to rounding order
("Flash Attention", introduction; handbook §3.2).

Readings where the pages leave a choice open:
  * ``scale`` is passed explicitly (the pages use 1/sqrt(d)); it multiplies q.k in float64.
  * LSE is the natural log of the normaliser of the *scaled* scores, one value per query row.
  * The inputs are upcast from exactly the tensors the GPU receives (bf16 or fp32), so the
    only differences measured are the kernel's own arithmetic.
  * A row with no visible key has no softmax; with N_q = N_k and the j <= i rule that cannot
    happen, and the oracle raises if it would.
"""
import numpy as np


def dense_scores(q, k, scale, causal, rows, query_offset=0, window=None, alibi_slope=None,
                 bias=None):
    """S = scale * q[rows] k^T (+ bias) with the masks applied (hidden keys -> -inf).

    q: [Nq, d], k: [N, d] float64; rows: int array of query indices into q. Query row i is token
    i + query_offset of the sequence (0 for self-attention over the same tokens), and the causal
    rule keeps keys j <= i + query_offset.
    Optional score modifiers ("Understanding FlashAttention Pt 1", §0.2: S = QK^T / sqrt(d) + B,
    B an additive mask or bias; §3.5 and §4.2: local/sliding-window attention and ALiBi-style
    bias), with positions i = row + query_offset and j = key index:
      window = (left, right): key j visible iff i - left <= j <= i + right (a negative bound is
               unbounded); combined with the causal rule when causal is set;
      alibi_slope = m: adds -m |i - j| to the scaled score;
      bias: [Nq, N] array added to the scaled score (its rows indexed like q).
    Returns S: [len(rows), N] float64.
    """
    rows = np.asarray(rows)
    s = float(scale) * (q[rows] @ k.T)
    key_pos = np.arange(k.shape[0])[None, :]
    qry_pos = rows[:, None] + int(query_offset)
    if bias is not None:
        s = s + np.asarray(bias, dtype=np.float64)[rows]
    if alibi_slope is not None:
        s = s - float(alibi_slope) * np.abs(qry_pos - key_pos)
    visible = np.ones(s.shape, dtype=bool)
    if causal:
        visible &= key_pos <= qry_pos
    if window is not None:
        left, right = window
        if left >= 0:
            visible &= key_pos >= qry_pos - left
        if right >= 0:
            visible &= key_pos <= qry_pos + right
    return np.where(visible, s, -np.inf)


def attention_head(q, k, v, scale, causal=False, rows=None, return_sp=False, query_offset=0,
                   window=None, alibi_slope=None, bias=None):
    """One head of naive attention in float64.

    q: [Nq, d], k: [N, d], v: [N, dv] (any float dtype; upcast to float64); Nq = N for
       self-attention. query_offset: position of query row 0 in the key sequence; window,
       alibi_slope, bias: optional score modifiers (see dense_scores).
    rows: optional sequence of query indices to evaluate (default: all Nq rows). Only those
          rows of S are formed, each against every key.
    Returns (O [R, dv], LSE [R]) and, if return_sp, also (S [R, N], P [R, N]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if rows is None:
        rows = np.arange(q.shape[0])
    rows = np.asarray(rows, dtype=np.int64)
    s = dense_scores(q, k, scale, causal, rows, query_offset, window, alibi_slope, bias)
    m = s.max(axis=1)
    if not np.all(np.isfinite(m)):
        raise ValueError("a query row has no visible key; its softmax is undefined")
    e = np.exp(s - m[:, None])
    ell = e.sum(axis=1)
    p = e / ell[:, None]
    o = p @ v
    lse = m + np.log(ell)
    if return_sp:
        return o, lse, s, p
    return o, lse


def attention(q, k, v, scale, causal=False, rows=None):
    """Batched naive attention over [B, H, N, d] arrays (numpy or anything np.asarray accepts).

    rows: optional per-head query rows, either one index array used for every (b, h) or an
          array of shape [B, H, R]. Returns (O [B, H, R, dv], LSE [B, H, R]) in float64.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, H = q.shape[0], q.shape[1]
    R = q.shape[2] if rows is None else np.asarray(rows).shape[-1]
    o = np.empty((B, H, R, v.shape[3]), dtype=np.float64)
    lse = np.empty((B, H, R), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            if rows is None:
                r = None
            else:
                ra = np.asarray(rows)
                r = ra if ra.ndim == 1 else ra[b, h]
            o[b, h], lse[b, h] = attention_head(q[b, h], k[b, h], v[b, h], scale, causal, r)
    return o, lse


def kv_head_of(h, H, H_kv):
    """K/V head that query head h attends with.

    "Understanding FlashAttention Pt 1", §4.1: the number of query heads is a multiple of the
    number of K/V heads and each query head is evaluated against its assigned K/V head (one per
    query head for MHA, a single shared one for MQA). The page does not spell the assignment out;
    the reading used here is the grouped one: the H query heads form H_kv consecutive groups of
    H / H_kv heads, and group j uses K/V head j.
    """
    if H_kv < 1 or H % H_kv != 0:
        raise ValueError("the query heads must divide evenly over the K/V heads")
    return h // (H // H_kv)


def attention_gqa(q, k, v, scale, causal=False, rows=None):
    """Batched naive attention with grouped K/V heads ("Understanding FlashAttention Pt 1", §4.1).

    q: [B, H, N, d]; k, v: [B, H_kv, N, d] with H a multiple of H_kv. Query head h attends with
    K/V head kv_head_of(h, H, H_kv); everything else is attention_head. rows as in attention().
    Returns (O [B, H, R, dv], LSE [B, H, R]) in float64.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, H = q.shape[0], q.shape[1]
    H_kv = k.shape[1]
    R = q.shape[2] if rows is None else np.asarray(rows).shape[-1]
    o = np.empty((B, H, R, v.shape[3]), dtype=np.float64)
    lse = np.empty((B, H, R), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            j = kv_head_of(h, H, H_kv)
            if rows is None:
                r = None
            else:
                ra = np.asarray(rows)
                r = ra if ra.ndim == 1 else ra[b, h]
            o[b, h], lse[b, h] = attention_head(q[b, h], k[b, j], v[b, j], scale, causal, r)
    return o, lse


def attention_decode(q, k, v, scale, causal=False):
    """Few queries against a longer key/value sequence, with grouped K/V heads, in float64.

    q: [B, H, N_q, d]; k, v: [B, H_kv, N_kv, d] with N_q <= N_kv when causal. The queries are the
    last N_q tokens of the N_kv-token sequence (query i is token N_kv - N_q + i), so with a causal
    mask query i sees keys j <= N_kv - N_q + i and without one every key; query head h uses K/V
    head kv_head_of(h, H, H_kv). This is the decoding problem of "FlashAttention-2 -- Deeper
    Math" ("What FA-2 does not fix"), written out densely: the split over keys and the merge of
    partial softmaxes are how the GPU reaches the same function.
    Returns (O [B, H, N_q, dv], LSE [B, H, N_q]).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, H, Nq = q.shape[0], q.shape[1], q.shape[2]
    H_kv, Nkv = k.shape[1], k.shape[2]
    if causal and Nq > Nkv:
        raise ValueError("with a causal mask the queries must be the last N_q of the N_kv tokens")
    o = np.empty((B, H, Nq, v.shape[3]), dtype=np.float64)
    lse = np.empty((B, H, Nq), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            j = kv_head_of(h, H, H_kv)
            o[b, h], lse[b, h] = attention_head(q[b, h], k[b, j], v[b, j], scale, causal,
                                                query_offset=Nkv - Nq)
    return o, lse


def attention_ext(q, k, v, scale, causal=False, window=None, alibi_slopes=None, bias=None,
                  rows=None):
    """Batched attention with grouped K/V heads and the optional score modifiers of dense_scores.

    q: [B, H, N, d]; k, v: [B, H_kv, N, d]; alibi_slopes: optional length-H sequence (one slope per
    query head); bias: optional [Bb, Hb, N, N] array with Bb in {1, B} and Hb in {1, H} (size-1
    dimensions are shared). rows as in attention(). Returns (O [B, H, R, dv], LSE [B, H, R]).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, H = q.shape[0], q.shape[1]
    H_kv = k.shape[1]
    R = q.shape[2] if rows is None else np.asarray(rows).shape[-1]
    o = np.empty((B, H, R, v.shape[3]), dtype=np.float64)
    lse = np.empty((B, H, R), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            j = kv_head_of(h, H, H_kv)
            if rows is None:
                r = None
            else:
                ra = np.asarray(rows)
                r = ra if ra.ndim == 1 else ra[b, h]
            bm = None
            if bias is not None:
                bb = np.asarray(bias)
                bm = bb[b if bb.shape[0] > 1 else 0, h if bb.shape[1] > 1 else 0]
            slope = None if alibi_slopes is None else float(alibi_slopes[h])
            o[b, h], lse[b, h] = attention_head(q[b, h], k[b, j], v[b, j], scale, causal, r,
                                                window=window, alibi_slope=slope, bias=bm)
    return o, lse

"""Helpers shared by the GPU parity tests: run the HIP path through the C-ABI binding, run the
CPU oracle on the same tensors (optionally on a thread pool over heads), compare."""
import concurrent.futures as cf
import os
import sys

import numpy as np
import torch

import exact_tiled_attention_05_amd as fa
from oracle import attention_head

# Parity bounds: max abs error of O (bf16 path / fp32 path) and of LSE.
TOL_O_BF16 = 2e-2
TOL_O_F32 = 1e-5
TOL_LSE = 1e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(q, k, v, scale, causal):
    """q, k, v: CPU tensors [B, H, N, d] (bf16 or fp32). Returns (o, lse) as CPU float64 numpy."""
    dev = torch.device("cuda:0")
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    o, lse = fa.forward(qd, kd, vd, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _as64(t):
    return t.float().numpy().astype(np.float64)


def oracle_rows(q, k, v, scale, causal, rows=None, heads=None, workers=None):
    """Oracle on every (b, h) in ``heads`` (default all) for the given query rows (default all).

    rows: None, a 1-D index array used for every head, or a dict {(b, h): rows}.
    Returns dict {(b, h): (rows, O [R, d], LSE [R])}.
    """
    B, H, N, _ = q.shape
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]

    def one(bh):
        b, h = bh
        r = rows.get(bh) if isinstance(rows, dict) else rows
        r = np.arange(N) if r is None else np.asarray(r)
        o, lse = attention_head(_as64(q[b, h]), _as64(k[b, h]), _as64(v[b, h]), scale, causal, r)
        return bh, (r, o, lse)

    workers = workers or min(16, os.cpu_count() or 1)
    out = {}
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        for bh, res in ex.map(one, heads):
            out[bh] = res
    return out


def compare(o_gpu, lse_gpu, ref):
    """Max abs errors of O and LSE over the rows the oracle evaluated."""
    eo = el = 0.0
    for (b, h), (r, o, lse) in ref.items():
        eo = max(eo, float(np.abs(o_gpu[b, h, r] - o).max()))
        el = max(el, float(np.abs(lse_gpu[b, h, r] - lse).max()))
    return eo, el

"""HIP graph capture of the library's calls.

The entry points only enqueue kernels on the caller's stream (no allocation, no memset, no
synchronisation; fa_fwd_splitkv_noalloc keeps its partials in the library's static scratch), so a
caller can capture them in a graph and replay it. Each case captures one call, then replays the
graph three times with new inputs copied into its buffers and the program's own eager GPU work in
between, and checks every replay bit for bit against an eager call on the same inputs into other
buffers. Cases: the bf16 forward on the wide-row kernel (causal, d = 128, N = 4096 + ragged) and on
the 8-wave kernel (d = 64), split-KV decoding through the allocation-free entry point, and the
backward pass with a caller workspace.
"""
import pytest
import torch

import exact_tiled_attention_05_amd as fa
from exact_tiled_attention_05_amd.workloads import make_inputs, softmax_scale, to_layout

from gpu_util import log

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _same(a, b):
    ia = a.contiguous().view(torch.int16 if a.element_size() == 2 else torch.int32)
    ib = b.contiguous().view(torch.int16 if b.element_size() == 2 else torch.int32)
    return bool(torch.equal(ia, ib))


def _replays(name, inputs, capture_call, eager_call, seeds):
    """inputs: static device tensors the graph reads; capture_call(): the call to capture (writes
    the static outputs it returns); eager_call(): the same call into fresh outputs."""
    capture_call()  # warm-up outside the capture (first-call setup such as the scratch address)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = capture_call()
    torch.cuda.synchronize()
    for r, seed in enumerate(seeds):
        gen = torch.Generator(device=DEV).manual_seed(seed)
        for x in inputs:
            x.copy_(torch.randn(x.shape, generator=gen, device=DEV, dtype=torch.float32).to(x.dtype))
        noise = torch.randn(1 << 20, device=DEV).sum()  # the program's own work between replays
        g.replay()
        torch.cuda.synchronize()
        ref = eager_call()
        torch.cuda.synchronize()
        log("graph %s replay %d (noise %.3f)" % (name, r, float(noise)))
        for i, (a, b) in enumerate(zip(outs, ref)):
            assert _same(a, b), "%s: replay %d output %d differs from the eager call" % (name, r, i)


@pytest.mark.parametrize("N,d,causal", [(4096 + 77, 128, True), (1000, 64, False)])
def test_forward_graph(N, d, causal):
    q, k, v = make_inputs(1, 4, N, d, "bf16", seed=3)
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((1, 4, N), dtype=torch.float32, device=DEV)
    sc = softmax_scale(d)

    def capture():
        fa.forward(qd, kd, vd, scale=sc, causal=causal, out=o, lse=lse)
        return o, lse

    def eager():
        return fa.forward(qd, kd, vd, scale=sc, causal=causal)

    _replays("forward N=%d d=%d" % (N, d), [qd, kd, vd], capture, eager, seeds=[11, 12, 13])


def test_decode_noalloc_graph():
    B, H, H_kv, Nq, Nkv, d = 4, 32, 8, 2, 5000, 128
    q, k, v = make_inputs(B, H, Nkv, d, "bf16", H_kv=H_kv, Nq=Nq, seed=5)
    qd, kd, vd = (to_layout(x, "bnhd").to(DEV) for x in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=DEV)
    sc = softmax_scale(d)

    def call(out, l_out):
        rc = fa.fa_fwd_splitkv_noalloc(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out.data_ptr(),
                                       l_out.data_ptr(), B, H, H_kv, Nq, Nkv, d, sc, 1,
                                       fa.FA_LAYOUT_BNHD, 0,
                                       torch.cuda.current_stream(DEV).cuda_stream)
        assert rc == fa.FA_OK, fa.fa_strerror(rc)
        return out, l_out

    def eager():
        return call(torch.empty_like(o), torch.empty_like(lse))

    _replays("decode noalloc", [qd, kd, vd], lambda: call(o, lse), eager, seeds=[21, 22, 23])


def test_backward_graph():
    B, H, N, d = 1, 4, 2048 + 33, 128
    q, k, v = make_inputs(B, H, N, d, "bf16", seed=7)
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    do = torch.randn(qd.shape, device=DEV).to(torch.bfloat16)
    sc = softmax_scale(d)
    o, lse = fa.forward(qd, kd, vd, scale=sc, causal=True)
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, H, N, d), dtype=torch.uint8, device=DEV)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)

    def capture():
        fa.backward(qd, kd, vd, o, lse, do, scale=sc, causal=True, dq=dq, dk=dk, dv=dv,
                    workspace=ws)
        return dq, dk, dv

    def eager():
        return fa.backward(qd, kd, vd, o, lse, do, scale=sc, causal=True)

    # the replays change dO (O and the logsumexp stay those of the forward call)
    _replays("backward", [do], capture, eager, seeds=[31, 32, 33])

"""Exact tiled attention for AMD MI355X (gfx950): Python binding of ``libfa.so``.

The library computes, per batch and head, O = softmax(scale * Q K^T [causal mask]) V and the
per-row logsumexp, tile by tile, without ever writing the N x N score matrix, and the gradients
dQ, dK, dV by recomputing those tiles (see ``include/fa.h`` for the full contract). This module only marshals arguments: every step of the
computation runs in the HIP kernels of ``libfa.so``. There is no CPU fallback; if the library
is missing the calls raise.

Raw entry points (same names and argument order as the C-ABI; pointers are integers):
    fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, stream) -> int
    fa_fwd_f32(q, k, v, o, lse, B, H, N, d, scale, causal, stream) -> int
    fa_fwd_gqa(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal, layout, stream) -> int
    fa_fwd_gqa_f32(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal, layout, stream) -> int
    fa_fwd_ext(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal, layout, window_left,
               window_right, alibi_slopes, bias, bias_batch_stride, bias_head_stride,
               bias_row_stride, stream) -> int
    fa_splitkv_workspace_bytes(B, H, H_kv, N_q, N_kv, d, causal, n_splits) -> int
    fa_fwd_splitkv(q, k, v, o, lse, B, H, H_kv, N_q, N_kv, d, scale, causal, layout, n_splits,
                   workspace, workspace_bytes, stream) -> int
    fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, H_kv, N_q, N_kv, d, scale, causal, layout,
                           n_splits, stream) -> int
    fa_bwd_workspace_bytes(B, H, H_kv, N, d) -> int
    fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, N, d, scale, causal, layout, workspace,
           workspace_bytes, stream) -> int
    fa_strerror(code) -> str
    fa_version() -> int
Tensor convenience (PyTorch supplies device memory and the stream):
    forward(q, k, v, scale=None, causal=False, out=None, lse=None, stream=None, layout="bhnd")
        -> (o, lse)
    forward_ext(q, k, v, scale=None, causal=False, layout="bhnd", window=(-1, -1),
                alibi_slopes=None, bias=None, out=None, lse=None, stream=None) -> (o, lse)
    decode(q, k, v, scale=None, causal=False, layout="bhnd", n_splits=0, out=None, lse=None,
           workspace=None, stream=None) -> (o, lse)
    backward(q, k, v, o, lse, dout, scale=None, causal=False, layout="bhnd", dq=None, dk=None,
             dv=None, workspace=None, stream=None) -> (dq, dk, dv)
"""
import contextlib
import ctypes
import math
import os

__all__ = ["fa_fwd", "fa_fwd_f32", "fa_fwd_gqa", "fa_fwd_gqa_f32", "fa_fwd_ext", "forward_ext",
           "fa_fwd_splitkv", "fa_fwd_splitkv_noalloc", "fa_bwd",
           "fa_bwd_workspace_bytes", "backward",
           "fa_splitkv_workspace_bytes", "fa_strerror", "fa_version", "forward", "decode", "FAError", "library_path", "race_check_library_path", "load_library", "using_library", "FA_OK", "FA_ERR_INVALID_ARG",
           "FA_ERR_UNSUPPORTED", "FA_ERR_ALIGNMENT", "FA_ERR_LAUNCH", "FA_ERR_TOO_LARGE",
           "FA_NOALLOC_SCRATCH_BYTES", "FA_LAYOUT_BHND", "FA_LAYOUT_BNHD"]

FA_OK = 0
FA_ERR_INVALID_ARG = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_ALIGNMENT = -3
FA_ERR_LAUNCH = -4
FA_ERR_TOO_LARGE = -5
FA_NOALLOC_SCRATCH_BYTES = 16 << 20
FA_LAYOUT_BHND = 0
FA_LAYOUT_BNHD = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def library_path():
    return os.path.join(_HERE, "libfa.so")


class FAError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        super().__init__("%s failed: %s (code %d)" % (where, fa_strerror(code), code))


def race_check_library_path():
    return os.path.join(_HERE, "libfa_race.so")


def load_library(path=None):
    """Load libfa.so from the package directory (built by ``exact_tiled_attention_05_amd.build``).

    With ``path`` (e.g. ``race_check_library_path()``) that build of the same C-ABI is loaded and
    returned instead; the module's own entry points keep using libfa.so.
    """
    global _LIB
    if path is not None:
        return _open(path)
    if _LIB is None:
        _LIB = _open(library_path())
    return _LIB


@contextlib.contextmanager
def using_library(lib):
    """Inside the block, this module's entry points call ``lib`` (a library returned by
    ``load_library(path)``) instead of libfa.so. Not thread-safe: it swaps a module global."""
    global _LIB
    prev = load_library()
    _LIB = lib
    try:
        yield lib
    finally:
        _LIB = prev


def _open(path):
    if not os.path.exists(path):
        raise RuntimeError("%s is not built (expected at %s); run "
                           "`python -m exact_tiled_attention_05_amd.build --all`"
                           % (os.path.basename(path), path))
    lib = ctypes.CDLL(path)
    fwd_args = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 4 + [ctypes.c_float, ctypes.c_int,
                                                               ctypes.c_void_p]
    gqa_args = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 5 + [ctypes.c_float, ctypes.c_int,
                                                               ctypes.c_int, ctypes.c_void_p]
    for name, argt in (("fa_fwd", fwd_args), ("fa_fwd_f32", fwd_args),
                       ("fa_fwd_gqa", gqa_args), ("fa_fwd_gqa_f32", gqa_args)):
        fn = getattr(lib, name)
        fn.argtypes = argt
        fn.restype = ctypes.c_int
    lib.fa_fwd_ext.argtypes = ([ctypes.c_void_p] * 5 + [ctypes.c_int] * 5 + [ctypes.c_float] +
                               [ctypes.c_int] * 4 + [ctypes.c_void_p] * 2 +
                               [ctypes.c_longlong] * 3 + [ctypes.c_void_p])
    lib.fa_fwd_ext.restype = ctypes.c_int
    lib.fa_splitkv_workspace_bytes.argtypes = [ctypes.c_int] * 8
    lib.fa_splitkv_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_fwd_splitkv.argtypes = ([ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 +
                                   [ctypes.c_float] + [ctypes.c_int] * 3 +
                                   [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p])
    lib.fa_fwd_splitkv.restype = ctypes.c_int
    lib.fa_fwd_splitkv_noalloc.argtypes = ([ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 +
                                           [ctypes.c_float] + [ctypes.c_int] * 3 +
                                           [ctypes.c_void_p])
    lib.fa_fwd_splitkv_noalloc.restype = ctypes.c_int
    lib.fa_bwd_workspace_bytes.argtypes = [ctypes.c_int] * 5
    lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_bwd.argtypes = ([ctypes.c_void_p] * 9 + [ctypes.c_int] * 5 + [ctypes.c_float] +
                           [ctypes.c_int] * 2 + [ctypes.c_void_p, ctypes.c_size_t,
                                                 ctypes.c_void_p])
    lib.fa_bwd.restype = ctypes.c_int
    lib.fa_strerror.argtypes = [ctypes.c_int]
    lib.fa_strerror.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = ctypes.c_int
    return lib


def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, stream=None):
    return load_library().fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, stream)


def fa_fwd_f32(q, k, v, o, lse, B, H, N, d, scale, causal, stream=None):
    return load_library().fa_fwd_f32(q, k, v, o, lse, B, H, N, d, scale, causal, stream)


def fa_fwd_gqa(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal, layout, stream=None):
    return load_library().fa_fwd_gqa(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal, layout,
                                     stream)


def fa_fwd_gqa_f32(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal, layout, stream=None):
    return load_library().fa_fwd_gqa_f32(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal,
                                         layout, stream)


def fa_fwd_ext(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal, layout, window_left,
               window_right, alibi_slopes, bias, bias_batch_stride, bias_head_stride,
               bias_row_stride, stream=None):
    return load_library().fa_fwd_ext(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal, layout,
                                     window_left, window_right, alibi_slopes, bias,
                                     bias_batch_stride, bias_head_stride, bias_row_stride, stream)


def fa_splitkv_workspace_bytes(B, H, H_kv, N_q, N_kv, d, causal, n_splits):
    return load_library().fa_splitkv_workspace_bytes(B, H, H_kv, N_q, N_kv, d, causal, n_splits)


def fa_fwd_splitkv(q, k, v, o, lse, B, H, H_kv, N_q, N_kv, d, scale, causal, layout, n_splits,
                   workspace, workspace_bytes, stream=None):
    return load_library().fa_fwd_splitkv(q, k, v, o, lse, B, H, H_kv, N_q, N_kv, d, scale, causal,
                                         layout, n_splits, workspace, workspace_bytes, stream)


def fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, H_kv, N_q, N_kv, d, scale, causal, layout,
                           n_splits, stream=None):
    return load_library().fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, H_kv, N_q, N_kv, d, scale,
                                                 causal, layout, n_splits, stream)


def fa_bwd_workspace_bytes(B, H, H_kv, N, d):
    return load_library().fa_bwd_workspace_bytes(B, H, H_kv, N, d)


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, N, d, scale, causal, layout, workspace,
           workspace_bytes, stream=None):
    return load_library().fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, N, d, scale,
                                 causal, layout, workspace, workspace_bytes, stream)


def fa_strerror(code):
    return load_library().fa_strerror(code).decode()


def fa_version():
    return load_library().fa_version()


def forward(q, k, v, scale=None, causal=False, out=None, lse=None, stream=None, layout="bhnd"):
    """Attention forward on CUDA/HIP tensors (bf16 or fp32, contiguous).

    layout "bhnd": q [B, H, N, d], k and v [B, H_kv, N, d]; layout "bnhd": q [B, N, H, d], k and
    v [B, N, H_kv, d]. H must be a multiple of H_kv (query head h uses K/V head h // (H // H_kv);
    H_kv = H is ordinary multi-head attention). Returns (o, lse) with o like q and lse float32
    [B, H, N]. ``out``/``lse`` may be passed to reuse buffers; ``stream`` defaults to torch's
    current stream on q's device.
    """
    import torch

    if layout not in ("bhnd", "bnhd"):
        raise ValueError("layout must be 'bhnd' or 'bnhd'")
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q, k, v must be 4-D and k, v must have the same shape")
    if layout == "bhnd":
        B, H, N, d = q.shape
        Bk, H_kv, Nk, dk = k.shape
    else:
        B, N, H, d = q.shape
        Bk, Nk, H_kv, dk = k.shape
    if (Bk, Nk, dk) != (B, N, d) or H_kv < 1 or H % H_kv != 0:
        raise ValueError("k, v must match q in batch, length and head dim, with H a multiple of "
                         "their head count")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q, k, v must all be bfloat16 or all float32")
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on the same GPU device")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if (out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous()
            or out.device != q.device):
        raise ValueError("out must be a contiguous tensor like q")
    if (tuple(lse.shape) != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous()
            or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr())
    if layout == "bhnd" and H_kv == H:
        fn = fa_fwd if q.dtype == torch.bfloat16 else fa_fwd_f32
        rc = fn(*ptrs, B, H, N, d, float(scale), int(bool(causal)), stream)
    else:
        fn = fa_fwd_gqa if q.dtype == torch.bfloat16 else fa_fwd_gqa_f32
        lay = FA_LAYOUT_BHND if layout == "bhnd" else FA_LAYOUT_BNHD
        rc = fn(*ptrs, B, H, H_kv, N, d, float(scale), int(bool(causal)), lay, stream)
    if rc != FA_OK:
        raise FAError(rc, fn.__name__)
    return out, lse


def decode(q, k, v, scale=None, causal=False, layout="bhnd", n_splits=0, out=None, lse=None,
           workspace=None, stream=None):
    """Split-KV attention of few queries against a long K/V sequence (bf16 CUDA/HIP tensors).

    layout "bhnd": q [B, H, N_q, d], k and v [B, H_kv, N_kv, d]; "bnhd": q [B, N_q, H, d], k and
    v [B, N_kv, H_kv, d]. Query i is token N_kv - N_q + i (causal: it sees keys up to there).
    Returns (o, lse) with o like q and lse float32 [B, H, N_q]. ``workspace`` (a uint8 tensor of
    at least fa_splitkv_workspace_bytes(...) bytes on q's device) is allocated here if not given.
    """
    import torch

    if layout not in ("bhnd", "bnhd"):
        raise ValueError("layout must be 'bhnd' or 'bnhd'")
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q, k, v must be 4-D and k, v must have the same shape")
    if layout == "bhnd":
        B, H, Nq, d = q.shape
        Bk, H_kv, Nkv, dk = k.shape
    else:
        B, Nq, H, d = q.shape
        Bk, Nkv, H_kv, dk = k.shape
    if (Bk, dk) != (B, d) or H_kv < 1 or H % H_kv != 0:
        raise ValueError("k, v must match q in batch and head dim, with H a multiple of their "
                         "head count")
    if not (q.dtype == k.dtype == v.dtype == torch.bfloat16):
        raise ValueError("q, k, v must all be bfloat16")
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on the same GPU device")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = fa_splitkv_workspace_bytes(B, H, H_kv, Nq, Nkv, d, int(bool(causal)), n_splits)
    if need == 0:
        raise ValueError("shape not supported by split-KV decoding (see fa_fwd_splitkv limits)")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    lay = FA_LAYOUT_BHND if layout == "bhnd" else FA_LAYOUT_BNHD
    rc = fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                        B, H, H_kv, Nq, Nkv, d, float(scale), int(bool(causal)), lay, n_splits,
                        workspace.data_ptr(), workspace.numel() * workspace.element_size(), stream)
    if rc != FA_OK:
        raise FAError(rc, "fa_fwd_splitkv")
    return out, lse


def backward(q, k, v, o, lse, dout, scale=None, causal=False, layout="bhnd", dq=None, dk=None,
             dv=None, workspace=None, stream=None):
    """Gradients of attention (bf16 CUDA/HIP tensors, contiguous) by recomputation.

    q, o, dout like forward()'s q and o; k, v its k and v; lse the float32 [B, H, N] logsumexp
    forward() returned for the same q, k, v, scale and mask. Returns (dq, dk, dv) shaped like q, k,
    v; for grouped K/V heads dk and dv hold the sums over each K/V head's query heads.
    ``workspace`` (a uint8 tensor of at least fa_bwd_workspace_bytes(B, H, H_kv, N, d) bytes) is
    allocated here if not given.
    """
    import torch

    if layout not in ("bhnd", "bnhd"):
        raise ValueError("layout must be 'bhnd' or 'bnhd'")
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or o.shape != q.shape or \
            dout.shape != q.shape:
        raise ValueError("q, o, dout must share a shape and k, v must share a shape (4-D)")
    if layout == "bhnd":
        B, H, N, d = q.shape
        Bk, H_kv, Nk, dk_ = k.shape
    else:
        B, N, H, d = q.shape
        Bk, Nk, H_kv, dk_ = k.shape
    if (Bk, Nk, dk_) != (B, N, d) or H_kv < 1 or H % H_kv != 0:
        raise ValueError("k, v must match q in batch, length and head dim, with H a multiple of "
                         "their head count")
    if not all(t.dtype == torch.bfloat16 for t in (q, k, v, o, dout)):
        raise ValueError("q, k, v, o, dout must all be bfloat16")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must be float32 [B, H, N]")
    ts = (q, k, v, o, dout, lse)
    if not all(t.is_cuda and t.device == q.device and t.is_contiguous() for t in ts):
        raise ValueError("all tensors must be contiguous and on the same GPU device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = fa_bwd_workspace_bytes(B, H, H_kv, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    lay = FA_LAYOUT_BHND if layout == "bhnd" else FA_LAYOUT_BNHD
    rc = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, H_kv, N, d,
                float(scale), int(bool(causal)), lay, workspace.data_ptr(),
                workspace.numel() * workspace.element_size(), stream)
    if rc != FA_OK:
        raise FAError(rc, "fa_bwd")
    return dq, dk, dv


def forward_ext(q, k, v, scale=None, causal=False, layout="bhnd", window=(-1, -1),
                alibi_slopes=None, bias=None, out=None, lse=None, stream=None):
    """forward() with a sliding window, ALiBi slopes and/or an additive bias (bf16 tensors).

    window: (left, right), key j visible to query i iff i - left <= j <= i + right (-1: that side
    unbounded). alibi_slopes: float32 tensor [H] on q's device (score -= slope_h |i - j|). bias: bf16
    tensor broadcastable to [B, H, N, N] (size-1 batch/head dimensions are shared), contiguous in
    its last dimension, added to the scaled scores. Returns (o, lse) like forward().
    """
    import torch

    if layout not in ("bhnd", "bnhd"):
        raise ValueError("layout must be 'bhnd' or 'bnhd'")
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q, k, v must be 4-D and k, v must have the same shape")
    if layout == "bhnd":
        B, H, N, d = q.shape
        Bk, H_kv, Nk, dk = k.shape
    else:
        B, N, H, d = q.shape
        Bk, Nk, H_kv, dk = k.shape
    if (Bk, Nk, dk) != (B, N, d) or H_kv < 1 or H % H_kv != 0:
        raise ValueError("k, v must match q in batch, length and head dim, with H a multiple of "
                         "their head count")
    if not (q.dtype == k.dtype == v.dtype == torch.bfloat16):
        raise ValueError("q, k, v must all be bfloat16")
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on the same GPU device")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    wl, wr = (int(window[0]), int(window[1]))
    sp = 0
    if alibi_slopes is not None:
        if alibi_slopes.dtype != torch.float32 or alibi_slopes.numel() != H or \
                alibi_slopes.device != q.device or not alibi_slopes.is_contiguous():
            raise ValueError("alibi_slopes must be a contiguous float32 tensor of H values on "
                             "q's device")
        sp = alibi_slopes.data_ptr()
    bp, bs, hs, rs = 0, 0, 0, 0
    if bias is not None:
        if bias.dtype != torch.bfloat16 or bias.dim() != 4 or bias.device != q.device:
            raise ValueError("bias must be a 4-D bfloat16 tensor on q's device")
        if bias.shape[0] not in (1, B) or bias.shape[1] not in (1, H) or \
                tuple(bias.shape[2:]) != (N, N) or bias.stride(3) != 1:
            raise ValueError("bias must broadcast to [B, H, N, N] and be contiguous in its last "
                             "dimension")
        if bias.data_ptr() % 16 or any(bias.stride(i) % 8 for i in range(3) if bias.shape[i] > 1):
            raise ValueError("bias rows must start 16-byte aligned: strides that are multiples of "
                             "8 elements (pad the last dimension)")
        bp = bias.data_ptr()
        bs = bias.stride(0) if bias.shape[0] > 1 else 0
        hs = bias.stride(1) if bias.shape[1] > 1 else 0
        rs = bias.stride(2) if N > 1 else 8  # one row: its stride is never used
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    lay = FA_LAYOUT_BHND if layout == "bhnd" else FA_LAYOUT_BNHD
    rc = fa_fwd_ext(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H,
                    H_kv, N, d, float(scale), int(bool(causal)), lay, wl, wr, sp or None,
                    bp or None, bs, hs, rs, stream)
    if rc != FA_OK:
        raise FAError(rc, "fa_fwd_ext")
    return out, lse

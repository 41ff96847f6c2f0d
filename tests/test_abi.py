"""The C-ABI boundary on the CPU: libfa.so loads, exports every function include/fa.h declares,
and refuses bad arguments with the documented codes before making any HIP call (no compute runs
here; the pointers below are never dereferenced)."""
import ctypes
import os
import re

import pytest
import torch

import exact_tiled_attention_05_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def _codes():
    text = open(HEADER).read()
    return {m[0]: int(m[1]) for m in re.findall(r"#define\s+(FA_[A-Z_]+)\s+\(?(-?\d+)\)?", text)}


def test_header_declares_the_expected_entry_points():
    assert _declared() == ["fa_bwd", "fa_bwd_workspace_bytes", "fa_fwd", "fa_fwd_ext",
                           "fa_fwd_f32", "fa_fwd_gqa", "fa_fwd_gqa_f32", "fa_fwd_splitkv",
                           "fa_fwd_splitkv_noalloc", "fa_splitkv_workspace_bytes", "fa_strerror",
                           "fa_version"]


@pytest.mark.parametrize("path", [fa.library_path(), fa.race_check_library_path()],
                         ids=["libfa", "libfa_race"])
def test_library_exports_every_declared_symbol(path):
    """Both builds (the fast library and its race-check twin) export the whole C-ABI."""
    lib = ctypes.CDLL(path)
    for name in _declared():
        assert hasattr(lib, name), name
    assert fa.load_library(path).fa_version() == fa.load_library().fa_version()


def test_python_codes_match_header():
    for name, value in _codes().items():
        assert getattr(fa, name) == value, name


def test_version_and_strerror():
    assert fa.fa_version() >= 100
    for code in (0, -1, -2, -3, -4, -5):
        assert fa.fa_strerror(code) and fa.fa_strerror(code) != "unknown error code"
    assert fa.fa_strerror(12345) == "unknown error code"


# Fake, 16-byte aligned, non-overlapping "device" addresses. Every call below fails validation,
# which happens before any HIP call, so they are never dereferenced.
A = 1 << 40
Q, K, V, O, L = (A + i * (1 << 32) for i in range(5))
GOOD = dict(q=Q, k=K, v=V, o=O, lse=L, B=2, H=3, N=100, d=64, scale=0.125, causal=0)


def _call(fn, **kw):
    a = dict(GOOD, **kw)
    return fn(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
              a["scale"], a["causal"], None)


BAD = [
    (dict(q=0), fa.FA_ERR_INVALID_ARG),
    (dict(k=0), fa.FA_ERR_INVALID_ARG),
    (dict(v=0), fa.FA_ERR_INVALID_ARG),
    (dict(o=0), fa.FA_ERR_INVALID_ARG),
    (dict(lse=0), fa.FA_ERR_INVALID_ARG),
    (dict(B=0), fa.FA_ERR_INVALID_ARG),
    (dict(H=-1), fa.FA_ERR_INVALID_ARG),
    (dict(N=0), fa.FA_ERR_INVALID_ARG),
    (dict(N=(1 << 22) + 1), fa.FA_ERR_INVALID_ARG),
    (dict(B=256, H=256), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(causal=-1), fa.FA_ERR_INVALID_ARG),
    (dict(scale=-0.5), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=512), fa.FA_ERR_UNSUPPORTED),
    (dict(d=0), fa.FA_ERR_UNSUPPORTED),
    (dict(q=Q + 8), fa.FA_ERR_ALIGNMENT),
    (dict(lse=L + 4), fa.FA_ERR_ALIGNMENT),
    (dict(o=Q), fa.FA_ERR_INVALID_ARG),            # o aliases q
    (dict(o=K + 16), fa.FA_ERR_INVALID_ARG),       # o overlaps k
    (dict(lse=O + 1024), fa.FA_ERR_INVALID_ARG),   # lse inside o
    (dict(lse=V), fa.FA_ERR_INVALID_ARG),          # lse aliases v
]


@pytest.mark.parametrize("fn_name", ["fa_fwd", "fa_fwd_f32"])
@pytest.mark.parametrize("kw,code", BAD, ids=[str(b[0]) for b in BAD])
def test_bad_arguments_are_refused(fn_name, kw, code):
    assert _call(getattr(fa, fn_name), **kw) == code


GOOD_GQA = dict(GOOD, H=4, H_kv=2, layout=fa.FA_LAYOUT_BNHD)


def _call_gqa(fn, **kw):
    a = dict(GOOD_GQA, **kw)
    return fn(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["H_kv"], a["N"], a["d"],
              a["scale"], a["causal"], a["layout"], None)


BAD_GQA = [(kw, code) for kw, code in BAD if "H" not in kw] + [
    (dict(H_kv=0), fa.FA_ERR_INVALID_ARG),
    (dict(H_kv=-2), fa.FA_ERR_INVALID_ARG),
    (dict(H_kv=3), fa.FA_ERR_INVALID_ARG),          # 4 query heads do not split over 3
    (dict(H_kv=8), fa.FA_ERR_INVALID_ARG),          # more K/V heads than query heads
    (dict(layout=2), fa.FA_ERR_INVALID_ARG),
    (dict(layout=-1), fa.FA_ERR_INVALID_ARG),
    (dict(H=256, H_kv=1, B=256), fa.FA_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("fn_name", ["fa_fwd_gqa", "fa_fwd_gqa_f32"])
@pytest.mark.parametrize("kw,code", BAD_GQA, ids=[str(b[0]) for b in BAD_GQA])
def test_bad_gqa_arguments_are_refused(fn_name, kw, code):
    assert _call_gqa(getattr(fa, fn_name), **kw) == code


def test_gqa_overlap_uses_kv_sizes():
    """k and v hold B*H_kv*N*d elements: an o placed right after a (smaller) k is accepted by the
    checks only if it does not overlap; one element into k is refused."""
    kv_bytes = 2 * 2 * 100 * 64 * 2  # B*H_kv*N*d bf16
    assert _call_gqa(fa.fa_fwd_gqa, o=K + kv_bytes - 16) == fa.FA_ERR_INVALID_ARG


def test_forward_checks_tensors_before_any_gpu_use():
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.forward(q, q, q)  # CPU tensors
    with pytest.raises(ValueError):
        fa.forward(q, q, q.float())  # mixed dtypes
    with pytest.raises(ValueError):
        fa.forward(q[0], q[0], q[0])  # not 4-D
    with pytest.raises(ValueError):
        fa.forward(q.half(), q.half(), q.half())  # fp16 is not a supported dtype


def test_forward_checks_gqa_shapes_before_any_gpu_use():
    q = torch.zeros(1, 4, 8, 64, dtype=torch.bfloat16)
    k3 = torch.zeros(1, 3, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.forward(q, k3, k3)  # 4 query heads do not split over 3 K/V heads
    with pytest.raises(ValueError):
        fa.forward(q, q, q, layout="nhbd")  # unknown layout
    k = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.forward(q, k, torch.zeros(1, 2, 9, 64, dtype=torch.bfloat16))  # k, v differ
    with pytest.raises(ValueError):
        fa.forward(q, k, k)  # CPU tensors (shapes are fine)



# ---- split-KV decoding ---------------------------------------------------------------------------
W_ = A + 8 * (1 << 32)
GOOD_DEC = dict(q=Q, k=K, v=V, o=O, lse=L, B=2, H=8, H_kv=2, Nq=1, Nkv=5000, d=128, scale=0.1,
                causal=1, layout=0, n_splits=0, ws=W_, ws_bytes=1 << 30)


def _call_dec(**kw):
    a = dict(GOOD_DEC, **kw)
    return fa.fa_fwd_splitkv(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["H_kv"],
                             a["Nq"], a["Nkv"], a["d"], a["scale"], a["causal"], a["layout"],
                             a["n_splits"], a["ws"], a["ws_bytes"], None)


BAD_DEC = [
    (dict(ws=0), fa.FA_ERR_INVALID_ARG),
    (dict(ws_bytes=16), fa.FA_ERR_INVALID_ARG),           # too small
    (dict(q=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nkv=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nkv=(1 << 22) + 1), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=6000), fa.FA_ERR_INVALID_ARG),               # causal needs N_q <= N_kv
    (dict(H_kv=3), fa.FA_ERR_INVALID_ARG),
    (dict(layout=5), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(n_splits=-1), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=129, causal=0), fa.FA_ERR_UNSUPPORTED),      # 4 heads x 129 queries > 512 rows
    (dict(H=1024, H_kv=1), fa.FA_ERR_UNSUPPORTED),       # 1024 heads share one K/V head
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(ws=W_ + 8), fa.FA_ERR_ALIGNMENT),
    (dict(ws=Q), fa.FA_ERR_INVALID_ARG),                  # workspace overlaps q
    (dict(o=K), fa.FA_ERR_INVALID_ARG),                   # o overlaps k
]


@pytest.mark.parametrize("kw,code", BAD_DEC, ids=[str(b[0]) for b in BAD_DEC])
def test_bad_splitkv_arguments_are_refused(kw, code):
    assert _call_dec(**kw) == code


def test_splitkv_workspace_bytes():
    f = fa.fa_splitkv_workspace_bytes
    # B * H_kv * splits * R * (d + 1) floats, the LSE part starting on a 256-byte boundary
    n = f(1, 8, 2, 1, 4096, 128, 1, 16)
    R, splits = 4, 16
    o_part = 2 * splits * R * 128 * 4
    assert n == (o_part + 255) // 256 * 256 + 2 * splits * R * 4
    assert f(1, 8, 2, 1, 4096, 128, 1, 0) > 0          # library's own split count
    assert f(1, 8, 2, 128, 4096, 128, 1, 0) > 0         # 512 rows per K/V head: the maximum
    assert f(1, 8, 2, 129, 4096, 128, 1, 0) == 0        # 516 rows per K/V head: not accepted
    # several row tiles per K/V head take fewer automatic splits (about 768 waves in all)
    one_tile = f(1, 8, 2, 8, 32768, 128, 1, 0) // (32 * (128 + 1) * 4)
    four_tiles = f(1, 8, 2, 32, 32768, 128, 1, 0) // (128 * (128 + 1) * 4)
    assert four_tiles < one_tile
    assert f(1, 8, 3, 1, 4096, 128, 1, 0) == 0          # uneven head groups
    assert f(1, 8, 2, 1, 40, 128, 1, 1000) == f(1, 8, 2, 1, 40, 128, 1, 2)  # at most 1 split / 32 keys


def _call_dec_noalloc(**kw):
    a = dict(GOOD_DEC, **kw)
    return fa.fa_fwd_splitkv_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                                     a["H_kv"], a["Nq"], a["Nkv"], a["d"], a["scale"], a["causal"],
                                     a["layout"], a["n_splits"], None)


# The allocation-free entry point refuses what fa_fwd_splitkv refuses (its workspace arguments
# aside), and a shape whose partials exceed the static scratch, before any HIP call.
BAD_DEC_NOALLOC = [(kw, code) for kw, code in BAD_DEC if not set(kw) & {"ws", "ws_bytes"}] + [
    # 256 x 8 K/V heads x 32 stacked rows: one split each already needs 34 MB of partials
    (dict(B=256, H=8, H_kv=8, Nq=32, Nkv=64, n_splits=1), fa.FA_ERR_TOO_LARGE),
    # the library's split plan for 8 x 8 K/V heads x 4 rows over 1M keys: 12 splits, 3.2 MB, fits;
    # an explicit 1024 splits does not
    (dict(B=8, H=32, H_kv=8, Nq=1, Nkv=1 << 20, n_splits=1024), fa.FA_ERR_TOO_LARGE),
]


@pytest.mark.parametrize("kw,code", BAD_DEC_NOALLOC, ids=[str(b[0]) for b in BAD_DEC_NOALLOC])
def test_bad_splitkv_noalloc_arguments_are_refused(kw, code):
    assert _call_dec_noalloc(**kw) == code


def test_noalloc_scratch_limit_matches_workspace_query():
    f = fa.fa_splitkv_workspace_bytes
    assert fa.FA_NOALLOC_SCRATCH_BYTES == 16 << 20
    assert f(256, 8, 8, 32, 64, 128, 1, 1) > fa.FA_NOALLOC_SCRATCH_BYTES
    assert f(8, 32, 8, 1, 1 << 20, 128, 1, 1024) > fa.FA_NOALLOC_SCRATCH_BYTES
    # the Llama-3-8B decoding batch (8 sequences, 32 query over 8 K/V heads, 32K keys) fits
    assert 0 < f(8, 32, 8, 1, 32768, 128, 1, 0) <= fa.FA_NOALLOC_SCRATCH_BYTES


# ---- backward ------------------------------------------------------------------------------------
DO_, DQ_, DK_, DV_, WB_ = (A + (9 + i) * (1 << 32) for i in range(5))
GOOD_BWD = dict(q=Q, k=K, v=V, o=O, do=DO_, lse=L, dq=DQ_, dk=DK_, dv=DV_, B=2, H=8, H_kv=2,
                N=300, d=128, scale=0.1, causal=1, layout=0, ws=WB_, ws_bytes=1 << 30)


def _call_bwd(**kw):
    a = dict(GOOD_BWD, **kw)
    return fa.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
                     a["B"], a["H"], a["H_kv"], a["N"], a["d"], a["scale"], a["causal"],
                     a["layout"], a["ws"], a["ws_bytes"], None)


BAD_BWD = [
    (dict(ws=0), fa.FA_ERR_INVALID_ARG),
    (dict(do=0), fa.FA_ERR_INVALID_ARG),
    (dict(dk=0), fa.FA_ERR_INVALID_ARG),
    (dict(o=0), fa.FA_ERR_INVALID_ARG),
    (dict(ws_bytes=2 * 8 * 300 * 4 - 1), fa.FA_ERR_INVALID_ARG),  # short of even the D part
    (dict(N=0), fa.FA_ERR_INVALID_ARG),
    (dict(H_kv=3), fa.FA_ERR_INVALID_ARG),
    (dict(layout=2), fa.FA_ERR_INVALID_ARG),
    (dict(causal=-1), fa.FA_ERR_INVALID_ARG),
    (dict(scale=-1.0), fa.FA_ERR_INVALID_ARG),
    (dict(d=256), fa.FA_ERR_UNSUPPORTED),
    (dict(dq=DQ_ + 4), fa.FA_ERR_ALIGNMENT),
    (dict(do=DO_ + 2), fa.FA_ERR_ALIGNMENT),
    (dict(dq=Q), fa.FA_ERR_INVALID_ARG),      # dq overlaps q
    (dict(dv=DO_), fa.FA_ERR_INVALID_ARG),    # dv overlaps dout
    (dict(dk=DV_), fa.FA_ERR_INVALID_ARG),    # dk overlaps dv
    (dict(ws=L), fa.FA_ERR_INVALID_ARG),      # workspace overlaps lse
]


@pytest.mark.parametrize("kw,code", BAD_BWD, ids=[str(b[0]) for b in BAD_BWD])
def test_bad_backward_arguments_are_refused(kw, code):
    assert _call_bwd(**kw) == code


def test_backward_workspace_bytes():
    f = fa.fa_bwd_workspace_bytes
    # D (B*H*N floats, 256-byte aligned) only, when no query-head split is needed (MHA)
    assert f(2, 8, 8, 300, 128) == 2 * 8 * 300 * 4
    # Llama-3-8B grouped layer: 32 key blocks x 8 K/V heads = 256 workgroups -> 2 splits at
    # d = 128 (about two workgroups per CU), 4 at d = 64 (about four), each with fp32 partial dK
    # and dV
    assert f(1, 32, 8, 8192, 128) == 32 * 8192 * 4 + 2 * 2 * 8 * 8192 * 128 * 4
    assert f(1, 32, 8, 8192, 64) == 32 * 8192 * 4 + 2 * 4 * 8 * 8192 * 64 * 4
    # few workgroups: the split is the largest divisor of the group size up to the need
    assert f(2, 8, 2, 300, 128) == 19200 + 2 * 4 * 2 * 2 * 300 * 128 * 4
    assert f(0, 8, 8, 300, 128) == 0
    assert f(1, 1, 1, (1 << 22) + 1, 128) == 0
    assert f(1, 8, 3, 300, 128) == 0
    assert f(1, 8, 8, 300, 96) == 0


def test_backward_binding_checks_tensors_before_calling():
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 2, 8)
    with pytest.raises(ValueError):
        fa.backward(q, q, q, q, lse, q, layout="bnhd ")
    with pytest.raises(ValueError):
        fa.backward(q, q, q, q, lse.double(), q)   # lse must be float32
    with pytest.raises(ValueError):
        fa.backward(q, q, q, q[:, :, :4].contiguous(), lse, q)  # o's shape differs from q's
    with pytest.raises(ValueError):
        fa.backward(q, q, q, q, lse, q)  # CPU tensors (shapes are fine)


# ---- score variants -------------------------------------------------------------------------------
SL_, BI_ = A + 15 * (1 << 32), A + 16 * (1 << 32)
GOOD_EXT = dict(q=Q, k=K, v=V, o=O, lse=L, B=2, H=8, H_kv=2, N=300, d=128, scale=0.1, causal=1,
                layout=0, wl=64, wr=-1, slopes=SL_, bias=BI_, bbs=0, bhs=300 * 304, brs=304)


def _call_ext(**kw):
    a = dict(GOOD_EXT, **kw)
    return fa.fa_fwd_ext(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["H_kv"],
                         a["N"], a["d"], a["scale"], a["causal"], a["layout"], a["wl"], a["wr"],
                         a["slopes"], a["bias"], a["bbs"], a["bhs"], a["brs"], None)


BAD_EXT = [
    (dict(wl=-2), fa.FA_ERR_INVALID_ARG),
    (dict(wr=-5), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(brs=299), fa.FA_ERR_INVALID_ARG),          # rows shorter than N
    (dict(brs=302), fa.FA_ERR_ALIGNMENT),             # row stride not a multiple of 8
    (dict(brs=308), fa.FA_ERR_ALIGNMENT),
    (dict(bias=BI_ + 2), fa.FA_ERR_ALIGNMENT),
    (dict(bias=BI_ + 8), fa.FA_ERR_ALIGNMENT),        # rows must start 16-byte aligned
    (dict(bhs=300 * 304 + 4), fa.FA_ERR_ALIGNMENT),
    (dict(bbs=12), fa.FA_ERR_ALIGNMENT),
    (dict(bhs=-1), fa.FA_ERR_INVALID_ARG),
    (dict(slopes=SL_ + 2), fa.FA_ERR_ALIGNMENT),
    (dict(N=40000, brs=40000, bhs=0), fa.FA_ERR_UNSUPPORTED),  # one matrix over 2 GiB
    (dict(bias=O), fa.FA_ERR_INVALID_ARG),            # bias overlaps o
    (dict(slopes=L), fa.FA_ERR_INVALID_ARG),          # slopes overlap lse
    (dict(H_kv=3), fa.FA_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("kw,code", BAD_EXT, ids=[str(b[0]) for b in BAD_EXT])
def test_bad_variant_arguments_are_refused(kw, code):
    assert _call_ext(**kw) == code


def test_d256_is_accepted_by_the_bf16_forward_only():
    # the fp32 path refuses d = 256 before any HIP call
    assert fa.fa_fwd_f32(Q, K, V, O, L, 1, 2, 64, 256, 0.1, 0, None) == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_fwd_gqa_f32(Q, K, V, O, L, 1, 2, 2, 64, 256, 0.1, 0, 0, None) == \
        fa.FA_ERR_UNSUPPORTED
    assert fa.fa_bwd(Q, K, V, O, DO_, L, DQ_, DK_, DV_, 1, 2, 2, 64, 256, 0.1, 0, 0, WB_, 1 << 30,
                     None) == fa.FA_ERR_UNSUPPORTED

"""The C-ABI library: it loads, exports what include/cgr.h declares, and its
host-side argument checks reject bad calls before anything is enqueued.

No compute call is made here: every call below fails validation first, with
pointers that are never dereferenced. These tests skip when a GPU is visible
(the GPU tests cover the same checks with real tensors).
"""

import ctypes
import os
import re
import subprocess

import pytest

import causal_gqa_rope_amd as cgr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cgr.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"CGR_API\s+[\w\s\*]+?\b(cgr_\w+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    assert declared_functions() == sorted(cgr.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = cgr.library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", cgr.library_path], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(declared_functions()) <= exported
    # Only the C entry points are exported: the kernels and helpers stay hidden.
    assert {s for s in exported if s.startswith("cgr")} == set(declared_functions())


def test_library_leaves_the_hip_runtime_to_the_process():
    out = subprocess.run(["readelf", "-d", cgr.library_path], capture_output=True, text=True,
                         check=True).stdout
    assert "amdhip64" not in out, "libcgr must not pull in its own HIP runtime"


def test_version_and_workspace_size():
    assert cgr.cgr_version() == 10000
    lib = cgr.library()
    assert lib.cgr_attn_fwd_workspace_size(0, 16, 2, 64) == 0
    # whole tiles of 64 keys (32 for head_dim 256), 2 bytes per element, then
    # 256 bytes for the attention kernel's work counter
    assert lib.cgr_attn_fwd_workspace_size(2, 100, 8, 128) == 2 * 8 * 2 * 64 * 128 * 2 + 256
    assert lib.cgr_attn_fwd_workspace_size(1, 64, 1, 32) == 64 * 32 * 2 + 256
    assert lib.cgr_attn_fwd_workspace_size(1, 33, 2, 256) == 2 * 2 * 32 * 256 * 2 + 256
    assert lib.cgr_attn_fwd_workspace_size(1, 16, 2, 96) == 0
    assert lib.cgr_attn_fwd_varlen_workspace_size(0, 10) == 0
    assert lib.cgr_attn_fwd_varlen_workspace_size(1, -1) == 0
    small = lib.cgr_attn_fwd_varlen_workspace_size(1, 1)
    big = lib.cgr_attn_fwd_varlen_workspace_size(32, 32226)
    assert 16 < small < big
    # one 8-byte item per (sequence, query block of >= 64 rows), plus a header
    assert big >= 16 + 8 * (32226 // 64 + 32)
    # with the once-rotated keys: the schedule, then (on a 256-byte boundary)
    # per K/V head ceil(total / BN) + num_seqs tile images
    up = lambda x: (x + 255) // 256 * 256
    rot = lib.cgr_attn_fwd_varlen_rotated_workspace_size
    assert rot(32, 32226, 1, 128) == up(big) + 1 * ((32226 + 63) // 64 + 32) * 64 * 128 * 2
    assert rot(3, 100, 2, 256) == (up(lib.cgr_attn_fwd_varlen_workspace_size(3, 100))
                                   + 2 * ((100 + 31) // 32 + 3) * 32 * 256 * 2)
    assert rot(0, 10, 1, 64) == 0 and rot(1, -1, 1, 64) == 0 and rot(1, 10, 0, 64) == 0
    assert rot(1, 10, 1, 96) == 0


no_gpu = pytest.mark.skipif(
    __import__("torch").cuda.is_available(), reason="host-only checks with placeholder pointers")

P = ctypes.c_void_p(0x10000)      # 16-byte aligned placeholder, never dereferenced
PMIS = ctypes.c_void_p(0x10002)   # misaligned placeholder


def dense(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, B=1, T=16, H=4, KV=2, D=64, dtype=1, cos=P, sin=P,
             P=16, style=0, mask=1, window=0, scale=0.0, qk=0, seqlens=None, ws=None, wsb=0)
    a.update(kw)
    lib = cgr.library()
    st = lib.cgr_gqa_rope_attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["T"], a["H"],
                                   a["KV"], a["D"], a["dtype"], a["cos"], a["sin"], a["P"],
                                   a["style"], a["mask"], a["window"], a["scale"], a["qk"], a["seqlens"],
                                   a["ws"], a["wsb"], None)
    return st, lib.cgr_last_error().decode()


@no_gpu
@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=None), 1, "non-null"),
    (dict(cos=None), 1, "non-null"),
    (dict(B=0), 1, ">= 1"),
    (dict(T=-3), 1, ">= 1"),
    (dict(H=0), 1, ">= 1"),
    (dict(H=6, KV=4), 1, "divisible"),
    (dict(D=63), 1, "even"),
    (dict(D=96), 2, "not one of"),
    (dict(D=512), 2, "not one of"),
    (dict(D=256, dtype=0), 2, "256"),
    (dict(dtype=7), 2, "dtype"),
    (dict(style=3), 2, "style"),
    (dict(mask=2), 2, "mask"),
    (dict(qk=9), 2, "qk operand"),
    (dict(scale=float("nan")), 1, "finite"),
    (dict(q=PMIS), 3, "aligned"),
    (dict(sin=PMIS), 3, "aligned"),
    (dict(P=15), 1, "positions"),
    (dict(window=-1), 1, "window"),
    (dict(window=8, mask=0), 1, "CGR_MASK_CAUSAL"),
    (dict(ws=P, wsb=100), 4, "needs"),
    (dict(seqlens=PMIS), 3, "seqlens"),
    # 32-bit byte offsets inside one sequence: (T + 256) * H * d * 4 must fit in int32
    (dict(T=130816, H=32, KV=8, D=128, P=130816), 2, "exceeds 2 GiB"),
    (dict(ws=PMIS, wsb=1 << 20), 3, "aligned"),
])
def test_dense_rejects_bad_arguments(kw, status, needle):
    st, msg = dense(**kw)
    assert st == status, msg
    assert needle in msg


def rotate_keys(**kw):
    a = dict(k=P, B=1, T=16, KV=2, D=64, dtype=1, cos=P, sin=P, P=16, style=0, qk=0, seqlens=None, ws=P,
             wsb=1 << 20)
    a.update(kw)
    lib = cgr.library()
    st = lib.cgr_attn_fwd_rotate_keys(a["k"], a["B"], a["T"], a["KV"], a["D"], a["dtype"], a["cos"], a["sin"],
                                      a["P"], a["style"], a["qk"], a["seqlens"], a["ws"], a["wsb"], None)
    return st, lib.cgr_last_error().decode()


def rotated(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, B=1, T=16, H=4, KV=2, D=64, dtype=1, cos=P, sin=P,
             P=16, style=0, mask=1, window=0, scale=0.0, qk=0, seqlens=None, ws=P, wsb=1 << 20)
    a.update(kw)
    lib = cgr.library()
    st = lib.cgr_gqa_rope_attn_fwd_rotated(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["T"], a["H"],
                                           a["KV"], a["D"], a["dtype"], a["cos"], a["sin"], a["P"], a["style"],
                                           a["mask"], a["window"], a["scale"], a["qk"], a["seqlens"], a["ws"],
                                           a["wsb"], None)
    return st, lib.cgr_last_error().decode()


@no_gpu
@pytest.mark.parametrize("fn,kw,status,needle", [
    (rotate_keys, dict(ws=None), 4, "workspace"),
    (rotate_keys, dict(wsb=100), 4, "needs"),
    (rotate_keys, dict(dtype=0), 2, "CGR_BF16"),
    (rotate_keys, dict(k=None), 1, "non-null"),
    (rotate_keys, dict(P=15), 1, "positions"),
    (rotate_keys, dict(D=96), 2, "not one of"),
    (rotate_keys, dict(ws=PMIS), 3, "aligned"),
    (rotated, dict(ws=None), 4, "workspace"),
    (rotated, dict(wsb=100), 4, "needs"),
    (rotated, dict(dtype=0), 2, "CGR_BF16"),
    (rotated, dict(H=6, KV=4), 1, "divisible"),
    (rotated, dict(window=4, mask=0), 1, "CGR_MASK_CAUSAL"),
])
def test_rotate_keys_and_rotated_reject_bad_arguments(fn, kw, status, needle):
    st, msg = fn(**kw)
    assert st == status, msg
    assert needle in msg


def varlen_noalloc(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, cu=P, n=2, total=100, maxs=60, H=4, KV=2, D=64, dtype=1, cos=P, sin=P,
             P=64, style=0, mask=1, window=0, scale=0.0, qk=0, status=None)
    a.update(kw)
    lib = cgr.library()
    st = lib.cgr_gqa_rope_attn_fwd_varlen_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu"], a["n"],
                                                  a["total"], a["maxs"], a["H"], a["KV"], a["D"], a["dtype"],
                                                  a["cos"], a["sin"], a["P"], a["style"], a["mask"], a["window"],
                                                  a["scale"], a["qk"], a["status"], None)
    return st, lib.cgr_last_error().decode()


@no_gpu
@pytest.mark.parametrize("kw,status,needle", [
    # 16 bytes + 8 per (sequence, 32-row block): past 1 MiB from ~4.19 M tokens
    (dict(total=4_200_000, maxs=4_200_000, P=4_200_000, H=1, KV=1, D=32), 4, "no-alloc scratch holds"),
    (dict(status=PMIS), 3, "device_status"),
    (dict(q=None), 1, "non-null"),
    (dict(cu=None), 1, "cu_seqlens"),
    (dict(n=0), 1, "num_seqs"),
    (dict(maxs=200), 1, "exceeds total_tokens"),
    (dict(H=6, KV=4), 1, "divisible"),
    (dict(window=3, mask=0), 1, "CGR_MASK_CAUSAL"),
])
def test_varlen_noalloc_rejects_bad_arguments(kw, status, needle):
    st, msg = varlen_noalloc(**kw)
    assert st == status, msg
    assert needle in msg


def fp8(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, B=1, T=16, H=4, KV=2, D=128, qd=0.01, kd=0.01, vd=0.01, cos=P, sin=P,
             P=16, style=0, mask=1, scale=0.0, seqlens=None, ws=P, wsb=1 << 20)
    a.update(kw)
    lib = cgr.library()
    st = lib.cgr_gqa_rope_attn_fwd_fp8(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["T"], a["H"], a["KV"],
                                       a["D"], a["qd"], a["kd"], a["vd"], a["cos"], a["sin"], a["P"], a["style"],
                                       a["mask"], a["scale"], a["seqlens"], a["ws"], a["wsb"], None)
    return st, lib.cgr_last_error().decode()


@no_gpu
@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=None), 1, "non-null"),
    (dict(T=0), 1, ">= 1"),
    (dict(H=6, KV=4), 1, "divisible"),
    (dict(D=64), 2, "head_dim 128"),
    (dict(qd=0.0), 1, "descales"),
    (dict(vd=float("inf")), 1, "descales"),
    (dict(style=5), 2, "style"),
    (dict(mask=3), 2, "mask"),
    (dict(k=PMIS), 3, "aligned"),
    (dict(P=15), 1, "positions"),
    (dict(ws=None), 4, "workspace"),
    (dict(wsb=100), 4, "needs"),
    (dict(qd=1e30, kd=1e30), 1, "out of range"),
    (dict(seqlens=ctypes.c_void_p(0x10002)), 3, "seqlens"),
])
def test_fp8_rejects_bad_arguments(kw, status, needle):
    st, msg = fp8(**kw)
    assert st == status, msg
    assert needle in msg


def test_fp8_workspace_size():
    lib = cgr.library()
    assert lib.cgr_attn_fwd_fp8_workspace_size(1, 16, 2, 64) == 0
    assert lib.cgr_attn_fwd_fp8_workspace_size(0, 16, 2, 128) == 0
    # two 8 KiB tile images (64 keys x 128 bytes) per (entry, K/V head, tile)
    assert lib.cgr_attn_fwd_fp8_workspace_size(2, 100, 3, 128) == 2 * 2 * 3 * 2 * 8192


def varlen(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, cu=P, nseq=2, total=100, maxlen=60, H=4, KV=1, D=128,
             dtype=1, cos=P, sin=P, P=60, style=0, mask=1, window=0, scale=0.0, qk=0, ws=P, wsb=1 << 20)
    a.update(kw)
    lib = cgr.library()
    st = lib.cgr_gqa_rope_attn_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu"],
                                          a["nseq"], a["total"], a["maxlen"], a["H"], a["KV"],
                                          a["D"], a["dtype"], a["cos"], a["sin"], a["P"],
                                          a["style"], a["mask"], a["window"], a["scale"], a["qk"],
                                          a["ws"], a["wsb"], None)
    return st, lib.cgr_last_error().decode()


@no_gpu
@pytest.mark.parametrize("kw,status,needle", [
    (dict(cu=None), 1, "cu_seqlens"),
    (dict(nseq=0), 1, "num_seqs"),
    (dict(total=-1), 1, ">= 0"),
    (dict(maxlen=101), 1, "exceeds"),
    (dict(P=59), 1, "positions"),
    (dict(ws=None), 4, "workspace"),
    (dict(wsb=16), 4, "needs"),
    (dict(ws=PMIS), 3, "aligned"),
    (dict(H=3, KV=2), 1, "divisible"),
    (dict(D=48), 2, "not one of"),
])
def test_varlen_rejects_bad_arguments(kw, status, needle):
    st, msg = varlen(**kw)
    assert st == status, msg
    assert needle in msg


@no_gpu
@pytest.mark.parametrize("args,needle", [
    ((0, 64, 1e4), ">= 1"),
    ((16, 63, 1e4), "even"),
    ((16, 0, 1e4), "even"),
    ((16, 64, 0.0), "positive"),
    ((16, 64, float("inf")), "positive"),
])
def test_rope_tables_rejects_bad_arguments(args, needle):
    lib = cgr.library()
    st = lib.cgr_rope_tables(args[0], args[1], args[2], P, P, None)
    assert st == 1
    assert needle in lib.cgr_last_error().decode()


@no_gpu
def test_python_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 4, 2, 64)
    with pytest.raises(cgr.CgrError):
        cgr.gqa_rope_attn_fwd(x, x, x, torch.zeros(4, 32), torch.zeros(4, 32))


def test_backward_workspace_size():
    lib = cgr.library()
    assert lib.cgr_attn_bwd_workspace_size(0, 16, 4, 2, 64) == 0
    assert lib.cgr_attn_bwd_workspace_size(1, 16, 4, 0, 64) == 0
    # rotated q and k (2 bytes each) on 256-byte boundaries, then 2 floats per
    # (head, row) over rows padded to 32, then 256 bytes of claim counters
    n = lib.cgr_attn_bwd_workspace_size(2, 100, 8, 2, 128)
    assert n == 2 * 100 * 8 * 128 * 2 + 2 * 100 * 2 * 128 * 2 + 2 * 8 * 4 * 64 * 4 + 256
    # more than 4 query heads per K/V head (G = 16): f32 partial sums of dk
    # and dv for ceil(16 / 4) = 4 head groups follow the per-tile values
    n = lib.cgr_attn_bwd_workspace_size(1, 100, 16, 1, 64)
    assert n == 100 * 16 * 64 * 2 + (100 * 64 * 2 + 255) // 256 * 256 + 16 * 4 * 64 * 4 + 2 * 4 * 100 * 64 * 4 + 256


def backward(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, dout=P, dq=P, dk=P, dv=P, B=1, T=16, H=4, KV=2, D=64,
             dtype=1, cos=P, sin=P, P=16, style=0, mask=1, window=0, scale=0.0, qk=0,
             ws=ctypes.c_void_p(0x10000), wsb=1 << 20)
    a.update(kw)
    lib = cgr.library()
    st = lib.cgr_gqa_rope_attn_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], a["dq"],
                                   a["dk"], a["dv"], a["B"], a["T"], a["H"], a["KV"], a["D"],
                                   a["dtype"], a["cos"], a["sin"], a["P"], a["style"], a["mask"],
                                   a["window"], a["scale"], a["qk"], a["ws"], a["wsb"], None)
    return st, lib.cgr_last_error().decode()


@no_gpu
@pytest.mark.parametrize("kw,status,needle", [
    (dict(lse=None), 1, "non-null"),
    (dict(dout=None), 1, "non-null"),
    (dict(dk=None), 1, "non-null"),
    (dict(dtype=0), 2, "bf16"),
    (dict(dq=PMIS), 3, "aligned"),
    (dict(ws=None), 4, "workspace"),
    (dict(wsb=100), 4, "needs"),
    (dict(ws=ctypes.c_void_p(0x10010)), 3, "256-byte"),
    (dict(H=6, KV=4), 1, "divisible"),
    (dict(D=80), 2, "not one of"),
    (dict(D=256), 2, "backward is built for"),
    (dict(T=0), 1, ">= 1"),
    (dict(P=15), 1, "positions"),
    (dict(window=4, mask=0), 1, "CGR_MASK_CAUSAL"),
])
def test_backward_rejects_bad_arguments(kw, status, needle):
    st, msg = backward(**kw)
    assert st == status, msg
    assert needle in msg


def test_backward_varlen_workspace_size():
    lib = cgr.library()
    assert lib.cgr_attn_bwd_varlen_workspace_size(0, 16, 4, 2, 64) == 0
    assert lib.cgr_attn_bwd_varlen_workspace_size(1, -1, 4, 2, 64) == 0
    assert lib.cgr_attn_bwd_varlen_workspace_size(1, 16, 4, 0, 64) == 0
    # rotated q and k over the packed rows on 256-byte boundaries, then 2
    # floats per (head, row) over ceil(total / 32) + num_seqs slots of 32 rows,
    # then 256 bytes of claim counters
    up = lambda x: (x + 255) // 256 * 256
    n = lib.cgr_attn_bwd_varlen_workspace_size(3, 100, 8, 2, 128)
    assert n == up(100 * 8 * 128 * 2) + up(100 * 2 * 128 * 2) + 8 * (4 + 3) * 64 * 4 + 256
    n = lib.cgr_attn_bwd_varlen_workspace_size(2, 33, 4, 1, 64)
    assert n == up(33 * 4 * 64 * 2) + up(33 * 1 * 64 * 2) + 4 * (2 + 2) * 64 * 4 + 256
    n = lib.cgr_attn_bwd_varlen_workspace_size(2, 33, 6, 1, 64)  # G = 6: two head groups
    assert n == up(33 * 6 * 64 * 2) + up(33 * 1 * 64 * 2) + up(6 * (2 + 2) * 64 * 4) + 2 * 2 * 33 * 64 * 4 + 256


def backward_varlen(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, dout=P, dq=P, dk=P, dv=P, cu=P, nseq=2, total=100, maxlen=60, H=4, KV=2,
             D=64, dtype=1, cos=P, sin=P, P=60, style=0, mask=1, window=0, scale=0.0, qk=0,
             ws=ctypes.c_void_p(0x10000), wsb=1 << 20)
    a.update(kw)
    lib = cgr.library()
    st = lib.cgr_gqa_rope_attn_bwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], a["dq"], a["dk"],
                                          a["dv"], a["cu"], a["nseq"], a["total"], a["maxlen"], a["H"], a["KV"],
                                          a["D"], a["dtype"], a["cos"], a["sin"], a["P"], a["style"], a["mask"],
                                          a["window"], a["scale"], a["qk"], a["ws"], a["wsb"], None)
    return st, lib.cgr_last_error().decode()


@no_gpu
@pytest.mark.parametrize("kw,status,needle", [
    (dict(cu=None), 1, "cu_seqlens"),
    (dict(nseq=0), 1, "num_seqs"),
    (dict(total=-1), 1, ">= 0"),
    (dict(maxlen=101), 1, "exceeds"),
    (dict(P=59), 1, "positions"),
    (dict(lse=None), 1, "non-null"),
    (dict(dv=None), 1, "non-null"),
    (dict(dtype=0), 2, "bf16"),
    (dict(dk=PMIS), 3, "aligned"),
    (dict(ws=None), 4, "workspace"),
    (dict(wsb=100), 4, "needs"),
    (dict(ws=ctypes.c_void_p(0x10010)), 3, "256-byte"),
    (dict(H=6, KV=4), 1, "divisible"),
    (dict(D=256), 2, "backward is built for"),
    (dict(window=4, mask=0), 1, "CGR_MASK_CAUSAL"),
])
def test_backward_varlen_rejects_bad_arguments(kw, status, needle):
    st, msg = backward_varlen(**kw)
    assert st == status, msg
    assert needle in msg


def test_decode_workspace_size():
    lib = cgr.library()
    assert lib.cgr_attn_decode_workspace_size(0, 1, 10, 4, 2, 64) == 0
    assert lib.cgr_attn_decode_workspace_size(2, 5, 4, 4, 2, 64) == 0   # max_seqlen < Tq
    assert lib.cgr_attn_decode_workspace_size(2, 1, 10, 6, 4, 64) == 0  # heads not divisible
    small = lib.cgr_attn_decode_workspace_size(1, 1, 32, 4, 2, 64)
    big = lib.cgr_attn_decode_workspace_size(16, 1, 8192, 32, 8, 128)
    assert 256 < small < big


def decode_call(**kw):
    a = dict(q=P, k=P, v=P, lens=P, o=P, lse=None, B=2, Tq=1, S=64, sb=64 * 2 * 64, st=2 * 64, sh=64,
             M=64, H=4, KV=2, D=64, dtype=1, cos=P, sin=P, P=64, style=0, window=0, scale=0.0,
             ws=ctypes.c_void_p(0x10000), wsb=1 << 20)
    a.update(kw)
    lib = cgr.library()
    st = lib.cgr_gqa_rope_attn_decode(a["q"], a["k"], a["v"], a["lens"], a["o"], a["lse"], a["B"], a["Tq"],
                                      a["S"], a["sb"], a["st"], a["sh"], a["M"], a["H"], a["KV"], a["D"],
                                      a["dtype"], a["cos"], a["sin"], a["P"], a["style"], a["window"],
                                      a["scale"], a["ws"], a["wsb"], None)
    return st, lib.cgr_last_error().decode()


@no_gpu
@pytest.mark.parametrize("kw,status,needle", [
    (dict(lens=None), 1, "cache_seqlens"),
    (dict(B=0), 1, ">= 1"),
    (dict(Tq=0), 1, ">= 1"),
    (dict(M=65), 1, "cache_capacity"),
    (dict(Tq=3, M=2), 1, "max_seqlen"),
    (dict(P=63), 1, "positions"),
    (dict(dtype=0), 2, "bf16"),
    (dict(st=60), 1, "multiples of 8"),
    (dict(sh=32), 1, "head_dim"),
    (dict(ws=None), 4, "workspace"),
    (dict(wsb=300), 4, "needs"),
    (dict(H=6, KV=4), 1, "divisible"),
    (dict(D=48), 2, "not one of"),
    (dict(D=256), 2, "decode is built for"),
    (dict(window=-2), 1, "window"),
])
def test_decode_rejects_bad_arguments(kw, status, needle):
    st, msg = decode_call(**kw)
    assert st == status, msg
    assert needle in msg


@no_gpu
@pytest.mark.parametrize("kw,status,needle", [
    (dict(x=None), 1, "non-null"),
    (dict(pos=None), 1, "non-null"),
    (dict(n=-1), 1, ">= 0"),
    (dict(nh=0), 1, ">= 1"),
    (dict(d=48), 2, "not one of"),
    (dict(dtype=5), 2, "dtype"),
    (dict(style=2), 2, "style"),
    (dict(x=PMIS), 3, "aligned"),
])
def test_rope_rotate_rejects_bad_arguments(kw, status, needle):
    a = dict(x=P, out=P, pos=P, n=4, nh=2, d=64, dtype=1, cos=P, sin=P, P=16, style=0, status=None)
    a.update(kw)
    lib = cgr.library()
    st = lib.cgr_rope_rotate(a["x"], a["out"], a["pos"], a["n"], a["nh"], a["d"], a["dtype"], a["cos"],
                             a["sin"], a["P"], a["style"], a["status"], None)
    assert st == status, lib.cgr_last_error().decode()
    assert needle in lib.cgr_last_error().decode()

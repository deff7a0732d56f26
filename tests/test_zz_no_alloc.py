"""The packed forward that allocates nothing (cgr_gqa_rope_attn_fwd_varlen_noalloc),
through the C-ABI, against the packed forward with a workspace: two calls in a
row, the second on a smaller batch, each giving the bits of the workspace call
(and so within the bf16 bar of the oracle); malformed cu_seqlens reported
through device_status with the output untouched."""

import numpy as np
import pytest
import torch

import causal_gqa_rope_amd as cgr
import oracle
from tests.gpu_cases import announce, assert_close, f64

pytestmark = pytest.mark.gpu


def packed(lengths, H, KV, d, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    total = sum(lengths)
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lengths), 0).to(torch.int32)
    q = torch.randn((total, H, d), generator=g).to(torch.bfloat16)
    k = torch.randn((total, KV, d), generator=g).to(torch.bfloat16)
    v = torch.randn((total, KV, d), generator=g).to(torch.bfloat16)
    return q, k, v, cu


@pytest.mark.parametrize("lengths,H,KV,d,causal,window", [
    # large then small: the second call reuses the array the first one filled
    ([1935, 16, 700, 1024, 33, 0, 2048], 16, 1, 128, True, 0),
    ([5, 1, 0, 130], 16, 1, 128, True, 0),
    ([300, 17, 64], 6, 2, 64, False, 0),
    ([120, 0, 77], 8, 2, 128, True, 40),
])
def test_noalloc_matches_the_workspace_call(gpu, lengths, H, KV, d, causal, window):
    announce(f"no-alloc packed forward lengths={lengths} H={H} KV={KV} d={d} causal={causal} W={window}")
    q, k, v, cu = packed(lengths, H, KV, d, seed=sum(lengths) + H)
    qd, kd, vd, cud = q.to(gpu), k.to(gpu), v.to(gpu), cu.to(gpu)
    ms = max(max(lengths), 1)
    cos, sin = cgr.rope_tables(ms, d, 5e5, device=gpu)
    kw = dict(causal=causal, window=window)
    o_ref, l_ref = cgr.gqa_rope_attn_fwd_varlen(qd, kd, vd, cud, ms, cos, sin, **kw)
    status = torch.full((1,), -7, dtype=torch.int32, device=gpu)
    for rep in range(2):
        o = torch.full_like(qd, float("nan"))
        lse = torch.full((H, qd.shape[0]), float("nan"), device=gpu)
        cgr.gqa_rope_attn_fwd_varlen_noalloc(qd, kd, vd, cud, ms, cos, sin, out=o, lse=lse, device_status=status,
                                             **kw)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), f"call {rep}"
    if sum(lengths):
        ro, rl = oracle.attention_varlen(q, k, v, cu.numpy(), causal=causal, base=5e5, window=window)
        assert_close("no-alloc", f64(o), ro, f64(lse), rl, "bf16")


def test_noalloc_two_calls_second_smaller(gpu):
    """Back to back on one stream without a sync between them: a large batch,
    then a smaller one; each matches its workspace call bit for bit."""
    announce("no-alloc: two calls in a row, the second smaller")
    big = packed([1500, 900, 3, 2048, 64], 16, 1, 128, seed=71)
    small = packed([40, 0, 129], 16, 1, 128, seed=72)
    outs = []
    for (q, k, v, cu) in (big, small):
        qd, kd, vd, cud = q.to(gpu), k.to(gpu), v.to(gpu), cu.to(gpu)
        ms = int((cu[1:] - cu[:-1]).max())
        cos, sin = cgr.rope_tables(ms, 128, 1e4, device=gpu)
        o = torch.empty_like(qd)
        lse = torch.empty((16, qd.shape[0]), device=gpu)
        cgr.gqa_rope_attn_fwd_varlen_noalloc(qd, kd, vd, cud, ms, cos, sin, out=o, lse=lse)
        outs.append((qd, kd, vd, cud, ms, cos, sin, o, lse))
    torch.cuda.synchronize()
    for (qd, kd, vd, cud, ms, cos, sin, o, lse) in outs:
        o_ref, l_ref = cgr.gqa_rope_attn_fwd_varlen(qd, kd, vd, cud, ms, cos, sin)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)


def test_noalloc_malformed_cu_seqlens(gpu):
    announce("no-alloc: malformed cu_seqlens")
    q = torch.randn(9, 2, 64, device=gpu).to(torch.bfloat16)
    kv = torch.randn(9, 1, 64, device=gpu).to(torch.bfloat16)
    cos, sin = cgr.rope_tables(8, 64, 1e4, device=gpu)
    status = torch.zeros(1, dtype=torch.int32, device=gpu)
    o = torch.full_like(q, float("nan"))
    cgr.gqa_rope_attn_fwd_varlen_noalloc(q, kv, kv, torch.tensor([0, 6, 4, 9], dtype=torch.int32, device=gpu), 6,
                                         cos, sin, out=o, lse=None, device_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 2
    assert torch.isnan(o).all()
    # The next well-formed call clears it again.
    cgr.gqa_rope_attn_fwd_varlen_noalloc(q, kv, kv, torch.tensor([0, 4, 9], dtype=torch.int32, device=gpu), 5,
                                         cos, sin, out=o, lse=None, device_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and not torch.isnan(o).any()

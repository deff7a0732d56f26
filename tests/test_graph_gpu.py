"""Forward calls captured in a HIP graph and replayed give the eager call's bits.

The calls launch only kernels on the caller's stream (no allocation, copy or
memset when the outputs and workspace are passed), so a graph can hold them.
Each case captures two back-to-back calls, then replays the graph three times
with eager work in between (the outputs overwritten by a fill, another eager
call on other tensors, a synchronisation), and compares every replay with the
eager result bit for bit."""

import numpy as np
import pytest
import torch

import causal_gqa_rope_amd as cgr
import workloads as W
from tests.gpu_cases import announce

pytestmark = pytest.mark.gpu


def _replays_match(gpu, call, outs, refs, other):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
        call()
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        other()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip(outs, refs):
            assert torch.equal(t, r), f"replay {rep} differs from the eager call"


@pytest.mark.parametrize("B,T,H,KV,d,io", [(2, 300, 8, 2, 128, "bf16"), (1, 64, 4, 2, 32, "f32"),
                                           (8, 256, 6, 2, 64, "bf16")])
def test_dense_forward_in_a_graph(gpu, B, T, H, KV, d, io):
    announce(f"graph replay dense B{B} T{T} H{H} KV{KV} d{d} {io}")
    w = W.custom("graph", B=B, T=T, n_head=H, n_kv_head=KV, head_dim=d, dtype=io, seed=T + d)
    x = W.make_inputs(w)
    q, k, v = (x[n].to(gpu) for n in ("q", "k", "v"))
    cos, sin = cgr.rope_tables(T, d, w.base, device=gpu)
    ws = (torch.empty(cgr.cgr_attn_fwd_workspace_size(B, T, KV, d), dtype=torch.uint8, device=gpu)
          if io == "bf16" else False)
    o_ref, l_ref = cgr.gqa_rope_attn_fwd(q, k, v, cos, sin, workspace=ws)
    o, lse = torch.empty_like(o_ref), torch.empty_like(l_ref)
    q2 = torch.randn_like(q.float()).to(q.dtype)
    o2, l2 = torch.empty_like(o), torch.empty_like(lse)
    torch.cuda.synchronize()
    _replays_match(gpu, lambda: cgr.gqa_rope_attn_fwd(q, k, v, cos, sin, out=o, lse=lse, workspace=ws),
                   (o, lse), (o_ref, l_ref),
                   lambda: cgr.gqa_rope_attn_fwd(q2, k, v, cos, sin, out=o2, lse=l2, workspace=ws))


def test_packed_forward_in_a_graph(gpu):
    lens = [5, 300, 0, 129, 1, 700]
    H, KV, d = 8, 2, 128
    announce(f"graph replay packed lens={lens}")
    gen = torch.Generator("cpu").manual_seed(97)
    total = sum(lens)
    q = torch.randn((total, H, d), generator=gen).to(torch.bfloat16).to(gpu)
    k = torch.randn((total, KV, d), generator=gen).to(torch.bfloat16).to(gpu)
    v = torch.randn((total, KV, d), generator=gen).to(torch.bfloat16).to(gpu)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=gpu)
    cos, sin = cgr.rope_tables(max(lens), d, 1e4, device=gpu)
    ws = torch.empty(cgr.cgr_attn_fwd_varlen_rotated_workspace_size(len(lens), total, KV, d), dtype=torch.uint8,
                     device=gpu)
    o_ref, l_ref = cgr.gqa_rope_attn_fwd_varlen(q, k, v, cu, max(lens), cos, sin, workspace=ws)
    o, lse = torch.empty_like(o_ref), torch.empty_like(l_ref)
    o2, l2 = torch.empty_like(o), torch.empty_like(lse)
    ws2 = torch.empty_like(ws)
    torch.cuda.synchronize()
    _replays_match(gpu, lambda: cgr.gqa_rope_attn_fwd_varlen(q, k, v, cu, max(lens), cos, sin, out=o, lse=lse,
                                                             workspace=ws),
                   (o, lse), (o_ref, l_ref),
                   lambda: cgr.gqa_rope_attn_fwd_varlen(k.repeat_interleave(H // KV, 1).contiguous(), k, v, cu,
                                                        max(lens), cos, sin, out=o2, lse=l2, workspace=ws2))

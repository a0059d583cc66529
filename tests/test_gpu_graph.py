"""fa_fwd, fa_bwd, fa_fwd_varlen and the decode entry points captured in one
HIP graph (torch.cuda.graph on the current stream): every replay reproduces
the eager calls bit for bit.  The library launches only kernels on the
caller's stream (no allocation, no memset, no synchronisation), which is what
capture needs; the replays are interleaved with eager work on other inputs
and host synchronisations, and each one is checked on its own."""
import pytest
import torch

import io_aware_exact_qk_amd as fa
from workloads import dense_case, decode_case, varlen_case
from _helpers import DEV, say

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t.view(torch.int32)


def test_graph_replays_match_eager():
    c = dense_case(B=2, Sq=700, Sk=700, Hq=4, Hkv=2, D=128, dtype="bf16", seed=61, causal=True)
    q, k, v, do = (t.to(DEV) for t in (c.q, c.k, c.v, c.dout))
    B, S, Hq, D = q.shape
    out, lse = torch.empty_like(q), torch.empty(B, Hq, S, device=DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.lib().fa_bwd_workspace_size(B, S, S, Hq, 2, D, 0), device=DEV, dtype=torch.uint8)

    vc = varlen_case([300, 5, 131], Hq=4, Hkv=4, D=64, seed=62, causal=True)
    vq, vk, vv = (t.to(DEV) for t in (vc.q, vc.k, vc.v))
    cq, ck = vc.cu_seqlens_q.to(DEV), vc.cu_seqlens_k.to(DEV)
    vout, vlse = torch.empty_like(vq), torch.empty(4, vq.shape[0], device=DEV)
    vws = torch.empty(fa.lib().fa_fwd_varlen_workspace_size(3, vq.shape[0], 4, 64), device=DEV, dtype=torch.uint8)

    dc = decode_case(B=3, Hq=8, Hkv=2, D=128, page=64, seqlens=[300, 77, 64], seed=63, rotary_dim=128)
    dqq = dc.q.to(DEV)
    kc, vcache = dc.k_cache.to(DEV), dc.v_cache.to(DEV)
    sl, bt = dc.cache_seqlens.to(DEV), dc.block_table.to(DEV)
    kn, vn = dc.k_new.to(DEV), dc.v_new.to(DEV)
    cos, sin = dc.rotary_cos.to(DEV), dc.rotary_sin.to(DEV)
    dout_a, dlse_a = torch.empty_like(dqq), torch.empty(3, 8, 1, device=DEV)
    dout_b, dlse_b = torch.empty_like(dqq), torch.empty(3, 8, 1, device=DEV)
    dws = torch.empty(fa.lib().fa_kvcache_workspace_size(3, 1, 8, 128, 4), device=DEV, dtype=torch.uint8)

    def calls():
        fa.fa_fwd(q, k, v, out=out, lse=lse, scale=c.scale, causal=True)
        fa.fa_bwd(q, k, v, out, do, lse, dq=dq, dk=dk, dv=dv, scale=c.scale, causal=True, workspace=ws)
        fa.fa_fwd_varlen(vq, vk, vv, cq, ck, vc.max_seqlen_q, vc.max_seqlen_k, out=vout, lse=vlse,
                         scale=vc.scale, causal=True, workspace=vws)
        # the append rewrites the same slots with the same values on every call
        fa.fa_fwd_kvcache(dqq, kc, vcache, sl, kn, vn, bt, cos, sin, 128, num_splits=4, out=dout_a,
                          lse=dlse_a, scale=dc.scale, workspace=dws)
        fa.fa_fwd_kvcache_noalloc(dqq, kc, vcache, sl, kn, vn, bt, cos, sin, 128, num_splits=3, out=dout_b,
                                  lse=dlse_b, scale=dc.scale)

    results = (out, lse, dq, dk, dv, vout, vlse, dout_a, dlse_a, dout_b, dlse_b, kc, vcache)
    say("graph: eager reference")
    calls()
    torch.cuda.synchronize()
    ref = [_bits(t).clone() for t in results]

    say("graph: capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()  # warm-up on a side stream, as torch recommends before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()

    other = dense_case(B=1, Sq=256, Sk=256, Hq=2, Hkv=2, D=64, dtype="fp16", seed=64)
    oq, ok_, ov = (t.to(DEV) for t in (other.q, other.k, other.v))
    for rep in range(3):
        for t in results[:-2]:
            t.zero_()  # outputs cleared (the caches keep their contents)
        torch.cuda.synchronize()
        say("graph: replay", rep)
        graph.replay()
        torch.cuda.synchronize()
        for i, (t, r) in enumerate(zip(results, ref)):
            assert torch.equal(_bits(t), r), f"replay {rep}: output {i} differs from the eager call"
        # eager work between replays
        fa.fa_fwd(oq, ok_, ov, causal=False)
        torch.cuda.synchronize()

"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph).

Outside the ATTN_VALIDATE test mode every entry point only enqueues kernels
on the caller's stream: it allocates nothing, issues no memset or copy and
never synchronises, and every buffer a kernel reads before writing is written
by an earlier kernel of the same call.  A captured prefill, backward, paged
decode and shared-prefix decode therefore replay to the same bits as the
eager calls.  Each of several replays is checked against the eager results,
with the outputs overwritten by NaN and the device synchronised between
replays (eager work between replays), so a replay that skipped or reused
anything would show.
"""

import math

import pytest
import torch

import exact_attention_34_amd as ea
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _dev(*ts):
    return [t.to(DEV) for t in ts]


def test_graph_replays_equal_eager_calls():
    g = torch.Generator().manual_seed(21)
    r = lambda *s: torch.randn(*s, generator=g).to(torch.bfloat16)
    # prefill and backward: GQA 8/2, causal, ragged 300 rows
    q, k, v, do = _dev(r(2, 300, 8, 128), r(2, 300, 2, 128), r(2, 300, 2, 128), r(2, 300, 8, 128))
    o = torch.empty_like(q)
    lse = torch.empty(2, 8, 300, device=DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_b = torch.empty(ea.attn_bwd_workspace_size(2, 300, 8), dtype=torch.uint8, device=DEV)
    # paged decode: mixed context lengths (one empty), shuffled table
    dec = workloads.decode_inputs([100, 700, 0, 33, 1500], 8, 2, 128, 16, "bf16", 22)
    dq_, kc, vc, tab, ctx = _dev(dec.q, dec.k_cache, dec.v_cache, dec.block_table,
                                 dec.context_lens)
    mcl = int(dec.context_lens.max())
    dout = torch.empty_like(dq_)
    dlse = torch.empty(5, 8, device=DEV)
    ws_d = torch.empty(ea.paged_attn_decode_workspace_size(5, 8, 2, 128, mcl), dtype=torch.uint8,
                       device=DEV)
    # shared-prefix decode: two groups sharing 300- and 64-token prefixes
    sh = workloads.shared_prefix_inputs([(300, [40, 7, 120]), (64, [0, 19])], 8, 2, 128, 16,
                                        "bf16", 23)
    sq, skc, svc, stab, sctx, sgs, spl = _dev(sh.q, sh.k_cache, sh.v_cache, sh.block_table,
                                              sh.context_lens, sh.group_starts, sh.prefix_lens)
    smcl = int(sh.context_lens.max())
    gsz = int((sh.group_starts[1:] - sh.group_starts[:-1]).max())
    mpl = int(sh.prefix_lens.max())
    sout = torch.empty_like(sq)
    slse = torch.empty(sq.shape[0], 8, device=DEV)
    ws_s = torch.empty(ea.paged_attn_decode_shared_workspace_size(
        sq.shape[0], sh.prefix_lens.numel(), gsz, 8, 2, 128, smcl, mpl),
        dtype=torch.uint8, device=DEV)
    scale = 1.0 / math.sqrt(128)

    def work():
        ea.attn_fwd(q, k, v, causal=True, scale=scale, out=o, lse=lse)
        ea.attn_bwd(q, k, v, o, do, lse, causal=True, scale=scale, dq=dq, dk=dk, dv=dv,
                    workspace=ws_b)
        ea.paged_attn_decode(dq_, kc, vc, tab, ctx, max_context_len=mcl, scale=dec.scale,
                             out=dout, lse=dlse, workspace=ws_d)
        ea.paged_attn_decode_shared(sq, skc, svc, stab, sctx, sgs, spl, max_context_len=smcl,
                                    max_group_size=gsz, max_prefix_len=mpl, scale=sh.scale,
                                    out=sout, lse=slse, workspace=ws_s)

    outs = (o, lse, dq, dk, dv, dout, dlse, sout, slse)
    work()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    for t in ref[:5] + [ref[5], ref[7]]:
        assert bool(torch.isfinite(t.float()).all())

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv", "decode o", "decode lse",
                               "shared o", "shared lse"), ref, outs):
            assert torch.equal(a, b), "replay %d: %s differs from the eager call" % (rep, name)

"""GPU parity of attn_fwd_paged (prefill over a paged KV cache) against the
fp64 oracle on each sequence's logical K/V, through the C ABI; and bitwise
equality with attn_fwd when the cache holds the same contiguous sequence."""

import numpy as np
import pytest
import torch

import exact_attention_34_amd as ea
import oracle
import workloads
from helpers import assert_close, assert_lse_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TDT = {"f16": torch.float16, "bf16": torch.bfloat16}


def _case(ctx, n_q, h_q, h_kv, d, dtype, causal, seed):
    rng = np.random.default_rng(seed)
    dt = TDT[dtype]
    B = len(ctx)
    q = workloads._round(rng.standard_normal((B, n_q, h_q, d)), dtype)
    kl = [workloads._round(rng.standard_normal((c, h_kv, d)), dtype) for c in ctx]
    vl = [workloads._round(rng.standard_normal((c, h_kv, d)), dtype) for c in ctx]
    kc, vc, table, cl = workloads.build_paged(kl, vl, 16, rng=rng, spare_blocks=3)
    mcl = max(1, max(ctx))
    print("case: ctx %s n_q %d hq %d hkv %d d %d %s causal %d" % (ctx, n_q, h_q, h_kv, d, dtype,
                                                                  causal), flush=True)
    out, lse = ea.attn_fwd_paged(q.to(DEV), kc.to(DEV), vc.to(DEV), table.to(DEV), cl.to(DEV),
                                 max_context_len=mcl, causal=causal, return_lse=True)
    torch.cuda.synchronize()
    ref = np.zeros((B, n_q, h_q, d))
    ref_lse = np.zeros((B, h_q, n_q))
    for b in range(B):
        o, l = oracle.sdpa(q[b:b + 1].double().numpy(), kl[b][None].double().numpy(),
                           vl[b][None].double().numpy(), 1.0 / np.sqrt(d), causal)
        ref[b], ref_lse[b] = o[0], l[0]
    what = "paged prefill ctx %s" % (ctx,)
    assert_close(out, ref, dt, what)
    assert_lse_close(lse, ref_lse, dt, what=what)
    return q, kl, vl, out, lse


def test_chunked_prefill_mixed_contexts():
    # 128 new tokens per sequence on top of cached contexts of various lengths
    _case([300, 1000, 129, 128], 128, 8, 2, 128, "bf16", True, seed=300)


def test_context_edges():
    _case([17, 63, 64, 65, 1023, 16], 16, 4, 4, 128, "bf16", True, seed=301)


def test_rows_without_keys():
    # 64 query rows on a 40-token context: the first 24 rows see no key
    q, kl, vl, out, lse = _case([40], 64, 2, 1, 128, "bf16", True, seed=302)
    assert (out[0, :24] == 0).all() and (lse[0, :, :24] == -np.inf).all()


def test_noncausal_head_dim_64_fp16():
    _case([90, 300], 50, 4, 2, 64, "f16", False, seed=303)


def test_equals_contiguous_prefill_bitwise():
    # a whole-sequence prefill: same tiles, same products, same bits
    q, kl, vl, out, lse = _case([512], 512, 8, 2, 128, "bf16", True, seed=304)
    o2, l2 = ea.attn_fwd(q.to(DEV), kl[0][None].to(DEV), vl[0][None].to(DEV), causal=True,
                         return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(lse, l2)


def test_block_table_rows_longer_than_the_staged_part():
    # contexts above 32,768 tokens: a workgroup stages the first 2,048 entries
    # of its sequence's table row in LDS and reads the rest from memory
    _case([40000, 33000, 2100], 200, 8, 2, 128, "bf16", True, seed=305)


def test_block_table_rows_longer_than_the_staged_part_noncausal_fp16():
    _case([36001], 130, 4, 4, 64, "f16", False, seed=306)


def test_validate_mode_on_valid_inputs(monkeypatch):
    monkeypatch.setenv("ATTN_VALIDATE", "1")
    _case([300, 129], 128, 8, 2, 128, "bf16", True, seed=307)

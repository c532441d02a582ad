"""GPU parity at the sizes where the kernels take their less common branches,
each compared element by element with the oracle (decode results from each
sequence's logical K/V, no block table on the oracle's side):

* decode batches of more than 64 sequences: the split kernel sums the list
  length and seeks its first block over several rounds of 64 sequences;
* (sequence, KV head) units cut into more than 64 partial results (contexts of
  64K and 128K tokens): the combine kernel folds partials lane + 64, lane +
  128, ... per lane and weighs them in later rounds of 64;
* shared prefixes cut into more than 64 chunks: more than 64 prefix partials
  per query;
* the same batches through sharing-aware decode.

The paged prefill whose block-table rows exceed the 2,048 entries staged in
LDS is in test_parity_prefill_paged.py.
"""

import numpy as np
import pytest
import torch

import exact_attention_34_amd as ea
import workloads
from helpers import assert_close, assert_lse_close, decode_reference

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TDT = {"f16": torch.float16, "bf16": torch.bfloat16}


def _plain(inp):
    out, lse = ea.paged_attn_decode(inp.q.to(DEV), inp.k_cache.to(DEV), inp.v_cache.to(DEV),
                                    inp.block_table.to(DEV), inp.context_lens.to(DEV),
                                    max_context_len=max(1, inp.max_context_len),
                                    scale=inp.scale, return_lse=True)
    torch.cuda.synchronize()
    return out, lse


def _shared(inp):
    sizes = np.diff(inp.group_starts.numpy())
    out, lse = ea.paged_attn_decode_shared(
        inp.q.to(DEV), inp.k_cache.to(DEV), inp.v_cache.to(DEV), inp.block_table.to(DEV),
        inp.context_lens.to(DEV), inp.group_starts.to(DEV), inp.prefix_lens.to(DEV),
        max_context_len=max(1, inp.max_context_len), max_group_size=max(1, int(sizes.max())),
        max_prefix_len=int(inp.prefix_lens.max()), scale=inp.scale, return_lse=True)
    torch.cuda.synchronize()
    return out, lse


def _check(inp, what, fn):
    print("case:", what, flush=True)
    out, lse = fn(inp)
    ref, ref_lse = decode_reference(inp)
    assert_close(out, ref, TDT[inp.dtype], what)
    assert_lse_close(lse, ref_lse, TDT[inp.dtype], what=what)
    return out, lse


# (sequences, lowest and highest context, seed)
MANY = [(200, 1, 3000, 400), (1000, 0, 300, 401), (130, 0, 5000, 402)]


@pytest.mark.parametrize("n,lo,hi,seed", MANY, ids=lambda x: str(x))
def test_decode_more_than_64_sequences(n, lo, hi, seed):
    rng = np.random.default_rng(seed)
    ctx = [int(c) for c in rng.integers(lo, hi, n, endpoint=True)]
    inp = workloads.decode_inputs(ctx, h_q=32, h_kv=8, d=128, block_size=16, dtype="bf16",
                                  seed=seed + 1)
    _check(inp, "%d sequences, contexts %d..%d" % (n, lo, hi), _plain)


def test_decode_more_than_64_sequences_fp16_d64_gqa8():
    rng = np.random.default_rng(403)
    ctx = [int(c) for c in rng.integers(0, 2000, 97, endpoint=True)]
    inp = workloads.decode_inputs(ctx, h_q=16, h_kv=2, d=64, block_size=16, dtype="f16",
                                  seed=404)
    _check(inp, "97 sequences, d=64 fp16, 8 query heads per KV head", _plain)


# contexts of 64K and 128K tokens at 32 query / 8 KV heads: with at most 2,048
# persistent waves of about 32 blocks each, every (sequence, KV head) of 4,096
# or 8,192 blocks is cut into 128 or 256 partial results
@pytest.mark.parametrize("ctx", [[65536, 65536], [131072], [131072 - 5, 17, 65536 + 9]],
                         ids=lambda c: "x".join(map(str, c)))
def test_decode_units_cut_into_more_than_64_partials(ctx):
    inp = workloads.decode_inputs(ctx, h_q=32, h_kv=8, d=128, block_size=16, dtype="bf16",
                                  seed=410 + len(ctx))
    _check(inp, "long contexts %s" % (ctx,), _plain)


def _groups(rng, n_groups, max_members, pre_hi, suf_hi):
    return [(int(rng.integers(0, pre_hi, endpoint=True)),
             [int(x) for x in rng.integers(0, suf_hi, int(rng.integers(1, max_members + 1)),
                                           endpoint=True)])
            for _ in range(n_groups)]


@pytest.mark.parametrize("seed,n_groups,members,pre_hi,suf_hi",
                         [(420, 25, 8, 1500, 500), (421, 250, 8, 300, 100)])
def test_shared_decode_more_than_64_sequences(seed, n_groups, members, pre_hi, suf_hi):
    rng = np.random.default_rng(seed)
    groups = _groups(rng, n_groups, members, pre_hi, suf_hi)
    inp = workloads.shared_prefix_inputs(groups, h_q=32, h_kv=8, d=128, block_size=16,
                                         dtype="bf16", seed=seed + 1)
    n = inp.q.shape[0]
    assert n > 64
    out, lse = _check(inp, "%d sequences in %d groups, shared" % (n, n_groups), _shared)
    plain, plain_lse = _plain(inp)
    d = (out.float() - plain.float()).abs().max().item()
    print("shared vs per-sequence decode max-abs %.3e" % d)
    assert d <= 2e-2


def test_shared_prefix_cut_into_more_than_64_chunks():
    # two groups with 64K- and 40K-token prefixes at 4 query heads per KV head:
    # the prefix work is cut into 128 chunks of 32 blocks, so every query
    # merges more than 64 prefix partials and its own suffix
    groups = [(65536, [16, 100, 0, 1000, 7, 300, 33, 2000]), (40000, [1, 5000, 64])]
    inp = workloads.shared_prefix_inputs(groups, h_q=8, h_kv=2, d=128, block_size=16,
                                         dtype="bf16", seed=430)
    _check(inp, "64K and 40K shared prefixes", _shared)

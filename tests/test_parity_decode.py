"""GPU parity of paged_attn_decode against the fp64 oracle, through the C ABI,
plus the layout invariants: a shuffled block table equals the identity
layout bit for bit, and a shared prefix equals private copies bit for bit."""

import numpy as np
import pytest
import torch

import exact_attention_34_amd as ea
import workloads
from helpers import assert_close, assert_lse_close, decode_reference

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TDT = {"f16": torch.float16, "bf16": torch.bfloat16}


def _run(inp, **kw):
    out, lse = ea.paged_attn_decode(inp.q.to(DEV), inp.k_cache.to(DEV), inp.v_cache.to(DEV),
                                    inp.block_table.to(DEV), inp.context_lens.to(DEV),
                                    max_context_len=max(1, inp.max_context_len),
                                    scale=inp.scale, return_lse=True, **kw)
    torch.cuda.synchronize()
    return out, lse


def _oracle(inp):
    return decode_reference(inp)


def _check(inp, what):
    print("case:", what, flush=True)
    out, lse = _run(inp)
    ref, ref_lse = _oracle(inp)
    assert_close(out, ref, TDT[inp.dtype], what)
    assert_lse_close(lse, ref_lse, TDT[inp.dtype], what=what)
    return out, lse


@pytest.fixture(scope="module")
def config4():
    return workloads.decode_config4()


def test_config4_full(config4):
    _check(config4, "64 seqs ctx U[512,8192] 32/8 heads shuffled table")


def test_config4_shapes_fp16():
    """The 64-sequence workload's context lengths and heads with fp16 K/V (the
    f16 matrix-core path of the split kernel at full size)."""
    c = workloads.DECODE_CONFIGS[4]
    ctx = np.random.default_rng(4).integers(c["ctx_lo"], c["ctx_hi"], size=c["num_seqs"],
                                            endpoint=True)
    inp = workloads.decode_inputs(ctx, c["h_q"], c["h_kv"], c["d"], c["block_size"], "f16", 44,
                                  max_blocks_per_seq=c["ctx_hi"] // c["block_size"])
    _check(inp, "64 seqs ctx U[512,8192] 32/8 heads shuffled table, fp16")


def test_config4_identity_layout_bitwise(config4):
    # the same logical sequences laid out contiguously (identity block order)
    out1, lse1 = _run(config4)
    kc, vc, tab, ctx = workloads.build_paged(config4.k_logical, config4.v_logical, 16,
                                             shuffle=False, max_blocks_per_seq=512)
    ident = workloads.DecodeInputs(config4.q, kc, vc, tab, ctx, 16, config4.scale, "bf16")
    out2, lse2 = _run(ident)
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


def test_config5_shared_prefix_full_and_bitwise_private():
    shared = workloads.decode_config5()
    out1, lse1 = _check(shared, "8x8 shared 4096 prefix + 256 suffix")
    private = workloads.decode_config5(private=True)
    assert private.k_cache.shape[0] > shared.k_cache.shape[0]
    out2, lse2 = _run(private)
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


EDGE_CTX = [1, 2, 15, 16, 17, 31, 33, 255, 511, 512, 513, 1023, 1024, 1025, 1536, 2049]


@pytest.mark.parametrize("group", [1, 2, 4, 8, 16])
def test_context_edges_and_groups(group):
    h_kv = 2
    inp = workloads.decode_inputs(EDGE_CTX, h_q=h_kv * group, h_kv=h_kv, d=128, block_size=16,
                                  dtype="bf16", seed=40 + group, spare_blocks=5)
    _check(inp, "edge contexts, group %d" % group)


def test_head_dim_64_fp16():
    inp = workloads.decode_inputs([1, 100, 700, 1500], h_q=8, h_kv=2, d=64, block_size=16,
                                  dtype="f16", seed=50)
    _check(inp, "d=64 fp16")


def test_zero_context_gives_zero_and_neg_inf():
    inp = workloads.decode_inputs([0, 40, 0, 600], h_q=8, h_kv=2, d=128, block_size=16,
                                  dtype="bf16", seed=51)
    out, lse = _check(inp, "zero contexts")
    assert (out[0] == 0).all() and (out[2] == 0).all()
    assert (lse[0] == -np.inf).all() and (lse[2] == -np.inf).all()


def test_max_context_bound_above_actual():
    # max_context_len larger than every context: extra partitions are idle
    inp = workloads.decode_inputs([100, 900], h_q=4, h_kv=1, d=128, block_size=16,
                                  dtype="bf16", seed=52, max_blocks_per_seq=256)
    print("case: max_context_len 4096 over contexts 100, 900", flush=True)
    out, lse = ea.paged_attn_decode(inp.q.to(DEV), inp.k_cache.to(DEV), inp.v_cache.to(DEV),
                                    inp.block_table.to(DEV), inp.context_lens.to(DEV),
                                    max_context_len=4096, scale=inp.scale, return_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = _oracle(inp)
    assert_close(out, ref, torch.bfloat16, "max_context_len bound")
    assert_lse_close(lse, ref_lse, torch.bfloat16)


def test_decode_equals_last_row_of_causal_prefill():
    ctx = [1, 77, 512, 1300]
    inp = workloads.decode_inputs(ctx, h_q=8, h_kv=2, d=128, block_size=16, dtype="bf16",
                                  seed=53)
    out, _ = _run(inp)
    for s, n in enumerate(ctx):
        rng = np.random.default_rng(s)
        qq = torch.from_numpy(rng.standard_normal((1, n, 8, 128))).to(torch.bfloat16)
        qq[0, -1] = inp.q[s]
        o = ea.attn_fwd(qq.to(DEV), inp.k_logical[s][None].to(DEV),
                        inp.v_logical[s][None].to(DEV), causal=True, scale=inp.scale)
        torch.cuda.synchronize()
        d = (o[0, -1].float() - out[s].float()).abs().max().item()
        print("seq", s, "ctx", n, "decode vs prefill last row max-abs", d)
        assert d <= 2e-2


def test_deterministic(config4):
    out1, lse1 = _run(config4)
    out2, lse2 = _run(config4)
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


def _long_case(h_q, h_kv, ctx_lo, ctx_hi, seed):
    # long contexts: every (sequence, KV head) is cut across several waves
    rng = np.random.default_rng(seed)
    ctx = [int(c) for c in rng.integers(ctx_lo, ctx_hi, 8, endpoint=True)]
    return workloads.decode_inputs(ctx, h_q=h_q, h_kv=h_kv, d=128, block_size=16,
                                   dtype="bf16", seed=seed)


def test_workspace_reused_with_garbage_contents():
    # the workspace contents on entry do not matter: a caller-provided buffer
    # filled with NaN bytes, reused for two calls, gives identical results
    inp = _long_case(32, 8, 2048, 2300, 60)
    mcl = int(inp.context_lens.max())
    need = ea.paged_attn_decode_workspace_size(8, 32, 8, 128, mcl)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    out1, lse1 = _run(inp, workspace=ws)
    out2, lse2 = _run(inp, workspace=ws)
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)
    ref, ref_lse = _oracle(inp)
    assert_close(out1, ref, torch.bfloat16, "long contexts, reused workspace")
    assert_lse_close(lse1, ref_lse, torch.bfloat16)


@pytest.mark.parametrize("group,h_kv,lo,hi", [(8, 4, 2560, 2800), (16, 2, 4800, 5200)])
def test_long_contexts_large_groups(group, h_kv, lo, hi):
    # groups of 8 and 16 query heads at d = 128 run one wave per SIMD
    inp = _long_case(group * h_kv, h_kv, lo, hi, 61 + group)
    _check(inp, "long contexts, group %d" % group)


def _random_cases(n, seed):
    """Seeded random decode batches: 1..40 sequences with contexts from 0 to
    3000 tokens (block edges included by chance), GQA ratios 1..16, both head
    dims and dtypes; NaN in every slot past a context."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        s = int(rng.integers(1, 41))
        ctx = [int(c) for c in rng.integers(0, 3001, s)]
        h_kv = int(rng.choice([1, 2, 4, 8]))
        group = int(rng.choice([1, 2, 4, 8, 16]))
        out.append((ctx, h_kv * group, h_kv, int(rng.choice([64, 128])),
                    str(rng.choice(["bf16", "f16"])), 3000 + i))
    return out


@pytest.mark.parametrize("case", _random_cases(12, 66), ids=lambda c: "seed%d" % c[5])
def test_random_batches(case):
    ctx, h_q, h_kv, d, dt, seed = case
    inp = workloads.decode_inputs(ctx, h_q=h_q, h_kv=h_kv, d=d, block_size=16, dtype=dt,
                                  seed=seed)
    _check(inp, "random %d seqs ctx<=%d %d/%d heads d=%d %s" % (len(ctx), max(ctx), h_q, h_kv,
                                                               d, dt))


def test_validate_mode_on_valid_inputs(config4, monkeypatch):
    # ATTN_VALIDATE=1: the call range-checks host copies of the table and the
    # context lengths first; valid inputs then give the same bits
    out1, lse1 = _run(config4)
    monkeypatch.setenv("ATTN_VALIDATE", "1")
    out2, lse2 = _run(config4)
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)

"""GPU parity of paged_attn_decode_shared (sharing-aware decode) against the
fp64 oracle, through the C ABI.  The oracle never sees the groups: it
attends each sequence to its own logical context, so these tests also check
that reading a prefix once per group changes nothing but the speed.  Layout
invariants: results do not depend on the physical block order, and without
sharing the call equals paged_attn_decode bit for bit."""

import numpy as np
import pytest
import torch

import exact_attention_34_amd as ea
import workloads
from helpers import assert_close, assert_lse_close, decode_reference

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TDT = {"f16": torch.float16, "bf16": torch.bfloat16}


def _bounds(inp):
    gs = inp.group_starts.numpy()
    sizes = np.diff(gs)
    return (max(1, inp.max_context_len), max(1, int(sizes.max()) if len(sizes) else 1),
            int(inp.prefix_lens.max()) if len(inp.prefix_lens) else 0)


def _run_shared(inp, workspace=None, bounds=None):
    mcl, mgs, mpl = bounds if bounds is not None else _bounds(inp)
    out, lse = ea.paged_attn_decode_shared(
        inp.q.to(DEV), inp.k_cache.to(DEV), inp.v_cache.to(DEV), inp.block_table.to(DEV),
        inp.context_lens.to(DEV), inp.group_starts.to(DEV), inp.prefix_lens.to(DEV),
        max_context_len=mcl, max_group_size=mgs, max_prefix_len=mpl, scale=inp.scale,
        workspace=workspace, return_lse=True)
    torch.cuda.synchronize()
    return out, lse


def _run_plain(inp):
    out, lse = ea.paged_attn_decode(inp.q.to(DEV), inp.k_cache.to(DEV), inp.v_cache.to(DEV),
                                    inp.block_table.to(DEV), inp.context_lens.to(DEV),
                                    max_context_len=max(1, inp.max_context_len),
                                    scale=inp.scale, return_lse=True)
    torch.cuda.synchronize()
    return out, lse


def _oracle(inp):
    return decode_reference(inp)


def _check(inp, what, **kw):
    print("case:", what, flush=True)
    out, lse = _run_shared(inp, **kw)
    ref, ref_lse = _oracle(inp)
    assert_close(out, ref, TDT[inp.dtype], what)
    assert_lse_close(lse, ref_lse, TDT[inp.dtype], what=what)
    return out, lse


@pytest.fixture(scope="module")
def config5():
    return workloads.decode_config5()


def test_config5_full(config5):
    # 8 groups x 8 sequences, 4096-token prefix per group, 256-token suffixes
    out, lse = _check(config5, "8x8 shared 4096 prefix + 256 suffix, prefix read once")
    plain, plain_lse = _run_plain(config5)
    d = (out.float() - plain.float()).abs().max().item()
    print("shared vs per-sequence decode max-abs %.3e" % d)
    assert d <= 2e-2


def test_config5_layout_independent_bitwise(config5):
    out1, lse1 = _run_shared(config5)
    c = workloads.DECODE_CONFIGS[5]
    groups = [(c["prefix"], [c["suffix"]] * c["per_group"])] * c["groups"]
    ident = workloads.shared_prefix_inputs(groups, c["h_q"], c["h_kv"], c["d"],
                                           c["block_size"], c["dtype"], 5, shuffle=False)
    assert torch.equal(ident.q, config5.q)
    assert not torch.equal(ident.block_table, config5.block_table)
    out2, lse2 = _run_shared(ident)
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


def test_deterministic_and_garbage_workspace(config5):
    mcl, mgs, mpl = _bounds(config5)
    need = ea.paged_attn_decode_shared_workspace_size(64, 8, mgs, 32, 8, 128, mcl, mpl)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    out1, lse1 = _run_shared(config5, workspace=ws)
    out2, lse2 = _run_shared(config5, workspace=ws)
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)
    out3, lse3 = _run_shared(config5)
    assert torch.equal(out1, out3) and torch.equal(lse1, lse3)


# (prefix tokens, [suffix tokens of each member]): no prefix; a one-block
# prefix with a member whose context is exactly the prefix; a prefix ending
# inside a block; more members than one 32-query tile holds (at 4 heads per
# KV head); an empty group; a group of one whose context is all prefix; long
# prefixes with short and long suffixes
EDGE_GROUPS = [
    (0, [5, 300]),
    (16, [0, 1, 17]),
    (100, [3, 250]),
    (1024, [64] * 9),
    (2048, []),
    (512, [0]),
    (4096, [1, 33, 700]),
]


@pytest.mark.parametrize("group", [1, 4, 8, 16])
def test_edge_groups(group):
    h_kv = 2
    inp = workloads.shared_prefix_inputs(EDGE_GROUPS, h_q=h_kv * group, h_kv=h_kv, d=128,
                                         block_size=16, dtype="bf16", seed=70 + group,
                                         spare_blocks=3)
    _check(inp, "edge groups, %d query heads per KV head" % group)


def test_head_dim_64_fp16():
    groups = [(256, [10, 40, 0]), (48, [200]), (1040, [16, 17])]
    inp = workloads.shared_prefix_inputs(groups, h_q=8, h_kv=2, d=64, block_size=16,
                                         dtype="f16", seed=80)
    _check(inp, "d=64 fp16 shared")


def test_understated_bounds_still_exact():
    # host bounds below the actual group size / prefix length: the members and
    # prefix blocks the prefix kernel does not cover fall back to the
    # per-sequence path, so the result is still exact
    groups = [(2048, [40] * 12), (1600, [7, 90])]
    inp = workloads.shared_prefix_inputs(groups, h_q=16, h_kv=4, d=128, block_size=16,
                                         dtype="bf16", seed=81)
    mcl, mgs, mpl = _bounds(inp)
    _check(inp, "understated max_group_size and max_prefix_len", bounds=(mcl, 5, 512))


def test_no_sharing_equals_plain_decode_bitwise():
    # every sequence its own group with no prefix: the same kernels, the same
    # partition, the same bits as paged_attn_decode
    rng = np.random.default_rng(82)
    ctx = [int(c) for c in rng.integers(1, 3000, 12)]
    groups = [(0, [c]) for c in ctx]
    inp = workloads.shared_prefix_inputs(groups, h_q=32, h_kv=8, d=128, block_size=16,
                                         dtype="bf16", seed=82)
    out1, lse1 = _run_shared(inp)
    out2, lse2 = _run_plain(inp)
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)
    ref, ref_lse = _oracle(inp)
    assert_close(out1, ref, torch.bfloat16, "no sharing")


def test_prefix_in_extreme_logit_range():
    # x20 prefix keys: the reference max moves inside the prefix chunks and
    # the merge of chunk partials must carry large max differences exactly
    groups = [(1024, [30, 30, 30, 30])]
    inp = workloads.shared_prefix_inputs(groups, h_q=32, h_kv=8, d=128, block_size=16,
                                         dtype="bf16", seed=83)
    kl = [k.clone() for k in inp.k_logical]
    rows = np.random.default_rng(84).choice(1024, 10, replace=False)
    for k in kl:
        k[rows] = (k[rows].double() * 20).to(torch.bfloat16)
    kc, vc, tab, ctx = workloads.build_paged(
        kl, inp.v_logical, 16, rng=np.random.default_rng(85),
        shared_blocks={(s, lb): ("p", lb) for s in range(4) for lb in range(64)})
    stressed = workloads.DecodeInputs(inp.q, kc, vc, tab, ctx, 16, inp.scale, "bf16", kl,
                                      inp.v_logical, inp.group_starts, inp.prefix_lens)
    _check(stressed, "x20 prefix keys")


def test_validate_mode_on_valid_inputs(config5, monkeypatch):
    # ATTN_VALIDATE=1 also checks the groups and that members share the
    # prefix's block ids; valid inputs give the same bits
    out1, lse1 = _run_shared(config5)
    monkeypatch.setenv("ATTN_VALIDATE", "1")
    out2, lse2 = _run_shared(config5)
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)

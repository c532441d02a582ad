"""GPU tests of the paged KV cache kernels (bit-exact against the oracle's
definition) and of the whole system path: the block manager's slots and
copy-on-write copies, applied with paged_kv_write / paged_kv_copy_blocks,
give block tables under which both decode entry points match the fp64
oracle on each sequence's logical context."""

import numpy as np
import pytest
import torch

import exact_attention_34_amd as ea
import oracle
import workloads
from helpers import assert_close, assert_lse_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BS = 16


def _same(got, want):
    """Equal element for element: NaN in the same places (the untouched NaN
    canaries; their bit pattern may differ after the reference's fp32 round
    trip), identical values everywhere else."""
    got = got.cpu()
    nan = torch.isnan(want)
    return torch.equal(torch.isnan(got), nan) and torch.equal(got[~nan], want[~nan])


def test_kv_write_matches_oracle_bitwise():
    rng = np.random.default_rng(100)
    nb, hkv, d, n = 12, 4, 128, 70
    kc = torch.full((nb, hkv, BS, d), float("nan"), dtype=torch.bfloat16)
    vc = kc.clone()
    # new K/V as views with a padded head axis (token stride 5 d, head stride d)
    wide_k = workloads._round(rng.standard_normal((n, hkv + 1, d)), "bf16")
    wide_v = workloads._round(rng.standard_normal((n, hkv + 1, d)), "bf16")
    kn, vn = wide_k[:, 1:], wide_v[:, 1:]
    slots = rng.permutation(nb * BS)[:n].astype(np.int32)
    slots[[3, 17]] = [-1, nb * BS + 5]              # padding / out of the pool: skipped
    ref_k, ref_v = oracle.paged_kv_write(kc.float().numpy(), vc.float().numpy(),
                                         kn.float().numpy(), vn.float().numpy(), slots, BS)
    gk, gv = kc.to(DEV), vc.to(DEV)
    ea.paged_kv_write(wide_k.to(DEV)[:, 1:], wide_v.to(DEV)[:, 1:],
                      torch.from_numpy(slots).to(DEV), gk, gv)
    torch.cuda.synchronize()
    want_k = torch.from_numpy(ref_k).to(torch.bfloat16)
    want_v = torch.from_numpy(ref_v).to(torch.bfloat16)
    assert _same(gk, want_k) and _same(gv, want_v)


def test_copy_blocks_matches_oracle_bitwise():
    rng = np.random.default_rng(101)
    nb, hkv, d = 10, 2, 64
    kc = workloads._round(rng.standard_normal((nb, hkv, BS, d)), "f16")
    vc = workloads._round(rng.standard_normal((nb, hkv, BS, d)), "f16")
    src = np.array([1, 4, 7, -1], dtype=np.int32)
    dst = np.array([6, 0, 9, 3], dtype=np.int32)
    ref_k, ref_v = oracle.paged_kv_copy_blocks(kc.float().numpy(), vc.float().numpy(), src, dst)
    gk, gv = kc.to(DEV), vc.to(DEV)
    ea.paged_kv_copy_blocks(gk, gv, torch.from_numpy(src).to(DEV), torch.from_numpy(dst).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(gk.cpu(), torch.from_numpy(ref_k).to(torch.float16))
    assert torch.equal(gv.cpu(), torch.from_numpy(ref_v).to(torch.float16))


@pytest.mark.parametrize("prompt,steps,samples", [(100, 20, 4), (64, 33, 3)])
def test_parallel_sampling_end_to_end(prompt, steps, samples):
    # a prompt written once, forked into `samples` sequences that each decode
    # `steps` tokens: shared prompt blocks, copy-on-write of the partial one
    rng = np.random.default_rng(200 + prompt)
    hq, hkv, d, nb = 8, 2, 128, 64
    dt = torch.bfloat16
    kc = torch.full((nb, hkv, BS, d), float("nan"), dtype=dt, device=DEV)
    vc = torch.full((nb, hkv, BS, d), float("nan"), dtype=dt, device=DEV)
    m = ea.BlockManager(nb, BS)
    logical_k, logical_v = {}, {}

    def write(seq, k_rows, v_rows):
        slots, copies = m.append(seq, k_rows.shape[0])
        if copies:
            src = torch.tensor([c[0] for c in copies], dtype=torch.int32, device=DEV)
            dst = torch.tensor([c[1] for c in copies], dtype=torch.int32, device=DEV)
            ea.paged_kv_copy_blocks(kc, vc, src, dst)
        ea.paged_kv_write(k_rows.to(DEV), v_rows.to(DEV), torch.from_numpy(slots).to(DEV), kc, vc)
        return copies

    pk = workloads._round(rng.standard_normal((prompt, hkv, d)), "bf16")
    pv = workloads._round(rng.standard_normal((prompt, hkv, d)), "bf16")
    m.add_sequence(0)
    write(0, pk, pv)
    children = list(range(1, samples + 1))
    for c in children:
        m.fork(0, c)
        logical_k[c], logical_v[c] = [pk], [pv]
    m.free_sequence(0)
    n_copies = 0
    for _ in range(steps):
        for c in children:
            tk = workloads._round(rng.standard_normal((1, hkv, d)), "bf16")
            tv = workloads._round(rng.standard_normal((1, hkv, d)), "bf16")
            n_copies += len(write(c, tk, tv))
            logical_k[c].append(tk)
            logical_v[c].append(tv)
    # a partial prompt block is copied once per sample but the last
    assert n_copies == (samples - 1 if prompt % BS else 0)
    max_blocks = (prompt + steps + BS - 1) // BS
    table, ctx = m.block_table(children, max_blocks)
    whole = prompt // BS
    assert (table[:, :whole] == table[0, :whole]).all()          # prompt blocks shared
    assert len(set(table[:, whole].tolist())) == samples          # the rest are private

    q = workloads._round(rng.standard_normal((samples, hq, d)), "bf16")
    tab, cl = torch.from_numpy(table).to(DEV), torch.from_numpy(ctx).to(DEV)
    print("case: prompt %d, %d samples x %d steps" % (prompt, samples, steps), flush=True)
    out, lse = ea.paged_attn_decode(q.to(DEV), kc, vc, tab, cl, max_context_len=int(ctx.max()),
                                    return_lse=True)
    gs = torch.tensor([0, samples], dtype=torch.int32, device=DEV)
    pl = torch.tensor([prompt], dtype=torch.int32, device=DEV)
    out2, lse2 = ea.paged_attn_decode_shared(q.to(DEV), kc, vc, tab, cl, gs, pl,
                                             max_context_len=int(ctx.max()),
                                             max_group_size=samples, max_prefix_len=prompt,
                                             return_lse=True)
    torch.cuda.synchronize()
    ref = np.zeros((samples, hq, d))
    ref_lse = np.zeros((samples, hq))
    for i, c in enumerate(children):
        kl = torch.cat(logical_k[c]).double().numpy()[None]
        vl = torch.cat(logical_v[c]).double().numpy()[None]
        o, l = oracle.sdpa(q[i].double().numpy()[None, None], kl, vl, 1.0 / np.sqrt(d))
        ref[i], ref_lse[i] = o[0, 0], l[0, :, 0]
    assert_close(out, ref, dt, "decode over manager-built tables")
    assert_lse_close(lse, ref_lse, dt, "decode over manager-built tables")
    assert_close(out2, ref, dt, "shared decode over manager-built tables")
    assert_lse_close(lse2, ref_lse, dt, "shared decode over manager-built tables")

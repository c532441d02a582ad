"""The C ABI without a GPU: the library loads, exports every function that
include/attn.h declares, and rejects invalid arguments on the host before any
device work (these calls never reach a launch)."""

import ctypes
import os
import re

import pytest

import exact_attention_34_amd as ea

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?([a-z_0-9]+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("attn_fwd", "paged_attn_decode", "paged_attn_decode_workspace_size",
              "paged_attn_decode_shared", "paged_attn_decode_shared_workspace_size",
              "attn_bwd", "attn_bwd_workspace_size",
              "attn_last_error", "attn_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = ea.lib()
    for n in declared_functions():
        assert hasattr(L, n), n


def test_abi_version():
    assert ea.abi_version() == 7


def test_workspace_size():
    # two partial slots per persistent wave, one per query head of a KV head's
    # group, each (head_dim + 2) floats; at most 2048 waves, at most one wave
    # per block of the largest possible block list
    assert ea.paged_attn_decode_workspace_size(0, 32, 8, 128, 8192) == 0
    assert ea.paged_attn_decode_workspace_size(64, 32, 0, 128, 8192) == 0
    # plus (first wave, wave count) per (sequence, KV head)
    assert ea.paged_attn_decode_workspace_size(64, 32, 8, 128, 8192) == \
        2048 * 2 * 4 * 130 * 4 + 64 * 8 * 8
    # 2 seqs x 1 kv head x ceil(513/16) = 33 blocks -> 66 waves
    assert ea.paged_attn_decode_workspace_size(2, 4, 1, 64, 513) == 66 * 2 * 4 * 66 * 4 + 2 * 8


FAKE = 1 << 20          # a 16-byte aligned, never dereferenced address
I64x3 = ctypes.c_int64 * 3


def _fwd(dtype=2, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, batch=1, n_q=128, n_k=128, h_q=4,
         h_kv=2, d=128, qs=(128 * 4 * 128, 4 * 128, 128), ks=(128 * 2 * 128, 2 * 128, 128),
         scale=0.088, causal=0, strides=True):
    L = ea.lib()
    st = [I64x3(*qs), I64x3(*ks), I64x3(*ks), I64x3(*qs)] if strides else [None] * 4
    code = L.attn_fwd(dtype, q, k, v, o, lse, batch, n_q, n_k, h_q, h_kv, d, *st, scale, causal,
                      None)
    return code, L.attn_last_error().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), 3),
    (dict(d=96), 3),
    (dict(h_q=3, h_kv=2), 2),
    (dict(h_kv=0), 2),
    (dict(n_q=-1), 2),
    (dict(scale=float("nan")), 2),
    (dict(scale=0.0), 2),
    (dict(causal=2), 2),
    (dict(q=None), 1),
    (dict(k=None), 1),
    (dict(strides=False), 1),
    (dict(q=FAKE + 8), 5),
    (dict(qs=(128 * 4 * 128, 4 * 128, 4)), 5),    # head stride of 8 bytes
    (dict(lse=FAKE + 2), 5),
])
def test_attn_fwd_rejects(kw, code):
    got, msg = _fwd(**kw)
    assert got == code, msg
    assert msg.startswith("attn_fwd")


def test_attn_fwd_empty_problem_is_noop():
    # nothing to compute: returns OK without touching any pointer
    assert _fwd(batch=0, q=None, o=None)[0] == 0
    assert _fwd(n_q=0, q=None, o=None)[0] == 0


def _dec(dtype=2, q=FAKE, k=FAKE, v=FAKE, table=FAKE, ctx=FAKE, o=FAKE, lse=None, S=4, h_q=32,
         h_kv=8, d=128, bs=16, mbps=512, mcl=8192, nb=100, scale=0.088, ws=FAKE, ws_bytes=None):
    L = ea.lib()
    if ws_bytes is None:
        ws_bytes = L.paged_attn_decode_workspace_size(S, h_q, h_kv, d, mcl)
    code = L.paged_attn_decode(dtype, q, k, v, table, ctx, o, lse, S, h_q, h_kv, d, bs, mbps, mcl,
                               nb, scale, ws, ws_bytes, None)
    return code, L.attn_last_error().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=0), 3),
    (dict(d=80), 3),
    (dict(bs=32), 3),
    (dict(h_q=64, h_kv=2), 3),       # group of 32
    (dict(h_q=30), 2),
    (dict(mbps=100), 2),             # 100 * 16 < 8192
    (dict(nb=0), 2),
    (dict(scale=-1.0), 2),
    (dict(q=None), 1),
    (dict(table=None), 1),
    (dict(ctx=None), 1),
    (dict(ws=None), 4),
    (dict(ws_bytes=100), 4),
    (dict(k=FAKE + 4), 5),
    (dict(ws=FAKE + 8), 5),
    (dict(table=FAKE + 2), 5),
])
def test_paged_decode_rejects(kw, code):
    got, msg = _dec(**kw)
    assert got == code, msg
    assert msg.startswith("paged_attn_decode")


def test_paged_decode_no_sequences_is_noop():
    assert _dec(S=0, q=None, o=None, ctx=None)[0] == 0


def _dsh(dtype=2, q=FAKE, k=FAKE, v=FAKE, table=FAKE, ctx=FAKE, gst=FAKE, plen=FAKE, o=FAKE,
         lse=None, S=64, G=8, mgs=8, h_q=32, h_kv=8, d=128, bs=16, mbps=512, mcl=8192, mpl=4096,
         nb=100, scale=0.088, ws=FAKE, ws_bytes=None):
    L = ea.lib()
    if ws_bytes is None:
        ws_bytes = L.paged_attn_decode_shared_workspace_size(S, G, mgs, h_q, h_kv, d, mcl, mpl)
    code = L.paged_attn_decode_shared(dtype, q, k, v, table, ctx, gst, plen, o, lse, S, G, mgs,
                                      h_q, h_kv, d, bs, mbps, mcl, mpl, nb, scale, ws, ws_bytes,
                                      None)
    return code, L.attn_last_error().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=0), 3),
    (dict(h_q=64, h_kv=2), 3),
    (dict(bs=8), 3),
    (dict(G=0), 2),
    (dict(mgs=0), 2),
    (dict(G=-1), 2),
    (dict(mpl=-16), 2),
    (dict(mpl=8193), 2),             # prefix bound above the context bound
    (dict(gst=None), 1),
    (dict(plen=None), 1),
    (dict(ctx=None), 1),
    (dict(ws=None), 4),
    (dict(ws_bytes=1000), 4),
    (dict(gst=FAKE + 2), 5),
    (dict(ws=FAKE + 4), 5),
])
def test_paged_decode_shared_rejects(kw, code):
    got, msg = _dsh(**kw)
    assert got == code, msg
    assert msg.startswith("paged_attn_decode_shared")


def test_paged_decode_shared_no_sequences_is_noop():
    assert _dsh(S=0, G=0, mgs=0, q=None, o=None, ctx=None, gst=None, plen=None)[0] == 0


def test_shared_workspace_size():
    L = ea.lib()
    assert L.paged_attn_decode_shared_workspace_size(0, 8, 8, 32, 8, 128, 8192, 4096) == 0
    assert L.paged_attn_decode_shared_workspace_size(64, 0, 8, 32, 8, 128, 8192, 4096) == 0
    # 8 groups x 8 members x 4 heads = one 32-query tile per (group, KV head);
    # 16,384 prefix blocks in all -> 32 blocks per chunk, 8 chunks: 512 items
    split = L.paged_attn_decode_workspace_size(64, 32, 8, 128, 4352)
    suf = 64 * 32 * 130 * 4
    pre = 512 * 32 * 130 * 4
    meta = 3 * 64 * 4
    assert L.paged_attn_decode_shared_workspace_size(64, 8, 8, 32, 8, 128, 4352, 4096) == \
        split + suf + pre + meta


def _bwd(dtype=2, q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
         batch=1, n_q=128, n_k=128, h_q=4, h_kv=2, d=128, qs=(128 * 4 * 128, 4 * 128, 128),
         ks=(128 * 2 * 128, 2 * 128, 128), scale=0.088, causal=1, ws=FAKE, ws_bytes=None):
    L = ea.lib()
    if ws_bytes is None:
        ws_bytes = L.attn_bwd_workspace_size(batch, n_q, h_q)
    st = [I64x3(*qs), I64x3(*ks), I64x3(*ks), I64x3(*qs), I64x3(*qs), I64x3(*qs), I64x3(*ks),
          I64x3(*ks)]
    code = L.attn_bwd(dtype, q, k, v, o, do, lse, dq, dk, dv, batch, n_q, n_k, h_q, h_kv, d, *st,
                      scale, causal, ws, ws_bytes, None)
    return code, L.attn_last_error().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=0), 3),              # fp32 backward is not built
    (dict(d=96), 3),
    (dict(h_q=3), 2),
    (dict(n_k=-1), 2),
    (dict(causal=3), 2),
    (dict(scale=float("inf")), 2),
    (dict(lse=None), 1),
    (dict(dk=None), 1),
    (dict(do=None), 1),
    (dict(ws=None), 4),
    (dict(ws_bytes=16), 4),
    (dict(dq=FAKE + 8), 5),
    (dict(lse=FAKE + 2), 5),
    (dict(qs=(128 * 4 * 128, 4 * 128, 4)), 5),
])
def test_attn_bwd_rejects(kw, code):
    got, msg = _bwd(**kw)
    assert got == code, msg
    assert msg.startswith("attn_bwd")


def test_attn_bwd_empty_is_noop():
    assert _bwd(batch=0, q=None, k=None)[0] == 0
    assert _bwd(n_q=0, n_k=0, q=None, k=None)[0] == 0


def test_attn_bwd_workspace_size():
    L = ea.lib()
    assert L.attn_bwd_workspace_size(0, 128, 4) == 0
    # two fp32 per query row (delta, log-sum-exp in log2 units), each array
    # rounded up to 16 bytes
    assert L.attn_bwd_workspace_size(2, 100, 3) == 2 * (2 * 100 * 3 * 4)   # 2400 = 16 * 150
    assert L.attn_bwd_workspace_size(1, 5, 1) == 2 * 32                     # 20 rounded up to 32


def test_last_error_cleared_on_success():
    _fwd(dtype=7)
    assert ea.lib().attn_last_error().decode() != ""
    assert _fwd(batch=0)[0] == 0
    assert ea.lib().attn_last_error().decode() == ""


# ----------------------------------------------------------------------------
# attn_validate_paged_tables: the check behind the ATTN_VALIDATE mode, on host
# arrays (no GPU involved)
# ----------------------------------------------------------------------------

def _tables():
    import numpy as np
    # 3 sequences of 40, 16 and 0 tokens in 16-token blocks; the first two
    # form a group sharing a 16-token prefix (block 7), the third its own group
    tab = np.full((3, 4), -1, dtype=np.int32)
    tab[0, :3] = [7, 2, 5]
    tab[1, :1] = [7]
    ctx = np.array([40, 16, 0], dtype=np.int32)
    gs = np.array([0, 2, 3], dtype=np.int32)
    pl = np.array([16, 0], dtype=np.int32)
    return tab, ctx, gs, pl


def test_validate_accepts_valid_tables():
    tab, ctx, gs, pl = _tables()
    ea.validate_paged_tables(tab, ctx, max_context_len=64, num_blocks=8)
    ea.validate_paged_tables(tab, ctx, 64, 8, group_starts=gs, prefix_lens=pl)
    # an empty batch, and entries past a context are never read (-1 there)
    ea.validate_paged_tables(tab[:0], ctx[:0], 64, 8)


def _rejects(match, **kw):
    tab, ctx, gs, pl = _tables()
    args = dict(block_table=tab, context_lens=ctx, max_context_len=64, num_blocks=8,
                group_starts=gs, prefix_lens=pl)
    mutate = kw.pop("mutate")
    mutate(args)
    args.update(kw)
    with pytest.raises(ea.AttnError) as ei:
        ea.validate_paged_tables(**args)
    assert ei.value.code == 2 and re.search(match, str(ei.value)), str(ei.value)


def test_validate_rejects_block_id_out_of_range():
    _rejects(r"block_table\[0\]\[2\] = 8 outside", mutate=lambda a: a["block_table"].__setitem__((0, 2), 8))
    _rejects(r"block_table\[0\]\[1\] = -1 outside", mutate=lambda a: a["block_table"].__setitem__((0, 1), -1))


def test_validate_rejects_context_lengths():
    _rejects(r"context_lens\[2\] = -3", mutate=lambda a: a["context_lens"].__setitem__(2, -3))
    _rejects(r"context_lens\[0\] = 40 outside", mutate=lambda a: None, max_context_len=39)
    # 65 tokens need 5 entries of a 4-entry row
    _rejects(r"needs 5 table entries", mutate=lambda a: a["context_lens"].__setitem__(0, 65),
             max_context_len=100)


def test_validate_rejects_bad_groups():
    _rejects(r"group_starts\[0\] must be 0", mutate=lambda a: a["group_starts"].__setitem__(0, 1))
    _rejects(r"must equal num_seqs", mutate=lambda a: a["group_starts"].__setitem__(2, 2))
    _rejects(r"non-decreasing", mutate=lambda a: a["group_starts"].__setitem__(1, 4))
    _rejects(r"prefix_lens\[1\] = -1", mutate=lambda a: a["prefix_lens"].__setitem__(1, -1))
    # a 17-token prefix is longer than member 1's 16-token context
    _rejects(r"exceeds context_lens\[1\]", mutate=lambda a: a["prefix_lens"].__setitem__(0, 17))


def test_validate_rejects_prefix_blocks_that_are_not_shared():
    def mutate(a):
        a["block_table"][1, 0] = 3
    _rejects(r"block_table\[1\]\[0\] = 3 differs", mutate=mutate)


def test_last_error_is_per_thread():
    """The error message store is per thread: threads that fail concurrently
    (the validator runs on the host; ctypes releases the interpreter lock
    during the call) each read their own message."""
    import threading
    failures = []

    def worker(t):
        tab, ctx, gs, pl = _tables()
        for i in range(300):
            bad = -(1000 * (t + 1) + i)
            ctx[2] = bad
            try:
                ea.validate_paged_tables(tab, ctx, max_context_len=64, num_blocks=8)
                failures.append((t, i, "accepted"))
            except ea.AttnError as e:
                if "context_lens[2] = %d" % bad not in str(e):
                    failures.append((t, i, str(e)))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(8)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not failures, failures[:5]


def test_noalloc_decode_rejects_sizes_beyond_its_scratch():
    # 16 query heads per KV head over 65,535 sequences x 64 KV heads need
    # more workspace than the library's scratch holds: rejected on the host,
    # before any device call
    need = ea.paged_attn_decode_workspace_size(65535, 1024, 64, 128, 1 << 20)
    assert need > ea.DECODE_SCRATCH_BYTES
    code = ea.lib().paged_attn_decode_noalloc(2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                              65535, 1024, 64, 128, 16, 1 << 16, 1 << 20, 1,
                                              0.1, None)
    assert code == 4, ea.lib().attn_last_error()
    assert b"scratch" in ea.lib().attn_last_error()
    # the capacity in the binding is the header's ATTN_DECODE_SCRATCH_BYTES
    text = open(HEADER).read()
    assert "#define ATTN_DECODE_SCRATCH_BYTES ((size_t)40 << 20)" in text
    assert ea.DECODE_SCRATCH_BYTES == 40 << 20

"""The block manager (host bookkeeping of the paged KV cache) on the CPU, and
the oracle's cache write pinned by a round trip through its paged gather.

The central property, checked on random operation sequences: after any mix
of adding, forking, appending to and freeing sequences -- with every block
copy the manager asks for applied to a simulated pool -- reading each live
sequence through its block table gives back exactly the tokens appended to
it (and to its ancestors before the fork), reference counts equal the number
of sequences holding each block, and the free blocks are exactly those no
sequence holds."""

import numpy as np
import pytest

import exact_attention_34_amd as ea
import oracle

BS = 16


def test_append_fork_copy_on_write():
    m = ea.BlockManager(8, BS)
    m.add_sequence(0)
    slots, copies = m.append(0, 20)
    assert list(slots) == list(range(20)) and copies == []
    m.fork(0, 1)
    table, ctx = m.block_table([0, 1], 4)
    assert (table[0] == table[1]).all() and list(ctx) == [20, 20]
    assert m.ref_count(table[0][0]) == 2 and m.ref_count(table[0][1]) == 2
    # the child's last block is partial and shared: it moves to a copy
    slots, copies = m.append(1, 3)
    assert len(copies) == 1 and copies[0][0] == table[0][1]
    new = copies[0][1]
    assert list(slots) == [new * BS + 4, new * BS + 5, new * BS + 6]
    t2, ctx2 = m.block_table([0, 1], 4)
    assert t2[0][1] == table[0][1] and t2[1][1] == new and t2[1][0] == t2[0][0]
    assert list(ctx2) == [20, 23]
    assert m.ref_count(t2[0][0]) == 2 and m.ref_count(t2[0][1]) == 1 and m.ref_count(new) == 1
    # the parent now holds its last block alone: it appends in place
    slots, copies = m.append(0, 1)
    assert copies == [] and slots[0] == t2[0][1] * BS + 4


def test_full_shared_blocks_stay_shared():
    m = ea.BlockManager(10, BS)
    m.add_sequence(7)
    m.append(7, 32)                   # two full blocks
    m.fork(7, 8)
    slots, copies = m.append(8, 5)    # a new block, no copy
    assert copies == []
    t, _ = m.block_table([7, 8], 3)
    assert (t[0][:2] == t[1][:2]).all() and t[0][2] == -1 and t[1][2] >= 0
    assert m.ref_count(t[0][0]) == 2 and m.ref_count(t[1][2]) == 1


def test_free_returns_blocks():
    m = ea.BlockManager(6, BS)
    m.add_sequence(1)
    m.append(1, 40)
    m.fork(1, 2)
    m.append(2, 10)
    # seq 1: blocks a, b, c (c holds 8 tokens); seq 2 shares a, b and moved
    # to a copy of c, plus one more block: 5 blocks in use
    assert m.num_free() == 1
    m.free_sequence(1)
    # a and b are still held by seq 2; only c becomes free
    assert m.num_free() == 2
    m.free_sequence(2)
    assert m.num_free() == 6
    assert all(m.ref_count(b) == 0 for b in range(6))


def test_out_of_blocks_changes_nothing():
    m = ea.BlockManager(3, BS)
    m.add_sequence(0)
    m.append(0, 40)                   # 3 blocks
    before = (m.num_free(), m.length(0), m.block_table([0], 3))
    with pytest.raises(ea.AttnError) as e:
        m.append(0, 20)
    assert e.value.code == 7
    after = (m.num_free(), m.length(0), m.block_table([0], 3))
    assert before[0] == after[0] and before[1] == after[1]
    assert (before[2][0] == after[2][0]).all()


@pytest.mark.parametrize("call,code", [
    (lambda m: m.add_sequence(0), 2),            # duplicate
    (lambda m: m.fork(5, 6), 2),                 # unknown parent
    (lambda m: m.fork(0, 0), 2),                 # existing child
    (lambda m: m.append(9, 1), 2),               # unknown sequence
    (lambda m: m.free_sequence(9), 2),
    (lambda m: m.block_table([0], 0), 2),        # table too narrow
])
def test_errors(call, code):
    m = ea.BlockManager(4, BS)
    m.add_sequence(0)
    m.append(0, 5)
    with pytest.raises(ea.AttnError) as e:
        call(m)
    assert e.value.code == code


def test_create_rejects_bad_sizes():
    with pytest.raises(ea.AttnError):
        ea.BlockManager(-1, BS)
    with pytest.raises(ea.AttnError):
        ea.BlockManager(4, 0)


def test_deterministic_ids():
    def run():
        m = ea.BlockManager(50, BS)
        m.add_sequence(0)
        m.append(0, 37)
        m.fork(0, 1)
        m.append(1, 9)
        m.free_sequence(0)
        m.add_sequence(2)
        m.append(2, 70)
        return m.block_table([1, 2], 8)
    a, b = run(), run()
    assert (a[0] == b[0]).all() and (a[1] == b[1]).all()


@pytest.mark.parametrize("seed", range(6))
def test_random_operations_keep_every_sequence_intact(seed):
    rng = np.random.default_rng(seed)
    nb = 40
    m = ea.BlockManager(nb, BS)
    pool = np.full(nb * BS, -1, dtype=np.int64)   # simulated cache: one value per slot
    logical = {}                                   # seq -> list of token values
    next_id, next_val = 0, 0
    for _ in range(300):
        op = rng.integers(0, 4)
        live = sorted(logical)
        if op == 0 or not live:
            m.add_sequence(next_id)
            logical[next_id] = []
            next_id += 1
        elif op == 1:
            parent = live[rng.integers(len(live))]
            m.fork(parent, next_id)
            logical[next_id] = list(logical[parent])
            next_id += 1
        elif op == 2:
            s = live[rng.integers(len(live))]
            n = int(rng.integers(1, 20))
            try:
                slots, copies = m.append(s, n)
            except ea.AttnError as e:
                assert e.code == 7   # out of blocks: nothing changed
                continue
            for src, dst in copies:        # copy-on-write first, then the writes
                pool[dst * BS:(dst + 1) * BS] = pool[src * BS:(src + 1) * BS]
            vals = list(range(next_val, next_val + n))
            next_val += n
            pool[slots] = vals
            logical[s] += vals
        else:
            s = live[rng.integers(len(live))]
            m.free_sequence(s)
            del logical[s]
        # invariants
        ids = sorted(logical)
        if ids:
            maxb = max((len(v) + BS - 1) // BS for v in logical.values()) or 1
            table, ctx = m.block_table(ids, maxb)
            refs = np.zeros(nb, dtype=int)
            for r, s in enumerate(ids):
                assert ctx[r] == len(logical[s])
                blocks = [b for b in table[r] if b >= 0]
                assert len(blocks) == (len(logical[s]) + BS - 1) // BS
                assert len(set(blocks)) == len(blocks)
                for b in blocks:
                    refs[b] += 1
                t = np.arange(len(logical[s]))
                got = pool[table[r][t // BS] * BS + t % BS] if len(t) else np.array([])
                assert list(got) == logical[s], "sequence %d reads wrong tokens" % s
            assert all(m.ref_count(b) == refs[b] for b in range(nb))
            assert m.num_free() == int((refs == 0).sum())
        else:
            assert m.num_free() == nb


def test_oracle_kv_write_round_trip():
    # pin: writing tokens and reading the sequence back through the oracle's
    # paged gather returns the written rows
    rng = np.random.default_rng(3)
    hkv, d, nb = 2, 8, 5
    kp = np.full((nb, hkv, BS, d), np.nan)
    vp = np.full((nb, hkv, BS, d), np.nan)
    table = np.array([3, 0, 4])
    n = 37
    t = np.arange(n)
    slots = table[t // BS] * BS + t % BS
    kn = rng.standard_normal((n, hkv, d))
    vn = rng.standard_normal((n, hkv, d))
    kp2, vp2 = oracle.paged_kv_write(kp, vp, kn, vn, np.concatenate([slots, [-1, 10 ** 6]]),
                                     BS)
    assert np.array_equal(oracle.gather_paged_kv(kp2, table, n, BS), kn)
    assert np.array_equal(oracle.gather_paged_kv(vp2, table, n, BS), vn)
    # untouched slots keep their contents
    assert np.isnan(kp2[1]).all() and np.isnan(kp2[2]).all()
    kc, vc = oracle.paged_kv_copy_blocks(kp2, vp2, [3], [1])
    assert np.array_equal(kc[1], kp2[3]) and np.array_equal(vc[1], vp2[3])

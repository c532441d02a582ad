"""Seeded synthetic inputs for exact attention and paged decode.

This module generates inputs only.  It holds none of the attention
arithmetic, and it is the one piece of code that both the fp64 oracle side
(tests, the CPU baseline) and the GPU side (tests, benchmark) use, so that the
two see bit-identical inputs.

Values are drawn as float64 from ``numpy.random.default_rng(seed)`` (PCG64),
N(0, 1), and rounded once to the target dtype with torch's round-to-nearest-
even conversion.  Tensors are returned on the CPU; the caller moves them to
the GPU.

The five standard workloads (sizes from the subject's benchmark list):

1. single-head non-causal prefill, batch 1, N=128, d=64, fp32;
2. causal prefill, batch 4, 16 heads, N=2048, d=128, bf16, with 1 % of the
   Q rows and 1 % of the K rows of every (batch, head) multiplied by 20 so the
   logits reach about +-1e3 (online-softmax stability stress);
3. causal prefill, batch 1, 32 query heads / 8 KV heads, N=16384, d=128, bf16;
4. paged decode, 64 sequences with context lengths uniform in [512, 8192],
   32 query heads / 8 KV heads, d=128, bf16, 16-token blocks, shuffled block
   table;
5. shared-prefix paged decode, 8 groups x 8 sequences sharing a 4096-token
   prefix per group through common block ids, each with a private 256-token
   suffix; 32 / 8 heads, d=128, bf16, 16-token blocks.
"""

import math
from dataclasses import dataclass, field

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _round(x64, dtype):
    """Round a float64 numpy array once to ``dtype`` (RNE) as a CPU tensor."""
    return torch.from_numpy(np.ascontiguousarray(x64)).to(DTYPES[dtype])


# ----------------------------------------------------------------------------
# prefill
# ----------------------------------------------------------------------------

PREFILL_CONFIGS = {
    1: dict(batch=1, n_q=128, n_k=128, h_q=1, h_kv=1, d=64, dtype="f32",
            causal=False, stress_frac=0.0),
    2: dict(batch=4, n_q=2048, n_k=2048, h_q=16, h_kv=16, d=128, dtype="bf16",
            causal=True, stress_frac=0.01),
    3: dict(batch=1, n_q=16384, n_k=16384, h_q=32, h_kv=8, d=128, dtype="bf16",
            causal=True, stress_frac=0.0),
}


@dataclass
class PrefillInputs:
    q: torch.Tensor          # [B][Nq][Hq][d]
    k: torch.Tensor          # [B][Nk][Hkv][d]
    v: torch.Tensor          # [B][Nk][Hkv][d]
    causal: bool
    scale: float
    dtype: str
    stress_rows_q: np.ndarray = None   # [B][Hq][n] token rows scaled x20 (or None)
    stress_rows_k: np.ndarray = None   # [B][Hkv][n]


def prefill_inputs(batch, n_q, n_k, h_q, h_kv, d, dtype, seed, causal=False,
                   stress_frac=0.0, stress_mult=20.0, scale=None):
    """Q, K, V ~ N(0, 1) drawn in the order Q, K, V, then the stress rows.

    With ``stress_frac > 0``, for every (batch, head) independently,
    ``round(stress_frac * N)`` distinct token rows of Q (and, separately, of
    K) are multiplied by ``stress_mult`` in float64 before the one rounding
    to ``dtype``.
    """
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((batch, n_q, h_q, d))
    k = rng.standard_normal((batch, n_k, h_kv, d))
    v = rng.standard_normal((batch, n_k, h_kv, d))
    rq = rk = None
    if stress_frac > 0:
        nq_s = int(round(stress_frac * n_q))
        nk_s = int(round(stress_frac * n_k))
        rq = np.zeros((batch, h_q, nq_s), dtype=np.int64)
        rk = np.zeros((batch, h_kv, nk_s), dtype=np.int64)
        for b in range(batch):
            for h in range(h_q):
                rq[b, h] = rng.choice(n_q, nq_s, replace=False)
                q[b, rq[b, h], h, :] *= stress_mult
            for h in range(h_kv):
                rk[b, h] = rng.choice(n_k, nk_s, replace=False)
                k[b, rk[b, h], h, :] *= stress_mult
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return PrefillInputs(_round(q, dtype), _round(k, dtype), _round(v, dtype),
                         bool(causal), float(scale), dtype, rq, rk)


def prefill_config(cfg_id, seed=None):
    """Inputs of standard prefill workload ``cfg_id`` (1, 2 or 3); seed = id."""
    c = dict(PREFILL_CONFIGS[cfg_id])
    return prefill_inputs(seed=cfg_id if seed is None else seed, **c)


def prefill_flops(batch, n_q, n_k, h_q, d, causal):
    """Algorithmic FLOP: 4*d per visible (query, key) pair (QK^T and PV)."""
    if causal:
        off = n_k - n_q
        # visible keys of row i: clamp(i + off + 1, 0, n_k)
        i = np.arange(n_q, dtype=np.int64)
        pairs = int(np.clip(i + off + 1, 0, n_k).sum())
    else:
        pairs = n_q * n_k
    return 4 * d * batch * h_q * pairs


# ----------------------------------------------------------------------------
# paged decode
# ----------------------------------------------------------------------------

DECODE_CONFIGS = {
    4: dict(num_seqs=64, ctx_lo=512, ctx_hi=8192, h_q=32, h_kv=8, d=128,
            block_size=16, dtype="bf16"),
    5: dict(groups=8, per_group=8, prefix=4096, suffix=256, h_q=32, h_kv=8,
            d=128, block_size=16, dtype="bf16"),
}


@dataclass
class DecodeInputs:
    q: torch.Tensor            # [S][Hq][d]
    k_cache: torch.Tensor      # [num_blocks][Hkv][block_size][d]
    v_cache: torch.Tensor      # [num_blocks][Hkv][block_size][d]
    block_table: torch.Tensor  # [S][max_blocks_per_seq] int32, -1 = unused
    context_lens: torch.Tensor  # [S] int32
    block_size: int
    scale: float
    dtype: str
    k_logical: list = field(default_factory=list)  # per sequence [ctx][Hkv][d]
    v_logical: list = field(default_factory=list)
    # shared-prefix groups (None when the inputs have no group structure):
    # group g is sequences group_starts[g] .. group_starts[g+1]-1, whose first
    # prefix_lens[g] tokens are the same logical data
    group_starts: torch.Tensor = None   # [G + 1] int32
    prefix_lens: torch.Tensor = None    # [G] int32

    @property
    def max_context_len(self):
        return int(self.context_lens.max()) if len(self.context_lens) else 0


def _fill_pool(pool, table, logical, block_size):
    """Write each sequence's logical rows into its physical blocks."""
    for s, rows in enumerate(logical):
        n = rows.shape[0]
        for lb in range((n + block_size - 1) // block_size):
            t0 = lb * block_size
            t1 = min(n, t0 + block_size)
            pool[int(table[s, lb]), :, : t1 - t0, :] = rows[t0:t1].transpose(0, 1)


def build_paged(k_logical, v_logical, block_size, rng=None, shared_blocks=None,
                max_blocks_per_seq=None, nan_fill=True, spare_blocks=0,
                shuffle=True):
    """Lay per-sequence logical K/V out in a paged pool and build its table.

    ``k_logical[s]`` is ``[ctx_s][Hkv][d]``.  Physical block ids are a random
    permutation of the pool (``shuffle``) or the identity order.
    ``shared_blocks`` optionally maps ``(s, lb) -> key``: entries with equal
    keys get one physical block (a shared prefix).  Unused slots of a
    sequence's last block, and ``spare_blocks`` extra blocks, hold NaN when
    ``nan_fill`` so that a kernel that reads past a context shows up.
    Returns (k_cache, v_cache, block_table, context_lens).
    """
    S = len(k_logical)
    ctx = [int(x.shape[0]) for x in k_logical]
    nblk = [(c + block_size - 1) // block_size for c in ctx]
    if max_blocks_per_seq is None:
        max_blocks_per_seq = max(nblk) if nblk else 0
    # logical block -> unique slot
    slot_of = {}
    order = []
    for s in range(S):
        for lb in range(nblk[s]):
            key = shared_blocks.get((s, lb), (s, lb)) if shared_blocks else (s, lb)
            if key not in slot_of:
                slot_of[key] = len(order)
                order.append(key)
    n_unique = len(order)
    num_blocks = n_unique + spare_blocks
    if shuffle:
        perm = rng.permutation(num_blocks)
    else:
        perm = np.arange(num_blocks)
    table = np.full((S, max(max_blocks_per_seq, 1)), -1, dtype=np.int32)
    for s in range(S):
        for lb in range(nblk[s]):
            key = shared_blocks.get((s, lb), (s, lb)) if shared_blocks else (s, lb)
            table[s, lb] = perm[slot_of[key]]
    h_kv, d = k_logical[0].shape[1], k_logical[0].shape[2]
    dt = k_logical[0].dtype
    fill = float("nan") if nan_fill else 0.0
    k_cache = torch.full((num_blocks, h_kv, block_size, d), fill, dtype=dt)
    v_cache = torch.full((num_blocks, h_kv, block_size, d), fill, dtype=dt)
    _fill_pool(k_cache, table, k_logical, block_size)
    _fill_pool(v_cache, table, v_logical, block_size)
    return (k_cache, v_cache, torch.from_numpy(table),
            torch.tensor(ctx, dtype=torch.int32))


def decode_inputs(context_lens, h_q, h_kv, d, block_size, dtype, seed,
                  nan_fill=True, spare_blocks=0, shuffle=True,
                  max_blocks_per_seq=None, scale=None):
    """Decode inputs with independent K/V per sequence.

    Draw order: q ``[S][Hq][d]``, then for each sequence its K then V rows
    ``[ctx][Hkv][d]``, then the block permutation.
    """
    rng = np.random.default_rng(seed)
    S = len(context_lens)
    q = _round(rng.standard_normal((S, h_q, d)), dtype)
    kl, vl = [], []
    for c in context_lens:
        kl.append(_round(rng.standard_normal((int(c), h_kv, d)), dtype))
        vl.append(_round(rng.standard_normal((int(c), h_kv, d)), dtype))
    kc, vc, table, ctx = build_paged(kl, vl, block_size, rng=rng,
                                     max_blocks_per_seq=max_blocks_per_seq,
                                     nan_fill=nan_fill, spare_blocks=spare_blocks,
                                     shuffle=shuffle)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return DecodeInputs(q, kc, vc, table, ctx, block_size, float(scale), dtype, kl, vl)


def decode_config4(seed=4, nan_fill=True):
    """64 sequences, context lengths uniform on {512..8192}, shuffled table.

    Draw order: the context lengths first (they fix every other shape), then
    as in :func:`decode_inputs`.  The table has 512 columns (8192 / 16).
    """
    c = DECODE_CONFIGS[4]
    rng = np.random.default_rng(seed)
    ctx = rng.integers(c["ctx_lo"], c["ctx_hi"], size=c["num_seqs"], endpoint=True)
    sub_seed = int(rng.integers(0, 2**31 - 1))
    return decode_inputs(ctx, c["h_q"], c["h_kv"], c["d"], c["block_size"], c["dtype"],
                         sub_seed, nan_fill=nan_fill,
                         max_blocks_per_seq=c["ctx_hi"] // c["block_size"])


def shared_prefix_inputs(groups, h_q, h_kv, d, block_size, dtype, seed, private=False,
                         nan_fill=True, spare_blocks=0, shuffle=True, max_blocks_per_seq=None,
                         scale=None):
    """Decode inputs for groups of sequences that share a prefix.

    ``groups`` is a list of ``(prefix_len, [suffix_len of each member])``.
    Member ``i`` of group ``g`` has context ``prefix_len + suffix_len``; its
    first ``prefix_len`` K/V rows are the group's prefix.  With
    ``private=False`` the prefix's whole blocks are one set of physical blocks
    repeated in every member's table row (a partial last prefix block also
    holds the member's own suffix tokens, so it stays private); with
    ``private=True`` every member owns copies.  Draw order: per group the
    prefix K then V ``[prefix_len][Hkv][d]``, then per member its q
    ``[Hq][d]``, suffix K then suffix V; then the block permutation.
    """
    rng = np.random.default_rng(seed)
    qs, kl, vl = [], [], []
    shared = {}
    starts, plens = [0], []
    for g, (plen, suffixes) in enumerate(groups):
        kp = _round(rng.standard_normal((plen, h_kv, d)), dtype)
        vp = _round(rng.standard_normal((plen, h_kv, d)), dtype)
        for sl in suffixes:
            s = len(qs)
            qs.append(_round(rng.standard_normal((h_q, d)), dtype))
            ks = _round(rng.standard_normal((sl, h_kv, d)), dtype)
            vs = _round(rng.standard_normal((sl, h_kv, d)), dtype)
            kl.append(torch.cat([kp, ks], 0))
            vl.append(torch.cat([vp, vs], 0))
            if not private:
                for lb in range(plen // block_size):
                    shared[(s, lb)] = ("prefix", g, lb)
        starts.append(len(qs))
        plens.append(plen)
    kc, vc, table, ctx = build_paged(kl, vl, block_size, rng=rng,
                                     shared_blocks=shared if not private else None,
                                     max_blocks_per_seq=max_blocks_per_seq, nan_fill=nan_fill,
                                     spare_blocks=spare_blocks, shuffle=shuffle)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    q = torch.stack(qs) if qs else torch.zeros((0, h_q, d), dtype=DTYPES[dtype])
    return DecodeInputs(q, kc, vc, table, ctx, block_size, float(scale), dtype, kl, vl,
                        torch.tensor(starts, dtype=torch.int32),
                        torch.tensor(plens, dtype=torch.int32))


def decode_config5(seed=5, nan_fill=True, private=False):
    """8 groups x 8 sequences sharing a 4096-token prefix per group.

    Every sequence has context 4096 + 256.  With ``private=False`` the 256
    prefix blocks of a group are the same physical ids in all 8 tables (3072
    blocks in the pool).  With ``private=True`` the same logical data is laid
    out with every sequence owning copies of its prefix (17408 blocks), for
    the shared == private check.  Draw order as in
    :func:`shared_prefix_inputs`.
    """
    c = DECODE_CONFIGS[5]
    groups = [(c["prefix"], [c["suffix"]] * c["per_group"])] * c["groups"]
    return shared_prefix_inputs(groups, c["h_q"], c["h_kv"], c["d"], c["block_size"],
                                c["dtype"], seed, private=private, nan_fill=nan_fill)


def decode_bytes(context_lens, h_kv, d, elem_bytes=2):
    """Algorithmic K+V bytes a per-sequence decode must read (logical)."""
    return int(np.asarray(context_lens, dtype=np.int64).sum()) * h_kv * d * elem_bytes * 2


def decode_unique_bytes(block_table, context_lens, block_size, h_kv, d, elem_bytes=2):
    """K+V bytes of the distinct (physical block, slot) pairs actually in use."""
    used = set()
    for s in range(len(context_lens)):
        n = int(context_lens[s])
        for t in range(0, n, block_size):
            used.add((int(block_table[s][t // block_size]), min(block_size, n - t)))
    toks = {}
    for b, n in used:
        toks[b] = max(toks.get(b, 0), n)
    return sum(toks.values()) * h_kv * d * elem_bytes * 2

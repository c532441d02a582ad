"""Plain fp64 CPU oracle: scaled-dot-product attention by its definition.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Nothing on the GPU
path may import this module.

Conventions (readings of the pages, fixed here because the pages leave them
open):

* Layout: q is ``[B][Nq][Hq][d]``, k and v are ``[B][Nk][Hkv][d]``, the output
  is ``[B][Nq][Hq][d]`` and the log-sum-exp is ``[B][Hq][Nq]``.
* Grouped-query attention: query head ``h`` reads key/value head
  ``h // (Hq // Hkv)`` (consecutive query heads share one KV head).  The pages
  do not describe GQA; this mapping is a declared convention.
* Causal mask: bottom-right aligned, key ``j`` is visible to query row ``i``
  when ``j <= i + (Nk - Nq)``.  The pages do not describe a mask; the decoder
  generating one token per step implies it.  With ``Nq == Nk`` this is the
  usual lower triangle.
* A row with no visible key (only possible when ``Nk == 0`` or, under the
  causal mask, ``Nq > Nk``) has output 0 and log-sum-exp ``-inf``.
* The log-sum-exp is in natural-log units: ``lse = m + log(sum_j exp(s_j - m))``.

Arithmetic is numpy float64 throughout.  Inputs that arrive as bf16/fp16/fp32
values are converted to float64 exactly before anything else happens.
"""

import numpy as np

_ROW_CHUNK = 2048


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def allowed_keys(n_q, n_k, causal, rows=None):
    """Boolean ``[len(rows)][n_k]`` matrix of the keys each query row may see.

    ``rows`` defaults to all ``n_q`` rows.  Non-causal: every key.  Causal:
    ``j <= i + (n_k - n_q)`` (bottom-right aligned; for ``n_q == n_k`` this is
    ``j <= i``).
    """
    i = (np.arange(n_q) if rows is None else np.asarray(rows, dtype=np.int64))[:, None]
    j = np.arange(n_k)[None, :]
    if not causal:
        return np.ones((i.shape[0], n_k), dtype=bool)
    return j <= i + (n_k - n_q)


def _two_pass_rows(q_rows, k_h, v_h, scale, allow):
    """Two-pass softmax attention for a set of query rows of one head.

    Follows the definition O = Softmax(Q K^T / sqrt(d_k)) V ("Other people's
    interview notes", question "explain FlashAttention", part 1): the score
    matrix S = scale * Q K^T is formed in full for these rows (as standard
    attention does, per the codelogiq.de FAQ), pass 1 takes the row maximum
    over the visible keys, pass 2 takes the exponentials relative to that
    maximum, their sum l, and O = (sum_j e_j v_j) / l.

    ``allow`` is the ``[rows][n_k]`` visibility mask.  Returns (o, lse).
    """
    s = (q_rows @ k_h.T) * scale                       # [r][n_k]
    s = np.where(allow, s, -np.inf)
    m = s.max(axis=1, initial=-np.inf)                 # pass 1: row max
    has = np.isfinite(m)
    m_safe = np.where(has, m, 0.0)
    e = np.where(allow, np.exp(s - m_safe[:, None]), 0.0)   # pass 2
    l = e.sum(axis=1)
    o = e @ v_h
    o = np.where(has[:, None], o / np.where(has, l, 1.0)[:, None], 0.0)
    lse = np.where(has, m_safe + np.log(np.where(has, l, 1.0)), -np.inf)
    return o, lse


def sdpa(q, k, v, scale=None, causal=False):
    """Exact attention output and log-sum-exp for every query row.

    ``q``: ``[B][Nq][Hq][d]``; ``k``, ``v``: ``[B][Nk][Hkv][d]``.  ``scale``
    defaults to ``1/sqrt(d)`` (the definition's 1/sqrt(d_k)).  Rows are
    processed in chunks of 2048 so that the score block of one chunk is the
    only N-sized temporary.  Returns ``(o [B][Nq][Hq][d], lse [B][Hq][Nq])``,
    both float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Nq, Hq, d = q.shape
    Bk, Nk, Hkv, dk = k.shape
    assert Bk == B and dk == d and v.shape == k.shape
    assert Hkv >= 1 and Hq % Hkv == 0
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    group = Hq // Hkv
    o = np.zeros((B, Nq, Hq, d))
    lse = np.full((B, Hq, Nq), -np.inf)
    if Nq == 0 or Nk == 0:
        return o, lse
    for b in range(B):
        for h in range(Hq):
            kvh = h // group
            k_h = k[b, :, kvh, :]
            v_h = v[b, :, kvh, :]
            for r0 in range(0, Nq, _ROW_CHUNK):
                r1 = min(Nq, r0 + _ROW_CHUNK)
                allow = allowed_keys(Nq, Nk, causal, np.arange(r0, r1))
                oo, ll = _two_pass_rows(q[b, r0:r1, h, :], k_h, v_h, scale, allow)
                o[b, r0:r1, h, :] = oo
                lse[b, h, r0:r1] = ll
    return o, lse


def sdpa_rows(q, k, v, rows, scale=None, causal=False):
    """The same definition as :func:`sdpa`, evaluated only at sampled outputs.

    ``rows`` is an integer array of shape ``[n][3]`` holding ``(b, i, h)``
    triples.  Returns ``(o [n][d], lse [n])``.  Used where the full output
    would take the CPU too long (a long causal sequence): each sampled row
    still sees the whole key/value sequence of its head.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    group = Hq // Hkv
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    o = np.zeros((len(rows), d))
    lse = np.full(len(rows), -np.inf)
    for n, (b, i, h) in enumerate(rows):
        kvh = h // group
        if Nk == 0:
            continue
        allow = allowed_keys(Nq, Nk, causal, [i])
        oo, ll = _two_pass_rows(q[b, i:i + 1, h, :], k[b, :, kvh, :], v[b, :, kvh, :],
                                scale, allow)
        o[n] = oo[0]
        lse[n] = ll[0]
    return o, lse


def sdpa_online(q, k, v, block, scale=None, causal=False):
    """Single-pass tiled attention with the online-softmax update.

    Follows "Other people's interview notes", question "explain
    FlashAttention", part 2: the key/value sequence is cut into blocks of
    ``block`` rows; for each query row the running maximum m and running sum
    l are kept, and for each new block

        m_new = max(m_old, max of the block's scores)
        l_new = exp(m_old - m_new) * l_old + sum_j exp(s_j - m_new)
        O     = exp(m_old - m_new) * O + sum_j exp(s_j - m_new) * v_j

    with O divided by l once, after the last block (the pages do not say when
    the division happens; dividing once at the end is the reading taken).
    The update is applied whether or not the maximum grew (the factor is 1
    when it did not).  This is a second, independent formulation used only
    to check that the tiled method reaches the two-pass result.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    group = Hq // Hkv
    allow_all = allowed_keys(Nq, Nk, causal)
    o = np.zeros((B, Nq, Hq, d))
    lse = np.full((B, Hq, Nq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            kvh = h // group
            qh = q[b, :, h, :]
            m = np.full(Nq, -np.inf)
            l = np.zeros(Nq)
            acc = np.zeros((Nq, d))
            for j0 in range(0, Nk, block):
                j1 = min(Nk, j0 + block)
                s = (qh @ k[b, j0:j1, kvh, :].T) * scale
                allow = allow_all[:, j0:j1]
                s = np.where(allow, s, -np.inf)
                m_new = np.maximum(m, s.max(axis=1))
                # rows that have seen no visible key yet keep m = -inf
                live = np.isfinite(m_new)
                mn = np.where(live, m_new, 0.0)
                alpha = np.where(np.isfinite(m), np.exp(m - mn), 0.0)
                p = np.where(allow, np.exp(s - mn[:, None]), 0.0)
                l = alpha * l + p.sum(axis=1)
                acc = alpha[:, None] * acc + p @ v[b, j0:j1, kvh, :]
                m = m_new
            has = np.isfinite(m)
            o[b, :, h, :] = np.where(has[:, None], acc / np.where(has, l, 1.0)[:, None], 0.0)
            lse[b, h, :] = np.where(has, np.where(has, m, 0.0) + np.log(np.where(has, l, 1.0)),
                                    -np.inf)
    return o, lse


def _bwd_rows(q_rows, k_h, v_h, do_rows, scale, allow):
    """Gradients contributed by a set of query rows of one head.

    The pages say only that the backward pass recomputes the attention
    probabilities from the Q, K, V blocks and the softmax statistics instead
    of storing the N x N matrix ("Other people's interview notes", question
    "explain FlashAttention", part 3; the codelogiq.de FAQ table, row on
    intermediate storage).  They give no formulas, so this is the derivative
    of the part-1 definition by the chain rule, for an upstream gradient dO of
    the output:

        S  = scale * Q K^T (invisible keys excluded)
        P  = softmax of each row of S
        dV = P^T dO                          (O = P V)
        dP = dO V^T
        dS = P * (dP - rowsum(P * dP))       (Jacobian of the row softmax)
        dQ = scale * dS K,    dK = scale * dS^T Q

    Returns ``(dq_rows, dk, dv)``: the rows' dQ, and their contributions to
    the head's dK and dV.
    """
    s = (q_rows @ k_h.T) * scale
    s = np.where(allow, s, -np.inf)
    m = s.max(axis=1, initial=-np.inf)
    has = np.isfinite(m)
    m_safe = np.where(has, m, 0.0)
    e = np.where(allow, np.exp(s - m_safe[:, None]), 0.0)
    l = e.sum(axis=1)
    p = e / np.where(has, l, 1.0)[:, None]              # rows with no key: all 0
    dv = p.T @ do_rows
    dp = do_rows @ v_h.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dq_rows = scale * (ds @ k_h)
    dk = scale * (ds.T @ q_rows)
    return dq_rows, dk, dv


def sdpa_bwd(q, k, v, do, scale=None, causal=False):
    """Gradients of :func:`sdpa`'s output with respect to q, k and v.

    ``do`` is the upstream gradient of the output, ``[B][Nq][Hq][d]``.  Rows
    are taken in chunks of 2048 (:func:`_bwd_rows`); a KV head's dK and dV sum
    the contributions of every query head that reads it (grouped-query
    attention, same head mapping as :func:`sdpa`).  Returns
    ``(dq [B][Nq][Hq][d], dk [B][Nk][Hkv][d], dv [B][Nk][Hkv][d])``, float64.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    assert do.shape == q.shape and v.shape == k.shape and Hq % Hkv == 0
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    group = Hq // Hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    if Nq == 0 or Nk == 0:
        return dq, dk, dv
    for b in range(B):
        for h in range(Hq):
            kvh = h // group
            for r0 in range(0, Nq, _ROW_CHUNK):
                r1 = min(Nq, r0 + _ROW_CHUNK)
                allow = allowed_keys(Nq, Nk, causal, np.arange(r0, r1))
                dqr, dkc, dvc = _bwd_rows(q[b, r0:r1, h, :], k[b, :, kvh, :], v[b, :, kvh, :],
                                          do[b, r0:r1, h, :], scale, allow)
                dq[b, r0:r1, h, :] = dqr
                dk[b, :, kvh, :] += dkc
                dv[b, :, kvh, :] += dvc
    return dq, dk, dv


def gather_paged_kv(pool, table_row, context_len, block_size):
    """Logical, contiguous K (or V) of one sequence read through its block table.

    PagedAttention ("Chapter 3 Advanced principles", section 3.0) keeps the
    KV cache in fixed-size physical blocks and a per-sequence block table
    mapping logical block index to physical block id; shared prefixes are the
    same physical id appearing in several tables.  ``pool`` is
    ``[num_blocks][Hkv][block_size][d]``; logical token ``t`` lives at
    ``pool[table_row[t // block_size], :, t % block_size, :]``.  Returns
    ``[context_len][Hkv][d]``.
    """
    t = np.arange(int(context_len))
    phys = np.asarray(table_row, dtype=np.int64)[t // block_size]
    return _f64(np.asarray(pool)[phys, :, t % block_size, :])


def paged_decode(q, k_pool, v_pool, block_table, context_lens, block_size, scale=None):
    """Single-token decode over a paged KV cache.

    For each sequence ``s`` the query ``q[s]`` (``[Hq][d]``) attends to all
    ``context_lens[s]`` cached tokens (the context length includes the
    current token; no other mask).  The cache is first read back into its
    logical order with :func:`gather_paged_kv`, then the plain definition
    (:func:`sdpa` with one query row, non-causal) is applied.  Returns
    ``(o [S][Hq][d], lse [S][Hq])``.
    """
    q = _f64(q)
    S, Hq, d = q.shape
    o = np.zeros((S, Hq, d))
    lse = np.full((S, Hq), -np.inf)
    for s in range(S):
        n = int(context_lens[s])
        if n == 0:
            continue
        kl = gather_paged_kv(k_pool, block_table[s], n, block_size)
        vl = gather_paged_kv(v_pool, block_table[s], n, block_size)
        oo, ll = sdpa(q[s][None, None], kl[None], vl[None], scale=scale, causal=False)
        o[s] = oo[0, 0]
        lse[s] = ll[0, :, 0]
    return o, lse


def paged_kv_write(k_pool, v_pool, k_new, v_new, slots, block_size):
    """The paged KV cache after writing new tokens (numpy copies).

    PagedAttention's cache keeps token t of a sequence at slot
    ``table[t // block_size] * block_size + t % block_size`` of a pool of
    fixed-size blocks ("Chapter 3 Advanced principles", section 3.0).  Token
    ``i``'s rows (``k_new[i]``, ``v_new[i]``: ``[Hkv][d]``) go to slot
    ``slots[i]``; slots outside the pool are skipped.  The pools are
    ``[num_blocks][Hkv][block_size][d]``.
    """
    k_pool, v_pool = np.array(k_pool, copy=True), np.array(v_pool, copy=True)
    n_slots = k_pool.shape[0] * block_size
    for i, slot in enumerate(np.asarray(slots, dtype=np.int64)):
        if 0 <= slot < n_slots:
            k_pool[slot // block_size, :, slot % block_size, :] = k_new[i]
            v_pool[slot // block_size, :, slot % block_size, :] = v_new[i]
    return k_pool, v_pool


def paged_kv_copy_blocks(k_pool, v_pool, src, dst):
    """The pools after copying block ``src[i]`` to block ``dst[i]`` (copy-on-
    write of a shared block before it is written, same section); pairs naming
    a block outside the pool are skipped."""
    k_pool, v_pool = np.array(k_pool, copy=True), np.array(v_pool, copy=True)
    nb = k_pool.shape[0]
    for s, d in zip(np.asarray(src), np.asarray(dst)):
        if 0 <= s < nb and 0 <= d < nb:
            k_pool[d] = k_pool[s]
            v_pool[d] = v_pool[s]
    return k_pool, v_pool

"""Pins for the fp64 oracle: it is checked against things other than itself.

* hand-derived examples from the definition (tests/golden/hand_examples.json);
* brute force in 50-digit arithmetic (mpmath) on tiny inputs, with its own
  mask and head mapping written independently of the oracle;
* closed forms (one key, zero query, identity V, constant V);
* invariants the mathematics fixes (shift, permutation, power-of-two scale,
  GQA == repeated-KV MHA, causal row == prefix attention, LSE normalises);
* torch's CPU scaled_dot_product_attention in float64 on small shapes;
* the tiled online-softmax formulation reaching the two-pass result;
* planted mistakes (in the oracle, on the CPU) that each pin must catch.

No GPU is used here.
"""

import json
import math
import os

import mpmath
import zlib

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oa
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _rand(shape, rng, scale=1.0):
    return rng.standard_normal(shape) * scale


# ----------------------------------------------------------------------------
# brute force, 50 digits
# ----------------------------------------------------------------------------

def brute_force(q, k, v, scale, causal):
    """Every output element from the definition, in 50-digit arithmetic.

    Softmax here is exp(s_j) / sum exp(s_j) with no max subtraction (50 digits
    hold it for the small logits used), the mask is written as "key j is at
    most (n_k - n_q) positions past row i", and query head h uses key head
    floor(h * Hkv / Hq).
    """
    mpmath.mp.dps = 50
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    o = np.zeros((B, Nq, Hq, d))
    lse = np.full((B, Hq, Nq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            kh = (h * Hkv) // Hq
            for i in range(Nq):
                vis = [j for j in range(Nk) if (not causal) or (j - (Nk - Nq) <= i)]
                if not vis:
                    continue
                s = {}
                for j in vis:
                    acc = mpmath.mpf(0)
                    for c in range(d):
                        acc += mpmath.mpf(float(q[b, i, h, c])) * mpmath.mpf(float(k[b, j, kh, c]))
                    s[j] = acc * mpmath.mpf(scale)
                z = mpmath.fsum(mpmath.exp(s[j]) for j in vis)
                for c in range(d):
                    num = mpmath.fsum(mpmath.exp(s[j]) * mpmath.mpf(float(v[b, j, kh, c]))
                                      for j in vis)
                    o[b, i, h, c] = float(num / z)
                lse[b, h, i] = float(mpmath.log(z))
    return o, lse


BRUTE_CASES = [
    # (B, Nq, Nk, Hq, Hkv, d, causal)
    (1, 1, 1, 1, 1, 1, False),
    (1, 2, 2, 1, 1, 2, True),
    (1, 3, 3, 2, 1, 4, True),
    (2, 5, 5, 2, 2, 2, False),
    (1, 8, 8, 4, 2, 4, True),
    (1, 3, 8, 2, 1, 2, True),      # bottom-right mask, Nq < Nk
    (1, 5, 3, 2, 1, 1, True),      # Nq > Nk: the first rows see nothing
    (1, 4, 7, 3, 1, 2, False),
]


@pytest.mark.parametrize("case", BRUTE_CASES)
def test_oracle_matches_brute_force(case):
    B, Nq, Nk, Hq, Hkv, d, causal = case
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()))
    q, k, v = _rand((B, Nq, Hq, d), rng), _rand((B, Nk, Hkv, d), rng), _rand((B, Nk, Hkv, d), rng)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.sdpa(q, k, v, scale, causal)
    ob, lb = brute_force(q, k, v, scale, causal)
    assert np.max(np.abs(o - ob)) <= 1e-13
    fin = np.isfinite(lb)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.max(np.abs(lse[fin] - lb[fin]), initial=0.0) <= 1e-13
    # rows with nothing visible: output 0, lse -inf
    assert np.all(o[np.broadcast_to(~fin.transpose(0, 2, 1)[..., None], o.shape)] == 0.0)


# ----------------------------------------------------------------------------
# hand-derived examples
# ----------------------------------------------------------------------------

def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_hand_examples(case):
    q, k, v = (np.array(case[x], dtype=np.float64) for x in ("q", "k", "v"))
    o, lse = oracle.sdpa(q, k, v, case["scale"], case["causal"])
    np.testing.assert_allclose(o, np.array(case["o"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, np.array(case["lse"]), rtol=0, atol=1e-14)


# ----------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------

def test_single_key_returns_v():
    rng = np.random.default_rng(1)
    q, k, v = _rand((2, 5, 3, 8), rng), _rand((2, 1, 3, 8), rng), _rand((2, 1, 3, 8), rng)
    o, lse = oracle.sdpa(q, k, v)
    np.testing.assert_array_equal(o, np.broadcast_to(v, o.shape))
    # lse of a single visible key is its logit
    s = np.einsum("bihc,bjhc->bhij", q, k)[..., 0] / math.sqrt(8)
    np.testing.assert_allclose(lse, s, rtol=0, atol=1e-14)


def test_two_keys_sigmoid():
    rng = np.random.default_rng(2)
    q, k, v = _rand((1, 6, 1, 4), rng), _rand((1, 2, 1, 4), rng), _rand((1, 2, 1, 4), rng)
    o, _ = oracle.sdpa(q, k, v, 0.7)
    s = 0.7 * (q[0, :, 0, :] @ k[0, :, 0, :].T)
    p1 = 1.0 / (1.0 + np.exp(s[:, 1] - s[:, 0]))   # sigmoid(s1 - s2)
    expect = p1[:, None] * v[0, 0, 0] + (1 - p1)[:, None] * v[0, 1, 0]
    np.testing.assert_allclose(o[0, :, 0, :], expect, rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_is_mean_of_visible_v(causal):
    rng = np.random.default_rng(3)
    N, d = 37, 5
    q = np.zeros((1, N, 2, d))
    k, v = _rand((1, N, 1, d), rng), _rand((1, N, 1, d), rng)
    o, lse = oracle.sdpa(q, k, v, causal=causal)
    if causal:
        expect = np.cumsum(v[0, :, 0, :], axis=0) / np.arange(1, N + 1)[:, None]
        cnt = np.arange(1, N + 1)
    else:
        expect = np.broadcast_to(v[0, :, 0, :].mean(0), (N, d))
        cnt = np.full(N, N)
    for h in range(2):
        np.testing.assert_allclose(o[0, :, h, :], expect, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[0, h], np.log(cnt), rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_identity_v_exposes_probability_rows(causal):
    rng = np.random.default_rng(4)
    N = 16
    q, k = _rand((1, N, 1, N), rng, 2.0), _rand((1, N, 1, N), rng, 2.0)
    v = np.eye(N)[None, :, None, :]
    o, _ = oracle.sdpa(q, k, v, causal=causal)
    P = o[0, :, 0, :]
    np.testing.assert_allclose(P.sum(1), 1.0, rtol=0, atol=1e-12)
    assert np.all(P >= 0)
    if causal:
        assert np.all(np.triu(P, 1) == 0.0)
    # against softmax written out row by row
    s = q[0, :, 0, :] @ k[0, :, 0, :].T / math.sqrt(N)
    for i in range(N):
        row = s[i, : (i + 1 if causal else N)]
        e = np.exp(row - row.max())
        np.testing.assert_allclose(P[i, : len(row)], e / e.sum(), rtol=1e-13, atol=1e-15)


def test_constant_v_returns_constant():
    rng = np.random.default_rng(5)
    q, k = _rand((2, 9, 4, 8), rng, 5.0), _rand((2, 9, 2, 8), rng, 5.0)
    c = rng.standard_normal(8)
    v = np.broadcast_to(c, (2, 9, 2, 8)).copy()
    for causal in (False, True):
        o, _ = oracle.sdpa(q, k, v, causal=causal)
        np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=0, atol=1e-14)


# ----------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("block", [1, 7, 64, 300])
@pytest.mark.parametrize("causal", [False, True])
def test_online_softmax_equals_two_pass(block, causal):
    rng = np.random.default_rng(block + 10 * causal)
    q, k, v = _rand((2, 70, 4, 16), rng, 3.0), _rand((2, 70, 2, 16), rng, 3.0), _rand((2, 70, 2, 16), rng)
    o1, l1 = oracle.sdpa(q, k, v, causal=causal)
    o2, l2 = oracle.sdpa_online(q, k, v, block=block, causal=causal)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=1e-12, atol=1e-13)


def test_shift_invariance_extreme_logits():
    # adding u to every key row adds q_i . u to every logit of row i
    rng = np.random.default_rng(6)
    d = 16
    q, k, v = _rand((1, 20, 2, d), rng), _rand((1, 20, 2, d), rng), _rand((1, 20, 2, d), rng)
    u = rng.standard_normal(d)
    u *= 1e3 * math.sqrt(d) / np.linalg.norm(u)      # shifts of order +-1e3
    o1, _ = oracle.sdpa(q, k, v, causal=True)
    o2, _ = oracle.sdpa(q, k + u, v, causal=True)
    assert np.all(np.isfinite(o2))
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-9)


def test_permutation_invariance_noncausal():
    rng = np.random.default_rng(7)
    q, k, v = _rand((1, 11, 2, 8), rng), _rand((1, 23, 1, 8), rng), _rand((1, 23, 1, 8), rng)
    perm = rng.permutation(23)
    o1, l1 = oracle.sdpa(q, k, v)
    o2, l2 = oracle.sdpa(q, k[:, perm], v[:, perm])
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-14)


def test_power_of_two_rescaling_is_exact():
    rng = np.random.default_rng(8)
    q, k, v = _rand((1, 33, 2, 16), rng), _rand((1, 33, 2, 16), rng), _rand((1, 33, 2, 16), rng)
    o1, l1 = oracle.sdpa(q, k, v, 0.25, causal=True)
    o2, l2 = oracle.sdpa(2.0 * q, k, v, 0.125, causal=True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_gqa_equals_repeated_kv_mha():
    rng = np.random.default_rng(9)
    Hq, Hkv = 8, 2
    q, k, v = _rand((2, 19, Hq, 8), rng), _rand((2, 19, Hkv, 8), rng), _rand((2, 19, Hkv, 8), rng)
    g = Hq // Hkv
    k_rep = np.repeat(k, g, axis=2)   # head h -> kv head h // g
    v_rep = np.repeat(v, g, axis=2)
    for causal in (False, True):
        o1, l1 = oracle.sdpa(q, k, v, causal=causal)
        o2, l2 = oracle.sdpa(q, k_rep, v_rep, causal=causal)
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)


def test_causal_row_equals_prefix_attention():
    rng = np.random.default_rng(10)
    Nq, Nk = 9, 14
    q, k, v = _rand((1, Nq, 1, 8), rng), _rand((1, Nk, 1, 8), rng), _rand((1, Nk, 1, 8), rng)
    o, _ = oracle.sdpa(q, k, v, causal=True)
    for i in range(Nq):
        n = i + (Nk - Nq) + 1
        oi, _ = oracle.sdpa(q[:, i:i + 1], k[:, :n], v[:, :n], causal=False)
        np.testing.assert_allclose(o[:, i], oi[:, 0], rtol=0, atol=1e-14)


def test_lse_normalises_probabilities():
    rng = np.random.default_rng(11)
    q, k, v = _rand((1, 25, 2, 8), rng, 4.0), _rand((1, 25, 2, 8), rng, 4.0), _rand((1, 25, 2, 8), rng)
    _, lse = oracle.sdpa(q, k, v, causal=True)
    for h in range(2):
        s = q[0, :, h, :] @ k[0, :, h, :].T / math.sqrt(8)
        for i in range(25):
            np.testing.assert_allclose(np.exp(s[i, : i + 1] - lse[0, h, i]).sum(), 1.0,
                                       rtol=0, atol=1e-13)


def test_sampled_rows_equal_full():
    rng = np.random.default_rng(12)
    q, k, v = _rand((2, 40, 4, 8), rng), _rand((2, 40, 2, 8), rng), _rand((2, 40, 2, 8), rng)
    o, lse = oracle.sdpa(q, k, v, causal=True)
    rows = np.array([[0, 0, 0], [1, 39, 3], [0, 17, 2], [1, 5, 1]])
    os_, ls_ = oracle.sdpa_rows(q, k, v, rows, causal=True)
    for n, (b, i, h) in enumerate(rows):
        # same definition; only the BLAS summation order may differ
        np.testing.assert_allclose(os_[n], o[b, i, h], rtol=0, atol=1e-14)
        np.testing.assert_allclose(ls_[n], lse[b, h, i], rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_float64(causal):
    rng = np.random.default_rng(13)
    q, k, v = _rand((2, 30, 3, 16), rng, 2.0), _rand((2, 30, 3, 16), rng, 2.0), _rand((2, 30, 3, 16), rng)
    o, _ = oracle.sdpa(q, k, v, causal=causal)
    t = lambda x: torch.from_numpy(x).permute(0, 2, 1, 3)   # -> [B][H][N][d]
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=causal)
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-13)


def test_empty_inputs():
    q = np.zeros((1, 0, 2, 8))
    k = np.zeros((1, 5, 1, 8))
    o, lse = oracle.sdpa(q, k, k)
    assert o.shape == (1, 0, 2, 8) and lse.shape == (1, 2, 0)
    q = np.ones((1, 3, 2, 8))
    k = np.zeros((1, 0, 1, 8))
    o, lse = oracle.sdpa(q, k, k)
    assert np.all(o == 0) and np.all(lse == -np.inf)


def test_stress_rows_stay_finite():
    # the stress workload's extreme logits (about +-1e3) must not overflow
    inp = workloads.prefill_inputs(1, 256, 256, 2, 2, 128, "bf16", seed=2, causal=True,
                                   stress_frac=0.05)
    q, k, v = (x.float().numpy() for x in (inp.q, inp.k, inp.v))
    o, lse = oracle.sdpa(q, k, v, inp.scale, True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    s_max = np.max(np.abs(np.einsum("bihc,bjhc->bhij", q, k))) * inp.scale
    assert s_max > 300.0
    # rows are convex combinations of V rows: bounded by V's range per column
    assert np.all(o <= v.max(axis=1, keepdims=True).max() + 1e-12)


# ----------------------------------------------------------------------------
# paged decode
# ----------------------------------------------------------------------------

def test_paged_gather_round_trip():
    ctx = [1, 15, 16, 17, 40]
    inp = workloads.decode_inputs(ctx, h_q=4, h_kv=2, d=8, block_size=16, dtype="f32",
                                  seed=3, spare_blocks=3)
    for s, n in enumerate(ctx):
        kl = oracle.gather_paged_kv(inp.k_cache.numpy(), inp.block_table[s].numpy(), n, 16)
        vl = oracle.gather_paged_kv(inp.v_cache.numpy(), inp.block_table[s].numpy(), n, 16)
        np.testing.assert_array_equal(kl, inp.k_logical[s].numpy())
        np.testing.assert_array_equal(vl, inp.v_logical[s].numpy())


def test_decode_equals_last_row_of_causal_prefill():
    ctx = [1, 16, 33, 70]
    inp = workloads.decode_inputs(ctx, h_q=4, h_kv=2, d=16, block_size=16, dtype="f32", seed=4)
    o, lse = oracle.paged_decode(inp.q.numpy(), inp.k_cache.numpy(), inp.v_cache.numpy(),
                                 inp.block_table.numpy(), inp.context_lens.numpy(), 16)
    assert np.all(np.isfinite(o))
    for s, n in enumerate(ctx):
        rng = np.random.default_rng(s)
        # a causal prefill over the sequence whose last query is the decode query
        qq = rng.standard_normal((1, n, 4, 16))
        qq[0, -1] = inp.q[s].numpy()
        op, lp = oracle.sdpa(qq, inp.k_logical[s].numpy()[None], inp.v_logical[s].numpy()[None],
                             inp.scale, causal=True)
        np.testing.assert_allclose(o[s], op[0, -1], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[s], lp[0, :, -1], rtol=0, atol=1e-13)


def test_shared_prefix_equals_private_copies():
    rng = np.random.default_rng(14)
    kp = torch.from_numpy(rng.standard_normal((48, 2, 8)))
    vp = torch.from_numpy(rng.standard_normal((48, 2, 8)))
    kl = [torch.cat([kp, torch.from_numpy(rng.standard_normal((n, 2, 8)))]) for n in (5, 16, 0)]
    vl = [torch.cat([vp, torch.from_numpy(rng.standard_normal((n, 2, 8)))]) for n in (5, 16, 0)]
    shared = {(s, lb): ("p", lb) for s in range(3) for lb in range(3)}
    kc, vc, tab, ctx = workloads.build_paged(kl, vl, 16, rng=rng, shared_blocks=shared)
    kc2, vc2, tab2, ctx2 = workloads.build_paged(kl, vl, 16, rng=rng)
    assert kc.shape[0] < kc2.shape[0]
    q = rng.standard_normal((3, 4, 8))
    o1, l1 = oracle.paged_decode(q, kc.numpy(), vc.numpy(), tab.numpy(), ctx.numpy(), 16)
    o2, l2 = oracle.paged_decode(q, kc2.numpy(), vc2.numpy(), tab2.numpy(), ctx2.numpy(), 16)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_decode_zero_context():
    inp = workloads.decode_inputs([0, 3], h_q=2, h_kv=1, d=4, block_size=16, dtype="f32", seed=5)
    o, lse = oracle.paged_decode(inp.q.numpy(), inp.k_cache.numpy(), inp.v_cache.numpy(),
                                 inp.block_table.numpy(), inp.context_lens.numpy(), 16)
    assert np.all(o[0] == 0) and np.all(lse[0] == -np.inf)
    assert np.all(np.isfinite(o[1]))


# ----------------------------------------------------------------------------
# planted mistakes: each must be caught by one of the pins above
# ----------------------------------------------------------------------------

def _run_brute_pins():
    for case in BRUTE_CASES:
        test_oracle_matches_brute_force(case)


def _mut_no_scale(q_rows, k_h, v_h, scale, allow):
    return _ORIG_TWO_PASS(q_rows, k_h, v_h, 1.0, allow)


def _mut_k_for_v(q_rows, k_h, v_h, scale, allow):
    return _ORIG_TWO_PASS(q_rows, k_h, k_h, scale, allow)


def _mut_sign(q_rows, k_h, v_h, scale, allow):
    return _ORIG_TWO_PASS(q_rows, k_h, v_h, -scale, allow)


def _mut_no_max(q_rows, k_h, v_h, scale, allow):
    s = np.where(allow, (q_rows @ k_h.T) * scale, -np.inf)
    with np.errstate(over="ignore", invalid="ignore"):
        e = np.exp(s)
        l = e.sum(1)
        return (e @ v_h) / l[:, None], np.log(l)


def _mut_mask_off_by_one(n_q, n_k, causal, rows=None):
    i = (np.arange(n_q) if rows is None else np.asarray(rows))[:, None]
    j = np.arange(n_k)[None, :]
    if not causal:
        return np.ones((i.shape[0], n_k), dtype=bool)
    return j < i + (n_k - n_q)


_ORIG_TWO_PASS = oa._two_pass_rows


@pytest.mark.parametrize("mutant", [_mut_no_scale, _mut_k_for_v, _mut_sign])
def test_planted_arithmetic_mistake_is_caught(monkeypatch, mutant):
    monkeypatch.setattr(oa, "_two_pass_rows", mutant)
    with pytest.raises(AssertionError):
        _run_brute_pins()


def test_planted_missing_max_subtraction_is_caught(monkeypatch):
    monkeypatch.setattr(oa, "_two_pass_rows", _mut_no_max)
    with pytest.raises(AssertionError):
        test_stress_rows_stay_finite()


def test_planted_mask_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(oa, "allowed_keys", _mut_mask_off_by_one)
    with pytest.raises(AssertionError):
        _run_brute_pins()


def test_planted_gqa_mapping_mistake_is_caught(monkeypatch):
    real = oa.sdpa

    def wrong_map(q, k, v, scale=None, causal=False):
        # query head h reads kv head h % Hkv instead of h // (Hq // Hkv)
        Hq, Hkv = q.shape[2], k.shape[2]
        idx = np.arange(Hq) % Hkv
        return real(q, np.asarray(k)[:, :, idx], np.asarray(v)[:, :, idx], scale, causal)

    monkeypatch.setattr(oracle, "sdpa", wrong_map)
    with pytest.raises(AssertionError):
        test_oracle_matches_brute_force((1, 8, 8, 4, 2, 4, True))


def test_planted_gather_mistake_is_caught(monkeypatch):
    def wrong_gather(pool, table_row, context_len, block_size):
        t = np.arange(int(context_len))
        phys = np.asarray(table_row, dtype=np.int64)[t // block_size]
        return np.asarray(pool, np.float64)[phys, :, (block_size - 1) - t % block_size, :]

    monkeypatch.setattr(oracle, "gather_paged_kv", wrong_gather)
    with pytest.raises(AssertionError):
        test_paged_gather_round_trip()

"""Pins of the oracle's backward pass (CPU only).

The gradients in ``oracle.sdpa_bwd`` are the chain rule applied to the
definition.  They are tied to things other than themselves:

* central finite differences of the forward oracle (itself pinned by brute
  force) on tiny inputs, for every input element;
* torch autograd through ``scaled_dot_product_attention`` in float64 on the
  CPU (a library routine);
* identities that hold for any input: dK sums to zero over the keys, dV sums
  to the sum of dO over the rows, constant V gives zero dQ and dK, a single
  key gives dV = dO;
* planted mistakes, each of which one of these pins must catch.
"""

import numpy as np
import pytest
import torch

import oracle
import oracle.attention as oa

FD_CASES = [
    # (n_q, n_k, h_q, h_kv, d, causal)
    (1, 1, 1, 1, 2, False),
    (3, 3, 1, 1, 2, True),
    (4, 4, 2, 1, 3, True),
    (5, 5, 2, 2, 2, False),
    (3, 5, 2, 1, 2, True),     # bottom-right aligned mask, n_q < n_k
    (4, 2, 1, 1, 2, False),
]


def _inputs(n_q, n_k, h_q, h_kv, d, seed, batch=1):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((batch, n_q, h_q, d))
    k = rng.standard_normal((batch, n_k, h_kv, d))
    v = rng.standard_normal((batch, n_k, h_kv, d))
    do = rng.standard_normal((batch, n_q, h_q, d))
    return q, k, v, do


def _finite_differences(q, k, v, do, scale, causal, h=1e-5):
    """Central differences of loss = sum(O * dO) for every element of q, k, v."""
    def loss(qq, kk, vv):
        o, _ = oracle.sdpa(qq, kk, vv, scale, causal)
        return float((o * do).sum())
    grads = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(args[which])
        it = np.nditer(g, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[which][idx] += h
            minus[which][idx] -= h
            g[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        grads.append(g)
    return grads


@pytest.mark.parametrize("case", FD_CASES)
def test_bwd_matches_finite_differences(case):
    n_q, n_k, h_q, h_kv, d, causal = case
    q, k, v, do = _inputs(n_q, n_k, h_q, h_kv, d, seed=sum(case[:5]))
    scale = 0.7
    got = oracle.sdpa_bwd(q, k, v, do, scale, causal)
    ref = _finite_differences(q, k, v, do, scale, causal)
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert np.allclose(g, r, rtol=1e-7, atol=1e-8), (name, np.abs(g - r).max())


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("group", [1, 2])
def test_bwd_matches_torch_autograd_float64(causal, group):
    q, k, v, do = _inputs(9, 9, 2 * group, 2, 8, seed=11 + group, batch=2)
    scale = 1.0 / np.sqrt(8)
    dq, dk, dv = oracle.sdpa_bwd(q, k, v, do, scale, causal)
    tq, tk, tv = (torch.tensor(x).permute(0, 2, 1, 3).requires_grad_() for x in (q, k, v))
    # repeat each KV head for its query heads; autograd sums the copies back
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(group, dim=1), tv.repeat_interleave(group, dim=1),
        is_causal=causal, scale=scale)
    o.backward(torch.tensor(do).permute(0, 2, 1, 3))
    for g, t in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.allclose(g, t.grad.permute(0, 2, 1, 3).numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_identities(causal):
    q, k, v, do = _inputs(12, 12, 4, 2, 6, seed=21)
    dq, dk, dv = oracle.sdpa_bwd(q, k, v, do, 0.5, causal)
    # rows of dS sum to zero, so the keys' dK sum to zero
    assert np.abs(dk.sum(axis=1)).max() < 1e-12
    # rows of P sum to one, so the keys' dV sum to the rows' dO (over the
    # query heads that read each KV head)
    want = do.sum(axis=1).reshape(1, 2, 2, 6).sum(axis=2)
    assert np.allclose(dv.sum(axis=1), want, atol=1e-12)


def test_bwd_constant_v_has_no_q_or_k_gradient():
    q, k, v, do = _inputs(7, 7, 1, 1, 4, seed=22)
    v[:] = v[:, :1]                      # every value row equal: O = that row
    dq, dk, dv = oracle.sdpa_bwd(q, k, v, do, 0.5, True)
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13


def test_bwd_single_key():
    q, k, v, do = _inputs(1, 1, 2, 1, 4, seed=23)
    dq, dk, dv = oracle.sdpa_bwd(q, k, v, do, 0.5, False)
    assert np.abs(dq).max() == 0 and np.abs(dk).max() == 0
    assert np.allclose(dv[0, 0, 0], do[0, 0].sum(axis=0), atol=1e-15)


def test_bwd_row_chunks_agree():
    # rows processed in chunks give the same gradients as one pass
    q, k, v, do = _inputs(40, 40, 2, 1, 4, seed=24)
    full = oracle.sdpa_bwd(q, k, v, do, 0.3, True)
    old = oa._ROW_CHUNK
    try:
        oa._ROW_CHUNK = 7
        chunked = oracle.sdpa_bwd(q, k, v, do, 0.3, True)
    finally:
        oa._ROW_CHUNK = old
    for a, b in zip(full, chunked):
        assert np.allclose(a, b, atol=1e-13)


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by the finite-difference pin
# ---------------------------------------------------------------------------

def _mutant(kind):
    real = oa._bwd_rows

    def bad(q_rows, k_h, v_h, do_rows, scale, allow):
        dq, dk, dv = real(q_rows, k_h, v_h, do_rows, scale, allow)
        s = np.where(allow, (q_rows @ k_h.T) * scale, -np.inf)
        m = s.max(axis=1, initial=-np.inf)
        e = np.where(allow, np.exp(s - np.where(np.isfinite(m), m, 0.0)[:, None]), 0.0)
        p = e / np.maximum(e.sum(axis=1, keepdims=True), 1e-300)
        dp = do_rows @ v_h.T
        if kind == "no_rowsum":          # softmax Jacobian without its second term
            ds = p * dp
            return scale * ds @ k_h, scale * ds.T @ q_rows, dv
        if kind == "no_scale_dq":
            return dq / scale, dk, dv
        if kind == "dv_from_dp":         # V's gradient through the wrong factor
            return dq, dk, dp.T @ do_rows
        if kind == "dk_sign":
            return dq, -dk, dv
        if kind == "mask_ignored_in_bwd":
            s2 = (q_rows @ k_h.T) * scale
            e2 = np.exp(s2 - s2.max(axis=1, keepdims=True))
            p2 = e2 / e2.sum(axis=1, keepdims=True)
            return dq, dk, p2.T @ do_rows
        raise AssertionError(kind)
    return bad


@pytest.mark.parametrize("kind", ["no_rowsum", "no_scale_dq", "dv_from_dp", "dk_sign",
                                  "mask_ignored_in_bwd"])
def test_planted_backward_mistake_is_caught(monkeypatch, kind):
    monkeypatch.setattr(oa, "_bwd_rows", _mutant(kind))
    with pytest.raises(AssertionError):
        test_bwd_matches_finite_differences((4, 4, 2, 1, 3, True))

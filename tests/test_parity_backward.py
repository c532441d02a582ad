"""GPU parity of attn_bwd (backward with recomputation) against the fp64
oracle's gradients, through the C ABI.

The GPU gradients are computed from the GPU forward pass's own output O and
log-sum-exp (as a training step would), the oracle's from the exact
definition.  The bound A below is built from the oracle's O, never from the
GPU's.  Tolerance, derived from the arithmetic (the subject states
tolerances for O only).  Each gradient element is bounded through A, the
same expression with every error-carrying factor replaced by its bound:
    A_dV = P^T |dO|
    A_dS = |dS| + P * (rowsum(|dO| * |O|) + d 2^-24 |dO| |V|^T)
    A_dQ = scale A_dS |K|,   A_dK = scale A_dS^T |Q|   (GQA heads summed)
The relative error sources, each at most about 2^-9 of A for bf16:
  * P and dS rounded to 16 bit for their products;
  * delta = rowsum(dO * O) taken from the 16-bit O;
  * the forward log-sum-exp, taken from the rounded probabilities (the
    log-sum-exp tolerance of the forward tests);
  * the fp32 accumulation of q.k in each pass, which reaches about 1.1e-3 of
    a logit for x20 stress keys.
These sum to at most about 1.0e-2 of A.  They are relative only while the
rounded values are normal numbers.  fp16 keeps the fp32 probabilities' range
only down to 2^-14; below it P and dS round to subnormals, with an absolute
error of up to u = 2^-25 each (half the subnormal spacing), which is a large
share of a tiny value.  Summed over a product, that adds the absolute term
    S_dV = u sum_q |dO|,   S_dQ = scale u sum_k |K|,   S_dK = scale u sum_q |Q|
over the visible (query, key) pairs (GQA heads summed); for bf16, whose
exponent range is fp32's, u = 2^-134 and S is nil.  The gate is
|gpu - oracle| <= half an output ulp + S + 2^-6 A elementwise (about 1.5x
margin on the relative part), with no NaN or Inf.
"""

import numpy as np
import pytest
import torch

import exact_attention_34_amd as ea
import oracle
import workloads
from helpers import half_ulp

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TDT = {"f16": torch.float16, "bf16": torch.bfloat16}
EPS = 2.0 ** -6


# half the smallest subnormal of each 16-bit type: the absolute rounding error
# of a value below its normal range
SUB = {"f16": 2.0 ** -25, "bf16": 2.0 ** -134}


def _abs_scale(q, k, v, do, o, scale, causal, dtype="bf16"):
    """A and S for dq, dk, dv (see the module docstring)."""
    q, k, v, do, o = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do, o))
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    u = SUB[dtype]
    aq, ak, av = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    sq, sk, sv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    allow = oracle.allowed_keys(Nq, Nk, causal)
    for b in range(B):
        for h in range(Hq):
            kv = h // g
            s = np.where(allow, (q[b, :, h] @ k[b, :, kv].T) * scale, -np.inf)
            m = s.max(axis=1, initial=-np.inf)
            m = np.where(np.isfinite(m), m, 0.0)
            e = np.where(allow, np.exp(s - m[:, None]), 0.0)
            p = e / np.maximum(e.sum(axis=1, keepdims=True), 1e-300)
            dp = do[b, :, h] @ v[b, :, kv].T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            ado = np.abs(do[b, :, h])
            av[b, :, kv] += p.T @ ado
            ads = np.abs(ds) + p * ((ado * np.abs(o[b, :, h])).sum(1)[:, None]
                                    + d * 2.0 ** -24 * (ado @ np.abs(v[b, :, kv]).T))
            aq[b, :, h] = scale * ads @ np.abs(k[b, :, kv])
            ak[b, :, kv] += scale * ads.T @ np.abs(q[b, :, h])
            vis = allow.astype(np.float64)
            sv[b, :, kv] += u * vis.T @ ado
            sq[b, :, h] = scale * u * vis @ np.abs(k[b, :, kv])
            sk[b, :, kv] += scale * u * vis.T @ np.abs(q[b, :, h])
    return (aq, ak, av), (sq, sk, sv)


def backward_gate(got, ref, a, s, dtype, what):
    g = got.detach().float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(g)), "%s: non-finite gradient" % what
    err = np.abs(g - ref)
    excess = np.maximum(0.0, err - half_ulp(ref, dtype) - s)
    ratio = excess / np.maximum(a, 1e-30)
    worst = float(ratio.max()) if ratio.size else 0.0
    print("%s: max-abs %.3e (max |ref| %.3e) mean-abs %.3e, worst excess / A = %.3e (gate %.3e)"
          % (what, err.max(), np.abs(ref).max(), err.mean(), worst, EPS), flush=True)
    assert worst <= EPS, "%s: error %.3e of A" % (what, worst)


def _case(batch, n_q, n_k, h_q, h_kv, d, dtype, causal, seed, stress=0.0, strided=False):
    inp = workloads.prefill_inputs(batch, n_q, n_k, h_q, h_kv, d, dtype, seed, causal=causal,
                                   stress_frac=stress)
    rng = np.random.default_rng(seed + 1000)
    do = workloads._round(rng.standard_normal((batch, n_q, h_q, d)), dtype)
    dt = TDT[dtype]
    q, k, v, g = (x.to(DEV) for x in (inp.q, inp.k, inp.v, do))
    if strided:
        # every tensor a view into a wider buffer (sequence stride > h * d)
        def widen(x):
            w = torch.zeros(x.shape[0], x.shape[1], x.shape[2] + 1, x.shape[3], dtype=dt,
                            device=DEV)
            w[:, :, 1:] = x
            return w[:, :, 1:]
        q, k, v, g = (widen(x) for x in (q, k, v, g))
    print("case: B=%d nq=%d nk=%d hq=%d hkv=%d d=%d %s causal=%d stress=%g strided=%d"
          % (batch, n_q, n_k, h_q, h_kv, d, dtype, causal, stress, strided), flush=True)
    o, lse = ea.attn_fwd(q, k, v, causal=causal, scale=inp.scale, return_lse=True)
    dq, dk, dv = ea.attn_bwd(q, k, v, o, g, lse, causal=causal, scale=inp.scale)
    torch.cuda.synchronize()
    qn, kn, vn, gn = (x.double().numpy() for x in (inp.q, inp.k, inp.v, do))
    rq, rk, rv = oracle.sdpa_bwd(qn, kn, vn, gn, inp.scale, causal)
    # the bound is built from the oracle's O, so that an error in the GPU's
    # forward output cannot widen the gate that checks the gradients
    o_ref, _ = oracle.sdpa(qn, kn, vn, inp.scale, causal)
    (aq, ak, av), (sq, sk, sv) = _abs_scale(qn, kn, vn, gn, o_ref, inp.scale, causal, dtype)
    what = "B=%d nq=%d nk=%d hq=%d/%d d=%d %s causal=%d" % (batch, n_q, n_k, h_q, h_kv, d,
                                                            dtype, causal)
    backward_gate(dq, rq, aq, sq, dt, what + " dq")
    backward_gate(dk, rk, ak, sk, dt, what + " dk")
    backward_gate(dv, rv, av, sv, dt, what + " dv")
    return q, k, v, o, g, lse, (dq, dk, dv)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_ragged(causal):
    # GQA 4:2, sequence lengths that are not tile multiples
    _case(2, 200, 200, 4, 2, 128, "bf16", causal, seed=90)


@pytest.mark.parametrize("causal", [False, True])
def test_head_dim_64_fp16(causal):
    _case(1, 130, 130, 2, 1, 64, "f16", causal, seed=91)


@pytest.mark.parametrize("n_q,n_k", [(100, 300), (300, 100), (1, 77), (77, 1)])
def test_unequal_lengths_causal(n_q, n_k):
    # bottom-right aligned mask; with n_q > n_k the first rows see no key
    _case(1, n_q, n_k, 2, 2, 128, "bf16", True, seed=92 + n_q)


def test_many_tiles_gqa8():
    _case(1, 1024, 1024, 8, 2, 128, "bf16", True, seed=93)


def test_stress_rows():
    # x20 rows of Q and K (logits to ~1e3), the stress workload's recipe
    _case(1, 512, 512, 2, 2, 128, "bf16", True, seed=94, stress=0.01)


def test_strided_views():
    _case(1, 190, 190, 2, 1, 128, "bf16", False, seed=95, strided=True)


@pytest.mark.parametrize("shape", [
    (2, 300, 300, 16, 16, 128, "bf16", True),    # 32 batch-heads in both kernels
    (1, 200, 200, 32, 8, 128, "bf16", True),     # 32 query heads (dQ), 8 KV heads (dK/dV)
    (4, 260, 260, 16, 16, 64, "f16", False),     # 64 batch-heads, d = 64
], ids=["bh32", "gqa_hq32", "bh64_d64"])
def test_head_groups_on_xcds(shape):
    """Batch-head counts that are multiples of 32, where both kernels take
    their items four batch-heads at a time per XCD."""
    _case(*shape, seed=97 + shape[3])


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_full_scale_sampled_heads(dtype):
    """The N=2048 causal workload (B=4, H=16, d=128, 1 % of Q/K rows x20; bf16
    as benchmarked, and the same shapes in fp16) in the benchmark's launch
    configuration, checked against the oracle on four whole (batch, head)
    slices, one per group of four batch-heads of different XCDs; every other
    gradient element is checked to be finite."""
    if dtype == "bf16":
        inp = workloads.prefill_config(2)
    else:
        c = dict(workloads.PREFILL_CONFIGS[2])
        c["dtype"] = dtype
        inp = workloads.prefill_inputs(seed=12, **c)
    B, N, H, d = inp.q.shape
    rng = np.random.default_rng(7)
    do = workloads._round(rng.standard_normal((B, N, H, d)), dtype)
    q, k, v, g = (x.to(DEV) for x in (inp.q, inp.k, inp.v, do))
    print("case: full-scale B=%d N=%d H=%d d=%d %s causal" % (B, N, H, d, dtype), flush=True)
    o, lse = ea.attn_fwd(q, k, v, causal=True, scale=inp.scale, return_lse=True)
    dq, dk, dv = ea.attn_bwd(q, k, v, o, g, lse, causal=True, scale=inp.scale)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t.float()).all())
    for b, h in ((0, 0), (1, 5), (2, 10), (3, 15)):
        sl = lambda x: x[b:b + 1, :, h:h + 1].double().numpy()
        qn, kn, vn, gn = sl(inp.q), sl(inp.k), sl(inp.v), sl(do)
        rq, rk, rv = oracle.sdpa_bwd(qn, kn, vn, gn, inp.scale, True)
        o_ref, _ = oracle.sdpa(qn, kn, vn, inp.scale, True)
        (aq, ak, av), (sq, sk, sv) = _abs_scale(qn, kn, vn, gn, o_ref, inp.scale, True, dtype)
        what = "full-scale %s b=%d h=%d" % (dtype, b, h)
        backward_gate(dq[b:b + 1, :, h:h + 1], rq, aq, sq, TDT[dtype], what + " dq")
        backward_gate(dk[b:b + 1, :, h:h + 1], rk, ak, sk, TDT[dtype], what + " dk")
        backward_gate(dv[b:b + 1, :, h:h + 1], rv, av, sv, TDT[dtype], what + " dv")


def _random_cases(n, seed):
    """Seeded random backward problems: ragged sizes around the 64- and
    128-row tiles, GQA ratios 1..4, both head dims and dtypes, both masks,
    and wide-buffer (strided) views."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        hkv = int(rng.choice([1, 2]))
        out.append((int(rng.integers(1, 3)), int(rng.integers(1, 300)), int(rng.integers(1, 300)),
                    hkv * int(rng.choice([1, 2, 3, 4])), hkv, int(rng.choice([64, 128])),
                    str(rng.choice(["bf16", "f16"])), bool(rng.integers(0, 2)), 2000 + i,
                    bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("case", _random_cases(12, 55), ids=lambda c: "seed%d" % c[8])
def test_random_problems(case):
    B, nq, nk, hq, hkv, d, dt, causal, seed, strided = case
    _case(B, nq, nk, hq, hkv, d, dt, causal, seed=seed, strided=strided)


def test_deterministic():
    q, k, v, o, g, lse, (dq, dk, dv) = _case(1, 300, 300, 4, 1, 128, "bf16", True, seed=96)
    dq2, dk2, dv2 = ea.attn_bwd(q, k, v, o, g, lse, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)


def test_no_queries_or_no_keys_give_zeros():
    dt = torch.bfloat16
    q = torch.randn(1, 0, 2, 128, device=DEV, dtype=dt)
    k = torch.randn(1, 50, 2, 128, device=DEV, dtype=dt)
    lse = torch.empty(1, 2, 0, device=DEV)
    dq, dk, dv = ea.attn_bwd(q, k, k, q, q, lse)
    torch.cuda.synchronize()
    assert (dk == 0).all() and (dv == 0).all()
    q = torch.randn(1, 40, 2, 128, device=DEV, dtype=dt)
    k = torch.randn(1, 0, 2, 128, device=DEV, dtype=dt)
    lse = torch.full((1, 2, 40), -float("inf"), device=DEV)
    dq, dk, dv = ea.attn_bwd(q, k, k, q, q, lse)
    torch.cuda.synchronize()
    assert (dq == 0).all()

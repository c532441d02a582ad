"""GPU parity of attn_fwd (prefill) against the fp64 oracle, through the C ABI.

Full-size cases use the standard workloads in the launch configuration the
benchmark times.  The long causal GQA workload (N = 16384, 32 query / 8 KV
heads) is compared element by element on all of its 524,288 output rows (the
oracle takes about a minute of host CPU for it); a fast subset of sampled
rows at tile edges runs first, and properties that hold at any size are
checked on the whole output.
"""

import math

import zlib

import numpy as np
import pytest
import torch

import exact_attention_34_amd as ea
import oracle
import workloads
from helpers import assert_close, assert_lse_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TDT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _np(t):
    return t.double().cpu().numpy()


def _run(inp, **kw):
    q, k, v = (x.to(DEV) for x in (inp.q, inp.k, inp.v))
    o, lse = ea.attn_fwd(q, k, v, causal=inp.causal, scale=inp.scale, return_lse=True, **kw)
    torch.cuda.synchronize()
    return o, lse


def _check_full(inp, what):
    print("case:", what, flush=True)
    o, lse = _run(inp)
    ref, ref_lse = oracle.sdpa(_np(inp.q), _np(inp.k), _np(inp.v), inp.scale, inp.causal)
    assert_close(o, ref, TDT[inp.dtype], what)
    assert_lse_close(lse, ref_lse, TDT[inp.dtype], what=what)


# ----------------------------------------------------------------------------
# standard workloads
# ----------------------------------------------------------------------------

def test_config1_fp32_single_head():
    _check_full(workloads.prefill_config(1), "N=128 d=64 fp32 non-causal")


def test_config2_causal_stress_full():
    inp = workloads.prefill_config(2)
    _check_full(inp, "B=4 H=16 N=2048 d=128 bf16 causal, stress rows x20")


def test_config2_shape_fp16_full():
    """The N=2048 workload's shapes and x20 stress rows in fp16 (the f16
    matrix-core path at full size), every output against the oracle."""
    c = dict(workloads.PREFILL_CONFIGS[2])
    c["dtype"] = "f16"
    _check_full(workloads.prefill_inputs(seed=12, **c),
                "B=4 H=16 N=2048 d=128 f16 causal, stress rows x20")


def test_config3_long_causal_gqa_sampled():
    inp = workloads.prefill_config(3)
    print("case: N=16384 Hq=32 Hkv=8 causal, sampled rows", flush=True)
    o, lse = _run(inp)
    B, N, Hq, d = inp.q.shape
    rng = np.random.default_rng(33)
    # every query head; rows at tile edges (first/last rows of 128-row tiles,
    # first and last rows overall) plus random rows
    edges = np.array([0, 1, 63, 64, 127, 128, 8191, 8192, N - 129, N - 128, N - 2, N - 1])
    rows = []
    for h in range(Hq):
        for i in np.concatenate([edges, rng.integers(0, N, 20)]):
            rows.append((0, int(i), h))
    rows = np.array(rows)
    ref, ref_lse = oracle.sdpa_rows(_np(inp.q), _np(inp.k), _np(inp.v), rows, inp.scale, True)
    ri = torch.from_numpy(rows).to(DEV)
    og = o[ri[:, 0], ri[:, 1], ri[:, 2]]
    assert_close(og, ref, torch.bfloat16, "N=16384 sampled %d rows" % len(rows))
    lg = lse[ri[:, 0], ri[:, 2], ri[:, 1]]
    assert_lse_close(lg, ref_lse, torch.bfloat16, what="N=16384 sampled lse")
    # properties of the whole output: finite, and every row is a convex
    # combination of V rows of its KV head, so it lies within V's range
    assert torch.isfinite(o).all()
    vmin = inp.v.float().amin(dim=1).to(DEV)   # [B][Hkv][d]
    vmax = inp.v.float().amax(dim=1).to(DEV)
    g = Hq // inp.k.shape[2]
    of = o.float()
    for h in range(Hq):
        assert (of[:, :, h, :] >= vmin[:, None, h // g, :] - 1e-2).all()
        assert (of[:, :, h, :] <= vmax[:, None, h // g, :] + 1e-2).all()


def test_config3_shapes_fp16_sampled():
    """The N=16384 GQA workload's shapes in fp16 (seed 13), 1,024 rows at tile
    edges and at random against the oracle, every output finite."""
    c = dict(workloads.PREFILL_CONFIGS[3])
    c["dtype"] = "f16"
    inp = workloads.prefill_inputs(seed=13, **c)
    print("case: N=16384 Hq=32 Hkv=8 causal fp16, sampled rows", flush=True)
    o, lse = _run(inp)
    B, N, Hq, d = inp.q.shape
    rng = np.random.default_rng(34)
    edges = np.array([0, 1, 127, 128, 255, 256, 8191, 8192, N - 257, N - 256, N - 2, N - 1])
    rows = np.array([(0, int(i), h) for h in range(Hq)
                     for i in np.concatenate([edges, rng.integers(0, N, 20)])])
    ref, ref_lse = oracle.sdpa_rows(_np(inp.q), _np(inp.k), _np(inp.v), rows, inp.scale, True)
    ri = torch.from_numpy(rows).to(DEV)
    assert_close(o[ri[:, 0], ri[:, 1], ri[:, 2]], ref, torch.float16,
                 "N=16384 fp16 sampled %d rows" % len(rows))
    assert_lse_close(lse[ri[:, 0], ri[:, 2], ri[:, 1]], ref_lse, torch.float16,
                     what="N=16384 fp16 sampled lse")
    assert torch.isfinite(o).all()


@pytest.mark.timeout(1200)
def test_config3_long_causal_gqa_full():
    # every output row and log-sum-exp of the N = 16384 workload against the
    # oracle (the launch the benchmark times: 2,048 work items of 256 rows,
    # 128 rows of each of two query heads of a GQA group, chunks of 2 items
    # per XCD)
    inp = workloads.prefill_config(3)
    print("case: N=16384 Hq=32 Hkv=8 causal, all rows", flush=True)
    o, lse = _run(inp)
    ref, ref_lse = oracle.sdpa(_np(inp.q), _np(inp.k), _np(inp.v), inp.scale, True)
    assert_close(o, ref, torch.bfloat16, "N=16384 all %d rows" % (ref.shape[1] * ref.shape[2]))
    assert_lse_close(lse, ref_lse, torch.bfloat16, what="N=16384 all rows lse")


# ----------------------------------------------------------------------------
# shapes: ragged tails, GQA ratios, head dims, dtypes, masks
# ----------------------------------------------------------------------------

SHAPES = [
    # (B, Nq, Nk, Hq, Hkv, d, dtype, causal)
    (1, 1, 1, 1, 1, 64, "bf16", False),
    (1, 1, 1, 1, 1, 128, "bf16", True),
    (2, 200, 200, 4, 4, 128, "bf16", True),
    (2, 200, 333, 4, 2, 128, "bf16", False),
    (1, 130, 500, 8, 2, 128, "bf16", True),     # Nq < Nk: bottom-right mask
    (1, 300, 100, 4, 1, 64, "bf16", True),      # Nq > Nk: leading rows see nothing
    (3, 129, 129, 2, 1, 64, "f16", True),
    (1, 257, 190, 8, 8, 64, "f16", False),
    (1, 640, 640, 16, 2, 128, "f16", True),
    (1, 384, 384, 8, 1, 128, "bf16", True),     # GQA 8:1
    (2, 300, 300, 3, 1, 128, "bf16", True),     # odd group: 256 rows of one head per workgroup
    (1, 600, 250, 6, 2, 128, "bf16", True),     # odd group, Nq > Nk: whole waves see no key
    (1, 64, 64, 2, 2, 128, "bf16", True),       # one key tile: first tile is also the last
    (1, 65, 65, 2, 1, 128, "bf16", False),      # a second tile with one key
    (1, 129, 129, 4, 2, 64, "f16", True),       # pipeline ends one row / key past a tile
    (2, 96, 96, 3, 1, 128, "f32", True),
    (1, 200, 77, 2, 2, 64, "f32", False),
    (1, 513, 513, 2, 1, 128, "f32", True),
]


def _random_cases(n, seed):
    """Seeded random prefill problems: sizes that straddle tile and block
    edges, GQA ratios 1..8, both head dims and 16-bit dtypes, both masks,
    and head-major (strided) layouts for some operands."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        hkv = int(rng.choice([1, 2, 4]))
        grp = int(rng.choice([1, 2, 3, 4, 8]))
        cases.append(dict(B=int(rng.integers(1, 3)), Nq=int(rng.integers(1, 400)),
                          Nk=int(rng.integers(1, 400)), Hq=hkv * grp, Hkv=hkv,
                          d=int(rng.choice([64, 128])), dt=str(rng.choice(["bf16", "f16"])),
                          causal=bool(rng.integers(0, 2)), strided=int(rng.integers(0, 8)),
                          seed=1000 + i))
    return cases


def _head_major(t):
    """The same values laid out [B][H][N][d] and viewed as [B][N][H][d]."""
    B, N, H, d = t.shape
    out = torch.empty(B, H, N, d, dtype=t.dtype, device=t.device).transpose(1, 2)
    out.copy_(t)
    return out


@pytest.mark.parametrize("case", _random_cases(24, 77), ids=lambda c: "seed%d" % c["seed"])
def test_random_shapes(case):
    c = case
    inp = workloads.prefill_inputs(c["B"], c["Nq"], c["Nk"], c["Hq"], c["Hkv"], c["d"], c["dt"],
                                   seed=c["seed"], causal=c["causal"])
    what = "random %s" % (c,)
    print("case:", what, flush=True)
    q, k, v = (x.to(DEV) for x in (inp.q, inp.k, inp.v))
    # bit i of `strided`: operand i (q, k, v) in head-major layout
    if c["strided"] & 1:
        q = _head_major(q)
    if c["strided"] & 2:
        k = _head_major(k)
    if c["strided"] & 4:
        v = _head_major(v)
    o, lse = ea.attn_fwd(q, k, v, causal=inp.causal, scale=inp.scale, return_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.sdpa(_np(inp.q), _np(inp.k), _np(inp.v), inp.scale, inp.causal)
    assert_close(o, ref, TDT[inp.dtype], what)
    assert_lse_close(lse, ref_lse, TDT[inp.dtype], what=what)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_shapes(shape):
    B, Nq, Nk, Hq, Hkv, d, dt, causal = shape
    inp = workloads.prefill_inputs(B, Nq, Nk, Hq, Hkv, d, dt, seed=zlib.crc32(repr(shape).encode()),
                                   causal=causal)
    _check_full(inp, "shape %s" % (shape,))


def test_empty_key_sequence_gives_zero_and_neg_inf():
    q = torch.randn(1, 5, 2, 128, device=DEV).to(torch.bfloat16)
    k = torch.zeros(1, 0, 1, 128, device=DEV, dtype=torch.bfloat16)
    o, lse = ea.attn_fwd(q, k, k, return_lse=True)
    torch.cuda.synchronize()
    assert (o == 0).all() and (lse == -math.inf).all()


def test_strided_views_of_packed_qkv():
    # q, k, v as views into one [B][N][Hq + 2 Hkv][d] buffer (non-contiguous)
    B, N, Hq, Hkv, d = 2, 190, 4, 2, 128
    rng = np.random.default_rng(5)
    packed = torch.from_numpy(rng.standard_normal((B, N, Hq + 2 * Hkv, d))).to(torch.bfloat16)
    q, k, v = packed[:, :, :Hq], packed[:, :, Hq:Hq + Hkv], packed[:, :, Hq + Hkv:]
    pd = packed.to(DEV)
    qd, kd, vd = pd[:, :, :Hq], pd[:, :, Hq:Hq + Hkv], pd[:, :, Hq + Hkv:]
    out = torch.empty(B, Hq, N, d, device=DEV, dtype=torch.bfloat16).transpose(1, 2)
    ea.attn_fwd(qd, kd, vd, causal=True, out=out)
    torch.cuda.synchronize()
    ref, _ = oracle.sdpa(_np(q), _np(k), _np(v), 1 / math.sqrt(d), True)
    assert_close(out, ref, torch.bfloat16, "strided views")


# ----------------------------------------------------------------------------
# invariants on the GPU
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_identity_v_exposes_probability_rows(causal):
    # with V = I (N = d) the output is the probability matrix itself
    N = d = 128
    rng = np.random.default_rng(21)
    q = torch.from_numpy(rng.standard_normal((1, N, 1, d)) * 2).to(torch.bfloat16).to(DEV)
    k = torch.from_numpy(rng.standard_normal((1, N, 1, d)) * 2).to(torch.bfloat16).to(DEV)
    v = torch.eye(N, dtype=torch.bfloat16, device=DEV)[None, :, None, :].contiguous()
    o = ea.attn_fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    P = o[0, :, 0, :].double().cpu().numpy()
    assert np.all(P >= 0)
    np.testing.assert_allclose(P.sum(1), 1.0, atol=2e-2)
    if causal:
        assert np.all(np.triu(P, 1) == 0.0)
    ref, _ = oracle.sdpa(_np(q), _np(k), _np(v), 1 / math.sqrt(d), causal)
    assert_close(o, ref, torch.bfloat16, "V = I")


def test_zero_query_gives_running_mean():
    N, d = 300, 128
    rng = np.random.default_rng(22)
    q = torch.zeros(1, N, 2, d, dtype=torch.bfloat16, device=DEV)
    k = torch.from_numpy(rng.standard_normal((1, N, 1, d))).to(torch.bfloat16).to(DEV)
    v = torch.from_numpy(rng.standard_normal((1, N, 1, d))).to(torch.bfloat16).to(DEV)
    o, lse = ea.attn_fwd(q, k, v, causal=True, return_lse=True)
    torch.cuda.synchronize()
    vv = v[0, :, 0, :].double().cpu().numpy()
    expect = np.cumsum(vv, 0) / np.arange(1, N + 1)[:, None]
    for h in range(2):
        assert_close(o[0, :, h, :], expect, torch.bfloat16, "Q = 0 head %d" % h)
        np.testing.assert_allclose(lse[0, h].cpu().numpy(), np.log(np.arange(1, N + 1)),
                                   rtol=0, atol=1e-5)


def test_power_of_two_rescaling_is_bitwise_exact():
    inp = workloads.prefill_inputs(1, 333, 333, 4, 2, 128, "bf16", seed=23, causal=True)
    q, k, v = (x.to(DEV) for x in (inp.q, inp.k, inp.v))
    o1 = ea.attn_fwd(q, k, v, causal=True, scale=0.0625)
    o2 = ea.attn_fwd(q * 2, k, v, causal=True, scale=0.03125)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_deterministic():
    inp = workloads.prefill_inputs(2, 700, 700, 8, 2, 128, "bf16", seed=24, causal=True)
    q, k, v = (x.to(DEV) for x in (inp.q, inp.k, inp.v))
    o1, l1 = ea.attn_fwd(q, k, v, causal=True, return_lse=True)
    o2, l2 = ea.attn_fwd(q, k, v, causal=True, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_gqa_equals_repeated_kv():
    inp = workloads.prefill_inputs(1, 256, 256, 8, 2, 128, "bf16", seed=25, causal=True)
    q, k, v = (x.to(DEV) for x in (inp.q, inp.k, inp.v))
    o1 = ea.attn_fwd(q, k, v, causal=True)
    o2 = ea.attn_fwd(q, k.repeat_interleave(4, dim=2).contiguous(),
                     v.repeat_interleave(4, dim=2).contiguous(), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_rows_sum_to_one_on_stress_logits():
    # V = all ones: every output is sum_j p_j = 1, also for rows whose logits
    # reach +-1e3
    inp = workloads.prefill_inputs(2, 512, 512, 4, 4, 128, "bf16", seed=26, causal=True,
                                   stress_frac=0.02)
    q, k = inp.q.to(DEV), inp.k.to(DEV)
    v = torch.ones_like(k)
    o = ea.attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    err = (o.float() - 1).abs().max().item()
    print("ones-V max-abs", err)
    assert err <= 1e-2

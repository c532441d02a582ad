"""Comparison gates shared by the GPU parity tests.

Tolerances (from the subject's acceptance bar):
  * fp32 outputs: max-abs error <= 1e-5 against the fp64 oracle;
  * bf16 / fp16 outputs: mean-abs error <= 1e-3, and max-abs error <= 1e-2
    measured beyond half an output ulp.  A 16-bit output cannot be closer to
    the exact value than half an ulp of its own format: for bf16 and
    |O| >= 4 that is 2^-6 = 0.0156 > 1e-2, so even the exactly rounded result
    would fail a raw 1e-2 bound on the rare large outputs of the stress
    workload.  The gate therefore charges max(0, |gpu - ref| - ulp/2); the raw
    max-abs error and the number of raw exceedances are reported as well.
No NaN or Inf is allowed anywhere.
"""

import numpy as np
import torch

import oracle

MANT_BITS = {torch.bfloat16: 7, torch.float16: 10, torch.float32: 23}


def half_ulp(ref, dtype):
    """Half an ulp of ``dtype`` at each |ref| (normal range)."""
    a = np.abs(ref)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return np.ldexp(1.0, (e - MANT_BITS[dtype] - 1).astype(np.int64))


def compare(gpu, ref, dtype):
    """Error report of a GPU output (tensor) against the fp64 oracle (ndarray)."""
    g = gpu.detach().float().cpu().numpy().astype(np.float64) if torch.is_tensor(gpu) else gpu
    ref = np.asarray(ref, dtype=np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    finite = bool(np.all(np.isfinite(g)))
    err = np.abs(g - ref)
    rep = {
        "finite": finite,
        "max_abs": float(err.max()) if err.size else 0.0,
        "mean_abs": float(err.mean()) if err.size else 0.0,
        "raw_exceed_1e-2": int((err > 1e-2).sum()),
    }
    if dtype == torch.float32:
        rep["gated_max"] = rep["max_abs"]
    else:
        rep["gated_max"] = float(np.max(np.maximum(0.0, err - half_ulp(ref, dtype)), initial=0.0))
    return rep


def assert_close(gpu, ref, dtype, what=""):
    rep = compare(gpu, ref, dtype)
    print("%s %s" % (what, rep), flush=True)
    assert rep["finite"], "%s: non-finite output" % what
    if dtype == torch.float32:
        assert rep["max_abs"] <= 1e-5, "%s: %s" % (what, rep)
    else:
        assert rep["mean_abs"] <= 1e-3, "%s: %s" % (what, rep)
        assert rep["gated_max"] <= 1e-2, "%s: %s" % (what, rep)
    return rep


# Log-sum-exp tolerance (the subject states tolerances for O only; this one
# is derived from the arithmetic).  Two terms:
#  * the kernels normalise by the sum of the probabilities *as rounded* for
#    the P V product (so that O's weights sum to exactly what it is divided
#    by); the log of that sum differs from the exact log-sum-exp by at most
#    ln(1 + 2^-(mantissa bits + 1)): 1.95e-3 for bf16, 2.4e-4 for fp16; fp32
#    inputs keep fp32 probabilities;
#  * the fp32 accumulation of q.k: at most d * 2^-24 * scale * sum_i |q_i k_i|,
#    about 1.1e-3 for a x20 stress key (d = 128, sum_i |q_i k_i| ~ 1.6e3), and
#    for random rows about sqrt(d) = 11 times |q.k| * d * 2^-24, i.e. ~1e-4 of
#    the logit itself (the stress rows reach logits of ~1e3).
# Absolute term = rounding + stress-key accumulation; relative term 1e-4.
LSE_TOL = {torch.bfloat16: 3.1e-3, torch.float16: 1.4e-3, torch.float32: 1e-5}


def assert_lse_close(gpu_lse, ref_lse, dtype, what=""):
    g = gpu_lse.detach().cpu().numpy().astype(np.float64)
    ref = np.asarray(ref_lse, dtype=np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(g)), "%s: lse finiteness differs" % what
    assert np.all(g[~fin] == -np.inf)
    if fin.any():
        err = np.abs(g[fin] - ref[fin])
        bound = LSE_TOL[dtype] + (1e-4 if dtype != torch.float32 else 1e-5) * np.abs(ref[fin])
        print("%s lse max-abs %.3e (worst err/bound %.2f)" % (what, err.max(), (err / bound).max()),
              flush=True)
        assert np.all(err <= bound), "%s: lse error %.3e" % (what, err.max())


def decode_reference(inp):
    """The oracle's single-token decode result, computed from each sequence's
    logical, contiguous K/V (``inp.k_logical``, ``inp.v_logical``): the query
    row of sequence s attends to all of its context by the definition, with
    no block table involved, so a layout mistake shared by the cache builder
    and the kernel cannot pass.  Returns (o [S][Hq][d], lse [S][Hq])."""
    S, Hq, d = inp.q.shape
    assert len(inp.k_logical) == S and len(inp.v_logical) == S
    o = np.zeros((S, Hq, d))
    lse = np.full((S, Hq), -np.inf)
    for s in range(S):
        k = inp.k_logical[s].double().numpy()[None]
        v = inp.v_logical[s].double().numpy()[None]
        oo, ll = oracle.sdpa(inp.q[s].double().numpy()[None, None], k, v, inp.scale, False)
        o[s] = oo[0, 0]
        lse[s] = ll[0, :, 0]
    return o, lse

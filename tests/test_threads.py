"""Calls from several host threads at once, each on its own stream.

Apart from paged_attn_decode_noalloc (one scratch array per GPU) every entry
point is re-entrant: it keeps no state between calls but the calling
thread's error message, and each call only enqueues kernels on the stream it
is given.  Threads that run prefill, backward and paged decode on their own
streams and buffers at the same time reproduce the results of the same calls
made one after another, bit for bit.
"""

import threading

import pytest
import torch

import exact_attention_34_amd as ea
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _problem(seed):
    g = torch.Generator().manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=g).to(torch.bfloat16).to(DEV)
    n = 200 + 37 * seed
    q, k, v, do = r(1, n, 8, 128), r(1, n, 2, 128), r(1, n, 2, 128), r(1, n, 8, 128)
    dec = workloads.decode_inputs([300 + 50 * seed, 17, 900], 8, 2, 128, 16, "bf16", 40 + seed)
    return q, k, v, do, dec


def _run(prob):
    q, k, v, do, dec = prob
    o, lse = ea.attn_fwd(q, k, v, causal=True, return_lse=True)
    dq, dk, dv = ea.attn_bwd(q, k, v, o, do, lse, causal=True)
    out, dlse = ea.paged_attn_decode(dec.q.to(DEV), dec.k_cache.to(DEV), dec.v_cache.to(DEV),
                                     dec.block_table.to(DEV), dec.context_lens.to(DEV),
                                     max_context_len=int(dec.context_lens.max()),
                                     scale=dec.scale, return_lse=True)
    return [o, lse, dq, dk, dv, out, dlse]


def test_threads_on_their_own_streams_match_serial_calls():
    probs = [_problem(s) for s in range(6)]
    ref = [_run(p) for p in probs]
    torch.cuda.synchronize()
    got = [None] * len(probs)
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(3):
                    got[i] = _run(probs[i])
            s.synchronize()
        except Exception as e:   # reported by the main thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(probs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i, (a, b) in enumerate(zip(ref, got)):
        for j, (x, y) in enumerate(zip(a, b)):
            assert torch.equal(x, y), "problem %d, output %d differs from the serial call" % (i, j)

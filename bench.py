"""Benchmark of the hot path on one MI355X.

One step = one causal prefill over the stress workload (batch 4, 16 heads,
N = 2048, d = 128, bf16, 1 % of Q/K rows x20), one long causal GQA prefill
(batch 1, 32 query / 8 KV heads, N = 16384, d = 128, bf16) and one paged
decode over 64 sequences (context lengths uniform in [512, 8192], 32 query /
8 KV heads, d = 128, bf16 KV cache in 16-token blocks, shuffled block table).
Inputs are synthetic (seeded) and resident in device memory before timing
starts.

Prints one JSON line:
  value          prefill TFLOP/s of the stress workload (algorithmic FLOP /
                 mean kernel time)
  roofline       that prefill kernel against the dense bf16 matrix-core peak
  long_prefill   the N = 16384 GQA prefill of the same step: TFLOP/s, its
                 roofline, and the oracle timed on sampled rows of it
  decode         decode GB/s (algorithmic K/V bytes / mean decode time, split +
                 combine kernels) and its roofline against HBM bandwidth
  achievable     what loops of the prefill's matrix op, of the exponential and
                 of random 4 KiB reads reach on this chip (libattn_probes.so);
                 each roofline also carries its fraction of these
  shared_decode  outside the step: the shared-prefix decode workload (8 groups
                 x 8 sequences, 4096-token common prefix, 256-token private
                 suffixes), per-sequence decode against sharing-aware decode,
                 warm (one pool, back-to-back calls) and cold (three pools
                 used in turn, 604 MB against the 256 MB last-level cache)
  backward       outside the step: attn_bwd on the prefill workload (its own
                 O and log-sum-exp, a seeded dO), TFLOP/s counted as 2.5x the
                 forward's algorithmic FLOP, against the bf16 peak
  paged_kv       outside the step: the prefill workload's K/V written into a
                 paged cache (shuffled blocks) with paged_kv_write (GB/s), and
                 the same prefill read back through the block table with
                 attn_fwd_paged (TFLOP/s, beside the contiguous attn_fwd)
  cpu_baseline   the fp64 CPU oracle timed on the host on a bounded sample
With --only long, the long causal GQA prefill alone, timed over back-to-back
calls, as {"long_prefill": ...}; --only probes runs the achievable-peak
probes alone.
Kernel times come from HIP events recorded on the stream the kernels run on;
the step's per-launch events skip the system-scope cache write-back that a
default event makes before its timestamp (LaunchEvent).

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --copy-calibration     # plain 1 GiB copies, for counters
    python bench.py --write-traffic FETCH WRITE COPY_FETCH COPY_WRITE [SFETCH SWRITE
                                    [BFETCH BWRITE]]
        # profiles/traffic.json from rocprofv3 --pmc output directories:
        # FETCH_SIZE and WRITE_SIZE of a --no-shared run, then of
        # --copy-calibration, then (optional) of an --only shared run and of
        # an --only backward run
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

METRIC = "prefill attention TFLOP/s (% MFMA peak) + paged decode GB/s (% HBM peak)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E bandwidth (published)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "exact_attention_34_amd", "csrc")


def source_hash():
    """Hash of the attention library's sources (the probes are not part of it)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name == "probes.hip":
            continue
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel):
    """HBM bytes per launch measured with counters, if the kernel is unchanged."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    ent = t.get(kernel)
    if not ent or ent.get("source_hash") != source_hash():
        return None
    return ent.get("bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-shared", action="store_true",
                    help="skip the shared-prefix decode measurement (for profiling)")
    ap.add_argument("--no-long", action="store_true",
                    help="leave the N=16384 prefill out of the step (for profiling)")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the achievable-peak probes")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode", "shared", "backward", "paged", "long",
                                       "probes"],
                    default=None,
                    help="run one kernel family only (for profiling)")
    ap.add_argument("--write-traffic", nargs="+", default=None, metavar="DIR")
    return ap.parse_args()


_FWD = "void attn::attn_fwd_mfma_kernel<attn::BF16, 128, true, false, 8>"
# entry name -> (kernel name prefix in rocprofv3 output, run, grid size in
# work-items or None).  The two prefills of the step are one kernel; their
# grids tell them apart: 512 workgroups of 512 threads (B=4, H=16, N=2048)
# and 2,048 of them (N=16384, 32 query heads).
TRAFFIC_KERNELS = {
    "attn_fwd_mfma_kernel": (_FWD, "main", 512 * 512),
    "attn_fwd_mfma_kernel_long": (_FWD, "main", 2048 * 512),
    "paged_decode_split_kernel": ("void attn::paged_decode_split_kernel<attn::BF16, 128, 4,",
                                  "main", None),
    "paged_decode_combine_kernel": ("void attn::paged_decode_combine_kernel<attn::BF16", "main",
                                    None),
    "paged_decode_prefix_kernel": ("void attn::paged_decode_prefix_kernel<attn::BF16, 128>",
                                   "shared", None),
    "attn_bwd_dkdv_kernel": ("void attn::attn_bwd_dkdv_kernel<attn::BF16, 128, true>", "backward",
                             None),
    "attn_bwd_dq_kernel": ("void attn::attn_bwd_dq_kernel<attn::BF16, 128, true>", "backward",
                           None),
}


def _counter_kib(directory, counter, prefix, grid=None):
    """Mean KiB per dispatch of `counter` over the kernels whose name starts
    with `prefix` (and, if given, whose grid has `grid` work-items), from
    rocprofv3 counter_collection.csv files."""
    import csv
    import glob
    vals = []
    for f in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter or not r["Kernel_Name"].startswith(prefix):
                    continue
                if grid is not None and int(float(r["Grid_Size"])) != grid:
                    continue
                vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit("no %s samples for %s in %s" % (counter, prefix, directory))
    return float(np.mean(vals)), len(vals)


def write_traffic(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, sfetch_dir=None,
                  swrite_dir=None, bfetch_dir=None, bwrite_dir=None):
    """HBM bytes per launch: counter KiB scaled by what the same counter reads
    for plain device copies of known size (bench.py --copy-calibration).
    Kernels of the shared-prefix decode come from the optional second pair
    of runs (bench.py --only shared)."""
    copy_bytes = 1 << 30
    cf, _ = _counter_kib(copy_fetch_dir, "FETCH_SIZE", "__amd_rocclr_copyBuffer")
    cw, _ = _counter_kib(copy_write_dir, "WRITE_SIZE", "__amd_rocclr_copyBuffer")
    ff, wf = copy_bytes / (cf * 1024.0), copy_bytes / (cw * 1024.0)
    out = {
        "_about": "HBM bytes per launch of each kernel on the benchmark workloads, from "
                  "rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE (KiB per dispatch) scaled by "
                  "the reading of the same counters for a plain 1 GiB device copy (fetch factor "
                  "%.4f, write factor %.4f). Valid only while the kernel sources hash to "
                  "source_hash." % (ff, wf),
        "fetch_factor": ff, "write_factor": wf,
    }
    for name, (prefix, run, grid) in TRAFFIC_KERNELS.items():
        fd, wd = {"main": (fetch_dir, write_dir), "shared": (sfetch_dir, swrite_dir),
                  "backward": (bfetch_dir, bwrite_dir)}[run]
        if fd is None:
            continue
        fk, n1 = _counter_kib(fd, "FETCH_SIZE", prefix, grid)
        wk, n2 = _counter_kib(wd, "WRITE_SIZE", prefix, grid)
        fb, wb = int(round(fk * 1024 * ff)), int(round(wk * 1024 * wf))
        out[name] = {"kernel_prefix": prefix, "grid_size": grid, "source_hash": source_hash(),
                     "fetch_kib_raw": fk, "write_kib_raw": wk, "dispatches": [n1, n2],
                     "fetch_bytes": fb, "write_bytes": wb, "bytes_per_launch": fb + wb}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


class LaunchEvent:
    """A HIP event recorded on torch's current stream (the stream the library
    launches on), created with hipEventDisableSystemFence.  A default event
    makes a system-scope release before it takes its timestamp, which writes
    the caches back after the kernel just timed: 1-2 us per launch that is
    not the kernel's and that rocprofv3's kernel time does not include.  The
    interface is torch.cuda.Event's record() / elapsed_time()."""

    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence

    @classmethod
    def runtime(cls):
        if cls._hip is None:
            import ctypes
            hip = ctypes.CDLL("libamdhip64.so.7")   # the HIP runtime torch has loaded
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = hip
        return cls._hip

    def __init__(self):
        import ctypes
        self._ct = ctypes
        self.ev = ctypes.c_void_p()
        rc = self.runtime().hipEventCreateWithFlags(ctypes.byref(self.ev), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError("hipEventCreateWithFlags failed (%d)" % rc)

    def record(self):
        rc = self.runtime().hipEventRecord(self.ev, torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError("hipEventRecord failed (%d)" % rc)

    def elapsed_time(self, other):
        """Milliseconds from this event to `other` (both completed)."""
        ms = self._ct.c_float()
        rc = self.runtime().hipEventElapsedTime(self._ct.byref(ms), self.ev, other.ev)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed (%d)" % rc)
        return ms.value

    def __del__(self):
        if self._hip is not None and self.ev:
            self._hip.hipEventDestroy(self.ev)


def copy_calibration():
    """Plain device copies of a known size (1 GiB), for scaling HBM counters."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    b = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    a.fill_(1)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 5}), flush=True)


def blas_info():
    """(threads, vendor) of the BLAS numpy uses, as threadpoolctl reports them."""
    try:
        from threadpoolctl import threadpool_info
        info = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        threads = max([p.get("num_threads", 1) for p in info] + [1])
        vendor = ", ".join("%s %s (%s)" % (p.get("internal_api"), p.get("version"),
                                            p.get("threading_layer", "?")) for p in info)
        return threads, vendor or "unknown"
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0)), "unknown"


def cpu_baseline(pre, dec, dec_bytes, pre_flops):
    """Time the fp64 oracle on a bounded sample of the same workloads."""
    import oracle
    threads, vendor = blas_info()
    q, k, v = (x.float().numpy() for x in (pre.q, pre.k, pre.v))
    # prefill sample: the whole stress workload (64 (batch, head) pairs)
    t0 = time.perf_counter()
    oracle.sdpa(q, k, v, pre.scale, True)
    t_pre = time.perf_counter() - t0
    flops_sample = pre_flops
    # decode sample: all 64 sequences
    ns = dec.q.shape[0]
    t0 = time.perf_counter()
    oracle.paged_decode(dec.q[:ns].double().numpy(), dec.k_cache.float().numpy(),
                        dec.v_cache.float().numpy(), dec.block_table[:ns].numpy(),
                        dec.context_lens[:ns].numpy(), dec.block_size, dec.scale)
    t_dec = time.perf_counter() - t0
    bytes_sample = int(dec.context_lens[:ns].to(torch.int64).sum()) * 8 * 128 * 2 * 2
    return {
        "value": flops_sample / t_pre / 1e12, "unit": "TFLOP/s", "cores": threads,
        "kind": "oracle", "blas": vendor,
        "sample": "one pass of each workload: prefill B=4 H=16 N=2048 causal (%.1f s), "
                  "decode of all 64 sequences (%.1f s)" % (t_pre, t_dec),
        "decode_value": bytes_sample / t_dec / 1e9, "decode_unit": "GB/s",
    }


def long_prefill_cpu_baseline(inp, n_rows=512, seed=33):
    """The oracle on sampled rows of the N = 16384 GQA prefill: n_rows
    (batch, row, head) triples, each attending to its whole visible key range
    (row i of a causal sequence sees i + 1 keys: 4 d (i + 1) FLOP)."""
    import oracle
    threads, vendor = blas_info()
    B, N, Hq, d = inp.q.shape
    rng = np.random.default_rng(seed)
    rows = np.stack([np.zeros(n_rows, dtype=np.int64), rng.integers(0, N, n_rows),
                     rng.integers(0, Hq, n_rows)], axis=1)
    q, k, v = (x.float().numpy() for x in (inp.q, inp.k, inp.v))
    t0 = time.perf_counter()
    oracle.sdpa_rows(q, k, v, rows, inp.scale, True)
    t = time.perf_counter() - t0
    flops = float(np.sum(4.0 * d * (rows[:, 1] + 1)))
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "blas": vendor,
            "sample": "%d random (row, head) outputs of the N=16384 causal GQA prefill, each "
                      "against its whole visible key range (%.2e FLOP, %.1f s)" % (n_rows, flops, t)}


def probe_lib():
    """libattn_probes.so with argument types declared (built beside libattn.so)."""
    import ctypes
    from exact_attention_34_amd import build as _b
    if not os.path.exists(_b.PROBE_LIB_PATH):
        raise RuntimeError("libattn_probes.so is not built; run python -m exact_attention_34_amd.build")
    L = ctypes.CDLL(_b.PROBE_LIB_PATH)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    L.attn_probe_mfma_bf16.argtypes = [vp, i32, i32, vp]
    L.attn_probe_exp2.argtypes = [vp, i32, i32, vp]
    L.attn_probe_random_read.argtypes = [vp, ctypes.c_size_t, vp, i32, vp, i32, vp]
    for f in (L.attn_probe_mfma_bf16, L.attn_probe_exp2, L.attn_probe_random_read):
        f.restype = i32
    return L


def achievable(dev, reps=10):
    """What simple loops reach on this chip: the prefill's matrix op
    (v_mfma_f32_32x32x16_bf16, independent chains, 4 waves per SIMD), the
    softmax's exponential (v_exp_f32 chains) and 4 KiB reads at random block
    ids (decode's access pattern: 2,048 waves, two blocks in flight each,
    non-temporal), each timed over `reps` launches with HIP events."""
    import ctypes
    L = probe_lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    def timed(fn):
        fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e-3

    def check(rc):
        if rc != 0:
            raise RuntimeError("probe launch failed: hip error %d" % rc)

    blocks, iters = 4096, 2000        # 4 waves per SIMD on 256 CUs
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    t = timed(lambda: check(L.attn_probe_mfma_bf16(ctypes.c_void_p(out.data_ptr()), blocks,
                                                     iters, stream)))
    mfma = blocks * 4 * iters * 8 * 32768 / t / 1e12
    t = timed(lambda: check(L.attn_probe_exp2(ctypes.c_void_p(out.data_ptr()), blocks, iters,
                                              stream)))
    exps = blocks * 256 * iters * 8 / t
    nbytes = 1 << 30                  # 1 GiB of 4 KiB blocks, read in a random order
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    ids = torch.randperm(nbytes // 4096, generator=torch.Generator().manual_seed(3)).to(
        torch.int32).to(dev)
    waves = 2048
    sink = torch.empty(waves * 64, dtype=torch.int32, device=dev)
    t = timed(lambda: check(L.attn_probe_random_read(
        ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(ids.data_ptr()), ids.numel(),
        ctypes.c_void_p(sink.data_ptr()), waves, stream)))
    rd = nbytes / t / 1e9
    del buf
    return {
        "mfma_bf16_TFLOPs": mfma, "exp2_per_s": exps, "random_4k_read_GBps": rd,
        "note": "libattn_probes.so loops on this chip: independent v_mfma_f32_32x32x16_bf16 "
                "chains (16,384 waves, varying operands); v_exp_f32 chains; 1 GiB read as "
                "4 KiB blocks in random order by 2,048 waves with non-temporal loads",
    }


def shared_decode(ea, workloads, dev, reps):
    """Per-sequence decode against sharing-aware decode on the shared-prefix
    workload, timed with HIP events on the current stream over `reps` calls:
    warm (the same pool, back-to-back calls) and cold (three pools of the same
    shape -- seeds 5, 105, 205 -- used in turn, 604 MB of K/V against the
    256 MB last-level cache, so a call finds little of its pool cached).
    GB/s are reported on the logical bytes (what a per-sequence kernel reads)
    and on the unique bytes (each shared block once)."""
    pools = []
    for seed in (5, 105, 205):
        inp = workloads.decode_config5(seed=seed, nan_fill=True)
        pools.append(dict(
            inp=inp, q=inp.q.to(dev), kc=inp.k_cache.to(dev), vc=inp.v_cache.to(dev),
            tab=inp.block_table.to(dev), ctx=inp.context_lens.to(dev),
            gs=inp.group_starts.to(dev), pl=inp.prefix_lens.to(dev)))
    inp = pools[0]["inp"]
    S, Hq, d = inp.q.shape
    Hkv = inp.k_cache.shape[1]
    G = inp.prefix_lens.shape[0]
    mcl = inp.max_context_len
    mgs = int(np.diff(inp.group_starts.numpy()).max())
    mpl = int(inp.prefix_lens.max())
    out = torch.empty_like(pools[0]["q"])
    ws_plain = torch.empty(ea.paged_attn_decode_workspace_size(S, Hq, Hkv, d, mcl),
                           dtype=torch.uint8, device=dev)
    ws_shared = torch.empty(ea.paged_attn_decode_shared_workspace_size(S, G, mgs, Hq, Hkv, d,
                                                                       mcl, mpl),
                            dtype=torch.uint8, device=dev)

    def plain(P):
        ea.paged_attn_decode(P["q"], P["kc"], P["vc"], P["tab"], P["ctx"], max_context_len=mcl,
                             scale=inp.scale, out=out, workspace=ws_plain)

    def shared(P):
        ea.paged_attn_decode_shared(P["q"], P["kc"], P["vc"], P["tab"], P["ctx"], P["gs"],
                                    P["pl"], max_context_len=mcl, max_group_size=mgs,
                                    max_prefix_len=mpl, scale=inp.scale, out=out,
                                    workspace=ws_shared)

    def timed(fn, rotate):
        for i in range(6):
            fn(pools[i % 3 if rotate else 0])
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for i in range(reps):
            fn(pools[i % 3 if rotate else 0])
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    warm_plain, warm_shared = timed(plain, False), timed(shared, False)
    cold_plain, cold_shared = timed(plain, True), timed(shared, True)
    logical = workloads.decode_bytes(inp.context_lens.numpy(), Hkv, d)
    unique = workloads.decode_unique_bytes(inp.block_table.numpy(), inp.context_lens.numpy(),
                                           inp.block_size, Hkv, d)

    def rates(t_plain, t_shared):
        return {"per_sequence_ms": t_plain, "shared_ms": t_shared, "speedup": t_plain / t_shared,
                "per_sequence_logical_GBps": logical / (t_plain * 1e-3) / 1e9,
                "shared_logical_GBps": logical / (t_shared * 1e-3) / 1e9,
                "shared_unique_GBps": unique / (t_shared * 1e-3) / 1e9,
                "shared_unique_frac_of_hbm": unique / (t_shared * 1e-3) / 1e9 / PEAK_HBM_GBS}

    return {
        "workload": "8 groups x 8 seqs, 4096-token shared prefix + 256-token private suffix, "
                    "Hq=32 Hkv=8 d=128 bf16 block 16 shuffled table",
        "logical_bytes": logical, "unique_bytes": unique,
        "cold": rates(cold_plain, cold_shared),
        "warm": rates(warm_plain, warm_shared),
        "note": "cold: three pools of this shape used in turn (each call's 201 MB of unique "
                "K/V was last read two calls, 402 MB, earlier); warm: one pool, back-to-back "
                "calls.  The per-sequence call streams K/V past the caches (non-temporal loads), "
                "so each sequence fetches the shared prefix again; the sharing-aware call reads "
                "each prefix block once, with ordinary loads",
        "prefix_kernel_traffic": load_traffic("paged_decode_prefix_kernel"),
    }


def backward(ea, pre, q, k, v, pre_flops, reps):
    """attn_bwd on the prefill workload, timed over `reps` back-to-back calls
    with HIP events on the current stream.  O and the log-sum-exp come from
    attn_fwd on the same inputs; dO is seeded N(0, 1) rounded to bf16."""
    o, lse = ea.attn_fwd(q, k, v, causal=True, scale=pre.scale, return_lse=True)
    g = torch.Generator().manual_seed(7)
    do = torch.randn(q.shape, generator=g, dtype=torch.float64).to(q.dtype).to(q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    B, N, Hq, _ = q.shape
    ws = torch.empty(max(1, ea.attn_bwd_workspace_size(B, N, Hq)), dtype=torch.uint8,
                     device=q.device)

    def run():
        ea.attn_bwd(q, k, v, o, do, lse, causal=True, scale=pre.scale, dq=dq, dk=dk, dv=dv,
                    workspace=ws)

    for _ in range(3):
        run()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        run()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    flops = 2.5 * pre_flops
    tf = flops / (ms * 1e-3) / 1e12
    return {
        "workload": "backward of the causal prefill B=4 Hq=Hkv=16 N=2048 d=128 bf16 "
                    "(1% Q/K rows x20)",
        "mean_ms": ms, "value": tf, "unit": "TFLOP/s",
        "flop_per_call": flops,
        "flop_convention": "2.5 x forward algorithmic FLOP (dV, dP, dQ, dK and the recomputed S); "
                           "the kernels execute 3.5 x (dP and S are recomputed for dQ)",
        "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": tf / PEAK_BF16_TFLOPS,
                     "traffic": {"dkdv": load_traffic("attn_bwd_dkdv_kernel"),
                                 "dq": load_traffic("attn_bwd_dq_kernel")},
                     "kernel": "attn_bwd_delta_kernel + attn_bwd_dkdv_kernel + "
                               "attn_bwd_dq_kernel <bf16,128,causal>"},
    }


def long_prefill(ea, workloads, dev, reps):
    """The long causal GQA prefill (B=1, 32 query / 8 KV heads, N=16384,
    d=128, bf16), timed over `reps` back-to-back calls with HIP events on the
    current stream."""
    inp = workloads.prefill_config(3)
    q, k, v = (x.to(dev) for x in (inp.q, inp.k, inp.v))
    o = torch.empty_like(q)
    B, N, Hq, d = q.shape
    flops = workloads.prefill_flops(B, N, N, Hq, d, True)

    def run():
        ea.attn_fwd(q, k, v, causal=True, scale=inp.scale, out=o)

    for _ in range(2):
        run()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        run()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    tf = flops / (ms * 1e-3) / 1e12
    return {
        "workload": "causal prefill B=1 Hq=32 Hkv=8 N=16384 d=128 bf16",
        "mean_ms": ms, "value": tf, "unit": "TFLOP/s", "flop_per_call": flops,
        "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": tf / PEAK_BF16_TFLOPS,
                     "kernel": "attn_fwd_mfma_kernel<bf16,128,causal>"},
        "note": "back-to-back calls",
    }


def paged_kv(ea, pre, q, k, v, pre_flops, reps):
    """paged_kv_write of the prefill workload's K and V into a shuffled paged
    cache, then attn_fwd_paged over it; each timed over `reps` back-to-back
    calls with HIP events on the current stream."""
    B, N, Hq, d = q.shape
    Hkv, bs = k.shape[2], 16
    per_seq = (N + bs - 1) // bs
    nb = B * per_seq
    g = torch.Generator().manual_seed(11)
    perm = torch.randperm(nb, generator=g).to(torch.int32)
    table = perm.view(B, per_seq).to(q.device)
    t = torch.arange(N, dtype=torch.int32)
    slots = (perm.view(B, per_seq)[:, t // bs] * bs + t % bs).reshape(-1).to(q.device)
    kc = torch.empty((nb, Hkv, bs, d), dtype=q.dtype, device=q.device)
    vc = torch.empty_like(kc)
    kf, vf = k.reshape(B * N, Hkv, d), v.reshape(B * N, Hkv, d)
    ctx = torch.full((B,), N, dtype=torch.int32, device=q.device)
    out = torch.empty_like(q)

    def timed(fn):
        for _ in range(3):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    t_write = timed(lambda: ea.paged_kv_write(kf, vf, slots, kc, vc))
    t_paged = timed(lambda: ea.attn_fwd_paged(q, kc, vc, table, ctx, max_context_len=N,
                                              causal=True, scale=pre.scale, out=out))
    t_flat = timed(lambda: ea.attn_fwd(q, k, v, causal=True, scale=pre.scale, out=out))
    moved = 2 * 2 * kf.numel() * kf.element_size()   # K and V, read once and written once
    return {
        "workload": "prefill workload's K/V (B=4 x 2048 tokens, 16 KV heads, d=128, bf16) in "
                    "%d shuffled 16-token blocks" % nb,
        "kv_write_ms": t_write, "kv_write_GBps": moved / (t_write * 1e-3) / 1e9,
        "kv_write_frac_of_hbm": moved / (t_write * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "paged_prefill_ms": t_paged,
        "paged_prefill_TFLOPs": pre_flops / (t_paged * 1e-3) / 1e12,
        "contiguous_prefill_ms": t_flat,
        "contiguous_prefill_TFLOPs": pre_flops / (t_flat * 1e-3) / 1e12,
        "note": "back-to-back calls on warm caches",
    }


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.write_traffic:
        if len(args.write_traffic) not in (4, 6, 8):
            raise SystemExit("--write-traffic takes 4, 6 or 8 directories")
        write_traffic(*args.write_traffic)
        return
    import exact_attention_34_amd as ea
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pre = workloads.prefill_config(2)
    B, N, Hq, d = pre.q.shape
    pre_flops = workloads.prefill_flops(B, N, N, Hq, d, True)
    q, k, v = (x.to(dev) for x in (pre.q, pre.k, pre.v))
    o = torch.empty_like(q)
    if args.only == "long":
        print(json.dumps({"long_prefill": long_prefill(ea, workloads, dev, args.steps)}),
              flush=True)
        return
    if args.only == "shared":
        print(json.dumps({"shared_decode": shared_decode(ea, workloads, dev, args.steps)}),
              flush=True)
        return
    if args.only == "backward":
        print(json.dumps({"backward": backward(ea, pre, q, k, v, pre_flops, args.steps)}),
              flush=True)
        return
    if args.only == "paged":
        print(json.dumps({"paged_kv": paged_kv(ea, pre, q, k, v, pre_flops, args.steps)}),
              flush=True)
        return

    if args.only == "probes":
        print(json.dumps({"achievable": achievable(dev)}), flush=True)
        return

    dec = workloads.decode_config4(nan_fill=True)
    dq = dec.q.to(dev)
    kc, vc = dec.k_cache.to(dev), dec.v_cache.to(dev)
    tab, ctx = dec.block_table.to(dev), dec.context_lens.to(dev)
    mcl = 8192
    dout = torch.empty_like(dq)
    ws = torch.empty(max(1, ea.paged_attn_decode_workspace_size(dq.shape[0], dq.shape[1],
                                                                kc.shape[1], 128, mcl)),
                     dtype=torch.uint8, device=dev)
    dec_bytes = workloads.decode_bytes(dec.context_lens.numpy(), 8, 128)

    run_pre = args.only in (None, "prefill")
    run_long = args.only is None and not args.no_long
    run_dec = args.only in (None, "decode")
    if run_long:
        lpre = workloads.prefill_config(3)
        lq, lk, lv = (x.to(dev) for x in (lpre.q, lpre.k, lpre.v))
        lo = torch.empty_like(lq)
        LB, LN, LHq, Ld = lq.shape
        long_flops = workloads.prefill_flops(LB, LN, LN, LHq, Ld, True)

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        if run_pre:
            mark(0)
            ea.attn_fwd(q, k, v, causal=True, scale=pre.scale, out=o)
            mark(1)
        if run_long:
            mark(2)
            ea.attn_fwd(lq, lk, lv, causal=True, scale=lpre.scale, out=lo)
            mark(3)
        if run_dec:
            mark(4)
            ea.paged_attn_decode(dq, kc, vc, tab, ctx, max_context_len=mcl, scale=dec.scale,
                                 out=dout, workspace=ws)
            mark(5)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[LaunchEvent() for _ in range(6)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step(events[i])
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)

    def mean_ms(a, b):
        return float(np.mean([e[a].elapsed_time(e[b]) for e in events]))

    pre_ms = mean_ms(0, 1) if run_pre else None
    long_ms = mean_ms(2, 3) if run_long else None
    dec_ms = mean_ms(4, 5) if run_dec else None

    res = {
        "metric": METRIC,
        "value": None, "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": total_ms / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {
            "workload": "causal prefill B=4 Hq=Hkv=16 N=2048 d=128 bf16 (1% Q/K rows x20) "
                        "+ causal GQA prefill B=1 Hq=32 Hkv=8 N=16384 d=128 bf16 "
                        "+ paged decode 64 seqs ctx~U[512,8192] Hq=32 Hkv=8 d=128 bf16 "
                        "block 16 shuffled table",
            "global_batch": B, "seq_len": N, "parallelism": "none (1 GPU)",
        },
    }
    ach = None
    if args.only is None and not args.no_probes:
        ach = achievable(dev)
        res["achievable"] = ach
    if run_pre:
        tflops = pre_flops / (pre_ms * 1e-3) / 1e12
        traffic = load_traffic("attn_fwd_mfma_kernel")
        res["value"] = tflops
        res["roofline"] = {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": tflops / PEAK_BF16_TFLOPS,
                           "traffic": traffic, "kernel": "attn_fwd_mfma_kernel<bf16,128,causal>",
                           "workload": "causal prefill B=4 Hq=Hkv=16 N=2048 d=128 bf16",
                           "flop_per_launch": pre_flops, "mean_ms": pre_ms}
        if ach:
            res["roofline"]["frac_of_achievable"] = tflops / ach["mfma_bf16_TFLOPs"]
    if run_long:
        ltf = long_flops / (long_ms * 1e-3) / 1e12
        res["long_prefill"] = {
            "workload": "causal GQA prefill B=1 Hq=32 Hkv=8 N=16384 d=128 bf16",
            "value": ltf, "unit": "TFLOP/s", "mean_ms": long_ms, "flop_per_launch": long_flops,
            "roofline": {"bound": "mfma", "achieved": ltf, "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": ltf / PEAK_BF16_TFLOPS,
                         "traffic": load_traffic("attn_fwd_mfma_kernel_long"),
                         "kernel": "attn_fwd_mfma_kernel<bf16,128,causal>"},
        }
        if ach:
            res["long_prefill"]["roofline"]["frac_of_achievable"] = ltf / ach["mfma_bf16_TFLOPs"]
    if run_dec:
        gbs = dec_bytes / (dec_ms * 1e-3) / 1e9
        res["decode"] = {
            "value": gbs, "unit": "GB/s", "mean_ms": dec_ms,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS,
                         "traffic": load_traffic("paged_decode_split_kernel"),
                         "kernel": "paged_decode_split_kernel + paged_decode_combine_kernel",
                         "bytes_per_launch": dec_bytes},
        }
        if ach:
            res["decode"]["roofline"]["frac_of_achievable"] = gbs / ach["random_4k_read_GBps"]
    if args.only is None and not args.no_shared:
        res["shared_decode"] = shared_decode(ea, workloads, dev, args.steps)
        res["backward"] = backward(ea, pre, q, k, v, pre_flops, args.steps)
        res["paged_kv"] = paged_kv(ea, pre, q, k, v, pre_flops, args.steps)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(pre, dec, dec_bytes, pre_flops)
        if run_long:
            res["long_prefill"]["cpu_baseline"] = long_prefill_cpu_baseline(lpre)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

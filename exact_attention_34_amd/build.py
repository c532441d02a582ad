"""Build the C-ABI libraries in-tree with hipcc for gfx950.

    python -m exact_attention_34_amd.build

compiles ``csrc/`` into
  * ``exact_attention_34_amd/libattn.so``: the attention library (the kernels
    and the C ABI of ``include/attn.h``);
  * ``exact_attention_34_amd/libattn_probes.so``: the achievable-peak probes
    that the benchmark divides by (measurement code only).
Each source is compiled to an object in parallel, then each library is
linked.  The libraries link only the HIP runtime.  Packed-fp32 instructions
are disabled (``-Xclang -target-feature -Xclang -packed-fp32-ops``); no
fast-math flags are used, so IEEE infinities and NaNs behave as written.
"""

import concurrent.futures
import os
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libattn.so")
PROBE_LIB_PATH = os.path.join(PKG_DIR, "libattn_probes.so")
SOURCES = ["attn_api.hip", "prefill.hip", "decode.hip", "backward.hip", "kv_cache.hip",
           "scratch.hip", "block_manager.cpp", "validate.cpp"]
PROBE_SOURCES = ["probes.hip"]
ARCH = "gfx950"
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def compile_command(src, obj):
    return [hipcc()] + FLAGS + ["-c", "-o", obj, os.path.join(CSRC, src)]


def link_command(objs, out_path):
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out_path] + objs


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in ln]
    return res.returncode, msgs


def build(verbose=False, jobs=None):
    """Compile both libraries; returns the attention library's path.  Raises
    on a compiler or linker error."""
    jobs = jobs or min(8, len(os.sched_getaffinity(0)))
    with tempfile.TemporaryDirectory(prefix="attn_build_") as td:
        srcs = SOURCES + PROBE_SOURCES
        objs = {s: os.path.join(td, s + ".o") for s in srcs}
        cmds = {s: compile_command(s, objs[s]) for s in srcs}
        if verbose:
            for s in srcs:
                print(" ".join(cmds[s]), flush=True)
        with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
            results = dict(zip(srcs, ex.map(_run, [cmds[s] for s in srcs])))
        for s in srcs:
            rc, msgs = results[s]
            if rc != 0:
                raise RuntimeError("hipcc failed on %s (%d):\n%s" % (s, rc, "\n".join(msgs)))
            if verbose and msgs:
                print("\n".join(msgs))
        for path, group in ((LIB_PATH, SOURCES), (PROBE_LIB_PATH, PROBE_SOURCES)):
            tmp = path + ".tmp%d" % os.getpid()
            cmd = link_command([objs[s] for s in group], tmp)
            if verbose:
                print(" ".join(cmd), flush=True)
            rc, msgs = _run(cmd)
            if rc != 0:
                if os.path.exists(tmp):
                    os.remove(tmp)
                raise RuntimeError("link of %s failed (%d):\n%s"
                                   % (os.path.basename(path), rc, "\n".join(msgs)))
            os.replace(tmp, path)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

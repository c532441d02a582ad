"""Build libattn.so (the C-ABI library) in-tree with hipcc for gfx950.

    python -m exact_attention_34_amd.build

compiles ``csrc/*.hip`` into ``exact_attention_34_amd/libattn.so``.  The
library links only the HIP runtime.  Packed-fp32 instructions are disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); no fast-math flags
are used, so IEEE infinities and NaNs behave as written.
"""

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libattn.so")
SOURCES = ["attn_api.hip", "prefill.hip", "decode.hip", "backward.hip", "kv_cache.hip",
           "block_manager.cpp", "validate.cpp"]
ARCH = "gfx950"


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def compile_command(out_path):
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-o", out_path] + [os.path.join(CSRC, s) for s in SOURCES]


def build(verbose=False):
    """Compile the library; returns its path.  Raises on a compiler error."""
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = compile_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so
    noise = "packed-fp32-ops"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, "\n".join(msgs)))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

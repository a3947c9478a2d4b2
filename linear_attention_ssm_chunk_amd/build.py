"""Build libgdn_prefill.so in-tree with hipcc for gfx950.

    python -m linear_attention_ssm_chunk_amd.build            # the library
    python -m linear_attention_ssm_chunk_amd.build --stamps   # and its section-stamp profiling build

The profiling build (libgdn_prefill_stamps.so, -DGDN_SECTION_STAMPS) is the same
sources with clock stamps at the spine's section marks, plus the streaming
kernel of stream_mix.hip; bench.py --section-stamps and --stream-ceiling load
it.  Nothing else loads it.

Every HIP source is compiled with packed FP32 math disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); the host pass warns
that it does not know the feature, which is harmless.  MFMA results are kept
in ordinary vector registers (``-amdgpu-mfma-vgpr-form``), which spares the
UT solve a register move per accumulator element it reads back.
"""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgdn_prefill.so")
LIB_STAMPS = os.path.join(PKG, "libgdn_prefill_stamps.so")
SOURCES = ["gdn_api.hip", "k1_chunk_cumsum_recompute_wu.hip", "k2_chunk_delta_h_fwd_o.hip",
           "k3_recurrent_decode.hip"]
ARCH = "gfx950"

FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose=False, stamps=False):
    """Compile every kernel and the C ABI into one shared library (with
    ``stamps``: the section-stamp profiling build)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    lib = LIB_STAMPS if stamps else LIB
    tmp = lib + ".tmp"
    if stamps:  # the measurement-only streaming kernel rides along in the profiling build
        srcs.append(os.path.join(CSRC, "stream_mix.hip"))
    cmd = [hipcc()] + FLAGS + (["-DGDN_SECTION_STAMPS"] if stamps else []) + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
    if "--stamps" in sys.argv[1:]:
        print(build(verbose=True, stamps=True))

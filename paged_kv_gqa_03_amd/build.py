"""Build libpaged_attn.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m paged_kv_gqa_03_amd.build [--resource-usage]

Every HIP translation unit is compiled to an object under _build/ (in
parallel) and linked into paged_kv_gqa_03_amd/libpaged_attn.so.  Device code
is compiled without packed-fp32 instructions (-packed-fp32-ops).
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpaged_attn.so")
SOURCES = ["api.hip", "decode.hip", "decode_mfma.hip", "prefill.hip", "swa.hip", "cache_ops.hip", "probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "-Wall", "-Wno-unused-function"]


# Per-source flags.  prefill.hip runs with the IEEE mode bit off (its
# arithmetic never produces or consumes NaN: masked scores are -inf and every
# -inf - -inf case is guarded), which lets fmax use MFMA results directly
# instead of quieting each input first.
SOURCE_FLAGS = {"prefill.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans"]}


def _compile(src, extra):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + SOURCE_FLAGS.get(src, []) + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    return src, obj, r


def build(resource_usage=False, verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(lambda s: _compile(s, extra), srcs))
    objs = []
    for src, obj, r in results:
        noise = [l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l]
        if verbose and noise:
            print("\n".join(noise), file=sys.stderr)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed on %s (exit %d)" % (src, r.returncode))
        objs.append(obj)
    tmp = LIB + ".tmp"
    subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH] + objs + ["-o", tmp], check=True)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB, flush=True)
    return LIB


if __name__ == "__main__":
    build(resource_usage="--resource-usage" in sys.argv)

"""Build ``libpkv.so`` (the HIP library behind include/pkv.h) in-tree for gfx950.

    python -m paged_kv_cache_259_amd.build          # or: python paged_kv_cache_259_amd/build.py

Each ``csrc/*.hip`` is compiled to an object in parallel under ``_build/``, then
linked into ``paged_kv_cache_259_amd/libpkv.so``.  Flags:
* ``--offload-arch=gfx950``, ``-O3``, no fast-math;
* ``-fhip-fp32-correctly-rounded-divide-sqrt``: the FP8 encode divides by the
  scale in IEEE single precision;
* ``-Xclang -target-feature -Xclang -packed-fp32-ops``: no packed-fp32
  (v_pk_*_f32) instructions are generated.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpkv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]

# Per-file code generation options.  The prefill kernel rescales its MFMA
# accumulators only on some steps; kept in AGPRs, the compiler copies all of
# them to VGPRs on every step to serve that branch, so its MFMAs use VGPRs.
FILE_FLAGS = {
    "prefill_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def _compile(src, extra=()):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), f"-I{os.path.dirname(src)}", *extra,
           "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    return obj, msgs


def build(verbose=True, defines=(), out=None, build_dir=None, csrc=None):
    """Compile and link; ``defines`` are extra -D flags (tuning constants), ``out`` the .so path,
    ``csrc`` another source directory with the same files (default: the package's csrc/)."""
    global BUILD
    lib = out or LIB
    src_dir = csrc or CSRC
    BUILD = build_dir or os.path.join(PKG, "_build")
    os.makedirs(BUILD, exist_ok=True)
    extra = [f"-D{d}" for d in defines]
    srcs = sorted(os.path.join(src_dir, f) for f in os.listdir(src_dir) if f.endswith(".hip"))
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(lambda f: _compile(f, extra), srcs))
    for obj, msgs in results:
        if msgs.strip() and verbose:
            print(msgs)
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *[o for o, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build()
    sys.exit(0)

"""Build ``libpkv.so`` (the HIP library behind include/pkv.h) in-tree for gfx950.

    python -m paged_kv_cache_259_amd.build          # or: python paged_kv_cache_259_amd/build.py

Each ``csrc/*.hip`` is compiled to an object in parallel under ``_build/``, then
linked into ``paged_kv_cache_259_amd/libpkv.so``.  The benchmark's HBM read
probes (``probe/*.hip``, include/pkv_probe.h) go into a library of their own,
``paged_kv_cache_259_amd/libpkv_probe.so``, so the paged-KV library holds only
the path.  Flags:
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
PROBE_SRC = os.path.join(PKG, "probe")
PROBE_LIB = os.path.join(PKG, "libpkv_probe.so")
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


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)


def build(verbose=True, defines=(), out=None, build_dir=None, csrc=None, probe=True):
    """Compile and link; ``defines`` are extra -D flags (tuning constants), ``out`` the .so path,
    ``csrc`` another source directory with the same files (default: the package's csrc/);
    ``probe`` also builds libpkv_probe.so (the default build does)."""
    global BUILD
    lib = out or LIB
    src_dir = csrc or CSRC
    BUILD = build_dir or os.path.join(PKG, "_build")
    os.makedirs(BUILD, exist_ok=True)
    extra = [f"-D{d}" for d in defines]
    srcs = sorted(os.path.join(src_dir, f) for f in os.listdir(src_dir) if f.endswith(".hip"))
    if probe:
        srcs += sorted(os.path.join(PROBE_SRC, f) for f in os.listdir(PROBE_SRC) if f.endswith(".hip"))
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(lambda f: _compile(f, extra), srcs))
    for obj, msgs in results:
        if msgs.strip() and verbose:
            print(msgs)
    objs = [o for o, _ in results]
    probe_objs = [o for o in objs if os.path.basename(o)[:-2] in os.listdir(PROBE_SRC)] if probe else []
    _link([o for o in objs if o not in probe_objs], lib)
    if verbose:
        print(f"built {lib}")
    if probe_objs:
        _link(probe_objs, PROBE_LIB)
        if verbose:
            print(f"built {PROBE_LIB}")
    return lib


if __name__ == "__main__":
    build()
    sys.exit(0)

"""Build libred.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m reduction_libred_amd.build      # or: python reduction_libred_amd/build.py

Every translation unit is compiled with hipcc for gfx950 only, with packed
FP32 instructions disabled, then linked into reduction_libred_amd/libred.so,
which exports only the red_* symbols declared in include/*.h.
"""
import concurrent.futures as cf
import hashlib
import json
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libred.so")
# sha256 of each compiled object, written beside the library: it identifies
# the machine code a measurement was taken on. hipcc would otherwise stamp a
# random compilation-unit id (__hip_cuid_*) into every object; -cuid=<name>
# fixes it per unit (unique, so the units still link together), so two
# builds of the same sources give byte-identical objects (checked in
# tests/test_build_repro.py), and an edit that leaves a unit's code unchanged
# leaves its hash unchanged.
MANIFEST = os.path.join(HERE, "libred_objects.json")

SOURCES = ["libred.cpp", "flat_sum_f32.hip", "flat_ops.hip", "flat_fused.hip", "flat_argmax.hip", "flat_argmin.hip",
           "flat_wide.hip", "rows_sum.hip", "rows_max.hip", "cols_reduce.hip", "ablate.hip", "probe.hip", "read_probe.hip", "rows_narrow.hip"]
ARCH = "gfx950"


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else shutil.which("hipcc") or "hipcc"


COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # Packed FP32 instructions stay off for all device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def compile_unit(src, obj):
    """Compile csrc/<src> with the library's flags into object file `obj`."""
    # A fixed compilation-unit id per unit instead of a random one: the
    # objects are reproducible.
    cuid = "libred_" + os.path.splitext(src)[0]
    cmd = [hipcc(), *COMMON, f"-cuid={cuid}", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def _compile(src):
    return compile_unit(src, os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o"))


def build(verbose=True):
    """Compile every source and link libred.so; return its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp,
           f"-Wl,--version-script={os.path.join(CSRC, 'libred.map')}", "-Wl,-soname,libred.so"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    digests = {}
    for src, obj in zip(SOURCES, objs):
        with open(obj, "rb") as fh:
            digests[src] = hashlib.sha256(fh.read()).hexdigest()
    with open(MANIFEST, "w") as fh:
        json.dump(digests, fh, indent=1, sort_keys=True)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()

"""Build libkda.so (all HIP sources, gfx950) in-tree with hipcc."""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libkda.so")
OBJ_DIR = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU instructions stay off: the compiler must not form them
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]

# Extra flags of single sources (none at present; MFMA accumulators in ordinary VGPRs for the
# walk kernel, -mllvm -amdgpu-mfma-vgpr-form, measured 5% slower than the compiler's choice).
FILE_FLAGS = {}


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{err}")
    if verbose and err.strip():
        print(err)


def build(verbose=False, extra=()):
    """Compile every source to an object (with its own extra flags), then link the library."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    jobs = []
    for src in sources():
        name = os.path.basename(src)
        obj = os.path.join(OBJ_DIR, name + ".o")
        jobs.append(([HIPCC, *FLAGS, *FILE_FLAGS.get(name, []), *extra, "-I",
                      os.path.join(ROOT, "include"), "-c", src, "-o", obj], obj))
    # the sources compile independently: one hipcc per source, a few at a time
    workers = max(1, min(len(jobs), 8, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(workers) as pool:
        for f in [pool.submit(_run, cmd, verbose) for cmd, _ in jobs]:
            f.result()
    objs = [obj for _, obj in jobs]
    _run([HIPCC, "--offload-arch=gfx950", "-fPIC", "-shared", *objs, "-o", LIB + ".tmp"], verbose)
    _check_defined(LIB + ".tmp")
    os.replace(LIB + ".tmp", LIB)
    return LIB


def _check_defined(lib):
    """Refuse a library that leaves any of its own symbols undefined: a source whose host
    pass failed to emit its kernels' launch stubs still compiles to an object (hipcc exits
    0), and a shared library links with the holes."""
    res = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"nm failed on {lib}:\n{res.stderr}")
    missing = [l.split()[-1] for l in res.stdout.splitlines()
               if "kda" in l or "device_stub" in l]
    if missing:
        os.remove(lib)
        raise RuntimeError("libkda.so would leave its own symbols undefined: " +
                           ", ".join(missing[:8]))


if __name__ == "__main__":
    build(verbose=True)

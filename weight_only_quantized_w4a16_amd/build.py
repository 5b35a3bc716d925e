"""Build the HIP library libwq.so for gfx950 with hipcc (in-tree)."""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libwq.so")
# measurement probe (streaming read), a library of its own outside the product ABI
PROBE_LIB = os.path.join(HERE, "libwq_probe.so")
# (source, object name, extra defines): the kernel files are compiled once
# per (activation dtype, code width) so the instantiations build in parallel.
SOURCES = [("wq_api.hip", "wq_api", []), ("wq_hadamard.hip", "wq_hadamard", [])]
for _k in ("wq_gemv", "wq_gemm"):
    for _dt, _dn in ((0, "f16"), (1, "bf16")):
        for _b in (2, 3, 4):
            SOURCES.append((_k + ".hip", f"{_k}_{_dn}_b{_b}", [f"-DWQ_DT={_dt}", f"-DWQ_BITS={_b}"]))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(os.path.dirname(HERE), "include")]


def _compile(item, verbose):
    src, name, defs = item
    obj = os.path.join(BUILD, name + ".o")
    cmd = [HIPCC, *FLAGS, *defs, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is expected
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip() and verbose:
        print(err, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", str(os.cpu_count() or 8))), 16)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    _link(objs, LIB, verbose)
    _link([_compile(("wq_probe.hip", "wq_probe", []), verbose)], PROBE_LIB, verbose)
    return LIB


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

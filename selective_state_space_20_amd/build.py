"""Build libsss.so (gfx950) in-tree with hipcc.  No JIT, no torch extension machinery.

Every source is compiled to an object in parallel (the selective scan once per state
count, see the explicit instances at the end of csrc/selective_scan.hip), then the objects
are linked into the shared library.  Objects live in _build/ at the repository root.
"""
from __future__ import annotations

import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsss.so")
# roofline calibration kernels (bench.py --probes only): a library of their own, so that
# libsss.so exports exactly the C ABI of include/sss.h
PROBE_SRC = os.path.join(CSRC, "probes", "roofline_probes.hip")
PROBE_LIB = os.path.join(PKG, "libsss_probes.so")
ARCH = "gfx950"
STATE_COUNTS = (1, 2, 4, 8, 16, 32, 64)

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU forms are kept out of the generated code on purpose
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]
NOISE = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.cpp")))


def compile_jobs():
    """(object path, extra flags, source) for every translation unit."""
    jobs = []
    for src in sources():
        stem = os.path.splitext(os.path.basename(src))[0]
        if stem == "selective_scan":
            jobs.append((os.path.join(OBJ, f"{stem}_host.o"), [], src))
            for n in STATE_COUNTS:
                jobs.append((os.path.join(OBJ, f"{stem}_n{n}.o"), [f"-DSSS_INST_NS={n}"], src))
        else:
            jobs.append((os.path.join(OBJ, f"{stem}.o"), [], src))
    return jobs


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if NOISE not in l)
    return r.returncode, msg


def build(verbose: bool = False, jobs: int = 0) -> str:
    os.makedirs(OBJ, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    work = compile_jobs()
    cmds = [["hipcc", *FLAGS, *extra, *inc, "-c", src, "-o", obj] for obj, extra, src in work]
    workers = jobs or max(1, min(len(cmds), os.cpu_count() or 1, 16))
    probe_cmd = ["hipcc", *FLAGS, "-shared", PROBE_SRC, "-o", PROBE_LIB + ".tmp"]
    with ThreadPoolExecutor(max_workers=workers) as ex:
        probe_job = ex.submit(_run, probe_cmd)
        results = list(ex.map(_run, cmds))
        results.append(probe_job.result())
    cmds.append(probe_cmd)
    for cmd, (rc, msg) in zip(cmds, results):
        if verbose:
            print(" ".join(cmd))
        if rc != 0:
            raise RuntimeError(f"hipcc failed ({rc}): {' '.join(cmd)}\n{msg}")
        if msg.strip() and verbose:
            print(msg)
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    tmp = LIB + ".tmp"
    rc, msg = _run(["hipcc", "-shared", "-fPIC", f"--offload-arch={ARCH}", *[obj for obj, _, _ in work], "-o", tmp])
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{msg}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=False))

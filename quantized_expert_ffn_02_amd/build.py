"""Build libmoe.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m quantized_expert_ffn_02_amd.build

Objects go to ``_build/`` at the repository root; the shared library is written
next to this file so that it travels with the source tree.
"""
import concurrent.futures
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep hipcc from emitting packed fp32 VALU instructions (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src):
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [_hipcc()] + FLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless
    noise = [ln for ln in (r.stderr or "").splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(noise))
    return obj, noise


# Host (CPU) sources, built with the host compiler.  host_ffn.cpp is built once per
# instruction set; the library picks one at run time.
HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-psabi", "-I", os.path.join(ROOT, "include")]
HOST_ISAS = {
    "avx512": ["-mavx512f", "-mavx512bw", "-mavx512vl", "-mavx512dq", "-mavx2", "-mfma", "-mf16c"],
    "avx2": ["-mavx2", "-mfma", "-mf16c"],
}


def _cxx():
    return os.environ.get("CXX") or "g++"


def _compile_host(job):
    src, isa = job
    tag = os.path.basename(src) + (f".{isa}" if isa else "")
    obj = os.path.join(OBJ, tag + ".o")
    cmd = [_cxx()] + HOST_FLAGS + ["-pthread", "-c", src, "-o", obj]
    if isa:
        cmd[1:1] = HOST_ISAS[isa] + [f"-DMOE_HOST_ISA_NS={isa}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = [ln for ln in (r.stderr or "").splitlines() if ln.strip()]
    if r.returncode != 0:
        raise RuntimeError(f"{_cxx()} failed on {src}:\n" + "\n".join(noise))
    return obj, noise


def _host_jobs():
    jobs = []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.cpp"))):
        if os.path.basename(src) == "host_ffn.cpp":
            jobs += [(src, isa) for isa in HOST_ISAS]
        else:
            jobs.append((src, None))
    return jobs


def build(verbose=False):
    os.makedirs(OBJ, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        hosts = ex.map(_compile_host, _host_jobs())
        results = list(ex.map(_compile, srcs)) + list(hosts)
    objs = []
    for obj, noise in results:
        objs.append(obj)
        if verbose and noise:
            print("\n".join(noise), file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

"""Build libfd.so (the C-ABI HIP library) in-tree with hipcc for gfx950."""
import concurrent.futures
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfd.so")
SOURCES = ["fd_kernels.hip", "fd_wide.hip", "fd_direct.hip", "fd_append.hip", "fd_check.hip", "fd_api.cpp"]
ARCH = "gfx950"

# -Xclang -target-feature -Xclang -packed-fp32-ops: keep the compiler from emitting packed
# fp32 VALU ops (v_pk_fma_f32 and friends) in device code.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-munsafe-fp-atomics",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return path


def build(verbose: bool = False) -> str:
    """Compile every source and link libfd.so (always recompiles)."""
    out_dir = os.path.join(PKG, "_build")
    os.makedirs(out_dir, exist_ok=True)
    cmds, objs = [], []
    for src in SOURCES:
        obj = os.path.join(out_dir, src + ".o")
        cmd = [hipcc(), *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        if verbose:
            print(" ".join(cmd), flush=True)
        cmds.append(cmd)
        objs.append(obj)
    # the sources compile independently: one process each, at most one per host core
    workers = max(1, min(len(cmds), os.cpu_count() or 1, 16))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        for r in ex.map(lambda c: subprocess.run(c, stderr=None if verbose else subprocess.PIPE), cmds):
            if r.returncode != 0:
                if r.stderr:
                    print(r.stderr.decode(errors="replace"), flush=True)
                raise subprocess.CalledProcessError(r.returncode, r.args)
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

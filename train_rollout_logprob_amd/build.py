"""Compile the HIP sources into the in-tree shared library ``libdrift.so`` (gfx950), and the
measurement-only read kernel into ``libdrift_ceiling.so``."""
from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdrift.so")
BUILD_DIR = os.path.join(PKG, "_build")
SOURCES = ["api.hip", "logprob.hip", "diagnostics.hip", "lmhead.hip", "dlogits.hip",
           "compact.hip"]
HEADERS = ["common.h", "classify.h", "exact.h", "lse.h", "rowio.h"]
CEILING_LIB = os.path.join(PKG, "libdrift_ceiling.so")
CEILING_SOURCE = "ceiling.hip"

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-mcode-object-version=5", "-Wall", "-Wno-unused-function",
    # packed fp32 vector instructions stay disabled in every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found; the drift library needs ROCm's hipcc")
    return p


def _fingerprint(hipcc: str) -> str:
    ver = subprocess.run([hipcc, "--version"], capture_output=True, text=True).stdout
    ver = " ".join(l.strip() for l in ver.splitlines() if "version" in l.lower())[:160]
    h = hashlib.sha256()
    for s in SOURCES + HEADERS:
        with open(os.path.join(CSRC, s), "rb") as f:
            h.update(f.read())
    with open(os.path.join(INCLUDE, "drift.h"), "rb") as f:
        h.update(f.read())
    return f"src:{h.hexdigest()[:16]} arch:{ARCH} flags:{' '.join(FLAGS[1:7])} {ver}"


def build(verbose: bool = False, defines=(), out: str = LIB, build_dir: str = BUILD_DIR) -> str:
    """Compile every source (always; no up-to-date check) and link the library.
    `defines` are extra -D options (e.g. another scoring block shape); they become part of
    the build fingerprint."""
    hipcc = _hipcc()
    os.makedirs(build_dir, exist_ok=True)
    fp = _fingerprint(hipcc).replace('"', "'")
    if defines:
        fp += " defs:" + ",".join(defines)
    defs = [f'-DDRIFT_BUILD_FINGERPRINT="{fp}"', f"-I{INCLUDE}", f"-I{CSRC}"]
    defs += [f"-D{d}" for d in defines]

    def compile_one(src):
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        cmd = [hipcc, *FLAGS, *defs, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
        if verbose and msg.strip():
            print(msg, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


def build_ceiling(out: str = CEILING_LIB) -> str:
    """Compile and link the measurement-only read kernel (no part of the drift library)."""
    hipcc = _hipcc()
    tmp = out + ".tmp"
    cmd = [hipcc, *FLAGS, f"-I{INCLUDE}", "-shared", "-o", tmp, os.path.join(CSRC, CEILING_SOURCE)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
        raise RuntimeError(f"hipcc failed on {CEILING_SOURCE}:\n{msg}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_ceiling())

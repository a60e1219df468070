"""Compile libgtc.so (HIP for gfx950) in-tree: graph_triangle_counting_amd/libgtc.so."""
from __future__ import annotations

import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(ROOT, "_build", "gtc")
LIB = os.path.join(PKG, "libgtc.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",  # the weight product is two separately rounded multiplies
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-result",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    err = "\n".join(line for line in r.stderr.splitlines() if "packed-fp32-ops" not in line
                    and "is not a recognized feature" not in line)
    if err.strip() and verbose:
        print(err)
    return obj


# kernel -> source file; build() writes <kernel>.fingerprint beside the library for each
FINGERPRINTED = {"k_triplet": "triplet.hip", "k_clique4": "clique4.hip"}


def fingerprint_path(kernel: str) -> str:
    return os.path.join(PKG, f"{kernel}.fingerprint")


def kernel_fingerprint_from_isa(kernel: str = "k_triplet") -> str:
    """sha256 (first 16 hex digits) of the gfx950 instructions of every instantiation of the
    kernel: the device assembly of its source with comments, labels' line comments and blank lines
    removed.  It changes with the kernel's machine code and with nothing else (host code, headers
    the kernel does not use, comments)."""
    import hashlib
    import re
    src = os.path.join(CSRC, FINGERPRINTED[kernel])
    r = subprocess.run([HIPCC, *FLAGS, "--cuda-device-only", "-S", src, "-o", "-"],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed on {src}:\n{r.stderr}")
    h = hashlib.sha256()
    inside = False
    for line in r.stdout.splitlines():
        if re.match(rf"^_ZN3gtc{len(kernel)}{kernel}\w*:", line):
            inside = True
        elif inside and line.startswith(".Lfunc_end"):
            inside = False
        if inside:
            code = line.split(";", 1)[0].rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with ThreadPoolExecutor(max_workers=min(8, len(srcs)) + len(FINGERPRINTED)) as ex:
        fps = {k: ex.submit(kernel_fingerprint_from_isa, k) for k in FINGERPRINTED}
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
        for k, fp in fps.items():
            with open(fingerprint_path(k), "w") as fh:
                fh.write(fp.result() + "\n")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

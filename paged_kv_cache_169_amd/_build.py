"""Build libkvcache.so (the HIP library) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkvcache.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    # packed fp32 VALU ops are kept out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]

# Sources whose fp32 results must match a plain IEEE evaluation exactly
# (INT4 codes, RoPE outputs) are built without multiply-add contraction.
SOURCES = {
    "api.cpp": [],
    "append.hip": ["-ffp-contract=off"],
    "int4.hip": ["-ffp-contract=off"],
    "rope.hip": ["-ffp-contract=off"],
    "copy.hip": [],
    "attention.hip": [],
    "blend.hip": [],
    "measure.hip": [],
    "noalloc.hip": [],
    "window.hip": [],
}


def sources_digest() -> str:
    """sha256 over every source and header the library is built from."""
    import hashlib
    h = hashlib.sha256()
    names = sorted(SOURCES) + sorted(f for f in os.listdir(CSRC) if f.endswith(".h"))
    for name in names:
        h.update(name.encode())
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    with open(os.path.join(ROOT, "include", "kvcache.h"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()


DIGEST_FILE = LIB + ".sources"  # sources_digest() of the sources LIB was last built from


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON + extra + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda kv: _compile(*kv), SOURCES.items()))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    with open(DIGEST_FILE, "w") as f:
        f.write(sources_digest() + "\n")
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)

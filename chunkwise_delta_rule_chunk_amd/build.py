"""Build librewy.so (gfx950) in-tree with hipcc.

Every translation unit under csrc/ is compiled in parallel to an object file,
then linked into chunkwise_delta_rule_chunk_amd/librewy.so.  Always rebuilds
when called (objects are cached by source hash only within one call tree).
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build", "obj")
LIB = os.path.join(HERE, "librewy.so")
ARCH = "gfx950"
SOURCES = ["api.hip", "k_fwd_prep.hip", "k_scan.hip", "k_bwd_chunk.hip", "k_recurrent.hip"]

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-ffp-contract=fast", "-I", INCLUDE, "-I", CSRC,
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _digest(src: str) -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hpp", ".h")):
            h.update(open(os.path.join(CSRC, name), "rb").read())
    h.update(open(os.path.join(INCLUDE, "rewy.h"), "rb").read())
    h.update(open(src, "rb").read())
    h.update(" ".join(CFLAGS).encode())
    return h.hexdigest()[:16]


def source_digest() -> str:
    """Digest of every library source (kernels, headers, the C header): names
    the exact code a measurement was taken on."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp", ".h")):
            h.update(name.encode())
            h.update(open(os.path.join(CSRC, name), "rb").read())
    h.update(open(os.path.join(INCLUDE, "rewy.h"), "rb").read())
    return h.hexdigest()[:16]


def _compile(name: str, force: bool) -> str:
    src = os.path.join(CSRC, name)
    obj = os.path.join(OBJDIR, f"{name}.{_digest(src)}.o")
    if force or not os.path.exists(obj):
        tmp = obj + ".tmp"
        r = subprocess.run([HIPCC, *CFLAGS, "-c", src, "-o", tmp], capture_output=True, text=True)
        err = "\n".join(x for x in r.stderr.splitlines() if "packed-fp32-ops" not in x)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {name}:\n{err}")
        os.replace(tmp, obj)
    return obj


def build(force: bool = False, jobs: int | None = None) -> str:
    """Compile the HIP sources (re-using objects whose inputs did not change
    unless ``force``) and link librewy.so.  Returns the library path."""
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, force), SOURCES))
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force="--force" in sys.argv))

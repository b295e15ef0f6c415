"""Build libmoe.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc.

    python -m sparse_mixture_experts_bias_amd.build

Cross-compiles for gfx950 on any machine with ROCm's hipcc; no GPU needed.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe.so")
SOURCES = ["moe_gemm_tall.hip", "moe_gemm_ws.hip", "moe_decode.hip", "moe_abi.hip", "moe_route.hip", "moe_gemm.hip",
           "moe_combine.hip", "moe_pack.hip"]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Wno-unused-result", "-munsafe-fp-atomics",
    # no packed fp32 ALU ops (v_pk_*_f32) in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe.so)")


def _compile(src: str, obj: str) -> None:
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-8000:]}")


def _key(src: str) -> str:
    """Hash of a source, every header of csrc/ and the flags (the incremental build's object key)."""
    h = hashlib.sha256(" ".join(FLAGS).encode())
    for f in sorted(os.listdir(CSRC)):
        if f == src or f.endswith(".h"):
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    return h.hexdigest()[:20]


def build(verbose: bool = True, incremental: bool = False) -> str:
    """Compile every source and link libmoe.so next to this file; returns its path.
    incremental: reuse objects under _build/ whose source, headers and flags are unchanged."""
    with tempfile.TemporaryDirectory(prefix="moe_build_") as tmp:
        if incremental:
            cache = os.path.join(PKG, "_build")
            os.makedirs(cache, exist_ok=True)
            objs = [os.path.join(cache, f"{s[:-4]}-{_key(s)}.o") for s in SOURCES]
            todo = [(s, o) for s, o in zip(SOURCES, objs) if not os.path.exists(o)]
        else:
            objs = [os.path.join(tmp, s.replace(".hip", ".o")) for s in SOURCES]
            todo = list(zip(SOURCES, objs))
        workers = min(max(len(todo), 1), max(1, (os.cpu_count() or 2)))
        with cf.ThreadPoolExecutor(workers) as ex:
            list(ex.map(lambda so: _compile(so[0], so[1] + ".part") or os.replace(so[1] + ".part", so[1]), todo))
        out_tmp = LIB + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out_tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stderr[-8000:]}")
        os.replace(out_tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(incremental="--incremental" in sys.argv)
    sys.exit(0)

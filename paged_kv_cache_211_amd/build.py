"""Build libpkv.so in-tree with hipcc for gfx950.

    python paged_kv_cache_211_amd/build.py          # or __graft_entry__.build()

Every HIP source is compiled with packed fp32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); the host compiler
warns that it does not know the feature, which is harmless.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpkv.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "host.cpp", "allocator.cpp", "kv_ops.hip", "decode.hip", "decode_f32.hip",
           "decode_bf16.hip", "decode_fp8.hip", "decode_mfma.hip", "decode_prefix.hip",
           "prefill.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (expected /opt/rocm/bin/hipcc)")


FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


def compile_cmd(src: str, obj: str) -> list[str]:
    return [hipcc(), *FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    noise = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if verbose and noise:
        print("\n".join(noise), file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel) and link libpkv.so; always recompiles."""
    from concurrent.futures import ThreadPoolExecutor
    with tempfile.TemporaryDirectory(prefix="pkv_build.", dir=PKG) as tmpdir:
        objs = [os.path.join(tmpdir, os.path.splitext(src)[0] + ".o") for src in SOURCES]
        workers = max(1, min(len(SOURCES), os.cpu_count() or 1, 16))
        with ThreadPoolExecutor(workers) as pool:
            for f in [pool.submit(_run, compile_cmd(src, obj), verbose)
                      for src, obj in zip(SOURCES, objs)]:
                f.result()
        tmp = os.path.join(tmpdir, "libpkv.so")
        _run([hipcc(), *FLAGS, "-shared", *objs, "-o", tmp], verbose)
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

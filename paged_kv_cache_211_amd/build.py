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
           "decode_bf16.hip", "decode_fp8.hip", "decode_mfma.hip", "decode_prefix.hip", "noalloc.hip",
           "prefill.hip", "paged_probe.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (expected /opt/rocm/bin/hipcc)")


# -amdgpu-atomic-optimizer-strategy=None: the persistent decode's work-counter
# add must not be rewritten into a wave-aggregated add whose result is
# broadcast (and so waited for) right away; its result is read a tile later.
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
         "-Wno-unused-command-line-argument"]


def compile_cmd(src: str, obj: str, defines=()) -> list[str]:
    return [hipcc(), *FLAGS, *[f"-D{d}" for d in defines], "-I", INCLUDE, "-I", CSRC, "-c",
            os.path.join(CSRC, src), "-o", obj]


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    noise = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if verbose and noise:
        print("\n".join(noise), file=sys.stderr)


def build(verbose: bool = False, out: str | None = None, defines=()) -> str:
    """Compile every source (in parallel) and link libpkv.so; always recompiles.

    out: where to put the library (default: in-tree, where the package loads
    it from); defines: extra NAME=VALUE macros for a measurement build, e.g.
    PKV_DECODE_MFMA=0 to serve every fp8 shape with the vector-ALU kernels
    (such a build is loaded through PKV_LIBRARY, never in-tree)."""
    from concurrent.futures import ThreadPoolExecutor
    if defines and out is None:
        raise ValueError("a build with extra defines needs its own output path")
    dst = os.path.abspath(out) if out else LIB
    with tempfile.TemporaryDirectory(prefix="pkv_build.", dir=PKG) as tmpdir:
        objs = [os.path.join(tmpdir, os.path.splitext(src)[0] + ".o") for src in SOURCES]
        workers = max(1, min(len(SOURCES), os.cpu_count() or 1, 16))
        with ThreadPoolExecutor(workers) as pool:
            for f in [pool.submit(_run, compile_cmd(src, obj, defines), verbose)
                      for src, obj in zip(SOURCES, objs)]:
                f.result()
        tmp = os.path.join(tmpdir, "libpkv.so")
        _run([hipcc(), *FLAGS, "-shared", *objs, "-o", tmp], verbose)
        os.replace(tmp, dst)
    return dst


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--out", default=None, help="library path (default: in-tree)")
    ap.add_argument("-D", dest="defines", action="append", default=[], metavar="NAME=VALUE")
    a = ap.parse_args()
    print(build(verbose=True, out=a.out, defines=a.defines))

"""Build liblvsa.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

Usage: python -m video_diffusion_transformer_lvsa_amd.build [--jobs N]

Every source is compiled to an object of its own (the Draft sources without
floating-point contraction, so their fixed fp32 evaluation order holds), then
linked into ``video_diffusion_transformer_lvsa_amd/liblvsa.so``.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblvsa.so")
ARCH = "gfx950"

SOURCES = {
    "api.cpp": [],
    "attn_bf16.hip": [],
    "attn_grp.hip": [],
    "attn_f32.hip": [],
    "lvsa_mask.hip": [],
    "draft.hip": ["-ffp-contract=off"],
    "fp8.hip": [],
    "attn_fp8.hip": [],
    "scratch.hip": [],
}

COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build liblvsa.so)")


def _compile(src: str, extra: list[str], out_dir: str = OUT_DIR) -> str:
    obj = os.path.join(out_dir, src + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc(), *COMMON, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 5, verbose: bool = False, lib: str = LIB, defines: tuple = ()) -> str:
    """Compile every source and link `lib`; `defines` are extra -D flags."""
    out_dir = OUT_DIR if lib == LIB else os.path.join(os.path.dirname(os.path.abspath(lib)), "_build")
    os.makedirs(out_dir, exist_ok=True)
    extra_d = [f"-D{d}" for d in defines]
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda kv: _compile(kv[0], kv[1] + extra_d, out_dir), SOURCES.items()))
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=5)
    ap.add_argument("--out", default=LIB, help="library path (default: in-tree liblvsa.so)")
    ap.add_argument("-D", dest="defines", action="append", default=[], help="extra preprocessor define")
    args = ap.parse_args(argv)
    build(args.jobs, verbose=True, lib=os.path.abspath(args.out), defines=tuple(args.defines))
    return 0


if __name__ == "__main__":
    sys.exit(main())

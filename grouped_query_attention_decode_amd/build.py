"""Build libgqa.so (HIP, gfx950 only) in-tree with hipcc.

Every source under csrc/ is compiled to an object in _build/ and linked into
grouped_query_attention_decode_amd/libgqa.so. Packed fp32 instructions are disabled
for all device code.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIBRARY = os.path.join(PKG, "libgqa.so")

SOURCES = [
    "gqa_api.hip",
    "attn_generic.hip",
    "splitkv_combine.hip",
    "kv_append.hip",
    "decode_valu.hip",
    "decode_mfma.hip",
    "prefill_mfma.hip",
    "hbm_stream.hip",
]

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# Host code only (the C ABI layer and launch code) under AddressSanitizer and
# UndefinedBehaviorSanitizer: each -fsanitize= is given to the host compilation alone
# (-Xarch_host), device code is built as usual. For the CPU tests of the C ABI, which run no
# kernel: point GQA_LIBRARY_PATH at this library and preload clang's ASan runtime (see README).
SANITIZED_LIBRARY = os.path.join(PKG, "libgqa_sanitized.so")
# Diagnostic build: the decode kernels record per-workgroup timestamps (gqa_timeline_read in
# include/gqa_measure.h). Never the library the binding loads by default.
TIMELINE_LIBRARY = os.path.join(PKG, "libgqa_timeline.so")
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src: str, extra, build_dir: str) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if r.stderr.strip():
        sys.stderr.write(r.stderr)
    return obj


def build(resource_usage: bool = False, jobs: int = 6, sanitize: bool = False, timeline: bool = False) -> str:
    """Compile every HIP source and link libgqa.so (with sanitize: libgqa_sanitized.so, host code
    under ASan and UBSan; with timeline: libgqa_timeline.so, the decode kernels stamping
    per-workgroup times). Returns the library path."""
    assert not (sanitize and timeline)
    build_dir = BUILD_DIR + ("_sanitized" if sanitize else "_timeline" if timeline else "")
    library = SANITIZED_LIBRARY if sanitize else TIMELINE_LIBRARY if timeline else LIBRARY
    os.makedirs(build_dir, exist_ok=True)
    extra = (["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []) + (SANITIZE_FLAGS if sanitize else []) \
        + (["-DGQA_TIMELINE"] if timeline else [])
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, build_dir), SOURCES))
    tmp = library + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, library)
    return library


if __name__ == "__main__":
    print(build(resource_usage="--resource-usage" in sys.argv, sanitize="--sanitize" in sys.argv,
                timeline="--timeline" in sys.argv))

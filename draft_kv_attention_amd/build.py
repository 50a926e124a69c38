"""Build libmasw.so in-tree with hipcc for gfx950.

    python -m draft_kv_attention_amd.build      # or draft_kv_attention_amd.build.build()

Every HIP source under csrc/ is compiled to an object in _build/ (in parallel), then
linked into draft_kv_attention_amd/libmasw.so next to this file.  The same sources are
also built once per entry of VARIANTS, with that entry's macros, into
libmasw_<name>.so: the measured designs that are not the defaults, kept selectable at
build time.  The package always loads libmasw.so; the GPU tests run parity cases
through each variant library as well.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libmasw.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.  The host
# pass prints a harmless "not a recognized feature" warning for it.
COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


# Build-time design alternatives (see the macro comments in csrc/decode_args.hpp,
# csrc/masw_device.hpp and csrc/masw_internal.hpp).
VARIANTS = {
    # decode tiles loaded straight into registers, a separate split-combine kernel after
    # the decode launch, and the verifier's earlier work-group-tiled kernel
    "regs_combine": ["-DMASW_DECODE_LDS_PIPE=0", "-DMASW_SPLIT_MERGE=0", "-DMASW_VERIFY_STREAM=0"],
    # register tiles double-buffered with non-temporal loads; in-launch merge with
    # device-scope fences around the ticket
    "dbuf_fence": ["-DMASW_DECODE_LDS_PIPE=0", "-DMASW_DECODE_DOUBLE_BUFFER=1", "-DMASW_DECODE_NT=1",
                   "-DMASW_SPLIT_MERGE=1"],
    # three LDS stages per decode wave instead of two
    "three_stages": ["-DMASW_DECODE_PIPE_STAGES=3"],
}


def variant_path(name: str) -> str:
    return os.path.join(HERE, f"libmasw_{name}.so")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, variant: str = "") -> str:
    out_dir = os.path.join(BUILD_DIR, variant) if variant else BUILD_DIR
    obj = os.path.join(out_dir, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, *VARIANTS.get(variant, []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, path: str) -> None:
    tmp = path + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = False, variants: bool = True) -> str:
    """Compile every csrc/*.hip and link libmasw.so (and, with `variants`, one library
    per VARIANTS entry); returns the path of libmasw.so."""
    names = [""] + (sorted(VARIANTS) if variants else [])
    for n in names:
        os.makedirs(os.path.join(BUILD_DIR, n) if n else BUILD_DIR, exist_ok=True)
    srcs = sources()
    jobs = [(src, n) for n in names for src in srcs]
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    for i, n in enumerate(names):
        _link(objs[i * len(srcs):(i + 1) * len(srcs)], variant_path(n) if n else LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {len(srcs)} sources"
              + (f" and {len(names) - 1} variant libraries" if variants else ""), file=sys.stderr)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)

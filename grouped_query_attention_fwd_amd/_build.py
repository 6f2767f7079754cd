"""Build step for libgqa.so (hipcc, gfx950).  Run as a module or through the
repository's build() entry point; it always recompiles.

    python -m grouped_query_attention_fwd_amd._build [-v]
    python -m grouped_query_attention_fwd_amd._build --trace

--trace builds libgqa_trace.so instead: the same library with the decode's
per-workgroup timing records compiled in (GQA_DECODE_TRACE), for
`bench.py --decode-trace`.  It is never loaded by the attention path."""

from __future__ import annotations

import concurrent.futures
import os
import sys

import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgqa.so")
TRACE_LIB = os.path.join(PKG, "libgqa_trace.so")
PROBE_LIB = os.path.join(PKG, "libgqa_probe.so")
SOURCES = ["gqa_api.hip", "decode.hip", "prefill.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; drop that noise
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "packed-fp32-ops" not in line and "not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def _library(lib, build_dir, defines):
    os.makedirs(build_dir, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *CFLAGS, *defines, "-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(4, len(cmds))) as ex:
        outs = list(ex.map(_run, cmds))
    vers = os.path.join(build_dir, "exports.map")
    with open(vers, "w") as f:
        f.write("{ global: gqa_*; local: *; };\n")
    tmp = lib + ".tmp"
    outs.append(_run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs,
                      f"-Wl,--version-script={vers}"]))
    os.replace(tmp, lib)
    return outs


ASAN_DIR = os.path.join(BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libgqa_asan.so")
# host code only: the device code of a sanitized build is the regular one
SANITIZE = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split()


def asan_runtime() -> str:
    """The compiler's shared ASan runtime (to preload into a process that
    loads the sanitized library)."""
    out = _run([HIPCC, "--print-file-name=libclang_rt.asan-x86_64.so"]).strip().splitlines()
    path = out[-1] if out else ""
    if not os.path.isabs(path) or not os.path.exists(path):
        import glob
        hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
        if not hits:
            raise RuntimeError("ASan runtime not found")
        path = hits[-1]
    return path


def build_sanitized() -> str:
    """CPU checking build: the C-ABI layer (gqa_api.hip) with its host code
    under AddressSanitizer and UndefinedBehaviorSanitizer, linked with the
    regular kernel objects of build().  For running the ABI checks on the
    CPU; never used on a GPU."""
    os.makedirs(ASAN_DIR, exist_ok=True)
    if not all(os.path.exists(os.path.join(BUILD, s.replace(".hip", ".o"))) for s in SOURCES[1:]):
        build()
    obj = os.path.join(ASAN_DIR, "gqa_api.o")
    _run([HIPCC, *CFLAGS, "-O1", "-g", *SANITIZE, "-Xarch_host", "-fno-omit-frame-pointer",
          "-c", os.path.join(CSRC, "gqa_api.hip"), "-o", obj])
    tmp = ASAN_LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *SANITIZE, "-shared-libasan",
          "-o", tmp, obj, *(os.path.join(BUILD, s.replace(".hip", ".o")) for s in SOURCES[1:])])
    os.replace(tmp, ASAN_LIB)
    return ASAN_LIB


def build(verbose: bool = False, trace: bool = False) -> str:
    if trace:
        outs = _library(TRACE_LIB, os.path.join(BUILD, "trace"), ["-DGQA_DECODE_TRACE=1"])
        lib = TRACE_LIB
    else:
        outs = _library(LIB, BUILD, [])
        # the HBM read-rate probe the benchmark uses for calibration: its own
        # library, not part of the attention path
        ptmp = PROBE_LIB + ".tmp"
        outs.append(_run([HIPCC, *CFLAGS, "-shared", os.path.join(CSRC, "read_probe.hip"),
                          "-o", ptmp]))
        os.replace(ptmp, PROBE_LIB)
        lib = LIB
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, trace="--trace" in sys.argv))

"""Builds libcsa2.so and the peak-probe library libcsa2_probe.so (gfx950)
in-tree with hipcc.

    python -m fp4_kv_cache_layer_amd.build
    python -m fp4_kv_cache_layer_amd.build --sanitized DIR

The second form builds a copy of the library whose host code carries
AddressSanitizer and UndefinedBehaviorSanitizer (the device code is built as
usual) into DIR, for running the host-side tests under the sanitizers.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libcsa2.so")
PROBE_LIB = os.path.join(PKG, "libcsa2_probe.so")
PROBE_SOURCE = "probe.hip"
SOURCES = ["api.hip", "append_quant.hip", "index_scan.hip", "prefill_scan.hip", "topk_select.hip", "sparse_attn.hip",
           "lse_merge.hip", "fake_quant.hip", "pool_index.hip", "prune.hip"]
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
    f"--offload-arch={ARCH}",
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results in ordinary VGPRs: the epilogues read every
    # accumulator, and an AGPR result would cost one copy per register
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-result",
]
SOURCE_FLAGS = {s: [] for s in SOURCES}
# the scan's one-lane reservation atomic is waited on only after the candidate
# listing; the atomic optimizer would rewrite it into a wave-wide form whose
# result is needed (waited on) at once
SOURCE_FLAGS["index_scan.hip"] = ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]
BUILD_DIR = os.path.join(ROOT, "_build")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    return "hipcc"


def _run(cmd, verbose: bool):
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


def _finish(proc, verbose: bool, what: str) -> None:
    text, _ = proc.communicate()
    out = "\n".join(l for l in text.splitlines()
                    if "packed-fp32-ops" not in l and "unknown target feature" not in l.lower())
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed on {what} ({proc.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    """Compiles every HIP source (in parallel, each with its own flags) and
    links them into one shared library, plus the probe library; returns the
    main library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    probe_tmp = PROBE_LIB + ".tmp"
    probe = _run([hipcc(), *FLAGS, *inc, "-shared", os.path.join(CSRC, PROBE_SOURCE), "-o", probe_tmp], verbose)
    objs, procs = [], []
    for s in SOURCES:
        obj = os.path.join(BUILD_DIR, s.replace(".hip", ".o"))
        objs.append(obj)
        procs.append((s, _run([hipcc(), *FLAGS, *SOURCE_FLAGS[s], *inc, "-c", os.path.join(CSRC, s), "-o", obj],
                              verbose)))
    for s, p in procs:
        _finish(p, verbose, s)
    tmp = LIB + ".tmp"
    _finish(_run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose), verbose, "link")
    os.replace(tmp, LIB)
    _finish(probe, verbose, PROBE_SOURCE)
    os.replace(probe_tmp, PROBE_LIB)
    return LIB


# host-only sanitizers: each -fsanitize= applies to the host pass alone
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
SANITIZED_NAME = "libcsa2_sanitized.so"


def asan_runtime() -> str | None:
    """The clang AddressSanitizer runtime that a host process must preload to
    load the sanitized library, or None when the toolchain has none."""
    import glob
    for d in sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux")):
        p = os.path.join(d, "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    return None


def build_sanitized(out_dir: str, verbose: bool = False) -> str:
    """Builds the library with host-side ASan and UBSan into out_dir (not the
    package: the product library is never replaced by it); returns its path."""
    os.makedirs(out_dir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs, procs = [], []
    for s in SOURCES:
        obj = os.path.join(out_dir, s.replace(".hip", ".o"))
        objs.append(obj)
        procs.append((s, _run([hipcc(), *FLAGS, *SOURCE_FLAGS[s], *SANITIZE, *inc, "-c", os.path.join(CSRC, s),
                               "-o", obj], verbose)))
    for s, p in procs:
        _finish(p, verbose, s)
    lib = os.path.join(out_dir, SANITIZED_NAME)
    _finish(_run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *SANITIZE, *objs, "-o", lib], verbose),
            verbose, "sanitized link")
    return lib


if __name__ == "__main__":
    if "--sanitized" in sys.argv:
        print(build_sanitized(sys.argv[sys.argv.index("--sanitized") + 1], verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))

"""Build libfa.so (the gfx950 FlashAttention-2 forward library) in-tree.

    python -m exact_attention_26_amd.build

Every translation unit is compiled with hipcc for gfx950 only, with packed
fp32 VALU instructions disabled, then linked into a shared library next to
this file. Object files go to ``_build/`` at the repository root.

Two debug libraries are built from the same sources; only the tests load
them:
  libfa_lds_poison.so (FA_DEBUG_POISON_LDS): before every LDS DMA copy is
    issued its destination is filled with NaN, so a read of a stage that is
    not ordered after the copy's completion shows up as NaN in the outputs;
  libfa_trace.so (FA_DEBUG_TRACE): the 16-bit forward can record the
    timestamps of each phase of one workgroup (fa_debug_fwd_trace).
"""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")
POISON_LIB = os.path.join(PKG, "libfa_lds_poison.so")
TRACE_LIB = os.path.join(PKG, "libfa_trace.so")
# Library variants: output path, extra compile flags, object directory.
VARIANTS = [(LIB, [], BUILD),
            (POISON_LIB, ["-DFA_DEBUG_POISON_LDS"], os.path.join(BUILD, "lds_poison")),
            (TRACE_LIB, ["-DFA_DEBUG_TRACE"], os.path.join(BUILD, "trace"))]

SOURCES = ["fa_api.hip", "fa_noalloc.hip", "fa_fwd_f32.hip", "fa_fwd_mfma16.hip", "fa_fwd_kvouter.hip",
           "fa_norm.hip",
           "fa_bwd.hip"]
# Per-source extra flags. The backward's key-block kernel runs one wave per
# SIMD with >256 live registers; left to itself the compiler gives every
# MFMA an AGPR destination, and the score and dP tiles then need a
# v_accvgpr_read per element before the VALU can use them. VGPR-form MFMAs
# keep those tiles in VGPRs (measured +4 % at d = 128, +25 % at d = 64).
EXTRA_FLAGS = {"fa_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        "-Wno-unused-function",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE,
        "-I", CSRC,
    ]


def source_stamp(extra: list[str] | None = None) -> str:
    """Hash of everything a library build reads: the compiler flags (with the
    variant's extra ones), the per-source flags, and the bytes of every
    source and header under csrc/ and include/."""
    h = hashlib.sha256()
    # Paths are left out: the same tree may sit at another absolute path.
    flags = [{INCLUDE: "<include>", CSRC: "<csrc>"}.get(f, f) for f in compile_flags()]
    h.update(repr((flags, extra or [], sorted(EXTRA_FLAGS.items()), SOURCES)).encode())
    for d in (CSRC, INCLUDE):
        for name in sorted(os.listdir(d)):
            if name.endswith((".hip", ".h", ".cpp")):
                h.update(name.encode())
                with open(os.path.join(d, name), "rb") as f:
                    h.update(f.read())
    return h.hexdigest()


def stamp_path(lib: str) -> str:
    """The file next to a built library that holds its source_stamp()."""
    return lib + ".stamp"


def is_current(lib: str = LIB) -> bool:
    """Whether the library variant at `lib` exists and was built from the
    sources and flags now in the tree (its stamp matches)."""
    extra = {path: ex for path, ex, _ in VARIANTS}.get(lib)
    try:
        with open(stamp_path(lib)) as f:
            recorded = f.read().strip()
    except OSError:
        return False
    return os.path.exists(lib) and extra is not None and recorded == source_stamp(extra)


def build(verbose: bool = False) -> str:
    """Compile all sources of every variant (in parallel) and link them.
    Returns the path of the product library, libfa.so."""
    cc = hipcc()
    procs = []
    links = []
    for lib, extra, objdir in VARIANTS:
        os.makedirs(objdir, exist_ok=True)
        objs = []
        for src in SOURCES:
            obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
            objs.append(obj)
            cmd = [cc, *compile_flags(), *extra, *EXTRA_FLAGS.get(src, []), "-c",
                   os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.STDOUT, text=True)))
        links.append((lib, objs))
    failed = []
    for src, pr in procs:
        out, _ = pr.communicate()
        # hipcc's host pass does not know the packed-fp32 feature; that
        # warning is expected and dropped.
        lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
        if lines and (verbose or pr.returncode != 0):
            print("\n".join(lines), file=sys.stderr)
        if pr.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    for (lib, objs), (_, extra, _) in zip(links, VARIANTS):
        tmp = lib + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib)
        # The stamp names the sources this library was built from, so that a
        # stale library (sources edited since) can be told apart from a
        # current one without rebuilding.
        with open(stamp_path(lib), "w") as f:
            f.write(source_stamp(extra) + "\n")
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

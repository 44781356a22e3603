"""Builds libmimo_attn.so (gfx950) from csrc/ with hipcc, in-tree next to this file, and two
checking variants that only the tests load: libmimo_attn_poison.so (every kernel fills its LDS
with NaN before it starts, see poison_lds in csrc/common.hpp) and libmimo_attn_hostsan.so (the
host code alone - validation, planning, error paths - built with AddressSanitizer and
UndefinedBehaviorSanitizer: api.hip, where it all lives, compiled with host-side sanitizers and
linked with the product objects of the kernel files; the test preloads the sanitizer runtime).

Usage: python -m sliding_window_sink_seeded_amd.build [-v]
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmimo_attn.so")
LIB_POISON = os.path.join(HERE, "libmimo_attn_poison.so")
LIB_HOSTSAN = os.path.join(HERE, "libmimo_attn_hostsan.so")
# sanitizers for the host compilation alone (each flag behind -Xarch_host)
HOSTSAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer"]
HOSTSAN_SOURCES = ["api.hip"]
SOURCES = ["api.hip", "prefill.hip", "decode.hip", "backward.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # keep hipcc from forming packed fp32 math (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _quiet(stderr: str) -> str:
    return "\n".join(l for l in stderr.splitlines() if "packed-fp32-ops" not in l)


def build(verbose: bool = False) -> str:
    """Compiles every source (always), for the product library and its LDS-poisoning variant, and
    links both; returns the product library's path."""
    hostsan_dir = os.path.join(OBJDIR, "hostsan")
    variants = [(LIB, OBJDIR, [], SOURCES),
                (LIB_POISON, os.path.join(OBJDIR, "poison"), ["-DMIMO_POISON_LDS=1"], SOURCES),
                (LIB_HOSTSAN, hostsan_dir, HOSTSAN_FLAGS, HOSTSAN_SOURCES)]
    procs = []
    for lib, objdir, extra, sources in variants:
        os.makedirs(objdir, exist_ok=True)
        for src in sources:
            obj = os.path.join(objdir, src.replace(".hip", ".o"))
            cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                                text=True)))
    failed = []
    for src, p in procs:
        out, err = p.communicate()
        err = _quiet(err)
        if p.returncode != 0:
            failed.append((src, err))
        elif verbose and err.strip():
            print(err, file=sys.stderr)
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(f"--- {s}\n{e}" for s, e in failed))
    for lib, objdir, _, sources in variants:
        # a variant that compiles only some sources takes the product objects of the rest
        objs = [os.path.join(objdir if src in sources else OBJDIR, src.replace(".hip", ".o")) for src in SOURCES]
        tmp = lib + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + _quiet(r.stderr))
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

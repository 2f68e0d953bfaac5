"""Build libgdn_prefill.so in-tree with hipcc for gfx950.

Each source compiles to its own object in parallel, then one link step makes
the shared library.

Usage: python -m gated_deltanet_chunked_varlen_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgdn_prefill.so")
SOURCES = ["gdn_host.hip", "k0_chunk_index.hip", "k1_intra.hip",
           "k2_state.hip", "k3_output.hip", "k4_decode.hip", "k5_cp.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # keep packed fp32 instructions out of device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _clean(stderr: str) -> str:
    return "\n".join(l for l in stderr.splitlines() if "packed-fp32-ops" not in l)


def build(verbose: bool = False, extra_flags=None, out: str = LIB) -> str:
    flags = FLAGS + list(extra_flags or [])
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    with tempfile.TemporaryDirectory(prefix="gdn_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(s) + ".o") for s in srcs]

        def compile_one(i):
            cmd = [HIPCC] + flags + ["-c", srcs[i], "-o", objs[i]]
            if verbose:
                print(" ".join(cmd), flush=True)
            return subprocess.run(cmd, capture_output=True, text=True)

        jobs = max(1, min(len(srcs), os.cpu_count() or 1, 16))
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(compile_one, range(len(srcs))))
        for s, r in zip(srcs, results):
            err = _clean(r.stderr)
            if r.returncode != 0:
                raise RuntimeError("hipcc failed on %s:\n%s" % (os.path.basename(s), err))
            if verbose and err.strip():
                print(err, file=sys.stderr)
        tmp = out + ".tmp%d" % os.getpid()
        cmd = [HIPCC] + flags + ["-shared", "-o", tmp] + objs
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc link failed:\n" + _clean(r.stderr))
        os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))

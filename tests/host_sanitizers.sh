#!/bin/bash
# The CPU test suite with AddressSanitizer and UndefinedBehaviorSanitizer in
# the host code: the oracle's C part and the host half of libgdn_prefill
# (argument checks, workspace planning, launch set-up; device code is built
# as usual).  Both are built with clang so that one sanitizer runtime serves
# the process; python itself is not instrumented, so the runtime is preloaded.
# Builds go to a temporary folder; the in-tree libraries are not touched.
set -euo pipefail
ROOT="$(cd "$(dirname "$0")/.." && pwd)"
OUT="$(mktemp -d /tmp/gdn_sanitize.XXXXXX)"
trap 'rm -rf "$OUT"' EXIT
CLANG=/opt/rocm/llvm/bin/clang
RTDIR="$(dirname "$($CLANG -print-file-name=libclang_rt.asan-x86_64.so)")"
[ -f "$RTDIR/libclang_rt.asan-x86_64.so" ] || RTDIR="$(ls -d /opt/rocm/llvm/lib/clang/*/lib/linux | head -1)"
SAN="-fsanitize=address,undefined -fno-omit-frame-pointer -shared-libsan -fno-sanitize-recover=undefined"
cd "$ROOT"
python3 - "$OUT" "$SAN" <<'PY'
import sys
out, san = sys.argv[1], sys.argv[2].split()
from oracle import oracle
oracle.build(out=out + "/liboracle_san.so", cc="/opt/rocm/llvm/bin/clang", extra_flags=san)
from gated_deltanet_chunked_varlen_amd import build
host = []
for f in san:
    host += ["-Xarch_host", f]
build.build(out=out + "/libgdn_san.so", extra_flags=host)
PY
export LD_LIBRARY_PATH="$RTDIR${LD_LIBRARY_PATH:+:$LD_LIBRARY_PATH}"
export LD_PRELOAD="$RTDIR/libclang_rt.asan-x86_64.so"
export ASAN_OPTIONS=detect_leaks=0:abort_on_error=1
export UBSAN_OPTIONS=print_stacktrace=1:halt_on_error=1
export GDN_PREFILL_LIB="$OUT/libgdn_san.so" ORACLE_LIB="$OUT/liboracle_san.so"
python3 -m pytest tests -q -m "not gpu" -p no:cacheprovider "$@"

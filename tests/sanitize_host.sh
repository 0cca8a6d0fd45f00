#!/bin/bash
# Host-side AddressSanitizer + UndefinedBehaviorSanitizer check of the library (CPU).
# Builds libmeo.so with the host code instrumented (device code as usual) into a
# scratch directory and runs the CPU test suite against it, the ASan runtime
# preloaded into the Python process. A report stops the run (halt_on_error); leak
# detection is off, since the interpreter itself is not instrumented.
# Usage: bash tests/sanitize_host.sh [scratch dir, default /tmp/meo_sanitize]
set -euo pipefail
R=$(cd "$(dirname "$0")/.." && pwd)
D=${1:-/tmp/meo_sanitize}
C=$R/memory_efficient_optimizers_amd/csrc
HIPCC=${HIPCC:-/opt/rocm/bin/hipcc}
mkdir -p "$D/obj"
FL="-x hip --offload-arch=gfx950 -O1 -g -std=c++17 -fPIC -Wno-unused-command-line-argument -Xclang -target-feature -Xclang -packed-fp32-ops -ffp-contract=off -I $R/include -I $C"
SAN="-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer"
pids=()
for f in abi.cpp passes.hip adafactor.hip came.hip lamb.hip shard.hip galore.hip galore_refresh.hip; do
  "$HIPCC" $FL $SAN -c "$C/$f" -o "$D/obj/${f%.*}.o" 2> "$D/obj/${f%.*}.log" & pids+=($!)
done
for p in "${pids[@]}"; do wait "$p"; done
"$HIPCC" --offload-arch=gfx950 -shared -fPIC -fsanitize=address -fsanitize=undefined -shared-libsan -fno-gpu-sanitize \
  "$D"/obj/*.o -o "$D/libmeo.so"
RT=$(/opt/rocm/llvm/bin/clang -print-file-name=libclang_rt.asan-x86_64.so)
cd "$R"
LD_PRELOAD=$RT ASAN_OPTIONS=detect_leaks=0:detect_odr_violation=0:alloc_dealloc_mismatch=0:halt_on_error=1 \
UBSAN_OPTIONS=print_stacktrace=1:halt_on_error=1 python3 - "$D/libmeo.so" <<'PY'
import sys
import memory_efficient_optimizers_amd._lib as L
L.LIB_PATH = sys.argv[1]
import pytest
rc = pytest.main(["-q", "-p", "no:cacheprovider", "-m", "not gpu", "tests"])
assert L.load()._name == sys.argv[1], "the instrumented library was not the one loaded"
print("sanitized library:", sys.argv[1])
sys.exit(rc)
PY

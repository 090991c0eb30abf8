#!/bin/bash
# The CPU test suite (-m "not gpu") under AddressSanitizer and
# UndefinedBehaviorSanitizer: the oracle and the host code of libspd.so and
# libspd_probe.so rebuilt with both (device code as usual, into
# _lib/sanitize/ and oracle/_build/sanitize/), the clang sanitizer runtime
# preloaded into Python, any finding fatal.  Extra arguments go to pytest.
set -euo pipefail
ROOT="$(cd "$(dirname "$0")/.." && pwd)"
cd "$ROOT"
python3 sparse_paged_decode_ragged_amd/build.py --sanitize
ORACLE=$(python3 -c "import oracle; print(oracle.build(sanitize=True))")
# the runtime the instrumented oracle was linked against
RT=$(ldd "$ORACLE" | awk '/libclang_rt.asan/ {print $3}')
test -f "$RT"
LD_PRELOAD="$RT" ASAN_OPTIONS=detect_leaks=0:abort_on_error=1 \
  UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 LD_LIBRARY_PATH=/opt/rocm/llvm/lib \
  SPD_LIB_DIR="$ROOT/sparse_paged_decode_ragged_amd/_lib/sanitize" SPD_ORACLE_LIB="$ORACLE" \
  SPD_EXPECT_SANITIZED=1 python3 -m pytest tests -m "not gpu" -q -p no:cacheprovider "$@"

#!/bin/bash
# Host-code sanitizer runs (CPU only; no GPU is touched):
#  1. the C oracle built by gcc with AddressSanitizer + UndefinedBehaviorSanitizer, under
#     the oracle's pin and mutation tests;
#  2. libsharq's host code (the C ABI's argument validation, the size queries and the
#     dispatch up to the device check) built by hipcc with both sanitizers on the host
#     side only, under the boundary and binding tests.
# Each run works in a scratch copy of the repository, so the in-tree libraries are left
# alone.  Usage: bash tests/sanitize_cpu.sh   (from the repository root)
set -euo pipefail
ROOT=$(cd "$(dirname "$0")/.." && pwd)
WORK=$(mktemp -d /tmp/sharq_sanitize.XXXXXX)
trap 'rm -rf "$WORK"' EXIT
copy_tree() {
  mkdir -p "$1"
  cp -r "$ROOT/oracle" "$ROOT/tests" "$ROOT/include" "$1"/
  mkdir -p "$1/activation_sparsity_fp4_sharq_amd"
  cp -r "$ROOT/activation_sparsity_fp4_sharq_amd/csrc" "$ROOT"/activation_sparsity_fp4_sharq_amd/*.py \
    "$1/activation_sparsity_fp4_sharq_amd"/
  rm -f "$1"/oracle/*.so "$1"/activation_sparsity_fp4_sharq_amd/*.so
}
SAN_OPTS="detect_leaks=0:halt_on_error=1:alloc_dealloc_mismatch=0:detect_odr_violation=0"

echo "== oracle: gcc -fsanitize=address,undefined"
copy_tree "$WORK/o"
gcc -O1 -g -std=c99 -ffp-contract=off -fno-fast-math -fopenmp -fPIC -shared -Wall -Wextra \
  -fsanitize=address,undefined -fno-sanitize-recover=undefined -fno-omit-frame-pointer \
  -o "$WORK/o/oracle/liboracle.so" "$WORK/o/oracle/sharq_oracle.c" -lm
nm -D "$WORK/o/oracle/liboracle.so" | grep -q __asan_report || { echo "oracle not instrumented"; exit 1; }
nm -D "$WORK/o/oracle/liboracle.so" | grep -q __ubsan_handle || { echo "oracle not instrumented (UB)"; exit 1; }
(cd "$WORK/o" && ASAN_OPTIONS=$SAN_OPTS UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 \
  LD_PRELOAD="$(gcc -print-file-name=libasan.so)" OMP_NUM_THREADS=4 \
  python3 -m pytest tests/test_oracle_pins.py tests/test_oracle_mutations.py -m "not gpu" -x -q -p no:cacheprovider)

echo "== libsharq host code: hipcc -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined"
copy_tree "$WORK/l"
D="$WORK/l/activation_sparsity_fp4_sharq_amd"
objs=()
for f in "$D"/csrc/*.hip; do
  /opt/rocm/bin/hipcc --offload-arch=gfx950 -O1 -g -std=c++17 -fPIC -ffp-contract=off \
    -Xclang -target-feature -Xclang -packed-fp32-ops \
    -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=undefined \
    -Xarch_host -fno-omit-frame-pointer -I "$WORK/l/include" -c "$f" -o "$f.o" 2>/dev/null
  objs+=("$f.o")
done
/opt/rocm/bin/hipcc --offload-arch=gfx950 -shared -fPIC -shared-libsan \
  -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -o "$D/libsharq.so" "${objs[@]}"
nm -D "$D/libsharq.so" | grep -q __asan_report || { echo "libsharq not instrumented"; exit 1; }
nm -D "$D/libsharq.so" | grep -q __ubsan_handle || { echo "libsharq not instrumented (UB)"; exit 1; }
ASAN_RT=$(/opt/rocm/bin/amdclang++ -print-file-name=libclang_rt.asan-x86_64.so)
(cd "$WORK/l" && ASAN_OPTIONS=$SAN_OPTS UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 LD_PRELOAD="$ASAN_RT" \
  python3 -m pytest tests/test_boundary.py tests/test_binding_checks.py -m "not gpu" -x -q -p no:cacheprovider)
echo "== both sanitized runs passed"

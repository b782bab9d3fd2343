#!/bin/bash
# Build the C-ABI host code with AddressSanitizer + UndefinedBehaviorSanitizer (host side
# only: every -fsanitize= sits after -Xarch_host) and run tests/sanitize/abi_driver.cpp
# against it.  Usage: build_and_run.sh <build dir>.  CPU only; the kernels are not run.
set -euo pipefail
OUT=${1:?build dir}
HERE=$(cd "$(dirname "$0")" && pwd)
ROOT=$(cd "$HERE/../.." && pwd)
CSRC=$ROOT/online_softmax_07_amd/csrc
HIPCC=${HIPCC:-/opt/rocm/bin/hipcc}
mkdir -p "$OUT"
SAN="-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=all"
COMMON="-O1 -g -std=c++17 -fno-omit-frame-pointer --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops -I$ROOT/include -I$CSRC"
for f in fa_api fa_calib; do
  $HIPCC $COMMON $SAN -c "$CSRC/$f.hip" -o "$OUT/$f.o" 2> "$OUT/$f.log" || { cat "$OUT/$f.log"; exit 1; }
done
# the kernel files, unsanitized (their host parts only launch kernels, which the driver never reaches)
for f in fa_fwd_bf16 fa_fwd_fp32 fa_decode fa_merge fa_bwd; do
  $HIPCC $COMMON -c "$CSRC/$f.hip" -o "$OUT/$f.o" 2> "$OUT/$f.log" || { cat "$OUT/$f.log"; exit 1; }
done
$HIPCC -O1 -g -std=c++17 $SAN -I$ROOT/include -x c++ "$HERE/abi_driver.cpp" -x none \
  "$OUT"/fa_api.o "$OUT"/fa_calib.o "$OUT"/fa_fwd_bf16.o "$OUT"/fa_fwd_fp32.o "$OUT"/fa_decode.o "$OUT"/fa_merge.o \
  "$OUT"/fa_bwd.o --offload-arch=gfx950 -o "$OUT/abi_driver" 2> "$OUT/link.log" || { cat "$OUT/link.log"; exit 1; }
ASAN_OPTIONS=detect_leaks=0:abort_on_error=1 UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 "$OUT/abi_driver"

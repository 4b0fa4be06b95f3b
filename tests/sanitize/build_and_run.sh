#!/bin/bash
# Build the library's host code (no device code) with AddressSanitizer and UndefinedBehaviorSanitizer
# into the abi_checks driver and run it. Usage: build_and_run.sh OUTDIR
set -euo pipefail
HERE="$(cd "$(dirname "$0")" && pwd)"
ROOT="$(cd "$HERE/../.." && pwd)"
OUT="${1:-$ROOT/_build/sanitize}"
mkdir -p "$OUT"
CSRC="$ROOT/attention_free_long_amd/csrc"
# device code is compiled as for the library (it only has to link; nothing here launches it);
# the sanitizers apply to the host code alone
FLAGS=(--offload-arch=gfx950 -O1 -g -std=c++17 -fno-omit-frame-pointer
       -Xclang -target-feature -Xclang -packed-fp32-ops
       -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined
       -Xarch_host -fno-sanitize-recover=all -I"$ROOT/include" -I"$CSRC")
OBJS=()
PIDS=()
for f in abi prepare maxsim_bf16 topk compress_bf16 dyn_bf16 gemm_bf16 simt_f32 peak_probe noalloc; do
  /opt/rocm/bin/hipcc "${FLAGS[@]}" -c "$CSRC/$f.hip" -o "$OUT/$f.o" 2>"$OUT/$f.log" &
  PIDS+=($!)
  OBJS+=("$OUT/$f.o")
done
for p in "${PIDS[@]}"; do
  wait "$p" || { grep -v packed-fp32 "$OUT"/*.log >&2; exit 1; }
done
g++ -O1 -g -std=c++17 -fno-omit-frame-pointer -fsanitize=address,undefined -fno-sanitize-recover=all \
    -I"$ROOT/include" -c "$HERE/abi_checks.cpp" -o "$OUT/abi_checks_main.o"
/opt/rocm/bin/hipcc --offload-arch=gfx950 -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -o "$OUT/abi_checks" \
    "$OUT/abi_checks_main.o" "${OBJS[@]}"
ASAN_OPTIONS=detect_leaks=0 UBSAN_OPTIONS=print_stacktrace=1:halt_on_error=1 "$OUT/abi_checks"

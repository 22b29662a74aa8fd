#!/bin/bash
# Build of the library's sources with the host side under AddressSanitizer +
# UndefinedBehaviorSanitizer (-Xarch_host: the device code is compiled as usual, without them),
# linked into the abi_checks driver, which never reaches a launch.
# Usage: build.sh OUT_DIR
set -e
HERE="$(cd "$(dirname "$0")" && pwd)"
ROOT="$(cd "$HERE/../.." && pwd)"
OUT="$1"
CSRC="$ROOT/gated_deltanet_linear_verify_amd/csrc"
HIPCC="${HIPCC:-/opt/rocm/bin/hipcc}"
SAN="-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=all"
mkdir -p "$OUT"
objs=()
DEV="--offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops"
pids=()
for f in gdn_abi.cpp gdn_prefill_abi.cpp gdn_linear_abi.cpp gdn_graph.cpp gdn_verify.hip gdn_rollback.hip \
         gdn_tree.hip gdn_prefill.hip gdn_linear.hip gdn_noalloc.hip gdn_scratch.cpp; do
    o="$OUT/${f%.*}.o"
    lang=""
    case "$f" in *.hip) lang="-x hip" ;; esac
    "$HIPCC" $DEV $lang -O1 -g -std=c++17 -fPIC -I"$ROOT/include" $SAN -c "$CSRC/$f" -o "$o" 2>"$o.log" &
    pids+=($!)
    objs+=("$o")
done
for p in "${pids[@]}"; do wait "$p"; done
"$HIPCC" -x c -O1 -g -I"$ROOT/include" $SAN -c "$HERE/abi_checks.c" -o "$OUT/abi_checks.o" 2>/dev/null
"$HIPCC" $DEV $SAN "$OUT/abi_checks.o" "${objs[@]}" -o "$OUT/abi_checks" 2>/dev/null

#!/bin/bash
# Build the host-side ABI driver against libmlra's sources with AddressSanitizer and
# UndefinedBehaviorSanitizer on the host code only (each -fsanitize= follows -Xarch_host, so
# the gfx950 device code is built as usual). Usage: build.sh OUT_DIR
set -euo pipefail
OUT=${1:?out dir}
HERE=$(cd "$(dirname "$0")" && pwd)
ROOT=$(cd "$HERE/../.." && pwd)
CSRC=$ROOT/rank_latent_kv_amd/csrc
mkdir -p "$OUT"
SAN="-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer"
FLAGS="-O1 -g -std=c++17 --offload-arch=gfx950 -I $ROOT/include -I $CSRC -Xclang -target-feature -Xclang -packed-fp32-ops -Wno-unused-result -Wno-inline-asm"
pids=()
for f in attn_mfma.hip attn_generic.hip merge.hip paged.hip prepare.hip read_probe.hip; do
  hipcc $FLAGS $SAN -c "$CSRC/$f" -o "$OUT/$f.o" & pids+=($!)
done
hipcc -x hip $FLAGS $SAN -c "$CSRC/mlra_api.cpp" -o "$OUT/mlra_api.o" & pids+=($!)
hipcc -x hip $FLAGS $SAN -c "$HERE/drive.cpp" -o "$OUT/drive.o" & pids+=($!)
for p in "${pids[@]}"; do wait "$p"; done
hipcc --offload-arch=gfx950 $SAN -o "$OUT/drive" "$OUT"/*.o

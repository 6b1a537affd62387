#!/bin/bash
# Host-sanitized build of libflarepp for the CPU tests: the C-ABI files
# (argument checks, plans, workspace layout, launch sequences) compiled
# with AddressSanitizer and UndefinedBehaviorSanitizer on the host side
# only, linked with the package build's kernel objects.  The result is
# never loaded on a GPU: the CPU tests run the ABI's validation paths
# through it.
# usage: build_host_sanitized.sh OUT_DIR   (after the package build)
set -e
OUT=$1
ROOT=$(cd "$(dirname "$0")/../.." && pwd)
PKG=$ROOT/rank_latent_attention_mixer_amd
OBJ=$PKG/_build
HIPCC=${HIPCC:-/opt/rocm/bin/hipcc}
CLANGXX=${CLANGXX:-/opt/rocm/llvm/bin/clang++}
mkdir -p "$OUT"
for f in flarepp_abi backward_abi frontend_abi; do
  "$HIPCC" -x hip -c "$PKG/csrc/$f.cpp" -o "$OUT/$f.o" -O1 -g -std=c++17 -fPIC \
    --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops \
    -Wno-unused-command-line-argument -I"$ROOT/include" -I"$PKG/csrc" \
    -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined \
    -Xarch_host -fno-omit-frame-pointer -Xarch_host -fno-sanitize-recover=all
done
"$CLANGXX" -shared -fPIC -fsanitize=address,undefined -shared-libasan -o "$OUT/libflarepp.so" \
  "$OUT/flarepp_abi.o" "$OUT/backward_abi.o" "$OUT/frontend_abi.o" \
  "$OBJ/encode_split.o" "$OBJ/combine.o" "$OBJ/decode.o" "$OBJ/backward.o" \
  "$OBJ/backward_valu.o" "$OBJ/frontend.o" \
  -L/opt/rocm/lib -lamdhip64 -Wl,-rpath,/opt/rocm/lib
"$CLANGXX" -print-file-name=libclang_rt.asan-x86_64.so > "$OUT/asan_runtime.txt"

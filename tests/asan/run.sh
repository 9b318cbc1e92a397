#!/bin/bash
# Host-side AddressSanitizer check of the C ABI, on the CPU (no GPU needed): the host sources
# api.cpp and qapi.cpp are compiled instrumented (-Xarch_host: device code is never built with
# the sanitizer), linked with the device objects of the normal build (run build() first), and
# driver.c calls every entry point's argument checks and no-device paths.
set -e
HERE=$(cd "$(dirname "$0")" && pwd)
R=$(cd "$HERE/../.." && pwd)
B=$R/tiled_matrix_multiply_amd/_build
O=$(mktemp -d)
trap 'rm -rf "$O"' EXIT
HIPCC=/opt/rocm/bin/hipcc
CLANG=/opt/rocm/llvm/bin/clang
for s in api qapi; do
  $HIPCC -O1 -g -std=c++17 -fPIC -fvisibility=hidden -Wall -I "$R/include" -I "$R/tiled_matrix_multiply_amd/csrc" \
    -Xarch_host -fsanitize=address -fno-omit-frame-pointer -c "$R/tiled_matrix_multiply_amd/csrc/$s.cpp" -o "$O/${s}_asan.o"
done
$CLANG -O1 -g -fsanitize=address -fno-omit-frame-pointer -I "$R/include" -c "$HERE/driver.c" -o "$O/driver.o"
OBJS=$(ls "$B"/*.o | grep -v -e '/api.o$' -e '/qapi.o$' -e '_lds_poison.o$')
$CLANG++ -fsanitize=address "$O/driver.o" "$O/api_asan.o" "$O/qapi_asan.o" $OBJS -L/opt/rocm/lib -lamdhip64 \
  -Wl,-rpath,/opt/rocm/lib -o "$O/driver"
ASAN_OPTIONS=detect_leaks=1 "$O/driver"

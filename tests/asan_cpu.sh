#!/bin/bash
# AddressSanitizer run of the CPU test suite (no GPU): the oracle (gcc ASan) and
# the host code of libqmm (argument validation, dispatch, launch set-up; hipcc
# with ASan on the host side only) are built into a scratch copy of the tree,
# and the -m "not gpu" tests run there against them, each group with its own
# sanitizer runtime preloaded.  Usage: bash tests/asan_cpu.sh
set -euo pipefail
SRC=$(cd "$(dirname "$0")/.." && pwd)
T=$(mktemp -d /tmp/qmm_asan.XXXXXX)
trap 'rm -rf "$T"' EXIT
cp -r "$SRC/oracle" "$SRC/bit_quantized_mat_quantize_amd" "$SRC/include" "$SRC/tests" "$T/"
rm -f "$T"/oracle/*.so "$T"/bit_quantized_mat_quantize_amd/*.so
cd "$T"
ORACLE_ASAN=1 python -c "import oracle; oracle.build()"
QMM_ASAN=1 python -m bit_quantized_mat_quantize_amd.build > /dev/null
export ASAN_OPTIONS=detect_leaks=0:abort_on_error=1
GCC_ASAN=$(gcc -print-file-name=libasan.so)
CLANG_ASAN=$(ls /opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so | head -1)
echo "== oracle under $GCC_ASAN"
LD_PRELOAD="$GCC_ASAN" python -m pytest -q -p no:cacheprovider -m "not gpu" tests/test_oracle.py tests/test_oracle_q6k.py \
    tests/test_oracle_q2k.py tests/test_oracle_moe.py
echo "== libqmm host code under $CLANG_ASAN"
LD_PRELOAD="$CLANG_ASAN" python -m pytest -q -p no:cacheprovider -m "not gpu" tests/test_abi.py tests/test_dispatch_log.py

"""The CPU test suite under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds, into a temporary directory, the oracle (oracle/kv4_oracle.c, with
clang) and libkv4 (hipcc; the sanitizers instrument the host code only, the
gfx950 code is built as usual), then runs `pytest -m "not gpu"` against those
two libraries (KV4_LIB, KV4_ORACLE_LIB) with clang's ASan runtime preloaded
into the Python process.  The run stops at the first report.  No GPU is
used: the CPU tests call only the host side of libkv4 (argument checks,
sizes, the partition arithmetic, status strings).

    python tests/sanitize_cpu.py [extra pytest arguments]
"""
import glob
import os
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from int8_mixed_precision_amd import build as B  # noqa: E402

LLVM = "/opt/rocm/llvm"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer"]


def asan_runtime():
    libs = sorted(glob.glob(os.path.join(LLVM, "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not libs:
        raise SystemExit("clang's ASan runtime (libclang_rt.asan-x86_64.so) was not found")
    return libs[-1]


def build(tmp):
    oracle_lib = os.path.join(tmp, "libkv4_oracle.so")
    subprocess.check_call([os.path.join(LLVM, "bin", "clang"), "-O1", "-g", *SAN, "-std=c11",
                           "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC",
                           "-Wall", "-Wno-unknown-pragmas",
                           os.path.join(ROOT, "oracle", "kv4_oracle.c"), "-o", oracle_lib, "-lm"])
    kv4_lib = os.path.join(tmp, "libkv4.so")
    host_san = [x for f in SAN for x in ("-Xarch_host", f)]
    subprocess.check_call([B.HIPCC, *B.HIPFLAGS, "-g", *host_san,
                           os.path.join(ROOT, "int8_mixed_precision_amd", "csrc", "kv4.hip"),
                           "-o", kv4_lib])
    return oracle_lib, kv4_lib


def main():
    with tempfile.TemporaryDirectory(prefix="kv4_san_") as tmp:
        oracle_lib, kv4_lib = build(tmp)
        env = dict(os.environ)
        env.update(
            LD_PRELOAD=asan_runtime(),
            ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:detect_odr_violation=0:"
                         "alloc_dealloc_mismatch=0:verify_asan_link_order=0",
            UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
            KV4_LIB=kv4_lib, KV4_ORACLE_LIB=oracle_lib,
            OMP_NUM_THREADS=env.get("OMP_NUM_THREADS", "8"))
        # the run must load the sanitized builds and the runtime, not the in-tree libraries
        check = ("import oracle, ctypes; from int8_mixed_precision_amd import kv4; oracle.lib(); "
                 "maps = open('/proc/self/maps').read(); "
                 f"assert {kv4_lib!r} in maps and {oracle_lib!r} in maps and 'libclang_rt.asan' in maps, maps")
        subprocess.check_call([sys.executable, "-c", check], env=env, cwd=ROOT)
        cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-m", "not gpu", "-x", "-q",
               "-p", "no:cacheprovider", *sys.argv[1:]]
        print("sanitized run:", " ".join(cmd), flush=True)
        return subprocess.call(cmd, env=env, cwd=ROOT)


if __name__ == "__main__":
    sys.exit(main())

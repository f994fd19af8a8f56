"""Host AddressSanitizer + UndefinedBehaviorSanitizer run of the CPU test suite.

    python tests/sanitize_host.py

Builds libmoe with its host code instrumented (hipcc: every sanitizer flag
behind -Xarch_host, the device code untouched) and the C oracle with clang and
the same sanitizers, both under _build/sanitize/, then runs
`pytest tests -m "not gpu"` with them loaded in place of the regular builds
(MOE_LIBRARY, ORACLE_LIBRARY) and clang's ASan runtime preloaded into the
uninstrumented Python.  Any report aborts the run.  CPU only: nothing is
launched on a GPU (the CPU suite exercises the ABI's argument checks, the
workspace and tier arithmetic on the host, and every oracle routine).
Exit status: pytest's.
"""
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_lib():
    sys.path.insert(0, os.path.join(ROOT, "bit_dequant_expert_router_amd"))
    import build as moe_build
    flags = [f for f in moe_build.FLAGS if f != "-O3"] + ["-O1", "-g"] + SAN_HOST + ["-shared-libsan"]
    out = os.path.join(OUT, "libmoe_san.so")
    subprocess.check_call([moe_build.HIPCC] + flags + moe_build.sources() + ["-o", out])
    return out


def build_oracle():
    out = os.path.join(OUT, "liboracle_san.so")
    subprocess.check_call([os.path.join(ROCM, "llvm", "bin", "clang"), "-O1", "-g", "-fno-omit-frame-pointer",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-shared-libsan",
                           "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC", "-std=c11",
                           os.path.join(ROOT, "oracle", "moe_oracle.c"), "-o", out, "-lm"])
    return out


def asan_runtime():
    found = sorted(glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    if not found:
        raise SystemExit("clang's ASan runtime (libclang_rt.asan-x86_64.so) not found under " + ROCM)
    return found[-1]


def main():
    os.makedirs(OUT, exist_ok=True)
    lib, orc, rt = build_lib(), build_oracle(), asan_runtime()
    env = dict(os.environ)
    env.update(MOE_LIBRARY=lib, ORACLE_LIBRARY=orc, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-m", "not gpu",
           "-p", "no:cacheprovider"] + sys.argv[1:]
    print("sanitized libraries:", lib, orc, "runtime:", rt, flush=True)
    # the bindings must map the sanitized builds, not the regular ones
    probe = ("import os, bit_dequant_expert_router_amd as m, oracle; oracle.lib(); "
             "maps = open('/proc/self/maps').read(); "
             "assert m.LIB_PATH == os.environ['MOE_LIBRARY'] and os.environ['MOE_LIBRARY'] in maps; "
             "assert os.environ['ORACLE_LIBRARY'] in maps and oracle.LIB_PATH not in maps; "
             "print('loaded:', m.LIB_PATH, os.environ['ORACLE_LIBRARY'])")
    subprocess.check_call([sys.executable, "-c", probe], env=env, cwd=ROOT)
    return subprocess.call(cmd, env=env, cwd=ROOT)


if __name__ == "__main__":
    sys.exit(main())

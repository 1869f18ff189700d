"""Run the CPU test suite against host-sanitized builds of the library and of
the oracle: AddressSanitizer + UndefinedBehaviorSanitizer on the host code
(argument checks, workspace layout, launch set-up of libmoeffn; every oracle
routine).  The kernels themselves are built as usual and are not run here.

    python tests/run_sanitized.py [extra pytest arguments]

Builds activation_sparse_expert_amd/_build_san/{libmoeffn_san,liboracle_san}.so,
then runs `pytest -m "not gpu"` in a child process that preloads clang's ASan
runtime and points MOEFFN_LIB / ORACLE_LIB at the sanitized builds.  Any report
aborts the run (halt_on_error), so exit status 0 means none was raised."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from activation_sparse_expert_amd import build as B  # noqa: E402
import oracle  # noqa: E402

CLANG = "/opt/rocm/llvm/bin/clang"


def main(argv):
    lib = B.build_sanitized()
    olib = oracle.build_sanitized(os.path.join(B.BUILD_SAN, "liboracle_san.so"))
    rt = subprocess.check_output([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                                 text=True).strip()
    if not os.path.exists(rt):
        raise SystemExit(f"ASan runtime not found: {rt}")
    env = dict(os.environ, MOEFFN_LIB=lib, ORACLE_LIB=olib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:protect_shadow_gap=0:halt_on_error=1:"
                            "detect_odr_violation=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-m", "not gpu",
           "-p", "no:cacheprovider", *argv]
    print("sanitized run:", lib, olib, "preload", rt, flush=True)
    return subprocess.call(cmd, env=env, cwd=ROOT)


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))

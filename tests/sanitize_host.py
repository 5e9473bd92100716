"""Runs the CPU test suite (-m "not gpu") on builds whose host code carries
AddressSanitizer and UndefinedBehaviorSanitizer: the C oracle, and the host
side of the HIP library (argument checks, workspace and launch planning, the
status strings, the static-scratch entry's refusals).

    python tests/sanitize_host.py [extra pytest arguments]

No GPU is needed.  Device code is compiled as usual: every -fsanitize= flag of
the library build goes to the host pass alone (-Xarch_host).  Both builds go
to a temporary directory that the loaders pick up through FLINT_SANITIZE_DIR,
and the sanitizers' shared runtime (clang's, which holds both) is preloaded
into the test process.  Any memory error or undefined behaviour ends the run
with a report and a non-zero exit status.  Leak detection is off: the Python
interpreter keeps memory to the end by design.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

SAN_HOST_FLAGS = []
for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-g"):
    SAN_HOST_FLAGS += ["-Xarch_host", flag]


def asan_runtime() -> str:
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise SystemExit("clang's AddressSanitizer runtime (libclang_rt.asan-x86_64.so) not found under /opt/rocm/llvm")
    return found[-1]


def instrumented(lib: str) -> bool:
    """The library calls into both sanitizers' runtimes."""
    out = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True, check=True).stdout
    return "__asan_report" in out and "__ubsan_handle" in out


# A read past the end of a buffer handed to the sanitized oracle: the run must
# end with AddressSanitizer's report, which shows that the runtime is live in a
# process set up as the suite's is.
CONTROL = """
import ctypes, numpy as np
from oracle import oracle
lib = ctypes.CDLL(oracle.LIBRARY)
a = np.zeros(8); b = np.zeros(8)
lib.oracle_round_bf16(a.ctypes.data_as(ctypes.c_void_p), b.ctypes.data_as(ctypes.c_void_p), ctypes.c_int64(9))
print("control: no report")
"""


def main(argv) -> int:
    from routed_expert_ffn_flint_amd import build

    tmp = tempfile.mkdtemp(prefix="flint_sanitize_")
    try:
        lib = build.build(extra_flags=SAN_HOST_FLAGS, lib=os.path.join(tmp, "libflint_moe.so"))
        env = dict(os.environ)
        env["FLINT_SANITIZE_DIR"] = tmp
        # the oracle is built by its loader in the same directory (clang, both sanitizers)
        r = subprocess.run([sys.executable, "-c", "from oracle import oracle; oracle.build()"], cwd=ROOT, env=env)
        if r.returncode:
            return r.returncode
        for path in (lib, os.path.join(tmp, "liboracle.so")):
            if not instrumented(path):
                print(f"{path}: no sanitizer calls in the build", file=sys.stderr)
                return 1
        env["LD_PRELOAD"] = asan_runtime()
        env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:detect_odr_violation=0"
        env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
        r = subprocess.run([sys.executable, "-c", CONTROL], cwd=ROOT, env=env, capture_output=True, text=True)
        if r.returncode == 0 or "heap-buffer-overflow" not in r.stderr:
            print("sanitizer control: an overflow went unreported\n" + r.stdout + r.stderr[-2000:], file=sys.stderr)
            return 1
        print("sanitizer control: overflow reported as expected", flush=True)
        cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-m", "not gpu", "-q", "-x",
               "-p", "no:cacheprovider"] + list(argv)
        print("FLINT_SANITIZE_DIR=%s LD_PRELOAD=%s %s" % (tmp, env["LD_PRELOAD"], " ".join(cmd)), flush=True)
        return subprocess.run(cmd, cwd=ROOT, env=env).returncode
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))

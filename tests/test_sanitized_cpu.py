"""The CPU parts under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle and the input generator (plain C) and the host code of the
library -- above all the host pass's thread pool and its vector kernels --
are rebuilt with clang's ASan + UBSan (UBSan without recovery: the first
report aborts), and the rest of the CPU suite is run against those builds in
a child process with the sanitizer runtime preloaded (the interpreter itself
is not instrumented).  The run must pass and print no sanitizer report.
Device code is not sanitized (no GPU is used here).
"""
import os
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g",
       "-shared-libasan"]


def _clang_so(src, out, extra):
    subprocess.check_call([CLANG, "-O1", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off"] + SAN + extra +
                          ["-o", out, src, "-lm"])


def test_cpu_suite_clean_under_asan_and_ubsan():
    runtime = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True,
                             check=True).stdout.strip()
    assert os.path.exists(runtime), runtime
    from expert_vram_slot_amd import build as b
    slot_lib = b.build(sanitize=True)
    with tempfile.TemporaryDirectory() as d:
        orc = os.path.join(d, "liboracle_san.so")
        syn = os.path.join(d, "libsynth_san.so")
        _clang_so(os.path.join(ROOT, "oracle", "oracle.c"), orc, [])
        _clang_so(os.path.join(ROOT, "synth", "synth.c"), syn, ["-mf16c", "-lpthread"])
        env = dict(os.environ, LD_PRELOAD=runtime, MOE_SLOT_LIB=slot_lib, MOE_ORACLE_LIB=orc, MOE_SYNTH_LIB=syn,
                   ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:allocator_may_return_null=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", PYTHONDONTWRITEBYTECODE="1")
        # everything on the CPU except this test and the mutation test (which builds oracles of its own)
        cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-m", "not gpu", "-x", "-q",
               "-p", "no:cacheprovider", "-k", "not sanitized and not mutations"]
        r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
        # the set-up itself catches a planted heap overflow and a planted signed overflow
        probe = os.path.join(d, "probe.c")
        with open(probe, "w") as f:
            f.write("#include <stdlib.h>\n"
                    "int heap_overflow(int n) { int* p = malloc(n * sizeof(int)); int v = p[n]; free(p); return v; }\n"
                    "int add_overflow(int a) { return a + 2147483647; }\n")
        so = os.path.join(d, "libprobe.so")
        _clang_so(probe, so, [])
        for fn, arg in (("heap_overflow", 4), ("add_overflow", 5)):
            pr = subprocess.run([sys.executable, "-c", f"import ctypes; ctypes.CDLL({so!r}).{fn}({arg})"], env=env,
                                capture_output=True, text=True, timeout=120)
            assert pr.returncode != 0 and ("AddressSanitizer" in pr.stderr or "runtime error" in pr.stderr), pr.stderr
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    for marker in ("ERROR: AddressSanitizer", "runtime error:", "SUMMARY: UndefinedBehaviorSanitizer"):
        assert marker not in out, out[-4000:]
    assert " passed" in out

"""The host-side C/C++ code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only; the GPU code is not built here).

* The library's planner (plan.cpp), its argument checks (validate.cpp) and its
  plan-cache policy, driven by tests/native/plan_check.cpp over 400 random
  lists (one in a hundred a 10,000-tensor list of log-uniform lengths),
  invalid lists and the cache's capture-pinning scenarios.
* The oracle (oracle/adamw_oracle.c), driven by tests/native/oracle_check.c
  over every exported function at lengths 0-70 and longer, every 16-bit
  pattern, and step indices up to 2^40.

Each driver is also built without sanitizers at the optimisation level the
code ships with; both builds must print the same checksum of everything they
computed.
"""
import os
import subprocess

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "adamw_optimizer_step_apply_amd", "csrc")
NATIVE = os.path.join(ROOT, "tests", "native")
SAN = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _build_and_run(cmd, exe, word):
    subprocess.run(cmd + ["-o", exe], check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, f"{os.path.basename(exe)} failed ({r.returncode}):\n{r.stdout}\n{r.stderr[-4000:]}"
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    line = [ln for ln in r.stdout.splitlines() if ln.startswith(word)]
    assert line and line[0].split()[1] == "ok", r.stdout
    return line[0].split()[2]


def test_planner_and_checks_under_sanitizers(tmp_path):
    srcs = [os.path.join(NATIVE, "plan_check.cpp"), os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "validate.cpp")]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    base = ["g++", "-std=c++17", "-Wall", "-Wextra", *inc]
    with_san = _build_and_run(base + SAN + srcs, str(tmp_path / "plan_check_san"), "plan_check")
    plain = _build_and_run(base + ["-O3"] + srcs, str(tmp_path / "plan_check"), "plan_check")
    assert with_san == plain


def test_oracle_under_sanitizers(tmp_path):
    srcs = [os.path.join(NATIVE, "oracle_check.c"), os.path.join(ROOT, "oracle", "adamw_oracle.c")]
    # the oracle's own arithmetic flags, without the shared-library ones
    flags = [f for f in oracle.CFLAGS if f not in ("-shared", "-fPIC")]
    base = ["gcc", "-Wall", "-Wextra", *flags]
    with_san = _build_and_run(base + SAN + srcs + ["-lm"], str(tmp_path / "oracle_check_san"), "oracle_check")
    plain = _build_and_run(base + srcs + ["-lm"], str(tmp_path / "oracle_check"), "oracle_check")
    assert with_san == plain


@pytest.mark.parametrize("planted", ["overflow", "ub"])
def test_sanitizers_catch_a_planted_fault(tmp_path, planted):
    """The sanitizer build reports a one-past-the-end read and a signed overflow
    in host code (so a clean run above means something)."""
    src = tmp_path / "planted.c"
    src.write_text(
        "#include <stdlib.h>\n#include <limits.h>\n"
        "int main(int argc, char** argv) { (void)argv;\n"
        "  int* a = malloc(4 * sizeof(int)); for (int i = 0; i < 4; ++i) a[i] = i;\n"
        + ("  int r = a[argc + 3];\n" if planted == "overflow" else "  int r = INT_MAX - 1 + argc * 2;\n")
        + "  free(a); return r == 12345; }\n")
    exe = str(tmp_path / "planted")
    subprocess.run(["gcc", *SAN, str(src), "-o", exe], check=True, capture_output=True)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=60)
    assert r.returncode != 0
    # the one-past-the-end read is reported by UBSan's object-size check or by ASan
    want = ("heap-buffer-overflow", "insufficient space") if planted == "overflow" else ("signed integer overflow",)
    assert any(w in r.stderr for w in want), r.stderr[-2000:]

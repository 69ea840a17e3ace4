"""The C-ABI from a plain C program: include/chunkkv.h compiles as strict C99
and as C++, and tests/c_consumer.c (no Python, no torch: HIP runtime
allocation and copies only) plans, is refused on invalid problems (CPU) and
compresses a two-layer problem that the oracle confirms (GPU)."""
import os
import subprocess

import pytest

import __graft_entry__ as entry

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_consumer.c")


def _consumer() -> str:
    exe = entry.C_CONSUMER
    if not os.path.exists(exe) or os.path.getmtime(exe) < os.path.getmtime(SRC):
        entry.build_c_consumer()
    return exe


@pytest.mark.parametrize("compiler,flags", [
    ("gcc", ["-x", "c", "-std=c99", "-pedantic"]),
    ("g++", ["-x", "c++", "-std=c++11", "-pedantic"]),
])
def test_header_is_plain_c_and_cpp(compiler, flags):
    src = '#include "chunkkv.h"\nint main(void) { chunkkv_problem p; (void)p; return CHUNKKV_OK; }\n'
    r = subprocess.run([compiler, *flags, "-Wall", "-Wextra", "-Werror", "-fsyntax-only",
                        "-I", os.path.join(ROOT, "include"), "-"], input=src, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_c_consumer_plans_and_validates():
    r = subprocess.run([_consumer(), "plan"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout


@pytest.mark.gpu
def test_c_consumer_compresses_like_the_oracle():
    exe = entry.C_CONSUMER
    assert os.path.exists(exe), "tests/c_consumer is built by __graft_entry__.build()"
    r = subprocess.run([exe, "run"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout

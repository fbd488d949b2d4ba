"""The oracle's C code under AddressSanitizer and UBSan (host code only).

The oracle is built with -fsanitize=address,undefined (every finding fatal)
and the oracle pins (tests/test_oracle_pins.py) run in a child process that
loads that build (DLM_ORACLE_LIB) with the sanitizer runtimes preloaded.
An out-of-bounds access, a use after free or undefined behaviour anywhere
the pins reach aborts the child, and this test fails.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_pass_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = oracle.build(force=True, sanitize=True, out=str(tmp_path / "libdlm_oracle_san.so"))
    env = dict(os.environ)
    # the sanitizer runtimes go first; anything already preloaded stays
    env["LD_PRELOAD"] = " ".join(x for x in (asan, ubsan, os.environ.get("LD_PRELOAD", "")) if x)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["DLM_ORACLE_LIB"] = lib
    probe = subprocess.run([sys.executable, "-c", "import oracle; oracle.num_threads(); print(oracle.library_path())"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0, probe.stderr[-2000:]
    assert probe.stdout.strip() == lib
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr


def test_the_sanitizer_build_catches_a_planted_overflow(tmp_path):
    """A heap overflow planted in a private copy of the oracle source aborts
    the child process that calls it: the leg above can fail."""
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc sanitizer runtimes not installed")
    with open(os.path.join(ROOT, "oracle", "dlm_oracle.c")) as f:
        src = f.read()
    marker = "int ora_num_threads(void)\n{"
    assert marker in src
    planted = src.replace(marker, marker + "\n    { int *p = (int *)malloc(4 * sizeof(int)); volatile int i = 4;"
                                           " p[i] = 1; free(p); }", 1)
    if "#include <stdlib.h>" not in planted:
        planted = "#include <stdlib.h>\n" + planted
    c = tmp_path / "planted.c"
    c.write_text(planted)
    lib = tmp_path / "libplanted.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", *oracle.SANITIZE_FLAGS,
                    str(c), "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ)
    env["LD_PRELOAD"] = " ".join(x for x in (asan, ubsan, os.environ.get("LD_PRELOAD", "")) if x)
    env["ASAN_OPTIONS"] = "detect_leaks=0"
    env["DLM_ORACLE_LIB"] = str(lib)
    r = subprocess.run([sys.executable, "-c", "import oracle; oracle.num_threads()"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    # UBSan's object-size check or ASan's redzone, whichever fires first
    assert "heap-buffer-overflow" in r.stderr or "runtime error: store" in r.stderr

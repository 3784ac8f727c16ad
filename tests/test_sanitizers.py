"""The CPU-side native code under AddressSanitizer and UndefinedBehaviorSanitizer.

The fp64 oracle (oracle/oracle.c), the seeded generator (synth/synth.c) and
the CPU replay of the kernels' data flow (tests/emu/qgemm_emu.cpp) are built
with clang's -fsanitize=address,undefined (errors fatal) into a temporary
folder, and the tests that exercise them (oracle pins, generator, replays of
the streaming, row-tiled and pass kernels) run again in a child process that
loads those builds (QG_ORACLE_LIB, QG_SYNTH_LIB, QG_EMU_LIB) with the ASan
runtime preloaded.  Host code only: nothing here touches a GPU.  A planted heap
overflow in a throwaway library shows that the set-up reports such errors.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-shared-libasan", "-fPIC", "-shared"]

pytestmark = pytest.mark.skipif(not os.path.exists(CLANG), reason="clang of the ROCm toolchain not found")


def _asan_runtime() -> str:
    return subprocess.check_output([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], text=True).strip()


def _env(libs: dict) -> dict:
    env = dict(os.environ)
    env.update(LD_PRELOAD=_asan_runtime(), PYTHONMALLOC="malloc",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", **libs)
    return env


@pytest.fixture(scope="module")
def san_libs(tmp_path_factory):
    d = tmp_path_factory.mktemp("san")
    libs = {"QG_ORACLE_LIB": str(d / "liboracle.so"), "QG_SYNTH_LIB": str(d / "libsynth.so"),
            "QG_EMU_LIB": str(d / "libqgemm_emu.so")}
    subprocess.check_call([CLANG, *SAN, "-std=c11", "-ffp-contract=off", os.path.join(ROOT, "oracle", "oracle.c"),
                           "-o", libs["QG_ORACLE_LIB"], "-lm", "-lpthread"])
    subprocess.check_call([CLANG, *SAN, "-std=c11", os.path.join(ROOT, "synth", "synth.c"),
                           "-o", libs["QG_SYNTH_LIB"], "-lm", "-lpthread"])
    subprocess.check_call([CLANG + "++", *SAN, "-std=c++17", "-ffp-contract=off",
                           os.path.join(ROOT, "tests", "emu", "qgemm_emu.cpp"), "-o", libs["QG_EMU_LIB"]])
    return libs


def test_instrumented_builds_are_the_ones_loaded(san_libs):
    code = ("import oracle, synth; from tests import emu; oracle.get(); synth.mix64(1); emu.lib(); "
            "maps = open('/proc/self/maps').read(); "
            "print(all(p in maps for p in %r), 'asan' in maps)" % (list(san_libs.values()),))
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=_env(san_libs), capture_output=True, text=True,
                         timeout=300)
    assert out.returncode == 0, out.stderr[-3000:]
    assert out.stdout.split() == ["True", "True"], out.stdout


def test_oracle_generator_and_replays_are_clean(san_libs):
    files = ["tests/test_oracle_pins.py", "tests/test_synth.py", "tests/test_pass_schedule.py",
             "tests/test_emulation.py"]
    out = subprocess.run([sys.executable, "-m", "pytest", *files, "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider"],
                         cwd=ROOT, env=_env(san_libs), capture_output=True, text=True, timeout=1500)
    tail = (out.stdout + out.stderr)[-4000:]
    assert out.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail


def test_a_planted_overflow_is_reported(tmp_path, san_libs):
    src = tmp_path / "planted.c"
    src.write_text("#include <stdlib.h>\n"
                   "unsigned planted(int n) { unsigned* a = calloc(n, sizeof(unsigned)); unsigned s = 0;\n"
                   "  for (int i = 0; i <= n; ++i) s += a[i];   /* one past the end */\n"
                   "  free(a); return s; }\n")
    so = tmp_path / "libplanted.so"
    subprocess.check_call([CLANG, *SAN, "-std=c11", str(src), "-o", str(so)])
    code = f"import ctypes; ctypes.CDLL({str(so)!r}).planted(16)"
    out = subprocess.run([sys.executable, "-c", code], env=_env(san_libs), capture_output=True, text=True, timeout=120)
    assert out.returncode != 0
    assert "heap-buffer-overflow" in out.stderr

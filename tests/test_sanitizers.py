"""Host code under sanitizers: the oracle (oracle/oracle.c) and the library's
host NVFP4 encoder (csrc/codec_host.cpp) are built with gcc/g++ and
AddressSanitizer + UndefinedBehaviorSanitizer (leak checks on), and again with
ThreadSanitizer (both split work over threads), and run through drivers that
call every entry point on seeded inputs, edge cases and error paths
(tests/sanitize/).  A report from any sanitizer fails the test.  The drivers
link one side each: the oracle and the library are never built together."""
import os
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
SAN = Path(__file__).resolve().parent / "sanitize"

TARGETS = {
    "oracle": ("gcc", ["-std=c11"], [SAN / "oracle_driver.c", ROOT / "oracle" / "oracle.c"], ["-lm"]),
    "codec": ("g++", ["-std=c++17"],
              [SAN / "codec_driver.cpp", ROOT / "nvfp4_bit_projection_amd" / "csrc" / "codec_host.cpp"], []),
}
MODES = {
    "asan_ubsan": ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"],
    "tsan": ["-fsanitize=thread"],
}
ENV = {
    "ASAN_OPTIONS": "detect_leaks=1:halt_on_error=1:abort_on_error=0:verify_asan_link_order=0",
    "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    "TSAN_OPTIONS": "halt_on_error=1:exitcode=66",
}


def _sanitizer_available(cc: str, flags: list, tmp: Path) -> bool:
    src = tmp / "probe.c"
    src.write_text("int main(void) { return 0; }\n")
    r = subprocess.run([cc, *flags, "-x", "c", str(src), "-o", str(tmp / "probe")], capture_output=True)
    return r.returncode == 0


@pytest.mark.parametrize("mode", sorted(MODES))
@pytest.mark.parametrize("target", sorted(TARGETS))
def test_host_code_under_sanitizer(target, mode, tmp_path):
    cc, std, srcs, libs = TARGETS[target]
    if shutil.which(cc) is None:
        pytest.skip(f"{cc} not found")
    if not _sanitizer_available(cc, MODES[mode], tmp_path):
        pytest.skip(f"{cc} has no {mode} runtime")
    exe = tmp_path / f"{target}_{mode}"
    build = subprocess.run([cc, *std, "-O1", "-g", *MODES[mode], *map(str, srcs), "-o", str(exe), *libs,
                            "-pthread"], capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-4000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env={**os.environ, **ENV})
    report = run.stderr
    assert run.returncode == 0, report[-4000:]
    for marker in ("ERROR: AddressSanitizer", "ERROR: LeakSanitizer", "runtime error:",
                   "WARNING: ThreadSanitizer"):
        assert marker not in report, report[-4000:]
    assert "all checks passed" in run.stdout

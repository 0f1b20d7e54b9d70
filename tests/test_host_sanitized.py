"""The library's host code (argument validation, workspace sizing and launch set-up in
kda_api.hip and the launchers) under AddressSanitizer and UndefinedBehaviorSanitizer, on the
CPU: every source is compiled with the sanitizers on its host side only (-Xarch_host), linked
with tests/host_abi_harness.c, and run with every GPU hidden.  The harness calls each entry
point with exactly-sized host arrays (ragged and empty sequences, 3000 sequences, pools,
prologues, invalid arguments) and checks each status; calls that pass validation stop at their
first launch, which fails with no device visible."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_49_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["kda_api.hip", "kda_chunk.hip", "kda_chunk32.hip", "kda_segments.hip", "kda_decode.hip", "kda_bwd.hip"]
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]


@pytest.mark.timeout(600)
def test_library_host_code_clean_under_sanitizers(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + CSRC]

    def compile_one(src):
        obj = str(tmp_path / (src + ".o"))
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + SAN + inc + \
              ["-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return obj

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    exe = str(tmp_path / "harness")
    cmd = [HIPCC, "--offload-arch=gfx950"] + SAN[:4] + inc + ["-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__",
                                                             "-x", "c", os.path.join(ROOT, "tests", "host_abi_harness.c"),
                                                             "-x", "none"] + objs + ["-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    # the sanitizer runtime is really linked into the library code under test
    nm = shutil.which("nm")
    if nm:
        syms = subprocess.run([nm, objs[0]], capture_output=True, text=True).stdout
        assert "__asan_report" in syms and "__ubsan_handle" in syms
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    if r.returncode == 77:
        pytest.skip("a GPU is visible: the harness passes fake device pointers and does not run")
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "0 failure(s)" in r.stdout

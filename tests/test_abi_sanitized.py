"""The C ABI's host-side tests (tests/test_abi.py) against a build whose host
code runs under AddressSanitizer and UndefinedBehaviorSanitizer: argument
validation, overlap and alignment checks, workspace plans, the fp64 RoPE
table and the adaptive tile table must neither read nor write out of bounds
nor hit undefined behaviour.  CPU only: the sanitized library is loaded into
a fresh process that never touches a GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_host_code_under_asan_and_ubsan():
    from joint_video_audio_rope_amd import build_sanitized as S
    try:
        lib = S.build()
        runtime = S.asan_runtime()
    except (RuntimeError, OSError, subprocess.CalledProcessError) as e:
        pytest.skip("sanitized build unavailable: %s" % e)
    code = ("import sys; sys.path.insert(0, %r); sys.path.insert(0, %r)\n"
            "import joint_video_audio_rope_amd._lib as L\n"
            "L.LIB_PATH = %r\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-x', '-m', 'not gpu', '-p', 'no:cacheprovider', %r]))\n"
            % (ROOT, os.path.join(ROOT, "tests"), lib, os.path.join(ROOT, "tests", "test_abi.py")))
    env = dict(os.environ)
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = runtime + ((" " + pre) if pre else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    p = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=600)
    print(p.stdout[-3000:])
    assert p.returncode == 0, p.stdout[-3000:]
    assert "passed" in p.stdout and "ERROR: AddressSanitizer" not in p.stdout and "runtime error" not in p.stdout

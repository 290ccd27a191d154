"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer: every
entry point on exactly-sized buffers (ragged lengths, all widths and block
sizes, both input types), see oracle_sanitize_check.c.  Host code only; the
oracle is built with the same numerics flags as its library build."""
import os
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_oracle_clean_under_address_and_ub_sanitizers():
    import oracle
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "oracle_sanitize")
        cmd = ["gcc", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
               "-fno-omit-frame-pointer", "-o", exe,
               os.path.join(HERE, "oracle_sanitize_check.c"),
               os.path.join(ROOT, "oracle", "lowbit_oracle.c"), "-lm"]
        try:
            subprocess.check_call(cmd)
        except (OSError, subprocess.CalledProcessError) as err:
            pytest.skip(f"sanitizer build unavailable here: {err}")
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1")
        r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), r.stdout + r.stderr
    del oracle

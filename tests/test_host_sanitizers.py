"""The C ABI's host-side validation and launch set-up, run under
AddressSanitizer and UndefinedBehaviorSanitizer: the ABI tests (every
rejection path, the size and workspace queries, the binding's buffer
checks) run in a fresh Python process against the host-sanitized build of
the library, with the sanitizer runtime preloaded. Any sanitizer report
aborts that process. CPU only."""
import os
import subprocess
import sys

import pytest

from microscaling_quantized_convolution_mxq_amd import build as b
from microscaling_quantized_convolution_mxq_amd import build_sanitize as san

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(not san.runtime(), reason="clang AddressSanitizer runtime not installed")
def test_abi_validation_under_host_sanitizers():
    if not os.path.exists(b.LIB):
        pytest.skip("libmqconv.so is not built")
    lib = san.build()
    env = dict(os.environ)
    env.update(LD_PRELOAD=san.runtime(), MQCONV_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the process maps the sanitizer runtime and the sanitized library
    maps = subprocess.run([sys.executable, "-c", "import microscaling_quantized_convolution_mxq_amd as mq; mq.lib(); "
                           "print(open('/proc/self/maps').read())"],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert maps.returncode == 0, maps.stderr[-2000:]
    assert "libclang_rt.asan" in maps.stdout and lib in maps.stdout
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out and "skipped" not in out, out[-2000:]

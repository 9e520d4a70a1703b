"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The packing and argument-validation tests of test_lib_host.py run again in a
child process against the host-sanitizer build of the library (the build
script's --sanitize mode: every -fsanitize goes to the host compilation only),
with the toolchain's shared sanitizer runtime preloaded. Any report ends the
child at once (halt_on_error, no recovery), so a clean pass means that the
host paths those tests drive (quantisation and packing of every format,
ragged shapes, expert strides, the validation of every entry point) made no
out-of-bounds or use-after-free access and hit no undefined behaviour (signed
overflow, misaligned or null access, bad shifts). CPU only: no kernel runs.
The instrumented build is cached under _build/san and redone when a source
changes."""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _sources_hash():
    h = hashlib.sha256()
    for d in ("bit_quantized_weight_amd/csrc", "include"):
        for name in sorted(os.listdir(os.path.join(ROOT, d))):
            with open(os.path.join(ROOT, d, name), "rb") as f:
                h.update(name.encode() + f.read())
    with open(os.path.join(ROOT, "bit_quantized_weight_amd", "build.py"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()


def test_host_code_under_sanitizers():
    sys.path.insert(0, ROOT)
    from bit_quantized_weight_amd import build as B
    try:
        B._hipcc()
    except RuntimeError:
        pytest.skip("no HIP toolchain")
    rt = B.sanitizer_runtime()
    if not rt or not os.path.exists(rt):
        pytest.skip("the toolchain has no shared AddressSanitizer runtime")
    stamp = os.path.join(B.SAN_DIR, "sources.sha256")
    want = _sources_hash()
    have = open(stamp).read() if os.path.exists(stamp) else ""
    if have != want or not os.path.exists(B.SAN_LIB):
        r = subprocess.run([sys.executable, "-m", "bit_quantized_weight_amd.build", "--sanitize"], cwd=ROOT,
                           capture_output=True, text=True, timeout=1200)
        assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
        with open(stamp, "w") as f:
            f.write(want)
    env = dict(os.environ, QGEMV_LIB=B.SAN_LIB, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_lib_host.py", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out and " failed" not in out, out[-2000:]

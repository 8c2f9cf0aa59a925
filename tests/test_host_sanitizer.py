"""The library's host code -- argument checks, workspace carving, launch
set-up -- under AddressSanitizer and UndefinedBehaviorSanitizer: the
sanitized build (host code instrumented, GPU code as usual) runs the CPU ABI
tests in a child process with the sanitizer runtime preloaded.  No GPU is
touched: every ABI test stops at the host checks."""
import os
import subprocess
import sys

import pytest

from long_context_hybrid_kv_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not found")

LOADED = """
from long_context_hybrid_kv_amd import _lib as L
L.lib()
maps = open('/proc/self/maps').read()
assert 'libhsa_attn_san.so' in maps, 'sanitized library not loaded'
assert 'libclang_rt.asan' in maps, 'sanitizer runtime not loaded'
assert 'libhsa_attn.so' not in maps, 'the plain library was loaded too'
print('sanitized build loaded')
"""


def test_abi_checks_under_host_sanitizers():
    lib = B.build(verbose=False, sanitize=True)
    env = dict(os.environ, LD_PRELOAD=B.sanitizer_runtime(), HSA_ATTN_LIB=lib,
               # leaks: the interpreter's own; the other two concern libraries
               # built without the sanitizer that share the process
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:detect_odr_violation=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", LOADED], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0 and "sanitized build loaded" in r.stdout, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join("tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out

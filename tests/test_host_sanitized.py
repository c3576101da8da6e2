"""The host code of libmoe under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU): the library built with the sanitizers on its host compilation
(expert_offload_amd.build.build(sanitize=True); rebuilt here when a source
is newer), then the host-side tests (exports, packing, errors, the AVX-512
and plain host executor) run in a child interpreter with the ASan runtime
preloaded.  Any sanitizer report fails the child."""
import glob
import os
import subprocess
import sys

from expert_offload_amd import build as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _stale() -> bool:
    if not os.path.exists(b.ASAN_LIB_PATH):
        return True
    t = os.path.getmtime(b.ASAN_LIB_PATH)
    srcs = b.sources() + glob.glob(os.path.join(b.CSRC, "*.h")) + glob.glob(os.path.join(ROOT, "include", "*.h"))
    return any(os.path.getmtime(s) > t for s in srcs)


def test_host_code_under_asan_and_ubsan():
    if _stale():
        b.build(sanitize=True)
    env = dict(os.environ)
    env["LD_PRELOAD"] = b.asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["MOE_LIB_PATH"] = b.ASAN_LIB_PATH
    p = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_lib_host.py"),
                        os.path.join(ROOT, "tests", "test_host_executor.py")],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    assert p.returncode == 0, p.stdout[-4000:]
    assert "AddressSanitizer" not in p.stdout and "runtime error" not in p.stdout, p.stdout[-4000:]

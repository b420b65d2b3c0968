"""The library's host code under AddressSanitizer (CPU only): a build with
-fsanitize=address on the host side runs the C ABI tests (argument checks,
option defaults, workspace sizing, tile-table queries, probe argument checks)
in a child process with the sanitizer runtime preloaded; any sanitizer report
fails the child."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_code_is_clean_under_asan():
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import asan_host_build

    lib = asan_host_build.build()
    env = dict(os.environ)
    env["RPA_LIBRARY"] = lib
    env["LD_PRELOAD"] = asan_host_build.runtime()
    # Python's own allocations are not instrumented; leaks at interpreter exit
    # are not the library's.
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=66"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert "AddressSanitizer" not in r.stderr + r.stdout, (r.stdout[-4000:] + r.stderr[-4000:])
    assert r.returncode == 0, (r.stdout[-4000:] + r.stderr[-4000:])

"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer: the library is rebuilt
with both sanitizers on its host code (post_quantization_mean_amd/build.py --sanitize; device code
unchanged) and the CPU ABI and binding tests run against it in a child process with the sanitizer
runtime preloaded. Any report (out-of-bounds access, signed overflow, misaligned access, ...) fails
the test. No GPU is needed: those tests only reach the host-side argument checks."""
import glob
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.timeout(600)
def test_abi_host_code_is_clean_under_asan_and_ubsan():
    rt = _asan_runtime()
    if rt is None or not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("no hipcc or clang sanitizer runtime")
    from post_quantization_mean_amd import build as bld

    lib = bld.build(sanitize=True)
    with tempfile.TemporaryDirectory() as logs:
        env = dict(os.environ)
        env["LD_PRELOAD"] = rt + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
        env["ASAN_OPTIONS"] = f"detect_leaks=0:log_path={logs}/asan"
        env["UBSAN_OPTIONS"] = f"print_stacktrace=1:halt_on_error=1:log_path={logs}/ubsan"
        code = ("import sys; sys.path.insert(0, %r)\n"
                "from post_quantization_mean_amd import binding as b\n"
                "b.load_library(%r)\n"
                "import pytest\n"
                "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', '-m', 'not gpu',"
                " 'tests/test_abi_cpu.py', 'tests/test_binding_cpu.py']))\n") % (ROOT, lib)
        r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                           timeout=500)
        logged = ""
        for f in sorted(glob.glob(os.path.join(logs, "*"))):
            logged += open(f, encoding="utf-8", errors="replace").read()
        # error reports fail the test; the runtime's own warnings (e.g. about format strings it does
        # not parse in the interpreter's printf calls) do not
        errors = "ERROR: AddressSanitizer" in logged or "runtime error:" in logged
        assert r.returncode == 0 and not errors, (r.stdout[-3000:] + r.stderr[-3000:] + logged[:6000])
        assert "passed" in r.stdout

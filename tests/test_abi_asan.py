"""The C ABI's host code under AddressSanitizer: the CPU ABI tests (every exported symbol,
the parameter struct layout, every host-checked error of every entry point, and the binding's
shape checks) run again in a child process that loads the library build whose host code is
instrumented (build.py's libskv_asan.so) with the ASan runtime preloaded. Any invalid host
memory access in validation or dispatch aborts the child and fails this test. No kernel is
launched on these paths."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _builder():
    spec = importlib.util.spec_from_file_location(
        "skv_build", os.path.join(ROOT, "streaming_kv_cache_write_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_host_abi_checks_under_asan():
    bld = _builder()
    assert os.path.exists(bld.ASAN_LIB), f"{bld.ASAN_LIB} missing: run build.py"
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": bld.asan_runtime(),
        "SKV_LIBRARY": bld.ASAN_LIB,
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1:allocator_may_return_null=1",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        "tests/test_abi.py", "tests/test_binding_shapes.py",
                        "-k", "not params_struct_layout"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out


def test_asan_build_is_instrumented():
    bld = _builder()
    syms = subprocess.run(["nm", "-D", bld.ASAN_LIB], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms or "__asan_init" in syms

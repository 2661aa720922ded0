"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The oracle, built with gcc's -fsanitize=address,undefined, runs every pin of
  ``test_oracle_pins``.
* libdsa, built with the sanitizers on its host pass only (device code is
  unchanged and never runs here), runs every check of ``test_abi_cpu``: the
  argument checks, workspace sizing, status strings and the timing session.

Each run is a child process with the sanitizer runtime preloaded (Python
itself is not instrumented); any report ends the child with a non-zero
status and the report in its output.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_CHILD = """
import sys
sys.path.insert(0, {root!r})
import {module} as M
M.LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main(["-q", "-x", "-s", "-p", "no:cacheprovider", "-m", "not gpu", {tests!r}]))
"""


def _run_child(module, lib, tests, runtime):
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime
    # the unsanitized Python and HIP runtimes free memory they did not get
    # from the instrumented allocator's point of view: leaks and odr are theirs
    env["ASAN_OPTIONS"] = "detect_leaks=0:alloc_dealloc_mismatch=0:detect_odr_violation=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    code = _CHILD.format(root=ROOT, module=module, lib=lib, tests=os.path.join(ROOT, "tests", tests))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600,
                       cwd=ROOT)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "runtime error" not in out and "AddressSanitizer" not in out, out[-6000:]
    assert " passed" in out, out[-3000:]


def test_oracle_pins_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    runtime = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(runtime) or not os.path.exists(runtime):
        pytest.skip("gcc's libasan not installed")
    import oracle
    lib = oracle.build(out=str(tmp_path / "liboracle_san.so"),
                       extra=["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                              "-fno-omit-frame-pointer", "-g"])
    _run_child("oracle", lib, "test_oracle_pins.py", runtime)


def test_library_host_code_under_sanitizers(tmp_path):
    from sparse_latent_attention_lightning_amd import build as B
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    clang = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc))), "llvm", "bin", "clang")
    if not os.path.exists(clang):
        pytest.skip("the ROCm clang is not installed")
    runtime = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                             text=True).stdout.strip()
    if not os.path.isabs(runtime) or not os.path.exists(runtime):
        pytest.skip("clang's ASan runtime not installed")
    lib = B.build(extra=B.HOST_SANITIZE_FLAGS, out=str(tmp_path / "libdsa_san.so"),
                  build_dir=str(tmp_path / "obj"))
    _run_child("sparse_latent_attention_lightning_amd._binding", lib, "test_abi_cpu.py", runtime)

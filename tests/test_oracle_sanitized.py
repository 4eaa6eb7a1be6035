"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer.

oracle/sanitize_driver.cpp calls every exported oracle function on small
cases (edge cases included) and checks the invariants that fix the results;
here it is compiled together with oracle/mage_oracle.cpp under
-fsanitize=address,undefined and run. Any out-of-bounds access, use after
free, leak or undefined arithmetic in the oracle aborts the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "oracle", "sanitize_driver.cpp"), os.path.join(ROOT, "oracle", "mage_oracle.cpp")]
FLAGS = ["-O1", "-g", "-std=c++17", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer"]


def _run(exe, leaks=True):
    env = dict(os.environ)
    # other preloaded libraries may precede the sanitizer runtime in this environment
    env["ASAN_OPTIONS"] = f"verify_asan_link_order=0:detect_leaks={1 if leaks else 0}:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["OMP_NUM_THREADS"] = "4"
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    if leaks and "LeakSanitizer has encountered a fatal error" in res.stderr:
        return _run(exe, leaks=False)   # the leak checker cannot attach in this sandbox
    return res


@pytest.fixture(scope="module")
def build_dir(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    return tmp_path_factory.mktemp("sanitized")


def test_sanitizers_are_active(build_dir):
    # a planted heap overflow in a separate program: the sanitized build must catch it
    src = build_dir / "overflow.cpp"
    src.write_text("#include <vector>\nint main(){std::vector<int> v(4); volatile int i = 4; "
                   "return v.data()[i];}\n")
    exe = str(build_dir / "overflow")
    subprocess.run(["g++", *FLAGS, "-o", exe, str(src)], check=True, capture_output=True, timeout=120)
    res = _run(exe)
    assert res.returncode != 0 and "AddressSanitizer" in res.stderr


def test_oracle_under_address_and_ub_sanitizers(build_dir):
    exe = str(build_dir / "oracle_sanitized")
    subprocess.run(["g++", *FLAGS, "-o", exe, *SRC], check=True, capture_output=True, timeout=300)
    res = _run(exe)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "ok: 0 failures" in res.stdout
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr

"""The host code under the address and undefined-behaviour sanitizers: the C ABI's validation and
workspace planning (api.cpp and plan.cpp, with launchers that report a device failure, so nothing
can be computed) and the C++ oracle are compiled with g++ -fsanitize=address,undefined, and the host
tests (argument checks, plans, oracle pins and cross-checks) run against those builds in a child
process with the sanitizer runtimes preloaded.  Any report fails the test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined"]
HOST_TESTS = ["tests/test_abi_host.py", "tests/test_oracle_pins.py", "tests/test_oracle_cpp.py",
              "tests/test_oracle_routing_pins.py", "tests/test_oracle_distill_pins.py",
              "tests/test_oracle_projection_pins.py"]


def _runtime(name):
    p = subprocess.run(["g++", f"-print-file-name={name}"], stdout=subprocess.PIPE, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(_runtime("libasan.so") is None or _runtime("libubsan.so") is None,
                    reason="g++ sanitizer runtimes not installed")
def test_host_code_under_sanitizers(tmp_path):
    csrc = os.path.join(ROOT, "cross_layer_token_amd", "csrc")
    abi = str(tmp_path / "libclsa_host_san.so")
    orc = str(tmp_path / "libclsa_oracle_san.so")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-Wall", *SAN, "-o", abi,
                    os.path.join(csrc, "api.cpp"), os.path.join(csrc, "plan.cpp"),
                    os.path.join(ROOT, "tests", "host", "launch_stubs.cpp")], check=True)
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-pthread", "-Wall", *SAN, "-o", orc,
                    os.path.join(ROOT, "oracle", "clsa_oracle.cpp")], check=True)
    env = dict(os.environ)
    env.update({"LD_PRELOAD": f"{_runtime('libasan.so')}:{_runtime('libubsan.so')}",
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
                "CLSA_TEST_SANITIZED_ABI": abi, "CLSA_TEST_SANITIZED_ORACLE": orc})
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider", "-m", "not gpu", *HOST_TESTS],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    tail = "\n".join(r.stdout.splitlines()[-30:])
    assert "AddressSanitizer" not in r.stdout and "runtime error:" not in r.stdout, tail
    assert r.returncode == 0, tail

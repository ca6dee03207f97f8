import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # tests/test_sanitizers.py re-runs the host tests against address/undefined-behaviour sanitizer
    # builds of the C ABI's host code and of the C++ oracle; these variables name those builds
    abi = os.environ.get("CLSA_TEST_SANITIZED_ABI")
    if abi:
        from cross_layer_token_amd import binding as B
        B.LIB = B._load(abi)
        B.LIB_PATH = abi
    orc = os.environ.get("CLSA_TEST_SANITIZED_ORACLE")
    if orc:
        from oracle import cpp as C
        C.LIB = C._load(orc)
        C._LIB_PATH = orc

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


# The sanitizer tests (test_sanitizers_cpu.py) rerun CPU test files in a
# child process against instrumented builds of the library and the oracle,
# named by these variables.
if os.environ.get("FA_TEST_LIBFA"):
    import tiled_attention_fa_amd._lib as _fa_lib

    _fa_lib._LIB_PATH = os.environ["FA_TEST_LIBFA"]
if os.environ.get("FA_TEST_LIBORACLE"):
    import oracle as _oracle

    _oracle._LIB = os.environ["FA_TEST_LIBORACLE"]

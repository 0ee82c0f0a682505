import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "full_coverage: full-size coverage runs (opt-in)")


FULL_COVERAGE_FILE = "test_gpu_full_coverage.py"


def pytest_addoption(parser):
    parser.addoption("--full-coverage", action="store_true", default=False,
                     help="also collect " + FULL_COVERAGE_FILE + ": whole outputs and 2,048-row "
                          "samples at full size, about 8 minutes, mostly fp64 oracle work")


def pytest_ignore_collect(collection_path, config):
    # the full-size coverage runs are collected only when asked for
    if collection_path.name == FULL_COVERAGE_FILE and not config.getoption("--full-coverage"):
        return True
    return None

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_addoption(parser):
    parser.addoption("--bimamba-lib", default=None,
                     help="load this build of libbimamba.so instead of the package's (e.g. the host-ASan build "
                          "that `python -m bidirectional_mamba_selective_amd.build --asan-host` writes)")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    lib = config.getoption("--bimamba-lib")
    if lib:
        from bidirectional_mamba_selective_amd import _lib

        _lib.LIB_PATH = os.path.abspath(lib)

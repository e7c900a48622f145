import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # use the library that is built; build it only if nothing is there
    lib = os.path.join(ROOT, "bit_quantized_fwht_amd", "libqift.so")
    if not os.path.exists(lib):
        from bit_quantized_fwht_amd.build import build
        build()

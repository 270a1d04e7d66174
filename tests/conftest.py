import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

LIB = os.path.join(ROOT, "post_weight_quantization_04_amd", "libgptq.so")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running test (tens of seconds, mostly host-side oracle work)")


def pytest_sessionstart(session):
    # The library is normally built beforehand (__graft_entry__.build()); build
    # it here only when it is missing, so that a fresh checkout can be tested.
    if not os.path.exists(LIB):
        from post_weight_quantization_04_amd import build
        build.build()

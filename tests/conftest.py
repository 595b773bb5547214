import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


# A stand-in build of the library (the host code under sanitizers, built by
# tests/test_host_sanitizers.py) replaces libpa.so when this is set.
if os.environ.get("PA_TEST_LIB"):
    import paged_kv_attention_22_amd as _pa

    _pa.LIB_PATH = os.environ["PA_TEST_LIB"]

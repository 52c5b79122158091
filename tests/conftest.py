import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    # GPU tests are selected with -m gpu and fail (not skip) where no device exists.
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Outputs, spectra and workspaces that the binding allocates for the library
# start as NaN in every test, so a kernel that reads memory it did not write
# fails parity instead of passing on stale values.
os.environ["HYENA_POISON"] = "1"
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running (large shapes)")

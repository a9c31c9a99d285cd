import os
import shutil
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")
    config.addinivalue_line("markers", "slow: full-size workload, tens of seconds")


def pytest_sessionstart(session):
    # A fresh checkout has no liblce.so (built files stay out of history): build it once, in tree,
    # when hipcc is there.  An existing build is used as it is.
    lib = os.path.join(ROOT, "vocabulary_cross_entropy_row_amd", "liblce.so")
    if not os.path.exists(lib) and (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")):
        from vocabulary_cross_entropy_row_amd import build
        build.build()

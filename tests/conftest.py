import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large-shape GPU parity case")


def announce_case(nodeid):
    """Name the GPU case about to run, before it touches the GPU: on stderr, and appended (with an
    fsync) to $MOE_TEST_LOG_DIR/gpu_test_progress.txt when that variable is set, so the case is
    known even if the process does not survive it."""
    sys.stderr.write("\nSTART %s\n" % nodeid)
    sys.stderr.flush()
    d = os.environ.get("MOE_TEST_LOG_DIR")
    if d:
        os.makedirs(d, exist_ok=True)
        with open(os.path.join(d, "gpu_test_progress.txt"), "a") as f:
            f.write("START %s\n" % nodeid)
            f.flush()
            os.fsync(f.fileno())


def progress(msg):
    """A progress line of a long GPU case (same destinations as announce_case)."""
    sys.stderr.write("  %s\n" % msg)
    sys.stderr.flush()
    d = os.environ.get("MOE_TEST_LOG_DIR")
    if d:
        os.makedirs(d, exist_ok=True)
        with open(os.path.join(d, "gpu_test_progress.txt"), "a") as f:
            f.write("  %s\n" % msg)
            f.flush()

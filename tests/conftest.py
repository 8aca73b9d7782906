import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")
    config.addinivalue_line("markers", "oracle_pool: runs the oracle in a pool of worker processes")


def pytest_collection_modifyitems(session, config, items):
    # the oracle pool is forked now, before any test touches the GPU: its workers never hold
    # GPU state and only run the numpy oracle
    if any(item.get_closest_marker("oracle_pool") for item in items):
        import parity
        parity.start_pool()


def pytest_sessionfinish(session, exitstatus):
    import parity
    parity.stop_pool()

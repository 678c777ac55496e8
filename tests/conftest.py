import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload on the GPU")
    # The full-size tests score every active row with the oracle in host worker processes.
    # The pool starts here, before any test touches the GPU, and only where GPU tests can
    # run (torch.cuda.device_count() counts devices without initialising the runtime).
    markexpr = " ".join((config.getoption("markexpr", "") or "").split())
    if "not gpu" in markexpr or "not slow" in markexpr:
        return
    import torch
    if torch.cuda.device_count() > 0:
        import helpers
        helpers.start_oracle_pool()


def pytest_unconfigure(config):
    import helpers
    helpers.stop_oracle_pool()

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


try:
    # Two hypothesis profiles.  "ci" (the default) draws the same examples on every run, so the suite's outcome
    # is reproducible; "explore" draws new examples (more of them) on every run, for searching:
    #     HYPOTHESIS_PROFILE=explore python -m pytest tests -m "not gpu" [--hypothesis-seed N]
    # (--hypothesis-seed replays one exploratory run exactly).
    from hypothesis import settings as _hyp_settings

    _hyp_settings.register_profile("ci", derandomize=True)
    _hyp_settings.register_profile("explore", derandomize=False, max_examples=300, database=None)
    _hyp_settings.load_profile(os.environ.get("HYPOTHESIS_PROFILE", "ci"))
except ImportError:  # pragma: no cover
    pass


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


@pytest.fixture(scope="session")
def require_gpu():
    if not gpu_available():
        pytest.skip("no GPU visible")

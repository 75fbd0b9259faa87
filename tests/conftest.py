import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    return oracle.load()


@pytest.fixture
def ntenv():
    """The library's tuning overrides (nt_set_override) with monkeypatch's
    setenv / delenv interface; every one touched is restored when the test
    ends."""
    import row_wise_reductions_amd as nt
    touched = set()

    class _Overrides:
        def setenv(self, name, value):
            touched.add(name)
            nt.set_override(name, value)

        def delenv(self, name, raising=True):
            touched.add(name)
            nt.set_override(name, None)

    yield _Overrides()
    for name in touched:
        nt.set_override(name, None)

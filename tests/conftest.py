import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: oracle cases that take more than a few seconds on the CPU")


@pytest.fixture
def rgt_env():
    """Set RGT_* environment settings for one test: rgt_env(NAME=value, ...)
    (None removes one). The library reads them only at its first call and on
    reload_env, so each change is followed by a reload, and the settings are
    restored (and reloaded) when the test ends."""
    saved = {}

    def reload():
        import router_gemv_top_amd as R
        R.reload_env()

    def set_env(**kv):
        for name, value in kv.items():
            if name not in saved:
                saved[name] = os.environ.get(name)
            if value is None:
                os.environ.pop(name, None)
            else:
                os.environ[name] = str(value)
        reload()

    yield set_env
    for name, value in saved.items():
        if value is None:
            os.environ.pop(name, None)
        else:
            os.environ[name] = value
    if saved:
        reload()

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


import pytest  # noqa: E402


@pytest.fixture
def w4_settings(monkeypatch):
    """Sets or clears a W4_* settings variable and makes the library re-read
    its settings; everything is restored (and re-read) after the test."""
    import bit_weight_only_02_amd as w4

    def set_(name, value=None):
        if value is None:
            monkeypatch.delenv(name, raising=False)
        else:
            monkeypatch.setenv(name, value)
        w4.w4_reload_settings()
    yield set_
    monkeypatch.undo()
    w4.w4_reload_settings()

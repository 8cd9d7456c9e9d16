import pytest

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture
def tune():
    """Set launch-policy overrides (dec_tuning) for the rest of the test; the previous
    overrides are restored at teardown."""
    import autoregressive_audio_token_amd as dec
    before = dec.dec_tuning_get()

    def set_(**fields):
        now = dec.dec_tuning_get()
        now.update(fields)
        dec.dec_tuning_set(**now)

    yield set_
    dec.dec_tuning_set(**before)

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size workload")


@pytest.fixture
def tune():
    """Set fields of the library's tuning (gqa_tuning_t) for one test and restore the previous
    tuning afterwards: `tune(shares=7, fold=2)`."""
    import decode_attention_04_amd as gd
    saved = gd.gqa_decode_get_tuning()

    def apply(**fields):
        t = gd.gqa_decode_get_tuning()
        for name, value in fields.items():
            if name not in t.as_dict():
                raise KeyError(f"no tuning field {name!r}")
            setattr(t, name, int(value))
        gd.gqa_decode_set_tuning(t)

    yield apply
    gd.gqa_decode_set_tuning(saved)

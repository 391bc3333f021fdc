import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def hf_available():
    try:
        import transformers  # noqa: F401
        from transformers import BloomConfig, BloomForCausalLM  # noqa: F401
    except Exception as exc:  # pragma: no cover
        pytest.skip(f"transformers BLOOM not importable: {exc}")
    return True

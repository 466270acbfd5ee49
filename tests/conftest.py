import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# A host-test run against another build of the library (the sanitized one, see
# test_host_sanitizers.py) names it here.
if os.environ.get("ZDIT_TEST_LIB"):
    from diffusion_transformer_text_s3_amd import binding as _binding
    _binding.LIB_PATH = os.environ["ZDIT_TEST_LIB"]


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def golden(name):
    """Rows of a tests/golden fixture, comments stripped."""
    rows = []
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows

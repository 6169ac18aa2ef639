import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # The sanitizer test runs CPU tests against a host-only build of libengram
    # made with AddressSanitizer and UBSan (tests/test_host_sanitizers.py).
    lib = os.environ.get("ENGRAM_TEST_LIB")
    if lib:
        from hashed_gram_embedding_engram_amd import engram as B
        B.LIB_PATH = lib
        B.load_library.__defaults__ = (lib,)


def read_golden(name):
    """Parse a tests/golden fixture: '#' comment lines, then 'key v1 v2 ...' lines of integers."""
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = [int(v) for v in vals]
    return out


@pytest.fixture(scope="session")
def golden_constants():
    return read_golden("printed_constants.txt")

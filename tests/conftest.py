import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def read_golden(name):
    """Parse a `key = value` fixture under tests/golden/ (comments start with #)."""
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = (s.strip() for s in line.split("=", 1))
            parts = v.split()
            conv = []
            for p in parts:
                if p.lower().startswith("0x"):
                    conv.append(int(p, 16))
                else:
                    try:
                        conv.append(int(p))
                    except ValueError:
                        conv.append(float(p))
            vals[k] = conv[0] if len(conv) == 1 else conv
    return vals

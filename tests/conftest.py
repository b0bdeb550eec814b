import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def read_golden(name):
    """Parse a golden fixture: '#' comments, then 'key v1 v2 ...' lines.
    Values stay strings; 'block <id>' lines open a new record."""
    records = [{}]
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            if key == "block":
                if records[-1]:
                    records.append({})
                records[-1]["block"] = vals
                continue
            records[-1][key] = vals
    return records


def read_table(name):
    """Two-column golden table -> list of (str, str)."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                a, b = line.split()
                rows.append((a, b))
    return rows


def gpu_available():
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


_MEASURES = []


def record_measure(line):
    """Keep one line of achieved parity figures (errors, exempt rows, recall); the terminal
    summary prints them even under -q, so a run's log records what each gate saw."""
    _MEASURES.append(str(line))


def pytest_terminal_summary(terminalreporter):
    if _MEASURES:
        terminalreporter.section("parity measures")
        for line in _MEASURES:
            terminalreporter.write_line(line)


def gpu_visible():
    """Whether this process can see a GPU (counting devices initialises no HIP context)."""
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


def read_golden(name):
    """Parse a tests/golden fixture: '#' lines are comments, other lines are
    'tag v1 v2 ...' or plain number rows.  Returns (tagged: dict[str, list[list[float]]],
    rows: list[list[float]])."""
    tagged, rows = {}, []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            try:
                rows.append([float(x) for x in parts])
            except ValueError:
                tagged.setdefault(parts[0], []).append([float(x) for x in parts[1:]])
    return tagged, rows

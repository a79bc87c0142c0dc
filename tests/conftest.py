"""Shared pytest configuration: the ``gpu`` marker and golden-fixture readers."""

import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def golden_lines(name):
    """Non-comment, non-empty lines of a golden fixture."""
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.lstrip().startswith("#")]


def golden_grid(name):
    """A golden fixture that is one integer grid."""
    return np.array([[int(v) for v in ln.split()] for ln in golden_lines(name)], dtype=np.int64)


def golden_sections(name):
    """A fixture made of ``[section] header...`` blocks: {section: (header tokens, [lines])}."""
    out = {}
    cur = None
    for ln in golden_lines(name):
        if ln.startswith("["):
            key, _, rest = ln[1:].partition("]")
            cur = key
            out[cur] = (rest.split(), [])
        else:
            out[cur][1].append(ln)
    return out

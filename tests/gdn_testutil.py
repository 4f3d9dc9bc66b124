"""Helpers shared by the test modules: golden-fixture readers and tolerance checks."""
import os

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def golden_path(name):
    return os.path.join(ROOT, "tests", "golden", name)


def read_golden_kv(name):
    out = {}
    with open(golden_path(name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            out[key] = [float(x) for x in val.split()]
    return out


def read_golden_rows(name):
    rows = []
    with open(golden_path(name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows

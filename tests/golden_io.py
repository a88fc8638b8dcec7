"""Readers for the hand-derived fixtures in tests/golden/."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _num(tok):
    tok = tok.strip()
    if tok.lower().startswith(("0x", "-0x")) and "p" not in tok.lower():
        return int(tok, 16)
    try:
        return int(tok)
    except ValueError:
        return float.fromhex(tok) if ("p" in tok.lower()) else float(tok)


def read_table(name):
    """Rows of `value code ...` lines (comments start with #)."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip() if line.lstrip().startswith("#") else line.strip()
            if not line:
                continue
            parts = line.split()
            rows.append((float.fromhex(parts[0]) if "p" in parts[0].lower() else float(parts[0]),
                         int(parts[1], 16)))
    return rows


def read_kv(name):
    """`key v1 v2 ...` lines -> dict of lists."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            s = line.strip()
            if not s or s.startswith("#"):
                continue
            parts = s.split()
            out[parts[0]] = [_num(p) for p in parts[1:]]
    return out

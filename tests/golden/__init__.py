"""Parser for the hand-worked fixtures in this folder (syntax: see each file's header)."""
from __future__ import annotations

import os
import re

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def _floats(text: str) -> np.ndarray:
    out = []
    for tok in text.split():
        if "*" in tok:
            v, n = tok.split("*")
            out.extend([float(v)] * int(n))
        else:
            out.append(float(tok))
    return np.array(out, dtype=np.float64).astype(np.float32)


def _hexbytes(text: str) -> bytes:
    s = re.sub(r"\{([0-9a-fA-F]{2})\*(\d+)\}", lambda m: m.group(1) * int(m.group(2)), text)
    return bytes.fromhex(s.replace(" ", ""))


def load(name: str) -> dict:
    """Return {section: {key: [raw values...]}} for golden file ``name``."""
    sections: dict = {}
    cur = None
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("["):
                cur = sections.setdefault(line.strip("[]"), {})
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            cur.setdefault(key, []).append(val)
    return sections


floats = _floats
hexbytes = _hexbytes

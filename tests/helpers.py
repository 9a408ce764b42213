"""Shared test helpers: golden-file readers and the parity metric."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_table(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            vals[int(c)] = float(v)
    return vals


def read_packing_examples():
    rows = []
    with open(os.path.join(GOLDEN, "packing_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            fmt, hexbytes, vals = [p.strip() for p in line.split("|")]
            rows.append((fmt, bytes.fromhex(hexbytes), [float(v) for v in vals.split()]))
    return rows


def read_format_variants():
    """Rows of golden/format_variants.txt: (format name, code bytes, scale bytes, values)."""
    rows = []
    with open(os.path.join(GOLDEN, "format_variants.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            fmt, codes, scales, vals = [p.strip() for p in line.split("|")]
            rows.append((fmt, bytes.fromhex(codes), bytes.fromhex(scales), [float(v) for v in vals.split()]))
    return rows


def max_rel_err(y, ref):
    """Max over elements of |y - ref| / max(|ref|, tau), tau = 1e-2 * max|ref|.

    The floor keeps outputs that cancel to near zero from dominating; it is the
    parity metric for floating-point outputs (bar: 2e-3)."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    tau = 1e-2 * np.max(np.abs(ref)) if ref.size else 0.0
    if ref.size == 0:
        return 0.0
    den = np.maximum(np.abs(ref), tau if tau > 0 else 1e-300)
    return float(np.max(np.abs(y - ref) / den))


PARITY_TOL = 2e-3

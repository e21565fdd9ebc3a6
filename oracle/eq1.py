"""The chiplet cache bandwidth model -- TEST INFRASTRUCTURE ONLY.

Source: HipKittens L2 note, section 4 ("方程物理意義", the paper's single explicit
equation) and section 2 (Pillar 3):

    BW = LLC_BW * LLC_hit + L2_BW * L2_hit

with hit rates as fractions.  Table 4 (same note, section 5) prints, per grid
order, the L2 and LLC hit rates and a "Mem BW" column.  Reading that column as
this equation's output, the two constants are recovered by least squares over
the six rows; the pages state L2 bandwidth is about 3x LLC bandwidth.
"""
from __future__ import annotations

import csv
import os

import numpy as np


def model_bw(l2_hit: float, llc_hit: float, l2_bw: float, llc_bw: float) -> float:
    return llc_bw * llc_hit + l2_bw * l2_hit


def load_table4(path: str) -> list[dict]:
    rows = []
    with open(path) as f:
        for r in csv.DictReader(line for line in f if not line.startswith("#")):
            rows.append({k: (v if k in ("order",) else float(v)) for k, v in r.items()})
    return rows


def fit(rows) -> tuple[float, float]:
    """Least-squares (L2_BW, LLC_BW) in TB/s from rows with l2_pct, llc_pct, bw_tbs."""
    X = np.array([[r["l2_pct"] / 100.0, r["llc_pct"] / 100.0] for r in rows])
    y = np.array([r["bw_tbs"] for r in rows])
    (l2_bw, llc_bw), *_ = np.linalg.lstsq(X, y, rcond=None)
    return float(l2_bw), float(llc_bw)


def default_table4_path() -> str:
    here = os.path.dirname(os.path.abspath(__file__))
    return os.path.join(os.path.dirname(here), "tests", "golden", "table4_chiplet_schedule.csv")

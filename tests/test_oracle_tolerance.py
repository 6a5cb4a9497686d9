"""Pins of the oracle's error metrics (``oracle.tolerance``) by values worked out by hand.

The bf16 forward bound is 2e-2 "max relative error"; the reading taken is the maximum
over (row, head) of max_k |O - O_ref| / max_k |O_ref| (comparison with a dense float64
reference: "Stream-CQSA: Exact Out-of-Memory Recovery for Attention", abstract).  The
case below is built so that every plausible slip gives another number: the mean over
(row, head) instead of the max, one norm over a whole row (all heads), a reduction over
the wrong axis, the output's norm in the denominator, an L1 or L2 norm, a global ratio.
"""
import numpy as np
import pytest

from oracle.tolerance import error_report, grad_rel_err, max_abs_err, rowwise_rel_err

# [R=2 rows][H=2 heads][d=3]
REF = np.array([[[1.0, -2.0, 0.5], [8.0, 2.5, 1.0]],
                [[4.0, 3.0, -1.0], [0.5, 0.25, -0.5]]])
OUT = np.array([[[1.1, -2.3, 0.5], [8.0, 2.5, 1.0]],
                [[4.0, 3.0, -1.2], [0.5, 0.25, -0.45]]])
# per (row, head): max|diff| / max|ref|
#   (0,0): 0.3 / 2   = 0.15      (0,1): 0 / 8 = 0
#   (1,0): 0.2 / 4   = 0.05      (1,1): 0.05 / 0.5 = 0.1
EXPECTED = 0.15


def test_rowwise_rel_err_by_hand():
    assert rowwise_rel_err(OUT, REF) == pytest.approx(EXPECTED, rel=1e-12)


def test_slips_give_other_values():
    diff = np.abs(OUT - REF)
    per = diff.max(-1) / np.abs(REF).max(-1)
    slips = {
        "mean over (row, head)": per.mean(),                                          # 0.075
        "one norm per row": (diff.max((1, 2)) / np.abs(REF).max((1, 2))).max(),       # 0.05
        "global ratio": diff.max() / np.abs(REF).max(),                               # 0.0375
        "over rows": (diff.max(0) / np.abs(REF).max(0)).max(),                        # 0.2
        "over heads": (diff.max(1) / np.abs(REF).max(1)).max(),                       # 0.2
        "output norm": (diff.max(-1) / np.abs(OUT).max(-1)).max(),                    # 0.1304
        "L1 norm": (diff.sum(-1) / np.abs(REF).sum(-1)).max(),                        # 0.1143
        "L2 norm": (np.sqrt((diff ** 2).sum(-1)) / np.sqrt((REF ** 2).sum(-1))).max(),  # 0.138
        "min over (row, head)": per.min(),                                            # 0
    }
    for name, value in slips.items():
        assert abs(value - EXPECTED) > 5e-3, name


def test_error_report_by_hand():
    rep = error_report(OUT, REF)
    # |diff| over the 12 elements: 0.1, 0.3, 0.2, 0.05 and eight zeros
    assert rep["max_abs"] == pytest.approx(0.3, rel=1e-12)
    assert rep["mean_abs"] == pytest.approx(0.65 / 12, rel=1e-12)
    assert rep["rowwise_rel"] == pytest.approx(EXPECTED, rel=1e-12)
    assert max_abs_err(OUT, REF) == pytest.approx(0.3, rel=1e-12)


def test_grad_rel_err_floor_by_hand():
    # largest row max|ref| = 8, floor = 8 * 2^-8 = 1/32.  Row (1,1) has max|ref| 0.5 > 1/32,
    # so nothing changes with this data; a tiny row is taken against the floor
    assert grad_rel_err(OUT, REF) == pytest.approx(EXPECTED, rel=1e-12)
    ref = REF.copy()
    out = OUT.copy()
    ref[1, 1] = [0.0, 0.01, 0.0]      # max|ref| 0.01 < 1/32
    out[1, 1] = [0.0, 0.01, 0.02]     # max|diff| 0.02 -> 0.02 / (1/32) = 0.64
    assert grad_rel_err(out, ref) == pytest.approx(0.64, rel=1e-12)
    # without the floor the same row would give 0.02 / 0.01 = 2
    assert rowwise_rel_err(out, ref) == pytest.approx(2.0, rel=1e-12)


def test_empty_inputs():
    z = np.zeros((0, 2, 3))
    assert rowwise_rel_err(z, z) == 0.0
    assert max_abs_err(z, z) == 0.0

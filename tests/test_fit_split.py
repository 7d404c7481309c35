"""Host check of the sequence-split cost-model fit (no GPU): timings generated
from known constants of T = lambda1 L + lambda2 segments + lambda0 (split) and
mu1 N w + mu0 (unsplit) are fitted back exactly, and noise shows up in the
reported residuals."""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from sub_quadratic_sequence_amd import fit_split  # noqa: E402

LAM = (3.1, 0.45, 9.0)   # lambda1, lambda2, lambda0 (us)
MU = (2.6, 7.5)          # mu1, mu0 (us)


def _rows(noise=0.0, seed=0):
    rng = np.random.default_rng(seed)
    rows = []
    for units in (1, 4, 16, 64):
        for nch in (16, 64, 256, 1024):
            waves = -(-units * 2 // 256)
            t = MU[0] * nch * waves + MU[1]
            rows.append({"units": units, "T": 64 * nch, "segments": 1, "L": nch, "waves": waves,
                         "us": t * (1 + noise * rng.standard_normal())})
            for n in (2, 4, 8, 16, 64):
                if n > nch or units * n > 256:
                    continue
                L = -(-nch // n)
                ns = -(-nch // L)
                t = LAM[0] * L + LAM[1] * ns + LAM[2]
                rows.append({"units": units, "T": 64 * nch, "segments": ns, "L": L, "waves": 1,
                             "us": t * (1 + noise * rng.standard_normal())})
    return rows


def test_fit_recovers_known_constants():
    f = fit_split.fit(_rows())
    assert f["lambda1"] == pytest.approx(LAM[0], rel=1e-9)
    assert f["lambda2"] == pytest.approx(LAM[1], rel=1e-9)
    assert f["lambda0"] == pytest.approx(LAM[2], rel=1e-9)
    assert f["mu1"] == pytest.approx(MU[0], rel=1e-9)
    assert f["mu0"] == pytest.approx(MU[1], rel=1e-9)
    assert f["split_rel_residual_max"] < 1e-9 and f["unsplit_rel_residual_max"] < 1e-9
    assert f["split_samples"] > 3 and f["unsplit_samples"] > 2


def test_fit_reports_noise_in_residuals():
    f = fit_split.fit(_rows(noise=0.05, seed=3))
    assert 0.005 < f["split_rel_residual_median"] < 0.2
    assert f["lambda1"] == pytest.approx(LAM[0], rel=0.1)

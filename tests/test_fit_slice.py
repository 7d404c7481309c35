"""Host check of the d_v slice-width search (no GPU): on timings generated from
the rounds model with known constants, the search finds pairs that lose nothing
and includes the true pair, the rule's choices follow the rounds, and a
threshold rule that ignores partial rounds shows its loss."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from sub_quadratic_sequence_amd import fit_slice  # noqa: E402

NCU = 256
WIDE, PARTIAL = 1.7, 0.6
C64 = 3.0   # us per chunk of a full round of 64-column items


def _rows():
    rows = []
    for T in (512, 2048):
        for dv in (128, 256):
            for units in range(16, 700, 24):
                i128 = units * dv // 128
                nch = T // 64
                rows.append({"T": T, "dv": dv, "units": units,
                             "us64": C64 * nch * fit_slice.rounds(2 * i128, NCU, PARTIAL) + 5.0,
                             "us128": WIDE * C64 * nch * fit_slice.rounds(i128, NCU, PARTIAL) + 5.0})
    return rows


def test_rounds():
    assert fit_slice.rounds(256, 256, 0.5) == 1.0
    assert fit_slice.rounds(512, 256, 0.5) == 2.0
    assert fit_slice.rounds(64, 256, 0.5) == pytest.approx(0.5 + 0.5 * 0.25)
    assert fit_slice.rounds(300, 256, 1.0) == 2.0   # a partial round at full cost: ceil
    assert fit_slice.rounds(0, 256, 0.5) == 0.0


def test_search_recovers_the_generating_model():
    rows = _rows()
    f = fit_slice.choose(rows, NCU)
    assert f["mean_loss"] == pytest.approx(0.0, abs=1e-12)
    assert (WIDE, PARTIAL) in f["optimal_pairs_kWide_kPartial"]
    # the generated timings favour each width somewhere, and the threshold rule loses time
    picks = fit_slice.choices(rows, NCU, WIDE, PARTIAL)
    assert set(picks) == {64, 128}
    assert f["threshold_rule_losses_mean_max"][0] > 0.0


def test_choices_against_hand_counted_rounds():
    # 256 CUs, kWide 1.8, kPartial 0.5: 192 units at dv 128 take 0.875 x 1.8 = 1.575
    # rounds of 128 columns against 1.75 of 64; 288 units 2.8125 against 2.625
    rows = [{"units": 192, "dv": 128}, {"units": 288, "dv": 128}, {"units": 128, "dv": 128}]
    assert fit_slice.choices(rows, 256, 1.8, 0.5) == [128, 64, 64]

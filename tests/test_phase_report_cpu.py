"""Host logic of the phase report (no GPU): stamps of a synthetic timeline are
turned into per-phase ends, lengths and wave lags, and a phase a row skipped
is left out of that phase and bridged in the next one's length."""
import numpy as np

from stable_top_selection_amd import phase_report as P


def _stamps(rows, skip=None):
    st = np.zeros(P.STAMP_ROWS * 2 * P.SLOTS, dtype=np.uint64)
    v = st.reshape(P.STAMP_ROWS, 2, P.SLOTS)
    for r in range(rows):
        base = 10_000 * (r + 1)  # rows start at different clocks
        v[r, 0, :len(P.PHASES) + 1] = base + np.arange(len(P.PHASES) + 1) * 100
        v[r, 1, :len(P.PHASES) + 1] = base + np.arange(len(P.PHASES) + 1) * 100 + 7 * (r + 1)
    if skip is not None:
        v[skip[0], :, skip[1]] = 0
    return st


def test_even_timeline():
    res = P._summarise(P._timelines(_stamps(3), 3))
    assert len(res) == len(P.PHASES)
    for p, (n, end, length, lag) in enumerate(res):
        assert n == 3
        assert end == 100 * (p + 1) + 14  # later wave: row 1's lag 14 is the median of 7, 14, 21
        assert length == 100 or (p == 0 and length == 114)
        assert lag == 14


def test_skipped_phase_is_bridged():
    res = P._summarise(P._timelines(_stamps(3, skip=(1, 6)), 3))
    assert res[5][0] == 2  # phase 6 (index 5) passed by two rows
    assert res[6][0] == 3
    # row 1's next length spans both phases: lengths 100, 200, 100 -> median 100
    assert res[6][2] == 100


def test_start_lags():
    assert P._start_lags(_stamps(3), 3) == [7, 14, 21]

"""Host-side replay of the split decode attention's index arithmetic (CPU).

The decode kernel splits the teacher window of one query at position pos
into pieces of split_len keys; each piece's four waves step through its keys
KPW at a time with two key steps in flight (the prologue fetches the first
two steps, each step then refills its buffer with the step two ahead), and
every fetch index is clamped to the split's first key when it would leave
the split.  This replays the host's choice of split count and every row
index a lane fetches, and checks that each fetched row lies in the window
[max(0, pos - w_T + 1), pos], so inside a cache of pos + 1 rows, and that
every launched split holds a key.
"""
import pytest


def plan(w_t: int):
    """split_len and the planned (maximum) split count for a teacher window."""
    sl = 128 if w_t <= 2048 else 512
    return sl, (w_t + sl - 1) // sl


def splits_used(w_t: int, pos: int, sl: int) -> int:
    keys = min(w_t, pos + 1)
    return (keys + sl - 1) // sl


def fetched_rows(w_t: int, pos: int, head_dim: int):
    """Every row index any lane of any launched split fetches."""
    sl, nplan = plan(w_t)
    ns = splits_used(w_t, pos, sl)
    assert 1 <= ns <= nplan
    lpk = head_dim // 8               # lanes per key
    kpw = 64 // lpk                   # keys per wave step
    jlo = max(0, pos - w_t + 1)
    rows = set()

    def fetch(j, ks, ke):
        rows.add(j if j < ke else ks)

    for s in range(ns):
        ks = jlo + s * sl
        ke = min(ks + sl, pos + 1)
        assert ks < ke, (w_t, pos, s)
        for wave in range(4):
            for kg in range(kpw):
                j = ks + wave * kpw + kg
                fetch(j, ks, ke)                         # prologue: step 0
                fetch(j + 4 * kpw, ks, ke)               # and step 1
                j0 = ks + wave * kpw
                while j0 < ke:
                    fetch(j0 + kg + 8 * kpw, ks, ke)     # step(j0) refills two ahead
                    if j0 + 4 * kpw >= ke:
                        break
                    fetch(j0 + 4 * kpw + kg + 8 * kpw, ks, ke)
                    j0 += 8 * kpw
    return rows, jlo


@pytest.mark.parametrize("w_t", [1, 7, 100, 128, 129, 1000, 2048, 2049, 8192])
@pytest.mark.parametrize("head_dim", [64, 128])
def test_every_fetched_row_is_inside_the_window(w_t, head_dim):
    for pos in list(range(0, min(w_t + 70, 600))) + [w_t - 1, w_t, w_t + 513, 65535]:
        if pos < 0:
            continue
        rows, jlo = fetched_rows(w_t, pos, head_dim)
        assert min(rows) >= jlo and max(rows) <= pos, (w_t, pos, min(rows), max(rows))


def test_short_cache_launches_fewer_splits():
    # a 257-row cache under a 1000-key window: 3 splits of 128 keys, not 8
    sl, nplan = plan(1000)
    assert (sl, nplan) == (128, 8)
    assert splits_used(1000, 256, sl) == 3

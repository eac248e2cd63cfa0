"""The documented split schedule, re-derived in Python, is itself valid."""
import numpy as np
import pytest

from tests import schedule_check as sc

CASES = [
    ([37, 130], 256), ([37, 130], 1), ([37, 130], 3), ([0, 0, 5], 4), ([131072] + [1024] * 31, 256),
    ([1, 16, 17, 64, 65, 0, 1000], 7), ([4096] * 64, 256), ([5], 1024), ([1] * 10, 64),
]


@pytest.mark.parametrize("lead", [0, 8, 16])
@pytest.mark.parametrize("seqlens,parts", CASES)
def test_expected_schedule_is_valid(seqlens, parts, lead):
    meta = sc.expected_metadata(seqlens, parts, lead)
    sc.check_valid(meta, seqlens, parts)
    n = np.maximum(np.asarray(seqlens), 0)
    ch = (n + 15) // 16
    TC = int(ch.sum() + lead * np.count_nonzero(ch))
    U = min(parts, TC)
    recs = meta[:8 * parts].reshape(parts, 8)
    assert np.all(recs[U:, 0] == -1)
    # a part's cost: its chunks plus a lead for every sequence it starts
    costs = []
    for p in range(U):
        s0, t0, s1, t1 = (int(v) for v in recs[p, :4])
        if s0 < 0:
            continue
        c = 0
        for s in range(s0, s1 + 1):
            a = t0 if s == s0 else 0
            e = t1 if s == s1 else n[s]
            if a < e:
                c += (e + 15) // 16 - a // 16 + (lead if a == 0 else 0)
        costs.append(c)
    if lead == 0:
        sizes = [((p + 1) * TC) // U - (p * TC) // U for p in range(U)]
        assert max(sizes) - min(sizes) <= 1 and min(sizes) >= 1 and np.all(recs[:U, 0] >= 0)
    # each part's cost is its unit range (TC/U, rounded) give or take one lead
    assert max(costs) <= -(-TC // U) + lead
    assert meta[8 * parts + len(seqlens)] <= len(seqlens) + U - 1


def test_lead_moves_cuts_to_sequence_starts():
    """With a lead, a part that starts a sequence takes fewer chunks."""
    seqlens, parts = [1024] * 8, 12
    even = sc.expected_metadata(seqlens, parts, 0).reshape(-1)[:8 * parts].reshape(parts, 8)
    led = sc.expected_metadata(seqlens, parts, 16).reshape(-1)[:8 * parts].reshape(parts, 8)
    assert not np.array_equal(even[:, :4], led[:, :4])


def test_checker_rejects_broken_schedules():
    seqlens, parts = [100, 40, 300], 5
    meta = sc.expected_metadata(seqlens, parts, 16)
    bad = meta.copy()
    bad[8 * 2 + 1] += 16        # part 2 starts one chunk late: a gap
    with pytest.raises(AssertionError):
        sc.check_valid(bad, seqlens, parts)
    bad = meta.copy()
    bad[8 * parts + 1] += 1     # split offsets inconsistent with the parts
    with pytest.raises(AssertionError):
        sc.check_valid(bad, seqlens, parts)

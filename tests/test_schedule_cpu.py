"""The documented split schedule, re-derived in Python, is itself valid."""
import numpy as np
import pytest

from tests import schedule_check as sc


@pytest.mark.parametrize("seqlens,parts", [
    ([37, 130], 256), ([37, 130], 1), ([37, 130], 3), ([0, 0, 5], 4), ([131072] + [1024] * 31, 256),
    ([1, 16, 17, 64, 65, 0, 1000], 7), ([4096] * 64, 256), ([5], 1024),
])
def test_expected_schedule_is_valid(seqlens, parts):
    meta = sc.expected_metadata(seqlens, parts)
    sc.check_valid(meta, seqlens, parts)
    T = int(meta[-1])
    U = min(parts, T)
    recs = meta[:8 * parts].reshape(parts, 8)
    assert np.all(recs[U:, 0] == -1) and np.all(recs[:U, 0] >= 0)
    sizes = [((p + 1) * T) // U - (p * T) // U for p in range(U)]
    assert max(sizes) - min(sizes) <= 1 and min(sizes) >= 1
    assert meta[8 * parts + len(seqlens)] <= len(seqlens) + U - 1


def test_checker_rejects_broken_schedules():
    seqlens, parts = [100, 40, 300], 5
    meta = sc.expected_metadata(seqlens, parts)
    bad = meta.copy()
    bad[8 * 2 + 1] += 16        # part 2 starts one chunk late: a gap
    with pytest.raises(AssertionError):
        sc.check_valid(bad, seqlens, parts)
    bad = meta.copy()
    bad[8 * parts + 1] += 1     # split offsets inconsistent with the parts
    with pytest.raises(AssertionError):
        sc.check_valid(bad, seqlens, parts)

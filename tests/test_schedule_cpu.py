"""The documented split schedule, re-derived in Python, is itself valid, and
its cuts are close to the best contiguous ones under a per-segment cost."""
import itertools

import numpy as np
import pytest

from mla_paged_kv_02_amd import inputs as gen
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


def _brute_best(seqlens, parts, cost):
    """All cuts of the chunk list into at most `parts` runs, by enumeration."""
    ch = (np.maximum(np.asarray(seqlens), 0) + 15) // 16
    units = [(b, i) for b in range(len(ch)) for i in range(int(ch[b]))]
    best = None
    for k in range(min(parts, len(units))):
        for cuts in itertools.combinations(range(1, len(units)), k):
            bounds = (0,) + cuts + (len(units),)
            worst = max(len(units[a:e]) + cost * len({b for b, _ in units[a:e]})
                        for a, e in zip(bounds, bounds[1:]))
            best = worst if best is None else min(best, worst)
    return best


@pytest.mark.parametrize("cost", [0, 1, 3])
@pytest.mark.parametrize("seqlens,parts", [([40, 100, 17], 2), ([40, 100, 17], 3),
                                           ([16, 16, 16, 16], 3), ([90, 0, 33, 60], 4),
                                           ([129], 3), ([1, 200, 1], 2)])
def test_best_max_cost_matches_enumeration(seqlens, parts, cost):
    assert sc.best_max_cost(seqlens, parts, cost) == _brute_best(seqlens, parts, cost)


def test_pick_lead_by_hand():
    """Two sequences of 40 chunks over 3 parts, 8 chunks a segment: the
    largest part (chunks + 8 per segment) is 43 with lead 0 (cuts at units
    26, 53), 40 with lead 8 (32, 64), 46 with lead 16, 48 with 24 and 32, so
    the schedule takes lead 8."""
    seqlens, parts = [640, 640], 3
    want = {0: 43, 8: 40, 16: 46, 24: 48, 32: 48}
    for lead, m in want.items():
        c = sc.segment_costs(sc.expected_metadata(seqlens, parts, lead), seqlens, parts, 8)
        assert int(c.max()) == m, lead
    assert sc.pick_lead(seqlens, parts, 8, (0, 8, 16, 24, 32)) == 8
    assert sc.pick_lead(seqlens, parts, 8, (0, 16)) == 0
    # an all-empty batch prices every lead at 0: the one nearest the cost
    assert sc.pick_lead([0, 0], 4, 24, (0, 24)) == 24


@pytest.mark.parametrize("name", ["memory_bound", "compute_bound", "skewed", "full_step",
                                  "multi_token_4", "multi_token_8", "len_1k", "len_5k"])
def test_cuts_near_best_partition(name):
    """With the segment cost the schedule prices, its cuts land within 3%
    (or two chunks) of the best largest part over all contiguous cuts into
    the same number of parts (at 256 compute units): a better cut rule has
    little to gain on these workloads."""
    seqlens, s_q, h_q, _ = gen.config_shape(name)
    parts = 256 // sc.row_tiles(s_q, h_q)
    cost = sc.segment_cost_for(s_q, h_q)
    meta = sc.expected_schedule(seqlens, parts, s_q, h_q)
    got = int(sc.segment_costs(meta, seqlens, parts, cost).max())
    best = sc.best_max_cost(seqlens, parts, cost)
    assert best <= got <= best + max(0.03 * best, 2), (got, best)

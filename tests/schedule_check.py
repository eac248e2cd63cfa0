"""Host-side checks of the split schedule written by mla_get_metadata.

The schedule is documented in include/mla_paged_kv.h: sequence b with ch_b
> 0 chunks of 16 tokens is `lead` cost units followed by its ch_b chunk
units; the concatenation (TC units) is cut into U = min(num_parts, TC) runs,
part p < U taking the chunks whose units lie in [floor(p*TC/U),
floor((p+1)*TC/U)); a run of lead units only, and parts >= U, are empty.
`expected_metadata` re-derives that layout independently in Python, by
walking the unit list one unit at a time; `check_valid` checks the properties
any correct schedule must have (every token covered exactly once, in order;
slot numbering consistent with the split offsets).
"""
import numpy as np

CHUNK = 16
WIDE_ROWS = 128
FEW_SPLITS = 32        # more splits than this: a heavy sequence
COMBINE_ROWS = 4       # rows per merge workgroup


MAX_SEQ_LEN = 1 << 21  # lengths are capped here on the device


def capped(seqlens):
    return np.clip(np.asarray(seqlens, dtype=np.int64), 0, MAX_SEQ_LEN)


def is_wide(s_q, h_q):
    """True when the 128-row kernel serves s_q * h_q rows (48 and more)."""
    r = s_q * h_q
    return r % WIDE_ROWS == 0 or r >= 48


def row_tiles(s_q, h_q):
    """Workgroups per part: 128-row tiles on the 128-row kernel, one on its
    32-row variant, 16-row tiles on the 16-row kernel."""
    r = s_q * h_q
    if is_wide(s_q, h_q):
        return -(-r // WIDE_ROWS)
    return 1 if r == 32 else -(-r // 16)


def segment_cost_for(s_q, h_q):
    """The schedule's price of one sequence segment, in chunks: 24 for the
    128-row kernel, 16 for the 16-row kernel."""
    return 24 if is_wide(s_q, h_q) else 16


def pick_lead(seqlens, num_parts, seg_cost, candidates):
    """Among the candidate leads, the one whose cuts have the smallest largest
    part when every segment costs seg_cost chunks (segment_costs); ties go
    to the candidate nearest seg_cost."""
    def key(lead):
        c = segment_costs(expected_metadata(seqlens, num_parts, lead), seqlens, num_parts,
                          seg_cost)
        return (int(c.max()) if len(c) else 0, abs(lead - seg_cost))
    return min(candidates, key=key)


def expected_schedule(seqlens, num_parts, s_q, h_q):
    """The full metadata mla_get_metadata writes for these lengths and rows:
    the 16-row kernel's schedule uses its segment cost as the lead; the
    128-row kernel's takes whichever of 0 and its segment cost prices
    lower."""
    cost = segment_cost_for(s_q, h_q)
    lead = pick_lead(seqlens, num_parts, cost, (0, cost)) if is_wide(s_q, h_q) else cost
    return expected_metadata(seqlens, num_parts, lead)


def expected_metadata(seqlens, num_parts, lead):
    n = capped(seqlens)
    B, P = len(n), int(num_parts)
    ch = (n + CHUNK - 1) // CHUNK
    # the unit list: (sequence, chunk index or -1 for a lead unit)
    units = []
    for b in range(B):
        if ch[b]:
            units += [(b, -1)] * lead + [(b, i) for i in range(int(ch[b]))]
    TC = len(units)
    U = min(P, TC)
    part_of_unit = np.zeros(TC, dtype=np.int64)
    for p in range(U):
        part_of_unit[(p * TC) // U:((p + 1) * TC) // U] = p
    # chunks of every part, in order
    chunks = [[] for _ in range(P)]
    for x, (b, i) in enumerate(units):
        if i >= 0:
            chunks[part_of_unit[x]].append((b, i))
    nsplit = np.zeros(B, dtype=np.int64)
    for b in range(B):
        nsplit[b] = sum(1 for p in range(P) if any(c[0] == b for c in chunks[p]))
    split_off = np.concatenate([[0], np.cumsum(nsplit)])
    recs = np.zeros((P, 8), dtype=np.int64)
    for p in range(P):
        if not chunks[p]:
            recs[p, :4] = [-1, 0, -1, 0]
            continue
        (s0, i0), (s1, i1) = chunks[p][0], chunks[p][-1]
        recs[p, 0] = s0
        recs[p, 1] = i0 * CHUNK
        recs[p, 2] = s1
        recs[p, 3] = min((i1 + 1) * CHUNK, n[s1])
        first_part_of_s0 = min(q for q in range(P) if any(c[0] == s0 for c in chunks[q]))
        recs[p, 4] = split_off[s0] + (p - first_part_of_s0)
    # merge section: extra workgroups of heavy (> 32-way split) sequences,
    # 4 rows x S dim slices per row group, S by the header's table
    def slices(k):
        return 16 if k >= 256 else 8 if k >= 128 else 4 if k >= 64 else 2

    extra = [COMBINE_ROWS * slices(int(k)) - 1 if k > FEW_SPLITS else 0 for k in nsplit]
    extra_off = np.concatenate([[0], np.cumsum(extra, dtype=np.int64)])
    return np.concatenate([recs.ravel(), split_off, [int(ch.sum())],
                           extra_off]).astype(np.int32)


def check_valid(meta, seqlens, num_parts):
    """Raise AssertionError unless the schedule covers each token once, in order."""
    n = capped(seqlens)
    B, P = len(n), int(num_parts)
    meta = np.asarray(meta, dtype=np.int64)
    recs = meta[:8 * P].reshape(P, 8)
    split_off = meta[8 * P:8 * P + B + 1]
    assert split_off[0] == 0 and np.all(np.diff(split_off) >= 0)
    assert split_off[-1] <= B + P, "more partial slots than the workspace holds"
    cursor = np.zeros(B, dtype=np.int64)        # next token expected per sequence
    slots_seen = [[] for _ in range(B)]
    last_seq = -1
    for p in range(P):
        s0, t0, s1, t1, slot0 = (int(v) for v in recs[p, :5])
        if s0 < 0:
            continue
        assert s0 >= last_seq and s0 <= s1 < B
        for s in range(s0, s1 + 1):
            a = t0 if s == s0 else 0
            e = t1 if s == s1 else n[s]
            if a >= e:
                assert n[s] == 0 or (s == s0 and False), "empty segment in part %d" % p
                continue
            assert a == cursor[s], "gap or overlap in sequence %d at token %d" % (s, a)
            assert e <= n[s]
            cursor[s] = e
            slots_seen[s].append(slot0 if s == s0 else split_off[s])
        last_seq = s1
    assert np.array_equal(cursor, n), "not every token covered"
    for s in range(B):
        want = list(range(split_off[s], split_off[s + 1]))
        assert slots_seen[s] == want, (s, slots_seen[s], want)


def segment_costs(meta, seqlens, num_parts, cost):
    """Per non-empty part: its 16-token chunks plus `cost` for every sequence
    segment it runs (query load, pipeline fill and result write, in chunks)."""
    n = capped(seqlens)
    P = int(num_parts)
    recs = np.asarray(meta, dtype=np.int64)[:8 * P].reshape(P, 8)
    out = []
    for p in range(P):
        s0, t0, s1, t1 = (int(v) for v in recs[p, :4])
        if s0 < 0:
            continue
        c = 0
        for s in range(s0, s1 + 1):
            a = t0 if s == s0 else 0
            e = t1 if s == s1 else int(n[s])
            if a < e:
                c += cost + (e + CHUNK - 1) // CHUNK - a // CHUNK
        out.append(c)
    return np.array(out, dtype=np.int64)


def best_max_cost(seqlens, num_parts, cost):
    """The smallest possible largest part cost (segment_costs) over all cuts of
    the chunk list, in order, into at most num_parts runs.  For a bound T,
    filling each part as far as T allows uses the fewest parts (taking more of
    the next sequence into a part never makes a later part costlier), so a
    binary search over T with that greedy count gives the optimum."""
    ch = [int(c) for c in (capped(seqlens) + CHUNK - 1) // CHUNK if c]
    if not ch:
        return 0

    def parts_needed(T):
        used, cur = 1, 0
        for rem in ch:
            while rem:
                if cur + cost + 1 > T:      # not even one chunk fits: next part
                    used, cur = used + 1, 0
                take = min(rem, T - cur - cost)
                cur += cost + take
                rem -= take
                if rem:
                    used, cur = used + 1, 0
        return used

    lo, hi = cost + 1, sum(ch) + cost * len(ch)
    while lo < hi:
        mid = (lo + hi) // 2
        if parts_needed(mid) <= num_parts:
            hi = mid
        else:
            lo = mid + 1
    return lo

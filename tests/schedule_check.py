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
FEW_SPLITS = 32        # more splits than this: two-level merge
HEAVY_CHUNK = 16       # splits per first-level merge workgroup
ROW_GROUPS_MAX = 512   # merge counters per heavy sequence


MAX_SEQ_LEN = 1 << 21  # lengths are capped here on the device


def capped(seqlens):
    return np.clip(np.asarray(seqlens, dtype=np.int64), 0, MAX_SEQ_LEN)


def lead_for(s_q, h_q):
    """Cost of starting a sequence, in chunks, for s_q*h_q rows: 16 below 128
    rows (the 16-row kernel, and partly empty 128-row tiles), 8 at exactly
    128 rows, 24 above (two or more 128-row tiles)."""
    r = s_q * h_q
    return 16 if r < WIDE_ROWS else 8 if r == WIDE_ROWS else 24


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
    # merge sections: extra workgroups of heavy (> 32-way split) sequences,
    # their ranks, zeroed counters
    heavy = nsplit > FEW_SPLITS
    extra = np.where(heavy, (nsplit + HEAVY_CHUNK - 1) // HEAVY_CHUNK - 1, 0)
    extra_off = np.concatenate([[0], np.cumsum(extra)])
    heavy_rank = np.concatenate([[0], np.cumsum(heavy)])[:B]
    counters = np.zeros(ROW_GROUPS_MAX * ((B + P) // (FEW_SPLITS + 1) + 1), dtype=np.int64)
    return np.concatenate([recs.ravel(), split_off, [int(ch.sum())], extra_off, heavy_rank,
                           counters]).astype(np.int32)


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

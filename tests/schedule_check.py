"""Host-side checks of the split schedule written by mla_get_metadata.

The schedule is documented in include/mla_paged_kv.h: the 16-token chunks of
all sequences, concatenated in batch order, are cut into P' = min(num_parts, T)
runs, part p < P' covering chunks [floor(p*T/P'), floor((p+1)*T/P')); later
parts are empty.  `expected_metadata`
re-derives that layout independently in Python; `check_valid` checks the
properties any correct schedule must have (every token covered exactly once,
in order; slot numbering consistent with the split offsets).
"""
import numpy as np

CHUNK = 16


def expected_metadata(seqlens, num_parts):
    n = np.maximum(np.asarray(seqlens, dtype=np.int64), 0)
    B, P = len(n), int(num_parts)
    ch = (n + CHUNK - 1) // CHUNK
    pre = np.concatenate([[0], np.cumsum(ch)])
    T = int(pre[-1])
    U = min(P, T)                      # used (non-empty) parts
    starts = [(p * T) // U for p in range(U + 1)] if U else [0]

    def part_of(f):
        # the used part whose chunk range holds chunk f
        p = 0
        while p + 1 < U and starts[p + 1] <= f:
            p += 1
        return p

    nsplit = np.zeros(B, dtype=np.int64)
    for b in range(B):
        if ch[b]:
            nsplit[b] = part_of(pre[b + 1] - 1) - part_of(pre[b]) + 1
    split_off = np.concatenate([[0], np.cumsum(nsplit)])
    recs = np.zeros((P, 8), dtype=np.int64)
    for p in range(P):
        if p >= U:
            recs[p, :4] = [-1, 0, -1, 0]
            continue
        f0, f1 = starts[p], starts[p + 1]
        s0 = int(np.searchsorted(pre, f0, side="right") - 1)
        s1 = int(np.searchsorted(pre, f1 - 1, side="right") - 1)
        recs[p, 0] = s0
        recs[p, 1] = (f0 - pre[s0]) * CHUNK
        recs[p, 2] = s1
        recs[p, 3] = min((f1 - pre[s1]) * CHUNK, n[s1])
        recs[p, 4] = split_off[s0] + (p - part_of(pre[s0]))
    return np.concatenate([recs.ravel(), split_off, [T]]).astype(np.int32)


def check_valid(meta, seqlens, num_parts):
    """Raise AssertionError unless the schedule covers each token once, in order."""
    n = np.maximum(np.asarray(seqlens, dtype=np.int64), 0)
    B, P = len(n), int(num_parts)
    meta = np.asarray(meta, dtype=np.int64)
    recs = meta[:8 * P].reshape(P, 8)
    split_off = meta[8 * P:8 * P + B + 1]
    assert split_off[0] == 0 and np.all(np.diff(split_off) >= 0)
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

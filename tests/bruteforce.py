"""Pure-Python brute force for tiny inputs (pins the fp64 oracle).

Written independently of the oracle: scalar loops, math.fsum for every sum,
its own bf16 decoding through struct, and the causal mask written in terms of
absolute positions (query i of a sequence of length n sits at position
n - s_q + i and sees the keys at positions <= its own).
"""
import math
import struct


def bf16(bits):
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def decode(q, kv, block_table, seqlens, s_q, h_q, scale, causal, page, d_v):
    """q: nested [B][s_q][h_q][d] of floats; kv: numpy uint16 [P][page][d].
    Returns (out [B][s_q][h_q][d_v], lse [B][s_q][h_q]) as nested lists."""
    out, lse = [], []
    for b, n in enumerate(seqlens):
        n = int(n)
        rows_o, rows_l = [], []
        for i in range(s_q):
            ho, hl = [], []
            for h in range(h_q):
                qv = q[b][i][h]
                keys = []
                for pos in range(n):
                    if causal and pos > n - s_q + i:
                        continue
                    page_id = int(block_table[b][pos // page])
                    keys.append([bf16(x) for x in kv[page_id][pos % page]])
                if not keys:
                    ho.append([0.0] * d_v)
                    hl.append(-math.inf)
                    continue
                logits = [float(scale) * math.fsum(a * c for a, c in zip(qv, k)) for k in keys]
                top = max(logits)
                w = [math.exp(s - top) for s in logits]
                tot = math.fsum(w)
                ho.append([math.fsum(w[t] * keys[t][e] for t in range(len(keys))) / tot
                           for e in range(d_v)])
                hl.append(top + math.log(tot))
            rows_o.append(ho)
            rows_l.append(hl)
        out.append(rows_o)
        lse.append(rows_l)
    return out, lse


def matmul_rows(x, w):
    """x [B][H][K] floats, w [H][K][N] floats -> [B][H][N] with fsum."""
    H = len(w)
    K = len(w[0])
    N = len(w[0][0])
    return [[[math.fsum(x[b][h][k] * w[h][k][n] for k in range(K)) for n in range(N)]
             for h in range(H)] for b in range(len(x))]

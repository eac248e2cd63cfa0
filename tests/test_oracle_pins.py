"""Pins of the fp64 oracle against things other than itself.

Each check fixes a part of the definition (see oracle/mla_oracle.c) with an
independent route: a pure-Python brute force, a closed form, an invariant, or
a hand-derived fixture.  Together they are chosen so that a dropped term, a
wrong sign or index, or a transposed operand in the oracle fails at least one
of them (tests/test_oracle_mutants.py plants such mistakes and checks that).
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import oracle as orc
from mla_paged_kv_02_amd import inputs as gen
from tests import bruteforce as bf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _small_case(seed, seqlens, *, s_q=1, h_q=2, d_qk=12, d_v=8, page=4, causal=False,
                poison=True):
    ss = np.random.SeedSequence(seed).spawn(5)
    rp, rq, rk = (np.random.default_rng(ss[i]) for i in (1, 2, 3))
    kv, bt = gen.paged_cache(np.asarray(seqlens), rp, rk, page=page, width=d_qk, poison=poison)
    q = gen.normal_bf16(rq, (len(seqlens), s_q, h_q, d_qk))
    return q, kv, bt, np.asarray(seqlens, dtype=np.int32)


def _brute(q_bits, kv, bt, seqlens, s_q, h_q, scale, causal, page, d_v):
    qf = [[[[bf.bf16(x) for x in q_bits[b, i, h]] for h in range(h_q)] for i in range(s_q)]
          for b in range(len(seqlens))]
    out, lse = bf.decode(qf, kv, bt, seqlens, s_q, h_q, scale, causal, page, d_v)
    return np.array(out, dtype=np.float64), np.array(lse, dtype=np.float64)


def _close(a, b, tol):
    a, b = np.asarray(a), np.asarray(b)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        diff = np.where(both_inf, 0.0, np.abs(a - b))
    if np.isnan(diff).any():
        return False
    return float(np.max(diff, initial=0.0)) <= tol


def test_bruteforce_tiny_config():
    """The tiny workload (2 sequences x 16 heads, lengths 37 and 130, shuffled
    64-token pages, NaN tails) against scalar fsum loops."""
    x = gen.make_config("tiny")
    out, lse = orc.attend(x.q, x.kv, x.block_table, x.seqlens, s_q=1, h_q=16,
                          scale=x.scale, causal=False)
    bo, bl = _brute(x.q, x.kv, x.block_table, x.seqlens, 1, 16, x.scale, False, 64, 512)
    assert _close(out, bo, 1e-12) and _close(lse, bl, 1e-12)
    assert np.all(np.isfinite(out))


@pytest.mark.parametrize("seed,seqlens,s_q,causal", [
    (1, [1, 5, 9], 1, False),
    (2, [4, 13, 0, 7], 1, False),
    (3, [6, 11, 2, 1], 3, True),
    (4, [17, 3], 4, True),
    (5, [8, 16], 2, False),
])
def test_bruteforce_random_small(seed, seqlens, s_q, causal):
    """Small widths and 4-token pages so many page boundaries are crossed;
    includes empty sequences and causal rows with no visible key."""
    q, kv, bt, sl = _small_case(seed, seqlens, s_q=s_q, causal=causal)
    scale = float(np.float32(0.37))
    out, lse = orc.attend(q, kv, bt, sl, s_q=s_q, h_q=2, scale=scale, causal=causal, page=4, d_v=8)
    bo, bl = _brute(q, kv, bt, sl, s_q, 2, scale, causal, 4, 8)
    assert _close(out, bo, 1e-12), np.max(np.abs(out - bo))
    assert _close(lse, bl, 1e-12)


def test_golden_fixture():
    g = json.load(open(os.path.join(GOLDEN, "three_keys_two_pages.json")))
    env = {"e": math.e, "ln": math.log, "__builtins__": {}}
    ev = lambda s: eval(str(s), env)  # noqa: E731  (fixture expressions only)
    page, d_qk, d_v = g["page"], g["d_qk"], g["d_v"]
    kv = np.zeros((g["num_pages"], page, d_qk), dtype=np.float32)
    for pid, rows in g["pages"].items():
        kv[int(pid)] = np.array([[float(v) for v in r] for r in rows], dtype=np.float32)
    kv_bits = gen.f32_to_bf16_bits(kv)
    bt = np.array([g["block_table"]], dtype=np.int32)
    q = np.array(g["q"], dtype=np.float64)
    out, lse = orc.attend(q.reshape(1, 1, 1, d_qk), kv_bits, bt, np.array([g["seqlen"]]),
                          s_q=1, h_q=1, scale=g["scale"], causal=False, page=page, d_v=d_v)
    assert np.allclose(out.ravel(), [ev(s) for s in g["expect_full"]["out"]], atol=1e-15, rtol=0)
    assert abs(lse.item() - ev(g["expect_full"]["lse"])) < 1e-15
    q2 = np.stack([q, q]).reshape(1, 2, 1, d_qk)
    out2, lse2 = orc.attend(q2, kv_bits, bt, np.array([g["seqlen"]]), s_q=2, h_q=1,
                            scale=g["scale"], causal=True, page=page, d_v=d_v)
    c = g["expect_causal_query0"]
    assert np.allclose(out2[0, 0, 0], [ev(s) for s in c["out"]], atol=1e-15, rtol=0)
    assert abs(lse2[0, 0, 0] - ev(c["lse"])) < 1e-15
    assert np.allclose(out2[0, 1, 0], out.ravel(), atol=0, rtol=0)
    cm = g["expect_combine"]
    o_parts = np.array([[[ev(v) for v in p]] for p in cm["o_parts"]])
    l_parts = np.array([[ev(v)] for v in cm["lse_parts"]])
    co, cl = orc.combine(o_parts, l_parts)
    assert np.allclose(co.ravel(), [ev(s) for s in cm["out"]], atol=1e-15, rtol=0)
    assert abs(cl.item() - ev(cm["lse"])) < 1e-15


def test_single_key_closed_form():
    """n = 1: the output is the value row itself, lse = scale * q.k."""
    x = gen.make_decode([1, 1, 1], s_q=1, h_q=16, causal=False, seed=11)
    out, lse = orc.attend(x.q, x.kv, x.block_table, x.seqlens, s_q=1, h_q=16,
                          scale=x.scale, causal=False)
    for b in range(3):
        row = orc.bf16_to_f64(x.kv[x.block_table[b, 0], 0])
        qb = orc.bf16_to_f64(x.q[b, 0])
        assert np.array_equal(out[b, 0], np.broadcast_to(row[:512], (16, 512)))
        for h in range(16):
            ref = x.scale * math.fsum(qb[h] * row)
            assert abs(lse[b, 0, h] - ref) < 1e-12


def test_zero_query_uniform_weights():
    """q = 0: all logits are 0, the output is the plain mean of the value rows
    and lse = ln n."""
    x = gen.make_decode([5, 70, 129], s_q=1, h_q=16, causal=False, seed=12)
    q = np.zeros_like(x.q)
    out, lse = orc.attend(q, x.kv, x.block_table, x.seqlens, s_q=1, h_q=16,
                          scale=x.scale, causal=False)
    for b, n in enumerate(x.seqlens):
        rows = np.stack([orc.bf16_to_f64(x.kv[x.block_table[b, j // 64], j % 64]) for j in range(n)])
        mean = np.array([math.fsum(rows[:, e]) / n for e in range(512)])
        assert np.allclose(out[b, 0], mean[None, :], atol=1e-13, rtol=0)
        assert np.allclose(lse[b, 0], math.log(n), atol=1e-13, rtol=0)


def test_identical_keys():
    """All keys equal: weights are uniform, out = that row's value part and
    lse = scale * q.k + ln n."""
    x = gen.make_decode([77], s_q=1, h_q=16, causal=False, seed=13)
    kv = x.kv.copy()
    row = kv[x.block_table[0, 0], 0].copy()
    for j in range(77):
        kv[x.block_table[0, j // 64], j % 64] = row
    out, lse = orc.attend(x.q, kv, x.block_table, x.seqlens, s_q=1, h_q=16, scale=x.scale,
                          causal=False)
    r = orc.bf16_to_f64(row)
    assert np.allclose(out[0, 0], r[None, :512], atol=1e-13, rtol=0)
    qb = orc.bf16_to_f64(x.q[0, 0])
    for h in range(16):
        assert abs(lse[0, 0, h] - (x.scale * math.fsum(qb[h] * r) + math.log(77))) < 1e-12


def test_constant_value_rows():
    """Value dims identical across tokens, rope dims random: a convex
    combination of equal vectors is that vector."""
    x = gen.make_decode([200, 64], s_q=2, h_q=16, causal=True, seed=14)
    kv = x.kv.copy()
    v = gen.f32_to_bf16_bits(np.linspace(-3, 3, 512).astype(np.float32))
    for b, n in enumerate(x.seqlens):
        for j in range(n):
            kv[x.block_table[b, j // 64], j % 64, :512] = v
    out, lse = orc.attend(x.q, kv, x.block_table, x.seqlens, s_q=2, h_q=16, scale=x.scale,
                          causal=True)
    assert np.allclose(out, orc.bf16_to_f64(v), atol=1e-14, rtol=0)


def test_page_permutation_invariance():
    """Moving pages to other physical slots (and remapping the block table)
    changes nothing, bit for bit."""
    x = gen.make_decode([130, 37, 64], s_q=1, h_q=16, causal=False, seed=15)
    out, lse = orc.attend(x.q, x.kv, x.block_table, x.seqlens, s_q=1, h_q=16, scale=x.scale,
                          causal=False)
    rng = np.random.default_rng(7)
    P = x.kv.shape[0]
    perm = rng.permutation(P)            # new slot of old page p is perm[p]
    kv2 = np.empty_like(x.kv)
    kv2[perm] = x.kv
    bt2 = np.where(x.block_table >= 0, perm[np.clip(x.block_table, 0, None)], -1).astype(np.int32)
    out2, lse2 = orc.attend(x.q, kv2, bt2, x.seqlens, s_q=1, h_q=16, scale=x.scale, causal=False)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


@pytest.mark.parametrize("seed", [21, 22, 23])
def test_split_combine_equals_unsplit(seed):
    """Any partition of the key range into contiguous splits (empty and
    one-token splits included), merged by lse weights, gives the unsplit
    result."""
    x = gen.make_decode([300, 65, 1, 129], s_q=2, h_q=16, causal=True, seed=seed)
    full_o, full_l = orc.attend(x.q, x.kv, x.block_table, x.seqlens, s_q=2, h_q=16,
                                scale=x.scale, causal=True)
    rng = np.random.default_rng(seed)
    n_parts = 5
    cuts = []
    for n in x.seqlens:
        c = np.sort(rng.integers(0, n + 1, n_parts - 1))
        if n > 2:
            c[0] = c[1]            # force an empty split
            c[-1] = min(c[-1], n - 1)
        cuts.append(np.concatenate([[0], c, [n]]))
    cuts = np.array(cuts, dtype=np.int64)
    o_parts, l_parts = [], []
    for p in range(n_parts):
        o, l = orc.attend(x.q, x.kv, x.block_table, x.seqlens, s_q=2, h_q=16, scale=x.scale,
                          causal=True, key_begin=cuts[:, p], key_end=cuts[:, p + 1])
        o_parts.append(o)
        l_parts.append(l)
    o, l = orc.combine(np.stack(o_parts), np.stack(l_parts))
    assert np.allclose(o, full_o, atol=1e-12, rtol=0)
    assert _close(l, full_l, 1e-12)


def test_causal_row_equals_shorter_decode():
    """Row i of a causal decode with s_q queries equals an s_q = 1 decode of
    the same query over the first n - s_q + 1 + i keys, bit for bit."""
    x = gen.make_decode([150, 3, 64], s_q=3, h_q=16, causal=True, seed=31)
    out, lse = orc.attend(x.q, x.kv, x.block_table, x.seqlens, s_q=3, h_q=16, scale=x.scale,
                          causal=True)
    for i in range(3):
        L = np.maximum(x.seqlens - 3 + 1 + i, 0).astype(np.int32)
        o1, l1 = orc.attend(x.q[:, i:i + 1], x.kv, x.block_table, L, s_q=1, h_q=16,
                            scale=x.scale, causal=False)
        assert np.array_equal(out[:, i], o1[:, 0]) and np.array_equal(lse[:, i], l1[:, 0])


def test_empty_rows():
    """No visible key: out = 0, lse = -inf (n = 0, and causal rows whose
    position is before the first key)."""
    x = gen.make_decode([0, 1, 2], s_q=3, h_q=16, causal=True, seed=41)
    out, lse = orc.attend(x.q, x.kv, x.block_table, x.seqlens, s_q=3, h_q=16, scale=x.scale,
                          causal=True)
    assert np.all(out[0] == 0) and np.all(lse[0] == -np.inf)
    assert np.all(lse[1, :2] == -np.inf) and np.all(np.isfinite(lse[1, 2]))
    assert np.all(lse[2, :1] == -np.inf) and np.all(np.isfinite(lse[2, 1:]))


def test_absorb_bmm_bruteforce():
    rng = np.random.default_rng(5)
    x = gen.normal_bf16(rng, (3, 2, 6))
    w = gen.normal_bf16(rng, (2, 6, 5), std=0.02)
    y = orc.absorb_bmm(x, w)
    xf = orc.bf16_to_f64(x).tolist()
    wf = orc.bf16_to_f64(w).tolist()
    ref = np.array(bf.matmul_rows(xf, wf))
    assert np.allclose(y, ref, atol=1e-15, rtol=1e-14)


def test_absorbed_equals_explicit_up_projection():
    """Attention over the shared latent with absorbed queries equals ordinary
    per-head attention with explicitly up-projected keys and values:
    K_h,j = [W_UK[h] c_j | rope_j] (192 dims) and V_h,j = W_UV[h]^T c_j
    (128 dims), same scale ("[Attention] MLA get rid of materialization", PR
    description: absorption as sequential matmuls)."""
    B, H, n = 2, 4, 150
    rng = np.random.default_rng(99)
    x = gen.make_decode([n, 97], s_q=1, h_q=H, causal=False, seed=51)
    q_nope = gen.normal_bf16(rng, (B, H, 128))
    q_rope = gen.normal_bf16(rng, (B, H, 64))
    w_uk = gen.normal_bf16(rng, (H, 128, 512), std=0.02)
    w_uv = gen.normal_bf16(rng, (H, 512, 128), std=0.02)
    _, _, lse, y = orc.full_step(q_nope, q_rope, w_uk, w_uv, x.kv, x.block_table, x.seqlens,
                                 scale=x.scale)
    Wuk, Wuv = orc.bf16_to_f64(w_uk), orc.bf16_to_f64(w_uv)
    qn, qr = orc.bf16_to_f64(q_nope), orc.bf16_to_f64(q_rope)
    for b, nb in enumerate(x.seqlens):
        C = np.stack([orc.bf16_to_f64(x.kv[x.block_table[b, j // 64], j % 64]) for j in range(nb)])
        for h in range(H):
            K = np.concatenate([C[:, :512] @ Wuk[h].T, C[:, 512:]], axis=1)   # [n, 192]
            V = C[:, :512] @ Wuv[h]                                           # [n, 128]
            s = x.scale * (K @ np.concatenate([qn[b, h], qr[b, h]]))
            m = s.max()
            w = np.exp(s - m)
            ref_y = (w @ V) / w.sum()
            ref_l = m + np.log(w.sum())
            assert np.allclose(y[b, h], ref_y, rtol=1e-10, atol=1e-13)
            assert abs(lse[b, h] - ref_l) < 1e-10


def test_nan_tails_and_unused_pages_ignored():
    """Rows past the length and unreferenced pages hold NaN; outputs are
    finite and equal to those from a cache with those slots zeroed."""
    x = gen.make_decode([37, 130], s_q=1, h_q=16, causal=False, seed=61, extra_pages=3)
    out, lse = orc.attend(x.q, x.kv, x.block_table, x.seqlens, s_q=1, h_q=16, scale=x.scale,
                          causal=False)
    kv0 = x.kv.copy()
    kv0[np.isnan(gen.bf16_bits_to_f32(kv0))] = 0
    out0, lse0 = orc.attend(x.q, kv0, x.block_table, x.seqlens, s_q=1, h_q=16, scale=x.scale,
                            causal=False)
    assert np.all(np.isfinite(out)) and np.array_equal(out, out0) and np.array_equal(lse, lse0)


def test_bad_block_table_is_reported():
    x = gen.make_decode([70], s_q=1, h_q=16, causal=False, seed=71)
    bt = x.block_table.copy()
    bt[0, 1] = x.kv.shape[0]
    with pytest.raises(ValueError):
        orc.attend(x.q, x.kv, bt, x.seqlens, s_q=1, h_q=16, scale=x.scale, causal=False)


# ---- fp8 weights: OCP FP8 E4M3 codes with one fp32 scale per 128 x 128 block,
# decompressed to bf16 before the bmm (the reading stated in the oracle of the
# absorption PR's "fp8 weights decompressed to 16-bit floats").

# Values the E4M3 format fixes (sign, exponent bias 7, 3 mantissa bits,
# subnormals m * 2^-9, max normal S.1111.110, NaN S.1111.111).
E4M3_KNOWN = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
              0x30: 0.5, 0x38: 1.0, 0x39: 1.125, 0x3C: 1.5, 0x40: 2.0, 0x70: 128.0,
              0x77: 240.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0, 0x81: -(2.0 ** -9)}


def test_e4m3_known_codes():
    for code, v in E4M3_KNOWN.items():
        assert orc.e4m3_to_f64(code) == v, hex(code)
    assert math.copysign(1.0, orc.e4m3_to_f64(0x80)) == -1.0 and orc.e4m3_to_f64(0x80) == 0.0
    assert math.isnan(orc.e4m3_to_f64(0x7F)) and math.isnan(orc.e4m3_to_f64(0xFF))


def test_e4m3_code_structure():
    """Positive codes increase with the code; inside a binade (exponent field
    e >= 1) neighbours are 2^(e - 10) apart, subnormals 2^-9; negative codes
    mirror; the only NaNs are 0x7F and 0xFF."""
    v = [orc.e4m3_to_f64(c) for c in range(256)]
    assert [c for c in range(256) if math.isnan(v[c])] == [0x7F, 0xFF]
    for c in range(0x7E):
        e = c >> 3
        step = 2.0 ** (e - 10) if e >= 1 else 2.0 ** -9
        assert v[c + 1] - v[c] == step, hex(c)   # also across binade edges
    for c in range(0x7F):
        assert v[c | 0x80] == -v[c]


def _bf16_exact_rne(x: float) -> float:
    """Nearest value with 8 significant bits (ties to even), by exact
    rational arithmetic -- normal range only."""
    from fractions import Fraction
    f = Fraction(x)
    if f == 0:
        return 0.0
    sign = -1 if f < 0 else 1
    f = abs(f)
    e = math.floor(math.log2(f))
    while Fraction(2) ** e > f:
        e -= 1
    while Fraction(2) ** (e + 1) <= f:
        e += 1
    unit = Fraction(2) ** (e - 7)
    q, r = divmod(f, unit)
    if r * 2 > unit or (r * 2 == unit and q % 2 == 1):
        q += 1
    return sign * float(q * unit)


def test_bf16_rounding_of_exact_products():
    """The decompression rounds e4m3 * scale once: ties go to even, and 500
    random products round as exact rational arithmetic says."""
    def val(bits):
        return float(gen.bf16_bits_to_f32(np.array([bits], dtype=np.uint16))[0])
    assert orc.f64_to_bf16(1 + 2.0 ** -8) == 0x3F80          # tie -> even (1.0)
    assert orc.f64_to_bf16(1 + 3 * 2.0 ** -8) == 0x3F82      # tie -> even (1 + 2^-6)
    assert orc.f64_to_bf16(-(1 + 2.0 ** -8)) == 0xBF80
    assert orc.f64_to_bf16(2.0 ** -133) == 0x0001            # smallest subnormal
    assert orc.f64_to_bf16(2.0 ** -134) == 0x0000            # half of it: tie -> even 0
    assert orc.f64_to_bf16(2.0 ** 128) == 0x7F80             # overflow -> infinity
    rng = np.random.default_rng(11)
    for _ in range(500):
        code = int(rng.integers(0, 256))
        if code & 0x7F == 0x7F:
            continue
        sc = float(np.float32(rng.uniform(1e-5, 1e-2)))
        x = orc.e4m3_to_f64(code) * sc
        assert val(orc.f64_to_bf16(x)) == _bf16_exact_rne(x), (hex(code), sc)


def test_dequant_block_scales_land_on_their_blocks():
    """2 heads of 256 x 384 (2 x 3 blocks, not square): with scale 1 every
    weight is its code's value (exact in bf16); with block (h, i, j) scaled
    by 2^-(6h + 3i + j) every weight of that block is scaled exactly so.  A
    swapped or mis-strided block index fails."""
    rng = np.random.default_rng(12)
    codes = rng.integers(0, 256, size=(2, 256, 384)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38
    ones = np.ones((2, 2, 3), dtype=np.float32)
    w1 = gen.bf16_bits_to_f32(orc.dequant_fp8(codes, ones)).astype(np.float64)
    table = np.array([orc.e4m3_to_f64(c) for c in range(256)])
    assert np.array_equal(w1, table[codes])
    sc = np.array([[[2.0 ** -(6 * h + 3 * i + j) for j in range(3)] for i in range(2)]
                   for h in range(2)], dtype=np.float32)
    w2 = gen.bf16_bits_to_f32(orc.dequant_fp8(codes, sc)).astype(np.float64)
    for h in range(2):
        for i in range(2):
            for j in range(3):
                blk = (h, slice(128 * i, 128 * i + 128), slice(128 * j, 128 * j + 128))
                assert np.array_equal(w2[blk], w1[blk] * sc[h, i, j]), (h, i, j)
    for code, v in E4M3_KNOWN.items():
        assert table[code] == v

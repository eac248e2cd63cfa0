"""Pins of the materialized-vs-sequential absorption oracle (oracle/materialize.py).

The two ways are pinned against scalar fsum loops on tiny shapes and against
each other (associativity: with unrounded materialized weights the chains
agree to fp64 rounding); the bf16 storage rounding against the scalar
rounding of the C oracle and against exact rational round-half-even; the
parameter counts against the products written out by hand for the PR's
shapes."""
import math
from fractions import Fraction

import numpy as np
import pytest

from mla_paged_kv_02_amd import inputs as gen
from oracle import materialize as mat
from oracle import oracle as orc


def _tiny(seed=1, B=3, H=2, r=5, dn=3, c=4, dv=3, dm=6):
    rng = np.random.default_rng(seed)
    return dict(c_q=gen.normal_bf16(rng, (B, r)), w_uq=gen.normal_bf16(rng, (H, r, dn)),
                w_uk=gen.normal_bf16(rng, (H, dn, c)), w_uv=gen.normal_bf16(rng, (H, c, dv)),
                w_o=gen.normal_bf16(rng, (H, dv, dm)), o_lat=gen.normal_bf16(rng, (B, H, c)))


def _f(a):
    return gen.bf16_bits_to_f32(a).astype(np.float64)


def test_products_against_fsum_loops():
    t = _tiny()
    c_q, w_uq, w_uk, w_uv, w_o, o = (_f(t[k]) for k in ("c_q", "w_uq", "w_uk", "w_uv", "w_o",
                                                         "o_lat"))
    B, H, r, dn, c, dv, dm = 3, 2, 5, 3, 4, 3, 6
    wq = mat.materialize_q_uk(t["w_uq"], t["w_uk"])
    wo = mat.materialize_uv_o(t["w_uv"], t["w_o"])
    for h in range(H):
        for i in range(r):
            for n in range(c):
                assert abs(wq[h, i, n] - math.fsum(w_uq[h, i, k] * w_uk[h, k, n]
                                                   for k in range(dn))) < 1e-13
        for i in range(c):
            for m in range(dm):
                assert abs(wo[h, i, m] - math.fsum(w_uv[h, i, e] * w_o[h, e, m]
                                                   for e in range(dv))) < 1e-13
    qs = mat.query_sequential(t["c_q"], t["w_uq"], t["w_uk"])
    for b in range(B):
        for h in range(H):
            nope = [math.fsum(c_q[b, i] * w_uq[h, i, k] for i in range(r)) for k in range(dn)]
            for n in range(c):
                ref = math.fsum(nope[k] * w_uk[h, k, n] for k in range(dn))
                assert abs(qs[b, h, n] - ref) < 1e-12
    ys = mat.output_sequential(t["o_lat"], t["w_uv"], t["w_o"])
    for b in range(B):
        v = [[math.fsum(o[b, h, i] * w_uv[h, i, e] for i in range(c)) for e in range(dv)]
             for h in range(H)]
        for m in range(dm):
            ref = math.fsum(v[h][e] * w_o[h, e, m] for h in range(H) for e in range(dv))
            assert abs(ys[b, m] - ref) < 1e-12


def test_materialized_chain_equals_sequential_chain():
    """Associativity: with the unrounded products the two ways agree to fp64
    rounding, at shapes where a wrong head, transpose or missing sum over
    heads would not."""
    t = _tiny(seed=2, B=4, H=3, r=16, dn=8, c=16, dv=8, dm=12)
    qs = mat.query_sequential(t["c_q"], t["w_uq"], t["w_uk"])
    qm = mat.query_materialized(t["c_q"], mat.materialize_q_uk(t["w_uq"], t["w_uk"]))
    assert np.max(np.abs(qs - qm)) <= 1e-12 * np.max(np.abs(qs))
    ys = mat.output_sequential(t["o_lat"], t["w_uv"], t["w_o"])
    ym = mat.output_materialized(t["o_lat"], mat.materialize_uv_o(t["w_uv"], t["w_o"]))
    assert np.max(np.abs(ys - ym)) <= 1e-12 * np.max(np.abs(ys))
    # the pin separates: one head's materialized weight taken from another head
    bad = mat.materialize_uv_o(t["w_uv"], t["w_o"])[[1, 0, 2]]
    assert np.max(np.abs(mat.output_materialized(t["o_lat"], bad) - ys)) > 1e-3


def test_round_bf16_matches_the_scalar_rounding_and_exact_ties():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(500) * 10.0 ** rng.integers(-30, 30, 500),
                        [0.0, -0.0, 1.0, -1.0, 3e38, 1e-40]])
    # exact midpoints between neighbouring bf16 values: ties to even
    lo = np.float64(1.0) + np.arange(8) * 2.0 ** -7
    x = np.concatenate([x, lo + 2.0 ** -8, -(lo + 2.0 ** -8)])
    got = orc.round_bf16(x)
    for xi, gi in zip(x, got):
        assert gi == orc.f64_to_bf16(xi)
    for k, v in enumerate(lo):
        # (1 + k 2^-7) + 2^-8 rounds to whichever neighbour has an even last bit
        want = v if k % 2 == 0 else v + 2.0 ** -7
        f = Fraction(float(gen.bf16_bits_to_f32(np.array([got[506 + k]], dtype=np.uint16))[0]))
        assert f == Fraction(want)


def test_weight_parameter_counts():
    """At 128 heads, c = 512, dn = dv = 128, r = 1536 and d_model = 7168."""
    p = mat.weight_params(128, 1536, 128, 512, 128, 7168)
    assert p["materialized"] == 128 * 1536 * 512 + 128 * 512 * 7168 == 570425344
    assert p["sequential"] == (128 * 1536 * 128 + 128 * 128 * 512 + 128 * 512 * 128
                               + 128 * 128 * 7168) == 159383552

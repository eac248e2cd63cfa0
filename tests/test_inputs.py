"""Host checks of the seeded input generator (no GPU)."""
import numpy as np

from mla_paged_kv_02_amd import inputs as gen


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.0e38, np.inf,
                  -np.inf, 0.0, -0.0, np.nan, 1.0 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    b = gen.f32_to_bf16_bits(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins;
    # 1 + 3*2^-8 ties between 1+2^-7 and 1+2^-6: even is 1 + 2^-6.
    assert b[0] == 0x3F80 and b[1] == 0x3F80 and b[2] == 0x3F82 and b[3] == 0x3F80
    assert b[4] == 0xC020 and b[6] == 0x7F80 and b[7] == 0xFF80
    assert b[8] == 0 and b[9] == 0x8000 and b[10] == gen.BF16_NAN and b[11] == 0x3F81
    assert gen.bf16_bits_to_f32(b[5:6])[0] > 2.9e38


def test_seeds_reproducible_and_distinct():
    a = gen.make_config("tiny")
    b = gen.make_config("tiny")
    c = gen.make_config("tiny", seed=5)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.kv, b.kv)
    assert not np.array_equal(a.q, c.q)


def test_block_table_and_poison():
    x = gen.make_decode([37, 130, 64, 0], s_q=1, h_q=16, causal=False, seed=3, extra_pages=2)
    nblk = x.blocks()
    used = np.concatenate([x.block_table[b, :nblk[b]] for b in range(x.batch)])
    assert len(np.unique(used)) == len(used) == nblk.sum()
    assert x.kv.shape[0] == nblk.sum() + 2
    for b in range(x.batch):
        assert np.all(x.block_table[b, nblk[b]:] == -1)
    f = gen.bf16_bits_to_f32(x.kv)
    for b, n in enumerate(x.seqlens):
        if n % 64:
            last = x.block_table[b, nblk[b] - 1]
            assert np.all(np.isnan(f[last, n % 64:])) and np.all(np.isfinite(f[last, :n % 64]))
    unused = np.setdiff1d(np.arange(x.kv.shape[0]), used)
    assert np.all(np.isnan(f[unused]))


def test_named_config_shapes():
    x = gen.make_config("tiny")
    assert x.q.shape == (2, 1, 16, 576) and list(x.seqlens) == [37, 130]
    assert abs(x.scale - 192 ** -0.5) < 1e-8 and np.float32(x.scale) == x.scale

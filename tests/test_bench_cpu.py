"""Host-side checks of bench.py: the algorithmic byte and flop counts that
every throughput and roofline figure divides by, against the sizes the
workloads fix (counted here from their definitions), and the one-GPU guard."""
import importlib.util
import os
import subprocess
import sys

import numpy as np

from mla_paged_kv_02_amd import inputs as gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_full_step_byte_and_flop_counts():
    """batch 128, 128 heads, 8192 tokens each: the attention moves Q (128 x 128
    x 576 bf16), every cache row once (128 x 8192 x 1152 B), out (128 x 128 x
    512 bf16) and lse (fp32); each bmm moves x, W and y once."""
    b = _bench()
    x = gen.make_config("full_step")
    assert x.batch == 128 and x.h_q == 128 and np.all(x.seqlens == 8192)
    att = b.algorithmic_bytes(x.seqlens, 1, 128)
    assert att == 128 * 128 * 576 * 2 + 128 * 8192 * 1152 + 128 * 128 * 512 * 2 + 128 * 128 * 4
    assert abs(att / 1e6 - 1243.7) < 0.1
    uk_b, uk_f = b.bmm_bytes_flops(128, 128, 128, 512)
    uv_b, uv_f = b.bmm_bytes_flops(128, 128, 512, 128)
    assert uk_b == uv_b == (128 * 128 * 128 + 128 * 128 * 512 + 128 * 128 * 512) * 2
    assert abs(uk_b / 1e6 - 37.7) < 0.1
    assert uk_f == uv_f == 2 * 128 * 128 * 128 * 512
    flops = b.algorithmic_flops(x.seqlens, 1, 128, False)
    assert flops == 2 * 128 * (128 * 8192) * (576 + 512)


def test_fp8_weight_bytes():
    """fp8 weights: one byte per weight plus an fp32 scale per 128 x 128 block;
    activations stay bf16."""
    b = _bench()
    uk_b, uk_f = b.bmm_bytes_flops(128, 128, 128, 512, True)
    assert uk_b == (128 * 128 * 128 + 128 * 128 * 512) * 2 + 128 * 128 * 512 + 128 * 1 * 4 * 4
    assert uk_f == 2 * 128 * 128 * 128 * 512
    uv_b, _ = b.bmm_bytes_flops(128, 128, 512, 128, True)
    assert uv_b == (128 * 128 * 512 + 128 * 128 * 128) * 2 + 128 * 512 * 128 + 128 * 4 * 1 * 4
    x = gen.make_config("full_step_fp8")
    assert x.extra["w_uk_fp8"].shape == (128, 128, 512) and x.extra["w_uk_scale"].shape == (128, 1, 4)
    assert x.extra["w_uv_fp8"].shape == (128, 512, 128) and x.extra["w_uv_scale"].shape == (128, 4, 1)
    assert not np.any((x.extra["w_uk_fp8"] & 0x7F) == 0x7F)   # no NaN codes


def test_causal_flops_count_each_query_row_once():
    """s_q = 2 causal: query i of a length-n sequence sees n - 1 + i keys."""
    b = _bench()
    seqlens = np.array([5, 1, 0, 9])
    f = b.algorithmic_flops(seqlens, 2, 3, True)
    keys = sum(max(n - 1, 0) + n for n in seqlens)
    assert f == 2 * 3 * keys * (576 + 512)
    assert b.algorithmic_flops(seqlens, 2, 3, False) == 2 * 3 * 2 * seqlens.sum() * (576 + 512)


def test_memory_bound_bytes_match_the_drawn_lengths():
    b = _bench()
    x = gen.make_config("memory_bound")
    rows = x.batch * x.s_q * x.h_q
    want = rows * 576 * 2 + int(x.seqlens.sum()) * 1152 + rows * 512 * 2 + rows * 4
    assert b.algorithmic_bytes(x.seqlens, x.s_q, x.h_q) == want


def test_percentiles_helper():
    b = _bench()
    r = b.pctl([3.0, 1.0, 2.0, 4.0, 5.0])
    assert r["ms"] == 3.0 and r["p10"] < r["ms"] < r["p90"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "1 GPU" in r.stderr or "--gpus 1" in r.stderr


def test_decode_kernel_rule_matches_the_library():
    """The bench names (and looks up traffic for) the kernel the library
    dispatches.  The library's default part count is CUs / row tiles, and
    the row tiles follow the kernel (128 rows for the wide one, one tile for
    its 32-row variant, 16 rows for the 16-row one), so the part count tells
    which kernel the library picks."""
    b = _bench()
    from mla_paged_kv_02_amd import _lib
    lib = _lib.load()
    for s_q, h_q in ((1, 16), (1, 32), (3, 16), (1, 64), (4, 16), (1, 128), (2, 128), (16, 128)):
        rows = s_q * h_q
        kern = b.decode_kernel(rows)
        tiles = (rows + 127) // 128 if kern == "decode_wide_kernel" \
            else 1 if kern == "decode_wide32_kernel" else (rows + 15) // 16
        assert lib.mla_default_num_parts(256, 1, s_q, h_q) == max(1, 256 // tiles), (s_q, h_q)

"""Seeded sweep of decode shapes against the fp64 oracle on the full batch:
every head count the library takes (16, 32, 64, 128), s_q from 1 to 16
(row counts 16 .. 2048, both kernels, partly empty 128-row tiles), causal or
not, batches of 1 to 6 sequences whose lengths mix empty, sub-page, page-edge
and multi-page values, and the default or a drawn scheduler part count.  The
draws are fixed by the seed, so a failure names a reproducible case."""
import numpy as np
import pytest

from mla_paged_kv_02_amd import inputs as gen
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

N_CASES = 24


def _case(i):
    rng = np.random.default_rng(5000 + i)
    h_q = int(rng.choice([16, 32, 64, 128]))
    s_q = int(rng.integers(1, 17))
    causal = bool(rng.integers(0, 2))
    batch = int(rng.integers(1, 7))
    kinds = rng.integers(0, 4, batch)
    lens = [int(v) for v in np.where(kinds == 0, rng.integers(0, 3, batch),
                             np.where(kinds == 1, rng.integers(1, 64, batch),
                             np.where(kinds == 2, 64 * rng.integers(1, 9, batch) + rng.integers(-1, 2, batch),
                                      rng.integers(64, 1200, batch))))]
    parts = None if rng.integers(0, 2) else int(rng.integers(1, 300))
    return dict(h_q=h_q, s_q=s_q, causal=causal, lens=lens, parts=parts, seed=6000 + i)


@pytest.mark.parametrize("i", range(N_CASES))
def test_sweep_case(i):
    c = _case(i)
    x = gen.make_decode(c["lens"], s_q=c["s_q"], h_q=c["h_q"], causal=c["causal"], seed=c["seed"])
    out, lse, meta, parts = gu.run_decode(gu.DeviceInputs(x), c["parts"])
    ro, rl = gu.oracle_decode(x)
    gu.compare(gu.dev_to_f64(out), lse.cpu().numpy().astype(np.float64), ro, rl,
               "sweep case %d %s" % (i, c))

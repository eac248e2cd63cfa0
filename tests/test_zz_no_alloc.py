"""GPU: mla_decode_noalloc (partials in the library's own scratch array)
against mla_decode (partials in a caller's workspace) and the oracle.

Two calls in a row on one device, the second with a smaller input, so the
second reads a scratch array that still holds the first call's partials."""
import numpy as np
import pytest
import torch

import mla_paged_kv_02_amd as mla
from mla_paged_kv_02_amd import inputs as gen
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _both(x):
    d = gu.DeviceInputs(x)
    meta, parts = mla.get_metadata(d.seqlens, x.s_q, x.h_q)
    ref_out, ref_lse = mla.decode(d.q, d.kv, d.bt, d.seqlens, meta, parts, scale=x.scale,
                                  causal=x.causal)
    out = torch.full_like(ref_out, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    mla.decode_noalloc(d.q, d.kv, d.bt, d.seqlens, meta, parts, scale=x.scale,
                       causal=x.causal, out=out, lse=lse)
    torch.cuda.synchronize()
    return out, lse, ref_out, ref_lse


def _check(x, what):
    out, lse, ref_out, ref_lse = _both(x)
    # same kernels, same schedule: bit for bit the workspace entry point's result
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), what
    assert torch.equal(lse, ref_lse), what
    ro, rl = gu.oracle_decode(x)
    gu.compare(gu.dev_to_f64(out), lse.cpu().numpy().astype(np.float64), ro, rl, what)


def test_noalloc_matches_decode_twice_second_smaller():
    # first: the compute-bound workload (128 sequences x 256 rows, its partials
    # near the top of the scratch array); second: a small batch at 16 rows
    # with empty, one-token and tile-edge lengths
    _check(gen.make_config("compute_bound"), "no-alloc compute-bound")
    _check(gen.make_decode([1, 15, 16, 17, 64, 65, 0, 700, 3000], s_q=1, h_q=16, causal=False,
                           seed=71), "no-alloc small")

"""The decode step captured into a HIP graph (torch.cuda.CUDAGraph): every
replay, with eager work of the program between replays, gives bitwise the
eager result.  The captured step holds no memset and the decode keeps no
state between calls (the metadata is only read), so nothing in a replay
depends on what the previous replay left."""
import numpy as np
import pytest
import torch

import mla_paged_kv_02_amd as mla
from mla_paged_kv_02_amd import inputs as gen
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _bufs(x, parts):
    dev = "cuda"
    return dict(
        meta=torch.empty(mla.metadata_ints(x.batch, parts), dtype=torch.int32, device=dev),
        ws=torch.empty(mla.workspace_bytes(x.batch, x.s_q, x.h_q, parts), dtype=torch.uint8,
                       device=dev),
        out=torch.empty((x.batch, x.s_q, x.h_q, 512), dtype=torch.bfloat16, device=dev),
        lse=torch.empty((x.batch, x.s_q, x.h_q), dtype=torch.float32, device=dev))


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("name", ["memory_bound", "skewed", "multi_token_4"])
def test_decode_graph_replays_match_eager(name):
    x = gen.make_config(name)
    d = gu.DeviceInputs(x)
    parts = mla.default_num_parts(x.batch, x.s_q, x.h_q)
    b = _bufs(x, parts)
    e = _bufs(x, parts)   # the program's own eager calls use other buffers

    def step(bb):
        mla.get_metadata(d.seqlens, x.s_q, x.h_q, parts, out=bb["meta"])
        mla.decode(d.q, d.kv, d.bt, d.seqlens, bb["meta"], parts, scale=x.scale,
                   causal=x.causal, workspace=bb["ws"], out=bb["out"], lse=bb["lse"])

    step(e)
    torch.cuda.synchronize()
    ref_out, ref_lse = e["out"].clone(), e["lse"].clone()
    g = _capture(lambda: step(b))
    for i in range(5):
        b["out"].fill_(float("nan"))
        b["ws"].view(torch.float32)[: b["ws"].numel() // 4].fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(b["out"].view(torch.int16), ref_out.view(torch.int16)), "replay %d" % i
        assert torch.equal(b["lse"], ref_lse), "replay %d" % i
        step(e)   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(e["out"].view(torch.int16), ref_out.view(torch.int16))


def test_full_step_fp8_graph_replays_match_eager():
    """The whole fp8-weight step (W_UK bmm, metadata, decode, W_UV bmm)."""
    x = gen.make_config("full_step_fp8")
    ex = x.extra
    d = gu.DeviceInputs(x)
    H = x.h_q
    parts = mla.default_num_parts(x.batch, 1, H)
    q_nope = gu.bits_to_dev(ex["q_nope"])
    w = [torch.from_numpy(ex[k]).cuda() for k in ("w_uk_fp8", "w_uk_scale", "w_uv_fp8",
                                                  "w_uv_scale")]
    b = _bufs(x, parts)
    y = torch.empty((x.batch, H, 128), dtype=torch.bfloat16, device="cuda")

    def step():
        mla.absorb_bmm_fp8w(q_nope, w[0], w[1], d.q[:, 0, :, :512])
        mla.get_metadata(d.seqlens, 1, H, parts, out=b["meta"])
        mla.decode(d.q, d.kv, d.bt, d.seqlens, b["meta"], parts, scale=x.scale,
                   workspace=b["ws"], out=b["out"], lse=b["lse"])
        mla.absorb_bmm_fp8w(b["out"][:, 0], w[2], w[3], y)

    step()
    torch.cuda.synchronize()
    ref = y.clone()
    g = _capture(step)
    for i in range(4):
        y.fill_(float("nan"))
        d.q[:, 0, :, :512].fill_(float("nan"))   # the replay must rewrite q_lat too
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), "replay %d" % i
        step()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16))

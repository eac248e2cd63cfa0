"""GPU checks of the measurement probes: the read probe leaves its sink
alone, the MFMA loop's per-wave result matches the 32x32x16 product of its
register operands worked out on the host, and the LDS probe reports a
cycle count and a real-time tick count for every wave."""
import numpy as np
import pytest
import torch

import mla_paged_kv_02_amd as mla
from mla_paged_kv_02_amd import inputs as gen

pytestmark = pytest.mark.gpu


def _bf16(v):
    return float(gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(np.array([v], dtype=np.float32)))[0])


def test_read_probe_writes_nothing_for_zeros():
    buf = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    mla.probe_read(buf, 2048, sink)
    mla.probe_read(buf[:4096 + 16], 3, sink)    # tail shorter than one unrolled pass
    torch.cuda.synchronize()
    assert int(sink.item()) == 7


def test_mfma_probe_sum_matches_host_product():
    """Lane 32g + m holds A[m][8g + j] = bf16(0.001 (lane + j)) and lane
    32g + n holds B[8g + j][n] = bf16(0.002 (lane - j)); lane 0 keeps rows
    8(r/4) + r%4 of column 0 of C = A B in its 16 accumulator registers.
    Each of the 8 chains adds C `iters` times; lane 0 writes the sum."""
    iters, wgs = 3, 2
    a = np.zeros((32, 16))
    b = np.zeros((16, 32))
    for lane in range(64):
        g, m = divmod(lane, 32)
        for j in range(8):
            a[m, 8 * g + j] = _bf16(np.float32(0.001) * np.float32(lane + j))
            b[8 * g + j, m] = _bf16(np.float32(0.002) * np.float32(lane - j))
    c = a @ b
    rows = [8 * (r // 4) + r % 4 for r in range(16)]
    want = 8 * iters * sum(c[r, 0] for r in rows)
    sink = torch.zeros(4 * wgs, dtype=torch.float32, device="cuda")
    flops = mla.probe_mfma(iters, wgs, sink)
    torch.cuda.synchronize()
    assert flops == wgs * 4 * iters * 8 * 32768
    got = sink.cpu().numpy().astype(np.float64)
    assert np.allclose(got, want, rtol=1e-5, atol=1e-6), (got, want)


def test_lds_probe_reports_every_wave():
    """Every wave of every workgroup writes (cycles, 100 MHz ticks); both grow
    with the iteration count, and the implied shader clock is plausible."""
    wgs, waves = 8, 4
    ticks = torch.zeros(2 * wgs * waves, dtype=torch.int32, device="cuda")
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    res = {}
    for iters in (256, 2048):
        ticks.zero_()
        per_wg = mla.probe_lds(waves, iters, wgs, ticks, sink, depth=8)
        torch.cuda.synchronize()
        assert per_wg == waves * iters * 8 * 1024
        t = ticks.view(wgs * waves, 2).cpu().numpy().astype(np.float64)
        assert np.all(t > 0), t
        res[iters] = t
    assert np.all(res[2048][:, 0] > res[256][:, 0])
    clock_ghz = res[2048][:, 0] / (res[2048][:, 1] * 10.0)   # cycles per 10 ns
    assert np.all((clock_ghz > 0.3) & (clock_ghz < 4.0)), clock_ghz
    assert int(sink.item()) == 7

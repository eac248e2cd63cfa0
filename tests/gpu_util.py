"""Helpers for the GPU parity tests: move generator inputs to the device, run
the library through its C ABI, and compare with the fp64 oracle."""
import numpy as np
import torch

import mla_paged_kv_02_amd as mla
from oracle import oracle as orc

# Tolerances on bf16 outputs against the fp64 oracle, and on lse.
MAX_ABS = 1e-2
MEAN_ABS = 1e-3
LSE_ABS = 1e-3


def bits_to_dev(a: np.ndarray, dev="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


def dev_to_f64(t: torch.Tensor) -> np.ndarray:
    """bf16 device tensor -> exact fp64 host array."""
    bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return orc.bf16_to_f64(bits)


class DeviceInputs:
    def __init__(self, x, dev="cuda"):
        self.x = x
        self.q = bits_to_dev(x.q, dev)
        self.kv = bits_to_dev(x.kv, dev)
        self.bt = torch.from_numpy(x.block_table).to(dev)
        self.seqlens = torch.from_numpy(x.seqlens).to(dev)


def run_decode(d: DeviceInputs, num_parts=None, q=None):
    x = d.x
    meta, parts = mla.get_metadata(d.seqlens, x.s_q, x.h_q, num_parts)
    out, lse = mla.decode(d.q if q is None else q, d.kv, d.bt, d.seqlens, meta, parts,
                          scale=x.scale, causal=x.causal)
    torch.cuda.synchronize()
    return out, lse, meta, parts


def compare(out_gpu: np.ndarray, lse_gpu: np.ndarray, out_ref: np.ndarray, lse_ref: np.ndarray,
            what: str = ""):
    """Assert the documented tolerances; return (max_abs, mean_abs, lse_max)."""
    assert out_gpu.shape == out_ref.shape, (out_gpu.shape, out_ref.shape)
    assert np.all(np.isfinite(out_gpu)), what + ": non-finite output"
    d = np.abs(out_gpu - out_ref)
    # where |ref| >= 4 a bf16 half-ulp exceeds 1e-2: allow one bf16 ulp there
    ulp = np.where(np.abs(out_ref) >= 4, 2.0 ** (np.floor(np.log2(np.abs(out_ref) + 1e-300)) - 7),
                   0.0)
    tol = np.maximum(MAX_ABS, ulp)
    worst = float(np.max(d - tol, initial=-1.0))
    mx, mean = float(d.max(initial=0.0)), float(d.mean()) if d.size else 0.0
    assert worst <= 0, "%s: max abs error %.3g" % (what, mx)
    assert mean <= MEAN_ABS, "%s: mean abs error %.3g" % (what, mean)
    inf_ref = np.isinf(lse_ref)
    assert np.array_equal(np.isinf(lse_gpu), inf_ref), what + ": lse -inf pattern differs"
    assert np.all(lse_gpu[inf_ref] < 0)
    lmax = float(np.max(np.abs(lse_gpu[~inf_ref] - lse_ref[~inf_ref]), initial=0.0))
    assert lmax <= LSE_ABS, "%s: lse error %.3g" % (what, lmax)
    return mx, mean, lmax


def oracle_decode(x, sel=None):
    """Oracle on all sequences, or on the batch subset `sel`."""
    if sel is None:
        return orc.attend(x.q, x.kv, x.block_table, x.seqlens, s_q=x.s_q, h_q=x.h_q,
                          scale=x.scale, causal=x.causal)
    sel = np.asarray(sel)
    return orc.attend(x.q[sel], x.kv, x.block_table[sel], x.seqlens[sel], s_q=x.s_q,
                      h_q=x.h_q, scale=x.scale, causal=x.causal)

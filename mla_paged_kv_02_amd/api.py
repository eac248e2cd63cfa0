"""Thin torch-facing wrappers over the C ABI (argument marshalling only).

Every op here checks tensor dtypes, devices and shapes, then calls the entry
point of the same name in libmla_paged_kv.so on the tensors' current HIP
stream.  torch provides device memory and streams; all arithmetic runs in
the library's kernels.  There is no fallback path: a missing library raises.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _lib

D_QK = 576
D_V = 512
PAGE = 64


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype, device=None, contiguous=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be on a GPU device" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if contiguous and not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def device_cus(device: Optional[int] = None) -> int:
    import ctypes
    if device is None:
        device = torch.cuda.current_device()
    v = ctypes.c_int(0)
    _lib.check(_lib.load().mla_device_cus(int(device), ctypes.byref(v)), "mla_device_cus")
    return int(v.value)


def default_num_parts(batch: int, s_q: int, h_q: int, device: Optional[int] = None,
                      num_cus: Optional[int] = None) -> int:
    if num_cus is None:
        num_cus = device_cus(device)
    return int(_lib.load().mla_default_num_parts(num_cus, batch, s_q, h_q))


def metadata_ints(batch: int, num_parts: int) -> int:
    return int(_lib.load().mla_metadata_ints(batch, num_parts))


def workspace_bytes(batch: int, s_q: int, h_q: int, num_parts: int) -> int:
    return int(_lib.load().mla_workspace_bytes(batch, s_q, h_q, num_parts))


def get_metadata(seqlens: torch.Tensor, s_q: int, h_q: int, num_parts: Optional[int] = None,
                 out: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, int]:
    """Split schedule for the current lengths -> (metadata int32 tensor, num_parts)."""
    _need(seqlens, "seqlens", torch.int32)
    batch = seqlens.shape[0]
    if num_parts is None:
        num_parts = default_num_parts(batch, s_q, h_q, seqlens.device.index)
    n = metadata_ints(batch, num_parts)
    if out is None:
        out = torch.empty(n, dtype=torch.int32, device=seqlens.device)
    _need(out, "metadata", torch.int32, seqlens.device)
    if out.numel() < n:
        raise ValueError("metadata buffer too small (%d < %d ints)" % (out.numel(), n))
    _lib.check(_lib.load().mla_get_metadata(seqlens.data_ptr(), batch, s_q, h_q, num_parts,
                                            out.data_ptr(), _stream(seqlens)),
               "mla_get_metadata")
    return out, num_parts


def split_offsets(metadata: torch.Tensor, batch: int, num_parts: int) -> torch.Tensor:
    """View of the per-sequence partial-slot offsets inside the metadata."""
    base = 8 * num_parts
    return metadata[base:base + batch + 1]


def decode(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
           seqlens: torch.Tensor, metadata: torch.Tensor, num_parts: int, *, scale: float,
           causal: bool = False, workspace: Optional[torch.Tensor] = None,
           out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None
           ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Paged MLA decode.  q [B, s_q, h_q, 576] bf16; kv_cache [P, 64, 576] bf16;
    block_table [B, S] int32; seqlens [B] int32.  Returns (out [B, s_q, h_q, 512]
    bf16, lse [B, s_q, h_q] fp32)."""
    dev = q.device
    _need(q, "q", torch.bfloat16)
    _need(kv_cache, "kv_cache", torch.bfloat16, dev)
    _need(block_table, "block_table", torch.int32, dev)
    _need(seqlens, "seqlens", torch.int32, dev)
    _need(metadata, "metadata", torch.int32, dev)
    if q.dim() != 4 or kv_cache.dim() != 3 or block_table.dim() != 2:
        raise ValueError("q must be 4-D, kv_cache 3-D and block_table 2-D")
    B, s_q, h_q, d_qk = q.shape
    num_pages, page, d_kv = kv_cache.shape
    if d_kv != d_qk:
        raise ValueError("q and kv_cache widths differ (%d vs %d)" % (d_qk, d_kv))
    if block_table.shape[0] != B or seqlens.shape[0] != B:
        raise ValueError("block_table and seqlens must have batch %d rows" % B)
    if metadata.numel() < metadata_ints(B, num_parts):
        raise ValueError("metadata was built for another batch or num_parts")
    need = workspace_bytes(B, s_q, h_q, num_parts)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, dev)
    if out is None:
        out = torch.empty((B, s_q, h_q, D_V), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, s_q, h_q), dtype=torch.float32, device=dev)
    _need(out, "out", torch.bfloat16, dev)
    _need(lse, "lse", torch.float32, dev)
    if tuple(out.shape) != (B, s_q, h_q, D_V) or tuple(lse.shape) != (B, s_q, h_q):
        raise ValueError("out / lse have the wrong shape")
    _lib.check(_lib.load().mla_decode(
        q.data_ptr(), kv_cache.data_ptr(), num_pages, block_table.data_ptr(),
        block_table.stride(0), seqlens.data_ptr(), B, s_q, h_q, d_qk, D_V, page, float(scale),
        int(bool(causal)), metadata.data_ptr(), num_parts, workspace.data_ptr(),
        workspace.numel(), out.data_ptr(), lse.data_ptr(), _stream(q)), "mla_decode")
    return out, lse



def decode_noalloc(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                   seqlens: torch.Tensor, metadata: torch.Tensor, num_parts: int, *,
                   scale: float, causal: bool = False, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """mla_decode_noalloc: the same decode with the split partials in the
    library's own per-device scratch array (no workspace argument; with `out`
    and `lse` given, nothing is allocated on this path either)."""
    dev = q.device
    _need(q, "q", torch.bfloat16)
    _need(kv_cache, "kv_cache", torch.bfloat16, dev)
    _need(block_table, "block_table", torch.int32, dev)
    _need(seqlens, "seqlens", torch.int32, dev)
    _need(metadata, "metadata", torch.int32, dev)
    if q.dim() != 4 or kv_cache.dim() != 3 or block_table.dim() != 2:
        raise ValueError("q must be 4-D, kv_cache 3-D and block_table 2-D")
    B, s_q, h_q, d_qk = q.shape
    num_pages, page, d_kv = kv_cache.shape
    if d_kv != d_qk:
        raise ValueError("q and kv_cache widths differ (%d vs %d)" % (d_qk, d_kv))
    if block_table.shape[0] != B or seqlens.shape[0] != B:
        raise ValueError("block_table and seqlens must have batch %d rows" % B)
    if metadata.numel() < metadata_ints(B, num_parts):
        raise ValueError("metadata was built for another batch or num_parts")
    if out is None:
        out = torch.empty((B, s_q, h_q, D_V), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, s_q, h_q), dtype=torch.float32, device=dev)
    _need(out, "out", torch.bfloat16, dev)
    _need(lse, "lse", torch.float32, dev)
    if tuple(out.shape) != (B, s_q, h_q, D_V) or tuple(lse.shape) != (B, s_q, h_q):
        raise ValueError("out / lse have the wrong shape")
    _lib.check(_lib.load().mla_decode_noalloc(
        q.data_ptr(), kv_cache.data_ptr(), num_pages, block_table.data_ptr(),
        block_table.stride(0), seqlens.data_ptr(), B, s_q, h_q, d_qk, D_V, page, float(scale),
        int(bool(causal)), metadata.data_ptr(), num_parts, out.data_ptr(), lse.data_ptr(),
        _stream(q)), "mla_decode_noalloc")
    return out, lse

def combine(o_part: torch.Tensor, lse_part: torch.Tensor, split_offsets: torch.Tensor,
            s_q: int, h_q: int, out: Optional[torch.Tensor] = None,
            lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Merge split partials.  o_part [T, s_q*h_q, 512] fp32, lse_part [T, s_q*h_q]
    fp32, split_offsets [B+1] int32."""
    dev = o_part.device
    _need(o_part, "o_part", torch.float32)
    _need(lse_part, "lse_part", torch.float32, dev)
    _need(split_offsets, "split_offsets", torch.int32, dev)
    B = split_offsets.shape[0] - 1
    if out is None:
        out = torch.empty((B, s_q, h_q, D_V), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, s_q, h_q), dtype=torch.float32, device=dev)
    _need(out, "out", torch.bfloat16, dev)
    _need(lse, "lse", torch.float32, dev)
    _lib.check(_lib.load().mla_combine(o_part.data_ptr(), lse_part.data_ptr(),
                                       split_offsets.data_ptr(), B, s_q, h_q, D_V,
                                       out.data_ptr(), lse.data_ptr(), _stream(o_part)),
               "mla_combine")
    return out, lse


def absorb_bmm(x: torch.Tensor, w: torch.Tensor, y: Optional[torch.Tensor] = None
               ) -> torch.Tensor:
    """y[b, h, :] = x[b, h, :] @ w[h].  x [B, H, K] bf16 (last dim contiguous,
    any batch/head strides), w [H, K, N] bf16 contiguous; y [B, H, N] may be a
    strided view (e.g. the first 512 columns of the decode query)."""
    dev = x.device
    _need(x, "x", torch.bfloat16, contiguous=False)
    _need(w, "w", torch.bfloat16, dev)
    if x.dim() != 3 or w.dim() != 3:
        raise ValueError("x must be [B, H, K] and w [H, K, N]")
    B, H, K = x.shape
    if w.shape[0] != H or w.shape[1] != K:
        raise ValueError("w must be [H=%d, K=%d, N]" % (H, K))
    N = w.shape[2]
    if y is None:
        y = torch.empty((B, H, N), dtype=torch.bfloat16, device=dev)
    _need(y, "y", torch.bfloat16, dev, contiguous=False)
    if tuple(y.shape) != (B, H, N) or y.stride(2) != 1 or x.stride(2) != 1:
        raise ValueError("x and y need unit stride in their last dim and y shape [B, H, N]")
    _lib.check(_lib.load().mla_absorb_bmm(x.data_ptr(), x.stride(0), x.stride(1), w.data_ptr(),
                                          H, K, N, y.data_ptr(), y.stride(0), y.stride(1), B,
                                          _stream(x)), "mla_absorb_bmm")
    return y


def absorb_bmm_fp8w(x: torch.Tensor, w: torch.Tensor, w_scale: torch.Tensor,
                    y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """absorb_bmm with fp8 weights: w [H, K, N] uint8 E4M3 codes (contiguous),
    w_scale [H, ceil(K/128), ceil(N/128)] float32 (one scale per 128 x 128
    block), decompressed to bf16 inside the kernel."""
    dev = x.device
    _need(x, "x", torch.bfloat16, contiguous=False)
    _need(w, "w", torch.uint8, dev)
    _need(w_scale, "w_scale", torch.float32, dev)
    if x.dim() != 3 or w.dim() != 3 or w_scale.dim() != 3:
        raise ValueError("x must be [B, H, K], w [H, K, N] and w_scale 3-D")
    B, H, K = x.shape
    if w.shape[0] != H or w.shape[1] != K:
        raise ValueError("w must be [H=%d, K=%d, N]" % (H, K))
    N = w.shape[2]
    if tuple(w_scale.shape) != (H, -(-K // 128), -(-N // 128)):
        raise ValueError("w_scale must be [%d, %d, %d]" % (H, -(-K // 128), -(-N // 128)))
    if y is None:
        y = torch.empty((B, H, N), dtype=torch.bfloat16, device=dev)
    _need(y, "y", torch.bfloat16, dev, contiguous=False)
    if tuple(y.shape) != (B, H, N) or y.stride(2) != 1 or x.stride(2) != 1:
        raise ValueError("x and y need unit stride in their last dim and y shape [B, H, N]")
    _lib.check(_lib.load().mla_absorb_bmm_fp8w(
        x.data_ptr(), x.stride(0), x.stride(1), w.data_ptr(), w_scale.data_ptr(), H, K, N,
        y.data_ptr(), y.stride(0), y.stride(1), B, _stream(x)), "mla_absorb_bmm_fp8w")
    return y


def probe_read(buf: torch.Tensor, workgroups: int, sink: Optional[torch.Tensor] = None) -> None:
    """Stream every byte of `buf` (uint8, 16-byte multiple) once on the device."""
    _need(buf, "buf", torch.uint8)
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    _lib.check(_lib.load().mla_probe_read(buf.data_ptr(), buf.numel(), int(workgroups),
                                          sink.data_ptr(), _stream(buf)), "mla_probe_read")


def probe_mfma(iters: int, workgroups: int, sink: torch.Tensor) -> int:
    """Run the dense bf16 MFMA loop; returns its flop count.  sink: float32
    [workgroups * 4] on the device."""
    _need(sink, "sink", torch.float32)
    if sink.numel() < 4 * workgroups:
        raise ValueError("sink needs %d floats" % (4 * workgroups))
    _lib.check(_lib.load().mla_probe_mfma(int(iters), int(workgroups), sink.data_ptr(),
                                          _stream(sink)), "mla_probe_mfma")
    return int(workgroups) * 4 * int(iters) * 8 * 32768


def probe_lds(waves: int, iters: int, workgroups: int, ticks: torch.Tensor,
              sink: Optional[torch.Tensor] = None, depth: int = 4) -> int:
    """Run the LDS read loop (`waves` waves in each of `workgroups`
    workgroups, one per CU, `depth` 1 KB reads in flight per wave); ticks:
    int32 [workgroups * waves * 2] on the device, receiving (shader cycles,
    100 MHz ticks) per wave.  Returns the bytes each workgroup reads."""
    _need(ticks, "ticks", torch.int32)
    if ticks.numel() < 2 * waves * workgroups:
        raise ValueError("ticks needs %d ints" % (2 * waves * workgroups))
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=ticks.device)
    _lib.check(_lib.load().mla_probe_lds(int(waves), int(depth), int(iters), int(workgroups),
                                         ticks.data_ptr(), sink.data_ptr(), _stream(ticks)),
               "mla_probe_lds")
    return int(waves) * int(iters) * int(depth) * 1024

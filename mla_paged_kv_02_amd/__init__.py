"""Multi-head latent attention decode over a paged latent KV cache for AMD
MI355X (gfx950): a C-ABI library of hand-written HIP kernels
(libmla_paged_kv.so, see include/mla_paged_kv.h) and a thin torch binding.

    meta, parts = get_metadata(seqlens, s_q, h_q)
    out, lse = decode(q, kv_cache, block_table, seqlens, meta, parts, scale=s)
"""
from .api import (absorb_bmm, absorb_bmm_fp8w, combine, decode, decode_noalloc, default_num_parts, device_cus, get_metadata,
                  metadata_ints, probe_lds, probe_mfma, probe_read, split_offsets, workspace_bytes)
from ._lib import MlaError

__all__ = ["MlaError", "absorb_bmm", "absorb_bmm_fp8w", "combine", "decode", "decode_noalloc",
           "default_num_parts", "device_cus",
           "get_metadata", "metadata_ints", "probe_lds", "probe_mfma", "probe_read", "split_offsets",
           "workspace_bytes"]

"""The two ways to apply MLA's absorbed projections, on the library's bmm.

"[Attention] MLA get rid of materialization" (PR description) weighs
precomputing the absorbed products W_Q_UK[h] = W_UQ[h] . W_UK[h] and
W_UV_O[h] = W_UV[h] . W_O[h] against applying the factors one after the
other, and keeps the latter: fewer weight bytes and fewer flops per token.
Every product here is one mla_absorb_bmm call (a per-head matmul with
arbitrary batch and head strides; a head stride of 0 broadcasts an operand
over heads, one head with the heads folded into K is a plain matmul), so
the arithmetic runs in the library's kernels; this module only lays out the
views.

Shapes: c_q [B, r] (compressed query), W_UQ [H, r, dn], W_UK [H, dn, c],
W_UV [H, c, dv], W_O [H, dv, d_model] (head h's rows of the [H * dv,
d_model] output projection), o_lat [B, H, c] (any strides with unit last
stride, e.g. the decode output), q_lat written into q[:, 0, :, :c].
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from .api import absorb_bmm


def materialize(w_uq: torch.Tensor, w_uk: torch.Tensor, w_uv: torch.Tensor,
                w_o: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """(W_Q_UK [H, r, c], W_UV_O [H, c, d_model]), bf16, each the per-head
    product of its two factors rounded once."""
    H, r, dn = w_uq.shape
    c, dv, dm = w_uk.shape[2], w_uv.shape[2], w_o.shape[2]
    w_q_uk = torch.empty((H, r, c), dtype=torch.bfloat16, device=w_uq.device)
    # rows i of W_UQ[h] as the batch: x[i, h, :] = W_UQ[h, i, :]
    absorb_bmm(w_uq.permute(1, 0, 2), w_uk, w_q_uk.permute(1, 0, 2))
    w_uv_o = torch.empty((H, c, dm), dtype=torch.bfloat16, device=w_uq.device)
    absorb_bmm(w_uv.permute(1, 0, 2), w_o, w_uv_o.permute(1, 0, 2))
    return w_q_uk, w_uv_o


def query_sequential(c_q: torch.Tensor, w_uq: torch.Tensor, w_uk: torch.Tensor,
                     q_lat_out: torch.Tensor, q_nope: Optional[torch.Tensor] = None
                     ) -> torch.Tensor:
    """q_nope = c_q . W_UQ[h] (c_q shared by every head), then
    q_lat = q_nope . W_UK[h] into q_lat_out [B, H, c] (a view may be strided)."""
    B = c_q.shape[0]
    H, r, dn = w_uq.shape
    if q_nope is None:
        q_nope = torch.empty((B, H, dn), dtype=torch.bfloat16, device=c_q.device)
    absorb_bmm(c_q.unsqueeze(1).expand(B, H, r), w_uq, q_nope)
    absorb_bmm(q_nope, w_uk, q_lat_out)
    return q_nope


def query_materialized(c_q: torch.Tensor, w_q_uk: torch.Tensor, q_lat_out: torch.Tensor) -> None:
    """q_lat = c_q . W_Q_UK[h] into q_lat_out [B, H, c]."""
    B = c_q.shape[0]
    H, r, _ = w_q_uk.shape
    absorb_bmm(c_q.unsqueeze(1).expand(B, H, r), w_q_uk, q_lat_out)


def output_sequential(o_lat: torch.Tensor, w_uv: torch.Tensor, w_o: torch.Tensor,
                      y: Optional[torch.Tensor] = None, v: Optional[torch.Tensor] = None
                      ) -> torch.Tensor:
    """v = o_lat . W_UV[h] ([B, H, dv]), then y = v . W_O summed over heads:
    one matmul over K = H * dv.  Returns y [B, d_model]."""
    B, H, _ = o_lat.shape
    dv, dm = w_uv.shape[2], w_o.shape[2]
    if v is None:
        v = torch.empty((B, H, dv), dtype=torch.bfloat16, device=o_lat.device)
    absorb_bmm(o_lat, w_uv, v)
    if y is None:
        y = torch.empty((B, dm), dtype=torch.bfloat16, device=o_lat.device)
    absorb_bmm(v.reshape(B, 1, H * dv), w_o.reshape(1, H * dv, dm), y.unsqueeze(1))
    return y


def output_materialized(o_lat: torch.Tensor, w_uv_o: torch.Tensor,
                        y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = sum_h o_lat[b, h, :] . W_UV_O[h]: one matmul over K = H * c.
    o_lat must be contiguous over (h, c) so that it reads as [B, H * c]."""
    B, H, c = o_lat.shape
    dm = w_uv_o.shape[2]
    if o_lat.stride(1) != c or o_lat.stride(2) != 1:
        raise ValueError("o_lat must be contiguous over heads and columns")
    if y is None:
        y = torch.empty((B, dm), dtype=torch.bfloat16, device=o_lat.device)
    x = o_lat.as_strided((B, 1, H * c), (o_lat.stride(0), H * c, 1))
    absorb_bmm(x, w_uv_o.reshape(1, H * c, dm), y.unsqueeze(1))
    return y

"""fp64 oracle of the two ways to apply MLA's absorbed projections.

TEST INFRASTRUCTURE ONLY: imported by the test suite and the benchmark's
comparison leg, never by the product package; it shares no code with the
GPU path.

"[Attention] MLA get rid of materialization" (PR description) compares two
ways to apply the query up-projection W_UQ (compressed query -> per-head
nope query), the key up-projection W_UK, the value up-projection W_UV and
the output projection W_O around the latent attention:

  materialized: precompute per head W_Q_UK[h] = W_UQ[h] . W_UK[h] and
    W_UV_O[h] = W_UV[h] . W_O[h], then
      q_lat[b,h,:] = c_q[b,:] . W_Q_UK[h]
      y[b,:]       = sum_h o_lat[b,h,:] . W_UV_O[h]
  sequential (the PR's choice, less weight memory and fewer flops):
      q_nope[b,h,:] = c_q[b,:] . W_UQ[h];   q_lat[b,h,:] = q_nope[b,h,:] . W_UK[h]
      v[b,h,:]      = o_lat[b,h,:] . W_UV[h]; y[b,:] = sum_h v[b,h,:] . W_O[h]

Shapes: c_q [B, r] (r = the query's compression rank), W_UQ [H, r, dn],
W_UK [H, dn, c], W_UV [H, c, dv], W_O [H, dv, d_model] (head h's rows of the
[H * dv, d_model] output projection), o_lat [B, H, c].  The pages give c =
512, dn = dv = 128 and 128 heads; r and d_model are not on them.

In exact arithmetic the two give the same q_lat and y (matrix products are
associative); stored materialized weights are rounded to bf16, which is the
one place they differ here.  Everything is fp64: bf16 inputs are widened
exactly, matrix products are NumPy fp64 products, nothing is rounded on the
way out except by round_bf16 where a caller asks for stored weights.
"""
from __future__ import annotations

import numpy as np

from .oracle import bf16_to_f64, round_bf16


def _f64(a) -> np.ndarray:
    return bf16_to_f64(a) if a.dtype == np.uint16 else np.asarray(a, dtype=np.float64)


def materialize_q_uk(w_uq, w_uk) -> np.ndarray:
    """W_Q_UK[h] = W_UQ[h] . W_UK[h], fp64 [H, r, c]."""
    return np.matmul(_f64(w_uq), _f64(w_uk))


def materialize_uv_o(w_uv, w_o) -> np.ndarray:
    """W_UV_O[h] = W_UV[h] . W_O[h], fp64 [H, c, d_model]."""
    return np.matmul(_f64(w_uv), _f64(w_o))


def query_sequential(c_q, w_uq, w_uk) -> np.ndarray:
    """q_lat [B, H, c] through q_nope [B, H, dn]."""
    q_nope = np.einsum("br,hrd->bhd", _f64(c_q), _f64(w_uq))
    return np.einsum("bhd,hdc->bhc", q_nope, _f64(w_uk))


def query_materialized(c_q, w_q_uk) -> np.ndarray:
    """q_lat [B, H, c] = c_q . W_Q_UK[h]."""
    return np.einsum("br,hrc->bhc", _f64(c_q), _f64(w_q_uk))


def output_sequential(o_lat, w_uv, w_o) -> np.ndarray:
    """y [B, d_model] through v [B, H, dv]."""
    v = np.einsum("bhc,hce->bhe", _f64(o_lat), _f64(w_uv))
    return np.einsum("bhe,hem->bm", v, _f64(w_o))


def output_materialized(o_lat, w_uv_o) -> np.ndarray:
    """y [B, d_model] = sum_h o_lat[b,h,:] . W_UV_O[h]."""
    return np.einsum("bhc,hcm->bm", _f64(o_lat), _f64(w_uv_o))


def stored(w: np.ndarray) -> np.ndarray:
    """A materialized weight as stored: bf16 bits, rounded once."""
    return round_bf16(w)


def weight_params(H: int, r: int, dn: int, c: int, dv: int, d_model: int) -> dict:
    """Parameter counts of the weights each way touches (one layer)."""
    return {"materialized": H * r * c + H * c * d_model,
            "sequential": H * r * dn + H * dn * c + H * c * dv + H * dv * d_model}

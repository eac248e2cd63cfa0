"""Seeded synthetic inputs for paged MLA decode.

This module only draws random numbers and lays them out (bf16 rounding of the
draws, the page permutation, the block table, NaN poisoning of unused cache
rows).  It holds none of the attention arithmetic, so both the GPU path and
the CPU oracle can be fed from it.

Workloads (MLA decode over a paged latent cache with 64-token pages, as in
"DeepSeek publica FlashMLA como codigo abierto", release bullets; sequential
absorption bmms as in "[Attention] MLA get rid of materialization", PR
description).  Every cache row is 576 bf16 values (512 latent + 64 rope).

  tiny           batch 2, s_q 1, h_q 16, lengths {37, 130}
  memory_bound   batch 64, s_q 1, h_q 16, lengths ~ N(4096, 1024) in [1, 8192]
  compute_bound  batch 128, s_q 2 causal, h_q 128, lengths ~ N(4096, 1024) in [2, 8192]
  skewed         batch 32, s_q 1, h_q 16, one length 131072 and 31 of 1024
  full_step      batch 128, h 128, length 8192 each; q_nope [.,.,128],
                 W_UK [128,128,512], W_UV [128,512,128] ~ N(0, 0.02)
  full_step_fp8  the same step with W_UK and W_UV stored as fp8 (E4M3 codes
                 and one fp32 scale per 128 x 128 block, spread near 0.02)

Wider query counts and the context-length sweep (the sequential-bmm PR
measures serving at 1000, 5000, 10000 and 32000 input tokens; these decode
steps at those context lengths stand in for it at the kernel level):

  multi_token_4  batch 64, s_q 4 causal, h_q 16, lengths ~ N(4096, 1024) in [4, 8192]
  multi_token_8  batch 64, s_q 8 causal, h_q 16 (128 rows), same lengths
  len_1k, len_5k, len_10k, len_32k
                 batch 64, s_q 1, h_q 128, every length 1000 / 5000 / 10000 / 32000

Q and the cache are N(0, 1) rounded once to bf16 (round to nearest even);
scale = fp32(192 ** -0.5).  N(mu, sigma) takes sigma as the standard
deviation; sampled lengths are rounded half-to-even, then clipped.

Seeds: numpy SeedSequence(seed).spawn(5) gives independent streams for
[lengths, page permutation, q, cache, weights].
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

D_QK = 576
D_V = 512
D_ROPE = 64
PAGE = 64
SCALE = float(np.float32(192.0 ** -0.5))
BF16_NAN = 0x7FC0

CONFIG_INDEX = {"tiny": 0, "memory_bound": 1, "compute_bound": 2, "skewed": 3, "full_step": 4,
                "multi_token_4": 5, "multi_token_8": 6, "len_1k": 7, "len_5k": 8, "len_10k": 9,
                "len_32k": 10, "full_step_fp8": 11}
SWEEP_LENGTHS = {"len_1k": 1000, "len_5k": 5000, "len_10k": 10000, "len_32k": 32000}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even; NaN -> quiet NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = BF16_NAN
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape, std: float = 1.0,
                chunk: int = 1 << 24) -> np.ndarray:
    """N(0, std) draws rounded to bf16, generated in chunks to bound memory."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        v = rng.standard_normal(e - s, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        out[s:e] = f32_to_bf16_bits(v)
    return out.reshape(shape)


def fp8_weights(rng: np.random.Generator, shape, blk: int = 128, std: float = 0.02):
    """Block-scaled fp8 weights as stored: E4M3 codes drawn as bit patterns
    (random sign, exponent field around 10 -- about 8 -- clipped to [0, 15],
    uniform mantissa; the NaN pattern S.1111.111 replaced by S.1111.110) and
    one positive fp32 scale per blk x blk block of each [K, N] matrix, near
    std / 16, so that code * scale has a standard deviation near std.  Returns (codes
    uint8 [H, K, N], scales float32 [H, ceil(K/blk), ceil(N/blk)])."""
    H, K, N = shape
    sign = rng.integers(0, 2, size=shape, dtype=np.uint8)
    expo = np.clip(np.rint(rng.normal(10.0, 1.0, size=shape)), 0, 15).astype(np.uint8)
    mant = rng.integers(0, 8, size=shape, dtype=np.uint8)
    mant[(expo == 15) & (mant == 7)] = 6
    codes = (sign << 7) | (expo << 3) | mant
    scales = (std / 16.0 * rng.uniform(0.5, 1.5, size=(H, -(-K // blk), -(-N // blk))))
    return codes.astype(np.uint8), scales.astype(np.float32)


@dataclass
class DecodeInputs:
    """Host-side inputs of one decode call (bf16 tensors as uint16 bits)."""
    q: np.ndarray             # uint16 [B, s_q, h_q, 576]
    kv: np.ndarray            # uint16 [num_pages, 64, 576]
    block_table: np.ndarray   # int32 [B, bt_stride]; -1 past each sequence's pages
    seqlens: np.ndarray       # int32 [B]
    s_q: int
    h_q: int
    causal: bool
    scale: float = SCALE
    name: str = "custom"
    extra: dict = field(default_factory=dict)   # full_step weights etc.

    @property
    def batch(self) -> int:
        return int(self.seqlens.shape[0])

    def blocks(self) -> np.ndarray:
        return (self.seqlens.astype(np.int64) + PAGE - 1) // PAGE


def _lengths(name: str, rng: np.random.Generator) -> np.ndarray:
    if name == "tiny":
        return np.array([37, 130], dtype=np.int32)
    if name == "memory_bound":
        return np.clip(np.rint(rng.normal(4096.0, 1024.0, 64)), 1, 8192).astype(np.int32)
    if name == "compute_bound":
        return np.clip(np.rint(rng.normal(4096.0, 1024.0, 128)), 2, 8192).astype(np.int32)
    if name == "skewed":
        n = np.full(32, 1024, dtype=np.int32)
        n[int(rng.integers(0, 32))] = 131072
        return n
    if name in ("full_step", "full_step_fp8"):
        return np.full(128, 8192, dtype=np.int32)
    if name in ("multi_token_4", "multi_token_8"):
        s_q = _SHAPES[name][0]
        return np.clip(np.rint(rng.normal(4096.0, 1024.0, 64)), s_q, 8192).astype(np.int32)
    if name in SWEEP_LENGTHS:
        return np.full(64, SWEEP_LENGTHS[name], dtype=np.int32)
    raise KeyError(name)


_SHAPES = {  # name -> (s_q, h_q, causal)
    "tiny": (1, 16, False),
    "memory_bound": (1, 16, False),
    "compute_bound": (2, 128, True),
    "skewed": (1, 16, False),
    "full_step": (1, 128, False),
    "full_step_fp8": (1, 128, False),
    "multi_token_4": (4, 16, True),
    "multi_token_8": (8, 16, True),
    "len_1k": (1, 128, False),
    "len_5k": (1, 128, False),
    "len_10k": (1, 128, False),
    "len_32k": (1, 128, False),
}


def paged_cache(seqlens: np.ndarray, rng_perm: np.random.Generator,
                rng_kv: np.random.Generator, *, extra_pages: int = 2,
                bt_slack: int = 1, poison: bool = True, permute: bool = True,
                page: int = PAGE, width: int = D_QK):
    """Build a shuffled paged latent cache for the given lengths.

    Logical block t of sequence b holds tokens [page*t, page*t+page); the data are
    drawn in logical order (so a different permutation keeps the content) and
    placed at physical page perm[first_block_of_b + t].  Rows past a
    sequence's length and the `extra_pages` unreferenced pages are NaN when
    `poison`.  Returns (kv uint16 [P, page, width], block_table int32 [B, S]).
    The defaults are the real cache geometry; tests of the oracle alone may
    shrink `page` and `width`.
    """
    seqlens = np.asarray(seqlens, dtype=np.int64)
    nblk = (seqlens + page - 1) // page
    total = int(nblk.sum())
    num_pages = total + extra_pages
    logical = normal_bf16(rng_kv, (total, page, width))
    perm = rng_perm.permutation(num_pages) if permute else np.arange(num_pages)
    kv = np.full((num_pages, page, width), BF16_NAN if poison else 0, dtype=np.uint16)
    kv[perm[:total]] = logical
    del logical
    stride = int(nblk.max(initial=0)) + bt_slack
    bt = np.full((len(seqlens), max(stride, 1)), -1, dtype=np.int32)
    first = np.concatenate([[0], np.cumsum(nblk)[:-1]]).astype(np.int64)
    for b in range(len(seqlens)):
        nb = int(nblk[b])
        bt[b, :nb] = perm[first[b]:first[b] + nb]
        tail = int(seqlens[b] % page)
        if poison and nb and tail:
            kv[bt[b, nb - 1], tail:, :] = BF16_NAN
    return kv, bt


def make_decode(seqlens, *, s_q: int, h_q: int, causal: bool, seed: int,
                name: str = "custom", extra_pages: int = 2, poison: bool = True,
                permute: bool = True, bt_slack: int = 1) -> DecodeInputs:
    """Decode inputs for explicit lengths (tests use this for edge cases)."""
    ss = np.random.SeedSequence(seed).spawn(5)
    rng_perm, rng_q, rng_kv = (np.random.default_rng(ss[i]) for i in (1, 2, 3))
    seqlens = np.asarray(seqlens, dtype=np.int32)
    kv, bt = paged_cache(seqlens, rng_perm, rng_kv, extra_pages=extra_pages,
                         poison=poison, permute=permute, bt_slack=bt_slack)
    q = normal_bf16(rng_q, (len(seqlens), s_q, h_q, D_QK))
    return DecodeInputs(q=q, kv=kv, block_table=bt, seqlens=seqlens, s_q=s_q, h_q=h_q,
                        causal=causal, name=name)


def config_shape(name: str, seed: Optional[int] = None):
    """(seqlens, s_q, h_q, causal) of a named workload: the lengths make_config
    draws with the same seed, without building its cache."""
    if seed is None:
        seed = 1000 + CONFIG_INDEX[name]
    rng_len = np.random.default_rng(np.random.SeedSequence(seed).spawn(5)[0])
    s_q, h_q, causal = _SHAPES[name]
    return _lengths(name, rng_len), s_q, h_q, causal


def make_config(name: str, seed: Optional[int] = None) -> DecodeInputs:
    """One of the named workloads; seed defaults to 1000 + its index."""
    if seed is None:
        seed = 1000 + CONFIG_INDEX[name]
    ss = np.random.SeedSequence(seed).spawn(5)
    rng_perm, rng_q, rng_kv, rng_w = (np.random.default_rng(s) for s in ss[1:])
    seqlens, s_q, h_q, causal = config_shape(name, seed)
    kv, bt = paged_cache(seqlens, rng_perm, rng_kv)
    if name in ("full_step", "full_step_fp8"):
        B, H = len(seqlens), h_q
        q_nope = normal_bf16(rng_q, (B, H, 128))
        q_rope = normal_bf16(rng_q, (B, H, D_ROPE))
        if name == "full_step":
            extra = dict(w_uk=normal_bf16(rng_w, (H, 128, D_V), std=0.02),
                         w_uv=normal_bf16(rng_w, (H, D_V, 128), std=0.02))
        else:
            uk, uk_s = fp8_weights(rng_w, (H, 128, D_V))
            uv, uv_s = fp8_weights(rng_w, (H, D_V, 128))
            extra = dict(w_uk_fp8=uk, w_uk_scale=uk_s, w_uv_fp8=uv, w_uv_scale=uv_s)
        q = np.zeros((B, 1, H, D_QK), dtype=np.uint16)
        q[:, 0, :, D_V:] = q_rope
        return DecodeInputs(q=q, kv=kv, block_table=bt, seqlens=seqlens, s_q=1, h_q=H,
                            causal=False, name=name,
                            extra=dict(q_nope=q_nope, q_rope=q_rope, **extra))
    q = normal_bf16(rng_q, (len(seqlens), s_q, h_q, D_QK))
    return DecodeInputs(q=q, kv=kv, block_table=bt, seqlens=seqlens, s_q=s_q, h_q=h_q,
                        causal=causal, name=name)



# The materialized-vs-sequential absorption comparison: the pages give 128
# heads, a 512-wide latent and 128-wide per-head nope query and value; the
# compressed-query rank (1536) and the model width (7168) are not on them
# and are taken from DeepSeek-V3 / R1, the model the pages serve.
ABSORB_AB_SHAPE = dict(B=128, H=128, r=1536, dn=128, c=512, dv=128, d_model=7168)


def make_absorb_ab(B=128, H=128, r=1536, dn=128, c=512, dv=128, d_model=7168,
                   seed: int = 1100) -> dict:
    """bf16 bits of the compressed query c_q [B, r] (N(0, 1)), the weights
    W_UQ [H, r, dn], W_UK [H, dn, c], W_UV [H, c, dv], W_O [H, dv, d_model]
    (N(0, 0.02)) and a latent attention output o_lat [B, H, c] (N(0, 0.25)),
    each from its own stream of SeedSequence(seed)."""
    ss = np.random.SeedSequence(seed).spawn(6)
    g = [np.random.default_rng(s) for s in ss]
    return dict(c_q=normal_bf16(g[0], (B, r)), w_uq=normal_bf16(g[1], (H, r, dn), std=0.02),
                w_uk=normal_bf16(g[2], (H, dn, c), std=0.02),
                w_uv=normal_bf16(g[3], (H, c, dv), std=0.02),
                w_o=normal_bf16(g[4], (H, dv, d_model), std=0.02),
                o_lat=normal_bf16(g[5], (B, H, c), std=0.25))

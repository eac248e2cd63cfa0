"""Python face of the fp64 CPU oracle for paged MLA decode.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the product package.  It shares
no code with the GPU path; the C file next to it holds the arithmetic and
states the definitions it follows (MLA decode over a 64-token paged latent
cache, "DeepSeek publica FlashMLA como codigo abierto", release bullets;
non-materialized absorption as sequential bmms, "[Attention] MLA get rid of
materialization", PR description).

All functions take NumPy arrays.  bf16 tensors are raw uint16 bit patterns;
they are widened exactly to fp64 here.  Results are fp64 and unrounded.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (plain IEEE fp64, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def bind(lib):
    """Declare the C signatures on a loaded oracle library."""
    P = ctypes.c_void_p
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    lib.oracle_attend.restype = ctypes.c_int
    lib.oracle_attend.argtypes = [P, P, i64, P, i64, P, i32, i32, i32, i32, i32, i32,
                                  ctypes.c_float, i32, P, P, P, P]
    lib.oracle_combine.restype = None
    lib.oracle_combine.argtypes = [P, P, i32, i64, i32, P, P]
    lib.oracle_absorb_bmm.restype = None
    lib.oracle_absorb_bmm.argtypes = [P, P, i32, i32, i32, i32, P]
    lib.oracle_e4m3_to_double.restype = ctypes.c_double
    lib.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
    lib.oracle_double_to_bf16.restype = ctypes.c_uint16
    lib.oracle_double_to_bf16.argtypes = [ctypes.c_double]
    lib.oracle_round_bf16_array.restype = None
    lib.oracle_round_bf16_array.argtypes = [P, i64, P]
    lib.oracle_dequant_fp8.restype = None
    lib.oracle_dequant_fp8.argtypes = [P, P, i32, i32, i32, i32, P]
    lib.oracle_set_threads.argtypes = [i32]
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = bind(ctypes.CDLL(_LIB))
    return _lib


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening: a bf16 pattern is the upper 16 bits of an fp32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def attend(q, kv_bits, block_table, seqlens, *, s_q, h_q, scale, causal,
           page=64, d_qk=None, d_v=512, key_begin=None, key_end=None):
    """MLA decode over a paged latent cache (the definition in mla_oracle.c).

    q           fp64 [B, s_q, h_q, d_qk] (or bf16 bits of that shape)
    kv_bits     uint16 [num_pages, page, d_qk]
    block_table int32 [B, bt_stride]
    seqlens     int32 [B]
    key_begin/key_end  optional int64 [B]: restrict every row of sequence b
                to keys in [key_begin[b], key_end[b]) (a split of the range).
    Returns (out fp64 [B, s_q, h_q, d_v], lse fp64 [B, s_q, h_q]).
    """
    lib = _load()
    if q.dtype == np.uint16:
        q = bf16_to_f64(q)
    q = np.ascontiguousarray(q, dtype=np.float64)
    kv = np.ascontiguousarray(kv_bits, dtype=np.uint16)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    sl = np.ascontiguousarray(seqlens, dtype=np.int32)
    B = sl.shape[0]
    if d_qk is None:
        d_qk = kv.shape[-1]
    assert q.shape == (B, s_q, h_q, d_qk), q.shape
    assert kv.ndim == 3 and kv.shape[1] == page and kv.shape[2] == d_qk
    assert bt.ndim == 2 and bt.shape[0] == B
    out = np.zeros((B, s_q, h_q, d_v), dtype=np.float64)
    lse = np.zeros((B, s_q, h_q), dtype=np.float64)
    kb = None if key_begin is None else np.ascontiguousarray(key_begin, dtype=np.int64)
    ke = None if key_end is None else np.ascontiguousarray(key_end, dtype=np.int64)
    rc = lib.oracle_attend(_ptr(q), _ptr(kv), kv.shape[0], _ptr(bt), bt.shape[1], _ptr(sl),
                           B, s_q, h_q, d_qk, d_v, page, float(np.float32(scale)), int(causal),
                           None if kb is None else _ptr(kb), None if ke is None else _ptr(ke),
                           _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_attend: block table or sequence length out of range")
    return out, lse


def combine(o_parts, lse_parts):
    """Merge partial results.  o_parts [P, ..., d_v], lse_parts [P, ...]."""
    lib = _load()
    o = np.ascontiguousarray(o_parts, dtype=np.float64)
    l = np.ascontiguousarray(lse_parts, dtype=np.float64)
    n_parts, d_v = o.shape[0], o.shape[-1]
    rows = int(np.prod(l.shape[1:]))
    assert o.shape[:-1] == l.shape
    out = np.zeros(o.shape[1:], dtype=np.float64)
    lse = np.zeros(l.shape[1:], dtype=np.float64)
    lib.oracle_combine(_ptr(o), _ptr(l), n_parts, rows, d_v, _ptr(out), _ptr(lse))
    return out, lse


def absorb_bmm(x, w_bits):
    """y[b,h,:] = x[b,h,:] @ W[h] in fp64.  x [B, H, K] fp64 or bf16 bits,
    w_bits uint16 [H, K, N].  Returns fp64 [B, H, N]."""
    lib = _load()
    if x.dtype == np.uint16:
        x = bf16_to_f64(x)
    x = np.ascontiguousarray(x, dtype=np.float64)
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    B, H, K = x.shape
    assert w.shape[0] == H and w.shape[1] == K
    N = w.shape[2]
    y = np.zeros((B, H, N), dtype=np.float64)
    lib.oracle_absorb_bmm(_ptr(x), _ptr(w), B, H, K, N, _ptr(y))
    return y


FP8_BLOCK = 128


def e4m3_to_f64(code: int) -> float:
    """Exact value of one OCP FP8 E4M3 code."""
    return float(_load().oracle_e4m3_to_double(int(code)))


def f64_to_bf16(x: float) -> int:
    """Bit pattern of the bf16 nearest to x (ties to even)."""
    return int(_load().oracle_double_to_bf16(float(x)))


def round_bf16(x) -> np.ndarray:
    """Bit patterns of x (fp64) rounded once to bf16, nearest even."""
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.zeros(a.shape, dtype=np.uint16)
    _load().oracle_round_bf16_array(_ptr(a), a.size, _ptr(out))
    return out


def dequant_fp8(codes, scales, blk: int = FP8_BLOCK):
    """Decompress E4M3 weights to bf16 bits: W = bf16(e4m3(code) * scale of its
    blk x blk block).  codes uint8 [H, K, N], scales fp32 [H, ceil(K/blk),
    ceil(N/blk)]."""
    lib = _load()
    q = np.ascontiguousarray(codes, dtype=np.uint8)
    sc = np.ascontiguousarray(scales, dtype=np.float32)
    H, K, N = q.shape
    assert sc.shape == (H, -(-K // blk), -(-N // blk)), sc.shape
    w = np.zeros((H, K, N), dtype=np.uint16)
    lib.oracle_dequant_fp8(_ptr(q), _ptr(sc), H, K, N, blk, _ptr(w))
    return w


def absorb_bmm_fp8(x, codes, scales, blk: int = FP8_BLOCK):
    """The absorption bmm with block-scaled fp8 weights decompressed to bf16
    first (fp64 product of x and the bf16 weights)."""
    return absorb_bmm(x, dequant_fp8(codes, scales, blk))


def full_step(q_nope_bits, q_rope_bits, w_uk_bits, w_uv_bits, kv_bits, block_table,
              seqlens, *, scale, page=64):
    """One decode step with non-materialized absorption, all in fp64:
    q_lat = q_nope . W_UK; q = [q_lat | q_rope]; attention over the latent
    cache (s_q = 1, no mask); y = o_lat . W_UV.

    q_nope_bits [B, H, dn], q_rope_bits [B, H, dr], w_uk_bits [H, dn, d_lat],
    w_uv_bits [H, d_lat, dv_head].  Returns (q_lat, o_lat, lse, y), fp64."""
    q_lat = absorb_bmm(q_nope_bits, w_uk_bits)                   # [B, H, d_lat]
    q = np.concatenate([q_lat, bf16_to_f64(q_rope_bits)], axis=-1)  # [B, H, d_lat+dr]
    B, H, d_qk = q.shape
    d_lat = q_lat.shape[-1]
    o_lat, lse = attend(q.reshape(B, 1, H, d_qk), kv_bits, block_table, seqlens,
                        s_q=1, h_q=H, scale=scale, causal=False, page=page, d_v=d_lat)
    o_lat = o_lat.reshape(B, H, d_lat)
    # the second bmm takes o_lat unrounded (fp64 chain end to end)
    y = absorb_bmm(o_lat, w_uv_bits)
    return q_lat, o_lat, lse.reshape(B, H), y

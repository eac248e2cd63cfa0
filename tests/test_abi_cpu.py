"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before any launch (no GPU needed).

Every call below fails validation by construction; none reaches a launch.
"""
import ctypes
import os
import re

import pytest

from mla_paged_kv_02_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "mla_paged_kv.h")
FAKE = 0x10000   # aligned non-null address; never dereferenced (validation fails first)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), "missing export " + n
    assert set(names) == set(_lib.SYMBOLS)


def test_status_strings(lib):
    assert _lib.status_str(0) == "MLA_OK"
    assert _lib.status_str(3) == "MLA_ERR_WORKSPACE"
    assert _lib.status_str(99) == "MLA_ERR_UNKNOWN"


def test_sizes(lib):
    # records, split offsets, total, extra merge offsets
    assert lib.mla_metadata_ints(64, 256) == 8 * 256 + (64 + 1) + 1 + (64 + 1)
    assert lib.mla_workspace_bytes(64, 1, 16, 256) == (64 + 256) * 16 * 513 * 4
    assert lib.mla_default_num_parts(256, 64, 1, 16) == 256
    assert lib.mla_default_num_parts(256, 128, 2, 128) == 128   # two 128-row tiles
    assert lib.mla_default_num_parts(256, 8, 1, 128) == 256     # one 128-row tile
    assert lib.mla_default_num_parts(256, 8, 3, 32) == 256      # 96 rows: one partial 128-row tile
    assert lib.mla_default_num_parts(256, 8, 5, 32) == 128      # 160 rows: two 128-row tiles
    assert lib.mla_default_num_parts(256, 8, 2, 16) == 256      # 32 rows: one 32-row tile
    assert lib.mla_default_num_parts(256, 8, 1, 16) == 256      # 16 rows: one 16-row tile


def _decode(lib, **kw):
    a = dict(q=FAKE, kv=FAKE, num_pages=10, bt=FAKE, bt_stride=4, seqlens=FAKE, batch=2, s_q=1,
             h_q=16, d_qk=576, d_v=512, page=64, scale=0.07, causal=0, meta=FAKE, parts=4,
             ws=FAKE, ws_bytes=0, out=FAKE, lse=FAKE)
    a.update(kw)
    return lib.mla_decode(a["q"], a["kv"], a["num_pages"], a["bt"], a["bt_stride"], a["seqlens"],
                          a["batch"], a["s_q"], a["h_q"], a["d_qk"], a["d_v"], a["page"],
                          a["scale"], a["causal"], a["meta"], a["parts"], a["ws"], a["ws_bytes"],
                          a["out"], a["lse"], None)


def test_decode_validation(lib):
    assert _decode(lib, q=None) == _lib.MLA_ERR_INVALID_ARG
    assert "non-null" in _lib.last_error()
    assert _decode(lib, h_q=8) == _lib.MLA_ERR_UNSUPPORTED
    assert _decode(lib, d_qk=512) == _lib.MLA_ERR_UNSUPPORTED
    assert _decode(lib, page=16) == _lib.MLA_ERR_UNSUPPORTED
    assert _decode(lib, s_q=0) == _lib.MLA_ERR_UNSUPPORTED
    assert _decode(lib, batch=0) == _lib.MLA_ERR_INVALID_ARG
    assert _decode(lib, causal=2) == _lib.MLA_ERR_INVALID_ARG
    assert _decode(lib, scale=float("nan")) == _lib.MLA_ERR_INVALID_ARG
    assert _decode(lib, scale=float("inf")) == _lib.MLA_ERR_INVALID_ARG
    # the softmax scale must be positive: the 128-row kernel masks and takes
    # row maxima before scaling, which preserves the order only for scale > 0
    assert _decode(lib, scale=0.0) == _lib.MLA_ERR_INVALID_ARG
    assert _decode(lib, scale=-0.07) == _lib.MLA_ERR_INVALID_ARG
    assert "positive" in _lib.last_error()
    assert _decode(lib, parts=0) == _lib.MLA_ERR_INVALID_ARG
    assert _decode(lib, q=FAKE + 2) == _lib.MLA_ERR_INVALID_ARG
    assert _decode(lib, ws_bytes=100) == _lib.MLA_ERR_WORKSPACE
    assert "workspace needs" in _lib.last_error()
    assert _decode(lib, ws=None, ws_bytes=1 << 30) == _lib.MLA_ERR_WORKSPACE


def _decode_noalloc(lib, **kw):
    a = dict(q=FAKE, kv=FAKE, num_pages=10, bt=FAKE, bt_stride=4, seqlens=FAKE, batch=2, s_q=1,
             h_q=16, d_qk=576, d_v=512, page=64, scale=0.07, causal=0, meta=FAKE, parts=4,
             out=FAKE, lse=FAKE)
    a.update(kw)
    return lib.mla_decode_noalloc(a["q"], a["kv"], a["num_pages"], a["bt"], a["bt_stride"],
                                  a["seqlens"], a["batch"], a["s_q"], a["h_q"], a["d_qk"],
                                  a["d_v"], a["page"], a["scale"], a["causal"], a["meta"],
                                  a["parts"], a["out"], a["lse"], None)


def test_decode_noalloc_validation(lib):
    """The same argument checks as mla_decode, and a shape whose partials do
    not fit the library's scratch array is refused before any device call."""
    assert _decode_noalloc(lib, q=None) == _lib.MLA_ERR_INVALID_ARG
    assert _decode_noalloc(lib, h_q=8) == _lib.MLA_ERR_UNSUPPORTED
    assert _decode_noalloc(lib, scale=0.0) == _lib.MLA_ERR_INVALID_ARG
    # (batch + parts) * rows * 513 * 4 bytes: 8192 sequences at 128 rows do not fit
    need = lib.mla_workspace_bytes(8192, 1, 128, 256)
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    assert _decode_noalloc(lib, batch=8192, h_q=128, parts=256) == _lib.MLA_ERR_WORKSPACE
    assert "scratch" in _lib.last_error() and str(need) in _lib.last_error()
    # the workloads' shapes fit: compute-bound (128 x 256 rows, 128 parts) and
    # full step (128 x 128 rows, 256 parts)
    assert lib.mla_workspace_bytes(128, 2, 128, 128) <= _lib.NOALLOC_SCRATCH_BYTES
    assert lib.mla_workspace_bytes(128, 1, 128, 256) <= _lib.NOALLOC_SCRATCH_BYTES


def test_noalloc_scratch_size_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define MLA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.NOALLOC_SCRATCH_BYTES


def test_other_validation(lib):
    assert lib.mla_get_metadata(None, 2, 1, 16, 4, FAKE, None) == _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_get_metadata(FAKE, 20000, 1, 16, 4, FAKE, None) == _lib.MLA_ERR_UNSUPPORTED
    assert lib.mla_get_metadata(FAKE, 2, 1, 16, 0, FAKE, None) == _lib.MLA_ERR_INVALID_ARG
    # part records are stored 16 bytes at a time
    assert lib.mla_get_metadata(FAKE, 2, 1, 16, 4, FAKE + 4, None) == _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_combine(FAKE, FAKE, FAKE, 2, 1, 16, 256, FAKE, FAKE, None) == \
        _lib.MLA_ERR_UNSUPPORTED
    assert lib.mla_combine(None, FAKE, FAKE, 2, 1, 16, 512, FAKE, FAKE, None) == \
        _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_absorb_bmm(FAKE, 0, 0, FAKE, 4, 100, 64, FAKE, 0, 0, 2, None) == \
        _lib.MLA_ERR_UNSUPPORTED
    assert lib.mla_absorb_bmm(FAKE, 3, 0, FAKE, 4, 128, 64, FAKE, 0, 0, 2, None) == \
        _lib.MLA_ERR_INVALID_ARG
    # (heads rounded up to 8) x (N / 64) x ceil(batch / 64) workgroups must stay below 2^24
    assert lib.mla_absorb_bmm(FAKE, 0, 0, FAKE, 65535, 32, 6400, FAKE, 0, 0, 192, None) == \
        _lib.MLA_ERR_UNSUPPORTED
    assert lib.mla_device_cus(0, None) == _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_absorb_bmm_fp8w(FAKE, 0, 0, FAKE, None, 4, 128, 64, FAKE, 0, 0, 2, None) == \
        _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_absorb_bmm_fp8w(FAKE, 0, 0, FAKE, FAKE, 4, 100, 64, FAKE, 0, 0, 2, None) == \
        _lib.MLA_ERR_UNSUPPORTED
    assert lib.mla_absorb_bmm_fp8w(FAKE, 0, 0, FAKE + 8, FAKE, 4, 128, 64, FAKE, 0, 0, 2,
                                   None) == _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_probe_read(FAKE, 100, 8, FAKE, None) == _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_probe_read(FAKE + 8, 1 << 20, 8, FAKE, None) == _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_probe_read(FAKE, 1 << 20, 0, FAKE, None) == _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_probe_mfma(0, 8, FAKE, None) == _lib.MLA_ERR_INVALID_ARG
    assert lib.mla_probe_mfma(16, 8, None, None) == _lib.MLA_ERR_INVALID_ARG


def test_default_library_has_no_timing_hook(lib):
    # per-workgroup timestamps exist only in the separately built instrumented
    # copy; the library the tests and the benchmark load writes none
    assert not hasattr(lib, "mla_stamps_set")
    from mla_paged_kv_02_amd import build
    assert build.STAMPS_LIB != _lib.LIB_PATH

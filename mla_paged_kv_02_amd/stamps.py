"""When each decode workgroup starts and ends, and where its time goes, from
the instrumented build.

    python -m mla_paged_kv_02_amd.build --stamps
    python -m mla_paged_kv_02_amd.stamps --config memory_bound --reps 20

The instrumented library (libmla_paged_kv_stamps.so: the same sources built
with MLA_STAMPS=1) makes every workgroup of the decode kernels write a
timing record (csrc/stamps.h): its start and end (s_memrealtime, 100 MHz)
and the ticks it spent in segment set-up, in the key loop and in the merge
and stores, with its segment count.  Workgroups are numbered in dispatch
order, x fastest, and consecutive numbers go to the eight XCDs in turn, so
number mod 8 is the XCD.  For each call the script measures times from the
first start and prints, as one JSON line, medians over the calls of: the
kernel span (last end), the median workgroup end, the tail (last end minus
median end), the median workgroup duration, the median per workgroup of
each phase and the mean segments per workgroup, per XCD the median and last
end, and the whole mla_decode call (decode and merge kernels) timed with HIP
events on its stream (host launch time included: each call is synchronized
before the next).  As in the benchmark, consecutive calls read different
copies of the cache (at least 1 GiB in all), so the last-level cache does
not serve a call what the previous one read.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys

import numpy as np


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--config", default="memory_bound")
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--num-parts", type=int, default=0)
    args = ap.parse_args(argv)

    import torch
    from . import _lib, api, inputs as gen
    from .build import STAMPS_LIB

    if not os.path.exists(STAMPS_LIB):
        print("build it first: python -m mla_paged_kv_02_amd.build --stamps", file=sys.stderr)
        return 2
    _lib._lib = None
    _lib.LIB_PATH = STAMPS_LIB
    lib = _lib.load()
    lib.mla_stamps_set.restype = ctypes.c_int
    lib.mla_stamps_set.argtypes = [ctypes.c_void_p]

    dev = torch.device("cuda:0")
    x = gen.make_config(args.config)

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    q, kv = to_dev(x.q), to_dev(x.kv)
    replicas = max(2, int(np.ceil((1 << 30) / kv.numel() / 2)))
    kvs = [kv] + [kv.clone() for _ in range(replicas - 1)]
    bt = torch.from_numpy(x.block_table).to(dev)
    seqlens = torch.from_numpy(x.seqlens).to(dev)
    parts = args.num_parts or api.default_num_parts(x.batch, x.s_q, x.h_q, 0)
    rows = x.s_q * x.h_q
    # an upper bound on the grid: parts x (16-row tiles), enough for either kernel
    wgs = parts * ((rows + 15) // 16)
    words = 8                                            # kStampWords in csrc/stamps.h
    stamps = torch.zeros(words * wgs, dtype=torch.int64, device=dev)
    _lib.check(lib.mla_stamps_set(stamps.data_ptr()), "mla_stamps_set")
    meta, parts = api.get_metadata(seqlens, x.s_q, x.h_q, parts)
    out = torch.empty((x.batch, x.s_q, x.h_q, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((x.batch, x.s_q, x.h_q), dtype=torch.float32, device=dev)
    ws = torch.empty(api.workspace_bytes(x.batch, x.s_q, x.h_q, parts), dtype=torch.uint8,
                     device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    spans, meds, tails, durs, per_xcd, calls, phases, segs = [], [], [], [], [], [], [], []
    try:
        for i in range(args.reps + 2):
            stamps.zero_()
            e0.record()
            api.decode(q, kvs[i % replicas], bt, seqlens, meta, parts, scale=x.scale,
                       causal=x.causal, workspace=ws, out=out, lse=lse)
            e1.record()
            torch.cuda.synchronize()
            if i < 2:
                continue                                 # warm-up calls
            calls.append(e0.elapsed_time(e1) * 1e3)
            raw = stamps.cpu().numpy().reshape(-1, words)
            ids = np.nonzero(raw[:, 0] > 0)[0]                  # launched workgroups only
            t = raw[ids, :5].astype(np.float64) / 100.0         # 100 MHz ticks -> µs
            phases.append(np.median(t[:, 2:5], axis=0))
            segs.append(raw[ids, 5].mean())
            t0 = t[:, 0].min()
            start, end = t[:, 0] - t0, t[:, 1] - t0
            spans.append(end.max())
            meds.append(np.median(end))
            tails.append(end.max() - np.median(end))
            durs.append(np.median(end - start))
            per_xcd.append([(np.median(end[ids % 8 == k]), end[ids % 8 == k].max())
                            for k in range(8) if np.any(ids % 8 == k)])
    finally:
        lib.mla_stamps_set(None)
    px = np.median(np.array(per_xcd), axis=0)
    print(json.dumps({
        "config": args.config, "workgroups": int(len(ids)), "calls": args.reps,
        "cache_replicas": replicas,
        "call_us": round(float(np.median(calls)), 2),
        "span_us": round(float(np.median(spans)), 2),
        "median_end_us": round(float(np.median(meds)), 2),
        "tail_us": round(float(np.median(tails)), 2),
        "median_workgroup_us": round(float(np.median(durs)), 2),
        "median_setup_us": round(float(np.median([v[0] for v in phases])), 2),
        "median_loop_us": round(float(np.median([v[1] for v in phases])), 2),
        "median_merge_us": round(float(np.median([v[2] for v in phases])), 2),
        "segments_per_workgroup": round(float(np.median(segs)), 3),
        "xcd_median_end_us": [round(float(v), 2) for v in px[:, 0]],
        "xcd_last_end_us": [round(float(v), 2) for v in px[:, 1]],
    }))
    return 0


if __name__ == "__main__":
    sys.exit(main())

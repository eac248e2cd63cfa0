"""Benchmark: paged MLA decode on one MI355X.

A step is one pass of the decode hot path over one batch: the split
schedule (mla_get_metadata) and the decode with its split-KV merge
(mla_decode); for the full-step workload also the two absorbed-weight bmms
around it (mla_absorb_bmm: q_nope . W_UK into the latent query, o_lat . W_UV
after), each stage timed on its own as well.  The default workload is the
memory-bound configuration
(batch 64, s_q 1, h_q 16, lengths ~ N(4096, 1024) clipped to [1, 8192],
shuffled 64-token pages of 576-wide bf16 latent rows); without --config the
line also carries the compute-bound configuration (batch 128, s_q 2 causal,
h_q 128) under "compute_bound", timed the same way, so that both halves of
the metric -- HBM GB/s and bf16 TFLOP/s -- come from one run.  Inputs are resident
in HBM before timing; the cache is replicated so consecutive steps read
different copies and no step is served from the 256 MB last-level cache
warmed by the previous one.

Prints one JSON line.  Throughput is algorithmic bytes (Q + each attended
cache row once per sequence + out + lse) per second; TFLOP/s uses
2 * h_q * keys * (576 + 512).  The roofline fraction is against the
published MI355X peaks; `measured_peaks` adds what a plain streaming read
and a dense bf16 MFMA loop reach on the same device, and the fraction of
that.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged MLA decode: achieved HBM GB/s + bf16 TFLOPS (% roofline), s_k≈4096"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
D_QK, D_V = 576, 512

HERE = os.path.dirname(os.path.abspath(__file__))

WORKLOADS = {
    "memory_bound": "batch 64, s_q 1, h_q 16, d 576/512, seqlens ~N(4096,1024) clipped [1,8192], "
                    "page 64, shuffled pages, bf16 N(0,1), scale 192^-0.5",
    "compute_bound": "batch 128, s_q 2 causal, h_q 128, d 576/512, seqlens ~N(4096,1024) clipped "
                     "[2,8192], page 64, shuffled pages, bf16 N(0,1), scale 192^-0.5",
    "skewed": "batch 32, s_q 1, h_q 16, one seq of 131072 + 31 of 1024, page 64, bf16 N(0,1)",
    "tiny": "batch 2, s_q 1, h_q 16, seqlens {37,130}, page 64",
    "multi_token_4": "batch 64, s_q 4 causal (multi-token / speculative decode), h_q 16, d 576/512, "
                     "seqlens ~N(4096,1024) clipped [4,8192], page 64, shuffled pages, bf16 N(0,1)",
    "multi_token_8": "batch 64, s_q 8 causal, h_q 16 (128 rows per sequence), d 576/512, "
                     "seqlens ~N(4096,1024) clipped [8,8192], page 64, shuffled pages, bf16 N(0,1)",
    "len_1k": "batch 64, s_q 1, h_q 128, every sequence 1000 tokens, page 64, shuffled pages",
    "len_5k": "batch 64, s_q 1, h_q 128, every sequence 5000 tokens, page 64, shuffled pages",
    "len_10k": "batch 64, s_q 1, h_q 128, every sequence 10000 tokens, page 64, shuffled pages",
    "len_32k": "batch 64, s_q 1, h_q 128, every sequence 32000 tokens, page 64, shuffled pages",
    "full_step": "batch 128, h 128, 8192 tokens each, page 64, shuffled pages; q_nope [.,128] x "
                 "W_UK[128,128,512] bmm -> latent q (+64 rope) -> paged attention -> o_lat x "
                 "W_UV[128,512,128] bmm; bf16 N(0,1) activations and cache, N(0,0.02) weights",
    "full_step_fp8": "full_step with W_UK and W_UV stored as fp8 (OCP E4M3 codes, one fp32 "
                     "scale per 128x128 block) and decompressed to bf16 inside the bmm kernels",
}


def measured_peaks(mla, torch, dev, read_gib=2, mfma_iters=4096, reps=10):
    """What this device reaches on a plain 16-byte streaming read of
    read_gib GiB (2 workgroups per CU) and on a dense bf16 MFMA loop (four
    workgroups of four waves per CU), medians of `reps` timed runs after two
    warm-up runs."""
    cus = mla.device_cus(dev.index or 0)
    stream = torch.cuda.current_stream(dev)
    buf = torch.empty(read_gib << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    wg_mfma = 4 * cus
    fsink = torch.zeros(4 * wg_mfma, dtype=torch.float32, device=dev)

    def timed(fn):
        for _ in range(2):
            fn()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b) / 1e3)
        return float(np.median(ts))

    t_read = timed(lambda: mla.probe_read(buf, 2 * cus, sink))
    flops = mla.probe_mfma(mfma_iters, wg_mfma, fsink)
    t_mfma = timed(lambda: mla.probe_mfma(mfma_iters, wg_mfma, fsink))
    del buf
    lds = {(w, d): lds_rate(mla, torch, dev, cus, w, d) for w in (1, 4, 8) for d in (4, 16)}
    return {"hbm_read_GBs": round((read_gib << 30) / t_read / 1e9, 1),
            "bf16_mfma_TFLOPs": round(flops / t_mfma / 1e12, 1),
            "lds_read_B_per_clk_per_CU": {"%d_waves_%d_deep" % k: r[0] for k, r in lds.items()},
            "lds_read_clk_per_KB_per_wave": {"%d_waves_%d_deep" % k: r[1] for k, r in lds.items()},
            "probe": "mla_probe_read over %d GiB, %d workgroups; mla_probe_mfma %d iters x 8 "
                     "v_mfma_f32_32x32x16_bf16 per wave, %d workgroups of 4 waves; mla_probe_lds "
                     "ds_read_b128 4 or 16 in flight per wave, one workgroup per CU, shader clock "
                     "cycles of the slowest wave" % (read_gib, 2 * cus, mfma_iters, wg_mfma)}


def lds_rate(mla, torch, dev, cus, waves, depth, iters=1024):
    """LDS bytes read per shader clock per CU with `waves` waves per CU each
    streaming ds_read_b128 with `depth` in flight (mla_probe_lds), and clocks
    per 1 KB read per wave; medians over the workgroups of a warm second run."""
    ticks = torch.zeros(2 * waves * cus, dtype=torch.int32, device=dev)
    for _ in range(2):
        per_wg = mla.probe_lds(waves, iters, cus, ticks, depth=depth)
        torch.cuda.synchronize()
    cyc = ticks.view(cus, waves, 2)[:, :, 0].cpu().numpy().astype(np.float64)
    slowest = cyc.max(axis=1)
    return (round(float(np.median(per_wg / slowest)), 1),
            round(float(np.median(cyc / (depth * iters))), 1))


def bmm_bytes_flops(batch, heads, k, n, fp8w=False):
    """One absorbed-weight bmm y[b,h,:] = x[b,h,:] . W[h]: x and y bf16, W bf16
    or (fp8w) one-byte codes plus an fp32 scale per 128 x 128 block."""
    w = heads * k * n * (1 if fp8w else 2)
    if fp8w:
        w += heads * -(-k // 128) * -(-n // 128) * 4
    return (batch * heads * k + batch * heads * n) * 2 + w, 2 * batch * heads * k * n


def pctl(v):
    v = np.asarray(v, dtype=np.float64)
    return {"ms": round(float(np.median(v)), 5), "p10": round(float(np.percentile(v, 10)), 5),
            "p90": round(float(np.percentile(v, 90)), 5)}


def algorithmic_bytes(seqlens, s_q, h_q):
    """Q + every attended cache row once per sequence + out (bf16) + lse (fp32)."""
    seqlens = np.asarray(seqlens, dtype=np.int64)
    rows = len(seqlens) * s_q * h_q
    return rows * D_QK * 2 + int(seqlens.sum()) * D_QK * 2 + rows * D_V * 2 + rows * 4


def algorithmic_flops(seqlens, s_q, h_q, causal):
    seqlens = np.asarray(seqlens, dtype=np.int64)
    keys = 0
    for i in range(s_q):
        L = seqlens - s_q + 1 + i if causal else seqlens
        keys += int(np.clip(L, 0, None).sum())
    return 2 * h_q * keys * (D_QK + D_V)


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_attend_rate(orc, x, sel, min_seconds, max_reps=200):
    """Median seconds of the fp64 oracle on the sequences `sel` of x (repeated
    until `min_seconds` have passed), and the algorithmic bytes of that
    sample."""
    q, bt, sl = x.q[sel], x.block_table[sel], x.seqlens[sel]
    times = []
    t_end = time.perf_counter() + min_seconds
    while True:
        t0 = time.perf_counter()
        orc.attend(q, x.kv, bt, sl, s_q=x.s_q, h_q=x.h_q, scale=x.scale, causal=x.causal)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() >= t_end or len(times) >= max_reps:
            break
    return (float(np.median(times)), algorithmic_bytes(sl, x.s_q, x.h_q), len(times),
            algorithmic_flops(sl, x.s_q, x.h_q, x.causal))


def cpu_baseline(x, min_seconds: float, one_core_seconds: float = 3.0):
    """The fp64 oracle on the host cores: its GB/s on the same algorithmic
    bytes, on all the host's threads and on one.  The all-thread figure
    covers the full batch when a pass fits in `min_seconds`, else the first
    sequences that do; the one-thread figure the first sequences that fit in
    about `one_core_seconds`.  For the full step: the oracle's fp64 chain on
    the first sequences, as many as fit the time."""
    from oracle import oracle as orc
    threads = orc.max_threads()
    base = {"kind": "oracle", "unit": "GB/s", "cpu_model": cpu_model(),
            "host_threads": os.cpu_count()}
    if x.name in ("full_step", "full_step_fp8"):
        e = x.extra
        fp8w = x.name == "full_step_fp8"
        if fp8w:   # decompressed once, outside the timed chain
            w_uk = orc.dequant_fp8(e["w_uk_fp8"], e["w_uk_scale"])
            w_uv = orc.dequant_fp8(e["w_uv_fp8"], e["w_uv_scale"])
        else:
            w_uk, w_uv = e["w_uk"], e["w_uv"]
        done, t_all, k = 0, 0.0, 1
        t_end = time.perf_counter() + min_seconds
        while done < x.batch and time.perf_counter() < t_end:
            k = min(k, x.batch - done)
            sel = np.arange(done, done + k)
            t0 = time.perf_counter()
            orc.full_step(e["q_nope"][sel], e["q_rope"][sel], w_uk, w_uv, x.kv,
                          x.block_table[sel], x.seqlens[sel], scale=x.scale)
            t_all += time.perf_counter() - t0
            done += k
            k *= 2
        sl = x.seqlens[:done]
        b1, _ = bmm_bytes_flops(done, x.h_q, 128, D_V, fp8w)
        b2, _ = bmm_bytes_flops(done, x.h_q, D_V, 128, fp8w)
        nb = b1 + algorithmic_bytes(sl, 1, x.h_q) + b2
        base.update({"value": round(nb / t_all / 1e9, 3), "cores": threads,
                     "sample": "%s chain (fp64) on the first %d of %d sequences, %.2f s"
                               % (x.name, done, x.batch, t_all)})
        return base
    # all threads: the full batch if one pass fits the time, else a prefix
    n = x.batch
    t_probe = _oracle_attend_rate(orc, x, np.arange(min(n, 4)), 0.0, 1)[0]
    per_seq = t_probe / min(n, 4)
    if per_seq * n > min_seconds:
        n = max(1, min(n, int(min_seconds / max(per_seq, 1e-9))))
    med, nb, reps, nf = _oracle_attend_rate(orc, x, np.arange(n), min_seconds)
    base.update({"value": round(nb / med / 1e9, 3), "cores": threads,
                 "tflops": round(nf / med / 1e12, 5),
                 "sample": "%s batch, first %d of %d sequences (fp64), median of %d repetitions, "
                           "%.3f s each" % (x.name, n, x.batch, reps, med)})
    # one thread
    orc.set_threads(1)
    try:
        t1 = _oracle_attend_rate(orc, x, np.arange(1), 0.0, 1)[0]
        n1 = max(1, min(x.batch, int(one_core_seconds / max(t1, 1e-9))))
        med1, nb1, _, nf1 = _oracle_attend_rate(orc, x, np.arange(n1), 0.0, 1)
    finally:
        orc.set_threads(threads)
    base["one_core"] = {"value": round(nb1 / med1 / 1e9, 4), "cores": 1,
                        "tflops": round(nf1 / med1 / 1e12, 6),
                        "sample": "first %d sequences, one pass, %.3f s" % (n1, med1)}
    return base


def source_digest():
    """sha256 over the library's kernel and ABI sources (names and bytes)."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(HERE, "mla_paged_kv_02_amd", "csrc", "*"))):
        if f.endswith((".hip", ".h", ".cpp")):
            h.update(os.path.basename(f).encode())
            with open(f, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def decode_kernel(rows):
    """The decode kernel the library runs for s_q * h_q = rows: the 128-row
    one for multiples of 128 and from 48 rows on, its shared-row 32-row
    variant for 32 rows, else the 16-row one."""
    if rows % 128 == 0 or rows >= 48:
        return "decode_wide_kernel"
    return "decode_wide32_kernel" if rows == 32 else "decode_r16_kernel"


def measured_traffic(config, x):
    """HBM bytes (fetched + written) of one mla_decode call (decode kernel +
    combine), from the rocprofv3 FETCH_SIZE / WRITE_SIZE runs recorded in
    profiles/hbm_traffic.json, scaled by the copy-kernel calibration there.
    None when no record exists for this workload or the sources have changed
    since it was taken."""
    path = os.path.join(HERE, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != source_digest() or config not in rec.get("per_launch", {}):
        return None
    k = rec["per_launch"][config]
    decode = decode_kernel(x.s_q * x.h_q)
    if decode not in k or "combine_kernel" not in k:
        return None
    return int(sum(k[n]["fetch_bytes"] + k[n]["write_bytes"] for n in (decode, "combine_kernel")))


def copy_reference(torch, dev, nbytes):
    """A plain device copy that moves `nbytes` in all (half read, half
    written), timed like a bmm stage (HIP events, median of 20): from one of
    16 source buffers in turn, so the last-level cache holds none of them.
    The yardstick for the absorbed-weight bmms, which move as many bytes."""
    half = nbytes // 2
    srcs = [torch.ones(half, dtype=torch.uint8, device=dev) for _ in range(16)]
    dst = torch.empty(half, dtype=torch.uint8, device=dev)
    times = []
    for i in range(24):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(srcs[i % 16])
        e1.record()
        torch.cuda.synchronize()
        if i >= 4:
            times.append(e0.elapsed_time(e1))
    ms = float(np.median(times))
    return {"ms": round(ms, 5), "bytes": 2 * half, "GB/s": round(2 * half / (ms / 1e3) / 1e9, 2)}


def time_workload(config, args, torch, mla, gen, dev):
    """Time one workload: `args.warmup` untimed steps, then `args.steps`
    steps bracketed by device synchronizations (ms_per_step), then the same
    steps again with HIP events on the launch stream around each call.
    Returns (record, inputs)."""
    x = gen.make_config(config)
    kv_bytes = x.kv.nbytes
    replicas = args.replicas or max(2, int(np.ceil((1 << 30) / kv_bytes)))

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    q = to_dev(x.q)
    kv0 = to_dev(x.kv)
    kvs = [kv0] + [kv0.clone() for _ in range(replicas - 1)]
    bt = torch.from_numpy(x.block_table).to(dev)
    seqlens = torch.from_numpy(x.seqlens).to(dev)
    parts = args.num_parts or mla.default_num_parts(x.batch, x.s_q, x.h_q, 0)
    meta = torch.empty(mla.metadata_ints(x.batch, parts), dtype=torch.int32, device=dev)
    ws = torch.empty(mla.workspace_bytes(x.batch, x.s_q, x.h_q, parts), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((x.batch, x.s_q, x.h_q, D_V), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((x.batch, x.s_q, x.h_q), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    full = config in ("full_step", "full_step_fp8")
    fp8w = config == "full_step_fp8"
    if full:
        q_nope = to_dev(x.extra["q_nope"])
        y = torch.empty((x.batch, x.h_q, 128), dtype=torch.bfloat16, device=dev)
        if fp8w:
            w_uk8 = torch.from_numpy(x.extra["w_uk_fp8"]).to(dev)
            w_uk_sc = torch.from_numpy(x.extra["w_uk_scale"]).to(dev)
            w_uv8 = torch.from_numpy(x.extra["w_uv_fp8"]).to(dev)
            w_uv_sc = torch.from_numpy(x.extra["w_uv_scale"]).to(dev)
        else:
            w_uk = to_dev(x.extra["w_uk"])
            w_uv = to_dev(x.extra["w_uv"])

    def bmm_uk():
        if fp8w:
            mla.absorb_bmm_fp8w(q_nope, w_uk8, w_uk_sc, q[:, 0, :, :D_V])
        else:
            mla.absorb_bmm(q_nope, w_uk, q[:, 0, :, :D_V])

    def bmm_uv():
        if fp8w:
            mla.absorb_bmm_fp8w(out[:, 0], w_uv8, w_uv_sc, y)
        else:
            mla.absorb_bmm(out[:, 0], w_uv, y)

    # events: [start, after metadata, after W_UK bmm, after decode, after W_UV bmm]
    def step(i, ev=None):
        if ev is not None:
            ev[0].record(stream)
        mla.get_metadata(seqlens, x.s_q, x.h_q, parts, out=meta)
        if ev is not None:
            ev[1].record(stream)
        if full:
            bmm_uk()
        if ev is not None:
            ev[2].record(stream)
        mla.decode(q, kvs[i % replicas], bt, seqlens, meta, parts, scale=x.scale,
                   causal=x.causal, workspace=ws, out=out, lse=lse)
        if ev is not None:
            ev[3].record(stream)
        if full:
            bmm_uv()
        if ev is not None:
            ev[4].record(stream)

    graphs = []
    if args.graph:
        # one captured step per cache replica; replay rotates through them
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for i in range(replicas):
                step(i)
        torch.cuda.synchronize()
        for i in range(replicas):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                step(i)
            graphs.append(gr)
        torch.cuda.synchronize()

    def run(i):
        if graphs:
            graphs[i % replicas].replay()
        else:
            step(i)

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run(i)
    t_issue = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps

    # per-call durations with HIP events on the launch stream (eager calls)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, events[i])
    torch.cuda.synchronize()
    st_meta = pctl([e[0].elapsed_time(e[1]) for e in events])
    st_decode = pctl([e[2].elapsed_time(e[3]) for e in events])
    decode_ms = st_decode["ms"]
    meta_ms = st_meta["ms"]

    nbytes = algorithmic_bytes(x.seqlens, x.s_q, x.h_q)
    flops = algorithmic_flops(x.seqlens, x.s_q, x.h_q, x.causal)
    stages = None
    step_bytes, step_flops = nbytes, flops
    if full:
        b1, f1 = bmm_bytes_flops(x.batch, x.h_q, 128, D_V, fp8w)
        b2, f2 = bmm_bytes_flops(x.batch, x.h_q, D_V, 128, fp8w)
        st_uk = pctl([e[1].elapsed_time(e[2]) for e in events])
        st_uv = pctl([e[3].elapsed_time(e[4]) for e in events])
        st_all = pctl([e[0].elapsed_time(e[4]) for e in events])

        def stage(st, b, f):
            sec = st["ms"] / 1e3
            d = dict(st)
            if b:
                d.update({"algorithmic_bytes": b, "GB/s": round(b / sec / 1e9, 2),
                          "hbm_frac": round(b / sec / 1e9 / HBM_PEAK_GBS, 4),
                          "TFLOP/s": round(f / sec / 1e12, 3),
                          "mfma_frac": round(f / sec / 1e12 / BF16_PEAK_TFLOPS, 4)})
            return d
        stages = {"metadata": stage(st_meta, 0, 0), "absorb_w_uk": stage(st_uk, b1, f1),
                  "decode": stage(st_decode, nbytes, flops), "absorb_w_uv": stage(st_uv, b2, f2),
                  "end_to_end": stage(st_all, b1 + nbytes + b2, f1 + flops + f2),
                  "copy_reference": copy_reference(torch, dev, b1)}
        step_bytes, step_flops = b1 + nbytes + b2, f1 + flops + f2
    value = step_bytes / (ms_step / 1e3) / 1e9
    achieved = nbytes / (decode_ms / 1e3) / 1e9
    tflops = flops / (decode_ms / 1e3) / 1e12
    # the bound is whichever peak the workload's arithmetic intensity meets first
    kernel = "mla_decode (%s + combine_kernel), HIP events" % decode_kernel(x.s_q * x.h_q)
    if flops / nbytes > BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        roofline = {"bound": "mfma", "achieved": round(tflops, 2), "peak": BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(tflops / BF16_PEAK_TFLOPS, 4)}
    else:
        roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    traffic = measured_traffic(config, x)
    roofline.update({"traffic": traffic, "kernel": kernel, "ms": round(decode_ms, 5),
                     "ms_p10": st_decode["p10"], "ms_p90": st_decode["p90"],
                     "GB/s": round(achieved, 2), "TFLOP/s": round(tflops, 2)})
    if traffic is not None:
        roofline["traffic_vs_algorithmic"] = round(traffic / nbytes, 4)
    rec = {
        "value": round(value, 2),
        "ms_per_step": round(ms_step, 5),
        "config": {"workload": "%s: %s" % (config, WORKLOADS[config]),
                   "global_batch": x.batch, "seq_len": int(round(float(x.seqlens.mean()))),
                   "s_q": x.s_q, "h_q": x.h_q, "num_parts": parts, "cache_replicas": replicas,
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "tflops": round(step_flops / (ms_step / 1e3) / 1e12, 3),
        "tflops_frac_of_bf16_peak": round(step_flops / (ms_step / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "metadata_ms": round(meta_ms, 5),
        "host_issue_ms_per_step": round(t_issue * 1e3 / args.steps, 5),
        "launch": "hip graph replay" if graphs else "eager",
        "algorithmic_bytes": step_bytes,
        "algorithmic_flops": step_flops,
    }
    if stages is not None:
        rec["stages"] = stages
    del kvs, kv0
    return rec, x


def absorb_ab(args, torch, mla, gen, dev):
    """Materialized vs sequential absorption at batch 128, 128 heads: HIP-event
    medians of the query side (c_q -> q_lat) and the output side (o_lat -> y)
    each way, with a 512 MiB write between timed calls so that no weight is
    served from the last-level cache, and the weight bytes and flops each
    way touches (every weight read once per call)."""
    from mla_paged_kv_02_amd import absorption as ab
    shp = gen.ABSORB_AB_SHAPE
    B, H, r, dn, c, dv, dm = (shp[k] for k in ("B", "H", "r", "dn", "c", "dv", "d_model"))
    t = gen.make_absorb_ab(**shp)

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    d = {k: to_dev(v) for k, v in t.items()}
    del t
    stream = torch.cuda.current_stream(dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    q = torch.empty((B, 1, H, 576), dtype=torch.bfloat16, device=dev)
    q_lat = q[:, 0, :, :c]
    q_nope = torch.empty((B, H, dn), dtype=torch.bfloat16, device=dev)
    v = torch.empty((B, H, dv), dtype=torch.bfloat16, device=dev)
    y = torch.empty((B, dm), dtype=torch.bfloat16, device=dev)

    def timed(fn, reps):
        ts = []
        for i in range(reps + 3):
            flush.fill_(i & 0xFF)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            if i >= 3:
                ts.append(a.elapsed_time(b) * 1e3)
        return round(float(np.median(ts)), 2)

    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record(stream)
    w_q_uk, w_uv_o = ab.materialize(d["w_uq"], d["w_uk"], d["w_uv"], d["w_o"])
    a1.record(stream)
    a1.synchronize()
    reps = max(5, min(args.steps, 30))
    res = {
        "sequential": {
            "query_us": timed(lambda: ab.query_sequential(d["c_q"], d["w_uq"], d["w_uk"], q_lat,
                                                          q_nope), reps),
            "output_us": timed(lambda: ab.output_sequential(d["o_lat"], d["w_uv"], d["w_o"], y,
                                                            v), reps)},
        "materialized": {
            "query_us": timed(lambda: ab.query_materialized(d["c_q"], w_q_uk, q_lat), reps),
            "output_us": timed(lambda: ab.output_materialized(d["o_lat"], w_uv_o, y), reps)},
    }
    act = 2  # bf16 bytes
    wq = {"sequential": H * r * dn + H * dn * c, "materialized": H * r * c}
    wo = {"sequential": H * c * dv + H * dv * dm, "materialized": H * c * dm}
    for way, rec in res.items():
        qb = wq[way] * act + (B * r + B * H * c) * act + (B * H * dn * 2 * act if way == "sequential" else 0)
        ob = wo[way] * act + (B * H * c + B * dm) * act + (B * H * dv * 2 * act if way == "sequential" else 0)
        rec.update({"query_weight_bytes": wq[way] * act, "output_weight_bytes": wo[way] * act,
                    "query_flops": 2 * B * wq[way], "output_flops": 2 * B * wo[way],
                    "query_GBs": round(qb / (rec["query_us"] * 1e-6) / 1e9, 1),
                    "output_GBs": round(ob / (rec["output_us"] * 1e-6) / 1e9, 1),
                    "total_us": round(rec["query_us"] + rec["output_us"], 2)})
    out = {"metric": "materialized vs sequential MLA absorption: weight bytes, flops and time "
                     "of the query and output projections",
           "config": {"batch": B, "heads": H, "q_lora_rank": r, "qk_nope": dn, "latent": c,
                      "v_head": dv, "d_model": dm,
                      "note": "q_lora_rank and d_model are DeepSeek-V3/R1 values, not on the pages"},
           "materialize_us": round(a0.elapsed_time(a1) * 1e3, 1),
           "kernel": "absorb_kernel (mla_absorb_bmm) for every product, HIP events",
           **res,
           "weight_bytes_ratio": round((wq["materialized"] + wo["materialized"]) /
                                       (wq["sequential"] + wo["sequential"]), 3),
           "time_ratio": round(res["materialized"]["total_us"] / res["sequential"]["total_us"], 3)}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default=None, choices=sorted(WORKLOADS),
                    help="one workload (default: the memory-bound workload, with the "
                         "compute-bound one reported beside it in the same line)")
    ap.add_argument("--replicas", type=int, default=0,
                    help="cache copies rotated over steps (0: enough for >= 1 GiB)")
    ap.add_argument("--num-parts", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step from a captured HIP graph (no host launch cost)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the read and MFMA probes (measured peaks)")
    ap.add_argument("--absorb-ab", action="store_true",
                    help="only compare the materialized and sequential absorption projections "
                         "(one JSON line)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB, five times (the known "
                         "byte count that scales the HBM traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import mla_paged_kv_02_amd as mla
    from mla_paged_kv_02_amd import inputs as gen

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 5}), flush=True)
        return

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    if args.absorb_ab:
        absorb_ab(args, torch, mla, gen, dev)
        return
    config = args.config or "memory_bound"
    body, x = time_workload(config, args, torch, mla, gen, dev)
    rec = {"metric": METRIC, "value": body.pop("value"), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": body.pop("ms_per_step"),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded N(0,1) bf16 cache and queries, shuffled pages)"}
    rec.update(body)
    second = None
    if args.config is None:
        # the metric's other half: bf16 TFLOP/s on the compute-bound workload
        second, x2 = time_workload("compute_bound", args, torch, mla, gen, dev)
        rec["compute_bound"] = second
    if not args.no_peaks:
        peaks = measured_peaks(mla, torch, dev)
        for r in (rec, second):
            if r is None:
                continue
            rf = r["roofline"]
            ref = peaks["hbm_read_GBs"] if rf["bound"] == "hbm" else peaks["bf16_mfma_TFLOPs"]
            rf["frac_of_measured_peak"] = round(rf["achieved"] / ref, 4)
        rec["measured_peaks"] = peaks
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(x, args.cpu_seconds)
        if second is not None:
            second["cpu_baseline"] = cpu_baseline(x2, min(args.cpu_seconds, 5.0), 1.0)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

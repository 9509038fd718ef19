#!/usr/bin/env python
"""Throughput of one MLA paged-latent decode step on one MI355X.

A step is the whole hot path over one batch of synthetic decode input, all in
the HIP library: the new tokens' cache write, query absorption, paged split-KV
decode (plan, split kernel, LSE merge) and the V up-projection.  Inputs are
resident in HBM before timing starts.  The KV pool is replicated R times and the
steps rotate over the copies so that the 256 MB Infinity Cache cannot serve one
step's pages to the next.

Prints ONE JSON line (stdout).  Usage:
    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload full_head]
    python bench.py --op gather_fp8|gather_bf16|merge_states|varlen_spec|upv_fp8_decode|upv_fp8_prefill|absorb_rope_decode|prefill_mha
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import mla_inputs as MI  # noqa: E402

METRIC = "MLA decode tokens/s + achieved HBM TB/s (% roofline), 128 heads, 1 MI355X"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16, published
MALL_BYTES = 256 * 2**20
DECODE_SRC = os.path.join(ROOT, "mla_paged_latent_amd", "csrc", "decode.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_work(w: MI.Workload) -> tuple[int, float, int]:
    """Bytes and flops a decode launch must move/compute, and the KV bytes alone.

    Every cached row is read once and shared by all heads and query rows; the
    query, output, LSE, block table and seq_lens are read/written once.  Flops:
    N * (2*576 + 2*512) per visible (query row, token) pair.  Split partials,
    LDS traffic and re-reads are implementation overhead and are not counted.
    """
    row = 1152 if w.kv_dtype == MI.KV_BF16 else 584
    kv = int(w.seq_lens.astype(np.int64).sum()) * row
    rows = w.B * w.q_len * w.N
    io = rows * 576 * 2 + rows * 512 * 2 + rows * 4
    pages = int(((w.seq_lens.astype(np.int64) + 63) // 64).sum())
    meta = pages * 4 + w.B * 4
    vis = 0
    for b in range(w.B):
        for t in range(w.q_len):
            vis += max(0, int(w.seq_lens[b]) - w.q_len + 1 + t)
    flops = float(vis) * w.N * (2 * 576 + 2 * 512)
    return kv + io + meta, flops, kv


def traffic_record(workload: str):
    """HBM bytes per decode launch measured with rocprofv3 PMC counters, if the
    committed record matches the current decode kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"decode_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    sha = hashlib.sha256(open(DECODE_SRC, "rb").read()).hexdigest()
    if rec.get("decode_hip_sha256") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def host_cores() -> int:
    """Threads the oracle's NumPy/BLAS work can use on this host."""
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = int(os.environ.get("OMP_NUM_THREADS", "1"))
    return min(len(os.sched_getaffinity(0)), blas)


def cpu_baseline(w: MI.Workload, budget_s: float = 12.0) -> dict:
    """The oracle (float64 NumPy) running the same step on this host's cores."""
    from oracle import mla_oracle as O
    cores = host_cores()
    kd = w.kv_dtype
    pool = O.encode_rows(w.kv_rows.reshape(-1, 576), kd).reshape(w.num_pages, 64, -1)
    T = w.B * w.q_len
    sc = O.default_scale()

    def step():
        p = O.cache_write(pool, w.new_rows[:, :512], w.new_rows[:, 512:], w.new_slots, kd)
        if w.q is None:
            q = O.round_to_bf16(O.absorb(O.bf16_bits_to_f64(w.q_nope.reshape(T, w.N, 128)),
                                         O.bf16_bits_to_f64(w.q_pe.reshape(T, w.N, 64)),
                                         O.bf16_bits_to_f64(w.w_uk_t))).reshape(w.B, w.q_len, w.N, 576)
        else:
            q = O.bf16_bits_to_f64(w.q)
        o, _ = O.decode(q, p, kd, w.block_table, w.seq_lens, sc)
        if w.w_uv is not None:
            O.up_v(O.round_to_bf16(o).reshape(T, w.N, 512), O.bf16_bits_to_f64(w.w_uv))

    times = []
    t_all = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        step()
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_all >= budget_s or len(times) >= 20:
            break
    mean = sum(times) / len(times)
    return {"value": T / mean, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"the full {w.name} batch ({w.B} requests x q_len {w.q_len}) through the "
                      f"float64 oracle step (cache write, absorb, decode, up-projection), "
                      f"{len(times)} repetition(s), mean {mean:.3f} s"}


def run(args) -> dict:
    import torch
    import mla_paged_latent_amd as M

    w = MI.CONFIGS[args.workload]()
    kd = w.kv_dtype
    dev = torch.device("cuda:0")
    T = w.B * w.q_len
    bytes_alg, flops_alg, kv_bytes = algorithmic_work(w)
    row = M.ROW_BYTES[kd]
    # enough pool copies that consecutive reuse of one copy is >= 3 MALL capacities apart
    R = min(8, max(2, math.ceil(3 * MALL_BYTES / max(kv_bytes, 1))))
    log(f"[bench] workload {w.name}: B={w.B} q_len={w.q_len} N={w.N} kv={'bf16' if kd == 0 else 'fp8'} "
        f"pages={w.num_pages} KV bytes/step={kv_bytes / 1e6:.1f} MB, pool copies={R}")

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    rows = bf16(w.kv_rows.reshape(-1, 576))
    slots = torch.arange(w.num_pages * 64, dtype=torch.int64, device=dev)
    pools = []
    for _ in range(R):
        pool = torch.empty((w.num_pages, 64, row), dtype=torch.uint8, device=dev)
        M.cache_write(rows[:, :512], rows[:, 512:], slots, pool, kd)
        pools.append(pool)
    del rows, slots
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(w.seq_lens).to(dev)
    new = bf16(w.new_rows)
    new_slots = torch.from_numpy(w.new_slots).to(dev)
    with_w = w.w_uk_t is not None
    if with_w:
        q_nope = bf16(w.q_nope.reshape(T, w.N, 128))
        q_pe = bf16(w.q_pe.reshape(T, w.N, 64))
        w_uk_t = bf16(w.w_uk_t)
        w_uv = bf16(w.w_uv)
        qf = torch.empty((T, w.N, 576), dtype=torch.bfloat16, device=dev)
        y = torch.empty((T, w.N * 128), dtype=torch.bfloat16, device=dev)
    else:
        qf = bf16(w.q.reshape(T, w.N, 576))
    out = torch.empty((w.B, w.q_len, w.N, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.q_len, w.N), dtype=torch.float32, device=dev)
    ws = torch.empty(M.decode_workspace_size(w.B, w.q_len, w.N, args.num_splits), dtype=torch.uint8,
                     device=dev)
    if args.copy_calibration_mb > 0:
        # one device-to-device copy of a known size: under a --pmc run its FETCH_SIZE /
        # WRITE_SIZE give the counters' scale (see --traffic-record)
        nb = args.copy_calibration_mb * 2**20
        src = torch.ones(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    torch.cuda.synchronize()

    def step_api(i: int):
        pool = pools[i % R]
        M.cache_write(new[:, :512], new[:, 512:], new_slots, pool, kd)
        if with_w:
            M.absorb_q(q_nope, q_pe, w_uk_t, q_fused=qf)
        M.decode(qf.view(w.B, w.q_len, w.N, 576), pool, kd, bt, sl, M.DEFAULT_SCALE, args.num_splits,
                 workspace=ws, out=out, lse=lse)
        if with_w:
            M.up_v(out.view(T, w.N, 512), w_uv, out=y)

    # The timed loops call the same C entry points with their arguments marshalled once
    # (the tensor-checking Python wrappers cost tens of microseconds per call, enough to
    # leave the GPU idle between the step's kernels); checked below against step_api.
    L = M.lib()
    stream = torch.cuda.current_stream().cuda_stream
    qv = qf.view(w.B, w.q_len, w.N, 576)
    kc_new, kp_new = new[:, :512], new[:, 512:]
    cw_args = [(kc_new.data_ptr(), kc_new.stride(0), kp_new.data_ptr(), kp_new.stride(0), new_slots.data_ptr(),
                new.shape[0], pool.data_ptr(), kd, w.num_pages, stream) for pool in pools]
    dec_args = [(qv.data_ptr(), qv.stride(0), qv.stride(1), qv.stride(2), pool.data_ptr(), kd, w.num_pages,
                 bt.data_ptr(), bt.stride(0), bt.shape[1], sl.data_ptr(), w.B, w.q_len, w.N,
                 float(M.DEFAULT_SCALE), args.num_splits, ws.data_ptr(), ws.numel(), out.data_ptr(),
                 out.stride(0), out.stride(1), out.stride(2), lse.data_ptr(), stream) for pool in pools]
    if with_w:
        ol = out.view(T, w.N, 512)
        ab_args = (q_nope.data_ptr(), q_nope.stride(0), q_nope.stride(1), q_pe.data_ptr(), q_pe.stride(0),
                   q_pe.stride(1), w_uk_t.data_ptr(), T, w.N, qf.data_ptr(), qf.stride(0), qf.stride(1), stream)
        uv_args = (ol.data_ptr(), ol.stride(0), ol.stride(1), w_uv.data_ptr(), T, w.N, y.data_ptr(), y.stride(0),
                   stream)
    f_cw, f_ab, f_dec, f_uv = L.mla_cache_write, L.mla_absorb_q, L.mla_decode, L.mla_up_v

    def step(i: int):
        j = i % R
        rc = f_cw(*cw_args[j])
        if with_w:
            rc |= f_ab(*ab_args)
        rc |= f_dec(*dec_args[j])
        if with_w:
            rc |= f_uv(*uv_args)
        if rc != 0:
            raise RuntimeError(f"an mla_* call failed in step {i} (status bits {rc})")

    def decode_only(i: int):
        if f_dec(*dec_args[i % R]) != 0:
            raise RuntimeError(f"mla_decode failed in call {i}")

    # the marshalled step computes what the checked wrappers compute, bit for bit
    step_api(0)
    torch.cuda.synchronize()
    ref = [t.clone() for t in ((out, lse, y) if with_w else (out, lse))]
    step(0)
    torch.cuda.synchronize()
    for a, b in zip(ref, (out, lse, y) if with_w else (out, lse)):
        assert torch.equal(a, b), "marshalled step differs from the API step"

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region 1: K whole steps, bracketed by one event pair (no events inside: an
    # event record between two kernels delays the next launch by several microseconds)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        step(i)
    stop.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    # timed region 2: K mla_decode calls back to back on the same stream (rotating cache
    # pools), bracketed by one event pair: the average launch duration of mla_decode
    for i in range(min(args.warmup, 3)):
        decode_only(i)
    torch.cuda.synchronize()
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    d0.record()
    for i in range(args.steps):
        decode_only(i)
    d1.record()
    torch.cuda.synchronize()
    dec_mean = d0.elapsed_time(d1) / args.steps
    log(f"[bench] step {ms_step * 1e3:.1f} us, mla_decode {dec_mean * 1e3:.1f} us per call "
        f"({args.steps} calls back to back)")

    achieved = bytes_alg / (dec_mean * 1e-3) / 1e9
    tflops = flops_alg / (dec_mean * 1e-3) / 1e12
    t_hbm = bytes_alg / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops_alg / (MFMA_BF16_PEAK_TFS * 1e12)
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFS,
                "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFS, 4)}
    roof["traffic"] = traffic_record(args.workload)
    roof["kernel"] = "mla_decode (split-KV decode with in-kernel split plan + LSE merge)"
    roof["algorithmic_bytes"] = bytes_alg
    roof["algorithmic_flops"] = flops_alg
    roof["mean_launch_us"] = round(dec_mean * 1e3, 2)
    roof["mfma_frac_bf16"] = round(tflops / MFMA_BF16_PEAK_TFS, 4)
    roof["hbm_frac"] = round(achieved / HBM_PEAK_GBS, 4)

    res = {
        "metric": METRIC,
        "value": round(T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if kd == MI.KV_BF16 else "fp8-e4m3 cache, bf16 mfma",
        "data": "synthetic (seeded N(0,1) latents/queries, N(0,1/512) weights; random page placement)",
        "config": {"workload": f"{w.name}: B={w.B}, q_len={w.q_len}, heads={w.N}, "
                               f"seq_lens={'all ' + str(int(w.seq_lens[0])) if len(set(w.seq_lens.tolist())) == 1 else 'mixed'}, "
                               f"kv={'bf16' if kd == 0 else 'fp8'} 576-d rows, 64-token pages, "
                               f"absorb + decode + up-proj",
                   "batch": w.B, "q_len": w.q_len, "heads": w.N, "kv_tokens": w.tokens,
                   "num_splits": args.num_splits, "pool_copies": R},
        "decode_latent_kv_tbs": round(kv_bytes / (dec_mean * 1e-3) / 1e12, 3),
        "roofline": roof,
    }
    return res


DECODE_KERNELS = ("decode_wide_kernel", "decode_narrow_kernel", "merge_kernel")
COPY_KERNEL = "copyBuffer"


def _counter_rows(d: str, counter: str):
    import csv
    import glob
    out = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                out.append((r["Kernel_Name"], int(r.get("Dispatch_Id", 0) or 0), float(r["Counter_Value"])))
    return out


def traffic_record_from_pmc(fetch_dir: str, write_dir: str, workload: str, copy_mb: int, command: str) -> dict:
    """HBM bytes per mla_decode call from two rocprofv3 --pmc runs of this script
    (FETCH_SIZE, then WRITE_SIZE, both in KiB per dispatch), each scaled by what the
    same counter reads for the calibration copy of copy_mb MiB in that run."""
    res = {"workload": workload, "command": command, "copy_calibration_bytes": copy_mb * 2**20}
    per_call = 0.0
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(d, name)
        copies = [v for k, _, v in rows if COPY_KERNEL in k]
        if not copies:
            raise SystemExit(f"no calibration copy found in {d}")
        scale = copy_mb * 2**20 / (max(copies) * 1024.0)
        kern = {}
        for k, _, v in rows:
            for kn in DECODE_KERNELS:
                if kn in k:
                    kern.setdefault(kn, []).append(v * 1024.0 * scale)
        med = {kn: sorted(v)[len(v) // 2] for kn, v in kern.items()}
        res[name] = {"scale": round(scale, 4), "bytes_per_dispatch": {k: round(v) for k, v in med.items()}}
        per_call += sum(med.values())
    res["hbm_bytes_per_launch"] = round(per_call)
    res["decode_hip_sha256"] = hashlib.sha256(open(DECODE_SRC, "rb").read()).hexdigest()
    return res


CONTEXT_OPS = {
    # the chunked-prefill workspace at its cap (64 x 1024 rows) gathered from 16
    # requests' 4096-token context chunks, fp8 cache upconverted to bf16
    "gather_fp8": dict(kind="gather", kv=MI.KV_FP8, requests=16, chunk=4096),
    "gather_bf16": dict(kind="gather", kv=MI.KV_BF16, requests=16, chunk=4096),
    # merging the context and new-token states of an 8192-token prefill, 128 heads,
    # v_head_dim 128
    "merge_states": dict(kind="merge", T=8192, N=128, D=128),
    # a speculative-decoding verification batch: 64 requests of 4096 cached tokens
    # with 1, 2 or 3 query tokens each (causal blocks), 128 heads, bf16 cache
    "varlen_spec": dict(kind="varlen", B=64, seq=4096, N=128, q_lens=(1, 2, 3)),
    # V up-projection with fp8 output in groups of 128: a 128-request decode batch
    # and an 8192-token prefill, 128 heads
    "upv_fp8_decode": dict(kind="upv", T=128, N=128, group=128),
    "upv_fp8_prefill": dict(kind="upv", T=8192, N=128, group=128),
    # query absorption with the rope part rotated on the way (rotate-half pairing,
    # positions drawn from a 32k table), a 128-request decode batch, 128 heads
    "absorb_rope_decode": dict(kind="rope", T=128, N=128, max_pos=32768),
    # prefill of new tokens: 4 requests of 2048 new tokens each (no context), causal,
    # 128 heads, keys [k_nope | k_pe] 192 wide, values 128 wide
    "prefill_mha": dict(kind="prefill", B=4, L=2048, N=128),
}


def run_context_op(args) -> dict:
    """One launch of mla_gather_cache, mla_merge_attn_states, mla_decode_varlen or
    mla_up_v_fp8, timed back to back.

    Algorithmic bytes: gather reads each source row (1152 or 584 B) and writes a
    1152 B bf16 row, plus 4 B of token_to_seq per row, 4 B per block-table entry
    and 12 B per request; merge reads two bf16 states and two LSEs and writes one
    of each.  The bound is HBM (no arithmetic to speak of).  mla_up_v_fp8 reads
    W_UV and o_lat once and writes one code byte per output plus a float32 scale
    per group; at 113 flops per byte it sits below the bf16 MFMA ridge, so HBM.
    """
    import ctypes
    import torch
    import mla_paged_latent_amd as M
    op = CONTEXT_OPS[args.op]
    dev = "cuda"
    L = M.lib()
    stream = torch.cuda.current_stream().cuda_stream
    if op["kind"] == "gather":
        kd, nreq, chunk = op["kv"], op["requests"], op["chunk"]
        total = nreq * chunk
        pages = total // 64
        rb = M.ROW_BYTES[kd]
        # replicated pools, rotated per call, so the 256 MB cache cannot hold the rows
        R = max(2, math.ceil(3 * MALL_BYTES / (pages * 64 * rb)))
        chunks = [MI.make_context_chunk([chunk] * nreq, [0] * nreq, pages, seed=500 + i) for i in range(R)]
        w = MI.make_workload("gather-pool", 1, 1, 16, [64], pages, kd, False, 501)
        rows = torch.from_numpy(np.ascontiguousarray(w.kv_rows.reshape(-1, 576)).view(np.int16)).view(
            torch.bfloat16).to(dev)
        slots = torch.arange(pages * 64, device=dev)
        pools = []
        for _ in range(R):
            pl = torch.empty((pages, 64, rb), dtype=torch.uint8, device=dev)
            M.cache_write(rows[:, :512], rows[:, 512:], slots, pl, kd)
            pools.append(pl)
        del rows
        out = torch.empty((total, 576), dtype=torch.bfloat16, device=dev)
        meta = [tuple(torch.from_numpy(a).to(dev) for a in (c.block_table, c.cu_seq_lens, c.token_to_seq))
                for c in chunks]
        calls = [(pools[i].data_ptr(), kd, pages, meta[i][0].data_ptr(), meta[i][0].stride(0),
                  meta[i][0].shape[1], meta[i][1].data_ptr(), None, meta[i][2].data_ptr(), nreq, total,
                  out.data_ptr(), out.stride(0), stream) for i in range(R)]
        f = L.mla_gather_cache
        bytes_alg = total * (rb + 1152 + 4) + pages * 4 + nreq * 12
        desc = (f"{args.op}: {total} rows (the 64x1024-row prefill workspace cap) from {nreq} requests' "
                f"{chunk}-token context chunks, {'fp8 rows upconverted' if kd == MI.KV_FP8 else 'bf16 rows'} "
                f"to bf16, random page placement, {R} rotating pool copies")
        metric = "context gather GB/s (% of HBM roofline), 1 MI355X"
        dtype = "fp8->bf16" if kd == MI.KV_FP8 else "bf16"
    elif op["kind"] == "varlen":
        B, N, seq = op["B"], op["N"], op["seq"]
        rng = np.random.default_rng(530)
        q_lens = rng.choice(op["q_lens"], size=B)
        qsl = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
        T = int(qsl[-1])
        w = MI.make_workload("varlen", B, 1, N, [seq] * B, None, MI.KV_BF16, False, 531, min_pool=8192)
        rb = 1152
        R = max(2, math.ceil(3 * MALL_BYTES / (w.num_pages * 64 * rb)))
        rows = torch.from_numpy(np.ascontiguousarray(w.kv_rows.reshape(-1, 576)).view(np.int16)).view(
            torch.bfloat16).to(dev)
        slots = torch.arange(w.num_pages * 64, device=dev)
        pools = []
        for _ in range(R):
            pl = torch.empty((w.num_pages, 64, rb), dtype=torch.uint8, device=dev)
            M.cache_write(rows[:, :512], rows[:, 512:], slots, pl, MI.KV_BF16)
            pools.append(pl)
        del rows
        q = torch.randn(T, N, 576, device=dev).to(torch.bfloat16)
        bt = torch.from_numpy(w.block_table).to(dev)
        sl = torch.from_numpy(w.seq_lens).to(dev)
        tq = torch.from_numpy(qsl).to(dev)
        out = torch.empty((T, N, 512), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((T, N), dtype=torch.float32, device=dev)
        ws = torch.empty(int(L.mla_decode_varlen_workspace_size(T, N, 0, bt.shape[1])), dtype=torch.uint8,
                         device=dev)
        calls = [(q.data_ptr(), q.stride(0), q.stride(1), pools[i].data_ptr(), MI.KV_BF16, w.num_pages,
                  bt.data_ptr(), bt.stride(0), bt.shape[1], tq.data_ptr(), sl.data_ptr(), B, T, N, 1,
                  float(M.DEFAULT_SCALE), 0, ws.data_ptr(), ws.numel(), out.data_ptr(), out.stride(0),
                  out.stride(1), lse.data_ptr(), stream) for i in range(R)]
        f = L.mla_decode_varlen
        pages = B * ((seq + 63) // 64)
        bytes_alg = B * seq * rb + T * N * (1152 + 1024 + 4) + pages * 4 + B * 8
        vis = sum(max(0, seq - int(ql) + 1 + t) for ql in q_lens for t in range(int(ql)))
        flops_alg = float(vis) * N * (2 * 576 + 2 * 512)
        desc = (f"{args.op}: B={B} requests x {seq} cached tokens, query tokens per request drawn from "
                f"{list(op['q_lens'])} (T={T} rows, causal), {N} heads, bf16 cache, {R} rotating pool copies")
        metric = "variable-length MLA decode GB/s (roofline: the binding one of HBM / bf16 MFMA), 1 MI355X"
        dtype = "bf16"
    elif op["kind"] == "upv":
        T, N, G = op["T"], op["N"], op["group"]
        per_copy = N * 512 * 128 * 2 + T * N * 512 * 2
        R = max(2, math.ceil(3 * MALL_BYTES / per_copy))
        gen = torch.Generator(device=dev).manual_seed(540)
        ws = [(torch.randn(N, 512, 128, device=dev, generator=gen) / math.sqrt(512)).to(torch.bfloat16)
              for _ in range(R)]
        ols = [torch.randn(T, N, 512, device=dev, generator=gen).to(torch.bfloat16) for _ in range(R)]
        codes = torch.empty((T, N * 128), dtype=torch.uint8, device=dev)
        scales = torch.empty((T, N * 128 // G), dtype=torch.float32, device=dev)
        calls = [(ols[i].data_ptr(), ols[i].stride(0), ols[i].stride(1), ws[i].data_ptr(), T, N, G,
                  codes.data_ptr(), codes.stride(0), scales.data_ptr(), scales.stride(0), stream)
                 for i in range(R)]
        f = L.mla_up_v_fp8
        bytes_alg = per_copy + T * N * 128 + T * N * 128 // G * 4
        flops_alg = 2.0 * T * N * 512 * 128
        # the bf16-output call on the same inputs, for comparison
        yb = torch.empty((T, N * 128), dtype=torch.bfloat16, device=dev)
        ref_calls = [(ols[i].data_ptr(), ols[i].stride(0), ols[i].stride(1), ws[i].data_ptr(), T, N,
                      yb.data_ptr(), yb.stride(0), stream) for i in range(R)]
        desc = (f"{args.op}: T={T} tokens x {N} heads, o_lat [T, N, 512] . W_UV [N, 512, 128] -> fp8 "
                f"e4m3 codes + float32 scales per group of {G}, {R} rotating input copies")
        metric = "V up-projection with fp8 group-quantized output GB/s (% of HBM roofline), 1 MI355X"
        dtype = "bf16->fp8"
    elif op["kind"] == "rope":
        T, N = op["T"], op["N"]
        per_copy = N * 128 * 512 * 2 + T * N * (128 + 64) * 2
        R = max(2, math.ceil(3 * MALL_BYTES / per_copy))
        gen = torch.Generator(device=dev).manual_seed(550)
        ws = [(torch.randn(N, 128, 512, device=dev, generator=gen) / math.sqrt(512)).to(torch.bfloat16)
              for _ in range(R)]
        qs = [torch.randn(T, N, 192, device=dev, generator=gen).to(torch.bfloat16) for _ in range(R)]
        table = torch.from_numpy(MI.rope_cos_sin(op["max_pos"])).to(dev)
        pos = torch.randint(0, op["max_pos"], (T,), device=dev, generator=gen)
        qf = torch.empty((T, N, 576), dtype=torch.bfloat16, device=dev)
        calls = [(qs[i].data_ptr(), qs[i].stride(0), qs[i].stride(1), qs[i].data_ptr() + 256, qs[i].stride(0),
                  qs[i].stride(1), ws[i].data_ptr(), T, N, pos.data_ptr(), table.data_ptr(), op["max_pos"], 1,
                  qf.data_ptr(), qf.stride(0), qf.stride(1), stream) for i in range(R)]
        f = L.mla_absorb_q_rope
        bytes_alg = per_copy + T * (8 + 256) + T * N * 576 * 2
        flops_alg = 2.0 * T * N * 128 * 512
        ref_calls = [(qs[i].data_ptr(), qs[i].stride(0), qs[i].stride(1), qs[i].data_ptr() + 256, qs[i].stride(0),
                      qs[i].stride(1), ws[i].data_ptr(), T, N, qf.data_ptr(), qf.stride(0), qf.stride(1), stream)
                     for i in range(R)]
        desc = (f"{args.op}: T={T} tokens x {N} heads, q_nope [T, N, 128] . W_UK_T [N, 128, 512] into a "
                f"[T, N, 576] fused query whose tail is RoPE(q_pe) (rotate-half, {op['max_pos']}-row table), "
                f"{R} rotating input copies")
        metric = "query absorption with fused RoPE GB/s (% of HBM roofline), 1 MI355X"
        dtype = "bf16"
    elif op["kind"] == "prefill":
        Bq, Lq, N = op["B"], op["L"], op["N"]
        T = S = Bq * Lq
        gen = torch.Generator(device=dev).manual_seed(560)
        q = torch.randn(T, N, 192, device=dev, generator=gen).to(torch.bfloat16)
        kvb = torch.randn(S, N, 256, device=dev, generator=gen).to(torch.bfloat16)
        kp = torch.randn(S, 64, device=dev, generator=gen).to(torch.bfloat16)
        cu = torch.arange(0, T + 1, Lq, dtype=torch.int32, device=dev)
        o = torch.empty(T, N, 128, dtype=torch.bfloat16, device=dev)
        lse_t = torch.empty(T, N, dtype=torch.float32, device=dev)
        kn, vv = kvb[..., :128], kvb[..., 128:]
        calls = [(q.data_ptr(), q.stride(0), q.stride(1), kn.data_ptr(), kn.stride(0), kn.stride(1), kp.data_ptr(),
                  kp.stride(0), vv.data_ptr(), vv.stride(0), vv.stride(1), cu.data_ptr(), cu.data_ptr(), Bq, T, S, N,
                  Lq, 1, float(M.DEFAULT_SCALE), o.data_ptr(), o.stride(0), o.stride(1), lse_t.data_ptr(), stream)]
        f = L.mla_prefill_mha
        pairs = Bq * Lq * (Lq + 1) / 2
        flops_alg = pairs * N * (2 * 192 + 2 * 128)
        bytes_alg = T * N * 192 * 2 + S * N * 256 * 2 + S * 64 * 2 + T * N * (128 * 2 + 4)
        desc = (f"{args.op}: {Bq} requests x {Lq} new tokens (no context), causal, {N} heads, keys 192 wide "
                f"([k_nope | shared k_pe]), values 128 wide, bf16")
        metric = "prefill MHA of new tokens TFLOP/s (% of bf16 MFMA roofline), 1 MI355X"
        dtype = "bf16"
    else:
        T, N, D = op["T"], op["N"], op["D"]
        po, pl, so, sl = MI.random_attn_states(T, N, D, seed=510)
        bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        tpo, tso = bf(po), bf(so)
        tpl, tsl = torch.from_numpy(pl).to(dev), torch.from_numpy(sl).to(dev)
        out = torch.empty_like(tpo)
        olse = torch.empty_like(tpl)
        calls = [(tpo.data_ptr(), tpl.data_ptr(), tso.data_ptr(), tsl.data_ptr(), T, N, D, tpo.stride(0),
                  tpo.stride(1), tpl.stride(0), tpl.stride(1), out.data_ptr(), olse.data_ptr(), stream)]
        f = L.mla_merge_attn_states
        bytes_alg = T * N * (3 * D * 2 + 3 * 4)
        desc = f"{args.op}: T={T} query rows x {N} heads x D={D} (bf16 states, fp32 LSE, ~10% empty rows)"
        metric = "attention-state merge GB/s (% of HBM roofline), 1 MI355X"
        dtype = "bf16"
    for i in range(max(args.warmup, 3)):
        if f(*calls[i % len(calls)]) != 0:
            raise RuntimeError(f"{args.op} failed")
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        f(*calls[i % len(calls)])
    e1.record()
    torch.cuda.synchronize()
    mean_ms = e0.elapsed_time(e1) / args.steps
    gbs = bytes_alg / (mean_ms * 1e-3) / 1e9
    log(f"[bench] {args.op}: {mean_ms * 1e3:.1f} us per call, {gbs:.0f} GB/s")
    bf16_out_us = None
    if op["kind"] in ("upv", "rope"):
        g = L.mla_up_v if op["kind"] == "upv" else L.mla_absorb_q
        for i in range(3):
            g(*ref_calls[i % len(ref_calls)])
        e0.record()
        for i in range(args.steps):
            g(*ref_calls[i % len(ref_calls)])
        e1.record()
        torch.cuda.synchronize()
        bf16_out_us = round(e0.elapsed_time(e1) / args.steps * 1e3, 2)
        log(f"[bench] the unfused call on the same inputs: {bf16_out_us:.1f} us per call")
    roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4)}
    if op["kind"] in ("varlen", "prefill") and flops_alg / (MFMA_BF16_PEAK_TFS * 1e12) > bytes_alg / (HBM_PEAK_GBS * 1e9):
        tfs = flops_alg / (mean_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(tfs, 1), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4)}
    roof.update({"traffic": None, "kernel": args.op, "algorithmic_bytes": bytes_alg,
                 "mean_launch_us": round(mean_ms * 1e3, 2), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)})
    if op["kind"] in ("varlen", "upv", "rope", "prefill"):
        roof["algorithmic_flops"] = flops_alg
    if bf16_out_us is not None:
        roof["unfused_call_us"] = bf16_out_us
    res = {"metric": metric, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(mean_ms, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": dtype, "data": "synthetic (seeded)", "config": {"workload": desc},
           "roofline": roof}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_context(args.op)
    return res


def cpu_baseline_context(name: str, budget_s: float = 10.0) -> dict:
    """The oracle's gather / merge on a bounded sample of the same workload."""
    from oracle import mla_oracle as O
    op = CONTEXT_OPS[name]
    times, n_items = [], 0
    t_all = time.perf_counter()
    if op["kind"] == "gather":
        c = MI.make_context_chunk([256] * 8, [0] * 8, 32, seed=520)
        w = MI.make_workload("gather-pool", 1, 1, 16, [64], 32, op["kv"], False, 521)
        pool = O.encode_rows(w.kv_rows.reshape(-1, 576), op["kv"]).reshape(32, 64, -1)
        while time.perf_counter() - t_all < budget_s and len(times) < 20:
            t0 = time.perf_counter()
            O.gather_cache(pool, op["kv"], c.block_table, c.cu_seq_lens, c.token_to_seq)
            times.append(time.perf_counter() - t0)
        n_items = c.total
        rb = 1152 if op["kv"] == MI.KV_BF16 else 584
        per_item = rb + 1152 + 4
        sample = f"{c.total} rows (8 requests x 256 tokens) through the oracle gather"
    elif op["kind"] == "varlen":
        B, N, seq = 4, op["N"], 1024
        w = MI.make_workload("varlen", B, 1, N, [seq] * B, None, MI.KV_BF16, False, 532)
        pool = O.encode_rows(w.kv_rows.reshape(-1, 576), MI.KV_BF16).reshape(w.num_pages, 64, -1)
        qsl = np.array([0, 1, 3, 6, 8], np.int32)
        q = np.random.default_rng(533).standard_normal((8, N, 576))
        while time.perf_counter() - t_all < budget_s and len(times) < 20:
            t0 = time.perf_counter()
            O.decode_varlen(q, qsl, pool, MI.KV_BF16, w.block_table, w.seq_lens, True, O.default_scale())
            times.append(time.perf_counter() - t0)
        n_items = 1
        per_item = B * seq * 1152 + 8 * N * (1152 + 1024 + 4)
        sample = f"{B} requests x {seq} tokens, 8 query rows, {N} heads through the oracle varlen decode"
    elif op["kind"] == "upv":
        T, N, G = 32, op["N"], op["group"]
        rng = np.random.default_rng(541)
        ol = O.bf16_bits_to_f64(MI.to_bf16_bits(rng.standard_normal((T, N, 512)).astype(np.float32)))
        wv = O.bf16_bits_to_f64(MI.to_bf16_bits((rng.standard_normal((N, 512, 128)) / np.sqrt(512)).astype(np.float32)))
        while time.perf_counter() - t_all < budget_s and len(times) < 20:
            t0 = time.perf_counter()
            y = O.f64_to_bf16_bits(O.up_v(ol, wv).reshape(T, N * 128))
            O.quantize_groups_fp8(y, G)
            times.append(time.perf_counter() - t0)
        n_items = 1
        per_item = N * 512 * 128 * 2 + T * N * (512 * 2 + 128 + 128 // G * 4)
        sample = f"T={T} tokens x {N} heads through the oracle up_v and group quantizer"
    elif op["kind"] == "rope":
        T, N = 32, op["N"]
        rng = np.random.default_rng(551)
        qn = O.bf16_bits_to_f64(MI.to_bf16_bits(rng.standard_normal((T, N, 128)).astype(np.float32)))
        qp = O.bf16_bits_to_f64(MI.to_bf16_bits(rng.standard_normal((T, N, 64)).astype(np.float32)))
        wk = O.bf16_bits_to_f64(MI.to_bf16_bits((rng.standard_normal((N, 128, 512)) / np.sqrt(512)).astype(np.float32)))
        table = MI.rope_cos_sin(op["max_pos"]).astype(np.float64)
        pos = rng.integers(0, op["max_pos"], T)
        while time.perf_counter() - t_all < budget_s and len(times) < 20:
            t0 = time.perf_counter()
            O.f64_to_bf16_bits(O.absorb_rope(qn, qp, wk, pos, table, True))
            times.append(time.perf_counter() - t0)
        n_items = 1
        per_item = N * 128 * 512 * 2 + T * N * (192 * 2 + 576 * 2) + T * (8 + 256)
        sample = f"T={T} tokens x {N} heads through the oracle absorb_rope"
    elif op["kind"] == "prefill":
        N, Lq = op["N"], 64
        rng = np.random.default_rng(561)
        q = rng.standard_normal((Lq, N, 192))
        kn, kp, vv = rng.standard_normal((Lq, N, 128)), rng.standard_normal((Lq, 64)), rng.standard_normal((Lq, N, 128))
        cu = np.array([0, Lq])
        while time.perf_counter() - t_all < budget_s and len(times) < 20:
            t0 = time.perf_counter()
            O.prefill_mha(q, kn, kp, vv, cu, cu, O.default_scale(), True)
            times.append(time.perf_counter() - t0)
        n_items = 1
        per_item = Lq * N * (192 * 2 + 256 * 2 + 128 * 2 + 4) + Lq * 64 * 2
        sample = f"1 request x {Lq} new tokens x {N} heads through the oracle prefill_mha"
    else:
        T, N, D = 256, op["N"], op["D"]
        po, pl, so, sl = MI.random_attn_states(T, N, D, seed=522)
        pof, sof = O.bf16_bits_to_f64(po), O.bf16_bits_to_f64(so)
        while time.perf_counter() - t_all < budget_s and len(times) < 20:
            t0 = time.perf_counter()
            O.merge_attn_states(pof, pl, sof, sl)
            times.append(time.perf_counter() - t0)
        n_items = T * N
        per_item = 3 * D * 2 + 3 * 4
        sample = f"{T} query rows x {N} heads x D={D} through the oracle merge"
    mean = sum(times) / len(times)
    return {"value": round(n_items * per_item / mean / 1e9, 3), "unit": "GB/s", "cores": host_cores(), "kind": "oracle",
            "sample": f"{sample}, {len(times)} repetition(s), mean {mean:.3f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="full_head", choices=sorted(MI.CONFIGS))
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--op", default="step", choices=["step"] + sorted(CONTEXT_OPS),
                    help="step: the decode step (default); the others time one other call on its own "
                         "workload (context gather, state merge, variable-length decode)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="run one device copy of this many MiB before the steps (counter calibration)")
    ap.add_argument("--traffic-record", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/decode_traffic_<workload>.json from two rocprofv3 --pmc runs "
                         "(FETCH_SIZE, WRITE_SIZE) of this script made with --copy-calibration-mb; no GPU")
    ap.add_argument("--traffic-command", default="", help="the profiling command, stored in the record")
    args = ap.parse_args()
    if args.traffic_record:
        rec = traffic_record_from_pmc(args.traffic_record[0], args.traffic_record[1], args.workload,
                                      args.copy_calibration_mb, args.traffic_command)
        path = os.path.join(ROOT, "profiles", f"decode_traffic_{args.workload}.json")
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "runs on one GPU only (--gpus 1): the decode path shards by "
                                   "request (attention-DP) or heads (TP) with no exchange inside the "
                                   "path, so only --gpus 1 is measured"}), flush=True)
        sys.exit(2)
    if args.op != "step":
        print(json.dumps(run_context_op(args)), flush=True)
        return
    res = run(args)
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(MI.CONFIGS[args.workload]())
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python
"""Throughput of one MLA paged-latent decode step on one MI355X.

A step is the whole hot path over one batch of synthetic decode input, all in
the HIP library: the new tokens' cache write, query absorption, paged split-KV
decode (plan, split kernel, LSE merge) and the V up-projection.  Inputs are
resident in HBM before timing starts.  The KV pool is replicated R times and the
steps rotate over the copies so that the 256 MB Infinity Cache cannot serve one
step's pages to the next.

Prints ONE JSON line (stdout).  Besides the headline step (default workload
full_head), the line carries one record per decode workload (tp_share, full_head,
fp8, spec_long: median / p10 / p90 of the mla_decode launch over >= 50 rounds,
fractions of the published and of the measured HBM and bf16 MFMA peaks, and the
throughput bar each is held to), the per-kernel launch durations of the step, the
measured peaks, and the CPU oracle baseline.  Usage:
    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload full_head]
    python bench.py --op gather_fp8|gather_bf16|merge_states|varlen_spec|upv_fp8_decode|upv_fp8_prefill|absorb_rope_decode|kv_b_proj_prefill|prefill_mha
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


def blas_threads() -> int:
    """Threads NumPy's BLAS uses on this host."""
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return int(os.environ.get("OMP_NUM_THREADS", "1"))


def host_cores() -> int:
    """Threads the oracle's NumPy/BLAS work can use on this host."""
    return min(len(os.sched_getaffinity(0)), blas_threads())


# the benchmark spec's throughput bars: (bound they are stated against, fraction)
TARGETS = {"tp_share": ("hbm", 0.75), "full_head": ("binding", 0.50), "fp8": ("binding", 0.50),
           "spec_long": ("binding", 0.50)}


def cpu_baseline(w: MI.Workload, budget_s: float = 10.0) -> dict:
    """The decode-level oracle (the plain MQA definition over the paged cache) timed on
    this host: float32 on every core the process may use (the reported value), the same
    pinned to one core with BLAS limited to one thread, and float64 (the parity
    precision) on every core.  A bounded sample of the workload's requests is used; the
    rate is in decode tokens (query rows) per second."""
    from oracle import mla_oracle as O
    kd = w.kv_dtype
    pool = O.encode_rows(w.kv_rows.reshape(-1, 576), kd).reshape(w.num_pages, 64, -1)
    sc = O.default_scale()
    if w.q is None:
        T = w.B * w.q_len
        q = O.round_to_bf16(O.absorb(O.bf16_bits_to_f64(w.q_nope.reshape(T, w.N, 128)),
                                     O.bf16_bits_to_f64(w.q_pe.reshape(T, w.N, 64)),
                                     O.bf16_bits_to_f64(w.w_uk_t))).reshape(w.B, w.q_len, w.N, 576)
    else:
        q = O.bf16_bits_to_f64(w.q)

    def timed(n_req: int, dtype, budget: float):
        qq = q[:n_req].astype(dtype)
        times = []
        t_all = time.perf_counter()
        while True:
            t0 = time.perf_counter()
            O.decode(qq, pool, kd, w.block_table[:n_req], w.seq_lens[:n_req], sc, dtype=dtype)
            times.append(time.perf_counter() - t0)
            if time.perf_counter() - t_all >= budget or len(times) >= 20:
                break
        mean = sum(times) / len(times)
        return n_req * w.q_len / mean, len(times), mean

    cores, blas = host_cores(), blas_threads()
    n_all = min(w.B, 16)
    v32, r32, m32 = timed(n_all, np.float32, budget_s)
    v64, r64, m64 = timed(n_all, np.float64, budget_s / 2)
    one = None
    try:
        from threadpoolctl import threadpool_limits
        keep = os.sched_getaffinity(0)
        os.sched_setaffinity(0, {min(keep)})
        try:
            with threadpool_limits(limits=1):
                v1, r1, m1 = timed(max(1, n_all // 4), np.float32, budget_s / 2)
            one = {"value": v1, "cores": 1, "sample": f"{max(1, n_all // 4)} requests, {r1} repetition(s), "
                                                      f"mean {m1:.3f} s"}
        finally:
            os.sched_setaffinity(0, keep)
    except Exception as e:                      # threadpoolctl missing: report why
        one = {"value": None, "error": str(e)}
    return {"value": v32, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"the first {n_all} of the {w.name} batch's {w.B} requests (q_len {w.q_len}, {w.N} heads) "
                      f"through the float32 decode oracle, {r32} repetition(s), mean {m32:.3f} s",
            "blas_threads": blas, "one_core": one,
            "float64": {"value": v64, "cores": cores, "sample": f"{n_all} requests, {r64} repetition(s), "
                                                                 f"mean {m64:.3f} s"}}


class Probe:
    """The measurement probes (libmla_probe.so): achievable HBM read and bf16 MFMA rates."""

    def __init__(self):
        import ctypes
        path = os.path.join(ROOT, "mla_paged_latent_amd", "libmla_probe.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} not found: build with `python -m mla_paged_latent_amd.build`")
        P = ctypes.CDLL(path)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        P.mla_probe_hbm_read.argtypes = [vp, ctypes.c_size_t, vp, vp]
        P.mla_probe_hbm_read.restype = i32
        P.mla_probe_mfma_bf16.argtypes = [vp, i32, vp]
        P.mla_probe_mfma_bf16.restype = i32
        P.mla_probe_sink_bytes.argtypes = []
        P.mla_probe_sink_bytes.restype = ctypes.c_size_t
        P.mla_probe_mfma_flops.argtypes = [i32]
        P.mla_probe_mfma_flops.restype = ctypes.c_double
        self.P = P

    def measure(self) -> dict:
        import torch
        P = self.P
        st = torch.cuda.current_stream().cuda_stream
        sink = torch.empty(P.mla_probe_sink_bytes(), dtype=torch.uint8, device="cuda")
        nb = 4 << 30                                        # 16x the 256 MB Infinity Cache
        buf = torch.ones(nb // 4, dtype=torch.int32, device="cuda")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(2):
            assert P.mla_probe_hbm_read(buf.data_ptr(), nb, sink.data_ptr(), st) == 0
        reads = []
        for _ in range(8):
            e0.record()
            assert P.mla_probe_hbm_read(buf.data_ptr(), nb, sink.data_ptr(), st) == 0
            e1.record()
            torch.cuda.synchronize()
            reads.append(nb / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        del buf
        iters = 20000
        for _ in range(2):
            assert P.mla_probe_mfma_bf16(sink.data_ptr(), iters, st) == 0
        rates = []
        for _ in range(5):
            e0.record()
            assert P.mla_probe_mfma_bf16(sink.data_ptr(), iters, st) == 0
            e1.record()
            torch.cuda.synchronize()
            rates.append(P.mla_probe_mfma_flops(iters) / (e0.elapsed_time(e1) * 1e-3) / 1e12)
        return {"hbm_read_gbs": round(max(reads), 1), "mfma_bf16_tflops": round(max(rates), 1),
                "method": "mla_probe_hbm_read: one pass over a 4 GiB buffer, 16-byte nontemporal loads, 8 in "
                          "flight per lane, 8 workgroups of 256 per CU (best of 8); mla_probe_mfma_bf16: four "
                          "independent v_mfma_f32_32x32x16_bf16 chains per wave, two waves per SIMD, register "
                          "operands (best of 5)"}


class DecodeSetup:
    """One workload's decode call on the device with R rotating copies of its cache pool,
    its C arguments marshalled once per copy."""

    def __init__(self, w: MI.Workload, num_splits: int, with_step: bool):
        import torch
        import mla_paged_latent_amd as M
        self.w = w
        kd = w.kv_dtype
        dev = torch.device("cuda:0")
        T = w.B * w.q_len
        self.bytes_alg, self.flops_alg, self.kv_bytes = algorithmic_work(w)
        row = M.ROW_BYTES[kd]
        # enough pool copies that consecutive reuse of one copy is >= 3 MALL capacities apart
        R = min(8, max(2, math.ceil(3 * MALL_BYTES / max(self.kv_bytes, 1))))
        self.R = R

        def bf16(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

        rows = bf16(w.kv_rows.reshape(-1, 576))
        slots = torch.arange(w.num_pages * 64, dtype=torch.int64, device=dev)
        self.pools = []
        for _ in range(R):
            pool = torch.empty((w.num_pages, 64, row), dtype=torch.uint8, device=dev)
            M.cache_write(rows[:, :512], rows[:, 512:], slots, pool, kd)
            self.pools.append(pool)
        del rows, slots
        self.bt = torch.from_numpy(w.block_table).to(dev)
        self.sl = torch.from_numpy(w.seq_lens).to(dev)
        self.new = bf16(w.new_rows)
        self.new_slots = torch.from_numpy(w.new_slots).to(dev)
        self.with_w = with_step and w.w_uk_t is not None
        if self.with_w:
            self.q_nope = bf16(w.q_nope.reshape(T, w.N, 128))
            self.q_pe = bf16(w.q_pe.reshape(T, w.N, 64))
            self.w_uk_t = bf16(w.w_uk_t)
            self.w_uv = bf16(w.w_uv)
            self.qf = torch.empty((T, w.N, 576), dtype=torch.bfloat16, device=dev)
            self.y = torch.empty((T, w.N * 128), dtype=torch.bfloat16, device=dev)
        elif w.q is not None:
            self.qf = bf16(w.q.reshape(T, w.N, 576))
        else:                                   # decode only on a weights workload: absorb once
            self.qf = M.absorb_q(bf16(w.q_nope.reshape(T, w.N, 128)), bf16(w.q_pe.reshape(T, w.N, 64)),
                                 bf16(w.w_uk_t))
        self.out = torch.empty((w.B, w.q_len, w.N, 512), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((w.B, w.q_len, w.N), dtype=torch.float32, device=dev)
        self.ws = torch.empty(M.decode_workspace_size(w.B, w.q_len, w.N, num_splits), dtype=torch.uint8,
                              device=dev)
        self.num_splits = num_splits
        L = M.lib()
        self.L = L
        st = torch.cuda.current_stream().cuda_stream
        qv = self.qf.view(w.B, w.q_len, w.N, 576)
        kc_new, kp_new = self.new[:, :512], self.new[:, 512:]
        self.cw_args = [(kc_new.data_ptr(), kc_new.stride(0), kp_new.data_ptr(), kp_new.stride(0),
                         self.new_slots.data_ptr(), self.new.shape[0], p.data_ptr(), kd, w.num_pages, st)
                        for p in self.pools]
        self.dec_args = [(qv.data_ptr(), qv.stride(0), qv.stride(1), qv.stride(2), p.data_ptr(), kd, w.num_pages,
                          self.bt.data_ptr(), self.bt.stride(0), self.bt.shape[1], self.sl.data_ptr(), w.B,
                          w.q_len, w.N, float(M.DEFAULT_SCALE), num_splits, self.ws.data_ptr(), self.ws.numel(),
                          self.out.data_ptr(), self.out.stride(0), self.out.stride(1), self.out.stride(2),
                          self.lse.data_ptr(), st) for p in self.pools]
        if self.with_w:
            ol = self.out.view(T, w.N, 512)
            self.ab_args = (self.q_nope.data_ptr(), self.q_nope.stride(0), self.q_nope.stride(1),
                            self.q_pe.data_ptr(), self.q_pe.stride(0), self.q_pe.stride(1), self.w_uk_t.data_ptr(),
                            T, w.N, self.qf.data_ptr(), self.qf.stride(0), self.qf.stride(1), st)
            self.uv_args = (ol.data_ptr(), ol.stride(0), ol.stride(1), self.w_uv.data_ptr(), T, w.N,
                            self.y.data_ptr(), self.y.stride(0), st)
            # the step's absorption and cache write as one launch (mla_absorb_q_cache_write)
            self.abcw_args = [self.ab_args[:-1] + a[:-1] + (st,) for a in self.cw_args]

    def step_api(self, i: int):
        """The step through the checked Python wrappers (used once, to check the fast path)."""
        import mla_paged_latent_amd as M
        w = self.w
        T = w.B * w.q_len
        pool = self.pools[i % self.R]
        M.cache_write(self.new[:, :512], self.new[:, 512:], self.new_slots, pool, w.kv_dtype)
        if self.with_w:
            M.absorb_q(self.q_nope, self.q_pe, self.w_uk_t, q_fused=self.qf)
        M.decode(self.qf.view(w.B, w.q_len, w.N, 576), pool, w.kv_dtype, self.bt, self.sl, M.DEFAULT_SCALE,
                 self.num_splits, workspace=self.ws, out=self.out, lse=self.lse)
        if self.with_w:
            M.up_v(self.out.view(T, w.N, 512), self.w_uv, out=self.y)

    def step(self, i: int):
        j = i % self.R
        L = self.L
        if self.with_w:
            rc = L.mla_absorb_q_cache_write(*self.abcw_args[j])
        else:
            rc = L.mla_cache_write(*self.cw_args[j])
        rc |= L.mla_decode(*self.dec_args[j])
        if self.with_w:
            rc |= L.mla_up_v(*self.uv_args)
        if rc != 0:
            raise RuntimeError(f"an mla_* call failed in step {i} (status bits {rc})")

    def outputs(self):
        return (self.out, self.lse, self.y) if self.with_w else (self.out, self.lse)


def time_back_to_back(fn, n: int, warm: int = 3) -> float:
    """Mean time (ms) of n calls of fn(i) enqueued back to back, one event pair around them."""
    import torch
    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def decode_distribution(s: DecodeSetup, rounds: int) -> list[float]:
    """Per-call mla_decode time (us) in each of `rounds` rounds; a round is R calls back to
    back (one per pool copy) under one event pair, so the copies rotate and no event sits
    between two calls."""
    import torch
    f = s.L.mla_decode
    # settle first: back-to-back calls for 0.2 s (the same steady state the step loop
    # is timed in; right after a setup the first ~100 calls run ~10 % slower)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.2:
        for i in range(20 * s.R):
            f(*s.dec_args[i % s.R])
        torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(rounds)]
    for r in range(rounds):
        ev[r][0].record()
        for j in range(s.R):
            f(*s.dec_args[j])
        ev[r][1].record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 / s.R for a, b in ev]


def pct(xs: list[float], q: float) -> float:
    ys = sorted(xs)
    return ys[min(len(ys) - 1, max(0, int(round(q * (len(ys) - 1)))))]


def roofline_record(bytes_alg: int, flops_alg: float, us: float, peaks: dict | None) -> dict:
    """Fractions of the published (and, when measured, the achievable) HBM and bf16 MFMA
    peaks for one launch of `us` microseconds; `binding` is the larger of the two
    published-peak times."""
    gbs = bytes_alg / (us * 1e-6) / 1e9
    tfs = flops_alg / (us * 1e-6) / 1e12
    t_hbm = bytes_alg / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops_alg / (MFMA_BF16_PEAK_TFS * 1e12)
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    rec = {"bound": bound, "hbm_gbs": round(gbs, 1), "mfma_tflops": round(tfs, 1),
           "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "mfma_frac_bf16": round(tfs / MFMA_BF16_PEAK_TFS, 4),
           "binding_frac": round(max(t_hbm, t_mfma) / (us * 1e-6), 4)}
    if peaks:
        m_hbm = bytes_alg / (peaks["hbm_read_gbs"] * 1e9)
        m_mfma = flops_alg / (peaks["mfma_bf16_tflops"] * 1e12)
        rec["hbm_frac_measured_peak"] = round(gbs / peaks["hbm_read_gbs"], 4)
        rec["mfma_frac_measured_peak"] = round(tfs / peaks["mfma_bf16_tflops"], 4)
        rec["binding_frac_measured_peaks"] = round(max(m_hbm, m_mfma) / (us * 1e-6), 4)
    return rec


def config_record(name: str, rounds: int, peaks: dict | None) -> dict:
    """mla_decode on one workload: distribution over rounds, rates, roofline fractions and
    the benchmark spec bar."""
    import torch
    w = MI.CONFIGS[name]()
    s = DecodeSetup(w, 0, with_step=False)
    us = decode_distribution(s, rounds)
    med = pct(us, 0.5)
    roof = roofline_record(s.bytes_alg, s.flops_alg, med, peaks)
    kind, bar = TARGETS.get(name, ("binding", None))
    got = roof["hbm_frac"] if kind == "hbm" else roof["binding_frac"]
    rec = {"workload": f"B={w.B}, q_len={w.q_len}, heads={w.N}, kv={'bf16' if w.kv_dtype == 0 else 'fp8'}, "
                       f"{w.tokens} cached tokens, {s.R} rotating pool copies",
           "us_median": round(med, 2), "us_p10": round(pct(us, 0.1), 2), "us_p90": round(pct(us, 0.9), 2),
           "rounds": rounds, "calls_per_round": s.R,
           "decode_tokens_per_s": round(w.B * w.q_len / (med * 1e-6), 1),
           "latent_kv_tbs": round(s.kv_bytes / (med * 1e-6) / 1e12, 3),
           "algorithmic_bytes": s.bytes_alg, "algorithmic_flops": s.flops_alg, **roof,
           "target": {"against": kind, "frac": bar, "met": (got >= bar) if bar is not None else None}}
    log(f"[bench] {name}: mla_decode median {med:.1f} us (p10 {rec['us_p10']:.1f}, p90 {rec['us_p90']:.1f}), "
        f"{roof['hbm_frac']:.3f} of HBM, {roof['mfma_frac_bf16']:.3f} of bf16 MFMA")
    del s
    torch.cuda.empty_cache()
    return rec


def run(args) -> dict:
    import torch
    import mla_paged_latent_amd as M

    peaks = None
    if not args.no_peaks:
        peaks = Probe().measure()
        log(f"[bench] measured peaks: HBM read {peaks['hbm_read_gbs']:.0f} GB/s, "
            f"bf16 MFMA {peaks['mfma_bf16_tflops']:.0f} TFLOP/s")

    w = MI.CONFIGS[args.workload]()
    kd = w.kv_dtype
    T = w.B * w.q_len
    s = DecodeSetup(w, args.num_splits, with_step=True)
    log(f"[bench] workload {w.name}: B={w.B} q_len={w.q_len} N={w.N} kv={'bf16' if kd == 0 else 'fp8'} "
        f"pages={w.num_pages} KV bytes/step={s.kv_bytes / 1e6:.1f} MB, pool copies={s.R}")
    if args.copy_calibration_mb > 0:
        # one device-to-device copy of a known size: under a --pmc run its FETCH_SIZE /
        # WRITE_SIZE give the counters' scale (see --traffic-record)
        nb = args.copy_calibration_mb * 2**20
        src = torch.ones(nb, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # The timed loops call the C entry points with their arguments marshalled once (the
    # tensor-checking Python wrappers cost tens of microseconds per call, enough to leave
    # the GPU idle between the step's kernels); checked here against the wrappers.
    s.step_api(0)
    torch.cuda.synchronize()
    ref = [t.clone() for t in s.outputs()]
    s.step(0)
    torch.cuda.synchronize()
    for a, b in zip(ref, s.outputs()):
        assert torch.equal(a, b), "marshalled step differs from the API step"

    # Untimed settling before the W warmup steps: right after the setup (host-side input
    # generation leaves the GPU idle for seconds) the step runs ~10 % slower for its
    # first ~100 repetitions; serving runs it back to back, so the timed steps start
    # from that steady state.  Steps are repeated until 0.2 s of them have run.
    settle = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < 0.2:
        for i in range(50):
            s.step(settle + i)
        settle += 50
        torch.cuda.synchronize()
    for i in range(args.warmup):
        s.step(i)
    torch.cuda.synchronize()
    # timed region 1: K whole steps, bracketed by one event pair (no events inside: an
    # event record between two kernels delays the next launch by several microseconds)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        s.step(i)
    stop.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    # timed region 2: each call of the step on its own, K calls back to back on the same
    # stream (rotating cache pools): the average launch durations, which add up to the step
    L = s.L
    kern = {"mla_cache_write": time_back_to_back(lambda i: L.mla_cache_write(*s.cw_args[i % s.R]), args.steps),
            "mla_decode": time_back_to_back(lambda i: L.mla_decode(*s.dec_args[i % s.R]), args.steps)}
    if s.with_w:
        kern["mla_absorb_q"] = time_back_to_back(lambda i: L.mla_absorb_q(*s.ab_args), args.steps)
        kern["mla_up_v"] = time_back_to_back(lambda i: L.mla_up_v(*s.uv_args), args.steps)
        kern["mla_absorb_q_cache_write"] = time_back_to_back(
            lambda i: L.mla_absorb_q_cache_write(*s.abcw_args[i % s.R]), args.steps)
    # timed region 3: the decode launch distribution (median / p10 / p90 over >= 50 rounds
    # of R back-to-back calls); its mean is the average launch duration the roofline uses
    # (150+ calls: region 2's K calls alone leave the mean to a few slow ones)
    dist = decode_distribution(s, max(50, args.steps))
    dec_mean = sum(dist) / len(dist) * 1e-3
    # the launches the step makes (the separate cache write and absorption are reported
    # beside them for reference)
    step_launches = (["mla_absorb_q_cache_write", "mla_decode", "mla_up_v"] if s.with_w
                     else ["mla_cache_write", "mla_decode"])
    step_sum = sum(kern[k] for k in step_launches)
    log(f"[bench] step {ms_step * 1e3:.1f} us; back to back per call: " +
        ", ".join(f"{k} {v * 1e3:.1f} us" for k, v in kern.items()) +
        f" (step's launches: sum {step_sum * 1e3:.1f} us); mla_decode median {pct(dist, 0.5):.1f} us")

    achieved = s.bytes_alg / (dec_mean * 1e-3) / 1e9
    tflops = s.flops_alg / (dec_mean * 1e-3) / 1e12
    t_hbm = s.bytes_alg / (HBM_PEAK_GBS * 1e9)
    t_mfma = s.flops_alg / (MFMA_BF16_PEAK_TFS * 1e12)
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFS,
                "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFS, 4)}
    roof["traffic"] = traffic_record(args.workload)
    roof["kernel"] = "mla_decode (split-KV decode with in-kernel split plan + LSE merge)"
    roof["algorithmic_bytes"] = s.bytes_alg
    roof["algorithmic_flops"] = s.flops_alg
    roof["mean_launch_us"] = round(dec_mean * 1e3, 2)
    roof["median_launch_us"] = round(pct(dist, 0.5), 2)
    roof["p10_launch_us"] = round(pct(dist, 0.1), 2)
    roof["p90_launch_us"] = round(pct(dist, 0.9), 2)
    roof["mfma_frac_bf16"] = round(tflops / MFMA_BF16_PEAK_TFS, 4)
    roof["hbm_frac"] = round(achieved / HBM_PEAK_GBS, 4)
    if peaks:
        roof["frac_measured_peak"] = round(achieved / peaks["hbm_read_gbs"], 4) if roof["bound"] == "hbm" else \
            round(tflops / peaks["mfma_bf16_tflops"], 4)

    res = {
        "metric": METRIC,
        "value": round(T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "settle_steps": settle,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if kd == MI.KV_BF16 else "fp8-e4m3 cache, bf16 mfma",
        "data": "synthetic (seeded N(0,1) latents/queries, N(0,1/512) weights; random page placement)",
        "config": {"workload": f"{w.name}: B={w.B}, q_len={w.q_len}, heads={w.N}, "
                               f"seq_lens={'all ' + str(int(w.seq_lens[0])) if len(set(w.seq_lens.tolist())) == 1 else 'mixed'}, "
                               f"kv={'bf16' if kd == 0 else 'fp8'} 576-d rows, 64-token pages, "
                               f"{'absorb + ' if s.with_w else ''}cache write + decode{' + up-proj' if s.with_w else ''}",
                   "batch": w.B, "q_len": w.q_len, "heads": w.N, "kv_tokens": w.tokens,
                   "num_splits": args.num_splits, "pool_copies": s.R},
        "decode_latent_kv_tbs": round(s.kv_bytes / (dec_mean * 1e-3) / 1e12, 3),
        "roofline": roof,
        "step_kernels_us": {k: round(v * 1e3, 2) for k, v in kern.items()},
        "step_launches": step_launches,
        "step_kernels_sum_us": round(step_sum * 1e3, 2),
    }
    if peaks:
        res["measured_peaks"] = peaks
    del s
    torch.cuda.empty_cache()
    if not args.no_configs:
        res["decode_configs"] = {}
        for name in args.configs.split(","):
            res["decode_configs"][name] = config_record(name, max(50, args.steps), peaks)
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
    # the keys and values those 8192 new tokens attend over, up-projected from their
    # latents: [k_nope | v][s, h] = kv_c[s] . W_KVB[h], 128 heads
    "kv_b_proj_prefill": dict(kind="kvb", S=8192, N=128),
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
    elif op["kind"] == "kvb":
        S, N = op["S"], op["N"]
        per_copy = N * 512 * 256 * 2 + S * 512 * 2
        R = max(2, min(8, math.ceil(3 * MALL_BYTES / per_copy)))
        gen = torch.Generator(device=dev).manual_seed(570)
        ws = [(torch.randn(N, 512, 256, device=dev, generator=gen) / math.sqrt(512)).to(torch.bfloat16)
              for _ in range(R)]
        kcs = [torch.randn(S, 576, device=dev, generator=gen).to(torch.bfloat16) for _ in range(R)]
        out = torch.empty((S, N, 256), dtype=torch.bfloat16, device=dev)
        calls = [(kcs[i].data_ptr(), kcs[i].stride(0), ws[i].data_ptr(), S, N, out.data_ptr(), out.stride(0),
                  out.stride(1), stream) for i in range(R)]
        f = L.mla_kv_b_proj
        bytes_alg = per_copy + S * N * 256 * 2
        flops_alg = 2.0 * S * N * 512 * 256
        desc = (f"{args.op}: S={S} latent rows (the [S, 576] rows' first 512) x {N} heads, "
                f"kv_c [S, 512] . W_KVB [N, 512, 256] -> [k_nope | v] [S, N, 256] bf16, {R} rotating input copies")
        metric = "prefill key / value up-projection TFLOP/s (% of bf16 MFMA roofline), 1 MI355X"
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
    # settle as the decode step does: 0.2 s of back-to-back calls before the timed ones
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < 0.2:
        for _ in range(10):
            f(*calls[i % len(calls)])
            i += 1
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
    if op["kind"] in ("varlen", "prefill", "kvb") and flops_alg / (MFMA_BF16_PEAK_TFS * 1e12) > bytes_alg / (HBM_PEAK_GBS * 1e9):
        tfs = flops_alg / (mean_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(tfs, 1), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4)}
    roof.update({"traffic": None, "kernel": args.op, "algorithmic_bytes": bytes_alg,
                 "mean_launch_us": round(mean_ms * 1e3, 2), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)})
    if op["kind"] in ("varlen", "upv", "rope", "prefill", "kvb"):
        roof["algorithmic_flops"] = flops_alg
    if bf16_out_us is not None:
        roof["unfused_call_us"] = bf16_out_us
    value, unit = (roof["achieved"], roof["unit"]) if roof["bound"] == "mfma" else (round(gbs, 1), "GB/s")
    res = {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(mean_ms, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": dtype, "data": "synthetic (seeded)", "config": {"workload": desc},
           "roofline": roof}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_context(args.op, unit)
    return res


def cpu_baseline_context(name: str, unit: str = "GB/s", budget_s: float = 10.0) -> dict:
    """The oracle on a bounded sample of the same workload, in the record's unit (GB/s, or
    TFLOP/s for the calls whose record is priced against the MFMA peak)."""
    from oracle import mla_oracle as O
    op = CONTEXT_OPS[name]
    times, n_items, flops_item = [], 0, None
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
    elif op["kind"] == "kvb":
        S, N = 64, op["N"]
        rng = np.random.default_rng(571)
        kc = rng.standard_normal((S, 512))
        w = rng.standard_normal((N, 512, 256)) / np.sqrt(512)
        while time.perf_counter() - t_all < budget_s and len(times) < 20:
            t0 = time.perf_counter()
            O.f64_to_bf16_bits(np.concatenate(O.kv_b_proj(kc, w), axis=-1))
            times.append(time.perf_counter() - t0)
        n_items = 1
        per_item = N * 512 * 256 * 2 + S * 512 * 2 + S * N * 256 * 2
        flops_item = 2.0 * S * N * 512 * 256
        sample = f"S={S} latent rows x {N} heads through the oracle kv_b_proj"
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
        flops_item = Lq * (Lq + 1) / 2 * N * (2 * 192 + 2 * 128)
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
    if unit == "TFLOP/s" and flops_item is not None:
        value = round(n_items * flops_item / mean / 1e12, 6)
    else:
        value, unit = round(n_items * per_item / mean / 1e9, 3), "GB/s"
    return {"value": value, "unit": unit, "cores": host_cores(), "kind": "oracle",
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
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured HBM / MFMA peaks")
    ap.add_argument("--no-configs", action="store_true",
                    help="time only the --workload step, not the per-config decode records")
    ap.add_argument("--configs", default="tp_share,full_head,fp8,spec_long",
                    help="workloads whose mla_decode gets a record of its own (comma separated)")
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

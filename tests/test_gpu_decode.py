"""GPU parity of mla_decode (and the whole step around it) against the oracle.

Gates (tests/mla_testlib.py): per request, the largest output error net of half a
bf16 ulp of the larger magnitude must stay within 2e-2 * RMS of that request's
reference output; max |lse_gpu - lse_ref| <= 1e-3; rows that see no token must give
o = 0 and lse = -inf exactly; the cache pool must match the oracle byte for byte.
"""

import math

import numpy as np
import pytest
import torch

import mla_inputs as MI
import mla_paged_latent_amd as M
from oracle import mla_oracle as O
from tests.mla_testlib import (check_lse, check_out, dev_bf16, gpu_decode, gpu_pool, host_bits,
                               oracle_pool, say, step_write_new_tokens_gpu,
                               step_write_new_tokens_oracle, to_f64)

pytestmark = pytest.mark.gpu

SC = O.default_scale()


def _run_step(w: MI.Workload, num_splits: int = 0, unabsorbed_samples=None):
    """The whole path on one workload: pool + new-token cache write (bit-exact),
    absorb (when the workload has weights), decode, up-projection."""
    kd = w.kv_dtype
    say(f"[{w.name}] pool write: {w.num_pages} pages, kv_dtype={kd}")
    pool = gpu_pool(w)
    ref_pool = oracle_pool(w)
    step_write_new_tokens_gpu(w, pool, kd)
    ref_pool = step_write_new_tokens_oracle(w, ref_pool, kd)
    torch.cuda.synchronize()
    assert np.array_equal(pool.cpu().numpy(), ref_pool), f"{w.name}: cache pool differs"

    if w.q is None:
        say(f"[{w.name}] absorb_q")
        T = w.B * w.q_len
        qf = M.absorb_q(dev_bf16(w.q_nope.reshape(T, w.N, 128)), dev_bf16(w.q_pe.reshape(T, w.N, 64)),
                        dev_bf16(w.w_uk_t))
        q_dev = qf.view(w.B, w.q_len, w.N, 576)
        # the oracle's own absorbed query, stored as bf16 like the pipeline's tensor
        q_ref = O.round_to_bf16(O.absorb(O.bf16_bits_to_f64(w.q_nope.reshape(T, w.N, 128)),
                                         O.bf16_bits_to_f64(w.q_pe.reshape(T, w.N, 64)),
                                         O.bf16_bits_to_f64(w.w_uk_t))).reshape(w.B, w.q_len, w.N, 576)
    else:
        q_dev = dev_bf16(w.q)
        q_ref = O.bf16_bits_to_f64(w.q)

    say(f"[{w.name}] decode num_splits={num_splits}")
    out, lse = M.decode(q_dev, pool, kd, torch.from_numpy(w.block_table).cuda(),
                        torch.from_numpy(w.seq_lens).cuda(), SC, num_splits)
    torch.cuda.synchronize()
    say(f"[{w.name}] oracle decode")
    o_ref, lse_ref = O.decode(q_ref, ref_pool, kd, w.block_table, w.seq_lens, SC)
    check_out(to_f64(out), o_ref, w.name)
    check_lse(lse.cpu().numpy(), lse_ref, w.name)

    if w.w_uv is not None:
        say(f"[{w.name}] up_v + un-absorbed oracle")
        T = w.B * w.q_len
        y = M.up_v(out.view(T, w.N, 512), dev_bf16(w.w_uv))
        torch.cuda.synchronize()
        y = to_f64(y).reshape(w.B, w.q_len, w.N, 128)
        qn = O.bf16_bits_to_f64(w.q_nope)
        qp = O.bf16_bits_to_f64(w.q_pe)
        wk = O.bf16_bits_to_f64(w.w_uk_t)
        wv = O.bf16_bits_to_f64(w.w_uv)
        if unabsorbed_samples is None:
            y_ref, l_ref = O.mla_unabsorbed(qn, qp, ref_pool, kd, w.block_table, w.seq_lens, wk, wv, SC)
            check_out(y, y_ref, w.name + " end-to-end y")
            e2e = float(np.max(np.abs(lse.cpu().numpy() - l_ref)))
        else:
            e2e = 0.0
            errs, refs = [], []
            bs, hs = unabsorbed_samples
            y_ref, l_ref = O.mla_unabsorbed(qn, qp, ref_pool, kd, w.block_table, w.seq_lens, wk, wv,
                                            SC, heads=hs, batches=bs)
            for b in bs:
                for h in hs:
                    errs.append(np.abs(y[b, :, h] - y_ref[b, :, h]))
                    refs.append(y_ref[b, :, h])
                    e2e = max(e2e, float(np.max(np.abs(lse.cpu().numpy()[b, :, h] - l_ref[b, :, h]))))
            rms = math.sqrt(float(np.mean(np.concatenate(refs) ** 2)))
            err = float(np.max(np.concatenate(errs)))
            say(f"  [{w.name} end-to-end y, sampled] max|err| = {err:.3e}, rms = {rms:.3e}")
            assert err <= 2e-2 * rms
        say(f"  [{w.name}] end-to-end lse max|err| vs un-absorbed oracle = {e2e:.3e} (reported)")


def test_tiny_workload_end_to_end():
    _run_step(MI.tiny())


def test_tp_share_workload():
    _run_step(MI.tp_share())


def test_full_head_workload_end_to_end():
    # the un-absorbed oracle up-projects every cached latent per head (~1 GFLOP per
    # request and head in float64): 6 requests x 6 heads, both head groups and both
    # ends of each
    _run_step(MI.full_head(), unabsorbed_samples=([0, 5, 13, 18, 26, 31], [0, 17, 63, 64, 100, 127]))


def test_fp8_workload():
    _run_step(MI.fp8())


def test_spec_long_workload():
    _run_step(MI.spec_long())


# ---------------------------------------------------------------------------
# split plans, determinism, paging
# ---------------------------------------------------------------------------
def _small(name, N, q_len, seq, kd=MI.KV_BF16, seed=60, pages=None):
    return MI.make_workload(name, len(seq), q_len, N, seq, pages, kd, False, seed)


@pytest.mark.parametrize("N,q_len", [(128, 1), (16, 1), (128, 2), (16, 2)])
def test_split_count_sweep(N, q_len):
    w = _small("sweep", N, q_len, [1, 64, 65, 700, 2049, 5000])
    pool = gpu_pool(w)
    ref_pool = oracle_pool(w)
    q_ref = O.bf16_bits_to_f64(w.q)
    o_ref, lse_ref = O.decode(q_ref, ref_pool, w.kv_dtype, w.block_table, w.seq_lens, SC)
    for ns in (1, 0, 2, 7, 64, 300):
        say(f"split sweep N={N} q_len={q_len} num_splits={ns}")
        out, lse = gpu_decode(w, pool, w.q, ns)
        check_out(to_f64(out), o_ref, f"N{N} q{q_len} splits{ns}")
        check_lse(lse.cpu().numpy(), lse_ref, f"N{N} q{q_len} splits{ns}")


@pytest.mark.parametrize("N", [128, 16])
def test_run_twice_bit_identical_and_page_permutation(N):
    w = _small("perm", N, 1, [3000, 100, 64, 1999], seed=61)
    pool = gpu_pool(w)
    for ns in (0, 1, 5):
        say(f"determinism N={N} num_splits={ns}")
        o1, l1 = gpu_decode(w, pool, w.q, ns)
        o2, l2 = gpu_decode(w, pool, w.q, ns)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        # permute the physical pages and remap the block table: identical bits
        perm = np.random.default_rng(ns).permutation(w.num_pages)
        inv = np.argsort(perm)
        bt2 = np.where(w.block_table >= 0, inv[np.maximum(w.block_table, 0)], -1).astype(np.int32)
        pool2 = pool[torch.from_numpy(perm).cuda()].contiguous()
        o3, l3 = gpu_decode(w, pool2, w.q, ns, block_table=bt2)
        assert torch.equal(o1, o3) and torch.equal(l1, l3)


def test_single_split_is_batch_invariant():
    """num_splits = 1: a request's result does not depend on the rest of the batch."""
    w = _small("inv", 128, 1, [500, 3000, 77], seed=62)
    pool = gpu_pool(w)
    o_all, l_all = gpu_decode(w, pool, w.q, 1)
    for b in range(w.B):
        o_b, l_b = gpu_decode(w, pool, w.q[b:b + 1].copy(), 1, seq_lens=w.seq_lens[b:b + 1],
                              block_table=w.block_table[b:b + 1].copy())
        assert torch.equal(o_b[0], o_all[b]) and torch.equal(l_b[0], l_all[b])


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("N", [1, 3, 16, 40, 100, 128])
def test_head_counts_and_ragged_tails(N):
    w = _small("heads", N, 1, [1, 63, 64, 65, 127, 129, 1000], seed=63 + N)
    pool = gpu_pool(w)
    o_ref, lse_ref = O.decode(O.bf16_bits_to_f64(w.q), oracle_pool(w), w.kv_dtype, w.block_table,
                              w.seq_lens, SC)
    for ns in (0, 3):
        say(f"heads N={N} ns={ns}")
        out, lse = gpu_decode(w, pool, w.q, ns)
        check_out(to_f64(out), o_ref, f"N{N}")
        check_lse(lse.cpu().numpy(), lse_ref, f"N{N}")


@pytest.mark.parametrize("N,q_len", [(128, 2), (8, 2), (16, 1), (128, 1)])
def test_empty_rows_and_zero_length_requests(N, q_len):
    # seq 0: every row empty; seq 1 with q_len 2: row 0 sees nothing
    w = _small("empty", N, q_len, [0, 1, 2, 70], seed=70 + N)
    pool = gpu_pool(w)
    o_ref, lse_ref = O.decode(O.bf16_bits_to_f64(w.q), oracle_pool(w), w.kv_dtype, w.block_table,
                              w.seq_lens, SC)
    for ns in (0, 1, 4):
        say(f"empty rows N={N} q_len={q_len} ns={ns}")
        out, lse = gpu_decode(w, pool, w.q, ns)
        o = to_f64(out)
        l = lse.cpu().numpy()
        empty = np.isneginf(lse_ref)
        assert empty.any()
        assert np.all(o[empty] == 0.0) and np.all(np.isneginf(l[empty]))
        check_out(o, o_ref, "empty")
        check_lse(l, lse_ref, "empty")


def test_single_token_context_is_exact():
    """One visible token: p = 1 exactly, so the output is that token's latent, bit for bit."""
    w = _small("one", 128, 1, [1, 1, 65], seed=80)
    pool = gpu_pool(w)
    out, lse = gpu_decode(w, pool, w.q, 0)
    pb = oracle_pool(w)
    for b in (0, 1):
        row = pb[w.block_table[b, 0], 0].view("<u2")
        assert np.array_equal(host_bits(out[b, 0]), np.broadcast_to(row[:512], (128, 512)))


def test_stale_nan_rows_past_the_end_are_ignored():
    """Pool rows past seq_len hold NaN bit patterns; they must not reach the output."""
    w = _small("nan", 128, 2, [70, 5, 129], seed=81)
    pool = gpu_pool(w)
    nan_row = torch.full((576,), float("nan"), dtype=torch.bfloat16, device="cuda")
    pv = pool.view(w.num_pages, 64, 576 * 2)
    for b, s in enumerate(w.seq_lens):
        last = int(w.block_table[b, (int(s) - 1) // 64])
        for off in range(int(s) % 64 or 64, 64):
            pv[last, off] = nan_row.view(torch.uint8)
    torch.cuda.synchronize()
    o_ref, lse_ref = O.decode(O.bf16_bits_to_f64(w.q), oracle_pool(w), w.kv_dtype, w.block_table,
                              w.seq_lens, SC)
    for ns in (0, 1):
        out, lse = gpu_decode(w, pool, w.q, ns)
        check_out(to_f64(out), o_ref, "nan tails")
        check_lse(lse.cpu().numpy(), lse_ref, "nan tails")


@pytest.mark.parametrize("N,q_len,kd", [(16, 1, MI.KV_BF16), (128, 1, MI.KV_BF16), (64, 2, MI.KV_BF16),
                                         (128, 1, MI.KV_FP8)])
def test_many_requests_plan_scan(N, q_len, kd):
    """More than 256 requests, many of them short or empty: the planner's scan spans
    several entries per thread and every stream runs through many pieces, so blocks of
    the next piece are prefetched across piece boundaries (both kernel variants)."""
    rng = np.random.default_rng(82 + N + q_len)
    seq = rng.integers(0, 300, size=600) * (rng.random(600) > 0.1)
    w = MI.make_workload("many", 600, q_len, N, seq, None, kd, False, 82)
    pool = gpu_pool(w)
    o_ref, lse_ref = O.decode(O.bf16_bits_to_f64(w.q), oracle_pool(w), w.kv_dtype, w.block_table,
                              w.seq_lens, SC)
    for ns in (0, 2):
        out, lse = gpu_decode(w, pool, w.q, ns)
        check_out(to_f64(out), o_ref, "many")
        check_lse(lse.cpu().numpy(), lse_ref, "many")


@pytest.mark.parametrize("N,kd", [(16, MI.KV_BF16), (128, MI.KV_BF16), (128, MI.KV_FP8)])
def test_wide_block_table_takes_the_64bit_plan_kernels(N, kd):
    """A block table 70000 pages wide puts a bound on the plan's products past 32 bits,
    so the kernels built with 64-bit plan arithmetic run (their 32-bit path, as these
    lengths are small): same bits as the kernels a narrow table selects, and parity."""
    w = _small("wide-bt", N, 1, [300, 1000, 4100, 64], kd=kd, seed=95)
    pool = gpu_pool(w)
    o_ref, lse_ref = O.decode(O.bf16_bits_to_f64(w.q), oracle_pool(w), w.kv_dtype, w.block_table,
                              w.seq_lens, SC)
    wide = np.full((w.B, 70000), -1, dtype=np.int32)
    wide[:, :w.block_table.shape[1]] = w.block_table
    for ns in (0, 3):
        say(f"wide block table N={N} kd={kd} ns={ns}")
        o_n, l_n = gpu_decode(w, pool, w.q, ns)
        o_w, l_w = gpu_decode(w, pool, w.q, ns, block_table=wide)
        assert torch.equal(o_n, o_w) and torch.equal(l_n, l_w)
        check_out(to_f64(o_w), o_ref, "wide block table")
        check_lse(l_w.cpu().numpy(), lse_ref, "wide block table")


@pytest.mark.parametrize("N", [128, 16])
def test_fp8_rows_with_distinct_k_and_v_scales(N):
    """fp8 rows whose K and V scales differ: each scale must be applied to its view."""
    rng = np.random.default_rng(90 + N)
    seq = [200, 64, 1]
    w = MI.make_workload("fp8s", 3, 1, N, seq, None, MI.KV_FP8, False, 90 + N)
    rows = MI.random_fp8_rows(rng, w.num_pages * 64, max_code_exp=8)
    ref_pool = rows.reshape(w.num_pages, 64, 584)
    pool = torch.from_numpy(ref_pool.copy()).cuda()
    o_ref, lse_ref = O.decode(O.bf16_bits_to_f64(w.q), ref_pool, MI.KV_FP8, w.block_table, w.seq_lens, SC)
    for ns in (0, 1):
        out, lse = gpu_decode(w, pool, w.q, ns)
        check_out(to_f64(out), o_ref, "fp8 scales")
        check_lse(lse.cpu().numpy(), lse_ref, "fp8 scales")


@pytest.mark.parametrize("N", [16, 128])
def test_fp8_rows_with_zero_v_scale(N):
    """fp8 rows whose v_scale is 0 have V = 0 but keep their weight in the softmax
    (a row's output must still be the convex combination the oracle forms), also when
    such a token holds a row's largest score: in every request one visible token gets
    a large K scale and a zero V scale."""
    rng = np.random.default_rng(190 + N)
    seq = [200, 64, 37]
    w = MI.make_workload("fp8v0", 3, 1, N, seq, None, MI.KV_FP8, False, 190 + N)
    rows = MI.random_fp8_rows(rng, w.num_pages * 64, max_code_exp=8)
    ks = rows[:, 576:580].copy().view("<f4").reshape(-1)
    vs = rows[:, 580:584].copy().view("<f4").reshape(-1)
    zero = rng.random(len(vs)) < 0.2
    for b, n in enumerate(seq):
        t = int(rng.integers(0, n))
        slot = int(w.block_table[b, t // 64]) * 64 + t % 64
        zero[slot] = True
        ks[slot] = 16.0
    vs[zero] = 0.0
    rows[:, 576:580] = ks.astype("<f4").view(np.uint8).reshape(-1, 4)
    rows[:, 580:584] = vs.astype("<f4").view(np.uint8).reshape(-1, 4)
    ref_pool = rows.reshape(w.num_pages, 64, 584)
    pool = torch.from_numpy(ref_pool.copy()).cuda()
    o_ref, lse_ref = O.decode(O.bf16_bits_to_f64(w.q), ref_pool, MI.KV_FP8, w.block_table, w.seq_lens, SC)
    for ns in (0, 1):
        say(f"fp8 zero v_scale N={N} ns={ns}")
        out, lse = gpu_decode(w, pool, w.q, ns)
        check_out(to_f64(out), o_ref, "fp8 zero v_scale")
        check_lse(lse.cpu().numpy(), lse_ref, "fp8 zero v_scale")


@pytest.mark.parametrize("N", [16, 128])
def test_large_score_range_triggers_reference_redo(N):
    """Scores that grow by far more than the reference slack within a unit: the
    kernel redoes the unit with a larger reference and still matches the oracle."""
    w = _small("range", N, 1, [640, 640], seed=83)
    rows = w.kv_rows.copy()
    # scale up the latents of one late page of each request by 2^7
    for b in range(2):
        pg = int(w.block_table[b, 8])
        f = O.bf16_bits_to_f64(rows[pg]) * 128.0
        rows[pg] = MI.to_bf16_bits(f.astype(np.float32))
    w.kv_rows = rows
    pool = gpu_pool(w)
    o_ref, lse_ref = O.decode(O.bf16_bits_to_f64(w.q), oracle_pool(w), w.kv_dtype, w.block_table,
                              w.seq_lens, SC)
    for ns in (1, 0):
        out, lse = gpu_decode(w, pool, w.q, ns)
        check_out(to_f64(out), o_ref, "range")
        check_lse(lse.cpu().numpy(), lse_ref, "range")


@pytest.mark.parametrize("N,q_len,wl", [(128, 1, "mixed"), (16, 1, "mixed"), (128, 2, "mixed"), (128, 1, "fp8")])
def test_device_split_plan_matches_the_cpu_model(N, q_len, wl):
    """The per-request record the decode kernels leave in the workspace ({first partial
    slot, number of pieces, -, clamped seq_len}) equals the CPU model of the plan."""
    from tests.test_split_plan_model import plan_auto
    if wl == "fp8":
        w = MI.fp8()
    else:
        rng = np.random.default_rng(70 + N + q_len)
        seq = (rng.integers(1, 6000, 48) * (rng.random(48) > 0.1)).tolist()
        w = _small("plan", N, q_len, [max(q_len, s) if s else 0 for s in seq], seed=70 + N)
    cus = (torch.cuda.get_device_properties(0).multi_processor_count + 7) // 8 * 8
    rows = 16 if q_len * N <= 16 else 64
    n_hg = -(-N // (rows // q_len))
    streams = cus if n_hg == 1 else max(8, cus // (8 * n_hg) * 8)
    width = w.block_table.shape[1]
    stretch = 4 + width
    p64 = w.B * stretch > 0xFFFFFFFF // (streams + 1) or stretch * width > 0xFFFFFFFF
    pool = gpu_pool(w)
    ws = torch.zeros(M.decode_workspace_size(w.B, w.q_len, w.N, 0), dtype=torch.uint8, device="cuda")
    q = dev_bf16(w.q) if w.q is not None else torch.zeros((w.B, w.q_len, w.N, 576), dtype=torch.bfloat16,
                                                          device="cuda")
    M.decode(q, pool, w.kv_dtype, torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda(),
             SC, 0, workspace=ws)
    torch.cuda.synchronize()
    dev = ws[: 16 * w.B].cpu().view(torch.int32).numpy().reshape(w.B, 4)
    seqm, pieces, req, _ = plan_auto(w.seq_lens.tolist(), streams, width * 64, p64)
    for b in range(w.B):
        first, n, _s = req[b][0]
        assert (int(dev[b, 0]), int(dev[b, 1]), int(dev[b, 3])) == (first, n, seqm[b]), (b, dev[b], req[b])

"""GPU parity of the steps either side of decode: the context gather
(mla_gather_cache, bit-exact against the oracle, bf16 and fp8) and the two-state
merge (mla_merge_attn_states, within one bf16 rounding of the float64 oracle),
plus the merge of two decodes over a split context against one decode."""

import math

import numpy as np
import pytest
import torch

import mla_inputs as MI
import mla_paged_latent_amd as M
from oracle import mla_oracle as O
from tests.mla_testlib import (bf16_half_ulp, check_lse, check_out, dev_bf16, gpu_decode, gpu_pool, host_bits,
                               oracle_pool, say, to_f64)

pytestmark = pytest.mark.gpu


def _chunk_on_gpu(c: MI.ContextChunk):
    return (torch.from_numpy(c.block_table).cuda(), torch.from_numpy(c.cu_seq_lens).cuda(),
            torch.from_numpy(c.token_to_seq).cuda(), torch.from_numpy(c.seq_starts).cuda())


def _pool_workload(num_pages, kd, seed):
    # a pool of random rows written by the cache write (the rows' content is what gets gathered)
    return MI.make_workload("ctx-pool", 1, 1, 16, [64], num_pages, kd, False, seed)


@pytest.mark.parametrize("kd", [MI.KV_BF16, MI.KV_FP8])
@pytest.mark.parametrize("with_starts", [False, True])
def test_gather_cache_bit_exact(kd, with_starts):
    lens = [130, 64, 1, 200, 4096, 63, 65]
    starts = [64, 0, 0, 128, 1024, 0, 192] if with_starts else [0] * 7
    c = MI.make_context_chunk(lens, starts, 200, seed=120 + kd)
    w = _pool_workload(c.num_pages, kd, 121)
    pool = gpu_pool(w, kd)
    ref_pool = oracle_pool(w, kd)
    bt, cu, t2s, ss = _chunk_on_gpu(c)
    say(f"gather kd={kd} starts={with_starts} rows={c.total}")
    out = M.gather_cache(pool, kd, bt, cu, t2s, ss if with_starts else None)
    torch.cuda.synchronize()
    ref = O.gather_cache(ref_pool, kd, c.block_table, c.cu_seq_lens, c.token_to_seq,
                         c.seq_starts if with_starts else None)
    assert np.array_equal(host_bits(out), ref)


def test_gather_cache_fp8_random_codes_and_scales_rounding():
    """Random codes with independent random K/V scales: ~10^7 products, some of them
    exactly halfway between two bf16 values, all rounded once like the oracle."""
    rng = np.random.default_rng(122)
    num_pages = 300
    rows = MI.random_fp8_rows(rng, num_pages * 64, max_code_exp=15)
    rows[:, :576][(rows[:, :576] & 0x7F) == 0x7F] = 0x7E          # no NaN codes here
    pool_np = rows.reshape(num_pages, 64, 584)
    pool = torch.from_numpy(pool_np.copy()).cuda()
    c = MI.make_context_chunk([num_pages * 64], [0], num_pages, seed=123)
    bt, cu, t2s, _ = _chunk_on_gpu(c)
    out = M.gather_cache(pool, MI.KV_FP8, bt, cu, t2s)
    torch.cuda.synchronize()
    ref = O.gather_cache(pool_np, MI.KV_FP8, c.block_table, c.cu_seq_lens, c.token_to_seq)
    got = host_bits(out)
    prod = O.e4m3_value(pool_np.reshape(-1, 584)[:, :576]) * \
        pool_np.reshape(-1, 584)[:, 576:580].copy().view("<f4").astype(np.float64)
    ties = np.count_nonzero((prod.astype(np.float32).view(np.uint32) & 0xFFFF) == 0x8000)
    say(f"fp8 gather: {got.size} values, {ties} of them with a float32 product on a bf16 tie")
    assert np.array_equal(got, ref)


def test_gather_cache_fp8_nan_codes_and_hand_values():
    pool_np = np.zeros((1, 64, 584), np.uint8)
    pool_np[0, :, :576] = np.arange(64)[:, None] * 2 + 1          # codes 1, 3, ..., 127 (127 = NaN)
    pool_np[0, :, 576:580] = np.array([1 + 2**-8], "<f4").view(np.uint8)
    pool_np[0, :, 580:584] = np.array([7.0], "<f4").view(np.uint8)
    pool = torch.from_numpy(pool_np.copy()).cuda()
    c = MI.make_context_chunk([64], [0], 1, seed=124)
    bt, cu, t2s, _ = _chunk_on_gpu(c)
    got = host_bits(M.gather_cache(pool, MI.KV_FP8, bt, cu, t2s))
    ref = O.gather_cache(pool_np, MI.KV_FP8, c.block_table, c.cu_seq_lens, c.token_to_seq)
    nan_g = (got & 0x7FFF) > 0x7F80
    nan_r = (ref & 0x7FFF) > 0x7F80
    assert np.array_equal(nan_g, nan_r) and nan_r.sum() == 576
    assert np.array_equal(got[~nan_r], ref[~nan_r])


@pytest.mark.parametrize("kd", [MI.KV_BF16, MI.KV_FP8])
def test_gather_cache_out_of_range_rows_are_zero(kd):
    say(f"gather out-of-range rows kd={kd}")
    c = MI.make_context_chunk([100, 50], [0, 64], 10, seed=125)
    w = _pool_workload(c.num_pages, kd, 126)
    pool = gpu_pool(w, kd)
    t2s = c.token_to_seq.copy()
    t2s[[3, 120]] = [-1, 7]                               # no such request
    bt = c.block_table.copy()
    bt[1, 1] = 10**6                                      # page id outside the pool
    out = M.gather_cache(pool, kd, torch.from_numpy(bt).cuda(), torch.from_numpy(c.cu_seq_lens).cuda(),
                         torch.from_numpy(t2s).cuda(), torch.from_numpy(c.seq_starts).cuda())
    got = host_bits(out)
    assert np.all(got[3] == 0) and np.all(got[120] == 0)
    # request 1 starts at its token 64 = page 1: its first 50 rows come from that page
    assert np.all(got[100:150] == 0)
    ref = O.gather_cache(oracle_pool(w, kd), kd, c.block_table, c.cu_seq_lens, c.token_to_seq, c.seq_starts)
    keep = np.ones(150, bool)
    keep[[3, 120]] = False
    keep[100:150] = False
    assert np.array_equal(got[keep], ref[keep])


def _check_merge(o_gpu, l_gpu, po, pl, so, sl, name):
    o_ref, l_ref = O.merge_attn_states(O.bf16_bits_to_f64(po), pl, O.bf16_bits_to_f64(so), sl)
    o = O.bf16_bits_to_f64(o_gpu)
    empty = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(l_gpu), empty) and np.all(o[empty] == 0)
    # one bf16 rounding of the result plus float32 arithmetic on the inputs' scale
    a = np.abs(o_ref)
    _, e = np.frexp(np.where(a > 0, a, 1.0))
    half_ulp = np.where(a > 0, np.ldexp(1.0, e - 9), 0.0)
    scale = np.maximum(np.abs(O.bf16_bits_to_f64(po)), np.abs(O.bf16_bits_to_f64(so)))
    err = np.abs(o - o_ref) - half_ulp - 1e-6 * scale
    say(f"  [{name}] merge: worst excess over half a bf16 ulp = {err.max():.3e}")
    assert err.max() <= 0
    fin = ~empty
    assert np.max(np.abs(l_gpu[fin] - l_ref[fin]) / np.maximum(1.0, np.abs(l_ref[fin]))) <= 1e-6


@pytest.mark.parametrize("T,N,D", [(1, 1, 8), (37, 16, 128), (300, 128, 512), (1000, 3, 64)])
def test_merge_attn_states_parity(T, N, D):
    po, pl, so, sl = MI.random_attn_states(T, N, D, seed=130 + D)
    say(f"merge T={T} N={N} D={D}")
    o, l = M.merge_attn_states(dev_bf16(po), torch.from_numpy(pl).cuda(), dev_bf16(so),
                               torch.from_numpy(sl).cuda())
    torch.cuda.synchronize()
    _check_merge(host_bits(o), l.cpu().numpy(), po, pl, so, sl, f"T{T} N{N} D{D}")


def test_merge_attn_states_strided_head_major_lse():
    """LSE stored head-major ([N, T]) and outputs inside a wider [T, N, 2D] buffer."""
    T, N, D = 50, 8, 64
    po, pl, so, sl = MI.random_attn_states(T, N, D, seed=140)
    big_p = torch.zeros((T, N, 2 * D), dtype=torch.bfloat16, device="cuda")
    big_s = torch.zeros_like(big_p)
    big_o = torch.full_like(big_p, 7.0)
    big_p[:, :, :D] = dev_bf16(po)
    big_s[:, :, :D] = dev_bf16(so)
    lp = torch.from_numpy(np.ascontiguousarray(pl.T)).cuda().t()     # [T, N] view of [N, T] storage
    ls = torch.from_numpy(np.ascontiguousarray(sl.T)).cuda().t()
    lo = torch.empty((N, T), dtype=torch.float32, device="cuda").t()
    o, l = M.merge_attn_states(big_p[:, :, :D], lp, big_s[:, :, :D], ls, out=big_o[:, :, :D], out_lse=lo)
    torch.cuda.synchronize()
    assert torch.all(big_o[:, :, D:] == 7.0)                         # nothing written outside the view
    _check_merge(host_bits(o), l.cpu().numpy(), po, pl, so, sl, "strided")


@pytest.mark.parametrize("N", [16, 128])
def test_merge_of_two_decodes_over_a_split_context_equals_one_decode(N):
    """Decode over the first k pages and over the rest, then merge: the same as one
    decode over all tokens (q_len 1: every token visible)."""
    w = MI.make_workload("split", 3, 1, N, [700, 130, 2049], None, MI.KV_BF16, False, 150)
    pool = gpu_pool(w)
    o_all, l_all = gpu_decode(w, pool, w.q, 0)
    k = np.array([5, 1, 16])                                         # pages in the prefix part
    pre_seq = np.minimum(w.seq_lens, 64 * k).astype(np.int32)
    suf_seq = (w.seq_lens - pre_seq).astype(np.int32)
    bt_suf = np.full_like(w.block_table, -1)
    for b in range(w.B):
        rest = w.block_table[b, k[b]:]
        bt_suf[b, :len(rest)] = rest
    o_p, l_p = gpu_decode(w, pool, w.q, 0, seq_lens=pre_seq)
    o_s, l_s = gpu_decode(w, pool, w.q, 0, seq_lens=suf_seq, block_table=bt_suf)
    T = w.B * w.q_len
    o_m, l_m = M.merge_attn_states(o_p.view(T, N, 512), l_p.view(T, N), o_s.view(T, N, 512), l_s.view(T, N))
    torch.cuda.synchronize()
    # the merge itself, against the oracle's merge of the same two bf16 states
    _check_merge(host_bits(o_m), l_m.cpu().numpy(), host_bits(o_p.view(T, N, 512)), l_p.view(T, N).cpu().numpy(),
                 host_bits(o_s.view(T, N, 512)), l_s.view(T, N).cpu().numpy(), f"split N{N}")
    # end to end, against one oracle decode over all tokens: the decode gate plus the
    # bf16 rounding the two partial outputs already carry (half an ulp of each)
    o_ref, l_ref = O.decode(O.bf16_bits_to_f64(w.q), oracle_pool(w), w.kv_dtype, w.block_table,
                            w.seq_lens, O.default_scale())
    o = to_f64(o_m).reshape(o_ref.shape)
    carried = bf16_half_ulp(np.abs(to_f64(o_p))) + bf16_half_ulp(np.abs(to_f64(o_s))) + \
        bf16_half_ulp(np.maximum(np.abs(o), np.abs(o_ref)))
    for b in range(w.B):
        rms = math.sqrt(float(np.mean(o_ref[b] ** 2)))
        excess = float(np.max(np.abs(o[b] - o_ref[b]) - carried[b]))
        say(f"  [split merge N{N}] request {b}: error beyond the carried roundings = {excess / rms:.3e} x rms")
        assert excess <= 2e-2 * rms
    check_lse(l_m.cpu().numpy().reshape(l_ref.shape), l_ref, f"split merge N{N}")
    check_out(to_f64(o_all), o_ref, f"one decode N{N}")

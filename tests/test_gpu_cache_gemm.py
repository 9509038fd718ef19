"""GPU parity: mla_cache_write (bit-exact against the oracle) and the two per-head
contractions mla_absorb_q / mla_up_v (element-wise rounding bound)."""

import numpy as np
import pytest
import torch

import mla_inputs as MI
import mla_paged_latent_amd as M
from oracle import mla_oracle as O
from tests.mla_testlib import dev_bf16, host_bits, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kd", [MI.KV_BF16, MI.KV_FP8])
def test_cache_write_bit_exact_with_guard_bands(kd):
    say(f"cache_write kd={kd}")
    rng = np.random.default_rng(30 + kd)
    T, pages = 300, 12
    rb = M.ROW_BYTES[kd]
    scale = rng.choice([1e-3, 1.0, 37.0, 3e4], size=(T, 1))
    rows = MI.to_bf16_bits((rng.standard_normal((T, 576)) * scale).astype(np.float32))
    rows[7] = 0                                            # all-zero row: scale 1
    rows[8, :] = MI.to_bf16_bits(np.full(576, -2.5, np.float32))
    slots = rng.permutation(pages * 64)[:T].astype(np.int64)
    slots[::17] = -1                                       # padding tokens are skipped
    guard = rng.integers(0, 256, size=(pages + 2, 64, rb), dtype=np.uint8)
    ref = O.cache_write(guard[1:-1], rows[:, :512], rows[:, 512:], slots, kd)
    buf = torch.from_numpy(guard.copy()).cuda()
    pool = buf[1:-1]
    # strided sources: kv_c and k_pe are views into one [T, 576 + 8] buffer
    src = torch.zeros((T, 584), dtype=torch.bfloat16, device="cuda")
    src[:, :576] = dev_bf16(rows)
    M.cache_write(src[:, :512], src[:, 512:576], torch.from_numpy(slots).cuda(), pool, kd)
    got = buf.cpu().numpy()
    assert np.array_equal(got[0], guard[0]) and np.array_equal(got[-1], guard[-1]), "guard page touched"
    assert np.array_equal(got[1:-1], ref)


def test_fp8_encode_covers_every_code_and_tie():
    """Rows built so that x / s hits every e4m3fn value, every midpoint and both
    neighbours of every midpoint: the GPU's rounding must match the oracle bit for bit."""
    say("fp8 encode exhaustive")
    pos = O.e4m3_value(np.arange(0, 127))
    mids = (pos[:-1] + pos[1:]) / 2
    targets = np.concatenate([pos, mids, -pos, -mids])
    # with amax fixed at 448 (s = 1) the quantizer sees the bf16 value itself; keep
    # only targets exactly representable in bf16 so the tie really is a tie
    t32 = targets.astype(np.float32)
    bits = MI.to_bf16_bits(t32)
    keep = O.bf16_bits_to_f64(bits) == targets
    vals = bits[keep]
    n_rows = (len(vals) + 574) // 575
    rows = np.zeros((n_rows, 576), np.uint16)
    flat = np.zeros(n_rows * 575, np.uint16)
    flat[:len(vals)] = vals
    rows[:, :575] = flat.reshape(n_rows, 575)
    rows[:, 575] = MI.to_bf16_bits(np.float32([448.0]))[0]      # amax 448 -> s = 1
    # plus rows at other scales, which exercise the float32 division
    rng = np.random.default_rng(31)
    extra = MI.to_bf16_bits((rng.standard_normal((256, 576)) * rng.uniform(1e-4, 1e4, (256, 1))).astype(np.float32))
    rows = np.concatenate([rows, extra])
    n = rows.shape[0]
    ref = O.encode_rows(rows, O.KV_FP8)
    pool = torch.zeros(((n + 63) // 64, 64, 584), dtype=torch.uint8, device="cuda")
    r = dev_bf16(rows)
    M.cache_write(r[:, :512], r[:, 512:], torch.arange(n, dtype=torch.int64, device="cuda"), pool, M.KV_FP8)
    got = pool.cpu().numpy().reshape(-1, 584)[:n]
    assert np.array_equal(got, ref)


def _gemm_bound(a, w, ref):
    """|gpu - ref| <= 2^-8 |ref| (bf16 rounding of the result) + K 2^-24 sum|a w|
    (float32 accumulation in any order) -- a rigorous bound for bf16 products."""
    K = a.shape[-1]
    absum = np.einsum("thk,hkn->thn", np.abs(a), np.abs(w))
    return 2.0 ** -8 * np.abs(ref) + 1.01 * K * 2.0 ** -24 * absum + 1e-30


@pytest.mark.parametrize("T,N", [(2, 16), (32, 128), (1, 3), (33, 40), (100, 128)])
def test_absorb_q(T, N):
    say(f"absorb_q T={T} N={N}")
    rng = np.random.default_rng(40 + T + N)
    qn = MI.to_bf16_bits(rng.standard_normal((T, N, 128)).astype(np.float32))
    qp = MI.to_bf16_bits(rng.standard_normal((T, N, 64)).astype(np.float32))
    w = MI.to_bf16_bits((rng.standard_normal((N, 128, 512)) / np.sqrt(512)).astype(np.float32))
    got = M.absorb_q(dev_bf16(qn), dev_bf16(qp), dev_bf16(w))
    torch.cuda.synchronize()
    gb = host_bits(got)
    a, ww = O.bf16_bits_to_f64(qn), O.bf16_bits_to_f64(w)
    ref = O.absorb(a, O.bf16_bits_to_f64(qp), ww)
    g = O.bf16_bits_to_f64(gb)
    bound = _gemm_bound(a, ww, ref[..., :512])
    assert np.all(np.abs(g[..., :512] - ref[..., :512]) <= bound)
    assert np.array_equal(gb[..., 512:], qp)                 # q_pe copied bit for bit


def test_absorb_q_strided_views_without_pe():
    """q_nope taken as a view of a [T, N, 192] query; output rows 512 wide."""
    say("absorb_q strided")
    rng = np.random.default_rng(45)
    T, N = 17, 24
    q = MI.to_bf16_bits(rng.standard_normal((T, N, 192)).astype(np.float32))
    w = MI.to_bf16_bits((rng.standard_normal((N, 128, 512)) / np.sqrt(512)).astype(np.float32))
    qd = dev_bf16(q)
    out = torch.full((T, N, 520), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.absorb_q(qd[..., :128], None, dev_bf16(w), q_fused=out[..., :512])
    torch.cuda.synchronize()
    ref = O.absorb(O.bf16_bits_to_f64(q[..., :128]), None, O.bf16_bits_to_f64(w))
    g = O.bf16_bits_to_f64(host_bits(out))
    assert np.all(np.abs(g[..., :512] - ref) <= _gemm_bound(O.bf16_bits_to_f64(q[..., :128]), O.bf16_bits_to_f64(w), ref))
    assert np.all(np.isnan(g[..., 512:]))                     # untouched padding


@pytest.mark.parametrize("T,N", [(2, 16), (32, 128), (1, 5), (77, 128), (127, 16), (128, 16), (256, 16), (300, 24), (700, 16), (513, 40)])
def test_up_v(T, N):
    say(f"up_v T={T} N={N}")
    rng = np.random.default_rng(50 + T + N)
    ol = MI.to_bf16_bits(rng.standard_normal((T, N, 512)).astype(np.float32))
    w = MI.to_bf16_bits((rng.standard_normal((N, 512, 128)) / np.sqrt(512)).astype(np.float32))
    got = M.up_v(dev_bf16(ol), dev_bf16(w))
    torch.cuda.synchronize()
    a, ww = O.bf16_bits_to_f64(ol), O.bf16_bits_to_f64(w)
    ref = O.up_v(a, ww)
    g = O.bf16_bits_to_f64(host_bits(got)).reshape(T, N, 128)
    assert np.all(np.abs(g - ref) <= _gemm_bound(a, ww, ref))


@pytest.mark.parametrize("kd", [MI.KV_BF16, MI.KV_FP8])
@pytest.mark.parametrize("T,N,T_new,with_pe", [(32, 128, 32, True), (3, 16, 70, False), (1, 128, 5, True),
                                               (0, 16, 9, True)])
def test_absorb_q_cache_write_equals_the_two_calls(kd, T, N, T_new, with_pe):
    """The single launch writes exactly what mla_absorb_q and mla_cache_write write:
    q_fused and the whole pool (guard pages included) compared byte for byte, with
    padding and out-of-range slots among the new rows."""
    say(f"absorb_q_cache_write kd={kd} T={T} N={N} T_new={T_new} pe={with_pe}")
    rng = np.random.default_rng(90 + 7 * kd + T + N)
    pages = 8
    rb = M.ROW_BYTES[kd]
    q_nope = dev_bf16(MI.to_bf16_bits(rng.standard_normal((T, N, 128)).astype(np.float32)))
    q_pe = dev_bf16(MI.to_bf16_bits(rng.standard_normal((T, N, 64)).astype(np.float32))) if with_pe else None
    w = dev_bf16(MI.to_bf16_bits((rng.standard_normal((N, 128, 512)) / 22.6).astype(np.float32)))
    rows = dev_bf16(MI.to_bf16_bits(rng.standard_normal((T_new, 576)).astype(np.float32)))
    slots = rng.permutation(pages * 64)[:T_new].astype(np.int64)
    slots[::4] = -1
    if T_new > 2:
        slots[2] = pages * 64 + 5                         # out of range: skipped
    slots_d = torch.from_numpy(slots).cuda()
    guard = torch.from_numpy(rng.integers(0, 256, size=(pages + 2, 64, rb), dtype=np.uint8)).cuda()
    buf_a, buf_b = guard.clone(), guard.clone()
    width = 576 if with_pe else 512
    qf_a = torch.full((T, N, width), 7.0, dtype=torch.bfloat16, device="cuda")
    qf_b = qf_a.clone()
    M.absorb_q(q_nope, q_pe, w, q_fused=qf_a)
    M.cache_write(rows[:, :512], rows[:, 512:], slots_d, buf_a[1:-1], kd)
    M.absorb_q_cache_write(q_nope, q_pe, w, rows[:, :512], rows[:, 512:], slots_d, buf_b[1:-1], kd, q_fused=qf_b)
    torch.cuda.synchronize()
    assert torch.equal(qf_a.view(torch.int16), qf_b.view(torch.int16))
    assert torch.equal(buf_a, buf_b)

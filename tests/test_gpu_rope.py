"""GPU parity of mla_absorb_q_rope: the absorbed query with the rotary embedding of
its rope part applied on the way into the tail, both pairings, against the oracle's
absorb_rope (element-wise rounding bound), with out-of-range positions, token counts
past one pass of the workgroup, and strided views."""
import numpy as np
import pytest
import torch

import mla_inputs as MI
import mla_paged_latent_amd as M
from oracle import mla_oracle as O
from tests.mla_testlib import dev_bf16, host_bits, say

pytestmark = pytest.mark.gpu

MAX_POS = 4096


def _gemm_bound(a, w, ref):
    K = a.shape[-1]
    absum = np.einsum("thk,hkn->thn", np.abs(a), np.abs(w))
    return 2.0 ** -8 * np.abs(ref) + 1.01 * K * 2.0 ** -24 * absum + 1e-30


def _rope_magnitude(x, positions, table, neox):
    """|a cos| + |b sin| per output value: the scale of the float32 rounding."""
    T, N, _ = x.shape
    mag = np.zeros_like(x)
    for t in range(T):
        p = positions[t]
        if p < 0 or p >= table.shape[0]:
            continue
        c, s = np.abs(table[p, :32]), np.abs(table[p, 32:])
        if neox:
            a, b = np.abs(x[t, :, :32]), np.abs(x[t, :, 32:])
            mag[t, :, :32], mag[t, :, 32:] = a * c + b * s, b * c + a * s
        else:
            a, b = np.abs(x[t, :, 0::2]), np.abs(x[t, :, 1::2])
            mag[t, :, 0::2], mag[t, :, 1::2] = a * c + b * s, b * c + a * s
    return mag


def _case(T, N, seed, bad=()):
    rng = np.random.default_rng(seed)
    qn = MI.to_bf16_bits(rng.standard_normal((T, N, 128)).astype(np.float32))
    qp = MI.to_bf16_bits(rng.standard_normal((T, N, 64)).astype(np.float32))
    w = MI.to_bf16_bits((rng.standard_normal((N, 128, 512)) / np.sqrt(512)).astype(np.float32))
    pos = rng.integers(0, MAX_POS, T).astype(np.int64)
    for i, p in bad:
        pos[i] = p
    return qn, qp, w, pos


def _check(got_bits, qn, qp, w, pos, table, neox):
    a, ww = O.bf16_bits_to_f64(qn), O.bf16_bits_to_f64(w)
    tab = table.astype(np.float64)
    ref = O.absorb_rope(a, O.bf16_bits_to_f64(qp), ww, pos, tab, neox)
    g = O.bf16_bits_to_f64(got_bits)
    assert np.all(np.abs(g[..., :512] - ref[..., :512]) <= _gemm_bound(a, ww, ref[..., :512]))
    bad = (pos < 0) | (pos >= table.shape[0])
    assert np.all(np.isnan(g[bad, :, 512:]))
    ok = ~bad
    mag = _rope_magnitude(O.bf16_bits_to_f64(qp), pos, tab, neox)
    tail_g, tail_r = g[ok, :, 512:], ref[ok, :, 512:]
    assert np.all(np.abs(tail_g - tail_r) <= 2.0 ** -8 * np.abs(tail_r) + 2.0 ** -22 * mag[ok] + 1e-30)


@pytest.mark.parametrize("T,N,neox", [(2, 16, True), (33, 128, False), (1, 5, True), (300, 40, False),
                                      (100, 128, True), (65, 3, False)])
def test_absorb_q_rope(T, N, neox):
    say(f"absorb_q_rope T={T} N={N} neox={neox}")
    bad = [(0, -1), (T - 1, MAX_POS)] if T > 2 else []
    qn, qp, w, pos = _case(T, N, 1300 + T + N + neox, bad)
    table = MI.rope_cos_sin(MAX_POS)
    got = M.absorb_q_rope(dev_bf16(qn), dev_bf16(qp), dev_bf16(w), torch.from_numpy(pos).cuda(),
                          torch.from_numpy(table).cuda(), neox)
    torch.cuda.synchronize()
    _check(host_bits(got), qn, qp, w, pos, table, neox)


def test_absorb_q_rope_strided_query_and_huge_positions():
    """q_nope and q_pe as views of one [T, N, 192] query; positions far outside the table."""
    say("absorb_q_rope strided")
    rng = np.random.default_rng(1350)
    T, N = 40, 24
    q = MI.to_bf16_bits(rng.standard_normal((T, N, 192)).astype(np.float32))
    w = MI.to_bf16_bits((rng.standard_normal((N, 128, 512)) / np.sqrt(512)).astype(np.float32))
    pos = rng.integers(0, MAX_POS, T).astype(np.int64)
    pos[3], pos[17] = 2 ** 40, -(2 ** 40)
    table = MI.rope_cos_sin(MAX_POS)
    qd = dev_bf16(q)
    out = torch.full((T, N, 584), float("nan"), dtype=torch.bfloat16, device="cuda")
    for neox in (True, False):
        M.absorb_q_rope(qd[..., :128], qd[..., 128:], dev_bf16(w), torch.from_numpy(pos).cuda(),
                        torch.from_numpy(table).cuda(), neox, q_fused=out[..., :576])
        torch.cuda.synchronize()
        _check(host_bits(out[..., :576]), q[..., :128], q[..., 128:], w, pos, table, neox)
        assert torch.isnan(out[..., 576:].float()).all()                  # untouched padding


def test_absorb_q_rope_at_position_zero_is_the_copying_absorb():
    """cos 1, sin 0 leaves every value as it is: the same bits as mla_absorb_q."""
    say("absorb_q_rope identity")
    qn, qp, w, _ = _case(50, 16, 1360)
    table = torch.from_numpy(MI.rope_cos_sin(8)).cuda()
    pos = torch.zeros(50, dtype=torch.int64, device="cuda")
    a, b, c = dev_bf16(qn), dev_bf16(qp), dev_bf16(w)
    ref = M.absorb_q(a, b, c)
    for neox in (True, False):
        got = M.absorb_q_rope(a, b, c, pos, table, neox)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(got), host_bits(ref))

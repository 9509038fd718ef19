"""GPU parity of mla_up_v_fp8: the V up-projection with its output quantized to fp8
per token group of 64 or 128 values, one float32 scale per group.

Two kinds of case.  With selection weights (one power-of-two entry per output
column, every other entry zero) the bf16 product is exact, so the expected codes
and scales are the oracle's quantizer applied to values computed from the inputs
alone, and the check is bit for bit; the chosen values put many groups on exact
e4m3 ties, in the subnormal range, on saturation and on all-zero groups.  With
random weights the dequantized output is held to a bound built from the float32
accumulation, the bf16 rounding and the e4m3 step.
"""
import numpy as np
import pytest
import torch

import mla_inputs as MI
import mla_paged_latent_amd as M
from oracle import mla_oracle as O
from tests.mla_testlib import dev_bf16, host_bits, say

pytestmark = pytest.mark.gpu


def _designed_outputs(rng, T, N, group):
    """bf16 values [T, N*128] whose groups exercise the quantizer's cases."""
    y = (rng.standard_normal((T, N * 128)) * 10.0 ** rng.uniform(-3, 3, (T, 1))).astype(np.float32)
    y = y.reshape(T, -1, group)
    G = y.shape[1]
    kind = rng.integers(0, 5, (T, G))
    codes_normal = np.array([c for c in range(0x08, 0x7e) if (c & 7) != 7], np.int64)
    for t in range(T):
        for g in range(G):
            j = float(2.0 ** rng.integers(-12, 12))
            sign = rng.choice([-1.0, 1.0], group)
            if kind[t, g] == 1:                      # exact ties: s = 2^j, midpoints of codes
                c = rng.choice(codes_normal, group)
                mid = (O.e4m3_value(c) + O.e4m3_value(c + 1)) / 2
                y[t, g] = (sign * mid * j).astype(np.float32)
                y[t, g, rng.integers(group)] = 448.0 * j * rng.choice([-1.0, 1.0])
            elif kind[t, g] == 2:                    # subnormal codes and their ties
                k = rng.integers(0, 16, group)
                y[t, g] = (sign * k * 2.0 ** -10 * j).astype(np.float32)
                y[t, g, rng.integers(group)] = 448.0 * j
            elif kind[t, g] == 3:                    # all-zero group: scale 1, codes 0
                y[t, g] = 0.0
            # kind 0 and 4: random values at the token's scale
    bits = MI.to_bf16_bits(y.reshape(T, N * 128))
    bits[bits == 0x8000] = 0                         # a sum of products never returns -0
    return bits


def _selection_case(rng, T, N, group):
    """o_lat and W_UV whose up-projection is exactly the designed values."""
    y_bits = _designed_outputs(rng, T, N, group)
    y = O.bf16_bits_to_f64(y_bits).reshape(T, N, 128)
    ol = rng.standard_normal((T, N, 512))
    w = np.zeros((N, 512, 128))
    for h in range(N):
        perm = rng.choice(512, 128, replace=False)
        e = rng.integers(-2, 3, 128)
        w[h, perm, np.arange(128)] = 2.0 ** e
        ol[:, h, perm] = y[:, h, :] * 2.0 ** -e    # exact: power-of-two scaling of bf16 values
    ol_bits = O.f64_to_bf16_bits(ol)
    w_bits = O.f64_to_bf16_bits(w)
    return ol_bits, w_bits, y_bits


@pytest.mark.parametrize("T,N,group", [(1, 16, 128), (33, 16, 64), (64, 128, 128), (77, 5, 64),
                                       (100, 128, 64), (3, 40, 128), (600, 16, 128), (517, 7, 128),
                                       (600, 16, 64), (191, 8, 128), (192, 8, 128), (301, 9, 128),
                                       (1030, 8, 128)])
def test_up_v_fp8_bit_exact_on_exact_products(T, N, group):
    say(f"up_v_fp8 selection T={T} N={N} group={group}")
    rng = np.random.default_rng(900 + T * 7 + N + group)
    ol, w, y_bits = _selection_case(rng, T, N, group)
    # the product really is exact: every output column has one nonzero term
    ref_y = O.up_v(O.bf16_bits_to_f64(ol), O.bf16_bits_to_f64(w)).reshape(T, N * 128)
    assert np.array_equal(O.f64_to_bf16_bits(ref_y), y_bits)
    ref_codes, ref_scales = O.quantize_groups_fp8(y_bits, group)
    codes, scales = M.up_v_fp8(dev_bf16(ol), dev_bf16(w), group)
    torch.cuda.synchronize()
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    assert np.array_equal(got_s.view(np.uint32), ref_scales.view(np.uint32))
    assert np.array_equal(got_c, ref_codes)


def test_up_v_fp8_ties_are_present():
    """The designed inputs do reach the tie and subnormal paths of the quantizer."""
    rng = np.random.default_rng(900 + 64 * 7 + 128 + 128)
    _, _, y_bits = _selection_case(rng, 64, 128, 128)
    y = O.bf16_bits_to_f64(y_bits).reshape(64, -1, 128)
    _, s = O.quantize_groups_fp8(y_bits, 128)
    q = y / s[:, :, None].astype(np.float64)
    frac_ties = np.mean(np.isin(q, (O.e4m3_value(np.arange(0x7e)) + O.e4m3_value(np.arange(1, 0x7f))) / 2))
    assert frac_ties > 0.1
    assert np.any((np.abs(q) < 2.0 ** -6) & (q != 0))


def _deq(codes, scales, group):
    T, C = codes.shape
    v = O.e4m3_value(codes.astype(np.int64)).reshape(T, C // group, group)
    return (v * scales.astype(np.float64)[:, :, None]).reshape(T, C)


@pytest.mark.parametrize("T,N,group", [(2, 16, 128), (32, 128, 64), (45, 128, 128), (7, 3, 64), (700, 16, 128), (270, 16, 128),
                                       (1100, 8, 128)])
def test_up_v_fp8_random_weights_within_bound(T, N, group):
    say(f"up_v_fp8 random T={T} N={N} group={group}")
    rng = np.random.default_rng(950 + T + N + group)
    ol = MI.to_bf16_bits(rng.standard_normal((T, N, 512)).astype(np.float32))
    w = MI.to_bf16_bits((rng.standard_normal((N, 512, 128)) / np.sqrt(512)).astype(np.float32))
    a, ww = O.bf16_bits_to_f64(ol), O.bf16_bits_to_f64(w)
    ref = O.up_v(a, ww)                                            # [T, N, 128] float64
    # |y_bf16 - ref| <= 2^-8 |ref| + K 2^-24 sum|a w| (float32 accumulation, one rounding)
    B = 2.0 ** -8 * np.abs(ref) + 1.01 * 512 * 2.0 ** -24 * np.einsum("thk,hkn->thn", np.abs(a), np.abs(ww))
    ref, B = ref.reshape(T, -1), B.reshape(T, -1)
    codes, scales = M.up_v_fp8(dev_bf16(ol), dev_bf16(w), group)
    torch.cuda.synchronize()
    c, s = codes.cpu().numpy(), scales.cpu().numpy().astype(np.float64)
    G = N * 128 // group
    amax = np.abs(ref).reshape(T, G, group).max(axis=2)
    bmax = B.reshape(T, G, group).max(axis=2)
    assert np.all(np.abs(s - amax / 448.0) <= bmax / 448.0 + 2.0 ** -23 * s)
    srep = np.repeat(s, group, axis=1)
    err = np.abs(_deq(c, s.astype(np.float32), group) - ref)
    # e4m3 half step: 2^-4 relative in the normal range, 2^-10 s below it
    assert np.all(err <= B + 2.0 ** -4 * (np.abs(ref) + B) * (1 + 2.0 ** -20) + 2.0 ** -10 * srep)
    assert np.all(c != 0x7f) and np.all(c != 0xff)                 # never a NaN code


def test_up_v_fp8_strided_outputs_and_empty_call():
    """Padded output rows keep their padding; T = 0 writes nothing."""
    say("up_v_fp8 strided")
    rng = np.random.default_rng(990)
    T, N, group = 9, 24, 64
    ol_full = MI.to_bf16_bits(rng.standard_normal((T, N, 600)).astype(np.float32))
    w = MI.to_bf16_bits((rng.standard_normal((N, 512, 128)) / np.sqrt(512)).astype(np.float32))
    old = dev_bf16(ol_full)[..., :512]
    wd = dev_bf16(w)
    codes = torch.full((T, N * 128 + 24), 0x7f, dtype=torch.uint8, device="cuda")
    scales = torch.full((T, N * 128 // group + 3), -1.0, dtype=torch.float32, device="cuda")
    M.up_v_fp8(old, wd, group, out_codes=codes[:, :N * 128], out_scales=scales[:, :N * 128 // group])
    c_ref, s_ref = M.up_v_fp8(old.contiguous(), wd, group)
    torch.cuda.synchronize()
    assert torch.equal(codes[:, :N * 128], c_ref) and torch.equal(scales[:, :N * 128 // group], s_ref)
    assert bool((codes[:, N * 128:] == 0x7f).all()) and bool((scales[:, N * 128 // group:] == -1).all())
    e_c = torch.full((0, N * 128), 1, dtype=torch.uint8, device="cuda")
    e_s = torch.full((0, N * 2), 1.0, dtype=torch.float32, device="cuda")
    M.up_v_fp8(old[:0], wd, group, out_codes=e_c, out_scales=e_s)
    torch.cuda.synchronize()

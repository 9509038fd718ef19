"""GPU parity of the large-token path of the per-head up-projections (mla_up_v from 128
tokens, mla_up_v_fp8 with groups of 128 from 192, mla_kv_b_proj from 128 rows), where a
workgroup keeps one head's weights for 128 output columns in registers and streams the
token rows; one or two such workgroups per CU depending on the call and its size.

Ragged and strided cases are checked in full against the oracle; the prefill sizes
(8192 rows, 128 heads, as bench.py times them) on sampled rows, the oracle computing
each sampled row from the same device inputs copied back to the host.

Bounds ([vLLM-MLA] §两套算法 and §Prefill: the up-projections are plain per-head
products): a bf16 result of K = 512 products accumulated in float32 and rounded once
is within 2^-8 |ref| + 1.01 K 2^-24 sum|a w| of the exact value; fp8 codes add half
an e4m3 step (2^-4 relative in the normal range, 2^-10 of the scale below it) on top
of that, and the group scale is amax / 448 of the bf16 values.
"""
import numpy as np
import pytest
import torch

import mla_inputs as MI
import mla_paged_latent_amd as M
from oracle import mla_oracle as O
from tests.mla_testlib import dev_bf16, host_bits, say

pytestmark = pytest.mark.gpu

F = O.bf16_bits_to_f64


def _bound(a, w, ref, spec):
    absum = np.einsum(spec, np.abs(a), np.abs(w))
    return 2.0 ** -8 * np.abs(ref) + 1.01 * 512 * 2.0 ** -24 * absum + 1e-30


def _check_fp8(codes, scales, ref, B, group):
    """codes uint8 [T, C], scales [T, C / group] against the exact product ref [T, C]
    with its bf16 + accumulation bound B."""
    T, C = ref.shape
    s = scales.astype(np.float64)
    G = C // group
    amax = np.abs(ref).reshape(T, G, group).max(axis=2)
    bmax = B.reshape(T, G, group).max(axis=2)
    assert np.all(np.abs(s - amax / 448.0) <= bmax / 448.0 + 2.0 ** -23 * s)
    srep = np.repeat(s, group, axis=1)
    deq = O.e4m3_value(codes.astype(np.int64)) * srep
    err = np.abs(deq - ref)
    assert np.all(err <= B + 2.0 ** -4 * (np.abs(ref) + B) * (1 + 2.0 ** -20) + 2.0 ** -10 * srep)
    assert np.all(codes != 0x7f) and np.all(codes != 0xff)


def _rand_bf16(rng, shape, scale=1.0):
    return MI.to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def test_up_v_large_t_strided_views():
    """Activations as a view with a padded head stride, output rows with padding."""
    say("up_v large T strided")
    rng = np.random.default_rng(1201)
    T, N = 600, 8
    ol = _rand_bf16(rng, (T, N, 520))
    w = _rand_bf16(rng, (N, 512, 128), 1 / np.sqrt(512))
    old = dev_bf16(ol)[..., :512]
    out = torch.full((T, N * 128 + 40), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.up_v(old, dev_bf16(w), out=out[:, :N * 128])
    torch.cuda.synchronize()
    a, ww = F(ol[..., :512]), F(w)
    ref = O.up_v(a, ww)
    g = F(host_bits(out))
    assert np.all(np.abs(g[:, :N * 128].reshape(T, N, 128) - ref) <= _bound(a, ww, ref, "thk,hkn->thn"))
    assert np.all(np.isnan(g[:, N * 128:]))


@pytest.mark.parametrize("S,N", [(600, 16), (513, 5), (512, 1), (511, 8), (130, 8), (128, 3), (127, 4)])
def test_kv_b_proj_large_s(S, N):
    """Latent rows taken from [S, 576] cache rows, output with a padded head stride."""
    say(f"kv_b_proj large S={S} N={N}")
    rng = np.random.default_rng(1210 + S + N)
    rows = _rand_bf16(rng, (S, 576))
    w = _rand_bf16(rng, (N, 512, 256), 1 / np.sqrt(512))
    out = torch.full((S, N, 264), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.kv_b_proj(dev_bf16(rows)[:, :512], dev_bf16(w), out=out[..., :256])
    torch.cuda.synchronize()
    kc, ww = F(rows[:, :512]), F(w)
    kn, v = O.kv_b_proj(kc, ww)
    ref = np.concatenate([kn, v], axis=-1)
    g = F(host_bits(out))
    assert np.all(np.abs(g[..., :256] - ref) <= _bound(kc, ww, ref, "sl,hlc->shc"))
    assert np.all(np.isnan(g[..., 256:]))


def _sample_rows(T, rng, n=20):
    fixed = [0, 1, 127, 128, T // 2, T - 129, T - 128, T - 1]
    return np.unique(np.concatenate([fixed, rng.integers(0, T, n)]))


def _device_inputs(seed, a_shape, w_shape):
    gen = torch.Generator(device="cuda").manual_seed(seed)
    a = torch.randn(*a_shape, device="cuda", generator=gen).to(torch.bfloat16)
    w = (torch.randn(*w_shape, device="cuda", generator=gen) / np.sqrt(512)).to(torch.bfloat16)
    return a, w


def test_up_v_prefill_size_sampled_rows():
    """T = 8192 tokens x 128 heads, bf16 output and fp8 output (groups of 128)."""
    say("up_v / up_v_fp8 T=8192 N=128 sampled")
    T, N = 8192, 128
    ol, w = _device_inputs(1220, (T, N, 512), (N, 512, 128))
    y = M.up_v(ol, w)
    codes, scales = M.up_v_fp8(ol, w, 128)
    torch.cuda.synchronize()
    rows = _sample_rows(T, np.random.default_rng(1221))
    idx = torch.from_numpy(rows).cuda()
    a, ww = F(host_bits(ol.index_select(0, idx))), F(host_bits(w))
    ref = O.up_v(a, ww)
    B = _bound(a, ww, ref, "thk,hkn->thn")
    g = F(host_bits(y.index_select(0, idx))).reshape(len(rows), N, 128)
    assert np.all(np.abs(g - ref) <= B)
    _check_fp8(codes.index_select(0, idx).cpu().numpy(), scales.index_select(0, idx).cpu().numpy(),
               ref.reshape(len(rows), -1), B.reshape(len(rows), -1), 128)


def test_kv_b_proj_prefill_size_sampled_rows():
    """S = 8192 latent rows (the first 512 of [S, 576] rows) x 128 heads."""
    say("kv_b_proj S=8192 N=128 sampled")
    S, N = 8192, 128
    rows_all, w = _device_inputs(1230, (S, 576), (N, 512, 256))
    out = M.kv_b_proj(rows_all[:, :512], w)
    torch.cuda.synchronize()
    rows = _sample_rows(S, np.random.default_rng(1231))
    idx = torch.from_numpy(rows).cuda()
    kc, ww = F(host_bits(rows_all.index_select(0, idx)[:, :512])), F(host_bits(w))
    kn, v = O.kv_b_proj(kc, ww)
    ref = np.concatenate([kn, v], axis=-1)
    g = F(host_bits(out.index_select(0, idx)))
    assert np.all(np.abs(g - ref) <= _bound(kc, ww, ref, "sl,hlc->shc"))

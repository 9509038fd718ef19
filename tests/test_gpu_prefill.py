"""GPU parity of the prefill of new tokens: mla_kv_b_proj (latents -> per-head keys and
values) and mla_prefill_mha (192/128 attention over ragged causal requests) against the
oracle's kv_b_proj and prefill_mha, per request, with the decode tests' output gate."""
import numpy as np
import pytest
import torch

import mla_inputs as MI
import mla_paged_latent_amd as M
from oracle import mla_oracle as O
from tests.mla_testlib import check_lse, check_out, dev_bf16, host_bits, say, to_f64

pytestmark = pytest.mark.gpu
SC = O.default_scale()


def _ragged(pairs):
    cu_q = np.concatenate([[0], np.cumsum([p[0] for p in pairs])]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum([p[1] for p in pairs])]).astype(np.int32)
    return cu_q, cu_k


def _bf16(rng, shape, std=1.0):
    return MI.to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))


def _check_requests(out, lse, ref_o, ref_l, cu_q, name):
    for b in range(len(cu_q) - 1):
        a, e = cu_q[b], cu_q[b + 1]
        if e == a:
            continue
        check_out(out[a:e][None], ref_o[a:e][None], f"{name} request {b}")
        check_lse(lse[a:e], ref_l[a:e], f"{name} request {b}")


@pytest.mark.parametrize("N,causal", [(16, True), (3, True), (16, False), (128, True)])
def test_prefill_mha_ragged(N, causal):
    # (query rows, keys): single token, equal lengths across q blocks, context before the
    # new tokens, no queries, more queries than keys (causal rows that see nothing)
    pairs = [(1, 1), (5, 5), (70, 70), (33, 100), (0, 10), (130, 200), (6, 3)]
    if N == 128:
        pairs = [(70, 150), (1, 64), (65, 65)]
    say(f"prefill_mha N={N} causal={causal} requests={pairs}")
    rng = np.random.default_rng(1500 + N + causal)
    cu_q, cu_k = _ragged(pairs)
    T, S = int(cu_q[-1]), int(cu_k[-1])
    q, kn, kp, v = _bf16(rng, (T, N, 192)), _bf16(rng, (S, N, 128)), _bf16(rng, (S, 64)), _bf16(rng, (S, N, 128))
    out, lse = M.prefill_mha(dev_bf16(q), dev_bf16(kn), dev_bf16(kp), dev_bf16(v), torch.from_numpy(cu_q).cuda(),
                             torch.from_numpy(cu_k).cuda(), max(p[0] for p in pairs), causal, SC)
    torch.cuda.synchronize()
    f = O.bf16_bits_to_f64
    ref_o, ref_l = O.prefill_mha(f(q), f(kn), f(kp), f(v), cu_q, cu_k, SC, causal)
    _check_requests(to_f64(out), lse.cpu().numpy(), ref_o, ref_l, cu_q, "prefill")


def test_kv_b_proj_and_prefill_end_to_end():
    """Latents -> mla_kv_b_proj -> mla_prefill_mha on strided views of its output, against
    the oracle's kv_b_proj (checked to its rounding bound) and the oracle's prefill_mha
    over that result rounded to bf16, as the kernel stores it."""
    say("kv_b_proj + prefill_mha")
    rng = np.random.default_rng(1550)
    N = 16
    pairs = [(40, 40), (20, 90)]
    cu_q, cu_k = _ragged(pairs)
    T, S = int(cu_q[-1]), int(cu_k[-1])
    rows = _bf16(rng, (S, 576))
    w = _bf16(rng, (N, 512, 256), 1 / np.sqrt(512))
    q = _bf16(rng, (T, N, 192))
    rd = dev_bf16(rows)
    kvb = M.kv_b_proj(rd[:, :512], dev_bf16(w))
    torch.cuda.synchronize()
    f = O.bf16_bits_to_f64
    kn_ref, v_ref = O.kv_b_proj(f(rows[:, :512]), f(w))
    got = f(host_bits(kvb))
    K = 512
    absum = np.einsum("sl,hlc->shc", np.abs(f(rows[:, :512])), np.abs(f(w)))
    ref = np.concatenate([kn_ref, v_ref], axis=-1)
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1.01 * K * 2.0 ** -24 * absum + 1e-30)
    out, lse = M.prefill_mha(dev_bf16(q), kvb[..., :128], rd[:, 512:], kvb[..., 128:], torch.from_numpy(cu_q).cuda(),
                             torch.from_numpy(cu_k).cuda(), 40, True, SC)
    torch.cuda.synchronize()
    # the GPU attends over its own bf16 keys and values: the oracle's, rounded to bf16 the
    # same way (at most a rare one-ulp difference from accumulation order remains)
    kn_b, v_b = f(O.f64_to_bf16_bits(kn_ref)), f(O.f64_to_bf16_bits(v_ref))
    ref_o, ref_l = O.prefill_mha(f(q), kn_b, f(rows[:, 512:]), v_b, cu_q, cu_k, SC, True)
    _check_requests(to_f64(out), lse.cpu().numpy(), ref_o, ref_l, cu_q, "kv_b_proj+prefill")

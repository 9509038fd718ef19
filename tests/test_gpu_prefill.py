"""GPU parity of the prefill of new tokens: mla_kv_b_proj (latents -> per-head keys and
values) and mla_prefill_mha (192/128 attention over ragged causal requests) against the
oracle's kv_b_proj and prefill_mha, per request, with the decode tests' output gate."""
import numpy as np
import pytest
import torch

import mla_inputs as MI
import mla_paged_latent_amd as M
from oracle import mla_oracle as O
from tests.mla_testlib import bf16_half_ulp, check_lse, check_out, dev_bf16, host_bits, say, to_f64

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


def _chunked_context_prefill(pool, kd, block_table, ctx_lens, new_rows, q, w_kvb, cu_q, W):
    """The chunked-context prefill of new tokens over their requests' cached context: per
    chunk of at most W context rows, gather -> kv_b_proj -> prefill_mha (not causal) ->
    merge into the running state; then the new tokens' causal attention over themselves,
    merged last.  Every step is one library call."""
    T, N = q.shape[0], q.shape[1]
    B = len(ctx_lens)
    dev = "cuda"
    bt = torch.from_numpy(block_table).to(dev)
    cuq = torch.from_numpy(cu_q).to(dev)
    max_q = int(np.max(np.diff(cu_q)))
    o_run = torch.zeros((T, N, 128), dtype=torch.bfloat16, device=dev)
    l_run = torch.full((T, N), -float("inf"), dtype=torch.float32, device=dev)
    starts, lens = M.plan_context_chunks(ctx_lens, W)
    for c in range(starts.shape[0]):
        cu = np.concatenate([[0], np.cumsum(lens[c])]).astype(np.int32)
        t2s = np.repeat(np.arange(B, dtype=np.int32), lens[c])
        rows = M.gather_cache(pool, kd, bt, torch.from_numpy(cu).to(dev), torch.from_numpy(t2s).to(dev),
                              seq_starts=torch.from_numpy(starts[c]).to(dev))
        assert rows.shape[0] <= W
        kvb = M.kv_b_proj(rows[:, :512], w_kvb)
        o_c, l_c = M.prefill_mha(q, kvb[..., :128], rows[:, 512:], kvb[..., 128:], cuq,
                                 torch.from_numpy(cu).to(dev), max_q, False, SC)
        o_run, l_run = M.merge_attn_states(o_run, l_run, o_c, l_c)
    kvb_n = M.kv_b_proj(new_rows[:, :512], w_kvb)
    o_n, l_n = M.prefill_mha(q, kvb_n[..., :128], new_rows[:, 512:], kvb_n[..., 128:], cuq, cuq, max_q, True, SC)
    return M.merge_attn_states(o_run, l_run, o_n, l_n), starts.shape[0]


def _chain_rounding_bound(q, kn, kp, v, key_off, ctx_lens, cu_q, plan):
    """Element bound on what the chain's bf16 stores add to the error: every piece's output
    and every intermediate running merge is stored in bf16 (half an ulp each) and reaches
    the final output scaled by its softmax weight exp(lse_piece - lse_final).  The pieces'
    exact values come from the oracle (float64)."""
    f = O.bf16_bits_to_f64
    T, N = q.shape[0], q.shape[1]
    B = len(ctx_lens)

    def piece(rows_of, causal):
        idx, cu = [], [0]
        for b in range(B):
            r = rows_of(b)
            idx.extend(r)
            cu.append(cu[-1] + len(r))
        idx = np.array(idx, np.int64)
        return O.prefill_mha(q, kn[idx], kp[idx], v[idx], cu_q, np.array(cu, np.int32), SC, causal)

    pieces = []
    for ch in plan:
        spans = {b: range(key_off[b] + s0, key_off[b] + s0 + t) for b, s0, t in ch}
        pieces.append(piece(lambda b: list(spans.get(b, ())), False))
    # the new tokens over themselves (square causal)
    pieces.append(piece(lambda b: list(range(key_off[b] + ctx_lens[b], key_off[b] + ctx_lens[b] + cu_q[b + 1] - cu_q[b])),
                        True))
    run_o, run_l = np.zeros_like(pieces[0][0]), np.full(pieces[0][1].shape, -np.inf)
    stores = []
    for o_c, l_c in pieces:
        stores.append((o_c, l_c))
        run_o, run_l = O.merge_attn_states(run_o, run_l, o_c, l_c)
        stores.append((run_o, run_l))
    stores.pop()                                  # the final output: its own half ulp is in the gate
    bound = np.zeros_like(run_o)
    for o_s, l_s in stores:
        wgt = np.where(np.isneginf(l_s), 0.0, np.exp(np.where(np.isneginf(l_s), 0.0, l_s) -
                                                      np.where(np.isneginf(run_l), 0.0, run_l)))
        bound += wgt[..., None] * bf16_half_ulp(o_s)
    return bound


@pytest.mark.parametrize("N,kd,ctx,new,W", [(16, MI.KV_BF16, [700, 3000, 130], [64, 100, 17], 1024),
                                          (16, MI.KV_FP8, [700, 3000, 130], [64, 100, 17], 1024),
                                          (128, MI.KV_BF16, [300, 900, 0], [20, 33, 5], 512)])
def test_chunked_context_prefill_matches_unchunked_oracle(N, kd, ctx, new, W):
    """A multi-chunk context prefill (row budget W below the batch's context) end to end
    against the oracle's plain prefill over the whole context followed by the new tokens
    (causal, bottom-right aligned): the context keys come from the oracle's gather of the
    same cache (fp8 rows upconverted with their K scale), keys and values from kv_b_proj."""
    from tests.mla_testlib import gpu_pool, oracle_pool
    say(f"chunked context prefill N={N} kd={kd} ctx={ctx} new={new} W={W}")
    rng = np.random.default_rng(1600 + N + kd)
    w = MI.make_workload("ctxpf", len(ctx), 1, N, [max(1, c) for c in ctx], None, kd, False, 1600 + N + kd)
    pool, ref_pool = gpu_pool(w), oracle_pool(w)
    ctx_lens = np.array(ctx, np.int32)
    cu_q = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    T = int(cu_q[-1])
    new_rows = _bf16(rng, (T, 576))
    q = _bf16(rng, (T, N, 192))
    wk = _bf16(rng, (N, 512, 256), 1 / np.sqrt(512))
    (out, lse), n_chunks = _chunked_context_prefill(pool, kd, w.block_table, ctx_lens, dev_bf16(new_rows),
                                                    dev_bf16(q), dev_bf16(wk), cu_q, W)
    torch.cuda.synchronize()
    assert n_chunks >= 2, "the case must take several chunks"
    f = O.bf16_bits_to_f64
    cu_ctx = np.concatenate([[0], np.cumsum(ctx_lens)]).astype(np.int32)
    ctx_bits = O.gather_cache(ref_pool, kd, w.block_table, cu_ctx, np.repeat(np.arange(len(ctx)), ctx_lens))
    lat, key_off, cu_k = [], [], [0]
    for b in range(len(ctx)):
        key_off.append(cu_k[-1])
        lat.append(ctx_bits[cu_ctx[b]:cu_ctx[b + 1]])
        lat.append(new_rows[cu_q[b]:cu_q[b + 1]])
        cu_k.append(cu_k[-1] + int(ctx_lens[b]) + new[b])
    lat = f(np.concatenate(lat))
    # keys and values as kv_b_proj stores them (bf16); the prefill itself in float64
    kn, v = (f(O.f64_to_bf16_bits(x)) for x in O.kv_b_proj(lat[:, :512], f(wk)))
    qf = f(q)
    ref_o, ref_l = O.prefill_mha(qf, kn, lat[:, 512:], v, cu_q, np.array(cu_k, np.int32), SC, True)
    bound = _chain_rounding_bound(qf, kn, lat[:, 512:], v, key_off, ctx_lens, cu_q,
                                  O.plan_context_chunks(ctx_lens.tolist(), W))
    got = to_f64(out)
    for b in range(len(ctx)):
        a, e = cu_q[b], cu_q[b + 1]
        # the chain's own bf16 stores are allowed on top of the single-call gate
        slack = np.where(np.abs(got[a:e] - ref_o[a:e]) > 0, np.minimum(np.abs(got[a:e] - ref_o[a:e]),
                                                                        bound[a:e]), 0.0)
        say(f"  request {b}: chain store bound max {float(np.max(bound[a:e])):.3e}")
        check_out((got[a:e] - np.sign(got[a:e] - ref_o[a:e]) * slack)[None], ref_o[a:e][None],
                  f"chunked prefill request {b}")
        check_lse(lse.cpu().numpy()[a:e], ref_l[a:e], f"chunked prefill request {b}")


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_mha_scores_rising_far_above_the_first_block(causal):
    """A key late in the request whose score exceeds every earlier block's maximum by far
    more than float32 can hold as a probability against a fixed reference (all-positive
    queries against a key of all 16s: a raw score near 16 * sum|q| ~ 2400, some 2^250 above
    the first block's reference): the attention must still equal the oracle's, its softmax
    concentrated on that key for the rows that see it."""
    say(f"prefill_mha rising scores causal={causal}")
    rng = np.random.default_rng(1700 + causal)
    N = 4
    pairs = [(200, 200), (70, 300)]
    cu_q, cu_k = _ragged(pairs)
    T, S = int(cu_q[-1]), int(cu_k[-1])
    q = MI.to_bf16_bits(np.abs(rng.standard_normal((T, N, 192))).astype(np.float32))
    kn, kp, v = _bf16(rng, (S, N, 128)), _bf16(rng, (S, 64)), _bf16(rng, (S, N, 128))
    big = MI.to_bf16_bits(np.full(1, 16.0, np.float32))[0]
    for key in (150, cu_k[1] + 260):                    # request 0: key 150; request 1: key 260
        kn[key] = big
        kp[key] = big
    out, lse = M.prefill_mha(dev_bf16(q), dev_bf16(kn), dev_bf16(kp), dev_bf16(v), torch.from_numpy(cu_q).cuda(),
                             torch.from_numpy(cu_k).cuda(), max(p[0] for p in pairs), causal, SC)
    torch.cuda.synchronize()
    f = O.bf16_bits_to_f64
    ref_o, ref_l = O.prefill_mha(f(q), f(kn), f(kp), f(v), cu_q, cu_k, SC, causal)
    _check_requests(to_f64(out), lse.cpu().numpy(), ref_o, ref_l, cu_q, "prefill rising")


def test_prefill_mha_bench_size_sampled_rows():
    """The benchmarked call: 4 requests x 2048 new tokens, causal, 128 heads, keys and
    values as strided views into one [S, N, 256] kv_b_proj-shaped tensor, seeded normal
    inputs drawn on the device.  Sampled query rows (first, last and interior rows of every
    request, all heads) against the oracle over each row's own visible keys, and the whole
    output and LSE are finite."""
    say("prefill_mha bench size, sampled rows")
    N, L, Bq = 128, 2048, 4
    T = Bq * L
    g = torch.Generator(device="cuda").manual_seed(1800)
    q = torch.randn(T, N, 192, device="cuda", generator=g).to(torch.bfloat16)
    kvb = torch.randn(T, N, 256, device="cuda", generator=g).to(torch.bfloat16)
    kp = torch.randn(T, 64, device="cuda", generator=g).to(torch.bfloat16)
    cu = torch.arange(0, T + 1, L, dtype=torch.int32, device="cuda")
    out, lse = M.prefill_mha(q, kvb[..., :128], kp, kvb[..., 128:], cu, cu, L, True, SC)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out.float()).all()) and bool(torch.isfinite(lse).all())
    f = O.bf16_bits_to_f64
    bits = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    for b, i in ((0, 0), (0, 1), (1, 255), (1, 256), (2, 1000), (2, 2047), (3, 63), (3, 1537)):
        row = b * L + i
        keys = slice(b * L, b * L + i + 1)
        kn_b = f(bits(kvb[keys, :, :128]))
        v_b = f(bits(kvb[keys, :, 128:]))
        ref_o, ref_l = O.prefill_mha(f(bits(q[row:row + 1])), kn_b, f(bits(kp[keys])), v_b,
                                     np.array([0, 1], np.int32), np.array([0, i + 1], np.int32), SC, True)
        check_out(to_f64(out[row:row + 1])[None], ref_o[None], f"bench-size row {b}:{i}")
        check_lse(lse[row:row + 1].cpu().numpy(), ref_l, f"bench-size row {b}:{i}")

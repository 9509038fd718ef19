"""Pins for the CPU oracle: each check ties it to something other than itself.

Printed numbers from the pages (tests/golden), closed forms, invariants that the
method's definition implies, brute force in pure Python loops, and library
routines (torch's float64 SDPA, logsumexp, bfloat16 and float8_e4m3fn codecs).
A plausible slip in the oracle (a dropped rope term, the 576-wide scale, a
transposed weight, a wrong causal offset, a lost scale factor) fails at least
one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import mla_oracle as O
import mla_inputs as MI

GOLD = os.path.join(os.path.dirname(__file__), "golden", "page_arithmetic.json")


# ----------------------------------------------------------------------------
# printed byte arithmetic
# ----------------------------------------------------------------------------
def test_printed_byte_arithmetic():
    g = json.load(open(GOLD))
    bf, f8 = O.row_bytes(O.KV_BF16), O.row_bytes(O.KV_FP8)
    assert bf == g["row_bytes_bf16"] and f8 == g["row_bytes_fp8"]
    mha = O.mha_row_bytes()
    assert mha == g["mha_row_bytes_128h_qk192_v128"]
    assert mha // bf == g["mha_over_mla_ratio_floor"]
    L, S = g["layers"], g["context_tokens"]
    assert bf * L == g["per_token_all_layers_bf16"]
    assert round(bf * L / 1024, 1) == g["per_token_all_layers_bf16_kib"]
    assert round(O.request_bytes(S, L, O.KV_BF16) / 1e9, 2) == g["request_128k_bf16_gb"]
    assert round(O.request_bytes(S, L, O.KV_BF16) / 2**30, 2) == g["request_128k_bf16_gib"]
    assert O.page_bytes(O.KV_BF16) == g["page_bytes_bf16"] == g["page_kib_bf16"] * 1024
    assert S // O.PAGE_TOKENS == g["pages_per_128k"]
    assert f8 * L == g["per_token_all_layers_fp8"]
    assert round(f8 * L / 1024, 1) == g["per_token_all_layers_fp8_kib"]
    assert round(O.request_bytes(S, L, O.KV_FP8) / 1e9, 2) == g["request_128k_fp8_gb"]
    assert round(O.request_bytes(S, L, O.KV_FP8) / 2**30, 2) == g["request_128k_fp8_gib"]
    assert round(mha * L * S / 1e9) == g["mha_request_128k_gb"]
    gqa = O.mha_row_bytes(num_heads=8, qk_dim=128, v_dim=128)
    assert gqa == g["gqa8_row_bytes"]
    assert round(gqa * L * S / 1e9, 1) == g["gqa8_request_128k_gb"]
    assert round(gqa / bf, 1) == g["gqa8_over_mla_ratio"]
    assert round(64 * 1024 * O.ROW_ELEMS * 2 / 1e6, 1) == g["gather_workspace_64k_rows_mb"]
    assert 128 * 128 * 2 == g["trtllm_mha_elems_per_token"]
    assert O.ROW_ELEMS == g["trtllm_mla_elems_per_token"]


def test_scale_is_192_wide():
    assert O.default_scale() == pytest.approx(1 / math.sqrt(192), rel=1e-15)
    assert O.default_scale() != pytest.approx(1 / math.sqrt(576), rel=1e-3)


# ----------------------------------------------------------------------------
# number formats against torch's codecs
# ----------------------------------------------------------------------------
def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**16, size=20000, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]       # drop inf/nan encodings
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(O.bf16_bits_to_f64(bits), ref)


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = O.e4m3_value(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert set(np.flatnonzero(np.isnan(got))) == {0x7F, 0xFF}
    assert np.nanmax(got) == 448.0 and np.nanmin(got) == -448.0


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(2)
    pos = O.e4m3_value(np.arange(0, 127))
    mids = (pos[:-1] + pos[1:]) / 2
    x = np.concatenate([
        rng.standard_normal(20000) * 50,
        rng.uniform(-448, 448, 20000),
        rng.standard_normal(5000) * 1e-2,
        mids, -mids, pos, -pos,
        np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
        np.nextafter(mids.astype(np.float32), np.float32(-np.inf)),
    ]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(x), ref)


def test_e4m3_encode_ties_and_saturation():
    # ties go to the even code
    assert O.e4m3_encode(np.float32(1.0625)) == 0x38          # between 1.0 (0x38) and 1.125 (0x39)
    assert O.e4m3_encode(np.float32(1.1875)) == 0x3A          # between 1.125 and 1.25 (0x3A)
    # half of the smallest subnormal rounds to zero, just above rounds up
    assert O.e4m3_encode(np.float32(2.0**-10)) == 0x00
    assert O.e4m3_encode(np.nextafter(np.float32(2.0**-10), np.float32(1))) == 0x01
    # saturation instead of NaN
    for v, c in [(448.0, 0x7E), (460.0, 0x7E), (470.0, 0x7E), (1e6, 0x7E), (-1e30, 0xFE)]:
        assert O.e4m3_encode(np.float32(v)) == c
    # round trip of every finite code
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(O.e4m3_encode(O.e4m3_value(codes).astype(np.float32)), codes)


def test_fp8_quantize_row_properties():
    rng = np.random.default_rng(3)
    x = MI.to_bf16_bits(rng.standard_normal(576).astype(np.float32) * 3)
    codes, s = O.fp8_quantize_row(x)
    xf = O.bf16_bits_to_f64(x)
    # the largest magnitude lands on 448 exactly
    assert np.max(np.abs(O.e4m3_value(codes))) == 448.0
    assert s == np.float32(np.float32(np.max(np.abs(xf))) / np.float32(448))
    # dequantized error within half a 3-bit-mantissa ulp (relative 2^-4), or the subnormal step
    deq = O.e4m3_value(codes) * np.float64(s)
    bound = np.maximum(np.abs(xf) * 2.0**-4, float(s) * 2.0**-10) * (1 + 1e-6)
    assert np.all(np.abs(deq - xf) <= bound)
    # an all-zero row uses scale 1 and code 0
    z_codes, z_s = O.fp8_quantize_row(np.zeros(576, np.uint16))
    assert z_s == 1.0 and np.all(z_codes == 0)


# ----------------------------------------------------------------------------
# cache write
# ----------------------------------------------------------------------------
def test_cache_write_bf16_is_bit_copy_and_touches_only_its_slots():
    rng = np.random.default_rng(4)
    pool = rng.integers(0, 256, size=(5, 64, 1152), dtype=np.uint8)
    kv = MI.to_bf16_bits(rng.standard_normal((4, 512)).astype(np.float32))
    pe = MI.to_bf16_bits(rng.standard_normal((4, 64)).astype(np.float32))
    slots = np.array([3 * 64 + 7, -1, 0, 4 * 64 + 63])
    out = O.cache_write(pool, kv, pe, slots, O.KV_BF16)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        row = out[s // 64, s % 64].view("<u2")
        assert np.array_equal(row[:512], kv[t]) and np.array_equal(row[512:], pe[t])
    touched = np.zeros((5, 64), bool)
    touched[3, 7] = touched[0, 0] = touched[4, 63] = True
    assert np.array_equal(out[~touched], pool[~touched])


def test_cache_write_fp8_layout():
    rng = np.random.default_rng(5)
    pool = np.zeros((2, 64, 584), dtype=np.uint8)
    kv = MI.to_bf16_bits(rng.standard_normal((1, 512)).astype(np.float32))
    pe = MI.to_bf16_bits(rng.standard_normal((1, 64)).astype(np.float32))
    out = O.cache_write(pool, kv, pe, np.array([70]), O.KV_FP8)
    row = out[1, 6]
    codes, s = O.fp8_quantize_row(np.concatenate([kv[0], pe[0]]))
    assert np.array_equal(row[:576], codes)
    assert row[576:580].view("<f4")[0] == s and row[580:584].view("<f4")[0] == s
    K, Vv = O.row_views(row[None], O.KV_FP8)
    assert K.shape == (1, 576) and Vv.shape == (1, 512)


# ----------------------------------------------------------------------------
# attention: closed forms and invariants
# ----------------------------------------------------------------------------
def _pool_from_rows(rows_bits):
    """bf16 pool whose page p holds rows_bits[p*64 : p*64+64] (pure byte packing)."""
    n = rows_bits.shape[0]
    pages = (n + 63) // 64
    buf = np.zeros((pages * 64, rows_bits.shape[1]), np.uint16)
    buf[:n] = rows_bits
    return buf.astype("<u2").view(np.uint8).reshape(pages, 64, -1)


def _rand_bits(rng, shape, std=1.0):
    return MI.to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))


def test_single_token_context_returns_v_exactly():
    rng = np.random.default_rng(6)
    rows = _rand_bits(rng, (1, 576))
    pool = _pool_from_rows(rows)
    q = O.bf16_bits_to_f64(_rand_bits(rng, (1, 1, 8, 576)))
    o, lse = O.decode(q, pool, O.KV_BF16, np.array([[0]]), np.array([1]), O.default_scale())
    v0 = O.bf16_bits_to_f64(rows[0, :512])
    assert np.array_equal(o[0, 0], np.broadcast_to(v0, (8, 512)))
    k0 = O.bf16_bits_to_f64(rows[0])
    assert np.allclose(lse[0, 0], O.default_scale() * (q[0, 0] @ k0), rtol=0, atol=1e-12)


def test_zero_query_gives_uniform_softmax():
    rng = np.random.default_rng(7)
    n = 150
    rows = _rand_bits(rng, (n, 576))
    pool = _pool_from_rows(rows)
    bt = np.arange(pool.shape[0])[None]
    q = np.zeros((1, 1, 4, 576))
    o, lse = O.decode(q, pool, O.KV_BF16, bt, np.array([n]), O.default_scale())
    V = O.bf16_bits_to_f64(rows[:, :512])
    assert np.allclose(lse, math.log(n), atol=1e-12)
    assert np.allclose(o[0, 0], V.mean(0)[None], atol=1e-12)


def test_identical_keys_give_that_value():
    rng = np.random.default_rng(8)
    n = 77
    row = _rand_bits(rng, (1, 576))
    pool = _pool_from_rows(np.repeat(row, n, axis=0))
    q = O.bf16_bits_to_f64(_rand_bits(rng, (1, 1, 3, 576)))
    o, lse = O.decode(q, pool, O.KV_BF16, np.arange(2)[None], np.array([n]), 0.1)
    s = 0.1 * (q[0, 0] @ O.bf16_bits_to_f64(row[0]))
    assert np.allclose(lse[0, 0], s + math.log(n), atol=1e-11)
    assert np.allclose(o[0, 0], O.bf16_bits_to_f64(row[0, :512])[None], atol=1e-12)


def test_decode_matches_torch_sdpa_and_logsumexp():
    """The decode oracle equals torch's float64 SDPA over the gathered rows (MQA broadcast)."""
    w = MI.make_workload("t", 3, 1, 8, [5, 64, 130], 8, MI.KV_BF16, False, 11)
    pool = O.cache_write(np.zeros((w.num_pages, 64, 1152), np.uint8),
                         w.kv_rows.reshape(-1, 576)[:, :512], w.kv_rows.reshape(-1, 576)[:, 512:],
                         np.arange(w.num_pages * 64), O.KV_BF16)
    q = O.bf16_bits_to_f64(w.q)
    sc = O.default_scale()
    o, lse = O.decode(q, pool, O.KV_BF16, w.block_table, w.seq_lens, sc)
    for b in range(w.B):
        n = int(w.seq_lens[b])
        j = np.arange(n)
        rows = w.kv_rows[w.block_table[b, j // 64], j % 64]
        K = torch.from_numpy(O.bf16_bits_to_f64(rows))
        qt = torch.from_numpy(q[b, 0])
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt[None, :, None, :], K[None, None].expand(1, w.N, n, 576),
            K[None, None, :, :512].expand(1, w.N, n, 512), scale=sc)[0, :, 0]
        assert np.allclose(o[b, 0], ref.numpy(), rtol=1e-12, atol=1e-13)
        ref_lse = torch.logsumexp(sc * qt @ K.T, dim=-1).numpy()
        assert np.allclose(lse[b, 0], ref_lse, rtol=0, atol=1e-12)


def test_probabilities_sum_to_one():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((5, 576))
    K = rng.standard_normal((40, 576))
    _, lse = O.attend(q, K, K[:, :512], 0.07)
    assert np.allclose(np.exp(0.07 * q @ K.T - lse[:, None]).sum(1), 1.0, atol=1e-13)


def test_empty_context_row():
    q = np.ones((1, 2, 2, 576))
    pool = np.zeros((1, 64, 1152), np.uint8)
    o, lse = O.decode(q, pool, O.KV_BF16, np.array([[0]]), np.array([1]), 0.1)
    # q_len 2 with seq_len 1: row 0 sees 0 tokens, row 1 sees 1
    assert np.all(o[0, 0] == 0) and np.all(np.isneginf(lse[0, 0]))
    assert np.all(np.isfinite(lse[0, 1]))


def test_merge_of_any_partition_equals_unsplit():
    rng = np.random.default_rng(10)
    q = rng.standard_normal((6, 576))
    K = rng.standard_normal((300, 576)) * 2
    o_all, lse_all = O.attend(q, K, K[:, :512], O.default_scale())
    for cuts in ([0, 300], [0, 1, 300], [0, 64, 128, 200, 300], [0, 0, 150, 150, 300]):
        parts = [O.attend(q, K[a:b], K[a:b, :512], O.default_scale()) for a, b in zip(cuts, cuts[1:])]
        o, lse = O.merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
        assert np.allclose(o, o_all, atol=1e-12) and np.allclose(lse, lse_all, atol=1e-12)
    o, lse = O.merge(np.zeros((3, 2, 4)), np.full((3, 2), -np.inf))
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_causal_rows_equal_single_token_decodes():
    w = MI.make_workload("t", 2, 2, 4, [70, 129], 8, MI.KV_BF16, False, 12)
    pool = O.cache_write(np.zeros((w.num_pages, 64, 1152), np.uint8),
                         w.kv_rows.reshape(-1, 576)[:, :512], w.kv_rows.reshape(-1, 576)[:, 512:],
                         np.arange(w.num_pages * 64), O.KV_BF16)
    q = O.bf16_bits_to_f64(w.q)
    o2, lse2 = O.decode(q, pool, O.KV_BF16, w.block_table, w.seq_lens, 0.1)
    for t in range(2):
        o1, lse1 = O.decode(q[:, t:t + 1], pool, O.KV_BF16, w.block_table,
                            w.seq_lens - 1 + t, 0.1)
        assert np.array_equal(o1[:, 0], o2[:, t]) and np.array_equal(lse1[:, 0], lse2[:, t])
    # row 0 really sees one token fewer than row 1
    assert not np.allclose(lse2[:, 0], lse2[:, 1])


def test_page_permutation_invariance():
    w = MI.make_workload("t", 2, 1, 4, [100, 65], 6, MI.KV_BF16, False, 13)
    pool = O.cache_write(np.zeros((w.num_pages, 64, 1152), np.uint8),
                         w.kv_rows.reshape(-1, 576)[:, :512], w.kv_rows.reshape(-1, 576)[:, 512:],
                         np.arange(w.num_pages * 64), O.KV_BF16)
    q = O.bf16_bits_to_f64(w.q)
    o, lse = O.decode(q, pool, O.KV_BF16, w.block_table, w.seq_lens, 0.1)
    perm = np.random.default_rng(0).permutation(w.num_pages)      # new page id -> old page id
    inv = np.argsort(perm)
    bt2 = np.where(w.block_table >= 0, inv[np.maximum(w.block_table, 0)], -1)
    o2, lse2 = O.decode(q, pool[perm], O.KV_BF16, bt2, w.seq_lens, 0.1)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_head_permutation_permutes_outputs():
    rng = np.random.default_rng(14)
    q = rng.standard_normal((7, 576))
    K = rng.standard_normal((50, 576))
    o, lse = O.attend(q, K, K[:, :512], 0.1)
    p = rng.permutation(7)
    o2, lse2 = O.attend(q[p], K, K[:, :512], 0.1)
    # BLAS blocking may change the last bits with row order; values must agree to rounding
    assert np.allclose(o2, o[p], rtol=1e-13, atol=1e-14) and np.allclose(lse2, lse[p], rtol=1e-14, atol=0)


# ----------------------------------------------------------------------------
# absorption identity: brute force in pure Python loops, tiny dims
# ----------------------------------------------------------------------------
def _brute_unabsorbed(qn, qp, C, KPE, WK, WV, scale):
    """Pure-Python MLA for one query row: up-project every latent, then softmax."""
    H, P = len(qn), len(qn[0])
    n, Lr = len(C), len(C[0])
    Vd = len(WV[0][0])
    ys, lses = [], []
    for h in range(H):
        scores = []
        vs = []
        for j in range(n):
            k_nope = [sum(WK[h][p][l] * C[j][l] for l in range(Lr)) for p in range(P)]
            s = sum(qn[h][p] * k_nope[p] for p in range(P)) + sum(qp[h][r] * KPE[j][r] for r in range(len(qp[h])))
            scores.append(scale * s)
            vs.append([sum(C[j][l] * WV[h][l][v] for l in range(Lr)) for v in range(Vd)])
        m = max(scores)
        z = sum(math.exp(s - m) for s in scores)
        lse = m + math.log(z)
        y = [sum(math.exp(scores[j] - lse) * vs[j][v] for j in range(n)) for v in range(Vd)]
        ys.append(y)
        lses.append(lse)
    return ys, lses


@pytest.mark.parametrize("n", [1, 3, 7])
def test_absorption_identity_brute_force(n):
    """up_v(decode(absorb(q))) == un-absorbed MLA, tiny dims, fp64."""
    rng = np.random.default_rng(100 + n)
    Ld, Rd, Pd, Vd, H = 8, 2, 4, 4, 3
    C = rng.standard_normal((n, Ld))
    KPE = rng.standard_normal((n, Rd))
    WK = rng.standard_normal((H, Pd, Ld))       # W_UK_T[h] : [P, L]
    WV = rng.standard_normal((H, Ld, Vd))       # W_UV[h]   : [L, V]
    qn = rng.standard_normal((H, Pd))
    qp = rng.standard_normal((H, Rd))
    scale = (Pd + Rd) ** -0.5
    y_ref, lse_ref = _brute_unabsorbed(qn.tolist(), qp.tolist(), C.tolist(), KPE.tolist(),
                                       WK.tolist(), WV.tolist(), scale)
    # oracle route: absorb -> decode over float64 rows -> up_v
    qf = O.absorb(qn[None], qp[None], WK)[0]                  # [H, L+R]
    rows = np.concatenate([C, KPE], axis=1)
    o, lse = O.attend(qf, rows, rows[:, :Ld], scale)
    y = O.up_v(o[None], WV)[0]
    assert np.allclose(y, np.array(y_ref), rtol=1e-10, atol=1e-12)
    assert np.allclose(lse, np.array(lse_ref), rtol=1e-12, atol=1e-12)
    # the 576-wide (here L+R-wide) scale breaks the identity
    o_bad, lse_bad = O.attend(qf, rows, rows[:, :Ld], (Ld + Rd) ** -0.5)
    if n > 1:
        assert not np.allclose(O.up_v(o_bad[None], WV)[0], np.array(y_ref), rtol=1e-6)
    assert not np.allclose(lse_bad, np.array(lse_ref), rtol=1e-6)


def test_absorption_identity_tiny_config_full_dims():
    """Same identity at the tiny workload's real dims, via the vectorised un-absorbed oracle."""
    w = MI.tiny()
    pool = O.cache_write(np.zeros((w.num_pages, 64, 1152), np.uint8),
                         w.kv_rows.reshape(-1, 576)[:, :512], w.kv_rows.reshape(-1, 576)[:, 512:],
                         np.arange(w.num_pages * 64), O.KV_BF16)
    qn = O.bf16_bits_to_f64(w.q_nope)
    qp = O.bf16_bits_to_f64(w.q_pe)
    wk = O.bf16_bits_to_f64(w.w_uk_t)
    wv = O.bf16_bits_to_f64(w.w_uv)
    sc = O.default_scale()
    y_ref, lse_ref = O.mla_unabsorbed(qn, qp, pool, O.KV_BF16, w.block_table, w.seq_lens, wk, wv, sc)
    qf = O.absorb(qn.reshape(-1, w.N, 128), qp.reshape(-1, w.N, 64), wk).reshape(w.B, w.q_len, w.N, 576)
    o, lse = O.decode(qf, pool, O.KV_BF16, w.block_table, w.seq_lens, sc)
    y = O.up_v(o.reshape(-1, w.N, 512), wv).reshape(w.B, w.q_len, w.N, 128)
    assert np.allclose(y, y_ref, rtol=1e-9, atol=1e-12)
    assert np.allclose(lse, lse_ref, rtol=0, atol=1e-10)
    # dropping the rope term of the key would be caught here
    y_norope, _ = O.mla_unabsorbed(qn, np.zeros_like(qp), pool, O.KV_BF16, w.block_table,
                                   w.seq_lens, wk, wv, sc)
    assert not np.allclose(y_norope, y_ref, rtol=1e-3)


def test_fp8_views_use_their_own_scales():
    """With k_scale != v_scale the un-absorbed and absorbed routes still agree,
    and swapping the scales changes the result."""
    rng = np.random.default_rng(15)
    rows = MI.random_fp8_rows(rng, 64, max_code_exp=7)
    pool = rows.reshape(1, 64, 584)
    N = 2
    qn = rng.standard_normal((1, 1, N, 128))
    qp = rng.standard_normal((1, 1, N, 64))
    wk = rng.standard_normal((N, 128, 512)) / 22
    wv = rng.standard_normal((N, 512, 128)) / 22
    sc = O.default_scale()
    y_ref, lse_ref = O.mla_unabsorbed(qn, qp, pool, O.KV_FP8, np.array([[0]]), np.array([50]), wk, wv, sc)
    qf = O.absorb(qn[0], qp[0], wk)[None]
    o, lse = O.decode(qf, pool, O.KV_FP8, np.array([[0]]), np.array([50]), sc)
    y = O.up_v(o[0], wv)[None]
    assert np.allclose(y, y_ref, rtol=1e-9, atol=1e-12) and np.allclose(lse, lse_ref, atol=1e-10)
    swapped = rows.copy()
    swapped[:, 576:580], swapped[:, 580:584] = rows[:, 580:584], rows[:, 576:580]
    o2, _ = O.decode(qf, swapped.reshape(1, 64, 584), O.KV_FP8, np.array([[0]]), np.array([50]), sc)
    assert not np.allclose(o2, o, rtol=1e-3)


def _hand_fp8_row(codes, k_scale: float, v_scale: float) -> np.ndarray:
    """One raw fp8 cache row written byte by byte: 576 code bytes, then the float32
    K scale, then the float32 V scale (the row format of [vLLM-MLA] §缓存的形状:
    scales appended after the data, one for K and one for V)."""
    import struct
    row = np.zeros(584, dtype=np.uint8)
    row[:576] = np.asarray(codes, dtype=np.uint8)
    row[576:580] = np.frombuffer(struct.pack("<f", k_scale), dtype=np.uint8)
    row[580:584] = np.frombuffer(struct.pack("<f", v_scale), dtype=np.uint8)
    return row


def test_fp8_scale_slots_hand_row():
    """Bytes 576..579 scale the K view (all 576 elements), bytes 580..583 the V view
    (the first 512).  Codes by the e4m3fn definition: 0x38 = +1.0 (exponent field 7 =
    bias, mantissa 0), 0x40 = +2.0, 0xB8 = -1.0, 0x30 = +0.5."""
    codes = np.full(576, 0x38, dtype=np.uint8)
    codes[1], codes[2], codes[3] = 0x40, 0xB8, 0x30
    row = _hand_fp8_row(codes, 2.0, 3.0)
    K, V = O.row_views(row[None], O.KV_FP8)
    assert K.shape == (1, 576) and V.shape == (1, 512)
    want = np.ones(576)
    want[1], want[2], want[3] = 2.0, -1.0, 0.5
    assert np.array_equal(K[0], 2.0 * want)
    assert np.array_equal(V[0], 3.0 * want[:512])


def test_fp8_one_token_context_returns_v_scale_times_code():
    """A one-token fp8 context: the softmax weight is exactly 1, so the output is
    code * v_scale element by element (3 * code here, never 2 * code), and the LSE is
    the single scaled score, scale * sum_i q_i * code_i * k_scale."""
    rng = np.random.default_rng(17)
    codes = rng.choice(np.array([0x38, 0x40, 0xB8, 0x30], dtype=np.uint8), size=576)
    vals = {0x38: 1.0, 0x40: 2.0, 0xB8: -1.0, 0x30: 0.5}
    c = np.array([vals[int(x)] for x in codes])
    pool = np.zeros((1, 64, 584), dtype=np.uint8)
    pool[0, 0] = _hand_fp8_row(codes, 2.0, 3.0)
    q = rng.standard_normal((1, 1, 2, 576))
    sc = O.default_scale()
    o, lse = O.decode(q, pool, O.KV_FP8, np.array([[0]]), np.array([1]), sc)
    for h in range(2):
        assert np.array_equal(o[0, 0, h], 3.0 * c[:512])
        s = sc * sum(float(q[0, 0, h, i]) * c[i] * 2.0 for i in range(576))
        assert abs(lse[0, 0, h] - s) <= 1e-12 * max(1.0, abs(s))


def test_fp8_two_token_context_closed_form():
    """Two fp8 tokens with all codes 1.0, K scales (1, 2), V scales (3, 5), query of
    ones: scores s_j = scale * 576 * k_j, so every output element is
    (3 e^{s_0} + 5 e^{s_1}) / (e^{s_0} + e^{s_1}) and lse = ln(e^{s_0} + e^{s_1}).
    Swapping the two scale slots of either row breaks both."""
    ones = np.full(576, 0x38, dtype=np.uint8)
    pool = np.zeros((1, 64, 584), dtype=np.uint8)
    pool[0, 0] = _hand_fp8_row(ones, 1.0, 3.0)
    pool[0, 1] = _hand_fp8_row(ones, 2.0, 5.0)
    q = np.ones((1, 1, 1, 576))
    sc = O.default_scale()
    o, lse = O.decode(q, pool, O.KV_FP8, np.array([[0]]), np.array([2]), sc)
    s0, s1 = sc * 576 * 1.0, sc * 576 * 2.0
    m = max(s0, s1)
    e0, e1 = math.exp(s0 - m), math.exp(s1 - m)
    want = (3.0 * e0 + 5.0 * e1) / (e0 + e1)
    assert np.allclose(o[0, 0, 0], want, rtol=1e-13, atol=0)
    assert abs(lse[0, 0, 0] - (m + math.log(e0 + e1))) <= 1e-12
    for j in range(2):
        sw = pool.copy()
        sw[0, j, 576:580], sw[0, j, 580:584] = pool[0, j, 580:584], pool[0, j, 576:580]
        o2, l2 = O.decode(q, sw, O.KV_FP8, np.array([[0]]), np.array([2]), sc)
        assert not np.allclose(o2[0, 0, 0], want, rtol=1e-6) or abs(l2[0, 0, 0] - lse[0, 0, 0]) > 1e-6


def test_absorb_and_up_v_against_loops():
    rng = np.random.default_rng(16)
    qn = rng.standard_normal((2, 3, 4))
    qp = rng.standard_normal((2, 3, 2))
    wk = rng.standard_normal((3, 4, 5))
    out = O.absorb(qn, qp, wk)
    for t in range(2):
        for h in range(3):
            for l in range(5):
                assert out[t, h, l] == pytest.approx(sum(qn[t, h, p] * wk[h, p, l] for p in range(4)), rel=1e-13)
            assert np.array_equal(out[t, h, 5:], qp[t, h])
    ol = rng.standard_normal((2, 3, 5))
    wv = rng.standard_normal((3, 5, 4))
    y = O.up_v(ol, wv)
    for t in range(2):
        for h in range(3):
            for v in range(4):
                assert y[t, h, v] == pytest.approx(sum(ol[t, h, l] * wv[h, l, v] for l in range(5)), rel=1e-13)


def test_encode_rows_matches_per_token_cache_write():
    rng = np.random.default_rng(17)
    rows = MI.to_bf16_bits((rng.standard_normal((128, 576)) * rng.uniform(0.01, 100, (128, 1))).astype(np.float32))
    rows[5] = 0                                        # an all-zero row
    for dt, rb in ((O.KV_BF16, 1152), (O.KV_FP8, 584)):
        pool = O.cache_write(np.zeros((2, 64, rb), np.uint8), rows[:, :512], rows[:, 512:],
                             np.arange(128), dt)
        assert np.array_equal(pool.reshape(128, rb), O.encode_rows(rows, dt))


def test_round_to_bf16_matches_torch():
    rng = np.random.default_rng(18)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-20, 20, 20000),
                        (rng.integers(-2**15, 2**15, 4000) + 0.5) * 2.0 ** -7])   # exact ties
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(O.round_to_bf16(x), ref)


def test_bf16_half_ulp_helper():
    from tests.mla_testlib import bf16_half_ulp
    x = np.array([1.0, 1.99, 0.5, -3.0, 2.0 ** -20, 0.0])
    assert np.array_equal(bf16_half_ulp(x), [2.0 ** -8, 2.0 ** -8, 2.0 ** -9, 2.0 ** -7, 2.0 ** -28, 0.0])
    # the exactly rounded value is always within half an ulp
    v = np.random.default_rng(0).standard_normal(10000)
    assert np.all(np.abs(O.round_to_bf16(v) - v) <= bf16_half_ulp(v))


# ----------------------------------------------------------------------------
# context gather and the two-part merge (the steps either side of decode)
# ----------------------------------------------------------------------------
def test_f64_to_bf16_bits_hand_values():
    x = np.array([1.0, -2.0, 1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-8 + 2**-30, 2**-133, 2**-134,
                  3 * 2**-134, 2**-126, np.nan, np.inf, -np.inf, 3.5e38, 0.0, -0.0, 448.0 * 0.5])
    want = [0x3F80, 0xC000, 0x3F80, 0x3F82, 0x3F81, 0x0001, 0x0000, 0x0002, 0x0080, 0x7FC0, 0x7F80,
            0xFF80, 0x7F80, 0x0000, 0x8000, 0x4360]
    assert [int(v) for v in O.f64_to_bf16_bits(x)] == want


def test_f64_to_bf16_bits_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(30)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-40, 38, 20000),
                        rng.standard_normal(2000) * 1e-39]).astype(np.float32)
    ours = O.f64_to_bf16_bits(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def _position_pool(num_pages):
    """bf16 pool whose every element encodes (page, offset, element)."""
    pg, off, el = np.meshgrid(np.arange(num_pages), np.arange(64), np.arange(576), indexing="ij")
    return ((pg * 64 + off) * 7 + el).astype(np.uint16).view(np.uint8).reshape(num_pages, 64, 1152)


def test_gather_cache_bf16_rows_come_from_their_logical_tokens():
    rng = np.random.default_rng(31)
    num_pages = 40
    pool = _position_pool(num_pages)
    seqs = [130, 64, 1, 200]                       # context lengths of the chunk's requests
    starts = [64, 0, 0, 128]                      # page-aligned chunk starts inside the requests
    bt = np.full((4, 6), -1, np.int32)
    perm = rng.permutation(num_pages)
    k = 0
    for b, (n, s0) in enumerate(zip(seqs, starts)):
        for p in range((s0 + n + 63) // 64):
            bt[b, p] = perm[k]
            k += 1
    cu = np.concatenate([[0], np.cumsum(seqs)]).astype(np.int32)
    t2s = np.repeat(np.arange(4), seqs).astype(np.int32)
    out = O.gather_cache(pool, O.KV_BF16, bt, cu, t2s, np.array(starts, np.int32))
    for r in range(len(t2s)):
        b = t2s[r]
        j = starts[b] + r - cu[b]
        page, offset = bt[b, j // 64], j % 64
        assert np.array_equal(out[r], ((page * 64 + offset) * 7 + np.arange(576)).astype(np.uint16))


def test_gather_cache_fp8_dequant_hand_values():
    """code x k_scale, rounded once to bf16 (v_scale is not used by the K view)."""
    cases = [  # (code, k_scale, expected bf16 bits)
        (0x38, 2.0, 0x4000),             # 1.0 x 2
        (0x7E, 0.5, 0x4360),             # 448 x 0.5 = 224
        (0xFE, 0.5, 0xC360),             # -224
        (0x01, 4.0, 0x3C00),             # subnormal 2^-9 x 4 = 2^-7
        (0x00, 3.0, 0x0000),
        (0x38, 1 + 2**-8, 0x3F80),       # exact tie 1 + 2^-8 -> even (1.0)
        (0x38, 1 + 3 * 2**-8, 0x3F82),   # exact tie -> even (1 + 2^-6)
        (0x3F, 1 + 2**-10, 0x3FF0),      # 1.875 (1 + 2^-10) = 1.87683... -> 1.875
        (0x3C, 1 + 2**-8, 0x3FC1),       # 1.5 (1 + 2^-8) = 1.505859375 -> 1.5078125
    ]
    n = len(cases)
    pool = np.zeros((1, 64, 584), np.uint8)
    for i, (code, ks, _) in enumerate(cases):
        pool[0, i, :576] = code
        pool[0, i, 576:580] = np.array([ks], "<f4").view(np.uint8)
        pool[0, i, 580:584] = np.array([1000.0], "<f4").view(np.uint8)   # v_scale: unused here
    out = O.gather_cache(pool, O.KV_FP8, np.zeros((1, 1), np.int32), np.array([0, n], np.int32),
                         np.zeros(n, np.int32))
    for i, (_, _, want) in enumerate(cases):
        assert np.all(out[i] == want), (i, hex(int(out[i, 0])), hex(want))


def test_merge_attn_states_closed_forms():
    rng = np.random.default_rng(32)
    o1, o2 = rng.standard_normal((2, 5, 3, 16))
    l1, l2 = rng.standard_normal((2, 5, 3))
    # an empty state weighs nothing
    o, lse = O.merge_attn_states(o1, l1, np.zeros_like(o2), np.full_like(l2, -np.inf))
    assert np.array_equal(o, o1) and np.array_equal(lse, l1)
    o, lse = O.merge_attn_states(np.zeros_like(o1), np.full_like(l1, -np.inf), o2, l2)
    assert np.array_equal(o, o2) and np.array_equal(lse, l2)
    # both empty: o = 0, lse = -inf
    o, lse = O.merge_attn_states(np.zeros_like(o1), np.full_like(l1, -np.inf), np.zeros_like(o2),
                                 np.full_like(l2, -np.inf))
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    # equal LSE: the plain average, LSE + ln 2
    o, lse = O.merge_attn_states(o1, l1, o2, l1)
    assert np.allclose(o, (o1 + o2) / 2, atol=1e-15) and np.allclose(lse, l1 + math.log(2), atol=1e-15)


def test_merge_attn_states_of_a_key_split_equals_attention_over_all_keys():
    rng = np.random.default_rng(33)
    q = rng.standard_normal((8, 192))
    K = rng.standard_normal((90, 192)) * 1.5
    V = rng.standard_normal((90, 128))
    o_all, l_all = O.attend(q, K, V, O.default_scale())
    for cut in (0, 1, 37, 89, 90):
        op, lp = O.attend(q, K[:cut], V[:cut], O.default_scale())
        os_, ls = O.attend(q, K[cut:], V[cut:], O.default_scale())
        o, lse = O.merge_attn_states(op, lp, os_, ls)
        assert np.allclose(o, o_all, atol=1e-12) and np.allclose(lse, l_all, atol=1e-12)


# ----------------------------------------------------------------------------
# variable query lengths (speculative-decoding verification batches)
# ----------------------------------------------------------------------------
def _varlen_case(seed, q_lens, seqs, kd=O.KV_BF16):
    w = MI.make_workload("vl", len(seqs), 1, 4, seqs, None, kd, False, seed)
    pool = O.encode_rows(w.kv_rows.reshape(-1, 576), kd).reshape(w.num_pages, 64, -1)
    rng = np.random.default_rng(seed)
    qsl = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    q = rng.standard_normal((int(qsl[-1]), 4, 576))
    return w, pool, qsl, q


def test_decode_varlen_with_uniform_lengths_is_the_uniform_decode():
    w, pool, qsl, q = _varlen_case(40, [2, 2, 2], [70, 129, 3])
    o, lse = O.decode_varlen(q, qsl, pool, w.kv_dtype, w.block_table, w.seq_lens, True, O.default_scale())
    o2, lse2 = O.decode(q.reshape(3, 2, 4, 576), pool, w.kv_dtype, w.block_table, w.seq_lens, O.default_scale())
    assert np.array_equal(o, o2.reshape(6, 4, 512)) and np.array_equal(lse, lse2.reshape(6, 4))


def test_decode_varlen_rows_are_single_row_decodes_at_their_lengths():
    """Causal: row t of a q_len-token block is a one-row decode over seq - q_len + 1 + t
    tokens; non-causal: over all seq tokens.  Brute force per row."""
    q_lens = [1, 3, 2, 4]
    w, pool, qsl, q = _varlen_case(41, q_lens, [65, 130, 2, 200])
    for causal in (True, False):
        o, lse = O.decode_varlen(q, qsl, pool, w.kv_dtype, w.block_table, w.seq_lens, causal, O.default_scale())
        for b, ql in enumerate(q_lens):
            for t in range(ql):
                r = qsl[b] + t
                n = max(0, int(w.seq_lens[b]) - ql + 1 + t) if causal else int(w.seq_lens[b])
                o1, l1 = O.decode(q[r][None, None], pool, w.kv_dtype, w.block_table[b:b + 1],
                                  np.array([n], np.int32), O.default_scale())
                assert np.array_equal(o[r], o1[0, 0]) and np.array_equal(lse[r], l1[0, 0])
    # non-causal: all rows of a block see the same keys, so equal queries give equal rows
    q2 = q.copy()
    q2[qsl[3]:qsl[4]] = q2[qsl[3]]
    o, _ = O.decode_varlen(q2, qsl, pool, w.kv_dtype, w.block_table, w.seq_lens, False, O.default_scale())
    assert all(np.array_equal(o[qsl[3]], o[r]) for r in range(qsl[3], qsl[4]))
    oc, _ = O.decode_varlen(q2, qsl, pool, w.kv_dtype, w.block_table, w.seq_lens, True, O.default_scale())
    assert not np.array_equal(oc[qsl[3]], oc[qsl[4] - 1])


# ----------------------------------------------------------------------------
# per-token-group fp8 quantization of the up-projected output
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("group", [64, 128])
def test_quantize_groups_fp8_properties(group):
    rng = np.random.default_rng(50)
    T, C = 6, 512
    y = MI.to_bf16_bits((rng.standard_normal((T, C)) * 10.0 ** rng.integers(-3, 3, (T, 1))).astype(np.float32))
    y[2, :group] = 0                                       # an all-zero group: scale 1, codes 0
    codes, s = O.quantize_groups_fp8(y, group)
    assert codes.shape == (T, C) and s.shape == (T, C // group) and s.dtype == np.float32
    x = O.bf16_bits_to_f64(y).reshape(T, C // group, group)
    c = codes.reshape(T, C // group, group)
    assert s[2, 0] == 1.0 and np.all(c[2, 0] == 0)
    for t in range(T):
        for g in range(C // group):
            if s[t, g] == 1.0 and np.all(x[t, g] == 0):
                continue
            # each group's largest magnitude becomes +-448 (code 0x7E / 0xFE) ...
            k = np.argmax(np.abs(x[t, g]))
            assert (c[t, g, k] & 0x7F) == 0x7E and (c[t, g, k] >> 7) == (x[t, g, k] < 0)
            assert s[t, g] == np.float32(np.float32(np.max(np.abs(x[t, g]))) / np.float32(448.0))
    # ... and dequantization is within half an e4m3 step of every value (relative 2^-4 above 2^-6 s)
    deq = O.e4m3_value(codes).reshape(T, C // group, group) * s[:, :, None]
    err = np.abs(deq - x)
    assert np.all(err <= np.maximum(np.abs(x) * 2.0**-4, 2.0**-10 * s[:, :, None]) * (1 + 1e-6))


def test_quantize_groups_fp8_matches_torch_cast_and_group_boundaries():
    """Codes equal torch's float8_e4m3fn cast of x / s; groups are consecutive elements."""
    rng = np.random.default_rng(51)
    T, C, group = 4, 256, 64
    y = MI.to_bf16_bits(rng.standard_normal((T, C)).astype(np.float32))
    y[:, 64:128] = MI.to_bf16_bits(rng.standard_normal((T, 64)).astype(np.float32) * 1000)   # a loud group
    codes, s = O.quantize_groups_fp8(y, group)
    xf = torch.from_numpy(O.bf16_bits_to_f64(y).astype(np.float32))
    st = torch.from_numpy(np.repeat(s, group, axis=1))
    ref = (xf / st).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    assert np.all(s[:, 1] > 100 * s[:, 0]) and np.all(s[:, 1] > 100 * s[:, 2])


# --- rope fused into the absorption -------------------------------------------
def _angles_table(ang):
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1)


def test_rope_is_complex_multiplication_in_both_pairings():
    """Each pair is a complex number multiplied by exp(i * angle): adjacent pairs
    (x[2i] + i x[2i+1]) and rotate-half pairs (x[i] + i x[i+32])."""
    rng = np.random.default_rng(1200)
    T, N = 5, 3
    x = rng.standard_normal((T, N, 64))
    ang = rng.uniform(-10, 10, (T, 32))
    table = _angles_table(ang)
    pos = np.arange(T)
    e = np.exp(1j * ang)[:, None, :]
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * e
    adj = np.empty_like(x)
    adj[..., 0::2], adj[..., 1::2] = z.real, z.imag
    assert np.allclose(O.rope(x, pos, table, False), adj, rtol=0, atol=1e-13)
    z = (x[..., :32] + 1j * x[..., 32:]) * e
    assert np.allclose(O.rope(x, pos, table, True), np.concatenate([z.real, z.imag], -1), rtol=0, atol=1e-13)


def test_rope_pairings_are_each_other_under_the_deinterleave_permutation():
    rng = np.random.default_rng(1201)
    x = rng.standard_normal((4, 2, 64))
    table = _angles_table(rng.uniform(-3, 3, (4, 32)))
    perm = np.concatenate([np.arange(0, 64, 2), np.arange(1, 64, 2)])   # adjacent -> halves
    a = O.rope(x, np.arange(4), table, False)
    b = O.rope(x[..., perm], np.arange(4), table, True)
    assert np.allclose(a[..., perm], b, rtol=0, atol=1e-14)


def test_rope_hand_values_and_identity():
    x = np.arange(1.0, 65.0).reshape(1, 1, 64)
    quarter = _angles_table(np.full((1, 32), np.pi / 2))
    # a quarter turn: (a, b) -> (-b, a)
    got = O.rope(x, np.array([0]), quarter, True)[0, 0]
    assert np.allclose(got[:32], -x[0, 0, 32:], atol=1e-12) and np.allclose(got[32:], x[0, 0, :32], atol=1e-12)
    got = O.rope(x, np.array([0]), quarter, False)[0, 0]
    assert np.allclose(got[0::2], -x[0, 0, 1::2], atol=1e-12) and np.allclose(got[1::2], x[0, 0, 0::2], atol=1e-12)
    ident = _angles_table(np.zeros((1, 32)))
    for neox in (True, False):
        assert np.array_equal(O.rope(x, np.array([0]), ident, neox), x)


def test_rope_scores_depend_only_on_the_position_difference():
    """<RoPE(q, p), RoPE(k, p')> is a function of p - p' (the reason for rotating)."""
    rng = np.random.default_rng(1202)
    table = MI.rope_cos_sin(64).astype(np.float64)
    q, k = rng.standard_normal((1, 1, 64)), rng.standard_normal((1, 1, 64))
    for neox in (True, False):
        dots = [np.sum(O.rope(q, np.array([p + d]), table, neox) * O.rope(k, np.array([p]), table, neox))
                for p in (0, 7, 30) for d in (5,)]
        assert np.allclose(dots, dots[0], rtol=1e-5)
        far = np.sum(O.rope(q, np.array([12]), table, neox) * O.rope(k, np.array([0]), table, neox))
        assert abs(far - dots[0]) > 1e-3
        # and rotation keeps each pair's length
        r = O.rope(q, np.array([9]), table, neox)
        assert np.isclose(np.sum(r * r), np.sum(q * q), rtol=1e-6)


def test_rope_out_of_range_positions_are_nan_and_absorb_rope_is_absorb_plus_rope():
    rng = np.random.default_rng(1203)
    T, N = 4, 2
    qn, qp = rng.standard_normal((T, N, 128)), rng.standard_normal((T, N, 64))
    w = rng.standard_normal((N, 128, 512))
    table = MI.rope_cos_sin(8)
    pos = np.array([0, 7, 8, -1])
    r = O.rope(qp, pos, table, True)
    assert np.all(np.isnan(r[2:])) and not np.any(np.isnan(r[:2]))
    assert np.array_equal(r[0], qp[0])                                    # position 0: cos 1, sin 0
    f = O.absorb_rope(qn, qp, w, pos, table, False)
    assert np.array_equal(f[..., :512], O.absorb(qn, None, w))
    assert np.array_equal(f[..., 512:], O.rope(qp, pos, table, False), equal_nan=True)


def test_rope_table_helper_follows_the_geometric_schedule():
    t = MI.rope_cos_sin(5, base=100.0, rope_dim=8)
    assert t.shape == (5, 8) and t.dtype == np.float32
    assert np.allclose(t[3, 1], math.cos(3 * 100.0 ** -0.25)) and np.allclose(t[3, 5], math.sin(3 * 100.0 ** -0.25))
    assert np.all(t[0, :4] == 1) and np.all(t[0, 4:] == 0)


# --- prefill of new tokens -----------------------------------------------------
def test_prefill_mha_over_kv_b_proj_equals_absorbed_decode():
    """The compute-friendly prefill (keys and values up-projected by kv_b_proj, 192/128
    MHA) equals the absorbed decode over the latent cache followed by the V
    up-projection, causal rows included (q_len 2: the first row sees one token less)."""
    rng = np.random.default_rng(1400)
    N, lens = 3, [37, 100]
    B, q_len = 2, 2
    pool = np.zeros((4, 64, 576))
    bt = np.array([[0, 1], [2, 3]])
    lat = rng.standard_normal((4 * 64, 576))
    pool[:] = lat.reshape(4, 64, 576)
    wk = rng.standard_normal((N, 128, 512)) / 22
    wv = rng.standard_normal((N, 512, 128)) / 22
    qn = rng.standard_normal((B, q_len, N, 128))
    qp = rng.standard_normal((B, q_len, N, 64))
    sc = O.default_scale()
    pool_bits = O.f64_to_bf16_bits(pool).reshape(4, 64, 576)
    qf = O.absorb(qn.reshape(-1, N, 128), qp.reshape(-1, N, 64), wk).reshape(B, q_len, N, 576)
    o, lse = O.decode(qf, pool_bits.view(np.uint8).reshape(4, 64, 1152), O.KV_BF16, bt, np.array(lens), sc)
    y = O.up_v(o.reshape(-1, N, 512), wv).reshape(B, q_len, N, 128)
    # the same tokens, packed per request, through kv_b_proj and the prefill MHA
    latv = O.bf16_bits_to_f64(pool_bits).reshape(-1, 576)
    rows = np.concatenate([latv[bt[b].repeat(64) * 64 + np.tile(np.arange(64), 2)][:lens[b]] for b in range(B)])
    w_kvb = np.concatenate([np.transpose(wk, (0, 2, 1)), wv], axis=-1)        # [N, L, P + V]
    k_nope, v = O.kv_b_proj(rows[:, :512], w_kvb)
    cu_k = np.array([0, lens[0], lens[0] + lens[1]])
    cu_q = np.array([0, 2, 4])
    q = np.concatenate([qn, qp], axis=-1).reshape(-1, N, 192)
    out, lse2 = O.prefill_mha(q, k_nope, rows[:, 512:], v, cu_q, cu_k, sc, causal=True)
    assert np.allclose(out, y.reshape(-1, N, 128), rtol=1e-9, atol=1e-12)
    assert np.allclose(lse2, lse.reshape(-1, N), rtol=0, atol=1e-10)
    # non-causal: both rows see the whole request, and differ from the causal first row
    out_nc, _ = O.prefill_mha(q, k_nope, rows[:, 512:], v, cu_q, cu_k, sc, causal=False)
    assert np.allclose(out_nc[1], out[1], rtol=1e-12) and not np.allclose(out_nc[0], out[0], rtol=1e-3)


def test_prefill_mha_matches_torch_sdpa_and_handles_empty_requests():
    rng = np.random.default_rng(1401)
    N, T = 2, 9
    q = rng.standard_normal((T, N, 192))
    kn, kp, v = rng.standard_normal((T, N, 128)), rng.standard_normal((T, 64)), rng.standard_normal((T, N, 128))
    sc = O.default_scale()
    out, lse = O.prefill_mha(q, kn, kp, v, np.array([0, T]), np.array([0, T]), sc, causal=True)
    K = np.concatenate([kn, np.broadcast_to(kp[:, None], (T, N, 64))], axis=-1)
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2))) for a in (q, K, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=sc)
    assert np.allclose(out, ref.numpy().transpose(1, 0, 2), rtol=1e-10, atol=1e-12)
    s = np.einsum("thd,shd->hts", q, K) * sc
    s = np.where(np.tril(np.ones((T, T), bool))[None], s, -np.inf)
    assert np.allclose(lse, torch.logsumexp(torch.from_numpy(s), dim=-1).numpy().T, atol=1e-12)
    # a request with queries but no keys, and one with keys but no queries
    out2, lse2 = O.prefill_mha(q[:3], kn[:4], kp[:4], v[:4], np.array([0, 3, 3]), np.array([0, 0, 4]), sc, True)
    assert np.all(out2 == 0) and np.all(np.isneginf(lse2))


def test_kv_b_proj_splits_keys_and_values():
    rng = np.random.default_rng(1402)
    c = rng.standard_normal((5, 512))
    w = rng.standard_normal((3, 512, 256))
    kn, v = O.kv_b_proj(c, w)
    assert kn.shape == (5, 3, 128) and v.shape == (5, 3, 128)
    assert np.allclose(kn[2, 1], c[2] @ w[1, :, :128]) and np.allclose(v[4, 2], c[4] @ w[2, :, 128:])


def test_prefill_workspace_rows_page_numbers():
    """[vLLM-MLA] §Prefill: W = min(max(8 L_max, 4 B_seq P_block), 64 * 1024); at the cap
    the 576-wide bf16 gather workspace is about 72 MiB (the page's 64 x 1024 x 576 x 2
    ~ 75.5 MB of its arithmetic section), and eight full requests or four pages per
    request decide below it."""
    W = O.prefill_workspace_rows
    assert W(163840, 256) == 65536 and W(65536, 1024) == 65536
    assert 65536 * 576 * 2 == 75497472 and abs(65536 * 576 * 2 / 2**20 - 72.0) < 1e-9
    assert W(4096, 16) == 8 * 4096                      # eight full-length requests
    assert W(1024, 64) == 4 * 64 * 64                   # four pages per request
    assert W(2048, 8, 128) == max(8 * 2048, 4 * 8 * 128)


def _check_chunk_plan(lens, W, chunks, P=64):
    seen = {b: [] for b in range(len(lens))}
    for ch in chunks:
        assert ch, "no empty chunk"
        assert sum(t for _, _, t in ch) <= W
        bs = [b for b, _, _ in ch]
        assert bs == sorted(bs) and len(set(bs)) == len(bs), "requests in order, once per chunk"
        for b, start, t in ch:
            assert t > 0 and start % P == 0
            seen[b].append((start, t))
    for b, n in enumerate(lens):
        pos = 0
        for start, t in seen[b]:
            assert start == pos
            pos += t
        assert pos == max(0, n)
    # only the first piece of a chunk can continue a request begun in an earlier chunk
    for ch in chunks:
        for b, start, _ in ch[1:]:
            assert start == 0


def test_plan_context_chunks_by_hand():
    W = 1024
    chunks = O.plan_context_chunks([700, 3000, 130], W)
    assert chunks == [[(0, 0, 700), (1, 0, 320)], [(1, 320, 1024)], [(1, 1344, 1024)],
                      [(1, 2368, 632), (2, 0, 130)]]
    _check_chunk_plan([700, 3000, 130], W, chunks)
    # a chunk with less than a page left closes; an exact fill closes too
    assert O.plan_context_chunks([1000, 100], W) == [[(0, 0, 1000)], [(1, 0, 100)]]
    assert O.plan_context_chunks([1024, 64], W) == [[(0, 0, 1024)], [(1, 0, 64)]]
    assert O.plan_context_chunks([0, 0], W) == []
    with pytest.raises(ValueError):
        O.plan_context_chunks([10], 63)


def test_plan_context_chunks_invariants():
    rng = np.random.default_rng(2700)
    for _ in range(300):
        B = int(rng.integers(1, 40))
        lens = (rng.integers(0, 9000, B) * (rng.random(B) > 0.2)).tolist()
        W = int(rng.choice([64, 100, 512, 1000, 4096, 65536]))
        _check_chunk_plan(lens, W, O.plan_context_chunks(lens, W), 64)

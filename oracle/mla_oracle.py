"""Plain, slow CPU oracle for MLA decode over a paged 576-element latent cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
constant generator with the HIP library; the two meet only on the seeded
inputs produced by ``mla_inputs``.

Everything here is float64 NumPy written straight from the definitions on the
source pages (cited per function).  Page short names used in citations:

* [vLLM-MLA]   "vLLM 源码完全拆解(三十七):MLA 注意力后端——矩阵吸收之后,576 维
                latent KV 如何被四种内核读走"
* [TRTLLM-TP]  "TensorRT-LLM 源码完全拆解(十二):注意力层的张量并行——head 怎么切、
                MLA 为什么不能照切"
* [Triton-MLA] "Triton und MLA: portable Attention und Latent-Space-Attention"

Conventions (readings of the pages, listed in the design doc):

* A cache row is ``[kv_c (L=512) | k_pe (R=64)]``; a page holds 64 rows
  ([vLLM-MLA] §缓存的形状, §FlashMLA).  bf16 rows are 1152 bytes; fp8 rows are
  576 e4m3fn codes followed by two float32 scales, K then V, 584 bytes.
* ``seq_lens[b]`` counts every cached token including the ``q_len`` new ones;
  query row ``t`` sees the first ``seq_lens[b] - q_len + 1 + t`` tokens
  ([vLLM-MLA] §Triton MLA, causal via per-row seq_len).
* Softmax scale is ``1/sqrt(qk_nope + qk_rope) = 1/sqrt(192)`` even though the
  absorbed dot product is 576 wide ([vLLM-MLA] §两套算法).
* ``lse`` is the natural-log log-sum-exp of the *scaled* scores
  ([Triton-MLA] §Entwurfsmotivation: lse_base_on_e).  A row that sees no token
  has ``o = 0`` and ``lse = -inf`` ([vLLM-MLA] §Prefill, empty partials).

Parity status: every public function below is pinned by a ``-m "not gpu"``
test in ``tests/test_oracle_pins.py`` (closed forms, brute force, library
routines, printed numbers); none is "parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np

# --- layout constants, as printed on the pages -------------------------------
KV_LORA_RANK = 512          # L  ([vLLM-MLA] §从模型层看)
ROPE_DIM = 64               # R
QK_NOPE_DIM = 128           # P
V_HEAD_DIM = 128            # V
ROW_ELEMS = KV_LORA_RANK + ROPE_DIM   # 576, the cached head_size
PAGE_TOKENS = 64            # FlashMLA page size ([vLLM-MLA] §缓存的形状)
E4M3_MAX = 448.0            # largest finite OCP e4m3fn value

KV_BF16 = 0
KV_FP8 = 1


def row_bytes(kv_dtype: int, row_elems: int = ROW_ELEMS) -> int:
    """Bytes of one cached token row.

    [vLLM-MLA] §缓存的形状: bf16 stores 2 bytes per element; fp8 stores one
    byte per element and appends two float32 scales (one for K, one for V).
    """
    if kv_dtype == KV_BF16:
        return 2 * row_elems
    if kv_dtype == KV_FP8:
        return row_elems + 2 * 4
    raise ValueError("unknown kv dtype")


def default_scale(qk_nope: int = QK_NOPE_DIM, qk_rope: int = ROPE_DIM) -> float:
    """Softmax scale of absorbed decode: ``(qk_nope + qk_rope) ** -0.5``.

    [vLLM-MLA] §两套算法: the absorbed and un-absorbed dot products are the same
    scalar, so the scale keeps the 192-wide value.
    """
    return (qk_nope + qk_rope) ** -0.5


# --- number formats ----------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Value of bfloat16 bit patterns: the top 16 bits of an IEEE float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value (ties to even) of float64 values, returned as float64.

    Used where the pages' pipeline stores an intermediate as a bf16 tensor (the
    absorbed query and the latent attention output are bf16 in the decode step,
    [vLLM-MLA] §一次 decode step 的完整走查).  Finite inputs only.
    """
    v = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(v)                          # v = m * 2^e, 0.5 <= |m| < 1
    q = np.round(m * 256.0) / 256.0             # 8 significant bits, ties to even
    return np.ldexp(q, e)


def e4m3_value(code: np.ndarray) -> np.ndarray:
    """Value of OCP e4m3fn codes from the format definition.

    1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 is
    subnormal (``2^-6 * m/8``); there is no infinity and only ``S.1111.111``
    is NaN, so the largest finite magnitude is ``2^8 * 1.75 = 448``.
    """
    c = np.asarray(code, dtype=np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = np.ldexp(m / 8.0, -6)
    mag = np.where(e == 0, sub, normal)
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


_E4M3_POS = e4m3_value(np.arange(0, 127))   # codes 0x00..0x7E, increasing


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round float values to e4m3fn codes: nearest, ties to even, saturating.

    Brute force over the 127 non-negative finite codes: pick the closest value;
    on an exact tie pick the even code (even mantissa); magnitudes at or above
    448 map to 448.  The sign bit is kept (so -0.0 and tiny negatives give
    0x80).  Input values are taken exactly as given (callers pass float32).
    """
    v = np.asarray(x, dtype=np.float64)
    a = np.abs(v)
    idx = np.searchsorted(_E4M3_POS, a)          # first table value >= a
    hi = np.clip(idx, 0, 126)
    lo = np.clip(idx - 1, 0, 126)
    d_hi = np.abs(_E4M3_POS[hi] - a)
    d_lo = np.abs(a - _E4M3_POS[lo])
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(pick_lo, lo, hi)
    code = np.where(a >= E4M3_MAX, 126, code)
    neg = np.signbit(v)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def fp8_quantize_row(x_bits: np.ndarray) -> tuple[np.ndarray, np.float32]:
    """Quantize one 576-element bf16 row to e4m3fn codes plus a float32 scale.

    The pages only say that fp8 rows carry one float32 scale for K and one for
    V ([vLLM-MLA] §缓存的形状) and that the multiply is skipped when the
    scale is 1 ([vLLM-MLA] §写缓存).  Reading used here: per-token scale
    ``s = amax / 448`` (float32 division; ``s = 1`` for an all-zero row) and
    ``code_i = e4m3(x_i / s)`` with an IEEE float32 division per element, so
    the row's largest magnitude maps to 448.
    """
    xf = bf16_bits_to_f64(x_bits).astype(np.float32)
    amax = np.float32(np.max(np.abs(xf))) if xf.size else np.float32(0.0)
    s = np.float32(amax / np.float32(E4M3_MAX))
    if s == 0:
        s = np.float32(1.0)
    q = (xf / s).astype(np.float32)
    return e4m3_encode(q), s


# --- a1: cache write ---------------------------------------------------------
def cache_write(pool: np.ndarray, kv_c_bits: np.ndarray, k_pe_bits: np.ndarray,
                slot_mapping: np.ndarray, kv_dtype: int) -> np.ndarray:
    """Scatter token rows into the paged pool; returns the updated pool.

    [vLLM-MLA] §写缓存: latent and k_pe of token ``t`` land in one row at
    ``slot_mapping[t]``; with 64-token pages the row is page ``slot // 64``,
    offset ``slot % 64``.  Negative slots are padding and are skipped.
    ``pool`` is a uint8 array ``[num_pages, 64, row_bytes]``.
    """
    out = pool.copy()
    rb = out.shape[2]
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        page, off = divmod(int(slot), PAGE_TOKENS)
        row_bits = np.concatenate([np.asarray(kv_c_bits[t], np.uint16),
                                   np.asarray(k_pe_bits[t], np.uint16)])
        if kv_dtype == KV_BF16:
            out[page, off, :] = row_bits.astype("<u2").view(np.uint8)
        else:
            codes, s = fp8_quantize_row(row_bits)
            n = row_bits.size
            out[page, off, :n] = codes
            out[page, off, n:n + 4] = np.array([s], "<f4").view(np.uint8)
            out[page, off, n + 4:n + 8] = np.array([s], "<f4").view(np.uint8)
            assert rb == n + 8
    return out


def encode_rows(rows_bits: np.ndarray, kv_dtype: int) -> np.ndarray:
    """Cache-row bytes for many token rows at once: ``[n, 576]`` bf16 bits ->
    ``[n, row_bytes]`` uint8.  The same definition as :func:`cache_write` applies
    per row (bit copy for bf16; per-row amax scale and e4m3fn codes for fp8),
    written with whole-array NumPy operations so full pools build quickly.
    """
    rows_bits = np.ascontiguousarray(rows_bits, dtype=np.uint16)
    n, e = rows_bits.shape
    if kv_dtype == KV_BF16:
        return rows_bits.astype("<u2").view(np.uint8).reshape(n, 2 * e)
    xf = bf16_bits_to_f64(rows_bits).astype(np.float32)
    amax = np.max(np.abs(xf), axis=1)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    s = np.where(s == 0, np.float32(1.0), s).astype(np.float32)
    q = (xf / s[:, None]).astype(np.float32)
    out = np.empty((n, e + 8), dtype=np.uint8)
    out[:, :e] = e4m3_encode(q)
    sb = s.astype("<f4").view(np.uint8).reshape(n, 4)
    out[:, e:e + 4] = sb
    out[:, e + 4:e + 8] = sb
    return out


def row_views(rows: np.ndarray, kv_dtype: int, row_elems: int = ROW_ELEMS,
              latent: int = KV_LORA_RANK, dtype=np.float64) -> tuple[np.ndarray, np.ndarray]:
    """Decode raw cache rows into the K view (all elements) and V view (latent).

    bf16: both views are the stored values.  fp8: K = code * k_scale over all
    elements, V = code * v_scale over the latent part ([vLLM-MLA] §缓存的形状:
    one scale for K and one for V; the latent doubles as V).
    """
    rows = np.asarray(rows, dtype=np.uint8)
    if kv_dtype == KV_BF16:
        vals = bf16_bits_to_f64(rows.reshape(rows.shape[0], -1).view("<u2")).astype(dtype, copy=False)
        return vals, vals[:, :latent]
    codes = rows[:, :row_elems]
    k_scale = rows[:, row_elems:row_elems + 4].copy().view("<f4").astype(np.float64)
    v_scale = rows[:, row_elems + 4:row_elems + 8].copy().view("<f4").astype(np.float64)
    vals = e4m3_value(codes)
    return (vals * k_scale).astype(dtype, copy=False), (vals[:, :latent] * v_scale).astype(dtype, copy=False)


def gather_rows(pool: np.ndarray, block_table_row: np.ndarray, n: int) -> np.ndarray:
    """Raw rows of logical tokens ``0..n-1`` of one request.

    Token ``j`` lives in physical page ``block_table_row[j // 64]`` at offset
    ``j % 64`` ([vLLM-MLA] §Metadata: block_table; §FlashMLA: paged cache).
    """
    j = np.arange(n)
    pages = np.asarray(block_table_row, dtype=np.int64)[j // PAGE_TOKENS]
    return pool[pages, j % PAGE_TOKENS, :]


# --- a4 + a5: absorbed MQA decode, definition form ---------------------------
def visible_tokens(seq_len: int, q_len: int, t: int) -> int:
    """Tokens seen by query row ``t``: ``seq_len - q_len + 1 + t``, floored at 0.

    [vLLM-MLA] §Triton MLA: multi-token decode adds ``arange(1 - q_len, 1)`` to
    ``seq_lens`` per row and clamps at 0, which is causality within the block.
    """
    return max(0, seq_len - q_len + 1 + t)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float
           ) -> tuple[np.ndarray, np.ndarray]:
    """Textbook softmax attention of query rows ``q[H, D]`` over ``n`` keys.

    ``s = scale * q K^T``, ``lse = m + ln sum exp(s - m)``, ``p = exp(s - lse)``,
    ``o = p V``.  With no keys: ``o = 0``, ``lse = -inf``.
    """
    H = q.shape[0]
    if K.shape[0] == 0:
        return np.zeros((H, V.shape[1]), dtype=q.dtype), np.full(H, -np.inf, dtype=q.dtype)
    s = scale * (q @ K.T)
    m = s.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
    p = np.exp(s - lse[:, None])
    return p @ V, lse


def decode(q: np.ndarray, pool: np.ndarray, kv_dtype: int, block_table: np.ndarray,
           seq_lens: np.ndarray, scale: float, row_elems: int = ROW_ELEMS,
           latent: int = KV_LORA_RANK, dtype=np.float64) -> tuple[np.ndarray, np.ndarray]:
    """Absorbed-MQA decode over the paged cache, as its plain definition.

    ``q`` is ``[B, q_len, N, row_elems]`` (absorbed query ``[q_l,nope | q_pe]``);
    returns ``o[B, q_len, N, latent]`` and ``lse[B, q_len, N]`` (float64).
    Every head scores against the whole row and the latent part is V
    ([vLLM-MLA] §两套算法 data-movement-friendly form; §FlashMLA: one KV head
    shared by all query heads; [Triton-MLA] §Datenfluss).  No splits, no online
    softmax: the gathered keys are attended in one pass.  ``dtype`` float32 runs the
    same definition in single precision (the timed CPU baseline only; parity uses
    float64).
    """
    q = np.asarray(q, dtype=dtype)
    B, q_len, N, _ = q.shape
    o = np.zeros((B, q_len, N, latent), dtype=dtype)
    lse = np.full((B, q_len, N), -np.inf, dtype=dtype)
    for b in range(B):
        n_all = int(seq_lens[b])
        if n_all <= 0:
            continue
        K_all, V_all = row_views(gather_rows(pool, block_table[b], n_all), kv_dtype,
                                 row_elems, latent, dtype)
        for t in range(q_len):
            n = visible_tokens(n_all, q_len, t)
            o[b, t], lse[b, t] = attend(q[b, t], K_all[:n], V_all[:n], dtype(scale))
    return o, lse


def decode_varlen(q: np.ndarray, query_start_loc: np.ndarray, pool: np.ndarray, kv_dtype: int,
                  block_table: np.ndarray, seq_lens: np.ndarray, causal: bool, scale: float,
                  row_elems: int = ROW_ELEMS, latent: int = KV_LORA_RANK) -> tuple[np.ndarray, np.ndarray]:
    """Decode with a different number of query tokens per request.

    [vLLM-MLA] §投机解码 (query 不是 1 时) and §Metadata (QueryLenSupport VARLEN):
    a verification batch mixes requests with 1, 2, 3 ... query tokens; request
    ``b`` owns query rows ``query_start_loc[b] .. query_start_loc[b+1]-1`` of the
    flat ``q[T, N, row_elems]``.  Causal blocks: row ``t`` of the block sees
    ``seq_lens[b] - q_len_b + 1 + t`` tokens (per-row sequence lengths);
    non-causal draft blocks: every row sees all ``seq_lens[b]`` tokens.
    Returns ``o[T, N, latent]``, ``lse[T, N]`` (float64).
    """
    q = np.asarray(q, dtype=np.float64)
    T, N, _ = q.shape
    o = np.zeros((T, N, latent))
    lse = np.full((T, N), -np.inf)
    for b in range(len(seq_lens)):
        r0, r1 = int(query_start_loc[b]), int(query_start_loc[b + 1])
        n_all = int(seq_lens[b])
        if r1 <= r0 or n_all <= 0:
            continue
        K_all, V_all = row_views(gather_rows(pool, block_table[b], n_all), kv_dtype, row_elems, latent)
        for t in range(r1 - r0):
            n = visible_tokens(n_all, r1 - r0, t) if causal else n_all
            o[r0 + t], lse[r0 + t] = attend(q[r0 + t], K_all[:n], V_all[:n], scale)
    return o, lse


def merge(o_parts: np.ndarray, lse_parts: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Combine attention partials over disjoint token sets (axis 0 = part).

    [vLLM-MLA] §Prefill (merge_attn_states): each part is re-weighted by
    ``exp(lse_s - max lse)``; parts with ``lse = -inf`` weigh zero.  Result
    ``o = sum w_s o_s / sum w_s``, ``lse = max + ln sum w_s``; all parts empty
    gives ``o = 0``, ``lse = -inf``.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    safe_m = np.where(np.isfinite(m), m, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - safe_m), 0.0)
    wsum = w.sum(axis=0)
    o = (w[..., None] * o_parts).sum(axis=0) / np.where(wsum > 0, wsum, 1.0)[..., None]
    lse = np.where(wsum > 0, safe_m + np.log(np.where(wsum > 0, wsum, 1.0)), -np.inf)
    return o, lse


# --- a2 / a6: absorption and up-projection ----------------------------------
def absorb(q_nope: np.ndarray, q_pe: np.ndarray | None, w_uk_t: np.ndarray) -> np.ndarray:
    """Absorbed query ``[q_nope . W_UK_T[h] | q_pe]`` per token and head.

    ``q_nope[T, N, P]``, ``W_UK_T[N, P, L]`` ([vLLM-MLA] §权重准备: W_UK is
    permuted to ``[N, P, L]`` so one batched GEMM serves all heads; §两套算法:
    ``q_l,nope = q_nope W_UK^T``); ``q_pe[T, N, R]`` is appended unchanged
    ([TRTLLM-TP] §吸收: the product is written into the front of a
    ``[T, N, L + R]`` fused query).  Returns float64 ``[T, N, L(+R)]``.
    """
    ql = np.einsum("thp,hpl->thl", np.asarray(q_nope, np.float64),
                   np.asarray(w_uk_t, np.float64))
    if q_pe is None:
        return ql
    return np.concatenate([ql, np.asarray(q_pe, np.float64)], axis=-1)


def rope(x_pe: np.ndarray, positions: np.ndarray, cos_sin: np.ndarray, neox: bool) -> np.ndarray:
    """Rotary position embedding of the 64-wide rope part of a query.

    [vLLM-MLA] §从模型层看: the model layer rotates the last ``qk_rope_head_dim``
    query values (and the shared ``k_pe``) by ``rotary_emb(positions, ...)``
    before MLA sees them; [TRTLLM-TP] §吸收 runs that rotation beside the
    absorption GEMM.  The pages give neither the pairing nor the frequencies,
    so the caller supplies both: ``cos_sin[p] = [cos(p w_0..w_31) | sin(...)]``
    (float, ``[max_pos, 64]``) and the pairing, either rotate-half
    (``neox``: value ``i`` pairs with ``i + 32``) or adjacent pairs (value
    ``2i`` with ``2i + 1``).  Pair ``(a, b)`` with frequency ``i`` becomes
    ``(a cos - b sin, b cos + a sin)``.  A row whose position lies outside
    ``[0, max_pos)`` has no defined rotation: it comes back as NaN.

    ``x_pe[T, N, 64]``, ``positions[T]``.  Returns float64 ``[T, N, 64]``.
    """
    x = np.asarray(x_pe, np.float64)
    T, N, R = x.shape
    half = R // 2
    table = np.asarray(cos_sin, np.float64)
    out = np.full_like(x, np.nan)
    for t in range(T):
        p = int(positions[t])
        if p < 0 or p >= table.shape[0]:
            continue
        c, sn = table[p, :half], table[p, half:]
        if neox:
            a, b = x[t, :, :half], x[t, :, half:]
            out[t, :, :half] = a * c - b * sn
            out[t, :, half:] = b * c + a * sn
        else:
            a, b = x[t, :, 0::2], x[t, :, 1::2]
            out[t, :, 0::2] = a * c - b * sn
            out[t, :, 1::2] = b * c + a * sn
    return out


def absorb_rope(q_nope: np.ndarray, q_pe: np.ndarray, w_uk_t: np.ndarray, positions: np.ndarray,
                cos_sin: np.ndarray, neox: bool) -> np.ndarray:
    """:func:`absorb` with the query's rope part rotated on the way into the tail.

    The fused query of [TRTLLM-TP] §吸收 holds ``[q_nope . W_UK_T[h] | RoPE(q_pe)]``;
    the rotation is :func:`rope`.  Returns float64 ``[T, N, L + R]``.
    """
    return np.concatenate([absorb(q_nope, None, w_uk_t), rope(q_pe, positions, cos_sin, neox)], axis=-1)


def up_v(o_lat: np.ndarray, w_uv: np.ndarray) -> np.ndarray:
    """Per-head up-projection ``o_lat[t,h,:] . W_UV[h]`` → ``[T, N, V]``.

    [vLLM-MLA] §两套算法 (_v_up_proj): ``[N, B, L] @ W_UV[N, L, V]`` written
    back token-major.
    """
    return np.einsum("thl,hlv->thv", np.asarray(o_lat, np.float64),
                     np.asarray(w_uv, np.float64))


# --- next to decode: context gather and the two-part state merge ------------
def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns of float64 values, rounded to nearest, ties to even.

    bfloat16 is the top half of an IEEE float32: 8 significant bits down to
    2^-126, then subnormals spaced 2^-133; values that round past the largest
    finite one become infinity; NaN becomes the quiet NaN 0x7FC0 (with the
    input's sign).  The rounding is done on the exact float64 input.
    """
    v = np.asarray(x, dtype=np.float64)
    a = np.abs(v)
    _, e = np.frexp(np.where(np.isfinite(a) & (a > 0), a, 1.0))
    quantum = np.ldexp(1.0, np.maximum(e, -125) - 8)        # 2^(e-8), 2^-133 below 2^-126
    with np.errstate(over="ignore", invalid="ignore"):
        q = np.round(a / quantum) * quantum                  # round half to even
        bits = (q.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(np.isnan(a), np.uint16(0x7FC0), bits)
    bits = np.where(np.isinf(a), np.uint16(0x7F80), bits)
    return (bits | np.where(np.signbit(v), np.uint16(0x8000), np.uint16(0))).astype(np.uint16)


def gather_cache(pool: np.ndarray, kv_dtype: int, block_table: np.ndarray, cu_seq_lens: np.ndarray,
                 token_to_seq: np.ndarray, seq_starts: np.ndarray | None = None,
                 row_elems: int = ROW_ELEMS) -> np.ndarray:
    """Gather context rows from the paged cache into a contiguous bf16 workspace.

    [vLLM-MLA] §Prefill (chunked context): the context rows a chunk needs are
    collected from the paged cache by ``block_table``, ``cu_seq_lens`` and
    ``token_to_seq`` into a contiguous workspace so that ``kv_b_proj`` can run
    as one GEMM; fp8 rows are upconverted to bf16 while gathering; a chunk may
    start part-way into a request, on a page boundary (``seq_starts``).

    Output row ``r`` belongs to request ``b = token_to_seq[r]`` and is that
    request's logical token ``seq_starts[b] + r - cu_seq_lens[b]``.  bf16 rows are
    copied bit for bit; an fp8 row becomes ``code * k_scale`` for all of its
    elements (the row's K view), rounded once to bf16.  Returns uint16 bf16 bit
    patterns ``[len(token_to_seq), row_elems]``.
    """
    pool = np.asarray(pool, dtype=np.uint8)
    total = len(token_to_seq)
    out = np.zeros((total, row_elems), dtype=np.uint16)
    for r in range(total):
        b = int(token_to_seq[r])
        start = 0 if seq_starts is None else int(seq_starts[b])
        j = start + r - int(cu_seq_lens[b])
        raw = pool[int(block_table[b][j // PAGE_TOKENS]), j % PAGE_TOKENS]
        if kv_dtype == KV_BF16:
            out[r] = raw[:2 * row_elems].view("<u2")
        else:
            k_scale = float(raw[row_elems:row_elems + 4].copy().view("<f4")[0])
            out[r] = f64_to_bf16_bits(e4m3_value(raw[:row_elems]) * k_scale)
    return out


def prefill_workspace_rows(max_model_len: int, max_num_seqs: int, page_tokens: int = PAGE_TOKENS) -> int:
    """Row budget W of the chunked-context workspace.

    [vLLM-MLA] §Prefill (determine_chunked_prefill_workspace_size):
    ``W = min(max(8 * L_max, 4 * B_seq * P_block), 64 * 1024)`` -- room for eight
    full-length requests or four pages per concurrent request, capped at 64k rows so
    that the workspace does not crowd out the KV cache.
    """
    return min(max(8 * int(max_model_len), 4 * int(max_num_seqs) * int(page_tokens)), 64 * 1024)


def plan_context_chunks(context_lens, row_budget: int, page_tokens: int = PAGE_TOKENS
                        ) -> list[list[tuple[int, int, int]]]:
    """Pack a prefill batch's context rows into chunks of at most ``row_budget`` rows.

    [vLLM-MLA] §Prefill (plan_mla_context_chunks, align_chunk_to_block): the requests'
    contexts are packed in request order; a request that does not fit in what is left
    of the current chunk is cut on a page boundary and continues in the next chunk, so
    that every chunk starts a request on a block boundary (the gather takes no other
    start).  Returns, per chunk, the ``(request, first token, tokens)`` pieces in order.
    A budget below one page cannot make progress and is rejected.
    """
    if row_budget < page_tokens:
        raise ValueError("row budget below one page")
    chunks: list[list[tuple[int, int, int]]] = []
    cur: list[tuple[int, int, int]] = []
    used = 0
    for b, n in enumerate(context_lens):
        n = max(0, int(n))
        pos = 0
        while pos < n:
            room = row_budget - used
            take = n - pos if n - pos <= room else room // page_tokens * page_tokens
            if take == 0:                      # no whole page left: the next chunk
                chunks.append(cur)
                cur, used = [], 0
                continue
            cur.append((b, pos, take))
            used += take
            pos += take
    if cur:
        chunks.append(cur)
    return chunks


def merge_attn_states(prefix_o: np.ndarray, prefix_lse: np.ndarray, suffix_o: np.ndarray,
                      suffix_lse: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Merge two attention states of the same query rows over disjoint key sets.

    [vLLM-MLA] §Prefill (merge_attn_states): the context-chunk result (prefix)
    and the new-token result (suffix) are re-weighted by ``exp(lse - max_lse)``
    per head and query row; a state with no keys (``o = 0``, ``lse = -inf``)
    weighs zero.  ``o[..., D]`` and ``lse[...]`` share their leading shape;
    returns float64 ``(o, lse)``.  This is :func:`merge` with two parts.
    """
    return merge(np.stack([np.asarray(prefix_o, np.float64), np.asarray(suffix_o, np.float64)]),
                 np.stack([np.asarray(prefix_lse, np.float64), np.asarray(suffix_lse, np.float64)]))


def quantize_groups_fp8(y_bits: np.ndarray, group: int) -> tuple[np.ndarray, np.ndarray]:
    """Per-token-group fp8 quantization of a bf16 output ``[T, C]`` (C % group == 0).

    [vLLM-MLA] §QuantKey: when the layer after MLA wants fp8, the W_UV output is
    quantized dynamically in groups of 128 or 64 consecutive elements of a token,
    one float32 scale per group (kFp8Dynamic128Sym / kFp8Dynamic64Sym).  The
    pages do not give the scale rule; the cache write's rule is used (as in
    :func:`fp8_quantize_row`): ``s = amax / 448`` (float32), ``s = 1`` for an
    all-zero group, ``code = e4m3(x / s)`` with a float32 division.  Returns
    ``codes uint8 [T, C]`` and ``scales float32 [T, C // group]``.
    """
    y = np.asarray(y_bits, dtype=np.uint16)
    T, C = y.shape
    assert C % group == 0
    xf = bf16_bits_to_f64(y).astype(np.float32).reshape(T, C // group, group)
    amax = np.max(np.abs(xf), axis=2)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    s = np.where(s == 0, np.float32(1.0), s).astype(np.float32)
    q = (xf / s[:, :, None]).astype(np.float32)
    return e4m3_encode(q).reshape(T, C), s


# --- prefill of new tokens: kv_b_proj and the 192/128 MHA --------------------
def kv_b_proj(kv_c: np.ndarray, w_kvb: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-head up-projection of latents into the prefill keys and values.

    [vLLM-MLA] §从模型层看 and §两套算法 (compute-friendly form): every latent
    ``kv_c[s]`` becomes ``k_nope[s,h] = kv_c[s] W_UK[h]`` (P values) and
    ``v[s,h] = kv_c[s] W_UV[h]`` (V values); §Prefill: ``kv_b_proj(kv_c)`` gives
    both at once.  ``w_kvb[N, L, P + V]`` holds ``[W_UK[h] | W_UV[h]]`` per head.
    Returns float64 ``k_nope[S, N, P]`` and ``v[S, N, V]``.
    """
    out = np.einsum("sl,hlc->shc", np.asarray(kv_c, np.float64), np.asarray(w_kvb, np.float64))
    return out[..., :QK_NOPE_DIM], out[..., QK_NOPE_DIM:]


def prefill_mha(q: np.ndarray, k_nope: np.ndarray, k_pe: np.ndarray, v: np.ndarray,
                cu_q: np.ndarray, cu_k: np.ndarray, scale: float, causal: bool
                ) -> tuple[np.ndarray, np.ndarray]:
    """Multi-head attention of a prefill batch with 192-wide keys and 128-wide values.

    [vLLM-MLA] §Prefill (run_prefill_new_tokens): the key of token ``s`` for head
    ``h`` is ``[k_nope[s,h] | k_pe[s]]`` (the single rope key broadcast to every
    head), the value ``v[s,h]``; the softmax scale is ``1/sqrt(192)``.  Request
    ``b`` owns query rows ``cu_q[b] .. cu_q[b+1]-1`` and keys
    ``cu_k[b] .. cu_k[b+1]-1``; with ``causal`` its query row ``i`` is the token
    at position ``klen - qlen + i`` and sees keys ``0 .. klen - qlen + i`` (the
    new tokens come after the request's context).  Returns ``out[T, N, V]`` and
    the natural-log ``lse[T, N]`` (``o = 0``, ``lse = -inf`` for a row that sees
    no key), the pair :func:`merge_attn_states` combines with a context part.
    """
    q = np.asarray(q, np.float64)
    kn, kp, vv = (np.asarray(a, np.float64) for a in (k_nope, k_pe, v))
    T, N, _ = q.shape
    out = np.zeros((T, N, vv.shape[-1]))
    lse = np.full((T, N), -np.inf)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        qlen, klen = q1 - q0, k1 - k0
        for i in range(qlen):
            nvis = klen - qlen + i + 1 if causal else klen
            nvis = max(0, min(klen, nvis))
            if nvis == 0:
                continue
            for h in range(N):
                K = np.concatenate([kn[k0:k0 + nvis, h], kp[k0:k0 + nvis]], axis=-1)
                o, l = attend(q[q0 + i, h][None, :], K, vv[k0:k0 + nvis, h], scale)
                out[q0 + i, h], lse[q0 + i, h] = o[0], l[0]
    return out, lse


# --- the un-absorbed oracle --------------------------------------------------
def mla_unabsorbed(q_nope: np.ndarray, q_pe: np.ndarray, pool: np.ndarray, kv_dtype: int,
                   block_table: np.ndarray, seq_lens: np.ndarray, w_uk_t: np.ndarray,
                   w_uv: np.ndarray, scale: float, heads: list[int] | None = None,
                   batches: list[int] | None = None, row_elems: int = ROW_ELEMS,
                   latent: int = KV_LORA_RANK) -> tuple[np.ndarray, np.ndarray]:
    """MLA attention computed the compute-friendly way, with no absorption.

    Every visible cached latent is up-projected per head to
    ``k_nope = W_UK[h] c`` (P values) and ``v = c W_UV[h]`` (V values); the key
    is ``[k_nope, k_pe]`` with the single rope key broadcast to all heads, and
    plain softmax attention runs with the 192-wide query ``[q_nope, q_pe]``
    ([vLLM-MLA] §从模型层看 decoupled RoPE, §两套算法 compute-friendly form).
    For fp8 rows the latent's K view uses ``k_scale`` and its V view
    ``v_scale``.

    ``q_nope[B, q_len, N, P]``, ``q_pe[B, q_len, N, R]``.  Returns
    ``y[B, q_len, N, V]`` and ``lse[B, q_len, N]`` (NaN where not computed when
    ``heads``/``batches`` restrict the work).
    """
    q_nope = np.asarray(q_nope, np.float64)
    q_pe = np.asarray(q_pe, np.float64)
    wk = np.asarray(w_uk_t, np.float64)
    wv = np.asarray(w_uv, np.float64)
    B, q_len, N, _ = q_nope.shape
    Vd = wv.shape[2]
    heads = list(range(N)) if heads is None else heads
    batches = list(range(B)) if batches is None else batches
    y = np.full((B, q_len, N, Vd), np.nan)
    lse = np.full((B, q_len, N), np.nan)
    for b in batches:
        n_all = max(0, int(seq_lens[b]))
        Kv, Vv = row_views(gather_rows(pool, block_table[b], n_all), kv_dtype, row_elems, latent) \
            if n_all > 0 else (np.zeros((0, row_elems)), np.zeros((0, latent)))
        c_k, k_pe = Kv[:, :latent], Kv[:, latent:]
        for h in heads:
            k_nope = c_k @ wk[h].T          # [n, P]
            v = Vv @ wv[h]                  # [n, V]
            K = np.concatenate([k_nope, k_pe], axis=1)
            for t in range(q_len):
                n = visible_tokens(n_all, q_len, t)
                qh = np.concatenate([q_nope[b, t, h], q_pe[b, t, h]])[None, :]
                o, l = attend(qh, K[:n], v[:n], scale)
                y[b, t, h], lse[b, t, h] = o[0], l[0]
    return y, lse


# --- byte arithmetic used as printed pins ------------------------------------
def mha_row_bytes(num_heads: int = 128, qk_dim: int = 192, v_dim: int = 128,
                  elem_bytes: int = 2) -> int:
    """Per-token per-layer bytes of an un-compressed MHA cache: ``N (QK + V)``."""
    return num_heads * (qk_dim + v_dim) * elem_bytes


def page_bytes(kv_dtype: int) -> int:
    """Bytes of one 64-token page of one layer."""
    return PAGE_TOKENS * row_bytes(kv_dtype)


def request_bytes(seq_len: int, layers: int, kv_dtype: int) -> int:
    """Cache bytes of one request across ``layers`` layers."""
    return seq_len * layers * row_bytes(kv_dtype)


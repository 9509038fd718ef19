"""Seeded synthetic inputs for MLA paged-latent decode.

This module holds only random draws and their packing into arrays: no step of
the method (no cache write, no quantization, no attention arithmetic).  Both the
HIP path's tests/bench and the CPU oracle consume what it produces.

Shapes follow DeepSeek-V3's MLA (kv_lora_rank 512, rope 64, qk_nope 128,
v_head 128, 64-token pages) as described on the source page "vLLM 源码完全拆解
(三十七):MLA 注意力后端" (§从模型层看, §缓存的形状).  The named workloads are:

* ``tiny``      B=2, q_len=1, N=16, seq {37, 100}, 16-page pool, bf16, with the
                absorption weights.
* ``tp_share``  B=64, q_len=1, N=16, seq ~ U{1024..4096}, 8192-page pool, bf16,
                absorbed query given directly.
* ``full_head`` B=32, q_len=1, N=128, seq 8192 each, 8192-page pool, bf16, with
                the absorption weights W_UK_T[128,128,512] and W_UV[128,512,128].
* ``fp8``       B=128, q_len=1, N=128, seq lognormal (median 2048, sigma 1.0,
                clipped to [64, 32768]), pool max(8192, 1.25 x needed), fp8 rows.
* ``spec_long`` B=8, q_len=2, N=128, seq {131072, 65536, ..., 1024},
                pool 1.25 x 4080 pages, bf16.

Every value is drawn N(0, 1) except the weights, N(0, 1/512) (variance), and
rounded to bfloat16 (round to nearest even) so that both sides see identical
bits.  Seeds are ``20260 + index``.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

L, R, P, V = 512, 64, 128, 128
ROW = L + R
PAGE = 64
KV_BF16, KV_FP8 = 0, 1


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 draws to bfloat16 bit patterns (nearest, ties to even)."""
    # finite inputs only: u + 0x8000 cannot wrap for any finite float32 pattern
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    q_len: int
    N: int
    kv_dtype: int
    num_pages: int
    seq_lens: np.ndarray          # int32 [B]
    block_table: np.ndarray       # int32 [B, max_pages], -1 past the used pages
    kv_rows: np.ndarray           # uint16 bf16 bits [num_pages, 64, 576]: source row of every slot
    new_slots: np.ndarray         # int64 [B*q_len]: slots of the step's new tokens
    new_rows: np.ndarray          # uint16 bf16 bits [B*q_len, 576]: the step's new token rows
    q: np.ndarray | None          # uint16 bf16 bits [B, q_len, N, 576] absorbed query
    q_nope: np.ndarray | None     # uint16 [B, q_len, N, 128]
    q_pe: np.ndarray | None       # uint16 [B, q_len, N, 64]
    w_uk_t: np.ndarray | None     # uint16 [N, 128, 512]
    w_uv: np.ndarray | None       # uint16 [N, 512, 128]
    seed: int

    @property
    def tokens(self) -> int:
        return int(self.seq_lens.astype(np.int64).sum())

    @property
    def max_pages(self) -> int:
        return self.block_table.shape[1]


def _normal_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return to_bf16_bits(x)


def make_workload(name: str, B: int, q_len: int, N: int, seq_lens, num_pages: int | None,
                  kv_dtype: int, with_weights: bool, seed: int, pool_factor: float = 1.25,
                  min_pool: int = 0) -> Workload:
    """Draw one synthetic decode batch.

    Pages are placed at random: a random permutation of the pool is dealt out to
    the requests in order, so logically adjacent pages are physically scattered.
    Block-table entries past a request's last page are -1.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    seq = np.asarray(seq_lens, dtype=np.int64)
    assert seq.shape == (B,)
    pages_per = (seq + PAGE - 1) // PAGE
    need = int(pages_per.sum())
    if num_pages is None:
        num_pages = max(min_pool, int(math.ceil(pool_factor * need)))
    assert num_pages >= need, "pool too small"
    max_pages = max(1, int(pages_per.max()))
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = np.full((B, max_pages), -1, dtype=np.int32)
    cur = 0
    for b in range(B):
        n = int(pages_per[b])
        bt[b, :n] = perm[cur:cur + n]
        cur += n
    kv_rows = _normal_bf16(rng, (num_pages, PAGE, ROW))
    T = B * q_len
    new_rows = _normal_bf16(rng, (T, ROW))
    new_slots = np.full(T, -1, dtype=np.int64)
    for b in range(B):
        for t in range(q_len):
            pos = int(seq[b]) - q_len + t
            if pos >= 0:
                new_slots[b * q_len + t] = int(bt[b, pos // PAGE]) * PAGE + pos % PAGE
    q = q_nope = q_pe = w_uk_t = w_uv = None
    if with_weights:
        q_nope = _normal_bf16(rng, (B, q_len, N, P))
        q_pe = _normal_bf16(rng, (B, q_len, N, R))
        w_uk_t = _normal_bf16(rng, (N, P, L), std=1.0 / math.sqrt(512.0))
        w_uv = _normal_bf16(rng, (N, L, V), std=1.0 / math.sqrt(512.0))
    else:
        q = _normal_bf16(rng, (B, q_len, N, ROW))
    return Workload(name, B, q_len, N, kv_dtype, num_pages, seq.astype(np.int32), bt,
                    kv_rows, new_slots, new_rows, q, q_nope, q_pe, w_uk_t, w_uv, seed)


def tiny() -> Workload:
    return make_workload("tiny", 2, 1, 16, [37, 100], 16, KV_BF16, True, 20260)


def tp_share() -> Workload:
    rng = np.random.Generator(np.random.PCG64(20261 + 1000))
    seq = rng.integers(1024, 4096, size=64, endpoint=True)
    return make_workload("tp_share", 64, 1, 16, seq, 8192, KV_BF16, False, 20261)


def full_head() -> Workload:
    return make_workload("full_head", 32, 1, 128, [8192] * 32, 8192, KV_BF16, True, 20262)


def fp8() -> Workload:
    rng = np.random.Generator(np.random.PCG64(20263 + 1000))
    seq = np.clip(np.rint(np.exp(rng.normal(math.log(2048.0), 1.0, size=128))), 64, 32768)
    return make_workload("fp8", 128, 1, 128, seq.astype(np.int64), None, KV_FP8, False, 20263,
                         min_pool=8192)


def spec_long() -> Workload:
    seq = [131072, 65536, 32768, 16384, 8192, 4096, 2048, 1024]
    return make_workload("spec_long", 8, 2, 128, seq, int(math.ceil(1.25 * 4080)), KV_BF16,
                         False, 20264)


CONFIGS = {"tiny": tiny, "tp_share": tp_share, "full_head": full_head, "fp8": fp8,
           "spec_long": spec_long}


def random_fp8_rows(rng: np.random.Generator, n_rows: int, max_code_exp: int = 8,
                    scale_lo: float = 0.25, scale_hi: float = 4.0) -> np.ndarray:
    """Raw fp8 cache rows with random codes and independent random K/V scales.

    Codes are drawn with exponent field <= ``max_code_exp`` (never NaN); the
    two float32 scales are drawn independently, so K and V dequantize
    differently.  Returns uint8 ``[n_rows, 584]``.
    """
    sign = rng.integers(0, 2, size=(n_rows, ROW)) << 7
    e = rng.integers(0, max_code_exp + 1, size=(n_rows, ROW)) << 3
    m = rng.integers(0, 8, size=(n_rows, ROW))
    codes = (sign | e | m).astype(np.uint8)
    ks = rng.uniform(scale_lo, scale_hi, size=n_rows).astype("<f4")
    vs = rng.uniform(scale_lo, scale_hi, size=n_rows).astype("<f4")
    rows = np.empty((n_rows, ROW + 8), dtype=np.uint8)
    rows[:, :ROW] = codes
    rows[:, ROW:ROW + 4] = ks.view(np.uint8).reshape(n_rows, 4)
    rows[:, ROW + 4:] = vs.view(np.uint8).reshape(n_rows, 4)
    return rows


@dataclasses.dataclass
class ContextChunk:
    """One chunk of prefill context to gather: which tokens of which requests."""
    block_table: np.ndarray       # int32 [B, max_pages], -1 past the used pages
    cu_seq_lens: np.ndarray       # int32 [B + 1]: output row offsets
    seq_starts: np.ndarray        # int32 [B]: first token of each request in the chunk (page-aligned)
    token_to_seq: np.ndarray      # int32 [total]
    num_pages: int

    @property
    def total(self) -> int:
        return int(self.cu_seq_lens[-1])


def make_context_chunk(chunk_lens, chunk_starts, num_pages: int, seed: int) -> ContextChunk:
    """A chunk of context rows: request b contributes ``chunk_lens[b]`` tokens
    starting at its token ``chunk_starts[b]`` (a multiple of 64).  The requests'
    pages (enough to cover start + length) are dealt from a random permutation of
    the pool, as in :func:`make_workload`."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = np.asarray(chunk_lens, dtype=np.int64)
    starts = np.asarray(chunk_starts, dtype=np.int64)
    assert np.all(starts % PAGE == 0)
    pages_per = (starts + lens + PAGE - 1) // PAGE
    assert int(pages_per.sum()) <= num_pages, "pool too small"
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = np.full((len(lens), max(1, int(pages_per.max()))), -1, dtype=np.int32)
    cur = 0
    for b, n in enumerate(pages_per):
        bt[b, :n] = perm[cur:cur + n]
        cur += int(n)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    t2s = np.repeat(np.arange(len(lens)), lens).astype(np.int32)
    return ContextChunk(bt, cu, starts.astype(np.int32), t2s, num_pages)


def random_attn_states(T: int, N: int, D: int, seed: int, empty_frac: float = 0.1):
    """Two attention states (prefix, suffix) of the same ``T x N`` query rows:
    outputs bf16 bits ``[T, N, D]`` ~ N(0, 1), LSEs float32 ~ N(0, 3^2); a fraction
    of rows is empty on one side or both (``o = 0``, ``lse = -inf``)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    po = _normal_bf16(rng, (T, N, D))
    so = _normal_bf16(rng, (T, N, D))
    pl = (rng.standard_normal((T, N)) * 3.0).astype(np.float32)
    sl = (rng.standard_normal((T, N)) * 3.0).astype(np.float32)
    for o, l in ((po, pl), (so, sl)):
        empty = rng.random((T, N)) < empty_frac
        o[empty] = 0
        l[empty] = -np.inf
    return po, pl, so, sl


def rope_cos_sin(max_pos: int, base: float = 10000.0, rope_dim: int = R) -> np.ndarray:
    """A rotary table ``[max_pos, rope_dim]`` in float32: ``cos(p w_i)`` for the
    ``rope_dim / 2`` frequencies ``w_i = base^(-2i / rope_dim)``, then ``sin(p w_i)``.

    This is the caller-side table the rope-fused absorption takes as input (the
    usual geometric frequencies; the pages leave the schedule to the model).
    """
    half = rope_dim // 2
    w = base ** (-np.arange(half, dtype=np.float64) * 2.0 / rope_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * w[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


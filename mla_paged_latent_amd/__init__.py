"""MI355X (gfx950) MLA paged-latent decode: thin Python binding over the C ABI.

Every step of the path runs in the HIP library ``libmla_paged_latent.so`` built
from ``mla_paged_latent_amd/csrc``; this module only marshals torch tensors into
pointers, strides and the current HIP stream, and allocates outputs/workspace
when the caller does not pass them.  There is no CPU fallback: if the library is
missing, :func:`lib` raises.

The calls mirror ``include/mla.h``: :func:`cache_write`, :func:`absorb_q`,
:func:`decode` and :func:`up_v`, plus :func:`decode_workspace_size`, the
variable-query-length decode :func:`decode_varlen`, and the two
steps either side of decode in chunked prefill, :func:`gather_cache` and
:func:`merge_attn_states`.
"""

from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla_paged_latent.so")

KV_BF16 = 0
KV_FP8 = 1
KV_LORA_RANK = 512
ROPE_DIM = 64
ROW_ELEMS = 576
PAGE_TOKENS = 64
ROW_BYTES = {KV_BF16: 1152, KV_FP8: 584}
DEFAULT_SCALE = 192 ** -0.5

_STATUS = {0: "MLA_OK", 1: "MLA_ERR_NULL", 2: "MLA_ERR_SHAPE", 3: "MLA_ERR_DTYPE",
           4: "MLA_ERR_ALIGN", 5: "MLA_ERR_WORKSPACE", 6: "MLA_ERR_HIP", 7: "MLA_ERR_DEVICE"}

_lib = None


class MLAError(RuntimeError):
    def __init__(self, call: str, status: int):
        self.status = status
        super().__init__(f"{call} failed: {_STATUS.get(status, status)} ({lib().mla_status_str(status).decode()})")


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} not found: build it with `python -m mla_paged_latent_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    L.mla_cache_write.argtypes = [vp, i64, vp, i64, vp, i64, vp, i32, i64, vp]
    L.mla_cache_write.restype = i32
    L.mla_absorb_q.argtypes = [vp, i64, i64, vp, i64, i64, vp, i64, i32, vp, i64, i64, vp]
    L.mla_absorb_q.restype = i32
    L.mla_absorb_q_cache_write.argtypes = [vp, i64, i64, vp, i64, i64, vp, i64, i32, vp, i64, i64,
                                           vp, i64, vp, i64, vp, i64, vp, i32, i64, vp]
    L.mla_absorb_q_cache_write.restype = i32
    L.mla_decode_workspace_size.argtypes = [i32, i32, i32, i32]
    L.mla_decode_workspace_size.restype = ctypes.c_size_t
    L.mla_decode.argtypes = [vp, i64, i64, i64, vp, i32, i64, vp, i64, i32, vp, i32, i32, i32,
                             ctypes.c_float, i32, vp, ctypes.c_size_t, vp, i64, i64, i64, vp, vp]
    L.mla_decode.restype = i32
    L.mla_decode_noalloc.argtypes = [vp, i64, i64, i64, vp, i32, i64, vp, i64, i32, vp, i32, i32, i32,
                                     ctypes.c_float, i32, vp, i64, i64, i64, vp, vp]
    L.mla_decode_noalloc.restype = i32
    L.mla_up_v.argtypes = [vp, i64, i64, vp, i64, i32, vp, i64, vp]
    L.mla_up_v.restype = i32
    L.mla_absorb_q_rope.argtypes = [vp, i64, i64, vp, i64, i64, vp, i64, i32, vp, vp, i64, i32, vp, i64,
                                    i64, vp]
    L.mla_absorb_q_rope.restype = i32
    L.mla_kv_b_proj.argtypes = [vp, i64, vp, i64, i32, vp, i64, i64, vp]
    L.mla_kv_b_proj.restype = i32
    L.mla_prefill_mha.argtypes = [vp, i64, i64, vp, i64, i64, vp, i64, vp, i64, i64, vp, vp, i32, i64, i64,
                                  i32, i32, i32, ctypes.c_float, vp, i64, i64, vp, vp]
    L.mla_prefill_mha.restype = i32
    L.mla_up_v_fp8.argtypes = [vp, i64, i64, vp, i64, i32, i32, vp, i64, vp, i64, vp]
    L.mla_up_v_fp8.restype = i32
    L.mla_decode_varlen_workspace_size.argtypes = [i64, i32, i32, i32]
    L.mla_decode_varlen_workspace_size.restype = ctypes.c_size_t
    L.mla_decode_varlen.argtypes = [vp, i64, i64, vp, i32, i64, vp, i64, i32, vp, vp, i32, i64, i32, i32,
                                    ctypes.c_float, i32, vp, ctypes.c_size_t, vp, i64, i64, vp, vp]
    L.mla_decode_varlen.restype = i32
    L.mla_gather_cache.argtypes = [vp, i32, i64, vp, i64, i32, vp, vp, vp, i32, i64, vp, i64, vp]
    L.mla_gather_cache.restype = i32
    L.mla_merge_attn_states.argtypes = [vp, vp, vp, vp, i64, i32, i32, i64, i64, i64, i64, vp, vp, vp]
    L.mla_merge_attn_states.restype = i32
    L.mla_prefill_workspace_rows.argtypes = [i64, i64, i32]
    L.mla_prefill_workspace_rows.restype = i64
    L.mla_plan_context_chunks.argtypes = [vp, i32, i64, vp, vp, i64]
    L.mla_plan_context_chunks.restype = i64
    L.mla_status_str.argtypes = [i32]
    L.mla_status_str.restype = ctypes.c_char_p
    _lib = L
    return L


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(call: str, status: int):
    if status != 0:
        raise MLAError(call, status)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _need_out(call: str, out: torch.Tensor, shape: tuple) -> None:
    """A caller-supplied output: bf16 of exactly ``shape`` with a contiguous last dim
    (the C call writes bf16 rows at the tensor's strides)."""
    if out.dtype != torch.bfloat16 or tuple(out.shape) != tuple(shape) or out.stride(-1) != 1:
        raise ValueError(f"{call}: out must be bfloat16 {tuple(shape)} with a contiguous last dim, got "
                         f"{out.dtype} {tuple(out.shape)} strides {out.stride()}")


def _need_lse(call: str, lse: torch.Tensor, shape: tuple) -> None:
    """A caller-supplied LSE: contiguous float32 of exactly ``shape`` (the C call
    writes it densely, without strides)."""
    if lse.dtype != torch.float32 or tuple(lse.shape) != tuple(shape) or not lse.is_contiguous():
        raise ValueError(f"{call}: lse must be contiguous float32 {tuple(shape)}, got "
                         f"{lse.dtype} {tuple(lse.shape)} strides {lse.stride()}")


def cache_write(kv_c: torch.Tensor, k_pe: torch.Tensor, slot_mapping: torch.Tensor,
                kv_cache: torch.Tensor, kv_dtype: int, stream=None) -> None:
    """Scatter rows ``[kv_c | k_pe]`` into ``kv_cache`` at ``slot_mapping`` (see mla.h).

    ``kv_c`` bf16 ``[T, 512]``, ``k_pe`` bf16 ``[T, 64]`` or ``[T, 1, 64]``,
    ``slot_mapping`` int64 ``[T]``, ``kv_cache`` the page pool (any dtype; its
    byte size gives the page count).
    """
    k_pe = k_pe.reshape(k_pe.shape[0], -1)
    assert kv_c.dtype == torch.bfloat16 and k_pe.dtype == torch.bfloat16
    assert slot_mapping.dtype == torch.int64 and kv_c.stride(-1) == 1 and k_pe.stride(-1) == 1
    T = kv_c.shape[0]
    num_pages = kv_cache.numel() * kv_cache.element_size() // (PAGE_TOKENS * ROW_BYTES[kv_dtype])
    _check("mla_cache_write", lib().mla_cache_write(
        _ptr(kv_c), kv_c.stride(0), _ptr(k_pe), k_pe.stride(0), _ptr(slot_mapping), T,
        _ptr(kv_cache), kv_dtype, num_pages, _stream(stream)))


def absorb_q(q_nope: torch.Tensor, q_pe: torch.Tensor | None, w_uk_t: torch.Tensor,
             q_fused: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """``q_fused[t,h] = [q_nope[t,h] . W_UK_T[h] | q_pe[t,h]]`` (bf16 ``[T, N, 576]``)."""
    T, N, P = q_nope.shape
    assert P == 128 and q_nope.dtype == torch.bfloat16 and w_uk_t.is_contiguous()
    assert w_uk_t.shape == (N, 128, KV_LORA_RANK) and w_uk_t.dtype == torch.bfloat16
    width = ROW_ELEMS if q_pe is not None else KV_LORA_RANK
    if q_fused is None:
        q_fused = torch.empty((T, N, width), dtype=torch.bfloat16, device=q_nope.device)
    qp_st = q_pe.stride(0) if q_pe is not None else 0
    qp_sh = q_pe.stride(1) if q_pe is not None else 0
    _check("mla_absorb_q", lib().mla_absorb_q(
        _ptr(q_nope), q_nope.stride(0), q_nope.stride(1), _ptr(q_pe), qp_st, qp_sh,
        _ptr(w_uk_t), T, N, _ptr(q_fused), q_fused.stride(0), q_fused.stride(1), _stream(stream)))
    return q_fused


def absorb_q_cache_write(q_nope: torch.Tensor, q_pe: torch.Tensor | None, w_uk_t: torch.Tensor,
                         kv_c: torch.Tensor, k_pe: torch.Tensor, slot_mapping: torch.Tensor,
                         kv_cache: torch.Tensor, kv_dtype: int, q_fused: torch.Tensor | None = None,
                         stream=None) -> torch.Tensor:
    """:func:`absorb_q` and :func:`cache_write` in one launch (same arguments, same
    results); returns ``q_fused``."""
    T, N, P = q_nope.shape
    assert P == 128 and q_nope.dtype == torch.bfloat16 and w_uk_t.is_contiguous()
    assert w_uk_t.shape == (N, 128, KV_LORA_RANK) and w_uk_t.dtype == torch.bfloat16
    k_pe = k_pe.reshape(k_pe.shape[0], -1)
    assert kv_c.dtype == torch.bfloat16 and k_pe.dtype == torch.bfloat16
    assert slot_mapping.dtype == torch.int64 and kv_c.stride(-1) == 1 and k_pe.stride(-1) == 1
    width = ROW_ELEMS if q_pe is not None else KV_LORA_RANK
    if q_fused is None:
        q_fused = torch.empty((T, N, width), dtype=torch.bfloat16, device=q_nope.device)
    qp_st = q_pe.stride(0) if q_pe is not None else 0
    qp_sh = q_pe.stride(1) if q_pe is not None else 0
    num_pages = kv_cache.numel() * kv_cache.element_size() // (PAGE_TOKENS * ROW_BYTES[kv_dtype])
    _check("mla_absorb_q_cache_write", lib().mla_absorb_q_cache_write(
        _ptr(q_nope), q_nope.stride(0), q_nope.stride(1), _ptr(q_pe), qp_st, qp_sh,
        _ptr(w_uk_t), T, N, _ptr(q_fused), q_fused.stride(0), q_fused.stride(1),
        _ptr(kv_c), kv_c.stride(0), _ptr(k_pe), k_pe.stride(0), _ptr(slot_mapping), kv_c.shape[0],
        _ptr(kv_cache), kv_dtype, num_pages, _stream(stream)))
    return q_fused


def absorb_q_rope(q_nope: torch.Tensor, q_pe: torch.Tensor, w_uk_t: torch.Tensor,
                  positions: torch.Tensor, cos_sin_cache: torch.Tensor, neox: bool = True,
                  q_fused: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """``q_fused[t,h] = [q_nope[t,h] . W_UK_T[h] | RoPE(q_pe[t,h], positions[t])]``.

    ``positions`` int64 ``[T]``; ``cos_sin_cache`` float32 ``[max_pos, 64]``
    (cos of the 32 frequencies, then sin); ``neox`` picks rotate-half pairing,
    else adjacent pairs.
    """
    T, N, P = q_nope.shape
    assert P == 128 and q_nope.dtype == torch.bfloat16 and w_uk_t.is_contiguous()
    assert w_uk_t.shape == (N, 128, KV_LORA_RANK) and w_uk_t.dtype == torch.bfloat16
    assert q_pe.shape == (T, N, 64) and q_pe.stride(-1) == 1
    assert positions.dtype == torch.int64 and positions.is_contiguous() and positions.numel() == T
    assert cos_sin_cache.dtype == torch.float32 and cos_sin_cache.is_contiguous()
    assert cos_sin_cache.dim() == 2 and cos_sin_cache.shape[1] == 64
    if q_fused is None:
        q_fused = torch.empty((T, N, ROW_ELEMS), dtype=torch.bfloat16, device=q_nope.device)
    _check("mla_absorb_q_rope", lib().mla_absorb_q_rope(
        _ptr(q_nope), q_nope.stride(0), q_nope.stride(1), _ptr(q_pe), q_pe.stride(0), q_pe.stride(1),
        _ptr(w_uk_t), T, N, _ptr(positions), _ptr(cos_sin_cache), cos_sin_cache.shape[0],
        1 if neox else 0, _ptr(q_fused), q_fused.stride(0), q_fused.stride(1), _stream(stream)))
    return q_fused


def decode_workspace_size(B: int, q_len: int, N: int, num_splits: int = 0) -> int:
    return int(lib().mla_decode_workspace_size(B, q_len, N, num_splits))


def decode(q: torch.Tensor, kv_cache: torch.Tensor, kv_dtype: int, block_table: torch.Tensor,
           seq_lens: torch.Tensor, softmax_scale: float = DEFAULT_SCALE, num_splits: int = 0,
           workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
           lse: torch.Tensor | None = None, stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """Absorbed-MQA decode over the paged cache.

    ``q`` bf16 ``[B, q_len, N, 576]``; ``block_table`` int32 ``[B, max_pages]``;
    ``seq_lens`` int32 ``[B]``.  Returns ``out`` bf16 ``[B, q_len, N, 512]`` and
    ``lse`` float32 ``[B, q_len, N]``.
    """
    B, q_len, N, D = q.shape
    assert D == ROW_ELEMS and q.dtype == torch.bfloat16 and q.stride(-1) == 1
    assert block_table.dtype == torch.int32 and seq_lens.dtype == torch.int32
    assert block_table.stride(-1) == 1
    num_pages = kv_cache.numel() * kv_cache.element_size() // (PAGE_TOKENS * ROW_BYTES[kv_dtype])
    if out is None:
        out = torch.empty((B, q_len, N, KV_LORA_RANK), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, q_len, N), dtype=torch.float32, device=q.device)
    _need_out("decode", out, (B, q_len, N, KV_LORA_RANK))
    _need_lse("decode", lse, (B, q_len, N))
    need = decode_workspace_size(B, q_len, N, num_splits)
    if need == 0:
        raise MLAError("mla_decode_workspace_size", 2)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check("mla_decode", lib().mla_decode(
        _ptr(q), q.stride(0), q.stride(1), q.stride(2), _ptr(kv_cache), kv_dtype, num_pages,
        _ptr(block_table), block_table.stride(0), block_table.shape[1], _ptr(seq_lens),
        B, q_len, N, float(softmax_scale), num_splits, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), out.stride(0), out.stride(1),
        out.stride(2), _ptr(lse), _stream(stream)))
    return out, lse


def decode_noalloc(q: torch.Tensor, kv_cache: torch.Tensor, kv_dtype: int, block_table: torch.Tensor,
                   seq_lens: torch.Tensor, softmax_scale: float = DEFAULT_SCALE, num_splits: int = 0,
                   out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                   stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """:func:`decode` through ``mla_decode_noalloc``: no workspace, the library's
    per-GPU scratch array instead (calls that overlap on one GPU race)."""
    B, q_len, N, D = q.shape
    assert D == ROW_ELEMS and q.dtype == torch.bfloat16 and q.stride(-1) == 1
    assert block_table.dtype == torch.int32 and seq_lens.dtype == torch.int32
    assert block_table.stride(-1) == 1
    num_pages = kv_cache.numel() * kv_cache.element_size() // (PAGE_TOKENS * ROW_BYTES[kv_dtype])
    if out is None:
        out = torch.empty((B, q_len, N, KV_LORA_RANK), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, q_len, N), dtype=torch.float32, device=q.device)
    _need_out("decode_noalloc", out, (B, q_len, N, KV_LORA_RANK))
    _need_lse("decode_noalloc", lse, (B, q_len, N))
    _check("mla_decode_noalloc", lib().mla_decode_noalloc(
        _ptr(q), q.stride(0), q.stride(1), q.stride(2), _ptr(kv_cache), kv_dtype, num_pages,
        _ptr(block_table), block_table.stride(0), block_table.shape[1], _ptr(seq_lens),
        B, q_len, N, float(softmax_scale), num_splits, _ptr(out), out.stride(0), out.stride(1),
        out.stride(2), _ptr(lse), _stream(stream)))
    return out, lse


def up_v(o_lat: torch.Tensor, w_uv: torch.Tensor, out: torch.Tensor | None = None,
         stream=None) -> torch.Tensor:
    """``out[t, h*128:(h+1)*128] = o_lat[t,h] . W_UV[h]`` (bf16 ``[T, N*128]``)."""
    T, N, Lr = o_lat.shape
    assert Lr == KV_LORA_RANK and o_lat.dtype == torch.bfloat16 and o_lat.stride(-1) == 1
    assert w_uv.shape == (N, KV_LORA_RANK, 128) and w_uv.is_contiguous()
    if out is None:
        out = torch.empty((T, N * 128), dtype=torch.bfloat16, device=o_lat.device)
    _check("mla_up_v", lib().mla_up_v(
        _ptr(o_lat), o_lat.stride(0), o_lat.stride(1), _ptr(w_uv), T, N, _ptr(out),
        out.stride(0), _stream(stream)))
    return out


def up_v_fp8(o_lat: torch.Tensor, w_uv: torch.Tensor, group: int = 128,
             out_codes: torch.Tensor | None = None, out_scales: torch.Tensor | None = None,
             stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """:func:`up_v` quantized to fp8 per token group of ``group`` (64 or 128) values.

    Returns ``codes`` uint8 ``[T, N*128]`` (e4m3fn) and ``scales`` float32
    ``[T, N*128 // group]``.
    """
    T, N, Lr = o_lat.shape
    assert Lr == KV_LORA_RANK and o_lat.dtype == torch.bfloat16 and o_lat.stride(-1) == 1
    assert w_uv.shape == (N, KV_LORA_RANK, 128) and w_uv.is_contiguous()
    if out_codes is None:
        out_codes = torch.empty((T, N * 128), dtype=torch.uint8, device=o_lat.device)
    if out_scales is None:
        out_scales = torch.empty((T, N * 128 // group), dtype=torch.float32, device=o_lat.device)
    assert out_codes.dtype == torch.uint8 and out_codes.stride(-1) == 1
    assert out_scales.dtype == torch.float32 and out_scales.stride(-1) == 1
    _check("mla_up_v_fp8", lib().mla_up_v_fp8(
        _ptr(o_lat), o_lat.stride(0), o_lat.stride(1), _ptr(w_uv), T, N, group, _ptr(out_codes),
        out_codes.stride(0), _ptr(out_scales), out_scales.stride(0), _stream(stream)))
    return out_codes, out_scales


def kv_b_proj(kv_c: torch.Tensor, w_kvb: torch.Tensor, out: torch.Tensor | None = None,
              stream=None) -> torch.Tensor:
    """``out[s, h] = kv_c[s] . w_kvb[h]`` (bf16 ``[S, N, 256]``: k_nope then v)."""
    S, Lr = kv_c.shape
    N = w_kvb.shape[0]
    assert Lr == KV_LORA_RANK and kv_c.dtype == torch.bfloat16 and kv_c.stride(-1) == 1
    assert w_kvb.shape == (N, KV_LORA_RANK, 256) and w_kvb.is_contiguous() and w_kvb.dtype == torch.bfloat16
    if out is None:
        out = torch.empty((S, N, 256), dtype=torch.bfloat16, device=kv_c.device)
    _check("mla_kv_b_proj", lib().mla_kv_b_proj(_ptr(kv_c), kv_c.stride(0), _ptr(w_kvb), S, N, _ptr(out),
                                                out.stride(0), out.stride(1), _stream(stream)))
    return out


def prefill_mha(q: torch.Tensor, k_nope: torch.Tensor, k_pe: torch.Tensor, v: torch.Tensor,
                cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor, max_q_len: int,
                causal: bool = True, softmax_scale: float = DEFAULT_SCALE,
                out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """Attention of a prefill batch's new tokens: ``q[T, N, 192]`` against keys
    ``[k_nope[S, N, 128] | k_pe[S, 64]]`` and values ``v[S, N, 128]``; returns
    ``out[T, N, 128]`` and ``lse[T, N]``."""
    T, N, D = q.shape
    S = k_nope.shape[0]
    assert D == 192 and q.dtype == torch.bfloat16 and q.stride(-1) == 1
    assert k_nope.shape[1:] == (N, 128) and v.shape == (S, N, 128) and k_pe.shape == (S, 64)
    assert k_nope.stride(-1) == 1 and v.stride(-1) == 1 and k_pe.stride(-1) == 1
    assert cu_seqlens_q.dtype == torch.int32 and cu_seqlens_k.dtype == torch.int32
    B = cu_seqlens_q.numel() - 1
    assert cu_seqlens_k.numel() == B + 1
    if out is None:
        out = torch.empty((T, N, 128), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((T, N), dtype=torch.float32, device=q.device)
    _need_out("prefill_mha", out, (T, N, 128))
    _need_lse("prefill_mha", lse, (T, N))
    _check("mla_prefill_mha", lib().mla_prefill_mha(
        _ptr(q), q.stride(0), q.stride(1), _ptr(k_nope), k_nope.stride(0), k_nope.stride(1), _ptr(k_pe),
        k_pe.stride(0), _ptr(v), v.stride(0), v.stride(1), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B, T, S, N,
        int(max_q_len), 1 if causal else 0, float(softmax_scale), _ptr(out), out.stride(0), out.stride(1),
        _ptr(lse), _stream(stream)))
    return out, lse


def prefill_workspace_rows(max_model_len: int, max_num_seqs: int, page_tokens: int = PAGE_TOKENS) -> int:
    """Row budget of the chunked-context workspace (see ``mla_prefill_workspace_rows``)."""
    return int(lib().mla_prefill_workspace_rows(int(max_model_len), int(max_num_seqs), int(page_tokens)))


def plan_context_chunks(context_lens, row_budget: int):
    """Chunk plan of a prefill batch's context (see ``mla_plan_context_chunks``): returns
    int32 numpy arrays ``starts[n_chunks, B]`` and ``lens[n_chunks, B]``."""
    import numpy as np
    cl = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    B = int(cl.size)
    n = int(lib().mla_plan_context_chunks(cl.ctypes.data, B, int(row_budget), None, None, 0))
    if n < 0:
        raise MLAError("mla_plan_context_chunks", -n)
    starts = np.zeros((max(n, 1), B), dtype=np.int32)
    lens = np.zeros((max(n, 1), B), dtype=np.int32)
    m = int(lib().mla_plan_context_chunks(cl.ctypes.data, B, int(row_budget), starts.ctypes.data,
                                          lens.ctypes.data, n))
    assert m == n
    return starts[:n], lens[:n]


def gather_cache(kv_cache: torch.Tensor, kv_dtype: int, block_table: torch.Tensor,
                 cu_seq_lens: torch.Tensor, token_to_seq: torch.Tensor,
                 seq_starts: torch.Tensor | None = None, out: torch.Tensor | None = None,
                 stream=None) -> torch.Tensor:
    """Context rows of the paged cache as a contiguous bf16 ``[total, 576]`` workspace.

    ``block_table`` int32 ``[B, max_pages]``, ``cu_seq_lens`` int32 ``[B + 1]``,
    ``token_to_seq`` int32 ``[total]``, ``seq_starts`` int32 ``[B]`` or None.
    """
    assert block_table.dtype == torch.int32 and block_table.stride(-1) == 1
    assert cu_seq_lens.dtype == torch.int32 and token_to_seq.dtype == torch.int32
    assert seq_starts is None or seq_starts.dtype == torch.int32
    B = block_table.shape[0]
    total = token_to_seq.numel()
    num_pages = kv_cache.numel() * kv_cache.element_size() // (PAGE_TOKENS * ROW_BYTES[kv_dtype])
    if out is None:
        out = torch.empty((total, ROW_ELEMS), dtype=torch.bfloat16, device=kv_cache.device)
    assert out.dtype == torch.bfloat16 and out.stride(-1) == 1
    _check("mla_gather_cache", lib().mla_gather_cache(
        _ptr(kv_cache), kv_dtype, num_pages, _ptr(block_table), block_table.stride(0),
        block_table.shape[1], _ptr(cu_seq_lens), _ptr(seq_starts), _ptr(token_to_seq), B, total,
        _ptr(out), out.stride(0), _stream(stream)))
    return out


def merge_attn_states(prefix_out: torch.Tensor, prefix_lse: torch.Tensor, suffix_out: torch.Tensor,
                      suffix_lse: torch.Tensor, out: torch.Tensor | None = None,
                      out_lse: torch.Tensor | None = None, stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """Merge two attention states ``(o [T, N, D] bf16, lse [T, N] fp32)`` of the same rows."""
    T, N, D = prefix_out.shape
    assert prefix_out.dtype == torch.bfloat16 and suffix_out.dtype == torch.bfloat16
    assert suffix_out.stride() == prefix_out.stride() and prefix_out.stride(-1) == 1
    assert prefix_lse.dtype == torch.float32 and suffix_lse.stride() == prefix_lse.stride()
    if out is None:
        out = torch.empty_strided(prefix_out.shape, prefix_out.stride(), dtype=torch.bfloat16,
                                  device=prefix_out.device)
    if out_lse is None:
        out_lse = torch.empty_strided(prefix_lse.shape, prefix_lse.stride(), dtype=torch.float32,
                                      device=prefix_lse.device)
    assert out.stride() == prefix_out.stride() and out_lse.stride() == prefix_lse.stride()
    _check("mla_merge_attn_states", lib().mla_merge_attn_states(
        _ptr(prefix_out), _ptr(prefix_lse), _ptr(suffix_out), _ptr(suffix_lse), T, N, D,
        prefix_out.stride(0), prefix_out.stride(1), prefix_lse.stride(0), prefix_lse.stride(1),
        _ptr(out), _ptr(out_lse), _stream(stream)))
    return out, out_lse


def decode_varlen(q: torch.Tensor, query_start_loc: torch.Tensor, kv_cache: torch.Tensor, kv_dtype: int,
                  block_table: torch.Tensor, seq_lens: torch.Tensor, causal: bool = True,
                  softmax_scale: float = DEFAULT_SCALE, num_splits: int = 0,
                  workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                  lse: torch.Tensor | None = None, stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """Decode of ``q`` bf16 ``[T, N, 576]`` whose request ``b`` owns rows
    ``query_start_loc[b] .. query_start_loc[b+1]-1``; returns ``out [T, N, 512]``, ``lse [T, N]``."""
    T, N, D = q.shape
    assert D == ROW_ELEMS and q.dtype == torch.bfloat16 and q.stride(-1) == 1
    assert query_start_loc.dtype == torch.int32 and seq_lens.dtype == torch.int32
    assert block_table.dtype == torch.int32 and block_table.stride(-1) == 1
    B = seq_lens.numel()
    assert query_start_loc.numel() == B + 1
    num_pages = kv_cache.numel() * kv_cache.element_size() // (PAGE_TOKENS * ROW_BYTES[kv_dtype])
    if out is None:
        out = torch.empty((T, N, KV_LORA_RANK), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((T, N), dtype=torch.float32, device=q.device)
    _need_out("decode_varlen", out, (T, N, KV_LORA_RANK))
    _need_lse("decode_varlen", lse, (T, N))
    need = int(lib().mla_decode_varlen_workspace_size(T, N, num_splits, block_table.shape[1]))
    if need == 0:
        raise MLAError("mla_decode_varlen_workspace_size", 2)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check("mla_decode_varlen", lib().mla_decode_varlen(
        _ptr(q), q.stride(0), q.stride(1), _ptr(kv_cache), kv_dtype, num_pages, _ptr(block_table),
        block_table.stride(0), block_table.shape[1], _ptr(query_start_loc), _ptr(seq_lens), B, T, N,
        int(bool(causal)), float(softmax_scale), num_splits, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), out.stride(0), out.stride(1), _ptr(lse),
        _stream(stream)))
    return out, lse

"""mla_decode_noalloc (decode with the library's per-GPU scratch array instead of a
caller workspace) against mla_decode through the C ABI: two calls in a row, the
second on a smaller batch, each bit-identical to mla_decode on the same inputs and
split mode (same kernels and plan) and within the oracle's gates."""

import numpy as np
import pytest
import torch

import mla_inputs as MI
import mla_paged_latent_amd as M
from oracle import mla_oracle as O
from tests.mla_testlib import check_lse, check_out, dev_bf16, gpu_pool, oracle_pool, say, to_f64

pytestmark = pytest.mark.gpu

SC = O.default_scale()


def _noalloc_call(w, pool, q, num_splits):
    """mla_decode_noalloc through ctypes with outputs allocated here."""
    out = torch.empty((w.B, w.q_len, w.N, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.q_len, w.N), dtype=torch.float32, device="cuda")
    bt = torch.from_numpy(w.block_table).cuda()
    sl = torch.from_numpy(w.seq_lens).cuda()
    st = M.lib().mla_decode_noalloc(
        q.data_ptr(), q.stride(0), q.stride(1), q.stride(2), pool.data_ptr(), w.kv_dtype, w.num_pages,
        bt.data_ptr(), bt.stride(0), bt.shape[1], sl.data_ptr(), w.B, w.q_len, w.N, SC, num_splits,
        out.data_ptr(), out.stride(0), out.stride(1), out.stride(2), lse.data_ptr(),
        torch.cuda.current_stream().cuda_stream)
    assert st == 0, M.lib().mla_status_str(st)
    return out, lse, bt, sl


@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_noalloc_matches_decode_twice_second_smaller(num_splits):
    rng = np.random.default_rng(300 + num_splits)
    big = MI.make_workload("na-big", 12, 2, 128, rng.integers(500, 9000, 12).tolist(), None, MI.KV_BF16,
                           False, 300 + num_splits)
    small = MI.make_workload("na-small", 3, 1, 16, [7, 130, 2000], None, MI.KV_FP8, False, 310 + num_splits)
    for w in (big, small):
        say(f"noalloc {w.name}: B={w.B} q_len={w.q_len} N={w.N} kv={w.kv_dtype} num_splits={num_splits}")
        pool = gpu_pool(w)
        q = dev_bf16(w.q)
        out, lse, bt, sl = _noalloc_call(w, pool, q, num_splits)
        ref_out, ref_lse = M.decode(q, pool, w.kv_dtype, bt, sl, SC, num_splits)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), "differs from mla_decode"
        o_ref, lse_ref = O.decode(O.bf16_bits_to_f64(w.q), oracle_pool(w), w.kv_dtype, w.block_table,
                                  w.seq_lens, SC)
        check_out(to_f64(out), o_ref, w.name)
        check_lse(lse.cpu().numpy(), lse_ref, w.name)


def test_noalloc_full_head_batch_fits_and_too_large_is_rejected():
    """The 128-head benchmark batch runs through the scratch; a batch whose partials
    cannot fit is refused with MLA_ERR_WORKSPACE before anything is enqueued."""
    w = MI.make_workload("na-fh", 32, 1, 128, [8192] * 32, 8192, MI.KV_BF16, False, 320)
    pool = gpu_pool(w)
    q = dev_bf16(w.q)
    out, lse, bt, sl = _noalloc_call(w, pool, q, 0)
    ref_out, ref_lse = M.decode(q, pool, w.kv_dtype, bt, sl, SC, 0)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
    # 4096 requests x 2 head groups x 64 rows of float32 partials is far beyond the scratch
    B = 4096
    qb = torch.zeros((B, 1, 128, 576), dtype=torch.bfloat16, device="cuda")
    btb = torch.zeros((B, 1), dtype=torch.int32, device="cuda")
    slb = torch.ones((B,), dtype=torch.int32, device="cuda")
    ob = torch.empty((B, 1, 128, 512), dtype=torch.bfloat16, device="cuda")
    lb = torch.empty((B, 1, 128), dtype=torch.float32, device="cuda")
    st = M.lib().mla_decode_noalloc(qb.data_ptr(), qb.stride(0), qb.stride(1), qb.stride(2), pool.data_ptr(),
                                    0, w.num_pages, btb.data_ptr(), 1, 1, slb.data_ptr(), B, 1, 128, SC, 0,
                                    ob.data_ptr(), ob.stride(0), ob.stride(1), ob.stride(2), lb.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream)
    assert st == 5, M.lib().mla_status_str(st)       # MLA_ERR_WORKSPACE

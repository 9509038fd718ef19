"""GPU parity of the variable-query-length decode (mla_decode_varlen, causal and
non-causal draft blocks) against the oracle, and a HIP-graph capture of the
calls (decode, varlen decode, gather, state merge) replayed several times."""

import numpy as np
import pytest
import torch

import mla_inputs as MI
import mla_paged_latent_amd as M
from oracle import mla_oracle as O
from tests.mla_testlib import check_lse, check_out, dev_bf16, gpu_pool, host_bits, oracle_pool, say, to_f64

pytestmark = pytest.mark.gpu

SC = O.default_scale()


def _varlen(N, kd, q_lens, seqs, seed):
    w = MI.make_workload("varlen", len(seqs), 1, N, seqs, None, kd, False, seed)
    qsl = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    q = MI.make_workload("varlen-q", int(qsl[-1]), 1, N, [1] * int(qsl[-1]), None, kd, False, seed + 1).q
    return w, qsl, q.reshape(int(qsl[-1]), N, 576)


@pytest.mark.parametrize("N,kd", [(16, MI.KV_BF16), (128, MI.KV_BF16), (128, MI.KV_FP8), (40, MI.KV_BF16)])
@pytest.mark.parametrize("causal", [True, False])
def test_decode_varlen_parity(N, kd, causal):
    q_lens = [1, 3, 2, 0, 4, 2, 1, 3]
    seqs = [700, 65, 3000, 50, 130, 2049, 1, 2]       # the last two: blocks longer than the context
    w, qsl, q = _varlen(N, kd, q_lens, seqs, 160 + N + kd)
    pool = gpu_pool(w)
    ref_pool = oracle_pool(w)
    o_ref, l_ref = O.decode_varlen(O.bf16_bits_to_f64(q), qsl, ref_pool, kd, w.block_table, w.seq_lens, causal, SC)
    for ns in (0, 1, 3):
        say(f"varlen N={N} kd={kd} causal={causal} num_splits={ns}")
        out, lse = M.decode_varlen(dev_bf16(q), torch.from_numpy(qsl).cuda(), pool, kd,
                                   torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda(),
                                   causal, SC, ns)
        torch.cuda.synchronize()
        o = to_f64(out)
        l = lse.cpu().numpy()
        empty = np.isneginf(l_ref)
        assert np.array_equal(np.isneginf(l), empty) and np.all(o[empty] == 0)
        check_out(o[~empty.all(axis=1)], o_ref[~empty.all(axis=1)], f"varlen N{N} causal={causal} ns{ns}")
        check_lse(l, l_ref, f"varlen N{N} causal={causal} ns{ns}")


def test_decode_varlen_matches_uniform_decode_rows():
    """Uniform 2-token causal blocks through the varlen call: the same rows as the
    uniform decode within the output gate, the same empty rows."""
    N = 128
    w = MI.make_workload("uni", 5, 2, N, [900, 2, 64, 1, 4000], None, MI.KV_BF16, False, 170)
    pool = gpu_pool(w)
    qsl = np.arange(0, 11, 2, dtype=np.int32)
    q = dev_bf16(w.q.reshape(10, N, 576))
    o_v, l_v = M.decode_varlen(q, torch.from_numpy(qsl).cuda(), pool, MI.KV_BF16,
                               torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda(), True)
    o_u, l_u = M.decode(dev_bf16(w.q), pool, MI.KV_BF16, torch.from_numpy(w.block_table).cuda(),
                        torch.from_numpy(w.seq_lens).cuda())
    torch.cuda.synchronize()
    o_ref, l_ref = O.decode(O.bf16_bits_to_f64(w.q), oracle_pool(w), MI.KV_BF16, w.block_table, w.seq_lens, SC)
    check_out(to_f64(o_v).reshape(o_ref.shape), o_ref, "varlen as uniform")
    check_out(to_f64(o_u), o_ref, "uniform")
    check_lse(l_v.cpu().numpy().reshape(l_ref.shape), l_ref, "varlen as uniform")


def test_graph_capture_replays_match_eager():
    """The calls enqueue only kernels on the caller's stream (no allocation, no host
    synchronisation, no memset), so a captured graph replays them: every replay,
    with eager work in between, gives the eager bits."""
    N = 128
    w = MI.make_workload("graph", 4, 1, N, [3000, 65, 700, 1], None, MI.KV_BF16, False, 180)
    pool = gpu_pool(w)
    bt = torch.from_numpy(w.block_table).cuda()
    sl = torch.from_numpy(w.seq_lens).cuda()
    q = dev_bf16(w.q)
    qsl = torch.tensor([0, 1, 3, 3, 4], dtype=torch.int32, device="cuda")
    qv = q.view(4, N, 576)
    c = MI.make_context_chunk([700, 65], [0, 0], w.num_pages, seed=181)
    cbt, ccu, ct2s = (torch.from_numpy(a).cuda() for a in (c.block_table, c.cu_seq_lens, c.token_to_seq))
    # every output and workspace allocated before capture
    outs = {}
    for ns in (0, 1):
        outs[ns] = (torch.empty((4, 1, N, 512), dtype=torch.bfloat16, device="cuda"),
                    torch.empty((4, 1, N), dtype=torch.float32, device="cuda"),
                    torch.empty(M.decode_workspace_size(4, 1, N, ns), dtype=torch.uint8, device="cuda"))
    vo = torch.empty((4, N, 512), dtype=torch.bfloat16, device="cuda")
    vl = torch.empty((4, N), dtype=torch.float32, device="cuda")
    vws = torch.empty(int(M.lib().mla_decode_varlen_workspace_size(4, N, 0, bt.shape[1])), dtype=torch.uint8,
                      device="cuda")
    g_out = torch.empty((c.total, 576), dtype=torch.bfloat16, device="cuda")
    mo = torch.empty((4, N, 512), dtype=torch.bfloat16, device="cuda")
    ml = torch.empty((4, N), dtype=torch.float32, device="cuda")
    # the contractions around decode, with their fused variants
    gen = torch.Generator(device="cuda").manual_seed(182)
    qn = torch.randn(37, N, 192, device="cuda", generator=gen).to(torch.bfloat16)
    wk = (torch.randn(N, 128, 512, device="cuda", generator=gen) / 23).to(torch.bfloat16)
    wv = (torch.randn(N, 512, 128, device="cuda", generator=gen) / 23).to(torch.bfloat16)
    ol = torch.randn(37, N, 512, device="cuda", generator=gen).to(torch.bfloat16)
    pos = torch.randint(0, 64, (37,), device="cuda", generator=gen)
    table = torch.from_numpy(MI.rope_cos_sin(64)).cuda()
    qf1 = torch.empty((37, N, 576), dtype=torch.bfloat16, device="cuda")
    qf2 = torch.empty_like(qf1)
    yv = torch.empty((37, N * 128), dtype=torch.bfloat16, device="cuda")
    yc = torch.empty((37, N * 128), dtype=torch.uint8, device="cuda")
    ys = torch.empty((37, N), dtype=torch.float32, device="cuda")

    def work():
        for ns in (0, 1):
            o, l, ws = outs[ns]
            M.decode(q, pool, MI.KV_BF16, bt, sl, SC, ns, workspace=ws, out=o, lse=l)
        M.decode_varlen(qv, qsl, pool, MI.KV_BF16, bt, sl, False, SC, 0, workspace=vws, out=vo, lse=vl)
        M.gather_cache(pool, MI.KV_BF16, cbt, ccu, ct2s, out=g_out)
        M.merge_attn_states(outs[0][0].view(4, N, 512), outs[0][1].view(4, N), vo, vl, out=mo, out_lse=ml)
        M.absorb_q(qn[..., :128], qn[..., 128:], wk, q_fused=qf1)
        M.absorb_q_rope(qn[..., :128], qn[..., 128:], wk, pos, table, True, q_fused=qf2)
        M.up_v(ol, wv, out=yv)
        M.up_v_fp8(ol, wv, 128, out_codes=yc, out_scales=ys)

    def snapshot():
        return [t.clone() for t in (outs[0][0], outs[0][1], outs[1][0], outs[1][1], vo, vl, g_out, mo, ml,
                                    qf1, qf2, yv, yc, ys)]

    work()                                    # eager, and warm-up before capture
    torch.cuda.synchronize()
    eager = snapshot()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            work()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (outs[0][0], outs[1][0], vo, g_out, mo, qf1, qf2, yv, yc, ys):   # eager work between replays
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot()
        say(f"graph replay {rep}")
        for a, b in zip(eager, got):
            assert torch.equal(a, b)

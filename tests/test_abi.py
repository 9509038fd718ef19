"""The C-ABI library on the CPU: it loads, exports every call include/mla.h
declares, sizes workspaces by pure host arithmetic, and rejects bad arguments
with a status before touching a device."""

import ctypes
import os
import re

import pytest

import mla_paged_latent_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")



def _ensure_library() -> None:
    """Build the library in-tree when it is missing (hipcc cross-compiles without a
    GPU); skip only if there is no hipcc either."""
    if os.path.exists(M.LIB_PATH):
        return
    from mla_paged_latent_amd import build as B
    try:
        B.hipcc()
    except RuntimeError:
        pytest.skip("HIP library not built and no hipcc to build it")
    B.build()


# every test here runs in both test jobs: the CPU one (-m "not gpu") and the GPU one
@pytest.fixture(autouse=True, params=[pytest.param("host"), pytest.param("gpu-job", marks=pytest.mark.gpu)])
def _library(request):
    _ensure_library()
    yield


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_calls():
    fns = declared_functions()
    for f in ("mla_cache_write", "mla_absorb_q", "mla_decode", "mla_up_v",
              "mla_up_v_fp8", "mla_absorb_q_rope", "mla_kv_b_proj", "mla_prefill_mha",
              "mla_decode_workspace_size", "mla_status_str"):
        assert f in fns


def test_library_exports_every_declared_symbol():
    L = M.lib()
    for f in declared_functions():
        assert hasattr(L, f), f


def test_probe_library_exports_its_header():
    """The measurement probes (libmla_probe.so) export what include/mla_probe.h declares."""
    import ctypes
    probe_h = os.path.join(ROOT, "include", "mla_probe.h")
    probe_so = os.path.join(os.path.dirname(M.LIB_PATH), "libmla_probe.so")
    if not os.path.exists(probe_so):
        from mla_paged_latent_amd import build as B
        B.build()
    P = ctypes.CDLL(probe_so)
    own = [f for f in declared_functions(probe_h) if f.startswith("mla_probe_")]
    assert own == ["mla_probe_hbm_read", "mla_probe_mfma_bf16", "mla_probe_mfma_flops", "mla_probe_sink_bytes"]
    for f in own:
        assert hasattr(P, f), f


def test_status_strings():
    L = M.lib()
    for code in range(8):
        assert L.mla_status_str(code).startswith(b"MLA_")
    assert b"unknown" in L.mla_status_str(99)


def test_workspace_size_arithmetic():
    ws = M.decode_workspace_size
    # invalid shapes give 0
    assert ws(0, 1, 16, 0) == 0 and ws(4, 3, 16, 0) == 0 and ws(4, 1, 0, 0) == 0
    assert ws(4, 1, 129, 0) == 0 and ws(4, 1, 16, -1) == 0 and ws(4, 1, 16, 5000) == 0
    # partials dominate: pairs x head groups x rows x (512 + 1) floats
    one = ws(32, 1, 128, 1)
    assert one >= (32 + 8) * 1 * 128 * 513 * 4
    assert ws(32, 1, 128, 8) > one
    assert ws(32, 1, 128, 0) >= (32 + 1024 + 8) * 128 * 513 * 4
    # q_len 2 with 128 heads needs two head groups of 128 rows
    assert ws(8, 2, 128, 1) >= (8 + 8) * 2 * 128 * 513 * 4
    assert ws(64, 1, 16, 1) >= (64 + 8) * 16 * 513 * 4
    assert ws(64, 1, 16, 1) % 256 == 0


def _decode_args(**over):
    vp = ctypes.c_void_p
    a = dict(q=vp(256), qsb=576, qst=576, qsh=576, kv=vp(256), kvd=0, pages=4, bt=vp(256),
             btsb=4, maxp=4, seq=vp(256), B=1, ql=1, N=16, scale=0.07, ns=0, ws=vp(256),
             wsb=1 << 30, out=vp(256), osb=512, ost=512, osh=512, lse=vp(256), stream=None)
    a.update(over)
    return list(a.values())


def test_decode_rejects_bad_arguments_before_any_device_call():
    L = M.lib()
    assert L.mla_decode(*_decode_args(kvd=7)) == 3                 # MLA_ERR_DTYPE
    assert L.mla_decode(*_decode_args(ql=3)) == 2                  # MLA_ERR_SHAPE
    assert L.mla_decode(*_decode_args(N=200)) == 2
    assert L.mla_decode(*_decode_args(B=0)) == 2
    assert L.mla_decode(*_decode_args(scale=0.0)) == 2
    assert L.mla_decode(*_decode_args(scale=float("nan"))) == 2
    assert L.mla_decode(*_decode_args(btsb=2)) == 2                # row stride < max pages
    assert L.mla_decode(*_decode_args(q=None)) == 1                # MLA_ERR_NULL
    assert L.mla_decode(*_decode_args(lse=None)) == 1
    assert L.mla_decode(*_decode_args(ws=None)) == 5               # MLA_ERR_WORKSPACE
    assert L.mla_decode(*_decode_args(wsb=100)) == 5
    assert L.mla_decode(*_decode_args(q=ctypes.c_void_p(258))) == 4   # MLA_ERR_ALIGN
    assert L.mla_decode(*_decode_args(qsh=577)) == 4
    assert L.mla_decode(*_decode_args(ws=ctypes.c_void_p(272))) == 4  # workspace needs 256 B


def test_other_calls_reject_bad_arguments():
    L = M.lib()
    vp = ctypes.c_void_p
    p = vp(256)
    # cache write
    assert L.mla_cache_write(p, 512, p, 64, p, 4, p, 9, 4, None) == 3
    assert L.mla_cache_write(p, 512, p, 64, p, 0, p, 0, 4, None) == 0      # T == 0 is a no-op
    assert L.mla_cache_write(None, 512, p, 64, p, 4, p, 0, 4, None) == 1
    assert L.mla_cache_write(p, 500, p, 64, p, 4, p, 0, 4, None) == 2
    assert L.mla_cache_write(p, 520, p, 64, vp(260), 4, p, 0, 4, None) == 4
    # absorb
    assert L.mla_absorb_q(p, 128, 128, p, 64, 64, p, 4, 0, p, 576, 576, None) == 2
    assert L.mla_absorb_q(p, 128, 128, None, 0, 0, p, 0, 16, p, 576, 576, None) == 0
    assert L.mla_absorb_q(None, 128, 128, None, 0, 0, p, 4, 16, p, 576, 576, None) == 1
    assert L.mla_absorb_q(p, 130, 128, None, 0, 0, p, 4, 16, p, 576, 576, None) == 4
    # absorb + cache write in one launch: the statuses of the two calls
    def acw(**o):
        a = dict(qn=p, qns=128, qnh=128, qp=p, qps=64, qph=64, w=p, T=4, N=16, qf=p, qfs=576, qfh=576,
                 kc=p, kcs=512, kp=p, kps=64, sl=p, Tn=4, pool=p, kd=0, pages=4, stream=None)
        a.update(o)
        return L.mla_absorb_q_cache_write(*a.values())
    assert acw(N=0) == 2 and acw(N=129) == 2 and acw(T=-1) == 2
    assert acw(qn=None) == 1 and acw(kc=None) == 1 and acw(sl=None) == 1
    assert acw(kd=9) == 3                                                  # MLA_ERR_DTYPE
    assert acw(kcs=500) == 2                                               # latent row stride < 512
    assert acw(qns=130) == 4 and acw(qp=vp(264)) == 4 and acw(sl=vp(260)) == 4
    assert acw(T=0, Tn=0) == 0                                             # nothing to do
    assert acw(T=0, Tn=4, kd=9) == 3                                       # T == 0: the cache write's checks
    # up_v
    assert L.mla_up_v(p, 512, 512, p, 4, 129, p, 128 * 129, None) == 2
    assert L.mla_up_v(p, 512, 512, p, 4, 16, p, 1024, None) == 2           # out row too short
    assert L.mla_up_v(p, 512, 512, None, 4, 16, p, 2048, None) == 1
    # absorb with the rope part rotated
    r = L.mla_absorb_q_rope
    assert r(p, 128, 128, p, 64, 64, p, 4, 0, p, p, 16, 1, p, 576, 576, None) == 2
    assert r(p, 128, 128, p, 64, 64, p, 4, 16, p, p, 0, 1, p, 576, 576, None) == 2     # empty table
    assert r(p, 128, 128, p, 64, 64, p, 0, 16, p, p, 16, 1, p, 576, 576, None) == 0     # T == 0
    assert r(p, 128, 128, None, 64, 64, p, 4, 16, p, p, 16, 1, p, 576, 576, None) == 1  # q_pe required
    assert r(p, 128, 128, p, 64, 64, p, 4, 16, None, p, 16, 1, p, 576, 576, None) == 1
    assert r(p, 128, 128, p, 64, 64, p, 4, 16, p, vp(264), 16, 1, p, 576, 576, None) == 4
    assert r(p, 128, 128, p, 64, 64, p, 4, 16, vp(260), p, 16, 1, p, 576, 576, None) == 4
    assert r(p, 128, 128, p, 66, 64, p, 4, 16, p, p, 16, 1, p, 576, 576, None) == 4
    # prefill: kv_b_proj and the 192/128 attention
    assert L.mla_kv_b_proj(p, 512, p, 4, 129, p, 4096, 256, None) == 2
    assert L.mla_kv_b_proj(p, 512, p, 0, 16, p, 4096, 256, None) == 0
    assert L.mla_kv_b_proj(p, 512, None, 4, 16, p, 4096, 256, None) == 1
    assert L.mla_kv_b_proj(p, 514, p, 4, 16, p, 4096, 256, None) == 4
    m = L.mla_prefill_mha
    args = lambda **o: [o.get(k, d) for k, d in [("q", p), ("qt", 3072), ("qh", 192), ("kn", p), ("knt", 2048),
                                                   ("knh", 128), ("kp", p), ("kpt", 64), ("v", p), ("vt", 2048),
                                                   ("vh", 128), ("cq", p), ("ck", p), ("B", 2), ("T", 8),
                                                   ("S", 8), ("N", 16), ("mq", 4), ("c", 1), ("sc", 0.07),
                                                   ("o", p), ("ot", 2048), ("oh", 128), ("l", p), ("s", None)]]
    assert m(*args(N=0)) == 2 and m(*args(B=-1)) == 2 and m(*args(B=70000)) == 2
    assert m(*args(T=0)) == 0 and m(*args(B=0)) == 0 and m(*args(mq=0)) == 0
    assert m(*args(kp=None)) == 1 and m(*args(ck=None)) == 1
    assert m(*args(qh=196)) == 4 and m(*args(l=vp(258))) == 4 and m(*args(v=vp(264))) == 4
    # up_v with fp8 group quantization of its output
    f = L.mla_up_v_fp8
    assert f(p, 512, 512, p, 4, 129, 128, p, 128 * 129, p, 129, None) == 2
    assert f(p, 512, 512, p, 4, 16, 32, p, 2048, p, 64, None) == 2           # group 32
    assert f(p, 512, 512, p, 0, 16, 64, p, 2048, p, 32, None) == 0           # T == 0 is a no-op
    assert f(p, 512, 512, p, 65535 * 32 + 1, 16, 64, p, 2048, p, 32, None) == 2
    assert f(p, 512, 512, None, 4, 16, 64, p, 2048, p, 32, None) == 1
    assert f(p, 512, 512, p, 4, 16, 64, p, 1024, p, 32, None) == 2          # codes row too short
    assert f(p, 512, 512, p, 4, 16, 128, p, 2048, p, 8, None) == 2          # scales row too short
    assert f(p, 512, 512, p, 4, 16, 64, p, 2052, p, 32, None) == 4          # codes stride % 8
    assert f(p, 512, 512, p, 4, 16, 64, p, 2048, vp(258), 32, None) == 4    # scales alignment


def test_context_calls_reject_bad_arguments_without_a_gpu():
    """Host-side checks of the gather and merge calls return before touching the device."""
    L = M.lib()
    vp = ctypes.c_void_p
    ok = vp(256)
    g = lambda **o: L.mla_gather_cache(*[o.get(k, v) for k, v in dict(
        kv=ok, kd=0, pages=4, bt=ok, btsb=4, maxp=4, cu=ok, ss=None, t2s=ok, B=1, total=10,
        out=ok, ostride=576, stream=None).items()])
    assert g(kd=7) == 3                          # MLA_ERR_DTYPE
    assert g(total=-1) == 2 and g(B=0) == 2 and g(btsb=3) == 2 and g(ostride=8) == 2
    assert g(total=0) == 0                       # nothing to do
    assert g(kv=None) == 1 and g(t2s=None) == 1
    assert g(out=vp(264)) == 4 and g(ostride=580) == 4 and g(t2s=vp(258)) == 4
    m = lambda **o: L.mla_merge_attn_states(*[o.get(k, v) for k, v in dict(
        po=ok, pl=ok, so=ok, sl=ok, T=4, N=2, D=64, ost=128, osh=64, lst=2, lsh=1, out=ok,
        ol=None, stream=None).items()])
    assert m(D=12) == 2 and m(D=0) == 2 and m(N=0) == 2 and m(T=-1) == 2 and m(D=8192) == 2
    assert m(T=0) == 0
    assert m(po=None) == 1 and m(out=None) == 1
    assert m(so=vp(264)) == 4 and m(osh=60) == 4 and m(pl=vp(258)) == 4


def test_varlen_call_rejects_bad_arguments_without_a_gpu():
    L = M.lib()
    vp = ctypes.c_void_p
    ok = vp(256)
    ws = L.mla_decode_varlen_workspace_size
    assert ws(0, 16, 0, 8) == 0 and ws(1 << 25, 16, 0, 8) == 0 and ws(4, 129, 0, 8) == 0 and ws(4, 16, 0, 0) == 0
    assert ws(4, 16, 0, 8) > 0 and ws(4, 16, 0, 800) > ws(4, 16, 0, 8)      # holds a block-table copy
    need = ws(4, 16, 0, 8)
    d = lambda **o: L.mla_decode_varlen(*[o.get(k, v) for k, v in dict(
        q=ok, qst=9216, qsh=576, kv=ok, kd=0, pages=4, bt=ok, btsb=8, maxp=8, qsl=ok, sl=ok, B=2, T=4, N=16,
        causal=1, scale=0.07, ns=0, ws=ok, wsb=need, out=ok, ost=8192, osh=512, lse=ok, stream=None).items()])
    assert d(kd=5) == 3
    assert d(T=0) == 2 and d(B=0) == 2 and d(N=0) == 2 and d(btsb=7) == 2 and d(scale=0.0) == 2
    assert d(qsl=None) == 1 and d(lse=None) == 1
    assert d(ws=None) == 5 and d(wsb=need - 1) == 5
    assert d(q=vp(264)) == 4 and d(qst=9220) == 4 and d(qsl=vp(258)) == 4 and d(ws=vp(512 + 16)) == 4


def test_binding_rejects_mismatched_out_and_lse():
    """Caller-supplied out / lse tensors of the wrong dtype, shape or layout raise
    before the C call (which would write bf16 rows at out's strides and a dense
    float32 lse)."""
    import torch
    B, q_len, N = 2, 1, 16
    q = torch.zeros((B, q_len, N, 576), dtype=torch.bfloat16)
    pool = torch.zeros((4, 64, 1152), dtype=torch.uint8)
    bt = torch.zeros((B, 4), dtype=torch.int32)
    sl = torch.ones((B,), dtype=torch.int32)
    good_out = torch.empty((B, q_len, N, 512), dtype=torch.bfloat16)
    good_lse = torch.empty((B, q_len, N), dtype=torch.float32)
    bad = [
        dict(out=torch.empty((B, q_len, N, 512), dtype=torch.float32), lse=good_lse),
        dict(out=torch.empty((B, q_len, N, 256), dtype=torch.bfloat16), lse=good_lse),
        dict(out=torch.empty((B, q_len, N, 1024), dtype=torch.bfloat16)[..., ::2], lse=good_lse),
        dict(out=good_out, lse=torch.empty((B, q_len, N), dtype=torch.bfloat16)),
        dict(out=good_out, lse=torch.empty((B, q_len, N - 1), dtype=torch.float32)),
        dict(out=good_out, lse=torch.empty((B, q_len, 2 * N), dtype=torch.float32)[..., ::2]),
    ]
    for kw in bad:
        with pytest.raises(ValueError):
            M.decode(q, pool, 0, bt, sl, M.DEFAULT_SCALE, 0, **kw)
    T = 3
    qv = torch.zeros((T, N, 576), dtype=torch.bfloat16)
    qsl = torch.tensor([0, 1, 3], dtype=torch.int32)
    with pytest.raises(ValueError):
        M.decode_varlen(qv, qsl, pool, 0, bt, sl, lse=torch.empty((T, N), dtype=torch.float32).t())
    with pytest.raises(ValueError):
        M.decode_varlen(qv, qsl, pool, 0, bt, sl, out=torch.empty((T, N, 512), dtype=torch.float16))
    qp = torch.zeros((T, N, 192), dtype=torch.bfloat16)
    kn = torch.zeros((T, N, 128), dtype=torch.bfloat16)
    kp = torch.zeros((T, 64), dtype=torch.bfloat16)
    cu = torch.tensor([0, T], dtype=torch.int32)
    with pytest.raises(ValueError):
        M.prefill_mha(qp, kn, kp, kn, cu, cu, T, out=torch.empty((T, N, 128), dtype=torch.float32))
    with pytest.raises(ValueError):
        M.prefill_mha(qp, kn, kp, kn, cu, cu, T, lse=torch.empty((N, T), dtype=torch.float32))


def test_context_chunk_plan_matches_the_oracle():
    """mla_plan_context_chunks / mla_prefill_workspace_rows (host arithmetic) give
    exactly the oracle's chunk plan and row budget."""
    import numpy as np
    from oracle import mla_oracle as O
    rng = np.random.default_rng(2800)
    for _ in range(200):
        B = int(rng.integers(1, 30))
        lens = (rng.integers(0, 7000, B) * (rng.random(B) > 0.2)).astype(np.int32)
        W = int(rng.choice([64, 100, 640, 1024, 4096, 65536]))
        starts, ls = M.plan_context_chunks(lens, W)
        ref = O.plan_context_chunks(lens.tolist(), W)
        assert len(ref) == starts.shape[0]
        for c, ch in enumerate(ref):
            want_s = np.zeros(B, np.int32)
            want_l = np.zeros(B, np.int32)
            for b, s0, t in ch:
                want_s[b], want_l[b] = s0, t
            assert np.array_equal(starts[c], want_s) and np.array_equal(ls[c], want_l)
    for L, S in ((163840, 256), (4096, 16), (1024, 64), (1, 1)):
        assert M.prefill_workspace_rows(L, S) == O.prefill_workspace_rows(L, S)
    L = M.lib()
    lens = np.array([100], np.int32)
    assert L.mla_plan_context_chunks(lens.ctypes.data, 1, 63, None, None, 0) == -2       # budget below a page
    assert L.mla_plan_context_chunks(None, 1, 1024, None, None, 0) == -1
    assert L.mla_prefill_workspace_rows(0, 1, 64) == 0

"""CPU model of the split plan the decode kernels derive from seq_lens on the device
("vLLM 源码完全拆解(三十七):MLA 注意力后端", §FlashMLA: a per-sequence split plan from
seq_lens and the compute-unit count; single-partition mode for batch invariance).

The model follows the kernels' planner step by step (the cost line of
kSegOverhead + pages per request, the equal cuts into streams, the front-loaded or
proportional mapping of a request's stretch onto its pages, the partial slot b + s,
the per-request {first slot, pieces} record) in both arithmetic forms the kernels
use: 32-bit unsigned products and quotients when a bound says they fit, exact
64-bit quotients (a bit-serial division) otherwise.  It checks what the merge and
the output rely on: every request's tokens covered once by page-aligned pieces in
stream order, one record per request that names exactly its pieces, consecutive
in-range partial slots, balanced streams, and the same plan from both arithmetic
forms wherever the 32-bit form is allowed.  The GPU tests run the kernels
themselves on these plans; this pins the planner's logic, including the 64-bit
branch that no realistic GPU batch reaches.
"""

from __future__ import annotations

import numpy as np
import pytest

OVERHEAD = 4            # pages' worth of cost for a piece's fixed work
PAGE = 64
U32 = 0xFFFFFFFF


def pages_of(s: int) -> int:
    return (s + PAGE - 1) // PAGE


def udiv64_slow(a: int, b: int) -> int:
    """The kernels' bit-serial 64-bit unsigned division, restated."""
    q = r = 0
    for i in range(63, -1, -1):
        r = (r << 1) | ((a >> i) & 1)
        if r >= b:
            r -= b
            q |= 1 << i
    return q


class Totals:
    """Cost-line totals and the cut arithmetic of one plan."""

    def __init__(self, total: int, n: int, p64: bool):
        self.total, self.n, self.p64 = total, n, p64

    def small(self) -> bool:
        return (not self.p64) or self.total <= U32 // (self.n + 1)

    def start(self, s: int) -> int:
        if self.small():
            return ((s * self.total) & U32) // self.n
        return udiv64_slow(s * self.total, self.n)

    def stream_of(self, x: int) -> int:
        if self.small():
            return ((((x + 1) & U32) * self.n - 1) & U32) // self.total
        return udiv64_slow((x + 1) * self.n - 1, self.total)


def scale_floor(x: int, np_: int, ln: int, p64: bool) -> int:
    if not p64 or ln * np_ <= U32:
        return ((x * np_) & U32) // ln
    return udiv64_slow(x * np_, ln)


def plan_auto(seq_lens, n_streams: int, cap: int, p64: bool):
    """All pieces (stream, b, t0, t1, pieces of b, slot) and the per-request records."""
    seq = [min(max(0, int(s)), cap) for s in seq_lens]
    B = len(seq)
    cost = [OVERHEAD + pages_of(s) for s in seq]
    prefix = np.concatenate([[0], np.cumsum(cost, dtype=np.int64)]).tolist()
    tot = Totals(int(prefix[-1]), min(n_streams, int(prefix[-1])), p64)
    pieces, req = [], {}
    for s in range(n_streams):
        if s >= tot.n:
            continue
        lo, hi = tot.start(s), tot.start(s + 1)
        # the request holding position lo and where it starts
        b = int(np.searchsorted(prefix, lo, side="right")) - 1
        c = prefix[b]
        while b < B and c < hi:
            sq = seq[b]
            np_ = pages_of(sq)
            ln = OVERHEAD + np_
            if np_ == 0:
                if c >= lo:
                    req.setdefault(b, []).append((0, 1, s))
                    pieces.append((s, b, 0, 0, 1, b + s))
            else:
                prop = tot.start(tot.stream_of(c)) == c
                first_end = (ln + np_ - 1) // np_ if prop else OVERHEAD + 1
                sf, sl = tot.stream_of(c + first_end - 1), tot.stream_of(c + ln - 1)
                if sf <= s <= sl:
                    xa = lo - c if lo > c else 0
                    xe = hi - c if hi < c + ln else ln
                    if prop:
                        pa, pe = scale_floor(xa, np_, ln, p64), scale_floor(xe, np_, ln, p64)
                    else:
                        pa, pe = max(xa - OVERHEAD, 0), max(xe - OVERHEAD, 0)
                    if s == sf:
                        req.setdefault(b, []).append((b + sf, sl - sf + 1, s))
                    t0, t1 = min(pa * PAGE, sq), min(pe * PAGE, sq)
                    pieces.append((s, b, t0, t1, sl - sf + 1, b + s))
            c += ln
            b += 1
    return seq, pieces, req, tot


def plan_forced(seq_lens, k: int, cap: int):
    """num_splits = k >= 1: stream s is split s % k of request s // k."""
    seq = [min(max(0, int(s)), cap) for s in seq_lens]
    pieces, req = [], {}
    for s in range(len(seq) * k):
        b, sp = divmod(s, k)
        sq = seq[b]
        chunk = max(PAGE, pages_of((sq + k - 1) // k) * PAGE)
        ns = (sq + chunk - 1) // chunk if sq > 0 else 1
        if sp == 0:
            req.setdefault(b, []).append((b * k, ns, s))
        if sp < ns:
            t0 = sp * chunk
            t1 = min(t0 + chunk, sq)
            pieces.append((s, b, t0, max(t1, t0), ns, s))
    return seq, pieces, req


def check_plan(seq, pieces, req, max_slots: int):
    B = len(seq)
    assert sorted(req) == list(range(B)), "a record for every request"
    for b in range(B):
        assert len(req[b]) == 1, f"request {b} recorded {len(req[b])} times"
    for b in range(B):
        first, n, _ = req[b][0]
        ps = sorted((p for p in pieces if p[1] == b), key=lambda p: p[0])
        assert len(ps) == n, (b, len(ps), n)
        assert all(p[4] == n for p in ps)
        if seq[b] == 0:
            assert [(p[2], p[3]) for p in ps] == [(0, 0)]
            continue
        # coverage in stream order, page-aligned starts; empty pieces allowed between
        pos = 0
        for p in ps:
            assert p[2] == pos and p[2] % PAGE == 0 and p[3] >= p[2], (b, ps)
            pos = p[3]
        assert pos == seq[b]
        if n > 1:
            slots = [p[5] for p in ps]
            assert slots == list(range(first, first + n)), (b, slots, first)
            assert 0 <= first and first + n <= max_slots
    split_slots = [p[5] for p in pieces if p[4] > 1]
    assert len(split_slots) == len(set(split_slots)), "one piece per partial slot"


def _cases():
    rng = np.random.default_rng(2026)
    cases = [([37, 100], 256), ([8192] * 32, 128), (list(rng.integers(1024, 4097, 64)), 256),
             (list(np.clip(np.round(np.exp(rng.normal(np.log(2048), 1.0, 128))), 64, 32768).astype(int)), 128),
             ([131072, 65536, 32768, 16384, 8192, 4096, 2048, 1024], 64), ([0, 0, 5, 0], 8), ([0], 8),
             ([1] * 600, 256), ([64] * 7, 256)]
    for _ in range(250):
        B = int(rng.integers(1, 300))
        seq = (rng.integers(0, 5000, B) * (rng.random(B) > 0.1)).tolist()
        cases.append((seq, int(rng.choice([8, 64, 80, 128, 256]))))
    return cases


@pytest.mark.parametrize("p64", [False, True])
def test_auto_plan_invariants(p64):
    cap = (2 ** 31 - 1) // PAGE * PAGE
    for seq_lens, G in _cases():
        seq, pieces, req, tot = plan_auto(seq_lens, G, cap, p64)
        check_plan(seq, pieces, req, len(seq) + G)
        # balance: no stream holds more than its equal share of the cost line plus one
        # page's rounding at each end
        load = {}
        for s, b, t0, t1, n, _ in pieces:
            load[s] = load.get(s, 0) + pages_of(t1) - t0 // PAGE
        if load:
            assert max(load.values()) <= -(-tot.total // tot.n) + 2


def test_forced_plan_invariants():
    cap = (2 ** 31 - 1) // PAGE * PAGE
    for seq_lens, _ in _cases()[:80]:
        for k in (1, 2, 3, 8, 64):
            seq, pieces, req = plan_forced(seq_lens, k, cap)
            check_plan(seq, pieces, req, len(seq) * k)
            if k == 1:
                assert all(p[2] == 0 and p[3] == seq[p[1]] for p in pieces)


def test_32_and_64_bit_forms_agree_where_the_32_bit_form_is_allowed():
    """Under the host's bound (B * (overhead + table width) * (streams + 1) and
    (overhead + width) * width both below 2^32) the 32-bit kernels' arithmetic gives
    the exact plan."""
    rng = np.random.default_rng(7)
    for _ in range(150):
        B = int(rng.integers(1, 400))
        width = int(rng.integers(1, 2000))
        G = int(rng.choice([8, 64, 128, 256, 1024]))
        stretch = OVERHEAD + width
        if B * stretch > U32 // (G + 1) or stretch * width > U32:
            continue
        seq = rng.integers(0, width * PAGE + 1, B).tolist()
        a = plan_auto(seq, G, width * PAGE, p64=False)
        b = plan_auto(seq, G, width * PAGE, p64=True)
        assert a[1] == b[1] and a[2] == b[2]


def test_64_bit_branch_on_batches_beyond_32_bits():
    """Batches whose cost line times the stream count exceeds 2^32 take the exact
    64-bit arithmetic; the plan keeps every invariant there."""
    cap = (2 ** 31 - 1) // PAGE * PAGE
    rng = np.random.default_rng(8)
    for B, G in ((200, 1024), (3000, 256), (64, 1024)):
        seq = rng.integers(cap // 2, cap + 1, B).tolist()
        seq[::7] = [0] * len(seq[::7])
        s, pieces, req, tot = plan_auto(seq, G, cap, p64=True)
        assert not tot.small(), "the case must take the 64-bit branch"
        check_plan(s, pieces, req, B + G)


def test_bit_serial_division():
    rng = np.random.default_rng(9)
    for _ in range(300):
        a = int(rng.integers(0, 2 ** 62)) * int(rng.integers(1, 4))
        b = int(rng.integers(1, 2 ** 40))
        assert udiv64_slow(a, b) == a // b
    assert udiv64_slow(2 ** 64 - 1, 1) == 2 ** 64 - 1 and udiv64_slow(5, 7) == 0

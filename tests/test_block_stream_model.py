"""CPU model of the wide decode kernel's block stream: copies into the LDS ring, the waits
for them, tail zeroing, reads and the epilogue's staging slot, with the workgroup barriers
between them ("vLLM 源码完全拆解(三十七):MLA 注意力后端", §FlashMLA: the paged cache of each
split streamed block by block; the ring and its bookkeeping are this library's design).

A workgroup walks the pieces of one stream of the split plan.  Their 32-token blocks form
one stream of copies into a 4-slot ring (slot = stream index mod 4).  The copying waves
keep an issue cursor that runs up to kWDepth blocks ahead, across piece boundaries, and
`landed`, the count of stream blocks they have waited for.  The model restates the
kernel's sequence (piece start, block steps, last PV, slack vote, epilogue, an optional
redo of a piece) and checks, with barriers as the only ordering between waves:
  * a block is read only in an interval after the one in which its copy was waited for;
  * a copy into a slot is issued only in an interval after every read of the slot's
    previous block and after the epilogue staging that used the slot;
  * a block's tail is zeroed after its copy landed and before any read of it;
  * the epilogue's staging slot holds no copy in flight and no block still to be read.
The plans come from the split-plan model, so the cases include streams with empty pieces
and pieces of one block, which exercise the cross-piece prefetch.  With `query_lds` (bf16
rows, one query row per head) a unit's first piece also copies its query into ring slots 2
and 3: block 0, the query, block 1, the wait, a barrier, the query reads, a barrier, and
only then block 2, which must not be copied over the query before it was read.
"""

from __future__ import annotations

import numpy as np
import pytest

import test_split_plan_model as plan

RING = 4
DEPTH = 3            # blocks issued ahead of the one being computed
BLK = 32
QUERY_SLOTS = (2, 3)  # where a unit's first query is staged (bf16 rows)


class Stream:
    def __init__(self, pieces, redo_pieces=(), guard_empty=True, query_lds=False):
        self.pieces = [max(0, -(-(t1 - t0) // BLK)) if t1 > t0 else 0 for (t0, t1) in pieces]
        self.redo = set(redo_pieces)
        self.guard_empty = guard_empty
        self.bar = 0                      # barriers passed so far (interval index)
        self.issued = 0
        self.landed = 0
        self.issue_at = {}                # block -> interval of its copy
        self.land_at = {}                 # block -> interval in which it was waited for
        self.reads = {}                   # block -> intervals of its reads
        self.zero_at = {}                 # block -> interval of its tail zeroing
        self.stage = []                   # (interval, slot) of epilogue staging
        self.slot_hist = {s: [] for s in range(RING)}
        self.query_lds = query_lds
        self.query_reads = []             # intervals in which the staged query was read
        self.query_copied_at = None

    # ---- events ----
    def barrier(self):
        self.bar += 1

    def issue(self, x):
        s = x % RING
        # the slot's previous block must be finished, and no staging in this interval
        prev = [y for y in self.slot_hist[s]]
        for y in prev:
            for r in self.reads.get(y, []):
                assert r < self.bar, f"copy of block {x} in interval {self.bar} while block {y} is read there"
        for (e, ss) in self.stage:
            if ss == s:
                assert e < self.bar, f"copy of block {x} into slot {s} during epilogue staging"
        if s in QUERY_SLOTS and self.query_copied_at is not None:
            assert self.query_reads and all(e < self.bar for e in self.query_reads), \
                f"copy of block {x} into slot {s} before the staged query was read"
        self.slot_hist[s].append(x)
        self.issue_at[x] = self.bar

    def land_upto(self, n):
        for x in range(self.landed, n):
            assert x in self.issue_at, f"wait counts block {x} as landed, but it was never issued"
            self.land_at.setdefault(x, self.bar)
        self.landed = max(self.landed, n)

    def read(self, x):
        assert x in self.land_at and self.land_at[x] < self.bar, \
            f"block {x} read in interval {self.bar} before a barrier after its wait ({self.land_at.get(x)})"
        if x in self.zero_pending:
            assert self.zero_at[x] < self.bar, f"block {x} read before its tail was zeroed"
        for (e, slot) in self.stage:
            assert not (slot == x % RING and self.land_at[x] <= e < self.bar), \
                f"block {x} read after the epilogue staged over its slot"
        self.reads.setdefault(x, []).append(self.bar)

    def zero(self, x):
        assert x < self.landed, f"tail of block {x} zeroed before its copy landed"
        assert not self.reads.get(x), f"tail of block {x} zeroed after it was read"
        self.zero_at[x] = self.bar

    def staging(self, slot):
        # no copy in flight into the slot (reads after it are checked in read())
        for y in self.slot_hist[slot]:
            assert y < self.landed, f"staging over block {y} still in flight"
        self.stage.append((self.bar, slot))

    # ---- the kernel's walk ----
    def run(self):
        P = self.pieces
        self.zero_pending = set()
        cur, nxt, nxt_known = 0, None, False
        ic_piece, ic_j, g0 = 0, 0, 0

        def next_copy():
            nonlocal ic_piece, ic_j
            if ic_piece == 0 and ic_j >= P[cur]:
                if not nxt_known or nxt is None:
                    return None
                ic_piece, ic_j = 1, 0
            if ic_piece == 1 and ic_j >= P[nxt]:
                return None
            x = self.issued
            self.issue(x)
            self.issued += 1
            ic_j += 1
            return x

        while True:
            nblk = P[cur]
            if self.query_lds and self.issued == 0:
                next_copy()                         # block 0
                for s in QUERY_SLOTS:               # the query copy: nothing of the ring there
                    assert not self.slot_hist[s], "query staged over a ring block"
                self.query_copied_at = self.bar
                before_q = self.issued
                next_copy()                         # block 1
                self.land_upto(before_q)            # the query and block 0 have landed
                self.barrier()
                self.query_reads.append(self.bar)   # score waves read their query
                self.barrier()
                next_copy()                         # block 2, into the query's slot
            else:
                for _ in range(DEPTH):
                    if self.issued >= g0 + DEPTH:
                        break
                    next_copy()
            nxt = cur + 1 if cur + 1 < len(P) else None
            nxt_known = True
            if (nblk > 0 or not self.guard_empty) and self.landed <= g0:
                self.land_upto(g0 + 1)
            for attempt in range(2):
                if attempt > 0 and nblk > 0:
                    # drop the stream's copies and restage the piece from block 0
                    self.land_upto(self.issued)
                    ic_piece, ic_j = 0, 0
                    g0 = self.issued
                    for _ in range(DEPTH):
                        next_copy()
                    self.land_upto(self.issued)
                if nblk == 1:
                    self.zero_pending.add(g0)
                    self.zero(g0)
                self.barrier()                      # block 0 visible
                for j in range(nblk):
                    g = g0 + j
                    self.read(g)                    # QK(j)
                    if j == 0 and attempt == 0:
                        self.barrier()              # reference-max exchange
                    if j > 0:
                        next_copy()                 # copy of stream block g+2 ...
                        self.read(g - 1)            # ... spread over PV(j-1)
                    if self.issued > g + 1:
                        self.land_upto(g + 2)
                        if j + 2 == nblk:
                            self.zero_pending.add(g + 1)
                            self.zero(g + 1)
                    self.barrier()                  # Y(j)
                if nblk > 0:
                    next_copy()
                    self.read(g0 + nblk - 1)        # last PV
                self.barrier()
                self.barrier()                      # slack vote
                if not (cur in self.redo and attempt == 0):
                    break
                self.barrier()
                self.barrier()                      # restart reference exchanged
            self.barrier()                          # row sums
            slot = (g0 + nblk + 3) % RING
            self.staging(slot)
            self.barrier()                          # stats and P free
            if nxt is None:
                break
            g0 += nblk
            cur, nxt_known = nxt, False
            if ic_piece == 1:
                ic_piece = 0
            else:
                ic_j = 0
        return True


def stream_pieces(seq, n_streams):
    sq, pieces, _, _ = plan.plan_auto(list(seq), n_streams, 10 ** 9, False)
    by = {}
    for (s, b, t0, t1, ns, slot) in pieces:
        by.setdefault(s, []).append((t0, t1))
    return by


def _cases():
    rng = np.random.default_rng(71)
    out = []
    seq = rng.integers(0, 300, size=600) * (rng.random(600) > 0.1)
    out.append(("many short, some empty", seq, 128))
    out.append(("many short, 256 streams", seq, 256))
    out.append(("long", np.full(32, 8192), 128))
    out.append(("lognormal", np.minimum(rng.lognormal(7.5, 1.0, 64).astype(int), 40000), 256))
    for k in range(12):
        n = int(rng.integers(1, 80))
        s = rng.integers(0, 3000, size=n) * (rng.random(n) > 0.3)
        out.append((f"random {k}", s, int(rng.choice([8, 16, 64, 128, 256]))))
    return out


@pytest.mark.parametrize("query_lds", [False, True], ids=["query in registers", "query staged in LDS"])
@pytest.mark.parametrize("name,seq,n_streams", _cases(), ids=[c[0] for c in _cases()])
def test_block_stream_orders_copies_waits_and_reads(name, seq, n_streams, query_lds):
    for s, pcs in stream_pieces(seq, n_streams).items():
        Stream(pcs, query_lds=query_lds).run()


def test_model_catches_block_2_copied_over_the_unread_query():
    """Issuing block 2 before the barrier that follows the query reads would copy it over
    the staged query: the model must reject that order."""
    st = Stream([(0, 9 * BLK)], query_lds=True)
    st.query_copied_at = 0
    st.query_reads.append(1)
    st.issue(0)
    st.bar = 1                                   # still the interval of the query reads
    with pytest.raises(AssertionError):
        st.issue(2)


def test_block_stream_with_redone_pieces():
    rng = np.random.default_rng(72)
    seq = rng.integers(0, 700, size=300) * (rng.random(300) > 0.2)
    for s, pcs in stream_pieces(seq, 64).items():
        redo = [i for i in range(len(pcs)) if rng.random() < 0.3]
        Stream(pcs, redo_pieces=redo).run()
        Stream(pcs, redo_pieces=redo, query_lds=True).run()


def test_model_catches_an_empty_piece_claiming_the_next_block():
    """Without the guard, an empty piece followed by a short one claims the short piece's
    first block as landed before its copy is issued: the model must reject that."""
    pcs = [(0, 9 * BLK), (0, 0), (0, 2 * BLK)]
    Stream(pcs).run()
    with pytest.raises(AssertionError):
        Stream(pcs, guard_empty=False).run()

"""The host-side paged cache allocator ("How the Ascend Computing Platform Achieves Same-Day
Inference Adaptation for Ultra-Large Sparse Models", §3.1, §3.2, §4.3), checked on the CPU.

The reference is the meaning of a paged cache: every sequence must read back, through its page
table, exactly the tokens written to it, whatever forks (shared prefixes), copy-on-write, growth
and frees happened in between. A simulated device memory (one token id per slot) is driven by
the allocator's page tables and copy-on-write pairs; reference counts, free-page accounting and
the coalescing of free runs are recomputed from scratch after every operation.
"""
import numpy as np
import pytest

from indexer_top_sparse_amd import binding as B


def _runs(free):
    """Maximal runs of consecutive page numbers in the set `free`."""
    runs, prev = [], None
    for p in sorted(free):
        if prev is not None and p == prev + 1:
            runs[-1][1] += 1
        else:
            runs.append([p, 1])
        prev = p
    return runs


class Sim:
    def __init__(self, pages, P, reserve=0):
        self.pool = B.Pool(pages, P, reserve)
        self.P, self.pages = P, pages
        self.mem = np.full((pages, P), -1, dtype=np.int64)  # token id per slot
        self.want = {}                                     # seq -> expected token ids
        self.next_tok = 0

    def new(self):
        s = self.pool.new()
        self.want[s] = []
        return s

    def fork(self, parent):
        s = self.pool.fork(parent)
        self.want[s] = list(self.want[parent])
        return s

    def append(self, s, n, urgent=False):
        old = len(self.want[s])
        cow = self.pool.reserve(s, old + n, urgent)
        for src, dst in cow:
            self.mem[dst] = self.mem[src]
        pt = self.pool.page_table(s)
        for t in range(old, old + n):
            self.mem[pt[t // self.P], t % self.P] = self.next_tok
            self.want[s].append(self.next_tok)
            self.next_tok += 1
        return cow

    def free(self, s):
        self.pool.free(s)
        del self.want[s]

    def check(self):
        held = {}
        for s, toks in self.want.items():
            pt = self.pool.page_table(s)
            assert self.pool.length(s) == len(toks)
            assert len(pt) == -(-len(toks) // self.P)
            got = [int(self.mem[pt[t // self.P], t % self.P]) for t in range(len(toks))]
            assert got == toks, f"sequence {s} reads back other tokens"
            for p in pt:
                held[p] = held.get(p, 0) + 1
        for p in range(self.pages):
            assert self.pool.refcount(p) == held.get(p, 0), f"page {p}"
        free = set(range(self.pages)) - set(held)
        f, r, m = self.pool.stats()
        runs = _runs(free)
        assert f == len(free)
        assert r == len(runs), "free runs are not coalesced"
        assert m == max([n for _, n in runs], default=0)


def test_random_operations_keep_every_sequence_intact():
    rng = np.random.default_rng(0)
    sim = Sim(pages=96, P=8, reserve=4)
    live = [sim.new()]
    for step in range(600):
        op = rng.random()
        if op < 0.45 and live:
            s = live[rng.integers(len(live))]
            try:
                sim.append(s, int(rng.integers(1, 20)))
            except B.SaError as e:
                assert e.status == B.SA_ERR_WORKSPACE  # pool exhausted: nothing changed
        elif op < 0.65 and live:
            live.append(sim.fork(live[rng.integers(len(live))]))
        elif op < 0.85 and len(live) > 1:
            s = live.pop(rng.integers(len(live)))
            sim.free(s)
        else:
            live.append(sim.new())
        sim.check()
    for s in live:
        sim.free(s)
    sim.check()
    assert sim.pool.stats() == (96, 1, 96)


def test_copy_on_write_only_for_a_shared_partial_page():
    sim = Sim(pages=16, P=4)
    a = sim.new()
    sim.append(a, 6)                 # pages: one full, one half full
    b = sim.fork(a)
    assert sim.append(b, 1)          # b writes into the shared half page: copy first
    assert not sim.append(a, 2)      # a's page is no longer shared
    c = sim.fork(a)                  # a holds 8 tokens: its pages are full
    assert not sim.append(c, 3)      # the next token opens a new page: nothing to copy
    sim.check()
    pa, pb = sim.pool.page_table(a), sim.pool.page_table(b)
    assert pa[0] == pb[0] and pa[1] != pb[1]  # the full first page stays shared
    assert sim.pool.refcount(pa[0]) == 3


def test_growth_prefers_the_next_page_then_best_fit():
    pool = B.Pool(32, 4)
    a, b, c = pool.new(), pool.new(), pool.new()
    pool.reserve(a, 12)              # pages 0-2
    pool.reserve(b, 20)              # pages 3-7
    pool.reserve(c, 12)              # pages 8-10
    assert pool.page_table(a) == [0, 1, 2]
    pool.reserve(a, 16)              # page 3 belongs to b: the only free run (11..31) serves
    assert pool.page_table(a) == [0, 1, 2, 11]
    pool.free(b)                     # a hole of 5 pages (3..7)
    d = pool.new()
    pool.reserve(d, 16)              # 4 pages: the 5-page hole fits better than 12..31
    assert pool.page_table(d) == [3, 4, 5, 6]
    pool.reserve(c, 16)              # page 11 belongs to a: best fit for one page is page 7
    assert pool.page_table(c) == [8, 9, 10, 7]
    pool.reserve(a, 20)              # page 12 follows a's last page and is free
    assert pool.page_table(a) == [0, 1, 2, 11, 12]


def test_emergency_reserve_only_for_urgent_requests():
    pool = B.Pool(10, 4, emergency_pages=3)
    a = pool.new()
    pool.reserve(a, 28)              # 7 pages: the 3 reserved remain
    with pytest.raises(B.SaError) as e:
        pool.reserve(a, 29)
    assert e.value.status == B.SA_ERR_WORKSPACE
    assert pool.length(a) == 28      # a failed request changes nothing
    pool.reserve(a, 40, urgent=True)
    assert pool.stats()[0] == 0
    with pytest.raises(B.SaError):
        pool.reserve(a, 41, urgent=True)


def test_free_runs_merge_and_split():
    pool = B.Pool(12, 2)
    s = [pool.new() for _ in range(6)]
    for x in s:
        pool.reserve(x, 4)           # two pages each: 0-1, 2-3, ..., 10-11
    assert pool.stats() == (0, 0, 0)
    pool.free(s[1])
    pool.free(s[3])
    assert pool.stats() == (4, 2, 2)  # two separate holes
    pool.free(s[2])
    assert pool.stats() == (6, 1, 6)  # 2..7 merged into one run
    t = pool.new()
    pool.reserve(t, 2)               # one page: the run is split
    assert pool.stats() == (5, 1, 5)


def test_invalid_calls():
    pool = B.Pool(4, 4)
    with pytest.raises(B.SaError):
        pool.free(7)
    with pytest.raises(B.SaError):
        pool.fork(3)
    with pytest.raises(B.SaError):
        B.Pool(0, 4)
    with pytest.raises(B.SaError):
        B.Pool(4, 4, emergency_pages=5)

"""Pins of the oracle's policy and compact work queue.

The compact queue holds tasks only for non-empty (row, KV head, split)
intervals, and the split ranges follow the true row lengths (PersistentKV
page, Methodology 1, "Row-Local Bounds" and "Compact Workqueue").  These
tests check the oracle builder against brute-force enumeration of every
(row, head, chunk) candidate on small grids and against the invariants that
follow: the items of each (row, head) tile [0, L_b) disjointly, no item is
empty, the count is sum_b ceil(L_b / C) * Hkv (split) or #non-empty rows *
Hkv (no split), and the partial slots of split items are distinct and dense.
"""

import itertools

import numpy as np
import pytest

from oracle import work_queue as wq
from paged_kv_attention_persistent_amd import workloads


def brute_force(lens, hkv, C, split):
    out = []
    for b, L in enumerate(lens):
        for h in range(hkv):
            nch = (max(1, -(-L // C)) if split else 1)
            for c in range(nch + 2):           # over-enumerate, then filter
                lo, hi = (c * C, min(L, (c + 1) * C)) if split else ((0, L) if c == 0 else (0, 0))
                if hi > lo:
                    out.append((b, h, c, lo, hi))
    return out


def check_invariants(q, lens, hkv, C):
    items = q["items"]
    assert items.dtype.itemsize == 16
    cover = {}
    for it in items:
        b, h, lo, hi = int(it["seq"]), int(it["kv_head"]), int(it["tok_begin"]), int(it["tok_end"])
        assert hi > lo, "empty item"
        if q["split"]:
            assert lo % C == 0 and hi - lo <= C and int(it["chunk"]) == lo // C
        cover.setdefault((b, h), []).append((lo, hi))
    for b, L in enumerate(lens):
        for h in range(hkv):
            segs = sorted(cover.get((b, h), []))
            if L == 0:
                assert not segs
                continue
            assert segs[0][0] == 0 and segs[-1][1] == L
            for (a0, a1), (b0, b1) in zip(segs, segs[1:]):
                assert a1 == b0, "gap or overlap"
            assert len(segs) == q["n_chunks"][b]
    # partial slots: distinct and dense over split items
    slots = [wq.partial_slot(it, q["part_off"], hkv) for it in items
             if q["n_chunks"][int(it["seq"])] > 1]
    assert sorted(slots) == list(range(len(slots)))
    assert q["part_off"][-1] * hkv == len(slots)
    assert list(q["merge_rows"]) == [b for b, L in enumerate(lens) if q["n_chunks"][b] != 1]


@pytest.mark.parametrize("split", [False, True])
def test_brute_force_small_grids(split):
    pol = wq.POLICY_SPLIT if split else wq.POLICY_NO_SPLIT
    for lens in itertools.product([0, 1, 15, 16, 17, 32, 33, 64], repeat=2):
        for hkv in (1, 3):
            q = wq.build_queue(list(lens), hkv, 256, 16, pol)
            got = [tuple(int(x) for x in it) for it in q["items"]]
            assert got == brute_force(list(lens), hkv, 16, split)
            check_invariants(q, list(lens), hkv, 16)


def test_policy_decisions_on_the_workloads():
    C, cus = 4096, 256
    t = workloads.tiny()
    assert not wq.decide_split(t.ctx_lens, 1, cus, C)
    lc = workloads.long_context()
    q = wq.build_queue(lc.ctx_lens, 8, cus, C)
    assert q["split"] and len(q["items"]) == 256 and q["n_chunks"][0] == 32
    mx = workloads.mixed()
    q = wq.build_queue(mx.ctx_lens, 8, cus, C)
    assert q["split"]
    assert len(q["items"]) == 8 * sum(-(-int(L) // C) for L in mx.ctx_lens)
    check_invariants(q, list(mx.ctx_lens), 8, C)
    sh = workloads.many_short()
    q = wq.build_queue(sh.ctx_lens, 8, cus, C)
    assert not q["split"] and len(q["items"]) == 512


def test_policy_boundaries():
    # fewer units than CUs and a row longer than one chunk -> split
    assert wq.decide_split([4097], 8, 256, 4096)
    assert not wq.decide_split([4096], 8, 256, 4096)      # fits one chunk
    assert not wq.decide_split([10 ** 6] * 32, 8, 256, 4096)   # 256 units fill 256 CUs
    assert wq.decide_split([10 ** 6] * 31, 8, 256, 4096)
    assert not wq.decide_split([], 8, 256, 4096)
    assert wq.decide_split([1], 8, 256, 4096, wq.POLICY_SPLIT)
    assert not wq.decide_split([10 ** 6], 8, 256, 4096, wq.POLICY_NO_SPLIT)


def test_lpt_order_is_a_stable_length_sort():
    lens = [5000, 100, 9000, 0, 4096]
    can = wq.build_queue(lens, 2, 256, 4096, wq.POLICY_SPLIT)
    lpt = wq.build_queue(lens, 2, 256, 4096, wq.POLICY_SPLIT, wq.ORDER_LPT)
    a = [tuple(int(x) for x in it) for it in can["items"]]
    b = [tuple(int(x) for x in it) for it in lpt["items"]]
    assert sorted(a) == sorted(b)
    want = sorted(a, key=lambda r: (-(r[4] - r[3]), a.index(r)))
    assert b == want
    for x, y in zip(b, b[1:]):
        assert x[4] - x[3] >= y[4] - y[3]


def test_item_bytes_little_endian():
    q = wq.build_queue([70000], 1, 256, 4096, wq.POLICY_SPLIT)
    raw = q["items"].tobytes()
    it = q["items"][17]
    off = 17 * 16
    assert int.from_bytes(raw[off:off + 4], "little") == int(it["seq"]) == 0
    assert int.from_bytes(raw[off + 6:off + 8], "little") == 17
    assert int.from_bytes(raw[off + 8:off + 12], "little") == 17 * 4096
    assert int.from_bytes(raw[off + 12:off + 16], "little") == min(70000, 18 * 4096)


# Chunk mode "fit": pins by closed forms, independent of the search.

def test_fit_chunk_one_row_is_the_ceiling_of_pages_over_the_budget():
    # one row of n pages and a budget of K ranges: T = ceil(n / K) (floor 1 here)
    for n, hkv, cus in [(8192, 8, 256), (8191, 8, 256), (100, 1, 7), (1, 4, 256), (33, 2, 8)]:
        K = max(1, cus // hkv)
        assert wq.fit_chunk([16 * n], hkv, cus, min_pages=1) == 16 * (-(-n // K))
        assert wq.fit_chunk([16 * n - 5], hkv, cus, min_pages=1) == 16 * (-(-n // K))
        assert wq.fit_chunk([16 * n], hkv, cus) == 16 * max(wq.FIT_MIN_PAGES, -(-n // K))
        assert wq.fit_chunk([16 * n], hkv, cus, min_pages=wq.FIT_MIN_PAGES_LOOP) == 16 * max(64, -(-n // K))


def test_fit_chunk_equal_rows():
    # B equal rows of n pages: each row gets floor(K / B) ranges, T = ceil(n / floor(K / B))
    for B, n in [(2, 1000), (3, 64), (5, 17), (16, 4096)]:
        K = 256 // 8
        assert wq.fit_chunk([16 * n] * B, 8, 256, min_pages=1) == 16 * (-(-n // (K // B)))
        assert wq.fit_chunk([16 * n] * B, 8, 256) == 16 * max(wq.FIT_MIN_PAGES, -(-n // (K // B)))


def test_fit_chunk_fallback_and_edges():
    assert wq.fit_chunk([], 8, 256, min_pages=1) == 16
    assert wq.fit_chunk([0, 0], 8, 256, min_pages=1) == 16
    assert wq.fit_chunk([], 8, 256) == 16 * wq.FIT_MIN_PAGES
    # more non-empty rows than the budget: no T fits, T = longest row
    assert wq.fit_chunk([16 * 5] * 40, 8, 256, min_pages=1) == 16 * 5
    assert wq.fit_chunk([16 * 500] * 40, 8, 256) == 16 * 500


def test_fit_mode_on_the_workloads():
    cus = 256
    t = workloads.tiny()
    q = wq.build_queue(t.ctx_lens, 1, cus, 0)
    assert not q["split"] and len(q["items"]) == 1 and q["chunk_tokens"] == 16 * wq.FIT_MIN_PAGES
    lc = workloads.long_context()
    q = wq.build_queue(lc.ctx_lens, 8, cus, 0)
    assert q["chunk_tokens"] == 4096 and len(q["items"]) == 256       # same as the fixed 4096
    for seed in (workloads.MEASURE_SEED, workloads.CALIBRATION_SEED):
        mx = workloads.mixed(seed)
        q = wq.build_queue(mx.ctx_lens, 8, cus, 0)
        C = q["chunk_tokens"]
        assert q["split"] and len(q["items"]) <= cus                  # one round
        check_invariants(q, list(mx.ctx_lens), 8, C)
        # a range one page shorter would need a second round
        pages = [-(-int(L) // 16) for L in mx.ctx_lens]
        assert sum(-(-n // (C // 16 - 1)) for n in pages) * 8 > cus
    sh = workloads.many_short()
    q = wq.build_queue(sh.ctx_lens, 8, cus, 0)
    assert not q["split"] and len(q["items"]) == 512


def test_fit_mode_brute_force_small_grids():
    # the fitted queue equals the fixed-chunk queue at the chunk it reports
    for lens in itertools.product([0, 1, 16, 17, 1500, 5000], repeat=3):
        for hkv, cus in [(1, 4), (2, 8), (1, 2)]:
            q = wq.build_queue(list(lens), hkv, cus, 0, wq.POLICY_SPLIT)
            C = q["chunk_tokens"]
            got = [tuple(int(x) for x in it) for it in q["items"]]
            assert got == brute_force(list(lens), hkv, C, True)
            fits = sum(1 for L in lens if L) <= max(1, cus // hkv)
            if fits:         # at most one range per workgroup
                assert len(got) <= max(max(1, cus // hkv) * hkv, sum(1 for L in lens if L) * hkv)
                if C > 1024:  # chosen by the bound, not the floor: one page less would not fit
                    assert sum(-(-(-(-L // 16)) // (C // 16 - 1)) for L in lens) > max(1, cus // hkv)


def test_a_row_needing_more_than_65535_ranges_is_an_error():
    # the item's range index is a 16-bit field: 65535 ranges encode, 65536 do not
    ok = wq.build_queue([65535 * 16], 1, 256, 16, wq.POLICY_SPLIT)
    assert ok["n_chunks"][0] == 65535 and int(ok["items"]["chunk"].max()) == 65534
    with pytest.raises(ValueError):
        wq.build_queue([65535 * 16 + 1], 1, 256, 16, wq.POLICY_SPLIT)

"""Host-side decode planner (lazyattn_decode_plan): CPU checks of the plan it
writes, through the C ABI (the planner is host code; no GPU is used).

A plan must cover every (sequence, KV head, table block) exactly once, give
each run of a sequence its own partial slot (the same run for every KV head),
cut runs only where the rules allow, put only runs that hold the same blocks
(with one offset each, and not a sequence's last) into one item, and place
the items of one (document, KV head) on one XCD (workgroup i runs on XCD
i mod 8)."""

import ctypes
from collections import defaultdict

import numpy as np
import pytest
import torch

import position_agnostic_kv_amd as pak
import workloads as W

XCDS = 8
INTS = 12


def _plan(table, lens, hq, hkv, max_item_blocks=0):
    return pak.decode_plan(torch.from_numpy(np.ascontiguousarray(table).view(np.int32)),
                           torch.from_numpy(np.asarray(lens, dtype=np.int32)), hq, hkv,
                           max_item_blocks=max_item_blocks)


def _decode_items(plan):
    ints = plan.ints.numpy()
    base = (plan.batch + 3) // 4 * 4
    counts = ints[:plan.batch]
    rows = ints[base:].reshape(-1, INTS)
    assert rows.shape[0] == plan.num_items
    items = []
    for r in rows.tolist():
        g, nmem = r[0] & 0xFFFF, r[0] >> 16
        assert r[3] == 0
        members = [(m & 0xFFFF, m >> 16) for m in r[4:4 + nmem]]
        starts = r[8:8 + nmem]
        assert all(m == 0 for m in r[4 + nmem:8] + r[8 + nmem:12])
        assert starts[0] == r[1], "the first member's start is the item's"
        items.append((g, nmem, r[1], r[2], members, starts))
    return counts, items


def _check_plan(table, lens, hq, hkv, max_item_blocks=0):
    """The plan's invariants; returns (counts, items, runs per sequence)."""
    table = np.asarray(table, dtype=np.uint32)
    plan = _plan(table, lens, hq, hkv, max_item_blocks)
    counts, items = _decode_items(plan)
    b_count, width = table.shape
    limit = max_item_blocks or 128
    most = min(4, 16 // (hq // hkv))
    nblk = [0 if (n < 0 or n > 16 * width) else -(-int(n) // 16) for n in lens]
    covered = defaultdict(int)
    runs = defaultdict(dict)          # b -> slot -> (start, end clipped)
    for g, nmem, start, end, members, starts in items:
        assert 0 <= g < hkv and 1 <= nmem <= most
        assert len({b for b, _ in members}) == nmem, "members are distinct sequences"
        assert 0 <= start <= end <= width
        for (b, slot), st in zip(members, starts):
            assert 0 <= b < b_count and 0 <= slot < counts[b]
            clipped = (st, min(st + end - start, nblk[b]))
            assert runs[b].setdefault(slot, clipped) == clipped, "one slot, one run, every KV head"
            for j in range(*clipped):
                covered[(b, g, j)] += 1
        if nmem > 1:
            ids = {tuple((table[b, st:st + end - start] & 0xFFFF).tolist()) for (b, _), st in zip(members, starts)}
            assert len(ids) == 1, "members read the same blocks"
            for (b, slot), st in zip(members, starts):
                assert len(set((table[b, st:st + end - start] >> 16).tolist())) == 1, "one offset over the run"
                assert slot < counts[b] - 1 and st + end - start <= nblk[b], "not the sequence's last run"
    for b in range(b_count):
        assert counts[b] == len(runs[b]) >= 1
        spans = sorted(runs[b].values())
        if nblk[b] == 0:
            assert spans == [(0, 0)]
            continue
        assert spans[0][0] == 0 and spans[-1][1] == nblk[b]
        for (s0, e0), (s1, _) in zip(spans, spans[1:]):
            assert e0 == s1, "runs are consecutive"
            edge = (table[b, s1] >> 16) != (table[b, s1 - 1] >> 16)
            assert e0 - s0 == limit or (edge and e0 - s0 >= 4), "a cut needs a document edge or the size limit"
        # the last run's items reach the end of the row
        last = max(runs[b], key=lambda s: runs[b][s][0])
        ends = {end for g, n, st, end, mem, _ in items if (b, last) in mem}
        assert ends == {width}
    want = {(b, g, j) for b in range(b_count) for g in range(hkv) for j in range(nblk[b])}
    assert set(covered) == want and all(v == 1 for v in covered.values())
    assert plan.max_items_per_seq == max(counts)
    return counts, items, runs


def test_plan_of_the_zipf_reuse_decode_workload():
    """The full Zipf mix: 128 sequences, 32 q / 8 KV heads.  Shared documents
    are read by items of up to four sequences; every (first block, KV head)
    group sits on one XCD, and the XCDs' loads are balanced."""
    case = W.make("zipf_reuse_decode")
    table = case.layout.table
    counts, items, runs = _check_plan(table, case.seq_lens, case.num_q_heads, case.num_kv_heads)
    groups = defaultdict(set)
    load = np.zeros(XCDS)
    for p, (g, nmem, start, end, members, _) in enumerate(items):
        b = members[0][0]
        groups[(int(table[b, start]) & 0xFFFF, g)].add(p % XCDS)
        load[p % XCDS] += min(end, -(-int(case.seq_lens[b]) // 16)) - start + 2
    assert all(len(x) == 1 for x in groups.values())
    assert load.max() / load.mean() < 1.05
    shared = sum(it[1] for it in items if it[1] > 1)
    assert shared > 0.5 * sum(it[1] for it in items)
    assert max(it[1] for it in items) == 4


@pytest.mark.parametrize("hq", [4, 8, 16, 32, 64])
def test_runs_follow_document_edges(hq):
    """Documents of 1..12 blocks shared by several sequences; members per
    item up to min(4, 16 / G)."""
    case = W.zipf_decode(seed=31, batch=12, catalogue=20, docs_per_seq=(2, 6), doc_blocks=(1, 12),
                         num_q_heads=hq, num_kv_heads=4)
    _, items, _ = _check_plan(case.layout.table, case.seq_lens, hq, 4)
    assert max(it[1] for it in items) == min(4, 16 // (hq // 4))


@pytest.mark.parametrize("limit", [1, 4, 7, 64])
def test_runs_respect_the_size_limit(limit):
    case = W.make("llama8b_decode")
    _, _, runs = _check_plan(case.layout.table[:6], case.seq_lens[:6], 8, 2, max_item_blocks=limit)
    for b in range(6):
        assert all(e - s <= limit for s, e in runs[b].values())


def test_empty_invalid_and_ragged_sequences():
    """Length 0, a negative length, a length past the table, and ragged
    documents: the first three get one empty item per head (the kernel
    writes zeros or NaN through it)."""
    case = W.ragged_case(41, "decode", 6, 8, 2, 128, docs_per_seq=(1, 4), doc_len=(1, 300), catalogue=5)
    table = case.layout.table
    lens = case.seq_lens.copy()
    lens[1] = 0
    lens[3] = -5
    lens[4] = 16 * table.shape[1] + 1
    counts, items, _ = _check_plan(table, lens, 8, 2)
    for b in (1, 3, 4):
        assert counts[b] == 1
        mine = [it for it in items if any(m[0] == b for m in it[4])]
        assert len(mine) == 2 and all(it[1] == 1 and it[2] == 0 and it[3] == table.shape[1] for it in mine)


def test_block_frame_tables():
    """Offsets that change at every block (each block carries its own first
    position): runs of 4 blocks, none shared."""
    case = W.make("llama8b_decode")
    table = W.block_frame_table(case.layout)[:4]
    _, items, runs = _check_plan(table, case.seq_lens[:4], 4, 1)
    sizes = [e - s for b in range(4) for s, e in runs[b].values()]
    assert max(sizes) == 4 and np.median(sizes) == 4
    assert all(it[1] == 1 for it in items)


def test_planner_errors():
    lib = pak.load_library()
    table = np.zeros((2, 4), dtype=np.uint32)
    lens = np.array([16, 30], dtype=np.int32)
    buf = np.zeros(256, dtype=np.int32)
    n, m = ctypes.c_int(0), ctypes.c_int(0)

    def call(tab=table.ctypes.data, ln=lens.ctypes.data, batch=2, width=4, hq=8, hkv=2, limit=0,
             out=buf.ctypes.data, cap=256, pn=ctypes.byref(n), pm=ctypes.byref(m)):
        return lib.lazyattn_decode_plan(ctypes.c_void_p(tab), ctypes.c_void_p(ln), batch, width, hq, hkv, limit,
                                        ctypes.c_void_p(out), cap, pn, pm)

    assert call() == 0 and n.value == 4 and m.value == 1
    assert call(batch=0) == -3
    assert call(hkv=0) == -3
    assert call(hq=6) == -3                   # group 3: not a power of two
    assert call(hq=7) == -3                   # not a multiple of the KV heads
    assert call(hq=64) == -3                  # groups up to 16
    assert call(limit=-1) == -3
    assert call(limit=5000) == -3
    assert call(width=5000) == -3
    assert call(tab=0) == -1
    assert call(out=0) == -1
    assert call(pn=None) == -1
    assert call(cap=4 + INTS * 3) == -4       # room for 3 of the 4 items
    assert call(cap=4 + INTS * 4) == 0
    assert lib.lazyattn_decode_plan_ints(2, 4, 2) == 4 + INTS * 2 * 4 * 2
    assert lib.lazyattn_decode_plan_ints(0, 4, 2) == 0

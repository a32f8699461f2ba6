"""Host-side decode planner (lazyattn_decode_plan): CPU checks of the plan it
writes, through the C ABI (the planner is host code; no GPU is used).

A plan must cover every (sequence, KV head, table block) exactly once, give
each run of a sequence its own partial slot (the same slot for every KV
head), cut runs only where the rules allow, and put the items of one shared
(document, KV head) on one XCD (workgroup i runs on XCD i mod 8)."""

import ctypes
from collections import defaultdict

import numpy as np
import pytest
import torch

import position_agnostic_kv_amd as pak
import workloads as W

XCDS = 8


def _items(plan):
    ints = plan.ints.numpy()
    base = (plan.batch + 3) // 4 * 4
    counts = ints[:plan.batch]
    items = ints[base:].reshape(-1, 4)
    assert items.shape[0] == plan.num_items
    return counts, items


def _plan(table, lens, hkv, max_item_blocks=0):
    return pak.decode_plan(torch.from_numpy(np.ascontiguousarray(table).view(np.int32)),
                           torch.from_numpy(np.asarray(lens, dtype=np.int32)), hkv,
                           max_item_blocks=max_item_blocks)


def _check_plan(table, lens, hkv, max_item_blocks=0):
    """The plan's invariants; returns (counts, items, runs per sequence)."""
    table = np.asarray(table, dtype=np.uint32)
    plan = _plan(table, lens, hkv, max_item_blocks)
    counts, items = _items(plan)
    b_count, width = table.shape
    limit = max_item_blocks or 128
    nblk = [0 if (n < 0 or n > 16 * width) else -(-int(n) // 16) for n in lens]
    covered = defaultdict(int)
    runs = defaultdict(dict)          # b -> slot -> (start, end clipped)
    for b, g, z, end in items.tolist():
        assert 0 <= b < b_count and 0 <= g < hkv
        slot, start = z & 0xFFFF, z >> 16
        assert 0 <= slot < counts[b]
        assert 0 <= start <= end <= width
        clipped = (start, min(end, nblk[b]))
        assert runs[b].setdefault(slot, clipped) == clipped, "one slot, one run, every KV head"
        for j in range(*clipped):
            covered[(b, g, j)] += 1
    for b in range(b_count):
        assert counts[b] == max(1, len(runs[b])) == len(runs[b])
        spans = sorted(runs[b].values())
        if nblk[b] == 0:
            assert spans == [(0, 0)]
            continue
        assert spans[0][0] == 0 and spans[-1][1] == nblk[b]
        for (s0, e0), (s1, _) in zip(spans, spans[1:]):
            assert e0 == s1, "runs are consecutive"
            n = e0 - s0
            offset_change = (table[b, s1] >> 16) != (table[b, s1 - 1] >> 16)
            assert n == limit or (offset_change and n >= 4), "a cut needs a document edge or the size limit"
        # the last item of a sequence reaches the end of the row
        last = max(runs[b], key=lambda s: runs[b][s][0])
        ends = {int(e) for bb, g, z, e in items.tolist() if bb == b and (z & 0xFFFF) == last}
        assert ends == {width}
    want = {(b, g, j) for b in range(b_count) for g in range(hkv) for j in range(nblk[b])}
    assert set(covered) == want and all(v == 1 for v in covered.values())
    assert plan.max_items_per_seq == max(counts)
    return counts, items, runs


def test_plan_of_the_zipf_reuse_decode_workload():
    """The full Zipf mix: 128 sequences, 8 KV heads.  Every (first block, KV
    head) group sits on one XCD, and the queues are balanced."""
    case = W.make("zipf_reuse_decode")
    table = case.layout.table
    counts, items, runs = _check_plan(table, case.seq_lens, case.num_kv_heads)
    groups = defaultdict(set)
    load = np.zeros(XCDS)
    for p, (b, g, z, e) in enumerate(items.tolist()):
        groups[(int(table[b, z >> 16]) & 0xFFFF, g)].add(p % XCDS)
        load[p % XCDS] += min(e, -(-int(case.seq_lens[b]) // 16)) - (z >> 16)
    assert all(len(x) == 1 for x in groups.values())
    assert load.max() / load.mean() < 1.05
    # documents are shared: fewer groups than items
    assert len(groups) < 0.5 * len(items)


def test_runs_follow_document_edges():
    """Documents of 1..12 blocks: cuts at document edges once a run holds 4
    blocks; shorter documents ride along with their neighbours."""
    case = W.zipf_decode(seed=31, batch=12, catalogue=20, docs_per_seq=(2, 6), doc_blocks=(1, 12),
                         num_q_heads=16, num_kv_heads=4)
    _check_plan(case.layout.table, case.seq_lens, 4)


@pytest.mark.parametrize("limit", [1, 4, 7, 64])
def test_runs_respect_the_size_limit(limit):
    case = W.make("llama8b_decode")
    counts, _, runs = _check_plan(case.layout.table[:6], case.seq_lens[:6], 2, max_item_blocks=limit)
    for b in range(6):
        for s, e in runs[b].values():
            assert e - s <= limit + 3   # a short last run joins the one before


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
    counts, items, _ = _check_plan(table, lens, 2)
    for b in (1, 3, 4):
        assert counts[b] == 1
        mine = [tuple(x) for x in items.tolist() if x[0] == b]
        assert len(mine) == 2 and all(z == 0 and e == table.shape[1] for _, _, z, e in mine)


def test_block_frame_tables():
    """Offsets that change at every block (each block carries its own first
    position): runs of 4 blocks."""
    case = W.make("llama8b_decode")
    table = W.block_frame_table(case.layout)[:4]
    _, _, runs = _check_plan(table, case.seq_lens[:4], 1)
    sizes = [e - s for b in range(4) for s, e in runs[b].values()]
    assert max(sizes) <= 7 and np.median(sizes) == 4


def test_planner_errors():
    lib = pak.load_library()
    table = np.zeros((2, 4), dtype=np.uint32)
    lens = np.array([16, 30], dtype=np.int32)
    buf = np.zeros(64, dtype=np.int32)
    n, m = ctypes.c_int(0), ctypes.c_int(0)

    def call(tab=table.ctypes.data, ln=lens.ctypes.data, batch=2, width=4, hkv=2, limit=0, out=buf.ctypes.data,
             cap=64, pn=ctypes.byref(n), pm=ctypes.byref(m)):
        return lib.lazyattn_decode_plan(ctypes.c_void_p(tab), ctypes.c_void_p(ln), batch, width, hkv, limit,
                                        ctypes.c_void_p(out), cap, pn, pm)

    assert call() == 0 and n.value == 4 and m.value == 1
    assert call(batch=0) == -3
    assert call(hkv=0) == -3
    assert call(limit=-1) == -3
    assert call(limit=5000) == -3
    assert call(width=5000) == -3
    assert call(tab=0) == -1
    assert call(out=0) == -1
    assert call(pn=None) == -1
    assert call(cap=4 + 4 * 3) == -4          # room for 3 of the 4 items
    assert call(cap=4 + 4 * 4) == 0
    assert lib.lazyattn_decode_plan_ints(2, 4, 2) == 4 + 4 * 2 * 4 * 2
    assert lib.lazyattn_decode_plan_ints(0, 4, 2) == 0

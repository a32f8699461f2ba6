"""Host logic of the input generators (no attention arithmetic): ragged
layouts place every document from a fresh block, record how many slots of
each block hold tokens, and count lengths in table slots."""

import numpy as np

import oracle
import workloads as W


def test_ragged_layout_counts_and_positions():
    for kind in ("decode", "prefill"):
        case = W.ragged_case(7, kind, 5, 8, 2, 64, (1, 6), (1, 400), prompt=(1, 90), catalogue=9,
                             offsets="random")
        lay = case.layout
        assert lay.block_fill.dtype == np.uint8 and lay.block_fill.shape == (lay.num_blocks,)
        for b in range(case.batch):
            row = lay.table[b]
            vs = oracle.valid_slots(row, case.seq_lens[b], lay.block_fill)
            assert vs.size == lay.total_lens[b]          # every token once, no slot too many
            # documents start at slot multiples of 16, in order, and fill
            # ceil(len / 16) blocks; the appended tail follows them
            col = 0
            for _, ln, off in lay.doc_spans[b]:
                nb = -(-ln // 16)
                ids = (row[col:col + nb] & np.uint32(0xFFFF)).astype(np.int64)
                assert np.all(row[col:col + nb] >> np.uint32(16) == off)
                assert lay.block_fill[ids[-1]] == ln - 16 * (nb - 1)
                assert np.all(lay.block_fill[ids[:-1]] == 16)
                col += nb
            assert case.seq_lens[b] == 16 * col + lay.tail_lens[b]
            tail_ids = (row[col:col + -(-int(lay.tail_lens[b]) // 16)] & np.uint32(0xFFFF)).astype(np.int64)
            assert int(lay.block_fill[tail_ids].astype(int).sum()) == lay.tail_lens[b]


def test_ragged_catalogue_has_edge_lengths_and_sharing():
    case = W.ragged_case(3, "decode", 6, 8, 2, 64, (3, 5), (1, 200), catalogue=8)
    lens = {d: ln for spans in case.layout.doc_spans for d, ln, _ in spans}
    assert {lens[d] for d in lens if d < 6} <= {1, 15, 16, 17, 31, 33}
    used = [d for spans in case.layout.doc_spans for d, _, _ in spans]
    assert len(used) > len(set(used))                   # some document is shared
    # a shared document is stored once: its table words name the same blocks
    first = {}
    for b, spans in enumerate(case.layout.doc_spans):
        col = 0
        for d, ln, _ in spans:
            nb = -(-ln // 16)
            ids = tuple((case.layout.table[b, col:col + nb] & np.uint32(0xFFFF)).tolist())
            assert first.setdefault(d, ids) == ids
            col += nb


def test_block_frame_table_on_ragged_layout():
    case = W.ragged_case(11, "prefill", 3, 8, 2, 64, (2, 4), (1, 100), prompt=(1, 40))
    lay = case.layout
    t = W.block_frame_table(lay)
    for b in range(case.batch):
        col = 0
        for _, ln, off in lay.doc_spans[b]:
            nb = -(-ln // 16)
            assert np.all((t[b, col:col + nb] >> np.uint32(16)) == off + 16 * np.arange(nb))
            col += nb
        # positions of the valid slots run off, off+1, ... within each document
        pos = oracle.key_positions(t[b], case.seq_lens[b], lay.block_fill)
        assert pos.size == lay.total_lens[b]


def test_fp8_lane_order_is_a_permutation_and_round_trips():
    from workloads import _fp8_lane_order
    ks, vs = _fp8_lane_order()
    assert sorted(ks.tolist()) == list(range(2048)) and sorted(vs.tolist()) == list(range(2048))
    rng = np.random.default_rng(1)
    k = rng.integers(0, 256, size=(3, 2, 16, 128)).astype(np.uint8)
    v = rng.integers(0, 256, size=(3, 2, 16, 128)).astype(np.uint8)
    kd, vd = W.fp8_pools_to_device_order(k, v)
    k2, v2 = W.fp8_pools_from_device_order(kd, vd)
    assert np.array_equal(k, k2) and np.array_equal(v, v2)
    # spot checks of the documented order: byte 1024 i + 16 l + x
    i, lane, x = 1, 37, 11            # g = 2, t = 5
    assert kd[0, 0].reshape(-1)[1024 * i + 16 * lane + x] == k[0, 0, 5, 32 * 2 + 16 * i + x]
    assert vd[0, 0].reshape(-1)[1024 * i + 16 * lane + x] == v[0, 0, 4 * 2 + x % 4, 16 * (4 * i + x // 4) + 5]

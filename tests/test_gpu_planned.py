"""GPU parity of the planned decode (lazyattn_decode_planned): the decode cut
at document boundaries by the host planner, with the sequences that share a
document reading it together.

* Shared-document (Zipf) batches at query-group sizes 1..16 against the
  oracle, twice (bit-identical repeats).
* Bit-level: on a table without offsets (no document cuts) and with the
  run-size limit equal to a split size, the plan's runs are exactly the
  uniform splits, so the output must equal lazyattn_decode's bit for bit;
  likewise one run per sequence against one split per sequence.
* Ragged documents (fill counts), an empty sequence (zeros) and an
  impossible length (NaN), small run limits (many partial slots), a plan
  built before the sequences grew by a block, and the full Zipf mix on
  sampled (sequence, head) rows as bench.py runs it.
"""

import numpy as np
import pytest
import torch

import oracle
import position_agnostic_kv_amd as pak
import workloads as W
from tests.gpu_helpers import DeviceCase, assert_parity, oracle_decode, say
from tests.test_gpu_parity import _gather

pytestmark = pytest.mark.gpu


def _planned(dc, case, plan, seq_lens=None, table=None):
    out = pak.lazyattn_decode_planned(dc.q, dc.q_pos, dc.k_pool, dc.v_pool, dc.table if table is None else table,
                                      dc.seq_lens if seq_lens is None else seq_lens, plan, scale=case.scale,
                                      rope_theta=case.rope_theta, block_fill=dc.fill)
    torch.cuda.synchronize()
    return out


def _bits(t):
    return t.view(torch.int16).clone()


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 4), (16, 4), (32, 4), (64, 4)])
def test_planned_shared_documents(hq, hkv):
    g = hq // hkv
    case = W.zipf_decode(seed=40 + g, batch=14, catalogue=24, docs_per_seq=(2, 6), doc_blocks=(1, 14),
                         num_q_heads=hq, num_kv_heads=hkv)
    say(f"[planned] zipf G{g} Hq{hq} Hkv{hkv} B{case.batch} NB{case.layout.num_blocks}")
    W.materialize_numpy(case)
    dc = DeviceCase(case)
    dc.append()
    plan = pak.decode_plan(dc.table, dc.seq_lens, hq, hkv)
    assert plan.max_items_per_seq > 1
    out = _planned(dc, case, plan)
    again = _planned(dc, case, plan)
    assert torch.equal(_bits(out), _bits(again)), "planned decode is not deterministic"
    assert_parity(W.to_float(out, case.dtype), oracle_decode(case), case.dtype, f"planned G{g}")


@pytest.mark.parametrize("limit", [8, 0])
def test_planned_runs_equal_to_splits_are_bit_identical(limit):
    """Zero offsets: runs are cut only at the size limit, so the runs are the
    uniform splits and the kernel sees the same partials."""
    ctx = [16 * 44, 16 * 23, 16 * 21, 16 * 12]   # + the new token: 45, 24, 22, 13 blocks
    case = W.decode_case(47, len(ctx), 16, 4, 128, ctx, (2, 9), offsets="random")
    W.materialize_numpy(case)
    dc = DeviceCase(case)
    dc.append()
    table0 = (dc.table & 0xFFFF).contiguous()
    plan = pak.decode_plan(table0, dc.seq_lens, 16, 4, max_item_blocks=limit)
    split = limit if limit else 1024
    say(f"[planned] bit-identical runs of {split} blocks, {plan.num_items} items")
    want = pak.lazyattn_decode(dc.q, dc.q_pos, dc.k_pool, dc.v_pool, table0, dc.seq_lens, scale=case.scale,
                               rope_theta=case.rope_theta, split_blocks=split)
    got = _planned(dc, case, plan, table=table0)
    assert torch.equal(_bits(got), _bits(want))


def test_planned_ragged_empty_and_invalid():
    case = W.ragged_case(48, "decode", 9, 16, 4, 128, docs_per_seq=(2, 5), doc_len=(1, 400), catalogue=7,
                         offsets="random")
    W.materialize_numpy(case)
    dc = DeviceCase(case)
    dc.append()
    lens = case.seq_lens.copy()
    lens[2] = 0
    lens[5] = 16 * case.layout.table.shape[1] + 3
    dlens = torch.from_numpy(lens.astype(np.int32)).to(dc.q.device)
    plan = pak.decode_plan(dc.table, dlens, 16, 4, max_item_blocks=6)
    say(f"[planned] ragged, {plan.num_items} items, up to {plan.max_items_per_seq} slots")
    out = W.to_float(_planned(dc, case, plan, seq_lens=dlens), case.dtype)
    assert np.all(out[2] == 0)
    assert np.all(np.isnan(out[5]))
    keep = [b for b in range(case.batch) if b not in (2, 5)]
    want = oracle_decode(case)
    assert_parity(out[keep], want[keep], case.dtype, "planned ragged")


def test_planned_plan_survives_growth():
    """A plan built while every sequence was one block shorter covers the
    appended block: its last run reaches the end of the row."""
    case = W.zipf_decode(seed=49, batch=10, catalogue=16, docs_per_seq=(2, 5), doc_blocks=(2, 10),
                         num_q_heads=32, num_kv_heads=8)
    W.materialize_numpy(case)
    dc = DeviceCase(case)
    dc.append()
    short = torch.from_numpy(case.layout.cached_lens.astype(np.int32)).to(dc.q.device)  # before the new token
    plan = pak.decode_plan(dc.table, short, 32, 8)
    out = _planned(dc, case, plan)
    assert_parity(W.to_float(out, case.dtype), oracle_decode(case), case.dtype, "planned after growth")


def test_full_size_zipf_planned_sampled():
    """The full Zipf mix, as bench.py runs it: against lazyattn_decode on every
    row, and against the oracle on sampled (sequence, head) rows."""
    case = W.make("zipf_reuse_decode")
    say(f"[planned] full zipf B={case.batch} NB={case.layout.num_blocks}")
    W.materialize_torch(case, "cuda:0")
    dc = DeviceCase(case)
    rng = np.random.default_rng(4)
    seqs = sorted(rng.choice(case.batch, size=4, replace=False).tolist())
    kp, vp, tab, fill = _gather(dc, case, seqs)
    dc.append()
    plan = pak.decode_plan(dc.table, dc.seq_lens, case.num_q_heads, case.num_kv_heads)
    got_t = _planned(dc, case, plan)
    ref_t = dc.decode()
    torch.cuda.synchronize()
    got = W.to_float(got_t, case.dtype)
    assert np.all(np.isfinite(got))
    assert_parity(got, W.to_float(ref_t, case.dtype), case.dtype, "planned vs per-sequence decode")
    q = W.to_float(case.q, case.dtype)
    g = case.num_q_heads // case.num_kv_heads
    rows_got, rows_want = [], []
    for i, b in enumerate(seqs):
        for h in rng.choice(case.num_q_heads, size=3, replace=False).tolist():
            rows_want.append(oracle.decode_one(q[b, h], int(case.q_pos[b]), kp, vp, tab[i], int(case.seq_lens[b]),
                                               h // g, case.scale, case.rope_theta, block_fill=fill))
            rows_got.append(got[b, h])
    assert_parity(np.stack(rows_got), np.stack(rows_want), case.dtype, "planned zipf sampled")

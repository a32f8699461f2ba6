"""GPU parity at the format's limits.

The table word gives block ids and offsets 16 bits each, so a pool holds at
most 65536 blocks and positions reach 65535; a table row of 4096 blocks
spans the whole position range.  Here:

* the pool has exactly 65536 blocks, and the table uses ids 0 and 65535;
* one sequence fills the widest row (4096 blocks, 65521 or 65536 slots) with
  documents at random offsets, the last of which ends at position 65535;
* the query (decode) or the prompt's last row (prefill) sits at 65535;
* a second sequence is a single token at position 65535 in block 65535.

Decode (automatic split, and the planned decode) and prefill are compared
with the oracle on every head of both sequences, using host copies of only
the blocks the sequences use.
"""

import numpy as np
import pytest
import torch

import oracle
import position_agnostic_kv_amd as pak
import workloads as W
from tests.gpu_helpers import DeviceCase, assert_parity, say
from tests.test_gpu_parity import _gather

pytestmark = pytest.mark.gpu

MAX_BLOCKS = 65536
WIDTH = 4096            # blocks of the widest row: 65536 slots
LAST = 65535            # the largest position


def _limits_case(kind, seed):
    rng = np.random.default_rng(seed)
    prompt = 1 if kind == "decode" else 96
    cached = WIDTH * 16 - 16 if kind == "decode" else WIDTH * 16 - prompt
    lens, left = [], cached
    while left:
        ln = min(16 * int(rng.integers(16, 129)), left)
        lens.append(ln)
        left -= ln
    offs = [int(rng.integers(0, LAST + 2 - ln)) for ln in lens]
    offs[-1] = LAST + 1 - lens[-1]                       # the last document ends at 65535
    doc_lens = lens + [16]
    seq_docs = [list(range(len(lens))), [len(lens)]]     # sequence 1: one 16-token document
    tails = [prompt, 1]
    tail_pos = [LAST + 1 - prompt, LAST]
    used_blocks = sum(-(-ln // 16) for ln in doc_lens) + sum(-(-t // 16) for t in tails)
    lay = W.build_layout(rng, seq_docs, doc_lens, tails, offsets=[offs, [0]], tail_pos=tail_pos,
                         spare_blocks=MAX_BLOCKS - used_blocks)
    assert lay.num_blocks == MAX_BLOCKS and lay.table.shape[1] == WIDTH
    # put ids 65535 and 0 into use: sequence 1's new-token block and sequence 0's first block
    perm = np.arange(MAX_BLOCKS, dtype=np.int64)

    def assign(old, new):   # perm[old] = new, perm stays a permutation
        x = int(np.nonzero(perm == new)[0][0])
        perm[old], perm[x] = new, perm[old]

    assign(int(lay.slot_mapping[-1]) // 16, MAX_BLOCKS - 1)
    assign(int(lay.table[0, 0]) & 0xFFFF, 0)
    ids = (lay.table & np.uint32(0xFFFF)).astype(np.int64)
    lay.table = ((lay.table & np.uint32(0xFFFF0000)) | perm[ids].astype(np.uint32)).astype(np.uint32)
    sm = lay.slot_mapping.astype(np.int64)
    lay.slot_mapping = (perm[sm // 16] * 16 + sm % 16).astype(np.int32)
    case = W.Case(f"limits_{kind}", kind, W.BF16, 4, 1, 128, 5.0e5, lay, seed=seed)
    W.materialize_numpy(case)
    used = set((lay.table[0, :WIDTH] & 0xFFFF).tolist()) | {int(lay.table[1, 0]) & 0xFFFF, int(lay.table[1, 1]) & 0xFFFF}
    assert {0, MAX_BLOCKS - 1} <= used
    return case


def test_decode_at_the_limits():
    case = _limits_case("decode", 61)
    say(f"[limits decode] seq_lens={case.seq_lens.tolist()} q_pos={case.q_pos.tolist()} NB={case.layout.num_blocks}")
    dc = DeviceCase(case)
    kp, vp, tab, fill = _gather(dc, case, [0, 1])
    dc.append()
    got = W.to_float(dc.decode(), case.dtype)
    plan = pak.decode_plan(dc.table, dc.seq_lens, case.num_q_heads, case.num_kv_heads)
    got_planned = W.to_float(pak.lazyattn_decode_planned(dc.q, dc.q_pos, dc.k_pool, dc.v_pool, dc.table,
                                                         dc.seq_lens, plan, scale=case.scale,
                                                         rope_theta=case.rope_theta), case.dtype)
    torch.cuda.synchronize()
    q = W.to_float(case.q, case.dtype)
    want = np.stack([np.stack([oracle.decode_one(q[b, h], int(case.q_pos[b]), kp, vp, tab[b], int(case.seq_lens[b]),
                                                 0, case.scale, case.rope_theta, block_fill=fill)
                               for h in range(case.num_q_heads)]) for b in range(2)])
    assert_parity(got, want, case.dtype, "decode at the limits")
    assert_parity(got_planned, want, case.dtype, "planned decode at the limits")


def test_prefill_at_the_limits():
    case = _limits_case("prefill", 62)
    say(f"[limits prefill] kv_lens={case.seq_lens.tolist()} prompts={case.layout.tail_lens.tolist()} "
        f"first={case.layout.tail_pos.tolist()}")
    dc = DeviceCase(case)
    kp, vp, tab, fill = _gather(dc, case, [0, 1])
    dc.append()
    got = W.to_float(dc.prefill(), case.dtype)
    torch.cuda.synchronize()
    q = W.to_float(case.q, case.dtype)
    want = oracle.prefill(q, case.cu_q_lens, case.layout.tail_pos, kp, vp, tab, case.seq_lens, case.scale,
                          case.rope_theta, block_fill=fill)
    assert_parity(got, want, case.dtype, "prefill at the limits")

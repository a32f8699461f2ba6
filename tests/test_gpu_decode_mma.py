"""GPU parity of the matrix-core decode kernel that bf16 pools with head_dim
128 take (decode_mma16_kernel): every query-group size from 1 to 64 under the
three position schemes (lazy RoPE, the eager baseline, ALiBi) against the
oracle, plus what only a bit-level check can see:

* repeated calls on the same inputs give bit-identical outputs (the block
  maximum once read matrix-core results before they were written, which
  showed up only as run-to-run rounding differences);
* the eager kernel on a table with cleared offsets equals the lazy kernel bit
  for bit;
* degenerate and invalid inputs in bf16: a one-token sequence returns its V
  row exactly, an empty sequence zeros, an impossible length or a table entry
  outside the pool NaN for that sequence only; splits whose last workgroup
  gives some waves no block at all."""

import numpy as np
import pytest
import torch

import oracle
import position_agnostic_kv_amd as pak
import workloads as W
from tests.gpu_helpers import DEV, DeviceCase, assert_parity, host_pools_after_append, say

pytestmark = pytest.mark.gpu

GROUPS = [
    # Hq, Hkv, ctx per sequence, doc blocks, offsets, split
    (8, 8, [640, 208, 1008], (2, 12), "random", 4),
    (16, 8, [1024, 96], (2, 20), "contiguous", 0),
    (16, 4, [512, 1504, 48], (1, 9), "random", 5),
    (64, 8, [2048, 336], (4, 16), "random", 8),
    (32, 2, [800, 112], (2, 10), "contiguous", 4),
    (32, 1, [704, 208], (2, 12), "random", 0),
    (64, 1, [480, 32], (2, 6), "contiguous", 6),
    # multi-query kernel: block streams of unequal length, single-block sequences
    (32, 4, [1504, 16, 336], (1, 9), "random", 5),
    (64, 1, [16, 48, 1008], (1, 3), "contiguous", 0),
    (64, 2, [2048, 272], (2, 30), "random", 7),
]


def _run(fn, dc, case, table, split, **kw):
    out = fn(dc.q, dc.q_pos, dc.k_pool, dc.v_pool, table, dc.seq_lens, scale=case.scale, split_blocks=split, **kw)
    torch.cuda.synchronize()
    return out


def _bits(t):
    return t.view(torch.int16).clone()


@pytest.mark.parametrize("hq,hkv,ctx,docs,offs,split", GROUPS)
def test_mma_decode_modes_and_determinism(hq, hkv, ctx, docs, offs, split):
    g = hq // hkv
    case = W.decode_case(301 + hq + 7 * hkv, len(ctx), hq, hkv, 128, ctx, docs, offsets=offs)
    say(f"[mma decode] G{g} Hq{hq} Hkv{hkv} ctx={ctx} {offs} split={split}")
    W.materialize_numpy(case)
    dc = DeviceCase(case)
    dc.append()
    kp, vp = host_pools_after_append(case)
    q = W.to_float(case.q, case.dtype)

    # lazy RoPE, twice
    lazy = _run(pak.lazyattn_decode, dc, case, dc.table, split, rope_theta=case.rope_theta)
    again = _run(pak.lazyattn_decode, dc, case, dc.table, split, rope_theta=case.rope_theta)
    assert torch.equal(_bits(lazy), _bits(again)), "lazy decode is not deterministic"
    want = oracle.decode(q, case.q_pos, kp, vp, case.layout.table, case.seq_lens, case.scale, case.rope_theta)
    assert_parity(W.to_float(lazy, case.dtype), want, case.dtype, f"mma lazy G{g}")

    # the eager baseline ignores offsets; on a cleared table lazy computes the same
    zero_host = (np.asarray(case.layout.table, dtype=np.uint32) & np.uint32(0xFFFF)).astype(np.uint32)
    zero_dev = (dc.table & 0xFFFF).contiguous()
    eager = _run(pak.lazyattn_decode_eager, dc, case, dc.table, split, rope_theta=case.rope_theta)
    eager2 = _run(pak.lazyattn_decode_eager, dc, case, dc.table, split, rope_theta=case.rope_theta)
    assert torch.equal(_bits(eager), _bits(eager2)), "eager decode is not deterministic"
    want0 = oracle.decode(q, case.q_pos, kp, vp, zero_host, case.seq_lens, case.scale, case.rope_theta)
    assert_parity(W.to_float(eager, case.dtype), want0, case.dtype, f"mma eager G{g}")
    lazy0 = _run(pak.lazyattn_decode, dc, case, zero_dev, split, rope_theta=case.rope_theta)
    assert torch.equal(_bits(eager), _bits(lazy0)), "eager != lazy on a zero-offset table"

    # ALiBi on block-frame offsets
    table = W.block_frame_table(case.layout)
    slopes = (oracle.alibi_slopes(hq) * 4.0).astype(np.float32)
    tab_dev = torch.from_numpy(table.view(np.int32)).to(DEV)
    sl_dev = torch.from_numpy(slopes).to(DEV)
    ali = pak.lazyattn_decode_alibi(dc.q, dc.q_pos, dc.k_pool, dc.v_pool, tab_dev, dc.seq_lens, sl_dev,
                                    scale=case.scale, split_blocks=split)
    ali2 = pak.lazyattn_decode_alibi(dc.q, dc.q_pos, dc.k_pool, dc.v_pool, tab_dev, dc.seq_lens, sl_dev,
                                     scale=case.scale, split_blocks=split)
    torch.cuda.synchronize()
    assert torch.equal(_bits(ali), _bits(ali2)), "ALiBi decode is not deterministic"
    wanta = oracle.decode_alibi(q, case.q_pos, kp, vp, table, case.seq_lens, case.scale, slopes)
    assert_parity(W.to_float(ali, case.dtype), wanta, case.dtype, f"mma alibi G{g}")


@pytest.mark.parametrize("hq,hkv", [(8, 2), (16, 1)])
def test_mma_decode_degenerate_and_invalid(hq, hkv):
    # 6 blocks per sequence (5 cached + the new token's); split 4 leaves a last
    # split of 2 blocks, so two of its four waves get none
    case = W.decode_case(331 + hq, 4, hq, hkv, 128, [80, 80, 80, 80], (1, 3))
    W.materialize_numpy(case)
    dc = DeviceCase(case)
    dc.append()
    g = hq // hkv
    say(f"[mma degenerate] G{g} Hq{hq} Hkv{hkv}")
    need = pak.decode_workspace_size(4, hq, hkv, 128, case.layout.table.shape[1], 4)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=DEV)
    a = dc.decode(split_blocks=4, workspace=ws)
    torch.cuda.synchronize()
    assert_parity(W.to_float(a, case.dtype), _oracle(case), case.dtype, f"mma short splits G{g}")
    a = a.clone()

    lens = torch.tensor([1, 0, -3, 16 * case.layout.table.shape[1] + 1], dtype=torch.int32, device=DEV)
    out = dc.decode(split_blocks=4, workspace=ws, seq_lens=lens)
    torch.cuda.synchronize()
    o = W.to_float(out, case.dtype)
    vp = W.to_float(case.v_pool, case.dtype)
    first = int(case.layout.table[0, 0]) & 0xFFFF
    for h in range(hq):
        assert np.array_equal(o[0, h], vp[first, h // g, 0]), "a one-token sequence must return its value exactly"
    assert np.all(o[1] == 0), "an empty sequence must give zeros"
    assert np.all(np.isnan(o[2])) and np.all(np.isnan(o[3])), "an impossible length must give NaN"

    # a table entry outside the pool poisons its own sequence only, whichever
    # wave of the workgroup meets it
    for blk in (0, 1, 2, 3, 5):
        tab = dc.table.clone()
        tab[2, blk] = (tab[2, blk] & ~0xFFFF) | 0xFFF0
        bad = pak.lazyattn_decode(dc.q, dc.q_pos, dc.k_pool, dc.v_pool, tab, dc.seq_lens, scale=case.scale,
                                  rope_theta=case.rope_theta, split_blocks=4, workspace=ws)
        torch.cuda.synchronize()
        ob = W.to_float(bad, case.dtype)
        assert np.all(np.isnan(ob[2])), f"block {blk} outside the pool must give NaN"
        assert np.array_equal(np.delete(ob, 2, axis=0), np.delete(W.to_float(a, case.dtype), 2, axis=0))
    c = dc.decode(split_blocks=4, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(_bits(c), _bits(a)), "a poisoned call changed a later result"


def _oracle(case):
    kp, vp = host_pools_after_append(case)
    return oracle.decode(W.to_float(case.q, case.dtype), case.q_pos, kp, vp, case.layout.table, case.seq_lens,
                         case.scale, case.rope_theta)


def test_mma_decode_split_counts_agree():
    """One input at several split sizes (each a different partition of the
    blocks over workgroups and waves) and at the automatic choice."""
    case = W.decode_case(351, 2, 32, 8, 128, [3008, 1504], (4, 24), offsets="random")
    W.materialize_numpy(case)
    dc = DeviceCase(case)
    dc.append()
    want = _oracle(case)
    outs = []
    for split in (4, 7, 16, 33, 0, 1024):
        out = dc.decode(split_blocks=split)
        torch.cuda.synchronize()
        got = W.to_float(out, case.dtype)
        assert_parity(got, want, case.dtype, f"mma split {split}")
        outs.append(got)
    for got in outs[1:]:
        assert np.abs(got - outs[0]).max() <= 2e-2

"""GPU parity with per-block fill counts: documents whose token count is not
a multiple of 16, so each document's last block is partly filled and the next
document starts a fresh block (block_fill says how many slots hold tokens;
lengths count table slots).  Decode, prefill, the non-lazy baseline and the
ALiBi variant against the fill-aware oracle; also arbitrary counts 0..16 on
every block (holes anywhere, including the new token's own block) and the
equivalence of an all-full fill array with none at all.

Documents draw lengths from 1 token up, with the edge lengths 1, 15, 16, 17,
31 and 33 always present; some documents are shared between sequences."""

import numpy as np
import pytest
import torch

import oracle
import position_agnostic_kv_amd as pak
import workloads as W
from tests.gpu_helpers import DEV, DeviceCase, assert_parity, host_pools_after_append, say

pytestmark = pytest.mark.gpu


def _case(seed, kind, hq, hkv, d, batch, docs, doc_len, offsets="contiguous", catalogue=None,
          prompt=(1, 300), dtype=W.BF16):
    case = W.ragged_case(seed, kind, batch, hq, hkv, d, docs, doc_len, prompt=prompt,
                         catalogue=catalogue, dtype=dtype, offsets=offsets)
    W.materialize_numpy(case)
    return case


def _q(case):
    return W.to_float(case.q, case.dtype)


DECODE = [
    # D, Hq, Hkv, batch, docs/seq, doc length, offsets, split, catalogue, dtype
    (128, 32, 8, 4, (2, 6), (1, 700), "contiguous", 0, None, W.BF16),
    (128, 32, 8, 5, (3, 8), (1, 90), "contiguous", 4, 12, W.BF16),
    (128, 16, 2, 3, (2, 5), (1, 1500), "random", 5, None, W.BF16),
    (128, 64, 1, 3, (1, 4), (1, 400), "contiguous", 0, 6, W.BF16),
    (64, 8, 8, 4, (2, 5), (1, 300), "random", 0, None, W.BF16),
    (128, 8, 2, 3, (2, 4), (1, 200), "contiguous", 4, None, W.F32),
]


@pytest.mark.parametrize("d,hq,hkv,batch,docs,dlen,offs,split,cat,dtype", DECODE)
def test_ragged_decode(d, hq, hkv, batch, docs, dlen, offs, split, cat, dtype):
    case = _case(101 + d + hq + batch, "decode", hq, hkv, d, batch, docs, dlen, offs, cat, dtype=dtype)
    say(f"[ragged decode] D{d} Hq{hq} Hkv{hkv} B{batch} docs={docs} len={dlen} {offs} split={split} "
        f"{dtype} slots={case.seq_lens.tolist()} tokens={case.layout.total_lens.tolist()}")
    dc = DeviceCase(case)
    dc.append()
    out = dc.decode(split_blocks=split)
    torch.cuda.synchronize()
    kp, vp = host_pools_after_append(case)
    want = oracle.decode(_q(case), case.q_pos, kp, vp, case.layout.table, case.seq_lens, case.scale,
                         case.rope_theta, block_fill=case.block_fill)
    assert_parity(W.to_float(out, dtype), want, dtype, f"ragged decode D{d} G{hq // hkv} split={split}")


def test_ragged_decode_eager_and_alibi():
    case = _case(131, "decode", 32, 8, 128, 4, (2, 6), (1, 500), "random")
    say("[ragged decode eager + alibi] D128 Hq32 Hkv8 B4")
    dc = DeviceCase(case)
    dc.append()
    kp, vp = host_pools_after_append(case)
    zero = (dc.table & 0xFFFF).contiguous()
    out = pak.lazyattn_decode_eager(dc.q, dc.q_pos, dc.k_pool, dc.v_pool, dc.table, dc.seq_lens,
                                    scale=case.scale, rope_theta=case.rope_theta, block_fill=dc.fill)
    lazy = pak.lazyattn_decode(dc.q, dc.q_pos, dc.k_pool, dc.v_pool, zero, dc.seq_lens,
                               scale=case.scale, rope_theta=case.rope_theta, block_fill=dc.fill)
    torch.cuda.synchronize()
    want = oracle.decode(_q(case), case.q_pos, kp, vp, (case.layout.table & np.uint32(0xFFFF)),
                         case.seq_lens, case.scale, case.rope_theta, block_fill=case.block_fill)
    assert_parity(W.to_float(out, case.dtype), want, case.dtype, "ragged eager decode")
    assert torch.equal(out.view(torch.int16), lazy.view(torch.int16))

    table = W.block_frame_table(case.layout)
    slopes = oracle.alibi_slopes(32).astype(np.float32)
    al = pak.lazyattn_decode_alibi(dc.q, dc.q_pos, dc.k_pool, dc.v_pool,
                                   torch.from_numpy(table.view(np.int32)).to(DEV), dc.seq_lens,
                                   torch.from_numpy(slopes).to(DEV), split_blocks=6, block_fill=dc.fill)
    torch.cuda.synchronize()
    want = oracle.decode_alibi(_q(case), case.q_pos, kp, vp, table, case.seq_lens, case.scale, slopes,
                               block_fill=case.block_fill)
    assert_parity(W.to_float(al, case.dtype), want, case.dtype, "ragged alibi decode")


PREFILL = [
    # D, Hq, Hkv, batch, docs/seq, doc length, prompt, offsets, catalogue
    (128, 32, 8, 3, (2, 5), (1, 600), (1, 300), "contiguous", None),
    (128, 8, 2, 4, (3, 7), (1, 80), (100, 260), "contiguous", 10),
    (128, 8, 1, 2, (1, 3), (1, 1200), (120, 140), "random", None),
    (64, 8, 4, 3, (2, 4), (1, 300), (1, 200), "random", None),
    (128, 4, 4, 3, (0, 2), (1, 50), (1, 40), "contiguous", None),
]


@pytest.mark.parametrize("d,hq,hkv,batch,docs,dlen,prompt,offs,cat", PREFILL)
def test_ragged_prefill(d, hq, hkv, batch, docs, dlen, prompt, offs, cat):
    case = _case(151 + d + hq + batch, "prefill", hq, hkv, d, batch, docs, dlen, offs, cat, prompt=prompt)
    say(f"[ragged prefill] D{d} Hq{hq} Hkv{hkv} B{batch} docs={docs} len={dlen} prompt={prompt} {offs} "
        f"q={case.layout.tail_lens.tolist()} slots={case.seq_lens.tolist()}")
    dc = DeviceCase(case)
    dc.append()
    out = dc.prefill()
    torch.cuda.synchronize()
    kp, vp = host_pools_after_append(case)
    want = oracle.prefill(_q(case), case.cu_q_lens, case.layout.tail_pos, kp, vp, case.layout.table,
                          case.seq_lens, case.scale, case.rope_theta, block_fill=case.block_fill)
    assert_parity(W.to_float(out, case.dtype), want, case.dtype, f"ragged prefill D{d} G{hq // hkv}")


def test_ragged_prefill_eager_and_alibi():
    case = _case(171, "prefill", 32, 8, 128, 3, (2, 5), (1, 500), "random", prompt=(60, 200))
    say("[ragged prefill eager + alibi] D128 Hq32 Hkv8 B3")
    dc = DeviceCase(case)
    dc.append()
    kp, vp = host_pools_after_append(case)
    out = pak.lazyattn_prefill_eager(dc.q, dc.cu, dc.q_pos_start, dc.k_pool, dc.v_pool, dc.table,
                                     dc.seq_lens, case.max_q_len, scale=case.scale,
                                     rope_theta=case.rope_theta, block_fill=dc.fill)
    torch.cuda.synchronize()
    want = oracle.prefill(_q(case), case.cu_q_lens, case.layout.tail_pos, kp, vp,
                          case.layout.table & np.uint32(0xFFFF), case.seq_lens, case.scale,
                          case.rope_theta, block_fill=case.block_fill)
    assert_parity(W.to_float(out, case.dtype), want, case.dtype, "ragged eager prefill")

    table = W.block_frame_table(case.layout)
    slopes = (oracle.alibi_slopes(32) * 4.0).astype(np.float32)
    al = pak.lazyattn_prefill_alibi(dc.q, dc.cu, dc.q_pos_start, dc.k_pool, dc.v_pool,
                                    torch.from_numpy(table.view(np.int32)).to(DEV), dc.seq_lens,
                                    case.max_q_len, torch.from_numpy(slopes).to(DEV), block_fill=dc.fill)
    torch.cuda.synchronize()
    want = oracle.prefill_alibi(_q(case), case.cu_q_lens, case.layout.tail_pos, kp, vp, table,
                                case.seq_lens, case.scale, slopes, block_fill=case.block_fill)
    assert_parity(W.to_float(al, case.dtype), want, case.dtype, "ragged alibi prefill")


def _holes(case, seed):
    """Arbitrary counts 0..16 on every block, a quarter of them 0 or 16."""
    rng = np.random.default_rng(seed)
    f = rng.integers(0, 17, size=case.layout.num_blocks).astype(np.uint8)
    pick = rng.random(case.layout.num_blocks)
    f[pick < 0.125] = 0
    f[(pick >= 0.125) & (pick < 0.25)] = 16
    return f


@pytest.mark.parametrize("split", [0, 4, 7])
def test_decode_arbitrary_fill_counts(split):
    case = _case(181 + split, "decode", 32, 8, 128, 4, (2, 6), (16, 600))
    fill = _holes(case, 5 + split)
    # sequence 0: every one of its blocks empty -> zeros
    row0 = case.layout.table[0, :(int(case.seq_lens[0]) + 15) // 16] & np.uint32(0xFFFF)
    fill[row0.astype(np.int64)] = 0
    say(f"[decode holes] split={split} empty blocks={int((fill == 0).sum())}/{fill.size}")
    dc = DeviceCase(case)
    dc.append()
    out = pak.lazyattn_decode(dc.q, dc.q_pos, dc.k_pool, dc.v_pool, dc.table, dc.seq_lens,
                              scale=case.scale, rope_theta=case.rope_theta, split_blocks=split,
                              block_fill=torch.from_numpy(fill).to(DEV))
    torch.cuda.synchronize()
    kp, vp = host_pools_after_append(case)
    want = oracle.decode(_q(case), case.q_pos, kp, vp, case.layout.table, case.seq_lens, case.scale,
                         case.rope_theta, block_fill=fill)
    got = W.to_float(out, case.dtype)
    assert np.all(got[0] == 0) and np.all(want[0] == 0)
    assert_parity(got, want, case.dtype, f"decode holes split={split}")


@pytest.mark.parametrize("alibi", [False, True])
def test_prefill_arbitrary_fill_counts(alibi):
    case = _case(191 + alibi, "prefill", 16, 4, 128, 3, (2, 5), (16, 700), prompt=(100, 300))
    fill = _holes(case, 9 + alibi)
    say(f"[prefill holes] alibi={alibi} empty blocks={int((fill == 0).sum())}/{fill.size}")
    dc = DeviceCase(case)
    dc.append()
    kp, vp = host_pools_after_append(case)
    fd = torch.from_numpy(fill).to(DEV)
    if alibi:
        table = W.block_frame_table(case.layout)
        slopes = oracle.alibi_slopes(16).astype(np.float32)
        out = pak.lazyattn_prefill_alibi(dc.q, dc.cu, dc.q_pos_start, dc.k_pool, dc.v_pool,
                                         torch.from_numpy(table.view(np.int32)).to(DEV), dc.seq_lens,
                                         case.max_q_len, torch.from_numpy(slopes).to(DEV), block_fill=fd)
        want = oracle.prefill_alibi(_q(case), case.cu_q_lens, case.layout.tail_pos, kp, vp, table,
                                    case.seq_lens, case.scale, slopes, block_fill=fill)
    else:
        out = pak.lazyattn_prefill(dc.q, dc.cu, dc.q_pos_start, dc.k_pool, dc.v_pool, dc.table, dc.seq_lens,
                                   case.max_q_len, scale=case.scale, rope_theta=case.rope_theta,
                                   block_fill=fd)
        want = oracle.prefill(_q(case), case.cu_q_lens, case.layout.tail_pos, kp, vp, case.layout.table,
                              case.seq_lens, case.scale, case.rope_theta, block_fill=fill)
    torch.cuda.synchronize()
    got = W.to_float(out, case.dtype)
    say(f"  rows with no visible token: {int((np.abs(want).sum(-1) == 0).sum())}")
    assert_parity(got, want, case.dtype, f"prefill holes alibi={alibi}")


def test_full_fill_array_equals_none():
    """All counts 16 must reproduce the no-fill kernels bit for bit."""
    case = W.decode_case(199, 3, 32, 8, 128, [512, 1024, 96], (2, 10))
    W.materialize_numpy(case)
    dc = DeviceCase(case)
    dc.append()
    full = torch.full((case.layout.num_blocks,), 16, dtype=torch.uint8, device=DEV)
    a = pak.lazyattn_decode(dc.q, dc.q_pos, dc.k_pool, dc.v_pool, dc.table, dc.seq_lens,
                            scale=case.scale, rope_theta=case.rope_theta, split_blocks=4)
    b = pak.lazyattn_decode(dc.q, dc.q_pos, dc.k_pool, dc.v_pool, dc.table, dc.seq_lens,
                            scale=case.scale, rope_theta=case.rope_theta, split_blocks=4, block_fill=full)
    pc = W.prefill_case(198, 2, 32, 8, 128, [512, 96], [256, 77], (2, 12))
    W.materialize_numpy(pc)
    pd = DeviceCase(pc)
    pd.append()
    pfull = torch.full((pc.layout.num_blocks,), 16, dtype=torch.uint8, device=DEV)
    c = pd.prefill()
    e = pak.lazyattn_prefill(pd.q, pd.cu, pd.q_pos_start, pd.k_pool, pd.v_pool, pd.table, pd.seq_lens,
                             pc.max_q_len, scale=pc.scale, rope_theta=pc.rope_theta, block_fill=pfull)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(c.view(torch.int16), e.view(torch.int16))

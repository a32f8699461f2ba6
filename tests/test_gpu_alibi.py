"""GPU parity of the ALiBi variant (lazyattn_decode_alibi / lazyattn_prefill_alibi)
against the ALiBi oracle, on block-frame tables (each block's offset is its
first token's position).  Geometric slopes 2^(-8 (h+1)/Hq), and steeper ones
(x16) that push every head's weights far from uniform; documents placed
contiguously or at random offsets (keys whose positions lie after the query
get positive biases: the running-max and reference paths must cope)."""

import numpy as np
import pytest
import torch

import oracle
import position_agnostic_kv_amd as pak
import workloads as W
from tests.gpu_helpers import DeviceCase, assert_parity, host_pools_after_append, say

pytestmark = pytest.mark.gpu

DECODE = [
    # D, Hq, Hkv, ctx, doc blocks, offsets, slope factor, split
    (128, 32, 8, [512, 1024, 96], (2, 10), "contiguous", 1.0, 0),
    (128, 8, 2, [640, 208], (2, 20), "contiguous", 16.0, 4),
    (128, 64, 8, [2048, 64], (4, 16), "contiguous", 1.0, 8),
    (64, 8, 8, [320, 16, 784], (1, 6), "random", 1.0, 0),
    (128, 32, 1, [400, 96], (2, 9), "contiguous", 1.0, 0),
]


def _slopes(hq, factor):
    return (oracle.alibi_slopes(hq) * factor).astype(np.float32)


@pytest.mark.parametrize("d,hq,hkv,ctx,docs,offs,factor,split", DECODE)
def test_alibi_decode(d, hq, hkv, ctx, docs, offs, factor, split):
    case = W.decode_case(71 + d + hq, len(ctx), hq, hkv, d, ctx, docs, offsets=offs)
    say(f"[alibi decode] D{d} Hq{hq} Hkv{hkv} ctx={ctx} {offs} slopes x{factor} split={split}")
    W.materialize_numpy(case)
    dc = DeviceCase(case)
    dc.append()
    table = W.block_frame_table(case.layout)
    slopes = _slopes(hq, factor)
    out = pak.lazyattn_decode_alibi(dc.q, dc.q_pos, dc.k_pool, dc.v_pool,
                                    torch.from_numpy(table.view(np.int32)).to(dc.q.device), dc.seq_lens,
                                    torch.from_numpy(slopes).to(dc.q.device), split_blocks=split)
    torch.cuda.synchronize()
    kp, vp = host_pools_after_append(case)
    want = oracle.decode_alibi(W.to_float(case.q, case.dtype), case.q_pos, kp, vp, table, case.seq_lens,
                               case.scale, slopes)
    assert_parity(W.to_float(out, case.dtype), want, case.dtype, f"alibi decode D{d} G{hq // hkv}")


PREFILL = [
    # D, Hq, Hkv, cached, prompt, doc blocks, offsets, slope factor
    (128, 32, 8, [512, 96], [256, 77], (2, 12), "contiguous", 1.0),
    (128, 8, 2, [224, 640], [300, 129], (2, 20), "contiguous", 16.0),
    (128, 8, 1, [1056], [130], (3, 40), "contiguous", 1.0),
    (64, 8, 4, [320, 48], [150, 31], (2, 10), "random", 1.0),
    (128, 4, 4, [0, 96], [77, 200], (1, 4), "contiguous", 4.0),
]


@pytest.mark.parametrize("d,hq,hkv,cached,prompt,docs,offs,factor", PREFILL)
def test_alibi_prefill(d, hq, hkv, cached, prompt, docs, offs, factor):
    case = W.prefill_case(73 + d + hq, len(prompt), hq, hkv, d, cached, prompt, docs, offsets=offs)
    say(f"[alibi prefill] D{d} Hq{hq} Hkv{hkv} cached={cached} prompt={prompt} {offs} slopes x{factor}")
    W.materialize_numpy(case)
    dc = DeviceCase(case)
    dc.append()
    table = W.block_frame_table(case.layout)
    slopes = _slopes(hq, factor)
    out = pak.lazyattn_prefill_alibi(dc.q, dc.cu, dc.q_pos_start, dc.k_pool, dc.v_pool,
                                     torch.from_numpy(table.view(np.int32)).to(dc.q.device), dc.seq_lens,
                                     case.max_q_len, torch.from_numpy(slopes).to(dc.q.device))
    torch.cuda.synchronize()
    kp, vp = host_pools_after_append(case)
    want = oracle.prefill_alibi(W.to_float(case.q, case.dtype), case.cu_q_lens, case.layout.tail_pos, kp, vp,
                                table, case.seq_lens, case.scale, slopes)
    assert_parity(W.to_float(out, case.dtype), want, case.dtype, f"alibi prefill D{d} G{hq // hkv}")


def test_alibi_zero_slopes_match_unrotated_rope_baseline():
    """With every slope 0 ALiBi is plain attention on unrotated keys; so is the
    eager RoPE baseline on a table whose offsets are all 0 with the query at
    position 0 (rotation by 0).  Same kernels' arithmetic elsewhere: the two
    must agree to rounding."""
    case = W.decode_case(79, 2, 8, 2, 128, [512, 208], (2, 12))
    W.materialize_numpy(case)
    dc = DeviceCase(case)
    dc.append()
    zero_q = torch.zeros_like(dc.q_pos)
    table = torch.from_numpy(W.block_frame_table(case.layout).view(np.int32)).to(dc.q.device)
    a = pak.lazyattn_decode_alibi(dc.q, dc.q_pos, dc.k_pool, dc.v_pool, table, dc.seq_lens,
                                  torch.zeros(8, dtype=torch.float32, device=dc.q.device))
    b = pak.lazyattn_decode_eager(dc.q, zero_q, dc.k_pool, dc.v_pool, dc.table, dc.seq_lens,
                                  rope_theta=case.rope_theta)
    torch.cuda.synchronize()
    diff = (a.float() - b.float()).abs().max().item()
    say(f"  alibi(0) vs eager rope at 0: max-abs {diff:.3e}")
    assert diff <= 2e-2

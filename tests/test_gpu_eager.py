"""GPU parity of the non-lazy baseline (lazyattn_decode_eager /
lazyattn_prefill_eager) that the method's overhead is measured against.

The baseline takes the pool's keys as already rotated to their absolute
positions and ignores the table's offsets.  Its oracle is therefore the
oracle's own attention with every table offset set to 0 (rot(k, 0) = k), and
the lazy kernel on such a table must give bit-identical results.
"""

import numpy as np
import pytest
import torch

import oracle
import position_agnostic_kv_amd as pak
import workloads as W
from tests.gpu_helpers import DeviceCase, assert_parity, host_pools_after_append, say

pytestmark = pytest.mark.gpu


def _zero_offsets_host(table):
    return (np.asarray(table, dtype=np.uint32) & np.uint32(0xFFFF)).astype(np.uint32)


def _zero_offsets_dev(table):
    return (table & 0xFFFF).contiguous()


EAGER_DECODE = [
    # D, Hq, Hkv, ctx, doc blocks, split
    (128, 32, 8, [512, 1024, 96], (2, 10), 0),
    (128, 16, 2, [2048, 64], (4, 16), 4),
    (64, 8, 8, [320, 16, 784], (1, 6), 0),
]


@pytest.mark.parametrize("d,hq,hkv,ctx,docs,split", EAGER_DECODE)
def test_eager_decode_matches_oracle_without_offsets(d, hq, hkv, ctx, docs, split):
    case = W.decode_case(91 + d + hq, len(ctx), hq, hkv, d, ctx, docs, offsets="random")
    say(f"[eager decode] D{d} Hq{hq} Hkv{hkv} ctx={ctx} split={split}")
    W.materialize_numpy(case)
    dc = DeviceCase(case)
    dc.append()
    out = pak.lazyattn_decode_eager(dc.q, dc.q_pos, dc.k_pool, dc.v_pool, dc.table, dc.seq_lens,
                                    scale=case.scale, rope_theta=case.rope_theta, split_blocks=split)
    torch.cuda.synchronize()
    kp, vp = host_pools_after_append(case)
    want = oracle.decode(W.to_float(case.q, case.dtype), case.q_pos, kp, vp,
                         _zero_offsets_host(case.layout.table), case.seq_lens, case.scale,
                         case.rope_theta)
    assert_parity(W.to_float(out, case.dtype), want, case.dtype, f"eager decode D{d} G{hq // hkv}")
    # the lazy kernel on the same table with its offsets cleared computes the same thing
    lazy = pak.lazyattn_decode(dc.q, dc.q_pos, dc.k_pool, dc.v_pool, _zero_offsets_dev(dc.table),
                               dc.seq_lens, scale=case.scale, rope_theta=case.rope_theta,
                               split_blocks=split)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), lazy.view(torch.int16))


EAGER_PREFILL = [
    # D, Hq, Hkv, cached, prompt, doc blocks
    (128, 32, 8, [512, 96], [256, 77], (2, 12)),
    (128, 8, 1, [1056], [130], (3, 40)),
    (64, 8, 4, [320, 48], [150, 31], (2, 10)),
]


@pytest.mark.parametrize("d,hq,hkv,cached,prompt,docs", EAGER_PREFILL)
def test_eager_prefill_matches_oracle_without_offsets(d, hq, hkv, cached, prompt, docs):
    case = W.prefill_case(93 + d + hq, len(prompt), hq, hkv, d, cached, prompt, docs, offsets="random")
    say(f"[eager prefill] D{d} Hq{hq} Hkv{hkv} cached={cached} prompt={prompt}")
    W.materialize_numpy(case)
    dc = DeviceCase(case)
    dc.append()
    out = pak.lazyattn_prefill_eager(dc.q, dc.cu, dc.q_pos_start, dc.k_pool, dc.v_pool, dc.table,
                                     dc.seq_lens, case.max_q_len, scale=case.scale,
                                     rope_theta=case.rope_theta)
    torch.cuda.synchronize()
    kp, vp = host_pools_after_append(case)
    want = oracle.prefill(W.to_float(case.q, case.dtype), case.cu_q_lens, case.layout.tail_pos, kp, vp,
                          _zero_offsets_host(case.layout.table), case.seq_lens, case.scale,
                          case.rope_theta)
    assert_parity(W.to_float(out, case.dtype), want, case.dtype, f"eager prefill D{d} G{hq // hkv}")
    lazy = pak.lazyattn_prefill(dc.q, dc.cu, dc.q_pos_start, dc.k_pool, dc.v_pool,
                                _zero_offsets_dev(dc.table), dc.seq_lens, case.max_q_len,
                                scale=case.scale, rope_theta=case.rope_theta)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), lazy.view(torch.int16))

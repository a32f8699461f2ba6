"""GPU: launches on a stream other than torch's current one.

The binding allocates its temporaries (output, split-K workspace, fill
counts padded to a multiple of 4) on the current stream.  Here every call
goes to a side stream with none of them supplied by the caller, and with a
fill-count array whose length is not a multiple of 4, so each temporary is
made by the binding.  The results must match the oracle and the same calls
on the current stream, bit for bit.  Between the calls the current stream
runs unrelated work that allocates and frees memory, which would reuse a
temporary still read by the side stream if the binding did not hold it.
"""

import pytest
import torch

import oracle
import position_agnostic_kv_amd as pak
import workloads as W
from tests.gpu_helpers import DEV, DeviceCase, assert_parity, host_pools_after_append, say

pytestmark = pytest.mark.gpu


def _churn():
    """Allocate, fill and free on the current stream (reuses freed blocks)."""
    for _ in range(4):
        x = torch.empty(1 << 20, dtype=torch.float32, device=DEV)
        x.fill_(float("nan"))
        del x


def _ragged(kind, seed):
    case = W.ragged_case(seed, kind, 3, 16, 2, 128, (2, 5), (1, 400), prompt=(40, 200))
    W.materialize_numpy(case)
    return case


def _odd_fill(dc):
    """Fill counts whose length is not a multiple of 4: the case's own, or,
    if its pool size is a multiple of 4, with one spare block appended to
    the pools and the counts (the table never refers to it)."""
    n = dc.fill.numel()
    if n % 4 != 0:
        return dc.fill
    dc.k_pool = torch.cat([dc.k_pool, dc.k_pool[:1]]).contiguous()
    dc.v_pool = torch.cat([dc.v_pool, dc.v_pool[:1]]).contiguous()
    return torch.cat([dc.fill, dc.fill.new_full((1,), 16)])


def test_side_stream_decode_allocates_safely():
    case = _ragged("decode", 401)
    say(f"[side stream decode] blocks={case.layout.num_blocks} slots={case.seq_lens.tolist()}")
    dc = DeviceCase(case)
    dc.append()
    fill = _odd_fill(dc)
    assert fill.numel() % 4 != 0
    kw = dict(scale=case.scale, rope_theta=case.rope_theta, split_blocks=4, block_fill=fill)
    ref = pak.lazyattn_decode(dc.q, dc.q_pos, dc.k_pool, dc.v_pool, dc.table, dc.seq_lens, **kw)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=DEV)
    outs = []
    for _ in range(3):
        outs.append(pak.lazyattn_decode(dc.q, dc.q_pos, dc.k_pool, dc.v_pool, dc.table, dc.seq_lens,
                                        stream=side, **kw))
        _churn()
    torch.cuda.synchronize()
    kp, vp = host_pools_after_append(case)
    want = oracle.decode(W.to_float(case.q, case.dtype), case.q_pos, kp, vp, case.layout.table,
                         case.seq_lens, case.scale, case.rope_theta, block_fill=case.block_fill)
    for i, out in enumerate(outs):
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"side-stream call {i} differs"
    assert_parity(W.to_float(outs[-1], case.dtype), want, case.dtype, "side-stream decode")


def test_side_stream_prefill_allocates_safely():
    case = _ragged("prefill", 402)
    say(f"[side stream prefill] blocks={case.layout.num_blocks} prompts={case.layout.tail_lens.tolist()}")
    dc = DeviceCase(case)
    dc.append()
    fill = _odd_fill(dc)
    assert fill.numel() % 4 != 0
    kw = dict(scale=case.scale, rope_theta=case.rope_theta, block_fill=fill)
    args = (dc.q, dc.cu, dc.q_pos_start, dc.k_pool, dc.v_pool, dc.table, dc.seq_lens, case.max_q_len)
    ref = pak.lazyattn_prefill(*args, **kw)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=DEV)
    outs = []
    for _ in range(3):
        outs.append(pak.lazyattn_prefill(*args, stream=side, **kw))
        _churn()
    torch.cuda.synchronize()
    kp, vp = host_pools_after_append(case)
    want = oracle.prefill(W.to_float(case.q, case.dtype), case.cu_q_lens, case.layout.tail_pos, kp, vp,
                          case.layout.table, case.seq_lens, case.scale, case.rope_theta,
                          block_fill=case.block_fill)
    for i, out in enumerate(outs):
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"side-stream call {i} differs"
    assert_parity(W.to_float(outs[-1], case.dtype), want, case.dtype, "side-stream prefill")


def test_side_stream_planned_decode_allocates_safely():
    case = _ragged("decode", 404)
    say(f"[side stream planned decode] blocks={case.layout.num_blocks} slots={case.seq_lens.tolist()}")
    dc = DeviceCase(case)
    dc.append()
    fill = _odd_fill(dc)
    assert fill.numel() % 4 != 0
    plan = pak.decode_plan(dc.table, dc.seq_lens, case.num_q_heads, case.num_kv_heads, max_item_blocks=5)
    kw = dict(scale=case.scale, rope_theta=case.rope_theta, block_fill=fill)
    args = (dc.q, dc.q_pos, dc.k_pool, dc.v_pool, dc.table, dc.seq_lens, plan)
    ref = pak.lazyattn_decode_planned(*args, **kw)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=DEV)
    outs = []
    for _ in range(3):
        outs.append(pak.lazyattn_decode_planned(*args, stream=side, **kw))
        _churn()
    torch.cuda.synchronize()
    kp, vp = host_pools_after_append(case)
    want = oracle.decode(W.to_float(case.q, case.dtype), case.q_pos, kp, vp, case.layout.table,
                         case.seq_lens, case.scale, case.rope_theta, block_fill=case.block_fill)
    for i, out in enumerate(outs):
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"side-stream call {i} differs"
    assert_parity(W.to_float(outs[-1], case.dtype), want, case.dtype, "side-stream planned decode")

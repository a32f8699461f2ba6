"""The C-ABI calls are stream-ordered and allocate nothing, so a whole step
(append + decode with split-K partials, append + prefill, the 8-bit pool's
append + decode, the planned decode with a plan built beforehand, the
precise prefill, and the 8-bit prefill's widening pass and prefill) can be
captured in a HIP graph and replayed.  Every
replay, with eager work on the same stream between replays, must give the
eager results bit for bit (the kernels are deterministic).  Outputs and the
decode workspace are allocated before capture; nothing inside the graph
clears memory with a memset."""

import numpy as np
import pytest
import torch

import position_agnostic_kv_amd as pak
import workloads as W
from tests.gpu_helpers import DEV, DeviceCase, say

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16).clone()


def test_graph_replays_equal_eager():
    dcase = W.decode_case(401, 3, 32, 8, 128, [1024, 512, 208], (2, 12), offsets="random")
    pcase = W.prefill_case(403, 2, 32, 8, 128, [512, 96], [256, 77], (2, 12))
    for c in (dcase, pcase):
        W.materialize_numpy(c)
    dd, pd = DeviceCase(dcase), DeviceCase(pcase)
    split = 4   # several splits: the combine kernel reads the workspace partials
    need = pak.decode_workspace_size(dcase.batch, dcase.num_q_heads, dcase.num_kv_heads, dcase.head_dim,
                                     dcase.layout.table.shape[1], split)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=DEV)
    dout, pout = torch.empty_like(dd.q), torch.empty_like(pd.q)
    shape = tuple(dd.k_pool.shape)
    k8 = W.e4m3_codes_torch(shape, DEV, 11)
    v8 = W.e4m3_codes_torch(shape, DEV, 12)
    out8 = torch.empty_like(dd.q)
    plan = pak.decode_plan(dd.table, dd.seq_lens, dcase.num_q_heads, dcase.num_kv_heads, max_item_blocks=8)
    pws = torch.empty(max(pak.decode_planned_workspace_size(dcase.batch, dcase.num_q_heads, dcase.num_kv_heads,
                                                            dcase.head_dim, plan.max_items_per_seq), 1),
                      dtype=torch.uint8, device=DEV)
    pl_out = torch.empty_like(dd.q)
    pre_out = torch.empty_like(pd.q)
    pshape = tuple(pd.k_pool.shape)
    pk8, pv8 = W.e4m3_codes_torch(pshape, DEV, 13), W.e4m3_codes_torch(pshape, DEV, 14)
    pws8 = torch.empty(max(pak.prefill_fp8_workspace_size(pcase.batch, pd.table.shape[1], pcase.num_kv_heads), 1),
                       dtype=torch.uint8, device=DEV)
    pout8 = torch.empty_like(pd.q)

    def step():
        pak.kvcache_append(dd.k_pool, dd.v_pool, dd.k_new, dd.v_new, dd.slots)
        pak.lazyattn_decode(dd.q, dd.q_pos, dd.k_pool, dd.v_pool, dd.table, dd.seq_lens, scale=dcase.scale,
                            rope_theta=dcase.rope_theta, split_blocks=split, out=dout, workspace=ws)
        pak.kvcache_append(pd.k_pool, pd.v_pool, pd.k_new, pd.v_new, pd.slots)
        pak.lazyattn_prefill(pd.q, pd.cu, pd.q_pos_start, pd.k_pool, pd.v_pool, pd.table, pd.seq_lens,
                             pcase.max_q_len, scale=pcase.scale, rope_theta=pcase.rope_theta, out=pout)
        pak.kvcache_append_fp8(k8, v8, dd.k_new, dd.v_new, dd.slots, 0.25, 0.125)
        pak.lazyattn_decode_fp8(dd.q, dd.q_pos, k8, v8, dd.table, dd.seq_lens, 0.25, 0.125, scale=dcase.scale,
                                rope_theta=dcase.rope_theta, split_blocks=split, out=out8, workspace=ws)
        pak.lazyattn_decode_planned(dd.q, dd.q_pos, dd.k_pool, dd.v_pool, dd.table, dd.seq_lens, plan,
                                    scale=dcase.scale, rope_theta=dcase.rope_theta, out=pl_out, workspace=pws)
        pak.lazyattn_prefill_precise(pd.q, pd.cu, pd.q_pos_start, pd.k_pool, pd.v_pool, pd.table, pd.seq_lens,
                                     pcase.max_q_len, scale=pcase.scale, rope_theta=pcase.rope_theta, out=pre_out)
        pak.kvcache_append_fp8(pk8, pv8, pd.k_new, pd.v_new, pd.slots, 0.25, 0.125)
        pak.lazyattn_prefill_fp8(pd.q, pd.cu, pd.q_pos_start, pk8, pv8, pd.table, pd.seq_lens, pcase.max_q_len,
                                 0.25, 0.125, scale=pcase.scale, rope_theta=pcase.rope_theta, out=pout8,
                                 workspace=pws8)

    outs = (dout, pout, out8, pl_out, pre_out, pout8)
    step()
    torch.cuda.synchronize()
    want = [_bits(t) for t in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        for t in outs:
            t.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        got = [_bits(t) for t in outs]
        say(f"[graph] replay {r}")
        for name, g, w in zip(("decode", "prefill", "decode fp8", "planned decode", "precise prefill",
                               "prefill fp8 (widening pass + prefill)"), got, want):
            assert torch.equal(g, w), f"replay {r}: {name} differs from the eager step"
        # eager work between replays, on the same buffers
        step()
        torch.cuda.synchronize()
        assert all(torch.equal(_bits(t), w) for t, w in zip(outs, want))
    assert np.isfinite(W.to_float(dout, W.BF16)).all()

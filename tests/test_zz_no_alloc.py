"""GPU: lazyattn_decode_noalloc (split-K partials in the library's fixed
per-GPU scratch) against lazyattn_decode with a caller workspace.

Two calls in a row, the second on a smaller input, each must equal the
workspace call bit for bit (same kernels, same split choice) and the oracle
within the bf16 tolerance; a size whose partials exceed the scratch is
rejected before any launch."""

import pytest
import torch

import position_agnostic_kv_amd as pak
import workloads as W
from tests.gpu_helpers import DEV, DeviceCase, assert_parity, oracle_decode, say

pytestmark = pytest.mark.gpu


def _check(case, split):
    W.materialize_numpy(case)
    dc = DeviceCase(case)
    dc.append()
    need = pak.decode_workspace_size(case.batch, case.num_q_heads, case.num_kv_heads, case.head_dim,
                                     case.layout.table.shape[1], split)
    say(f"[noalloc] {case.name} B={case.batch} Hq={case.num_q_heads} Hkv={case.num_kv_heads} split={split} "
        f"partials={need} B")
    assert 0 < need <= 8 << 20
    kw = dict(scale=case.scale, rope_theta=case.rope_theta, split_blocks=split)
    ref = pak.lazyattn_decode(dc.q, dc.q_pos, dc.k_pool, dc.v_pool, dc.table, dc.seq_lens, **kw)
    out = torch.empty_like(dc.q)
    got = pak.lazyattn_decode_noalloc(dc.q, dc.q_pos, dc.k_pool, dc.v_pool, dc.table, dc.seq_lens, out=out, **kw)
    torch.cuda.synchronize()
    assert got is out
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), "differs from the workspace call"
    assert_parity(W.to_float(out, case.dtype), oracle_decode(case), case.dtype, f"noalloc {case.name}")


def test_noalloc_decode_two_calls_second_smaller():
    big = W.decode_case(501, 6, 32, 8, 128, [4096, 2048, 1024, 512, 3008, 16], (2, 24), offsets="random",
                        name="noalloc_big")
    small = W.decode_case(502, 2, 16, 2, 128, [400, 96], (2, 8), name="noalloc_small")
    _check(big, 4)
    _check(small, 4)


def test_noalloc_decode_multi_query_automatic_splits():
    """A 64-head group (the 8-wave multi-query kernel) and a 32-head group,
    splits chosen by the library, partials in the fixed scratch."""
    wide = W.decode_case(503, 2, 64, 1, 128, [3008, 1200], (2, 16), offsets="random", name="noalloc_g64")
    mid = W.decode_case(504, 3, 32, 1, 128, [896, 2048, 64], (2, 10), name="noalloc_g32")
    _check(wide, 0)
    _check(mid, 0)


def test_noalloc_decode_rejects_partials_beyond_the_scratch():
    b, hq, hkv, d, max_blocks = 256, 64, 8, 128, 2048
    need = pak.decode_workspace_size(b, hq, hkv, d, max_blocks, 4)
    assert need > 8 << 20
    q = torch.zeros((b, hq, d), dtype=torch.bfloat16, device=DEV)
    pool = torch.zeros((1, hkv, 16, d), dtype=torch.bfloat16, device=DEV)
    table = torch.zeros((b, max_blocks), dtype=torch.int32, device=DEV)
    ints = torch.zeros(b, dtype=torch.int32, device=DEV)
    with pytest.raises(pak.LazyAttnError, match="status -6"):
        pak.lazyattn_decode_noalloc(q, ints, pool, pool, table, ints, out=torch.empty_like(q), split_blocks=4)
    torch.cuda.synchronize()

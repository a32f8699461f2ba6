"""End to end on the GPU: block tables from the host pool manager drive
kvcache_append and lazyattn_decode, checked against the oracle.

Round 1 places every request's documents for the first time (all misses): the
test writes each missed document's content-only K/V into the blocks the
manager handed out.  Round 2 asks for the same documents in other orders:
they hit, nothing is written, and the same physical blocks are read at new
positions (zero-copy reuse, LazyAttention summary "Metodologia").  Both rounds
must match the oracle on the manager's tables.
"""

import numpy as np
import pytest
import torch

import oracle
import position_agnostic_kv_amd as pak
import workloads as W
from position_agnostic_kv_amd.cache import CacheManager
from tests.gpu_helpers import DEV, assert_parity, say

pytestmark = pytest.mark.gpu

HQ, HKV, D, THETA = 8, 2, 128, 5.0e5


def _round(mgr, requests, docs, k_pool, v_pool, kh, vh, rng, label):
    """Acquire every request, append missed documents (device and host
    mirrors), decode one new query per request, compare with the oracle."""
    rows, rids, lens = [], [], []
    for ids in requests:
        row, miss, rid = mgr.acquire(ids, [docs[i][0].shape[0] for i in ids], 16)
        rows.append(row)
        rids.append(rid)
        lens.append(int(sum(docs[i][0].shape[0] for i in ids)) + 16)
        p = 0
        for i, m in zip(ids, miss):
            n = docs[i][0].shape[0]
            if m:
                blocks = (row[p // 16: (p + n) // 16] & 0xFFFF).astype(np.int64)
                slots = (blocks[:, None] * 16 + np.arange(16)[None, :]).reshape(-1).astype(np.int32)
                kd, vd = docs[i]
                pak.kvcache_append(k_pool, v_pool, torch.from_numpy(W.f32_to_bf16_bits(kd)).view(torch.bfloat16).to(DEV),
                                   torch.from_numpy(W.f32_to_bf16_bits(vd)).view(torch.bfloat16).to(DEV),
                                   torch.from_numpy(slots).to(DEV))
                kh[slots // 16, :, slots % 16, :] = W.bf16_bits_to_f32(W.f32_to_bf16_bits(kd))
                vh[slots // 16, :, slots % 16, :] = W.bf16_bits_to_f32(W.f32_to_bf16_bits(vd))
            p += n
        # the prompt's one block: a new token's K/V at the last slot range
        pb = int(row[-1] & 0xFFFF)
        kn = rng.standard_normal((16, HKV, D)).astype(np.float32) * 0.5
        vn = rng.standard_normal((16, HKV, D)).astype(np.float32) * 0.5
        slots = np.arange(pb * 16, pb * 16 + 16, dtype=np.int32)
        pak.kvcache_append(k_pool, v_pool, torch.from_numpy(W.f32_to_bf16_bits(kn)).view(torch.bfloat16).to(DEV),
                           torch.from_numpy(W.f32_to_bf16_bits(vn)).view(torch.bfloat16).to(DEV),
                           torch.from_numpy(slots).to(DEV))
        kh[pb] = W.bf16_bits_to_f32(W.f32_to_bf16_bits(kn)).transpose(1, 0, 2)
        vh[pb] = W.bf16_bits_to_f32(W.f32_to_bf16_bits(vn)).transpose(1, 0, 2)
    mb = max(len(r) for r in rows)
    table = np.zeros((len(rows), mb), dtype=np.uint32)
    for b, r in enumerate(rows):
        table[b, :len(r)] = r
    seq_lens = np.array(lens, dtype=np.int32)
    q_pos = seq_lens - 1
    qf = W.bf16_bits_to_f32(W.f32_to_bf16_bits(rng.standard_normal((len(rows), HQ, D)).astype(np.float32)))
    q = torch.from_numpy(W.f32_to_bf16_bits(qf)).view(torch.bfloat16).to(DEV)
    out = pak.lazyattn_decode(q, torch.from_numpy(q_pos).to(DEV), k_pool, v_pool,
                              torch.from_numpy(table.view(np.int32)).to(DEV), torch.from_numpy(seq_lens).to(DEV),
                              rope_theta=THETA, split_blocks=8)
    torch.cuda.synchronize()
    want = oracle.decode(qf, q_pos, kh, vh, table, seq_lens, 1.0 / np.sqrt(D), THETA)
    assert_parity(W.to_float(out, W.BF16), want, W.BF16, label)
    for rid in rids:
        mgr.release(rid)


def test_manager_tables_drive_append_and_decode():
    rng = np.random.default_rng(44)
    ndocs, nblocks = 10, 512
    docs = {}
    for i in range(ndocs):
        n = 16 * int(rng.integers(2, 12))
        docs[i] = (rng.standard_normal((n, HKV, D)).astype(np.float32) * 0.5,
                   rng.standard_normal((n, HKV, D)).astype(np.float32) * 0.5)
    k_pool = torch.zeros((nblocks, HKV, 16, D), dtype=torch.bfloat16, device=DEV)
    v_pool = torch.zeros_like(k_pool)
    kh = np.zeros((nblocks, HKV, 16, D), dtype=np.float32)
    vh = np.zeros_like(kh)
    mgr = CacheManager(nblocks, "agnostic")
    say("[cache] round 1: first placements")
    _round(mgr, [[0, 1, 2], [3, 4], [5, 6, 7, 8, 9]], docs, k_pool, v_pool, kh, vh, rng, "cache round 1")
    before = mgr.stats()
    say("[cache] round 2: the same documents in other orders")
    _round(mgr, [[2, 0, 1], [9, 4, 3, 7], [8, 6, 5]], docs, k_pool, v_pool, kh, vh, rng, "cache round 2")
    after = mgr.stats()
    assert after["doc_misses"] == before["doc_misses"], "round 2 must reuse every document"
    assert after["doc_hits"] - before["doc_hits"] == 10

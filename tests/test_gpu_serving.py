"""The whole path in a serving loop on the GPU, against the oracle.

The host pool manager places three requests whose documents overlap (one
document sits in two requests at different positions, stored once:
LazyAttention summary, "Metodologia").  The test then, through the C ABI:

1. appends every missed document's content-only K/V into the blocks the
   manager handed out (kvcache_append), and each prompt's K/V after them;
2. prefills the three prompts in one call (lazyattn_prefill);
3. runs three decode steps, each appending one new token per request into the
   room the manager reserved, then attending (lazyattn_decode);
4. prefills each prompt extended by the three generated tokens, whose rows
   for those tokens must reproduce the three decode outputs: incremental
   decoding equals the full recompute (the pages' decode appends the new row
   and attends 1 x (t + 1), KV Cache page, "Construa").

Every output is compared with the float64 oracle on host mirrors of the pool.
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

HQ, HKV, D, THETA = 16, 4, 128, 5.0e5
SCALE = 1.0 / np.sqrt(D)
STEPS = 3


def _bf16(x):
    """(device bf16 tensor, host float32 copy of the same rounded values)."""
    bits = W.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))
    return torch.from_numpy(bits).view(torch.bfloat16).to(DEV), W.bf16_bits_to_f32(bits)


def _i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(DEV)


def test_serving_loop_prefill_then_decode_steps():
    rng = np.random.default_rng(81)
    nblocks = 256
    doc_len = {i: 16 * int(rng.integers(2, 10)) for i in range(6)}
    docs = {i: (rng.standard_normal((n, HKV, D)) * 0.5, rng.standard_normal((n, HKV, D)) * 0.5)
            for i, n in doc_len.items()}
    requests = [[0, 1, 2], [3, 1], [2, 4, 5]]     # documents 1 and 2 at two positions each
    prompts = [70, 33, 150]
    k_pool = torch.zeros((nblocks, HKV, 16, D), dtype=torch.bfloat16, device=DEV)
    v_pool = torch.zeros_like(k_pool)
    kh = np.zeros((nblocks, HKV, 16, D), dtype=np.float32)
    vh = np.zeros_like(kh)

    def append(kx, vx, slots):
        kd, kf = _bf16(kx)
        vd, vf = _bf16(vx)
        pak.kvcache_append(k_pool, v_pool, kd, vd, _i32(slots))
        kh[slots // 16, :, slots % 16, :] = kf
        vh[slots // 16, :, slots % 16, :] = vf

    mgr = CacheManager(nblocks, "agnostic")
    rows, cached = [], []
    for ids, plen in zip(requests, prompts):
        row, miss, _ = mgr.acquire(ids, [doc_len[i] for i in ids], plen + STEPS)
        p = 0
        for i, m in zip(ids, miss):
            if m:
                blocks = (row[p // 16:(p + doc_len[i]) // 16] & 0xFFFF).astype(np.int64)
                append(*docs[i], (blocks[:, None] * 16 + np.arange(16)[None, :]).reshape(-1))
            p += doc_len[i]
        rows.append(np.asarray(row, dtype=np.uint32))
        cached.append(p)
    assert mgr.stats()["doc_hits"] == 2, "documents 1 and 2 are reused, not copied"

    def prompt_slots(b, r):
        """Table slots of prompt tokens r (array) of request b."""
        nd = cached[b] // 16
        return (rows[b][nd + r // 16] & 0xFFFF).astype(np.int64) * 16 + r % 16

    mb = max(len(r) for r in rows)
    table = np.zeros((len(rows), mb), dtype=np.uint32)
    for b, r in enumerate(rows):
        table[b, :len(r)] = r
    tab = torch.from_numpy(table.view(np.int32)).to(DEV)
    q_rows = []
    for b, plen in enumerate(prompts):
        r = np.arange(plen)
        append(rng.standard_normal((plen, HKV, D)) * 0.5, rng.standard_normal((plen, HKV, D)) * 0.5,
               prompt_slots(b, r))
        q_rows.append(rng.standard_normal((plen, HQ, D)))

    # ---- prefill of the three prompts
    say("[serving] prefill")
    cu = np.concatenate([[0], np.cumsum(prompts)])
    kv_lens = np.array([c + p for c, p in zip(cached, prompts)])
    qd, qf = _bf16(np.concatenate(q_rows))
    out = pak.lazyattn_prefill(qd, _i32(cu), _i32(cached), k_pool, v_pool, tab, _i32(kv_lens), max(prompts),
                               scale=SCALE, rope_theta=THETA)
    torch.cuda.synchronize()
    want = oracle.prefill(qf, cu, np.array(cached), kh, vh, table, kv_lens, SCALE, THETA)
    assert_parity(W.to_float(out, W.BF16), want, W.BF16, "serving prefill")

    # ---- decode steps: append the new token, attend
    dec_out, dec_q = [], []
    for t in range(STEPS):
        say(f"[serving] decode step {t}")
        for b, plen in enumerate(prompts):
            append(rng.standard_normal((1, HKV, D)) * 0.5, rng.standard_normal((1, HKV, D)) * 0.5,
                   prompt_slots(b, np.array([plen + t])))
        seq_lens = kv_lens + t + 1
        q_pos = np.array(cached) + np.array(prompts) + t
        qd, qf = _bf16(rng.standard_normal((len(rows), HQ, D)))
        out = pak.lazyattn_decode(qd, _i32(q_pos), k_pool, v_pool, tab, _i32(seq_lens), scale=SCALE,
                                  rope_theta=THETA)
        torch.cuda.synchronize()
        got = W.to_float(out, W.BF16)
        want = oracle.decode(qf, q_pos, kh, vh, table, seq_lens, SCALE, THETA)
        assert_parity(got, want, W.BF16, f"serving decode step {t}")
        dec_out.append(got)
        dec_q.append(qf)

    # ---- full recompute: each prompt extended by the generated tokens
    say("[serving] prefill of the extended prompts")
    ext = [p + STEPS for p in prompts]
    cu2 = np.concatenate([[0], np.cumsum(ext)])
    qx = np.concatenate([np.concatenate([q_rows[b]] + [dec_q[t][b:b + 1] for t in range(STEPS)])
                         for b in range(len(rows))])
    qd, qf = _bf16(qx)
    out = pak.lazyattn_prefill(qd, _i32(cu2), _i32(cached), k_pool, v_pool, tab, _i32(kv_lens + STEPS),
                               max(ext), scale=SCALE, rope_theta=THETA)
    torch.cuda.synchronize()
    full = W.to_float(out, W.BF16)
    want = oracle.prefill(qf, cu2, np.array(cached), kh, vh, table, kv_lens + STEPS, SCALE, THETA)
    assert_parity(full, want, W.BF16, "serving extended prefill")
    last = np.stack([np.stack([full[cu2[b] + prompts[b] + t] for b in range(len(rows))]) for t in range(STEPS)])
    assert_parity(np.stack(dec_out), last.astype(np.float64), W.BF16, "decode steps vs the full recompute's rows")

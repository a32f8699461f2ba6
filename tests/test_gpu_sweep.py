"""GPU parity over a seeded random sweep of shapes, and chunked prefill.

The fixed grids elsewhere pick their cases by hand.  Here each seed draws a
whole configuration from the space the C ABI accepts:

* decode: bf16 or fp32; head_dim 64 or 128 (fp32 also 16); 1, 2, 4 or 8 KV
  heads; group sizes 1..64; 1..4 sequences; documents of whole blocks or of any
  token count (per-block fill counts); contiguous or random offsets; automatic
  or explicit split-K partitions;
* prefill: head_dim 64 or 128; group sizes 1..64; 1..3 sequences; whole-block
  or any-length documents; prompts of 1..300 rows; lazyattn_prefill or
  lazyattn_prefill_precise.

Every case is compared element by element with the float64 oracle at the
stated tolerances (the method claims to reach the eager result exactly:
LazyAttention summary, "Equivalência Matemática").

Chunked prefill: a prompt run in two calls -- the first chunk, then the rest
with the first chunk's K/V already in the table as stored tokens -- gives the
one-shot prefill's rows (the pages' prefill attends query tiles to whatever
the table holds before them: "Implementação Técnica", Prefilling).
"""

import numpy as np
import pytest
import torch

import position_agnostic_kv_amd as pak
import workloads as W
from tests.gpu_helpers import DEV, DeviceCase, assert_parity, oracle_decode, oracle_prefill, say

pytestmark = pytest.mark.gpu

SEEDS = list(range(24))


def _decode_case(seed):
    rng = np.random.default_rng(9100 + seed)
    dtype = W.F32 if rng.random() < 0.3 else W.BF16
    d = int(rng.choice([16, 64, 128] if dtype == W.F32 else [64, 128]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8, 16, 32, 64]))
    while hkv * g > 64:
        hkv //= 2
    batch = int(rng.integers(1, 5))
    offsets = "random" if rng.random() < 0.5 else "contiguous"
    split = int(rng.choice([0, 0, 4, 7, 32]))
    if rng.random() < 0.4:
        case = W.ragged_case(9100 + seed, "decode", batch, hkv * g, hkv, d, (1, 5), (1, 400),
                             dtype=dtype, offsets=offsets)
        kind = "any-length documents"
    else:
        ctx = [16 * int(x) for x in rng.integers(1, 80, size=batch)]
        case = W.decode_case(9100 + seed, batch, hkv * g, hkv, d, ctx, (1, 12), dtype=dtype, offsets=offsets)
        kind = "whole-block documents"
    return case, split, f"seed {seed}: {dtype} D{d} Hkv{hkv} G{g} B{batch} {offsets} {kind} split {split}"


@pytest.mark.parametrize("seed", SEEDS)
def test_decode_random_sweep(seed):
    case, split, label = _decode_case(seed)
    say(f"[sweep decode] {label}")
    W.materialize_numpy(case)
    dc = DeviceCase(case)
    dc.append()
    out = dc.decode(split_blocks=split)
    torch.cuda.synchronize()
    assert_parity(W.to_float(out, case.dtype), oracle_decode(case), case.dtype, label)


def _prefill_case(seed):
    rng = np.random.default_rng(9300 + seed)
    d = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8, 16, 32, 64]))
    while hkv * g > 64:
        hkv //= 2
    batch = int(rng.integers(1, 4))
    offsets = "random" if rng.random() < 0.5 else "contiguous"
    precise = bool(rng.random() < 0.3)
    if rng.random() < 0.4:
        case = W.ragged_case(9300 + seed, "prefill", batch, hkv * g, hkv, d, (1, 4), (1, 300),
                             prompt=(1, 300), offsets=offsets)
        kind = "any-length documents"
    else:
        cached = [16 * int(x) for x in rng.integers(0, 40, size=batch)]
        prompt = [int(x) for x in rng.integers(1, 301, size=batch)]
        case = W.prefill_case(9300 + seed, batch, hkv * g, hkv, d, cached, prompt, (1, 10), offsets=offsets)
        kind = "whole-block documents"
    return case, precise, (f"seed {seed}: D{d} Hkv{hkv} G{g} B{batch} {offsets} {kind}"
                           f"{' precise' if precise else ''}")


@pytest.mark.parametrize("seed", SEEDS)
def test_prefill_random_sweep(seed):
    case, precise, label = _prefill_case(seed)
    say(f"[sweep prefill] {label}")
    W.materialize_numpy(case)
    dc = DeviceCase(case)
    dc.append()
    out = dc.prefill(precise=precise)
    torch.cuda.synchronize()
    assert_parity(W.to_float(out, case.dtype), oracle_prefill(case), case.dtype, label)


@pytest.mark.parametrize("seed,hq,hkv,d,cached,prompt,cut,offs", [
    (9501, 32, 8, 128, [512, 256], [300, 170], [165, 1], "random"),
    (9502, 8, 2, 64, [0, 384], [257, 129], [128, 64], "contiguous"),
    (9503, 16, 1, 128, [96], [200], [33], "random"),
])
def test_chunked_prefill_matches_one_shot(seed, hq, hkv, d, cached, prompt, cut, offs):
    """Prefill of rows [0, cut) then [cut, P) of each prompt, the second call
    seeing the first chunk as stored tokens, equals the one-shot prefill."""
    case = W.prefill_case(seed, len(prompt), hq, hkv, d, cached, prompt, (2, 10), offsets=offs)
    say(f"[chunked prefill] seed {seed} Hq{hq} Hkv{hkv} D{d} prompt {prompt} cut {cut} {offs}")
    W.materialize_numpy(case)
    dc = DeviceCase(case)
    dc.append()
    whole = dc.prefill()
    cu = [int(x) for x in case.cu_q_lens]
    kv = [int(x) for x in case.seq_lens]
    start = [int(x) for x in case.layout.tail_pos]
    parts = []
    for first in (True, False):
        rows, lens, cus, pos = [], [], [0], []
        for b, c in enumerate(cut):
            p = prompt[b]
            lo, hi = (0, c) if first else (c, p)
            rows.extend(range(cu[b] + lo, cu[b] + hi))
            lens.append(kv[b] - (p - hi))
            cus.append(cus[-1] + hi - lo)
            pos.append(start[b] + lo)
        idx = torch.tensor(rows, dtype=torch.long, device=DEV)
        q = dc.q.index_select(0, idx).contiguous()
        t = lambda x: torch.tensor(x, dtype=torch.int32, device=DEV)
        out = pak.lazyattn_prefill(q, t(cus), t(pos), dc.k_pool, dc.v_pool, dc.table, t(lens),
                                   max(cus[i + 1] - cus[i] for i in range(len(cut))),
                                   scale=case.scale, rope_theta=case.rope_theta, block_fill=dc.fill)
        parts.append((idx, out))
    torch.cuda.synchronize()
    chunked = torch.empty_like(whole)
    for idx, out in parts:
        chunked.index_copy_(0, idx, out)
    want = oracle_prefill(case)
    assert_parity(W.to_float(chunked, case.dtype), want, case.dtype, "chunked prefill vs oracle")
    assert_parity(W.to_float(chunked, case.dtype), W.to_float(whole, case.dtype).astype(np.float64),
                  case.dtype, "chunked prefill vs one-shot prefill")

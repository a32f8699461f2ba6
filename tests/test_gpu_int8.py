"""GPU parity of the int8 KV pool (kvcache_append_int8, lazyattn_decode_int8,
lazyattn_prefill_int8) against the int8 oracle.  Pools hold random int8
codes; the step's new rows are bf16 or f32 values that the append quantises
bit for bit as the oracle does (ties to even, the clamp to +-127, infinities,
NaN to 0).  The device pools hold the codes in the 8-bit pools' lane order;
the tests move host codes into it and back with the documented permutation.
Decode covers GQA 4 and 8, a 32-query-head group, split-K, random offsets
and documents of any length; prefill covers GQA 1 to 8, random offsets,
documents of any length, and bit-equality with the bf16 prefill on the
dequantised pool."""

import numpy as np
import pytest
import torch

import oracle
import position_agnostic_kv_amd as pak
import workloads as W
from tests.gpu_helpers import DEV, DeviceCase, assert_parity, say

pytestmark = pytest.mark.gpu


def _dev8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _host8(t):
    return t.cpu().numpy().view(np.int8)


@pytest.mark.parametrize("rows_dtype", [W.BF16, W.F32])
@pytest.mark.parametrize("ks,vs", [(1.0, 1.0), (0.05, 0.37), (0.5, 1.0e-3)])
def test_append_int8_bit_exact(rows_dtype, ks, vs):
    rng = np.random.default_rng(31)
    nb, hkv, d, t = 8, 4, 128, 70
    x = rng.standard_normal((2, t, hkv, d)).astype(np.float32) * np.float32(40.0 * ks)
    flat = x.reshape(-1)
    pick = rng.permutation(flat.size)
    flat[pick[:40]] = 1e5                                # clamps
    flat[pick[40:80]] = -3e4
    halves = (rng.integers(-120, 120, 60) + 0.5).astype(np.float32)
    flat[pick[80:140]] = halves * np.float32(ks)         # ties (exact where the scale is a power of two)
    flat[pick[140:150]] = -0.0
    flat[pick[150:155]] = np.inf
    flat[pick[155:158]] = -np.inf
    flat[pick[158:163]] = np.nan
    if rows_dtype == W.BF16:
        bits = W.f32_to_bf16_bits(x)
        x = W.bf16_bits_to_f32(bits)
        kd = torch.from_numpy(bits[0].view(np.int16)).to(DEV).view(torch.bfloat16)
        vd = torch.from_numpy(bits[1].view(np.int16)).to(DEV).view(torch.bfloat16)
    else:
        kd, vd = torch.from_numpy(x[0]).to(DEV), torch.from_numpy(x[1]).to(DEV)
    slots = rng.permutation(nb * 16)[:t].astype(np.int32)
    slots[:5] = -1                                       # padding rows
    slots[5] = nb * 16 + 3                               # past the pool: skipped
    say(f"[int8 append] rows {rows_dtype} k_scale {ks} v_scale {vs}")
    init_k = W.int8_codes(np.random.default_rng(5), (nb, hkv, 16, d))
    init_v = W.int8_codes(np.random.default_rng(6), (nb, hkv, 16, d))
    dk, dv = W.fp8_pools_to_device_order(init_k, init_v)
    kp, vp = _dev8(dk), _dev8(dv)
    pak.kvcache_append_int8(kp, vp, kd, vd, _dev8(slots), ks, vs)
    torch.cuda.synchronize()
    wk, wv = oracle.append_int8(init_k, init_v, x[0], x[1], slots, np.float32(ks), np.float32(vs))
    gk, gv = W.fp8_pools_from_device_order(_host8(kp), _host8(vp))
    bad = int((gk != wk).sum() + (gv != wv).sum())
    say(f"  mismatching bytes: {bad}")
    assert bad == 0


def _codes(case, seed):
    rng = np.random.default_rng(seed)
    shape = (case.layout.num_blocks, case.num_kv_heads, 16, case.head_dim)
    return W.int8_codes(rng, shape), W.int8_codes(rng, shape)


def _run_decode(case, seed, ks, vs, split=0):
    W.materialize_numpy(case)
    kc, vc = _codes(case, seed)
    dc = DeviceCase(case)
    k8, v8 = (_dev8(x) for x in W.fp8_pools_to_device_order(kc, vc))
    if dc.k_new.shape[0]:
        pak.kvcache_append_int8(k8, v8, dc.k_new, dc.v_new, dc.slots, ks, vs)
    out = pak.lazyattn_decode_int8(dc.q, dc.q_pos, k8, v8, dc.table, dc.seq_lens, ks, vs, scale=case.scale,
                                   rope_theta=case.rope_theta, split_blocks=split, block_fill=dc.fill)
    torch.cuda.synchronize()
    kn, vn = W.to_float(case.k_new, case.dtype), W.to_float(case.v_new, case.dtype)
    kc2, vc2 = oracle.append_int8(kc, vc, kn, vn, case.layout.slot_mapping, np.float32(ks), np.float32(vs))
    gk, gv = W.fp8_pools_from_device_order(_host8(k8), _host8(v8))
    assert np.array_equal(gk, kc2) and np.array_equal(gv, vc2), "append bytes"
    want = oracle.decode_int8(W.to_float(case.q, case.dtype), case.q_pos, kc2, vc2, case.layout.table,
                              case.seq_lens, case.scale, case.rope_theta, np.float32(ks), np.float32(vs),
                              block_fill=case.block_fill)
    return W.to_float(out, case.dtype), want


DECODE = [
    # Hq, Hkv, ctx, doc blocks, offsets, split, k_scale, v_scale
    (32, 8, [512, 1024, 96], (2, 10), "contiguous", 0, 0.01, 0.005),
    (64, 8, [1024, 16, 336], (2, 12), "random", 0, 0.01, 0.02),
    (32, 1, [400, 96], (2, 9), "contiguous", 4, 0.008, 0.004),
    (16, 8, [320, 16, 784], (1, 6), "random", 4, 0.012, 0.003),
]


@pytest.mark.parametrize("hq,hkv,ctx,docs,offs,split,ks,vs", DECODE)
def test_decode_int8(hq, hkv, ctx, docs, offs, split, ks, vs):
    case = W.decode_case(281 + hq + hkv, len(ctx), hq, hkv, 128, ctx, docs, offsets=offs)
    say(f"[int8 decode] Hq{hq} Hkv{hkv} ctx={ctx} {offs} split={split} k_scale {ks} v_scale {vs}")
    got, want = _run_decode(case, 7 + hq, ks, vs, split)
    assert_parity(got, want, W.BF16, f"int8 decode G{hq // hkv}")


def test_decode_int8_ragged_documents():
    case = W.ragged_case(291, "decode", 4, 32, 8, 128, (2, 6), (1, 700))
    say("[int8 decode] ragged documents, fill counts")
    got, want = _run_decode(case, 9, 0.01, 0.005, 4)
    assert_parity(got, want, W.BF16, "int8 decode ragged")


def test_single_token_reads_every_code_exactly():
    """A one-token sequence gives out = v_scale * code exactly (the softmax of
    one key is 1; a power-of-two scale keeps the product exact), for every
    code -128 .. 127 in one head's value row."""
    hkv, hq, d = 2, 8, 128
    nb = 4
    vc = np.zeros((nb, hkv, 16, d), dtype=np.int8)
    vc[1, 0, 0] = np.arange(-128, 0, dtype=np.int64).astype(np.int8)
    vc[1, 1, 0] = np.arange(0, 128, dtype=np.int64).astype(np.int8)
    rng = np.random.default_rng(2)
    kc = W.int8_codes(rng, (nb, hkv, 16, d))
    q = torch.from_numpy(W.f32_to_bf16_bits(rng.standard_normal((1, hq, d)).astype(np.float32)).view(np.int16))
    q = q.to(DEV).view(torch.bfloat16)
    table = _dev8(np.array([[1 | (7 << 16)]], dtype=np.uint32).view(np.int32))
    kd, vd = W.fp8_pools_to_device_order(kc, vc)
    out = pak.lazyattn_decode_int8(q, _dev8(np.array([7], np.int32)), _dev8(kd), _dev8(vd), table,
                                   _dev8(np.array([1], np.int32)), 0.25, 0.5)
    torch.cuda.synchronize()
    got = W.to_float(out, W.BF16)[0]
    for h in range(hq):
        want = (np.arange(-128, 0) if h < hq // hkv else np.arange(0, 128)) * 0.5
        assert np.array_equal(got[h], want), f"head {h}"


def _run_prefill(case, seed, ks, vs, precise=False):
    W.materialize_numpy(case)
    kc, vc = _codes(case, seed)
    dc = DeviceCase(case)
    k8, v8 = (_dev8(x) for x in W.fp8_pools_to_device_order(kc, vc))
    pak.kvcache_append_int8(k8, v8, dc.k_new, dc.v_new, dc.slots, ks, vs)
    fn = pak.lazyattn_prefill_int8_precise if precise else pak.lazyattn_prefill_int8
    out = fn(dc.q, dc.cu, dc.q_pos_start, k8, v8, dc.table, dc.seq_lens, case.max_q_len,
             ks, vs, scale=case.scale, rope_theta=case.rope_theta, block_fill=dc.fill)
    torch.cuda.synchronize()
    kn, vn = W.to_float(case.k_new, case.dtype), W.to_float(case.v_new, case.dtype)
    kc2, vc2 = oracle.append_int8(kc, vc, kn, vn, case.layout.slot_mapping, np.float32(ks), np.float32(vs))
    gk, gv = W.fp8_pools_from_device_order(_host8(k8), _host8(v8))
    assert np.array_equal(gk, kc2) and np.array_equal(gv, vc2), "append bytes"
    want = oracle.prefill_int8(W.to_float(case.q, case.dtype), case.cu_q_lens, case.layout.tail_pos, kc2, vc2,
                               case.layout.table, case.seq_lens, case.scale, case.rope_theta, np.float32(ks),
                               np.float32(vs), block_fill=case.block_fill)
    return W.to_float(out, case.dtype), want


PREFILL = [
    # Hq, Hkv, cached per sequence, prompt per sequence, doc blocks, offsets, k_scale, v_scale
    (32, 8, [512, 96], [256, 77], (2, 12), "contiguous", 0.01, 0.005),
    (16, 8, [224, 640], [300, 129], (2, 20), "random", 0.012, 0.003),
    (8, 8, [320, 48], [150, 31], (2, 10), "random", 0.008, 0.02),
]


@pytest.mark.parametrize("hq,hkv,cached,prompt,docs,offs,ks,vs", PREFILL)
def test_prefill_int8(hq, hkv, cached, prompt, docs, offs, ks, vs):
    case = W.prefill_case(301 + hq + hkv, len(prompt), hq, hkv, 128, cached, prompt, docs, offsets=offs)
    say(f"[int8 prefill] Hq{hq} Hkv{hkv} cached={cached} prompt={prompt} {offs} k_scale {ks} v_scale {vs}")
    got, want = _run_prefill(case, 17 + hq, ks, vs)
    assert_parity(got, want, W.BF16, f"int8 prefill G{hq // hkv}")


def test_prefill_int8_ragged_documents():
    case = W.ragged_case(311, "prefill", 3, 32, 8, 128, (2, 5), (1, 600), prompt=(1, 300))
    say("[int8 prefill] ragged documents, fill counts")
    got, want = _run_prefill(case, 19, 0.01, 0.005)
    assert_parity(got, want, W.BF16, "int8 prefill ragged")


def test_prefill_int8_equals_bf16_prefill_on_dequantised_pool():
    """Every int8 code times a power-of-two scale is a bf16 value, and a
    power-of-two K scale folded into the rotated query rounds exactly as the
    unscaled query does, so the int8 prefill must equal the bf16 prefill on
    the dequantised pool bit for bit (byte order and widening, element by
    element)."""
    ks, vs = 2.0 ** -6, 2.0 ** -7
    case = W.prefill_case(321, 2, 64, 8, 128, [704, 160], [190, 64], (2, 16), offsets="random")
    say("[int8 prefill == bf16 prefill]")
    W.materialize_numpy(case)
    kc, vc = _codes(case, 23)
    dc = DeviceCase(case)
    k8, v8 = (_dev8(x) for x in W.fp8_pools_to_device_order(kc, vc))
    pak.kvcache_append_int8(k8, v8, dc.k_new, dc.v_new, dc.slots, ks, vs)
    out8 = pak.lazyattn_prefill_int8(dc.q, dc.cu, dc.q_pos_start, k8, v8, dc.table, dc.seq_lens, case.max_q_len,
                                     ks, vs, scale=case.scale, rope_theta=case.rope_theta)
    torch.cuda.synchronize()
    kc2, vc2 = W.fp8_pools_from_device_order(_host8(k8), _host8(v8))

    def bf16_pool(codes, sc):
        x = oracle.dequantize_int8(codes, np.float32(sc)).astype(np.float32)
        bits = W.f32_to_bf16_bits(x)
        assert np.array_equal(W.bf16_bits_to_f32(bits), x), "dequantised codes are bf16 values"
        return torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    out16 = pak.lazyattn_prefill(dc.q, dc.cu, dc.q_pos_start, bf16_pool(kc2, ks), bf16_pool(vc2, vs), dc.table,
                                 dc.seq_lens, case.max_q_len, scale=case.scale, rope_theta=case.rope_theta)
    torch.cuda.synchronize()
    assert torch.equal(out8.view(torch.int16), out16.view(torch.int16))


def test_full_size_decode_int8_sampled():
    """The 8B decode shape over an int8 pool at full size (automatic split),
    against the oracle on sampled (sequence, head) rows.  Pools: random int8
    codes drawn on the GPU; the oracle reads the sampled sequences' blocks as
    generated and appends the new rows itself."""
    ks, vs = 0.01, 0.005
    case = W.make("llama8b_decode")
    say(f"[full int8 decode] B={case.batch} NB={case.layout.num_blocks}")
    W.materialize_torch(case, DEV)
    dc = DeviceCase(case)
    shape = tuple(dc.k_pool.shape)
    dc.k_pool = dc.v_pool = None
    case.k_pool = case.v_pool = None
    torch.cuda.empty_cache()
    k8 = W.int8_codes_torch(shape, DEV, case.seed + 7000)
    v8 = W.int8_codes_torch(shape, DEV, case.seed + 8000)
    lay = case.layout
    rng = np.random.default_rng(7)
    seqs = sorted(rng.choice(case.batch, size=4, replace=False).tolist())
    ids = []
    for b in seqs:
        ids.extend((lay.table[b, :-(-int(case.seq_lens[b]) // 16)] & 0xFFFF).tolist())
    uniq = np.unique(np.array(ids, dtype=np.int64))
    remap = {int(x): i for i, x in enumerate(uniq)}
    sel = torch.from_numpy(uniq).to(DEV)
    kc, vc = W.fp8_pools_from_device_order(_host8(k8.index_select(0, sel)), _host8(v8.index_select(0, sel)))
    rows, slots = [], []
    for t, sl in enumerate(lay.slot_mapping.tolist()):
        if sl >= 0 and sl // 16 in remap:
            rows.append(t)
            slots.append(remap[sl // 16] * 16 + sl % 16)
    r = torch.tensor(rows, device=DEV)
    kc, vc = oracle.append_int8(kc, vc, W.to_float(dc.k_new.index_select(0, r), W.BF16),
                                W.to_float(dc.v_new.index_select(0, r), W.BF16), np.array(slots),
                                np.float32(ks), np.float32(vs))
    kf, vf = oracle.dequantize_int8(kc, np.float32(ks)), oracle.dequantize_int8(vc, np.float32(vs))
    tab = np.zeros((len(seqs), lay.table.shape[1]), dtype=np.uint32)
    for i, b in enumerate(seqs):
        for j in range(-(-int(case.seq_lens[b]) // 16)):
            w = int(lay.table[b, j])
            tab[i, j] = (w & 0xFFFF0000) | remap[w & 0xFFFF]
    pak.kvcache_append_int8(k8, v8, dc.k_new, dc.v_new, dc.slots, ks, vs)
    out = pak.lazyattn_decode_int8(dc.q, dc.q_pos, k8, v8, dc.table, dc.seq_lens, ks, vs, scale=case.scale,
                                   rope_theta=case.rope_theta)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    q = W.to_float(case.q, W.BF16)
    got = W.to_float(out, W.BF16)
    g = case.num_q_heads // case.num_kv_heads
    rows_got, rows_want = [], []
    for i, b in enumerate(seqs):
        for h in rng.choice(case.num_q_heads, size=3, replace=False).tolist():
            rows_want.append(oracle.decode_one(q[b, h], int(case.q_pos[b]), kf, vf, tab[i], int(case.seq_lens[b]),
                                               h // g, case.scale, case.rope_theta))
            rows_got.append(got[b, h])
    assert_parity(np.stack(rows_got), np.stack(rows_want), W.BF16, "llama8b_decode int8 sampled")


@pytest.mark.parametrize("hq,hkv,cached,prompt,docs,offs,ks,vs", PREFILL + [
    (32, 8, [512, 96], [256, 77], (2, 12), "random", 0.08, 0.005),   # a K scale that spreads the scores
])
def test_prefill_int8_precise(hq, hkv, cached, prompt, docs, offs, ks, vs):
    """lazyattn_prefill_int8_precise against the oracle, including a K scale
    that spreads each row's scores several units wide."""
    case = W.prefill_case(331 + hq + int(ks * 1000), len(prompt), hq, hkv, 128, cached, prompt, docs,
                          offsets=offs)
    say(f"[int8 precise prefill] Hq{hq} Hkv{hkv} k_scale {ks} v_scale {vs} {offs}")
    got, want = _run_prefill(case, 67, ks, vs, precise=True)
    assert_parity(got, want, W.BF16, f"int8 precise prefill k_scale {ks}")

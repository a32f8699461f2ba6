"""GPU parity of the 8-bit KV pool (kvcache_append_fp8, lazyattn_decode_fp8,
lazyattn_prefill_fp8) against the E4M3 oracle.  Pools hold random E4M3 byte patterns (every
exponent from subnormal to 2^2, both signs); the step's new rows are bf16 or
f32 values that the append quantises, bit for bit as the oracle does,
including saturation, subnormals, signed zero, infinities and NaN.  The
device pools hold the codes in the library's lane order; the tests move host
codes into it and back with the index permutation the header documents.  Decode
covers GQA 4, GQA 8 (two workgroups per KV head), a 32-query-head group,
split-K, random offsets and documents of any length (fill counts); prefill
covers GQA 1 to 8, multi-query, random offsets, a prompt with no cached
document, documents of any length, and bit-equality with the bf16 prefill on
the dequantised pool."""

import numpy as np
import pytest
import torch

import oracle
import position_agnostic_kv_amd as pak
import workloads as W
from tests.gpu_helpers import DEV, DeviceCase, assert_parity, say

pytestmark = pytest.mark.gpu


def _u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


@pytest.mark.parametrize("rows_dtype", [W.BF16, W.F32])
@pytest.mark.parametrize("ks,vs", [(1.0, 1.0), (0.05, 0.37), (3.0, 1.0e-3)])
def test_append_fp8_bit_exact(rows_dtype, ks, vs):
    rng = np.random.default_rng(11)
    nb, hkv, d, t = 8, 4, 128, 70
    x = rng.standard_normal((2, t, hkv, d)).astype(np.float32) * np.float32(4.0)
    flat = x.reshape(-1)
    pick = rng.permutation(flat.size)
    flat[pick[:40]] = 1e5                              # saturates
    flat[pick[40:80]] = -3e4
    flat[pick[80:120]] = rng.standard_normal(40) * 1e-4  # subnormal codes and zeros
    flat[pick[120:130]] = -0.0
    flat[pick[130:135]] = np.inf
    flat[pick[135:140]] = np.nan
    if rows_dtype == W.BF16:
        bits = W.f32_to_bf16_bits(x)
        x = W.bf16_bits_to_f32(bits)
        kd = torch.from_numpy(bits[0].view(np.int16)).to(DEV).view(torch.bfloat16)
        vd = torch.from_numpy(bits[1].view(np.int16)).to(DEV).view(torch.bfloat16)
    else:
        kd, vd = torch.from_numpy(x[0]).to(DEV), torch.from_numpy(x[1]).to(DEV)
    slots = rng.permutation(nb * 16)[:t].astype(np.int32)
    slots[:5] = -1                                     # padding rows
    slots[5] = nb * 16 + 3                             # past the pool: skipped
    say(f"[fp8 append] rows {rows_dtype} k_scale {ks} v_scale {vs}")
    init_k = np.random.default_rng(5).integers(0, 256, (nb, hkv, 16, d)).astype(np.uint8)
    init_v = np.random.default_rng(6).integers(0, 256, (nb, hkv, 16, d)).astype(np.uint8)
    dk, dv = W.fp8_pools_to_device_order(init_k, init_v)
    kp, vp = _u8(dk), _u8(dv)
    pak.kvcache_append_fp8(kp, vp, kd, vd, _u8(slots), ks, vs)
    torch.cuda.synchronize()
    wk, wv = oracle.append_fp8(init_k, init_v, x[0], x[1], slots, np.float32(ks), np.float32(vs))
    gk, gv = W.fp8_pools_from_device_order(kp.cpu().numpy(), vp.cpu().numpy())
    bad = int((gk != wk).sum() + (gv != wv).sum())
    say(f"  mismatching bytes: {bad}")
    assert bad == 0


def _fp8_case(case, seed):
    rng = np.random.default_rng(seed)
    shape = (case.layout.num_blocks, case.num_kv_heads, 16, case.head_dim)
    return W.e4m3_codes(rng, shape), W.e4m3_codes(rng, shape)


def _run(case, seed, ks, vs, split=0):
    W.materialize_numpy(case)
    kc, vc = _fp8_case(case, seed)
    dc = DeviceCase(case)
    k8, v8 = (_u8(x) for x in W.fp8_pools_to_device_order(kc, vc))
    if dc.k_new.shape[0]:
        pak.kvcache_append_fp8(k8, v8, dc.k_new, dc.v_new, dc.slots, ks, vs)
    out = pak.lazyattn_decode_fp8(dc.q, dc.q_pos, k8, v8, dc.table, dc.seq_lens, ks, vs, scale=case.scale,
                                  rope_theta=case.rope_theta, split_blocks=split, block_fill=dc.fill)
    torch.cuda.synchronize()
    kn, vn = W.to_float(case.k_new, case.dtype), W.to_float(case.v_new, case.dtype)
    kc2, vc2 = oracle.append_fp8(kc, vc, kn, vn, case.layout.slot_mapping, np.float32(ks), np.float32(vs))
    gk, gv = W.fp8_pools_from_device_order(k8.cpu().numpy(), v8.cpu().numpy())
    assert np.array_equal(gk, kc2) and np.array_equal(gv, vc2), "append bytes"
    want = oracle.decode_fp8(W.to_float(case.q, case.dtype), case.q_pos, kc2, vc2, case.layout.table,
                             case.seq_lens, case.scale, case.rope_theta, np.float32(ks), np.float32(vs),
                             block_fill=case.block_fill)
    return W.to_float(out, case.dtype), want


DECODE = [
    # Hq, Hkv, ctx, doc blocks, offsets, split, k_scale, v_scale
    (32, 8, [512, 1024, 96], (2, 10), "contiguous", 0, 0.25, 0.125),
    (64, 8, [2048, 64], (4, 16), "contiguous", 8, 0.25, 0.5),
    (64, 8, [1024, 16, 336], (2, 12), "random", 0, 0.25, 0.5),
    (32, 1, [400, 96], (2, 9), "contiguous", 0, 0.2, 0.1),
    (64, 1, [272, 48], (2, 9), "contiguous", 4, 0.2, 0.1),
    (16, 1, [208, 512], (1, 8), "random", 0, 0.2, 0.1),
    (16, 8, [320, 16, 784], (1, 6), "random", 4, 0.3, 0.07),
    (8, 8, [1056, 48], (3, 40), "contiguous", 5, 0.25, 1.0),
]


@pytest.mark.parametrize("hq,hkv,ctx,docs,offs,split,ks,vs", DECODE)
def test_decode_fp8(hq, hkv, ctx, docs, offs, split, ks, vs):
    case = W.decode_case(201 + hq + hkv, len(ctx), hq, hkv, 128, ctx, docs, offsets=offs)
    say(f"[fp8 decode] Hq{hq} Hkv{hkv} ctx={ctx} {offs} split={split} k_scale {ks} v_scale {vs}")
    got, want = _run(case, 7 + hq, ks, vs, split)
    assert_parity(got, want, W.BF16, f"fp8 decode G{hq // hkv}")


def test_decode_fp8_ragged_documents():
    case = W.ragged_case(221, "decode", 4, 32, 8, 128, (2, 6), (1, 700))
    say("[fp8 decode] ragged documents, fill counts")
    got, want = _run(case, 9, 0.25, 0.125, 4)
    assert_parity(got, want, W.BF16, "fp8 decode ragged")


def test_single_token_reads_every_code_exactly():
    """A sequence of one token gives out = v_scale * decode(v code) exactly (the
    softmax of one key is 1); v_scale a power of two keeps the product exact,
    so all 256 codes (NaN patterns included) must come out bit for bit."""
    hkv, hq, d = 2, 8, 128
    nb = 4
    vc = np.zeros((nb, hkv, 16, d), dtype=np.uint8)
    vc[1, 0, 0] = np.arange(128, dtype=np.uint8)
    vc[1, 1, 0] = np.arange(128, 256, dtype=np.uint8)
    rng = np.random.default_rng(2)
    kc = W.e4m3_codes(rng, (nb, hkv, 16, d))
    q = torch.from_numpy(W.f32_to_bf16_bits(rng.standard_normal((1, hq, d)).astype(np.float32)).view(np.int16))
    q = q.to(DEV).view(torch.bfloat16)
    table = _u8(np.array([[1 | (7 << 16)]], dtype=np.uint32).view(np.int32))
    kd, vd = W.fp8_pools_to_device_order(kc, vc)
    out = pak.lazyattn_decode_fp8(q, _u8(np.array([7], np.int32)), _u8(kd), _u8(vd), table,
                                  _u8(np.array([1], np.int32)), 0.25, 0.5)
    torch.cuda.synchronize()
    got = W.to_float(out, W.BF16)[0]                       # [Hq, D]
    ref = oracle.e4m3_decode(np.arange(256, dtype=np.uint8)) * 0.5
    for h in range(hq):
        want = ref[:128] if h < hq // hkv else ref[128:]
        same = (got[h] == want) | (np.isnan(got[h]) & np.isnan(want))
        assert same.all(), f"head {h}: {np.flatnonzero(~same)[:8]}"


@pytest.mark.parametrize("name", ["llama8b_decode", "llama70b_decode"])
def test_full_size_decode_fp8_sampled(name):
    """The bench's 8-bit shapes at full size, in its launch configuration
    (automatic split), against the oracle on sampled (sequence, head) rows.
    Pools: random E4M3 bytes drawn on the GPU; the oracle reads the sampled
    sequences' blocks as generated and appends the new rows itself."""
    ks, vs = 0.25, 0.125
    case = W.make(name)
    say(f"[full fp8 decode] {name} B={case.batch} NB={case.layout.num_blocks}")
    W.materialize_torch(case, DEV)
    dc = DeviceCase(case)
    shape = tuple(dc.k_pool.shape)
    dc.k_pool = dc.v_pool = None
    case.k_pool = case.v_pool = None
    torch.cuda.empty_cache()
    k8 = W.e4m3_codes_torch(shape, DEV, case.seed + 5000)
    v8 = W.e4m3_codes_torch(shape, DEV, case.seed + 6000)
    lay = case.layout
    rng = np.random.default_rng(5)
    seqs = sorted(rng.choice(case.batch, size=min(4, case.batch), replace=False).tolist())
    ids = []
    for b in seqs:
        ids.extend((lay.table[b, :-(-int(case.seq_lens[b]) // 16)] & 0xFFFF).tolist())
    uniq = np.unique(np.array(ids, dtype=np.int64))
    remap = {int(x): i for i, x in enumerate(uniq)}
    sel = torch.from_numpy(uniq).to(DEV)
    kc, vc = W.fp8_pools_from_device_order(k8.index_select(0, sel).cpu().numpy(),
                                           v8.index_select(0, sel).cpu().numpy())
    rows, slots = [], []
    for t, sl in enumerate(lay.slot_mapping.tolist()):
        if sl >= 0 and sl // 16 in remap:
            rows.append(t)
            slots.append(remap[sl // 16] * 16 + sl % 16)
    r = torch.tensor(rows, device=DEV)
    kc, vc = oracle.append_fp8(kc, vc, W.to_float(dc.k_new.index_select(0, r), W.BF16),
                               W.to_float(dc.v_new.index_select(0, r), W.BF16), np.array(slots),
                               np.float32(ks), np.float32(vs))
    kf, vf = oracle.dequantize(kc, np.float32(ks)), oracle.dequantize(vc, np.float32(vs))
    tab = np.zeros((len(seqs), lay.table.shape[1]), dtype=np.uint32)
    for i, b in enumerate(seqs):
        for j in range(-(-int(case.seq_lens[b]) // 16)):
            w = int(lay.table[b, j])
            tab[i, j] = (w & 0xFFFF0000) | remap[w & 0xFFFF]
    pak.kvcache_append_fp8(k8, v8, dc.k_new, dc.v_new, dc.slots, ks, vs)
    out = pak.lazyattn_decode_fp8(dc.q, dc.q_pos, k8, v8, dc.table, dc.seq_lens, ks, vs, scale=case.scale,
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
    assert_parity(np.stack(rows_got), np.stack(rows_want), W.BF16, f"{name} fp8 sampled")


# ---------------------------------------------------------------- prefill
def _run_prefill(case, seed, ks, vs, precise=False):
    """Append the prompts' rows into an 8-bit pool of random codes, prefill,
    and return (got, want) with the oracle on the same codes (the append
    bytes checked exactly on the way)."""
    W.materialize_numpy(case)
    kc, vc = _fp8_case(case, seed)
    dc = DeviceCase(case)
    k8, v8 = (_u8(x) for x in W.fp8_pools_to_device_order(kc, vc))
    pak.kvcache_append_fp8(k8, v8, dc.k_new, dc.v_new, dc.slots, ks, vs)
    fn = pak.lazyattn_prefill_fp8_precise if precise else pak.lazyattn_prefill_fp8
    out = fn(dc.q, dc.cu, dc.q_pos_start, k8, v8, dc.table, dc.seq_lens, case.max_q_len,
             ks, vs, scale=case.scale, rope_theta=case.rope_theta, block_fill=dc.fill)
    torch.cuda.synchronize()
    kn, vn = W.to_float(case.k_new, case.dtype), W.to_float(case.v_new, case.dtype)
    kc2, vc2 = oracle.append_fp8(kc, vc, kn, vn, case.layout.slot_mapping, np.float32(ks), np.float32(vs))
    gk, gv = W.fp8_pools_from_device_order(k8.cpu().numpy(), v8.cpu().numpy())
    assert np.array_equal(gk, kc2) and np.array_equal(gv, vc2), "append bytes"
    want = oracle.prefill_fp8(W.to_float(case.q, case.dtype), case.cu_q_lens, case.layout.tail_pos, kc2, vc2,
                              case.layout.table, case.seq_lens, case.scale, case.rope_theta, np.float32(ks),
                              np.float32(vs), block_fill=case.block_fill)
    return W.to_float(out, case.dtype), want


PREFILL = [
    # Hq, Hkv, cached per sequence, prompt per sequence, doc blocks, offsets, k_scale, v_scale
    (32, 8, [512, 96], [256, 77], (2, 12), "contiguous", 0.25, 0.125),
    (64, 8, [1056], [130], (3, 40), "random", 0.25, 0.5),
    (16, 8, [224, 640], [300, 129], (2, 20), "contiguous", 0.3, 0.07),
    (8, 8, [320, 48], [150, 31], (2, 10), "random", 0.2, 1.0),
    (32, 1, [416, 96], [200, 70], (2, 9), "random", 0.2, 0.1),
    (32, 8, [0, 96], [77, 200], (1, 4), "contiguous", 0.5, 0.25),
]


@pytest.mark.parametrize("hq,hkv,cached,prompt,docs,offs,ks,vs", PREFILL)
def test_prefill_fp8(hq, hkv, cached, prompt, docs, offs, ks, vs):
    case = W.prefill_case(241 + hq + hkv, len(prompt), hq, hkv, 128, cached, prompt, docs, offsets=offs)
    say(f"[fp8 prefill] Hq{hq} Hkv{hkv} cached={cached} prompt={prompt} {offs} k_scale {ks} v_scale {vs}")
    got, want = _run_prefill(case, 17 + hq, ks, vs)
    assert_parity(got, want, W.BF16, f"fp8 prefill G{hq // hkv}")


def test_prefill_fp8_ragged_documents():
    case = W.ragged_case(251, "prefill", 3, 32, 8, 128, (2, 5), (1, 600), prompt=(1, 300))
    say("[fp8 prefill] ragged documents, fill counts")
    got, want = _run_prefill(case, 19, 0.25, 0.125)
    assert_parity(got, want, W.BF16, "fp8 prefill ragged")


@pytest.mark.parametrize("kind", ["documents", "ragged"])
def test_prefill_fp8_equals_bf16_prefill_on_dequantised_pool(kind):
    """Every E4M3 value times a power-of-two scale is a bf16 value, and a
    power-of-two K scale folded into the rotated query rounds exactly as the
    unscaled query does, so the 8-bit prefill must equal the bf16 prefill on
    the dequantised pool bit for bit: this checks the codes' byte order and
    the widening pass element by element."""
    ks, vs = 0.25, 0.5
    if kind == "ragged":
        case = W.ragged_case(261, "prefill", 2, 32, 8, 128, (2, 4), (1, 500), prompt=(1, 200))
    else:
        case = W.prefill_case(263, 2, 64, 8, 128, [704, 160], [190, 64], (2, 16), offsets="random")
    say(f"[fp8 prefill == bf16 prefill] {kind}")
    W.materialize_numpy(case)
    kc, vc = _fp8_case(case, 23)
    dc = DeviceCase(case)
    k8, v8 = (_u8(x) for x in W.fp8_pools_to_device_order(kc, vc))
    pak.kvcache_append_fp8(k8, v8, dc.k_new, dc.v_new, dc.slots, ks, vs)
    out8 = pak.lazyattn_prefill_fp8(dc.q, dc.cu, dc.q_pos_start, k8, v8, dc.table, dc.seq_lens, case.max_q_len,
                                    ks, vs, scale=case.scale, rope_theta=case.rope_theta, block_fill=dc.fill)
    torch.cuda.synchronize()
    kc2, vc2 = W.fp8_pools_from_device_order(k8.cpu().numpy(), v8.cpu().numpy())

    def bf16_pool(codes, sc):
        x = oracle.dequantize(codes, np.float32(sc)).astype(np.float32)
        bits = W.f32_to_bf16_bits(x)
        assert np.array_equal(W.bf16_bits_to_f32(bits), x), "dequantised codes are bf16 values"
        return torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    out16 = pak.lazyattn_prefill(dc.q, dc.cu, dc.q_pos_start, bf16_pool(kc2, ks), bf16_pool(vc2, vs), dc.table,
                                 dc.seq_lens, case.max_q_len, scale=case.scale, rope_theta=case.rope_theta,
                                 block_fill=dc.fill)
    torch.cuda.synchronize()
    assert torch.equal(out8.view(torch.int16), out16.view(torch.int16))


def test_prefill_fp8_caller_workspace_contents_are_irrelevant():
    """The widened copy lives in the caller's workspace: a workspace full of
    NaN patterns (slots the batch cannot see are never written or read), the
    same workspace again for a smaller batch, and the binding's own
    workspace all give the same bits."""
    ks, vs = 0.25, 0.125
    case = W.prefill_case(271, 3, 32, 8, 128, [512, 96, 304], [256, 77, 40], (2, 12), offsets="random")
    say("[fp8 prefill] caller workspace, NaN-filled, reused")
    W.materialize_numpy(case)
    kc, vc = _fp8_case(case, 29)
    dc = DeviceCase(case)
    k8, v8 = (_u8(x) for x in W.fp8_pools_to_device_order(kc, vc))
    pak.kvcache_append_fp8(k8, v8, dc.k_new, dc.v_new, dc.slots, ks, vs)
    need = pak.prefill_fp8_workspace_size(case.batch, dc.table.shape[1], case.num_kv_heads)
    assert need > 0
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)

    def run(workspace, nseq):
        tq = int(case.cu_q_lens[nseq])
        return pak.lazyattn_prefill_fp8(dc.q[:tq], dc.cu[:nseq + 1], dc.q_pos_start[:nseq], k8, v8,
                                        dc.table[:nseq], dc.seq_lens[:nseq], case.max_q_len, ks, vs,
                                        scale=case.scale, rope_theta=case.rope_theta, block_fill=dc.fill,
                                        workspace=workspace)
    own = run(None, case.batch)
    mine = run(ws, case.batch)
    again = run(ws, 2)
    torch.cuda.synchronize()
    assert torch.isfinite(mine.float()).all()
    assert torch.equal(own.view(torch.int16), mine.view(torch.int16))
    assert torch.equal(again.view(torch.int16), own[:again.shape[0]].view(torch.int16))
    with pytest.raises(pak.LazyAttnError):
        run(ws[:need - 1], case.batch)


def test_full_size_prefill_fp8_sampled():
    """The 8B prefill shape over an 8-bit pool at full size, as bench.py
    --shapes runs it, against the oracle on sampled prompt rows of two
    sequences.  Pools: random E4M3 bytes drawn on the GPU; the oracle reads
    the sampled sequences' blocks as generated and appends the prompts itself."""
    ks, vs = 0.25, 0.125
    case = W.make("llama8b_prefill")
    say(f"[full fp8 prefill] B={case.batch} prompt={case.max_q_len} NB={case.layout.num_blocks}")
    W.materialize_torch(case, DEV)
    dc = DeviceCase(case)
    shape = tuple(dc.k_pool.shape)
    dc.k_pool = dc.v_pool = None
    case.k_pool = case.v_pool = None
    torch.cuda.empty_cache()
    k8 = W.e4m3_codes_torch(shape, DEV, case.seed + 5000)
    v8 = W.e4m3_codes_torch(shape, DEV, case.seed + 6000)
    lay = case.layout
    seqs = [0, 3]
    ids = []
    for b in seqs:
        ids.extend((lay.table[b, :-(-int(case.seq_lens[b]) // 16)] & 0xFFFF).tolist())
    uniq = np.unique(np.array(ids, dtype=np.int64))
    remap = {int(x): i for i, x in enumerate(uniq)}
    sel = torch.from_numpy(uniq).to(DEV)
    kc, vc = W.fp8_pools_from_device_order(k8.index_select(0, sel).cpu().numpy(),
                                           v8.index_select(0, sel).cpu().numpy())
    rows, slots = [], []
    for t, sl in enumerate(lay.slot_mapping.tolist()):
        if sl >= 0 and sl // 16 in remap:
            rows.append(t)
            slots.append(remap[sl // 16] * 16 + sl % 16)
    r = torch.tensor(rows, device=DEV)
    kc, vc = oracle.append_fp8(kc, vc, W.to_float(dc.k_new.index_select(0, r), W.BF16),
                               W.to_float(dc.v_new.index_select(0, r), W.BF16), np.array(slots),
                               np.float32(ks), np.float32(vs))
    kf, vf = oracle.dequantize(kc, np.float32(ks)), oracle.dequantize(vc, np.float32(vs))
    tab = np.zeros((len(seqs), lay.table.shape[1]), dtype=np.uint32)
    for i, b in enumerate(seqs):
        for j in range(-(-int(case.seq_lens[b]) // 16)):
            w = int(lay.table[b, j])
            tab[i, j] = (w & 0xFFFF0000) | remap[w & 0xFFFF]
    pak.kvcache_append_fp8(k8, v8, dc.k_new, dc.v_new, dc.slots, ks, vs)
    out = pak.lazyattn_prefill_fp8(dc.q, dc.cu, dc.q_pos_start, k8, v8, dc.table, dc.seq_lens, case.max_q_len,
                                   ks, vs, scale=case.scale, rope_theta=case.rope_theta)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    q = W.to_float(case.q, W.BF16)
    got = W.to_float(out, W.BF16)
    g = case.num_q_heads // case.num_kv_heads
    rng = np.random.default_rng(6)
    qrows = np.array([0, 1, 2, 127, 128, 129, 1023, 1024, 2046, 2047])
    gots, wants = [], []
    for i, b in enumerate(seqs):
        q0 = int(case.cu_q_lens[b])
        for h in rng.choice(case.num_q_heads, size=3, replace=False).tolist():
            wants.append(oracle.prefill_rows(q[q0 + qrows, h], qrows, case.max_q_len, int(lay.tail_pos[b]), kf, vf,
                                             tab[i], int(case.seq_lens[b]), h // g, case.scale, case.rope_theta))
            gots.append(got[q0 + qrows, h])
    assert_parity(np.concatenate(gots), np.concatenate(wants), W.BF16, "llama8b_prefill fp8 sampled")


@pytest.mark.parametrize("hq,hkv,cached,prompt,docs,offs,ks,vs", PREFILL[:3] + [
    (32, 8, [512, 96], [256, 77], (2, 12), "random", 3.0, 0.25),   # a K scale that spreads the scores
])
def test_prefill_fp8_precise(hq, hkv, cached, prompt, docs, offs, ks, vs):
    """lazyattn_prefill_fp8_precise (rotated query as bf16 hi + lo, tiles cut
    at document ends) against the oracle, including a K scale of 3 on codes up
    to 7.5, where lazyattn_prefill_fp8 misses the tolerance."""
    case = W.prefill_case(233 + hq + int(ks * 10), len(prompt), hq, hkv, 128, cached, prompt, docs, offsets=offs)
    say(f"[fp8 precise prefill] Hq{hq} Hkv{hkv} k_scale {ks} v_scale {vs} {offs}")
    got, want = _run_prefill(case, 61, ks, vs, precise=True)
    assert_parity(got, want, W.BF16, f"fp8 precise prefill k_scale {ks}")

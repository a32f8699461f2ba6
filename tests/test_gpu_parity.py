"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Small cases compare every output element; the full-size workloads (run in the
launch configuration bench.py times) compare sampled (sequence, head) rows,
which the oracle computes one by one.
"""

import numpy as np
import pytest
import torch

import oracle
import position_agnostic_kv_amd as pak
import workloads as W
from tests.gpu_helpers import (DeviceCase, assert_parity, host_pools_after_append, oracle_decode,
                               oracle_prefill, say)

pytestmark = pytest.mark.gpu


def run_decode_case(case, split_blocks=0, label=None):
    label = label or case.name
    say(f"[decode] {label} B={case.batch} Hq={case.num_q_heads} Hkv={case.num_kv_heads} "
        f"D={case.head_dim} {case.dtype} split={split_blocks}")
    W.materialize_numpy(case)
    dc = DeviceCase(case)
    dc.append()
    out = dc.decode(split_blocks=split_blocks)
    torch.cuda.synchronize()
    got = W.to_float(out, case.dtype)
    want = oracle_decode(case)
    assert_parity(got, want, case.dtype, label)
    return dc, out


# ------------------------------------------------------------------ append
@pytest.mark.parametrize("dtype,d", [(W.F32, 16), (W.BF16, 128), (W.BF16, 64), (W.F32, 128)])
def test_append_bit_exact(dtype, d):
    say(f"[append] {dtype} D={d}")
    rng = np.random.default_rng(7)
    case = W.Case("append", "decode", dtype, 4, 2, d, 1e4,
                  W.build_layout(rng, [[0], [1]], [32, 48], [20, 5]), seed=7)
    W.materialize_numpy(case)
    dc = DeviceCase(case)
    # a padding slot (-1) and a slot past the pool are skipped
    slots = case.layout.slot_mapping.copy()
    slots[3] = -1
    slots[7] = case.layout.num_blocks * 16 + 5
    dc.slots = torch.from_numpy(slots).to("cuda:0")
    case.layout.slot_mapping = slots
    dc.append()
    torch.cuda.synchronize()
    kw, vw = host_pools_after_append(case)
    kg = W.to_float(dc.k_pool, dtype)
    vg = W.to_float(dc.v_pool, dtype)
    assert np.array_equal(kg.view(np.uint32), kw.astype(np.float32).view(np.uint32))
    assert np.array_equal(vg.view(np.uint32), vw.astype(np.float32).view(np.uint32))


# -------------------------------------------------------------- decode small
@pytest.mark.parametrize("layer", range(4))
@pytest.mark.parametrize("swap", [False, True])
def test_decode_tiny_fp32(layer, swap):
    """Tiny fp32 decode step: 4 layers x 4 heads, d_h=16, two 16-token docs at 0 and 16."""
    run_decode_case(W.tiny_decode(layer=layer, swap_docs=swap), label=f"tiny L{layer} swap={swap}")


DECODE_SMALL = [
    # dtype, D, Hq, Hkv, ctx list, doc_blocks, offsets, split
    (W.BF16, 128, 8, 2, [640, 1024, 208], (2, 20), "contiguous", 4),
    (W.BF16, 128, 8, 2, [640, 1024, 208], (2, 20), "contiguous", 0),
    (W.BF16, 128, 32, 8, [512, 96], (4, 12), "random", 8),
    (W.BF16, 128, 8, 8, [400, 16, 1008], (1, 30), "contiguous", 4),
    (W.BF16, 128, 16, 2, [784, 320], (3, 9), "random", 4),
    (W.BF16, 64, 8, 4, [672, 48], (2, 10), "contiguous", 4),
    (W.BF16, 64, 16, 2, [320], (2, 10), "random", 0),
    (W.F32, 16, 4, 4, [32, 96, 400], (1, 4), "contiguous", 4),
    (W.F32, 64, 8, 2, [512, 80], (2, 8), "random", 4),
    (W.F32, 128, 8, 1, [384, 208], (2, 8), "contiguous", 4),
    (W.F32, 128, 8, 4, [256], (2, 8), "random", 0),
    # multi-query attention (one KV head; G = 16..64 query heads per KV head)
    (W.BF16, 128, 32, 1, [704, 208], (2, 12), "random", 0),
    (W.BF16, 128, 64, 1, [512, 48], (2, 12), "contiguous", 8),
    (W.BF16, 64, 16, 1, [336], (1, 9), "random", 4),
    (W.F32, 64, 16, 1, [272, 64], (2, 6), "random", 4),
]


@pytest.mark.parametrize("dtype,d,hq,hkv,ctx,docs,offs,split", DECODE_SMALL)
def test_decode_small(dtype, d, hq, hkv, ctx, docs, offs, split):
    case = W.decode_case(11 + d + hq, len(ctx), hq, hkv, d, ctx, docs, dtype=dtype, offsets=offs)
    run_decode_case(case, split, label=f"{dtype} D{d} G{hq // hkv} {offs} split{split}")


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_decode_ragged_no_append_poisoned_slots(dtype):
    """Lengths not a multiple of 16 and NaN in the unused slots of last blocks."""
    case = W.decode_case(31, 3, 8, 2, 128, [1000, 17, 333], (2, 12), dtype=dtype, new_token=False)
    W.materialize_numpy(case)
    lay = case.layout
    nan_bits = np.uint16(0x7fc0) if dtype == W.BF16 else np.float32(np.nan)
    for b in range(case.batch):
        n = int(lay.cached_lens[b])
        if n % 16:
            blk = int(lay.table[b, n // 16]) & 0xFFFF
            case.k_pool[blk, :, n % 16:, :] = nan_bits
            case.v_pool[blk, :, n % 16:, :] = nan_bits
    dc = DeviceCase(case)
    out = dc.decode(split_blocks=4)
    torch.cuda.synchronize()
    kp, vp = W.to_float(case.k_pool, dtype), W.to_float(case.v_pool, dtype)
    want = oracle.decode(W.to_float(case.q, dtype), case.q_pos, kp, vp, lay.table, case.seq_lens,
                         case.scale, case.rope_theta)
    assert_parity(W.to_float(out, dtype), want, dtype, f"ragged+poison {dtype}")


def test_decode_split_and_shuffle_invariance():
    case = W.decode_case(41, 2, 16, 4, 128, [1504, 800], (3, 20))
    W.materialize_numpy(case)
    dc = DeviceCase(case)
    dc.append()
    want = oracle_decode(case)
    outs = {}
    for split in (4, 8, 16, 64, 128):
        outs[split] = W.to_float(dc.decode(split_blocks=split), case.dtype)
        assert_parity(outs[split], want, case.dtype, f"split {split}")
    # physical placement must not matter: permute the pool and remap the table
    nb = case.layout.num_blocks
    perm = np.random.default_rng(5).permutation(nb)
    inv = np.argsort(perm)
    kp2 = dc.k_pool[torch.from_numpy(perm).cuda()].contiguous()
    vp2 = dc.v_pool[torch.from_numpy(perm).cuda()].contiguous()
    tab = case.layout.table.copy()
    ids = tab & 0xFFFF
    tab = (tab & 0xFFFF0000) | inv[ids].astype(np.uint32)
    dc2 = DeviceCase(case)
    dc2.k_pool, dc2.v_pool = kp2, vp2
    dc2.table = torch.from_numpy(tab.view(np.int32)).cuda()
    out2 = W.to_float(dc2.decode(split_blocks=8), case.dtype)
    torch.cuda.synchronize()
    assert np.array_equal(out2, outs[8]), "block shuffle changed the result"


def _one_hot_case():
    """Decode case in which query head kvh * G + 1 of each sequence has
    scale * |q|^2 ~ 600 and its exact rotation rot(q, n - off1) is stored as
    slot 5 of the first block (offset off1) and, again, as slot 5 of the first
    block of another document (offset off2).  Returns (case, picks) with picks
    (b, h, kv head, block 1, block 2, table column of block 1, of block 2)."""
    case = W.decode_case(61, 2, 8, 2, 128, [640, 512], (4, 10), new_token=False, kv_std=0.05)
    W.materialize_numpy(case)
    lay = case.layout
    g = case.num_q_heads // case.num_kv_heads
    picks = []
    for b in range(case.batch):
        nb = -(-int(case.seq_lens[b]) // 16)
        offs = (lay.table[b, :nb] >> 16).astype(np.int64)
        c1, c2 = 0, int(np.nonzero(offs != offs[0])[0][0])
        id1, id2 = int(lay.table[b, c1]) & 0xFFFF, int(lay.table[b, c2]) & 0xFFFF
        for kvh in range(case.num_kv_heads):
            h = kvh * g + 1
            qf = W.to_float(case.q[b, h], case.dtype).astype(np.float64)
            qf *= np.sqrt(600.0 / case.scale) / np.linalg.norm(qf)
            case.q[b, h] = W.f32_to_bf16_bits(qf.astype(np.float32))
            qb = W.to_float(case.q[b, h], case.dtype).astype(np.float64)
            key = oracle.rope(qb[None, :], int(case.q_pos[b]) - int(offs[c1]), case.rope_theta)[0]
            for blk in (id1, id2):
                case.k_pool[blk, kvh, 5] = W.f32_to_bf16_bits(key.astype(np.float32))
            picks.append((b, h, kvh, id1, id2, c1, c2))
    return case, picks


def test_decode_one_hot_dominant_key():
    """Under the right offsets the matched key's weight is 1 and every other
    weight underflows to 0, so the output is that token's V bit for bit.  On
    the oracle, exchanging the two blocks' offsets hands the win to the other
    copy: the case tells a right offset from a wrong one."""
    case, picks = _one_hot_case()
    lay = case.layout
    say("[one-hot] dominant key under its own offset")
    kp, vp = W.to_float(case.k_pool, case.dtype), W.to_float(case.v_pool, case.dtype)
    q = W.to_float(case.q, case.dtype)
    want = oracle.decode(q, case.q_pos, kp, vp, lay.table, case.seq_lens, case.scale, case.rope_theta)
    wrong_tab = lay.table.copy()
    for b, c1, c2 in sorted({(p[0], p[5], p[6]) for p in picks}):   # once per sequence
        w1, w2 = int(wrong_tab[b, c1]), int(wrong_tab[b, c2])
        wrong_tab[b, c1] = (w2 & 0xFFFF0000) | (w1 & 0xFFFF)
        wrong_tab[b, c2] = (w1 & 0xFFFF0000) | (w2 & 0xFFFF)
    wrong = oracle.decode(q, case.q_pos, kp, vp, wrong_tab, case.seq_lens, case.scale, case.rope_theta)
    for b, h, kvh, id1, id2, c1, c2 in picks:
        assert np.abs(want[b, h] - vp[id1, kvh, 5]).max() < 1e-9, "the matched key dominates"
        assert np.abs(wrong[b, h] - vp[id2, kvh, 5]).max() < 1e-9, "a wrong offset selects the other copy"
        assert np.abs(vp[id1, kvh, 5] - vp[id2, kvh, 5]).max() > 1e-3
    dc = DeviceCase(case)
    for split in (0, 4):
        out = dc.decode(split_blocks=split)
        torch.cuda.synchronize()
        bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
        for b, h, kvh, id1, id2, c1, c2 in picks:
            assert np.array_equal(bits[b, h], case.v_pool[id1, kvh, 5]), f"split {split}: seq {b} head {h}"


def test_decode_workspace_reuse_and_degenerate_lengths():
    case = W.decode_case(51, 4, 8, 2, 128, [800, 800, 800, 800], (2, 20), dtype=W.F32)
    W.materialize_numpy(case)
    dc = DeviceCase(case)
    dc.append()
    import position_agnostic_kv_amd as pak
    need = pak.decode_workspace_size(4, 8, 2, 128, case.layout.table.shape[1], 4)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda:0")
    a = dc.decode(split_blocks=4, workspace=ws).clone()
    b = dc.decode(split_blocks=4, workspace=ws).clone()
    assert torch.equal(a, b), "a reused workspace changed the result"
    lens = torch.tensor([1, 0, -3, 801], dtype=torch.int32, device="cuda:0")
    out = dc.decode(split_blocks=4, workspace=ws, seq_lens=lens)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    vp = W.to_float(case.v_pool, case.dtype)
    first = int(case.layout.table[0, 0]) & 0xFFFF
    for h in range(8):
        assert np.array_equal(o[0, h], vp[first, h // 4, 0]), "single token must return its value exactly"
    assert np.all(o[1] == 0), "empty sequence must give zeros"
    assert np.all(np.isnan(o[2])), "negative length must give NaN"
    # a table entry pointing past the pool poisons only its own sequence
    tab = dc.table.clone()
    tab[3, 2] = (tab[3, 2] & ~0xFFFF) | 0xFFF0
    out = pak.lazyattn_decode(dc.q, dc.q_pos, dc.k_pool, dc.v_pool, tab, dc.seq_lens,
                              scale=case.scale, rope_theta=case.rope_theta, split_blocks=4, workspace=ws)
    o2 = out.cpu().numpy()
    assert np.all(np.isnan(o2[3])) and np.all(np.isfinite(o2[:3]))
    c = dc.decode(split_blocks=4, workspace=ws)
    assert torch.equal(c, a), "a poisoned call changed a later result"


# ------------------------------------------------------------- prefill small
PREFILL_SMALL = [
    # D, Hq, Hkv, cached, prompt, docs, offsets
    (128, 8, 2, [224, 640], [300, 129], (2, 20), "contiguous"),
    (128, 32, 8, [512], [256], (4, 12), "contiguous"),
    (128, 4, 4, [0, 96], [77, 200], (1, 4), "random"),
    (128, 16, 2, [1056], [64], (3, 40), "random"),
    (64, 8, 4, [320, 48], [150, 31], (2, 10), "contiguous"),
    (64, 8, 1, [160], [260], (2, 5), "random"),
    (128, 32, 1, [416, 96], [200, 70], (2, 9), "random"),   # multi-query attention
]


@pytest.mark.parametrize("d,hq,hkv,cached,prompt,docs,offs", PREFILL_SMALL)
def test_prefill_small(d, hq, hkv, cached, prompt, docs, offs):
    case = W.prefill_case(61 + d + hq, len(prompt), hq, hkv, d, cached, prompt, docs, offsets=offs)
    say(f"[prefill] D{d} Hq{hq} Hkv{hkv} cached={cached} prompt={prompt} {offs}")
    W.materialize_numpy(case)
    dc = DeviceCase(case)
    dc.append()
    out = dc.prefill()
    torch.cuda.synchronize()
    want = oracle_prefill(case)
    assert_parity(W.to_float(out, case.dtype), want, case.dtype, f"prefill D{d} G{hq // hkv} {offs}")


# Scores with a large common part per query row (up to ~2^300 before
# normalisation): the kernels must leave exp's range safely -- overflow on the
# first tile, underflow on the first tile, and a jump mid-row when the prompt's
# keys arrive -- and still agree with the oracle.
SHIFT_CASES = [
    # kind, D, k_x of cached keys, k_x of appended keys
    ("prefill", 128, 4.0, 4.0),
    ("prefill", 128, 0.0, 4.0),
    ("prefill", 128, -4.0, 4.0),
    ("prefill", 64, 4.0, -4.0),
    ("decode", 128, -4.0, 4.0),
    ("decode", 128, 4.0, -4.0),
]


@pytest.mark.parametrize("kind,d,kc,kn", SHIFT_CASES)
def test_large_score_shift(kind, d, kc, kn):
    if kind == "prefill":
        case = W.prefill_case(81 + d, 2, 8, 2, d, [512, 240], [300, 129], (2, 10), theta=1e30)
    else:
        case = W.decode_case(82 + d, 6, 8, 2, d, [512, 800, 16, 1024, 304, 96], (2, 10), theta=1e30)
    W.materialize_numpy(case)
    W.add_score_shift(case, 600.0, kc, kn, seed=d)
    qx = W.to_float(case.q, case.dtype)[..., d // 2 - 1]
    span = float(np.abs(qx).max()) * max(abs(kc), abs(kn)) * case.scale / np.log(2.0)
    assert span > 200.0  # log2 units: far past fp32's exp range
    say(f"[shift] {kind} D{d} k_cached={kc} k_new={kn} span 2^{span:.0f}")
    dc = DeviceCase(case)
    dc.append()
    want = oracle_prefill(case) if kind == "prefill" else oracle_decode(case)
    for split in ([0] if kind == "prefill" else [0, 4]):
        out = dc.prefill() if kind == "prefill" else dc.decode(split_blocks=split)
        torch.cuda.synchronize()
        assert_parity(W.to_float(out, case.dtype), want, case.dtype, f"shift {kind} D{d} split {split}")


def test_incremental_decode_matches_prefill_rows():
    """Decoding row t after the prompt is appended equals prefill row t."""
    case = W.prefill_case(71, 1, 8, 2, 128, [400 - 400 % 16], [150], (2, 10))
    W.materialize_numpy(case)
    dc = DeviceCase(case)
    dc.append()
    pre = W.to_float(dc.prefill(), case.dtype)
    p = 150
    c0 = int(case.layout.cached_lens[0])
    rows = [0, 1, 63, 64, 127, 128, 149]
    qd = dc.q[rows].contiguous()
    tab = dc.table.repeat(len(rows), 1).contiguous()
    lens = torch.tensor([c0 + r + 1 for r in rows], dtype=torch.int32, device="cuda:0")
    qpos = torch.tensor([int(case.layout.tail_pos[0]) + r for r in rows], dtype=torch.int32, device="cuda:0")
    import position_agnostic_kv_amd as pak
    dec = pak.lazyattn_decode(qd, qpos, dc.k_pool, dc.v_pool, tab, lens, scale=case.scale,
                              rope_theta=case.rope_theta)
    dec = W.to_float(dec, case.dtype)
    assert_parity(dec, pre[rows], W.BF16, "decode rows vs prefill rows")
    assert p == case.max_q_len


# ------------------------------------------------------- full-size workloads
def _gather(dc, case, seqs, table=None):
    """Oracle pools for the sampled sequences: host copies of the blocks they
    use, taken from the generated pools BEFORE the library's append, ids
    remapped, then the step's new rows that land there written by the
    oracle's own append.  `table`: the table rows the kernel reads (the
    layout's by default).  Returns (k, v, remapped table rows, the blocks'
    fill counts under the new ids or None)."""
    lay = case.layout
    src = lay.table if table is None else table
    ids = []
    for b in seqs:
        nb = -(-int(case.seq_lens[b]) // 16)
        ids.extend((lay.table[b, :nb] & 0xFFFF).tolist())
    uniq = np.unique(np.array(ids, dtype=np.int64))
    remap = {int(x): i for i, x in enumerate(uniq)}
    sel = torch.from_numpy(uniq).to("cuda:0")
    kp = W.to_float(dc.k_pool.index_select(0, sel), case.dtype)
    vp = W.to_float(dc.v_pool.index_select(0, sel), case.dtype)
    rows, slots = [], []
    for t, sl in enumerate(lay.slot_mapping.tolist()):
        if sl >= 0 and sl // 16 in remap:
            rows.append(t)
            slots.append(remap[sl // 16] * 16 + sl % 16)
    if rows:
        r = torch.tensor(rows, device="cuda:0")
        kp, vp = oracle.append(kp, vp, W.to_float(dc.k_new.index_select(0, r), case.dtype),
                               W.to_float(dc.v_new.index_select(0, r), case.dtype), np.array(slots))
    tab = np.zeros((len(seqs), lay.table.shape[1]), dtype=np.uint32)
    for i, b in enumerate(seqs):
        nb = -(-int(case.seq_lens[b]) // 16)
        for j in range(nb):
            w = int(src[b, j])
            tab[i, j] = (w & 0xFFFF0000) | remap[w & 0xFFFF]
    fill = None if case.block_fill is None else np.asarray(case.block_fill)[uniq]
    return kp, vp, tab, fill


@pytest.mark.parametrize("name", ["llama8b_decode", "llama70b_decode", "zipf_reuse_decode", "llama8b_decode_ragged"])
def test_full_size_decode_sampled(name):
    case = W.make(name)
    say(f"[full decode] {name} B={case.batch} NB={case.layout.num_blocks}")
    W.materialize_torch(case, "cuda:0")
    dc = DeviceCase(case)
    rng = np.random.default_rng(3)
    seqs = sorted(rng.choice(case.batch, size=min(4, case.batch), replace=False).tolist())
    kp, vp, tab, fill = _gather(dc, case, seqs)   # generated pools + the oracle's append
    dc.append()
    out = dc.decode()  # automatic split, as bench.py runs it
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    q = W.to_float(case.q, case.dtype)
    got = W.to_float(out, case.dtype)
    g = case.num_q_heads // case.num_kv_heads
    rows_got, rows_want = [], []
    for i, b in enumerate(seqs):
        for h in rng.choice(case.num_q_heads, size=3, replace=False).tolist():
            want = oracle.decode_one(q[b, h], int(case.q_pos[b]), kp, vp, tab[i], int(case.seq_lens[b]),
                                     h // g, case.scale, case.rope_theta, block_fill=fill)
            rows_got.append(got[b, h])
            rows_want.append(want)
    assert_parity(np.stack(rows_got), np.stack(rows_want), case.dtype, f"{name} sampled")


def test_full_size_append_bit_exact_sampled():
    case = W.make("llama8b_prefill")
    W.materialize_torch(case, "cuda:0")
    dc = DeviceCase(case)
    dc.append()
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    for t in rng.choice(len(case.layout.slot_mapping), size=64, replace=False).tolist():
        s = int(case.layout.slot_mapping[t])
        assert torch.equal(dc.k_pool[s // 16, :, s % 16], dc.k_new[t])
        assert torch.equal(dc.v_pool[s // 16, :, s % 16], dc.v_new[t])


@pytest.mark.parametrize("name", ["llama8b_prefill", "llama8b_prefill_ragged"])
def test_full_size_prefill_sampled(name):
    case = W.make(name)
    say(f"[full prefill] {name} B={case.batch} prompt={case.max_q_len}")
    W.materialize_torch(case, "cuda:0")
    dc = DeviceCase(case)
    rng = np.random.default_rng(4)
    seqs = [0, 3]
    kp, vp, tab, fill = _gather(dc, case, seqs)   # generated pools + the oracle's append
    dc.append()
    out = dc.prefill()
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    q = W.to_float(case.q, case.dtype)
    got = W.to_float(out, case.dtype)
    g = case.num_q_heads // case.num_kv_heads
    rows = np.array([0, 1, 2, 127, 128, 129, 1023, 1024, 2046, 2047])
    gots, wants = [], []
    for i, b in enumerate(seqs):
        q0 = int(case.cu_q_lens[b])
        for h in rng.choice(case.num_q_heads, size=3, replace=False).tolist():
            want = oracle.prefill_rows(q[q0 + rows, h], rows, case.max_q_len, int(case.layout.tail_pos[b]),
                                       kp, vp, tab[i], int(case.seq_lens[b]), h // g, case.scale,
                                       case.rope_theta, block_fill=fill)
            gots.append(got[q0 + rows, h])
            wants.append(want)
    assert_parity(np.concatenate(gots), np.concatenate(wants), case.dtype, f"{name} sampled")


def test_full_size_decode_alibi_sampled():
    """The 8B decode inputs read with ALiBi biases (block-frame table words),
    as bench.py --shapes times them, on 4 sampled sequences (all heads)."""
    case = W.make("llama8b_decode")
    say(f"[full decode alibi] B={case.batch}")
    W.materialize_torch(case, "cuda:0")
    dc = DeviceCase(case)
    frame = W.block_frame_table(case.layout)
    rng = np.random.default_rng(5)
    seqs = sorted(rng.choice(case.batch, size=4, replace=False).tolist())
    kp, vp, tab, fill = _gather(dc, case, seqs, table=frame)
    dc.append()
    slopes = oracle.alibi_slopes(case.num_q_heads)
    out = pak.lazyattn_decode_alibi(dc.q, dc.q_pos, dc.k_pool, dc.v_pool,
                                    torch.from_numpy(frame.view(np.int32)).to("cuda:0"), dc.seq_lens,
                                    torch.from_numpy(slopes.astype(np.float32)).to("cuda:0"))
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    q = W.to_float(case.q, case.dtype)[seqs]
    want = oracle.decode_alibi(q, case.q_pos[seqs], kp, vp, tab, case.seq_lens[seqs], case.scale,
                               slopes.astype(np.float32), block_fill=fill)
    assert_parity(W.to_float(out, case.dtype)[seqs], want, case.dtype, "llama8b_decode alibi sampled")

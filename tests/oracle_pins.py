"""Checks that pin the CPU oracle to facts other than itself.

Each ``check_*`` takes the oracle module and raises AssertionError on a
mismatch.  ``test_oracle_pins.py`` runs them against the real oracle;
``test_oracle_mutations.py`` runs them against copies with planted mistakes
and requires that every mistake is caught by at least one check.

What each check pins against:
  * complex-number rotation with hand-derived frequencies (RoPE sign,
    pairing, frequency law),
  * the relative-offset identity, composition and orthogonality of rotations,
  * scipy's softmax and a hand-worked closed form (running softmax),
  * torch's CPU scaled_dot_product_attention (scale, softmax, GQA mapping),
  * pure-Python brute force with its own table decoding (paging, offsets,
    causal visibility),
  * degenerate cases with exact answers, and the page's cache-size values.
"""

import cmath
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

BLOCK = 16


def _close(a, b, tol, what):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


# ------------------------------------------------------------------ helpers
def _word(block_id, offset):
    return block_id + 65536 * offset


def _pool_case(rng, n_blocks, hkv, d, seqs, scale_v=1.0):
    """Random pools plus per-sequence (words, length) with random offsets.

    seqs: list of lists of (n_tokens_in_block, offset) per block.
    """
    k_pool = rng.standard_normal((n_blocks, hkv, BLOCK, d))
    v_pool = rng.standard_normal((n_blocks, hkv, BLOCK, d)) * scale_v
    ids = rng.permutation(n_blocks)
    width = max(len(s) for s in seqs)
    table = np.zeros((len(seqs), width), dtype=np.uint64)
    lens = []
    used = 0
    for b, blocks in enumerate(seqs):
        n = 0
        for i, (cnt, off) in enumerate(blocks):
            table[b, i] = _word(int(ids[used]), off)
            used += 1
            n += cnt
        lens.append(n)
    return k_pool, v_pool, table, np.array(lens)


def _brute_rotate(vec, pos, theta_base):
    """Rotate by complex multiplication: z_i = x_i + i x_{i+D/2} times e^{i pos w_i}."""
    d = len(vec)
    out = [0.0] * d
    for i in range(d // 2):
        w = math.exp(-(2.0 * i / d) * math.log(theta_base))
        z = complex(vec[i], vec[i + d // 2]) * cmath.exp(1j * pos * w)
        out[i], out[i + d // 2] = z.real, z.imag
    return out


def _brute_attention(q_vec, q_pos, k_pool, v_pool, words, n_keys, kv_head, scale, theta):
    """Triple-loop attention of one query over the first n_keys logical tokens."""
    qr = _brute_rotate(list(q_vec), q_pos, theta)
    scores, vals = [], []
    for j in range(n_keys):
        w = int(words[j // BLOCK])
        off, blk = divmod(w, 65536)
        kr = _brute_rotate(list(k_pool[blk][kv_head][j % BLOCK]), off, theta)
        scores.append(scale * sum(a * b for a, b in zip(qr, kr)))
        vals.append(list(v_pool[blk][kv_head][j % BLOCK]))
    if not scores:
        return [0.0] * len(q_vec)
    m = max(scores)
    e = [math.exp(s - m) for s in scores]
    tot = sum(e)
    return [sum(e[j] * vals[j][c] for j in range(n_keys)) / tot for c in range(len(q_vec))]


def _brute_attention_fill(q_vec, q_pos, k_pool, v_pool, words, n_slots, kv_head, scale, theta, fill,
                          last_slot=None):
    """Triple-loop attention over the first n_slots table slots, skipping
    slots past their block's fill count; with last_slot, only slots <= it."""
    qr = _brute_rotate(list(q_vec), q_pos, theta)
    scores, vals = [], []
    for j in range(n_slots):
        off, blk = divmod(int(words[j // BLOCK]), 65536)
        if j % BLOCK >= int(fill[blk]) or (last_slot is not None and j > last_slot):
            continue
        kr = _brute_rotate(list(k_pool[blk][kv_head][j % BLOCK]), off, theta)
        scores.append(scale * sum(a * b for a, b in zip(qr, kr)))
        vals.append(list(v_pool[blk][kv_head][j % BLOCK]))
    m = max(scores)
    e = [math.exp(x - m) for x in scores]
    tot = sum(e)
    return [sum(e[i] * vals[i][c] for i in range(len(e))) / tot for c in range(len(q_vec))]


# ------------------------------------------------------------------- checks
def check_rope_frequency_closed_forms(O):
    # theta = 1e4, D = 16: theta^(-2i/16) = 10^(-i/2)
    _close(O.rope_frequencies(16, 1.0e4), [10.0 ** (-i / 2.0) for i in range(8)], 1e-15, "freq 1e4/16")
    # theta = 5e5, D = 128: w_32 = 5e5^(-1/2), w_0 = 1, consecutive ratio 5e5^(-1/64)
    w = O.rope_frequencies(128, 5.0e5)
    _close(w[0], 1.0, 0, "w0")
    _close(w[32], 1.0 / math.sqrt(5.0e5), 1e-17, "w32")
    _close(w[1:] / w[:-1], np.full(63, 5.0e5 ** (-1.0 / 64)), 1e-14, "ratio")


def check_rope_matches_complex_rotation(O):
    rng = np.random.default_rng(11)
    for d, theta in ((16, 1.0e4), (64, 1.0e4), (128, 5.0e5)):
        x = rng.standard_normal(d)
        for pos in (0, 1, 7, 1000, 32767, 65535):
            _close(O.rope(x, pos, theta), _brute_rotate(list(x), pos, theta), 1e-9, f"rope d={d} pos={pos}")


def check_rope_relative_identity(O):
    """rot(q, n) . rot(k, m) == rot(q, n - m) . k  (RoPE depends on n - m only)."""
    rng = np.random.default_rng(12)
    for d in (16, 128):
        for n, m in ((5, 3), (8192, 77), (32768, 12345), (100, 60000)):
            q, k = rng.standard_normal(d), rng.standard_normal(d)
            lhs = O.rope(q, n, 5.0e5) @ O.rope(k, m, 5.0e5)
            rhs = O.rope(q, n - m, 5.0e5) @ k
            _close(lhs, rhs, 1e-9, f"relative identity n={n} m={m}")


def check_rope_composition_and_norm(O):
    rng = np.random.default_rng(13)
    x = rng.standard_normal(128)
    _close(O.rope(x, 0, 1.0e4), x, 0, "rot(x, 0) == x")
    _close(O.rope(O.rope(x, 300, 1.0e4), 4000, 1.0e4), O.rope(x, 4300, 1.0e4), 1e-9, "composition")
    _close(np.linalg.norm(O.rope(x, 12345, 1.0e4)), np.linalg.norm(x), 1e-12, "norm")


def check_softmax(O):
    import scipy.special
    rng = np.random.default_rng(14)
    s = rng.standard_normal((5, 37)) * 10
    p = O.softmax(s)
    _close(p, scipy.special.softmax(s, axis=-1), 1e-15, "softmax vs scipy")
    _close(p.sum(axis=-1), np.ones(5), 1e-14, "rows sum to 1")
    _close(O.softmax(np.array([1.0, 0.0])), [math.e / (1 + math.e), 1 / (1 + math.e)], 1e-16, "2-way")


def check_blockwise_softmax(O):
    import scipy.special
    with open(os.path.join(GOLDEN, "tiled_softmax_example.json")) as f:
        g = json.load(f)
    e = math.e
    want = [(e + 3 + 5 * e * e) / (e + 1 + e * e), (2 * e + 4 - e * e) / (e + 1 + e * e)]
    for tile in (1, 2, 4):
        _close(O.blockwise_softmax_dot(g["q"], g["K"], g["V"], tile), want, 1e-14, f"worked example tile={tile}")
    rng = np.random.default_rng(15)
    q, k, v = rng.standard_normal(16), rng.standard_normal((53, 16)), rng.standard_normal((53, 16))
    one_shot = scipy.special.softmax(k @ q) @ v
    for tile in (1, 3, 4, 16, 53, 60):
        _close(O.blockwise_softmax_dot(q, k, v, tile), one_shot, 1e-13, f"tiled == one-shot tile={tile}")


def check_decode_vs_torch_sdpa(O):
    """One document at offset 0 and a query at position 0: no rotation at all,
    so the result is plain GQA attention, which torch computes independently."""
    import torch
    rng = np.random.default_rng(16)
    hq, hkv, d, n = 8, 2, 32, 45
    blocks = [(16, 0), (16, 0), (13, 0)]
    k_pool, v_pool, table, lens = _pool_case(rng, 5, hkv, d, [blocks])
    q = rng.standard_normal((1, hq, d))
    scale = 1 / math.sqrt(d)
    out = O.decode(q, np.array([0]), k_pool, v_pool, table, lens, scale, 1.0e4)
    # gather K, V in logical order with this file's own table decoding
    ks = np.stack([k_pool[int(table[0, j // 16]) % 65536, :, j % 16] for j in range(n)], axis=1)
    vs = np.stack([v_pool[int(table[0, j // 16]) % 65536, :, j % 16] for j in range(n)], axis=1)
    g = hq // hkv
    kt = torch.from_numpy(ks).repeat_interleave(g, dim=0)[None]
    vt = torch.from_numpy(vs).repeat_interleave(g, dim=0)[None]
    qt = torch.from_numpy(q[0])[None, :, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)[0, :, 0].numpy()
    _close(out[0], ref, 1e-12, "decode vs torch sdpa")


def check_decode_bruteforce(O):
    rng = np.random.default_rng(17)
    hq, hkv, d = 4, 2, 8
    seqs = [[(16, 40), (16, 40), (16, 1000), (5, 7)],
            [(16, 3), (9, 65000)],
            [(1, 12)]]
    k_pool, v_pool, table, lens = _pool_case(rng, 7, hkv, d, seqs)
    q = rng.standard_normal((3, hq, d))
    qpos = np.array([53, 9, 30000])
    scale = 0.37
    out = O.decode(q, qpos, k_pool, v_pool, table, lens, scale, 1.0e4)
    for b in range(3):
        for h in range(hq):
            ref = _brute_attention(q[b, h], qpos[b], k_pool, v_pool, table[b], lens[b], h // 2, scale, 1.0e4)
            _close(out[b, h], ref, 1e-11, f"decode brute b={b} h={h}")


def check_decode_one_matches_decode(O):
    rng = np.random.default_rng(18)
    k_pool, v_pool, table, lens = _pool_case(rng, 4, 2, 16, [[(16, 5), (16, 900), (3, 2)]])
    q = rng.standard_normal((1, 4, 16))
    full = O.decode(q, np.array([77]), k_pool, v_pool, table, lens, 0.25, 1.0e4)
    for h in range(4):
        one = O.decode_one(q[0, h], 77, k_pool, v_pool, table[0], lens[0], h // 2, 0.25, 1.0e4)
        _close(one, full[0, h], 1e-14, "decode_one")


def check_shift_invariance(O):
    """Adding the same shift to the query position and every offset changes nothing."""
    rng = np.random.default_rng(19)
    seqs = [[(16, 100), (16, 100), (16, 2000), (11, 50)]]
    k_pool, v_pool, table, lens = _pool_case(rng, 4, 1, 32, seqs)
    q = rng.standard_normal((1, 2, 32))
    a = O.decode(q, np.array([3000]), k_pool, v_pool, table, lens, 0.2, 1.0e4)
    shifted = table + np.uint64(65536 * 1234)
    b = O.decode(q, np.array([3000 + 1234]), k_pool, v_pool, shifted, lens, 0.2, 1.0e4)
    _close(a, b, 1e-10, "shift invariance")


def check_prefill_bruteforce(O):
    rng = np.random.default_rng(20)
    hq, hkv, d = 4, 2, 8
    # two cached documents, then a 21-token prompt appended in 2 blocks at offset 600
    seqs = [[(16, 0), (16, 300), (16, 600), (5, 600)],
            [(7, 40)]]
    k_pool, v_pool, table, lens = _pool_case(rng, 6, hkv, d, seqs)
    q_lens = [21, 7]
    qps = [600, 40]
    cu = np.array([0, 21, 28])
    q = rng.standard_normal((28, hq, d))
    out = O.prefill(q, cu, np.array(qps), k_pool, v_pool, table, lens, 0.4, 1.0e4)
    for b in range(2):
        for r in range(q_lens[b]):
            t = lens[b] - q_lens[b] + r
            for h in range(hq):
                ref = _brute_attention(q[cu[b] + r, h], qps[b] + r, k_pool, v_pool, table[b], t + 1,
                                       h // 2, 0.4, 1.0e4)
                _close(out[cu[b] + r, h], ref, 1e-11, f"prefill brute b={b} r={r} h={h}")


def check_decode_fill_bruteforce(O):
    """Blocks partly filled in the middle of a sequence (documents whose
    length is not a multiple of 16): the unused slots are skipped."""
    rng = np.random.default_rng(27)
    hq, hkv, d = 4, 2, 8
    seqs = [[(16, 0), (16, 0), (16, 37), (16, 900)], [(16, 5), (16, 400)]]
    k_pool, v_pool, table, lens = _pool_case(rng, 8, hkv, d, seqs)
    fill = rng.integers(1, 17, size=8)
    fill[int(table[1, 1]) % 65536] = 16
    q = rng.standard_normal((2, hq, d))
    qpos = np.array([2000, 430])
    out = O.decode(q, qpos, k_pool, v_pool, table, lens, 0.3, 1.0e4, block_fill=fill)
    for b in range(2):
        for h in range(hq):
            ref = _brute_attention_fill(q[b, h], qpos[b], k_pool, v_pool, table[b], lens[b], h // 2, 0.3,
                                        1.0e4, fill)
            _close(out[b, h], ref, 1e-11, f"decode fill brute b={b} h={h}")


def check_prefill_fill_bruteforce(O):
    """Prefill after partly filled document blocks: a prompt row sees the
    document tokens actually stored and the prompt up to itself."""
    rng = np.random.default_rng(28)
    hq, hkv, d = 2, 1, 8
    seqs = [[(16, 0), (16, 0), (16, 21), (16, 55), (3, 55)]]   # docs of 25 and 34 tokens, then a 19-token prompt
    k_pool, v_pool, table, lens = _pool_case(rng, 6, hkv, d, seqs)
    fill = np.full(6, 16)
    fill[int(table[0, 1]) % 65536] = 9
    fill[int(table[0, 2]) % 65536] = 13
    p = 19
    q = rng.standard_normal((p, hq, d))
    out = O.prefill(q, np.array([0, p]), np.array([55]), k_pool, v_pool, table, lens, 0.4, 1.0e4, block_fill=fill)
    for r in range(p):
        t = lens[0] - p + r
        for h in range(hq):
            ref = _brute_attention_fill(q[r, h], 55 + r, k_pool, v_pool, table[0], lens[0], 0, 0.4, 1.0e4, fill,
                                        last_slot=t)
            _close(out[r, h], ref, 1e-11, f"prefill fill brute r={r} h={h}")


def check_incremental_equals_full(O):
    """Decoding token t after appending it equals row t of the causal prefill."""
    rng = np.random.default_rng(21)
    seqs = [[(16, 0), (16, 0), (16, 32), (16, 32), (16, 64), (4, 64)]]
    k_pool, v_pool, table, lens = _pool_case(rng, 6, 2, 16, seqs)
    p = 36  # the prompt is the last 36 logical tokens of the table (blocks 3..5)
    q = rng.standard_normal((p, 4, 16))
    pre = O.prefill(q, np.array([0, p]), np.array([1000]), k_pool, v_pool, table, lens, 0.25, 1.0e4)
    for r in range(p):
        t = int(lens[0]) - p + r
        dec = O.decode(q[r][None], np.array([1000 + r]), k_pool, v_pool, table, np.array([t + 1]), 0.25, 1.0e4)
        _close(dec[0], pre[r], 1e-12, f"incremental row {r}")


def check_degenerate_cases(O):
    rng = np.random.default_rng(22)
    seqs = [[(16, 10), (16, 500), (7, 3)]]
    k_pool, v_pool, table, lens = _pool_case(rng, 3, 1, 16, seqs)
    q = rng.standard_normal((1, 1, 16))
    # constant values -> output equals that value
    v_const = np.ones_like(v_pool) * 0.75
    _close(O.decode(q, np.array([9]), k_pool, v_const, table, lens, 0.3, 1.0e4)[0, 0], np.full(16, 0.75),
           1e-14, "constant V")
    # zero query -> uniform weights -> mean of the visible values
    out = O.decode(np.zeros_like(q), np.array([9]), k_pool, v_pool, table, lens, 0.3, 1.0e4)
    vis = np.stack([v_pool[int(table[0, j // 16]) % 65536, 0, j % 16] for j in range(lens[0])])
    _close(out[0, 0], vis.mean(axis=0), 1e-13, "uniform weights")
    # a single visible token -> its value exactly
    one = O.decode(q, np.array([9]), k_pool, v_pool, table, np.array([1]), 0.3, 1.0e4)
    _close(one[0, 0], v_pool[int(table[0, 0]) % 65536, 0, 0], 0, "single token")
    # empty sequence -> zeros
    _close(O.decode(q, np.array([9]), k_pool, v_pool, table, np.array([0]), 0.3, 1.0e4), np.zeros((1, 1, 16)),
           0, "empty sequence")


def check_append(O):
    rng = np.random.default_rng(23)
    k_pool = rng.standard_normal((4, 2, 16, 8)).astype(np.float32)
    v_pool = rng.standard_normal((4, 2, 16, 8)).astype(np.float32)
    k_before, v_before = k_pool.copy(), v_pool.copy()
    k_new = rng.standard_normal((5, 2, 8)).astype(np.float32)
    v_new = rng.standard_normal((5, 2, 8)).astype(np.float32)
    slots = np.array([0, 17, -1, 63, 64 + 7])  # -1: padding; 71: past the 4-block pool
    k2, v2 = O.append(k_pool, v_pool, k_new, v_new, slots)
    for t, s in enumerate(slots):
        if 0 <= s < 64:
            assert np.array_equal(k2[s // 16, :, s % 16], k_new[t]), "append K"
            assert np.array_equal(v2[s // 16, :, s % 16], v_new[t]), "append V"
    touched = np.zeros((4, 16), dtype=bool)
    for s in slots:
        if 0 <= s < 64:
            touched[s // 16, s % 16] = True
    for blk in range(4):
        for sl in range(16):
            if not touched[blk, sl]:
                assert np.array_equal(k2[blk, :, sl], k_pool[blk, :, sl]), "untouched slot changed"
    assert np.array_equal(k_pool, k_before) and np.array_equal(v_pool, v_before), "input pool changed"


def check_cache_bytes_golden(O):
    with open(os.path.join(GOLDEN, "cache_bytes.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        got = O.cache_bytes(c["L"], c["H"], c["d_h"], c["S"], c["B"], c["s"])
        assert got == c["bytes"], f"{c['name']}: {got} != {c['bytes']}"


def check_rotation_overhead_golden(O):
    """The pages' printed overhead of one relative rotation per tile, and its
    independence of the key tile's size and the head dimension."""
    with open(os.path.join(GOLDEN, "rotation_overhead.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        pct = 100.0 * O.relative_rotation_overhead(c["M"], c["N"], c["D"])
        assert round(pct, c["printed_digits"]) == c["percent"], f"{c['name']}: {pct}"
        for n, d in ((16, 64), (256, 128), (64, 16)):
            assert O.relative_rotation_overhead(c["M"], n, d) == O.relative_rotation_overhead(c["M"], c["N"], c["D"])


ALL_CHECKS = [v for k, v in sorted(globals().items()) if k.startswith("check_")]

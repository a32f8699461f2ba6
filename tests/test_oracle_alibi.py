"""Pins of the ALiBi oracle (oracle/alibi_oracle.py) against things other than
itself: torch's CPU scaled_dot_product_attention when every slope is zero, a
pure-Python loop on tiny inputs, invariance to a common shift of all
positions (the bias is relative), and the steep-slope limit, which must pick
the value of the key with the largest position (the sign of the bias, and
positions read as block offset + slot, not as logical index)."""

import math

import numpy as np
import pytest
import torch

import oracle

BT = oracle.BLOCK_TOKENS


def _case(rng, nblocks, hq=4, hkv=2, d=16, offsets=None, pool=None):
    pool = pool or nblocks + 3
    k = rng.standard_normal((pool, hkv, BT, d))
    v = rng.standard_normal((pool, hkv, BT, d))
    ids = rng.permutation(pool)[:nblocks]
    offs = offsets if offsets is not None else [int(x) for x in rng.integers(0, 4000, size=nblocks)]
    row = (np.asarray(ids, np.uint64) | (np.asarray(offs, np.uint64) << 16)).astype(np.uint32)
    return k, v, row


def test_zero_slopes_equal_sdpa():
    rng = np.random.default_rng(1)
    k, v, row = _case(rng, 5)
    n = 5 * BT - 7
    q = rng.standard_normal((1, 4, 16))
    got = oracle.decode_alibi(q, [9000], k, v, row[None, :], [n], 0.25, np.zeros(4))
    kk, vv = oracle.alibi_oracle.gather_sequence(k, v, row, n, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q[0, :2])[None, :, None, :], torch.from_numpy(kk)[None, None].expand(1, 2, n, 16),
        torch.from_numpy(vv)[None, None].expand(1, 2, n, 16), scale=0.25)
    np.testing.assert_allclose(got[0, :2], ref[0, :, 0].numpy(), atol=1e-12)


def test_pure_python_loop():
    rng = np.random.default_rng(2)
    k, v, row = _case(rng, 2, hq=2, hkv=1, d=4)
    n, qpos, scale = 2 * BT - 3, 77, 0.5
    slopes = [0.3, 0.05]
    q = rng.standard_normal((1, 2, 4))
    got = oracle.decode_alibi(q, [qpos], k, v, row[None, :], [n], scale, slopes)
    for h in range(2):
        sc = []
        for j in range(n):
            w = int(row[j // BT])
            blk, off = w & 0xFFFF, w >> 16
            dot = sum(float(q[0, h, e]) * float(k[blk, 0, j % BT, e]) for e in range(4))
            sc.append(scale * dot + slopes[h] * ((off + j % BT) - qpos))
        m = max(sc)
        ex = [math.exp(s - m) for s in sc]
        tot = sum(ex)
        for e in range(4):
            want = sum(ex[j] * float(v[int(row[j // BT]) & 0xFFFF, 0, j % BT, e]) for j in range(n)) / tot
            assert abs(got[0, h, e] - want) < 1e-12


def test_shift_invariance():
    rng = np.random.default_rng(3)
    k, v, row = _case(rng, 4, offsets=[10, 400, 26, 900])
    q = rng.standard_normal((1, 4, 16))
    s = oracle.alibi_slopes(4)
    a = oracle.decode_alibi(q, [1000], k, v, row[None, :], [60], 0.25, s)
    shifted = (row & 0xFFFF) | (((row >> 16) + 777) << 16)
    b = oracle.decode_alibi(q, [1777], k, v, shifted[None, :].astype(np.uint32), [60], 0.25, s)
    np.testing.assert_allclose(a, b, atol=1e-12)
    # (a shift of the query alone adds one constant to its row: no change
    # either); moving one block relative to the others does change it
    moved = row.copy()
    moved[1] = (row[1] & 0xFFFF) | (((row[1] >> 16) + 300) << 16)
    c = oracle.decode_alibi(q, [1000], k, v, moved[None, :], [60], 0.25, s)
    assert np.abs(a - c).max() > 1e-3


def test_steep_slope_selects_the_latest_position():
    rng = np.random.default_rng(4)
    # logical order: block 0 at positions 100..115, block 1 at 50..65; the
    # latest position is logical token 15 (block 0, slot 15)
    k, v, row = _case(rng, 2, hq=2, hkv=1, d=8, offsets=[100, 50])
    q = rng.standard_normal((1, 2, 8)) * 0.1
    out = oracle.decode_alibi(q, [120], k, v, row[None, :], [2 * BT], 0.1, [60.0, 60.0])
    latest = v[int(row[0]) & 0xFFFF, 0, 15]
    np.testing.assert_allclose(out[0, 0], latest, atol=1e-12)
    np.testing.assert_allclose(out[0, 1], latest, atol=1e-12)


def test_prefill_rows_equal_truncated_decode():
    rng = np.random.default_rng(5)
    k, v, row = _case(rng, 4, hq=4, hkv=2, d=16, offsets=[0, 16, 32, 48])
    p, kv = 20, 60
    q = rng.standard_normal((p, 4, 16))
    s = oracle.alibi_slopes(4)
    pre = oracle.prefill_alibi(q, [0, p], [40], k, v, row[None, :], [kv], 0.25, s)
    for r in range(p):
        t = kv - p + r
        dec = oracle.decode_alibi(q[r][None], [40 + r], k, v, row[None, :], [t + 1], 0.25, s)
        np.testing.assert_allclose(pre[r], dec[0], atol=1e-12)


def test_slopes_formula():
    s = oracle.alibi_slopes(8)
    assert s[0] == 0.5 and s[-1] == 2.0 ** -8
    assert np.allclose(s[1:] / s[:-1], 0.5)

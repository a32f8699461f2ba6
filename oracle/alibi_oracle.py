"""Plain float64 reference of the ALiBi variant of the paged, position-free
KV attention (test infrastructure; see oracle/__init__.py).

The pages state that deferring position information to the attention kernel
also works for ALiBi ([LA] "Principais Contribuições" 4, "Generalizabilidade")
but do not define ALiBi.  Readings taken here:

* ALiBi (linear biases): the score of query position n against a key at
  position p is  scale * q . k + slope_h * (p - n)  for query head h; no
  rotation anywhere (queries, keys and values carry no position).  Slopes are
  an input, one per query head.
* Keys and values are stored by content only, exactly as in the RoPE path.
  Since no position is baked into a stored key, a key's position comes from
  the table alone: each block's table word carries the absolute position of
  the block's first token (its offset half), so the token in slot s sits at
  offset + s.  (For RoPE the offset is where the token's encoding frame
  starts; a block frame is the special case where every block starts its own
  frame.)
* Visibility is by logical index, as in the RoPE path; a sequence with no
  visible key outputs zeros.
"""

import numpy as np

from .lazy_oracle import BLOCK_TOKENS, unpack_block_word, valid_slots


def key_positions(table_row, length, block_fill=None):
    """Absolute position of each token of the sequence's first `length` table
    slots: the offset of its block plus its slot."""
    j = valid_slots(table_row, length, block_fill)
    _, offs = unpack_block_word(np.asarray(table_row)[j // BLOCK_TOKENS])
    return offs + j % BLOCK_TOKENS


def gather_sequence(k_pool, v_pool, table_row, length, kv_head, block_fill=None):
    """The sequence's stored keys and values in logical order ([tokens, D],
    float64), untouched: ALiBi never rotates them."""
    j = valid_slots(table_row, length, block_fill)
    ids, _ = unpack_block_word(np.asarray(table_row)[j // BLOCK_TOKENS])
    slots = j % BLOCK_TOKENS
    return (np.asarray(k_pool)[ids, kv_head, slots, :].astype(np.float64),
            np.asarray(v_pool)[ids, kv_head, slots, :].astype(np.float64))


def _attend_bias(q_rows, k, v, scale, bias, visible):
    """softmax(scale * Q K^T + bias) V on explicit matrices, masked; rows with
    no visible key give zeros."""
    out = np.zeros((q_rows.shape[0], v.shape[1]))
    if k.shape[0] == 0:
        return out
    s = scale * (q_rows @ k.T) + bias
    s = np.where(visible, s, -np.inf)
    rows = visible.any(axis=1)
    if rows.any():
        m = np.max(s[rows], axis=1, keepdims=True)
        e = np.exp(s[rows] - m)
        out[rows] = (e / e.sum(axis=1, keepdims=True)) @ v
    return out


def decode_alibi(q, q_pos, k_pool, v_pool, block_table, seq_lens, scale, slopes, block_fill=None):
    """Decode with ALiBi: q [B, Hq, D]; out [B, Hq, D] float64.  Query head h
    reads KV head h // (Hq / Hkv) and takes bias slopes[h] * (p - q_pos[b])."""
    q = np.asarray(q, dtype=np.float64)
    slopes = np.asarray(slopes, dtype=np.float64)
    bsz, hq, d = q.shape
    group = hq // k_pool.shape[1]
    out = np.zeros((bsz, hq, d))
    for b in range(bsz):
        n = int(seq_lens[b])
        pos = key_positions(block_table[b], n, block_fill).astype(np.float64)
        for h in range(hq):
            k, v = gather_sequence(k_pool, v_pool, block_table[b], n, h // group, block_fill)
            bias = (slopes[h] * (pos - float(q_pos[b])))[None, :]
            out[b, h] = _attend_bias(q[b, h][None, :], k, v, scale, bias,
                                     np.ones((1, pos.size), bool))[0]
    return out


def prefill_alibi(q, cu_q_lens, q_pos_start, k_pool, v_pool, block_table, kv_lens, scale, slopes,
                  block_fill=None):
    """Prefill with ALiBi: prompt row r of sequence b is logical index
    kv_len - P + r at position q_pos_start + r and sees keys of logical
    index <= its own (causal by table order)."""
    q = np.asarray(q, dtype=np.float64)
    slopes = np.asarray(slopes, dtype=np.float64)
    tq, hq, d = q.shape
    group = hq // k_pool.shape[1]
    out = np.zeros((tq, hq, d))
    for b in range(len(cu_q_lens) - 1):
        s0, s1 = int(cu_q_lens[b]), int(cu_q_lens[b + 1])
        p = s1 - s0
        if p == 0:
            continue
        kv = int(kv_lens[b])
        rows = np.arange(p)
        t = kv - p + rows
        npos = float(q_pos_start[b]) + rows
        pos = key_positions(block_table[b], kv, block_fill).astype(np.float64)
        vis = valid_slots(block_table[b], kv, block_fill)[None, :] <= t[:, None]
        for h in range(hq):
            k, v = gather_sequence(k_pool, v_pool, block_table[b], kv, h // group, block_fill)
            bias = slopes[h] * (pos[None, :] - npos[:, None])
            out[s0:s1, h] = _attend_bias(q[s0:s1, h], k, v, scale, bias, vis)
    return out


def alibi_slopes(num_heads):
    """The geometric slopes 2^(-8 (h+1) / H) for H heads (a power of two),
    used by the workloads."""
    h = np.arange(1, num_heads + 1, dtype=np.float64)
    return np.power(2.0, -8.0 * h / num_heads)

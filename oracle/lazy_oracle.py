"""Plain float64 reference of deferred-RoPE paged attention (test infrastructure).

Readings of the pages that this file fixes (they are silent or loose there):

* Table word: one 32-bit word per 16-token block; bits 0..15 hold the
  physical block id, bits 16..31 the (unsigned) position offset of that
  block's frame.  [LA] "Implementação Técnica", Decoding, only says that the
  (block id, offset) pair lives in a single register.
* Storage frame: a stored key is position-free in the sense of [LA]
  "Metodologia": it carries the rotation of its place inside its own
  document (frame origin 0), never the place the document is put at.  The key
  that a placed token really has is the stored key rotated by its block's
  offset.  This is the eager "position-adjusted copy" of [LA] "Declaração do
  Problema", which this oracle materialises.
* RoPE: rotate-half layout, pairs (i, i + D/2), frequency theta**(-2i/D).
  The pages name RoPE without defining it.
* Values carry no position; only queries and keys rotate.
* Softmax scale is passed explicitly (1/sqrt(D) in [WHY] "Lo que hace el
  decoding autorregresivo"); the page's tiled routine has none.
* Visibility (causal mask) uses the logical token index in table order,
  never the RoPE position.
* A sequence with no visible key has output zeros.
"""

import numpy as np

BLOCK_TOKENS = 16  # [KVF] "PagedAttention": the cache is allocated in 16-token blocks


def unpack_block_word(words):
    """Split packed table words into (block_id, offset).

    [LA] "Implementação Técnica", Decoding: block id and offset share one
    register.  Layout read here: id in the low 16 bits, offset in the high 16.
    """
    w = np.asarray(words, dtype=np.uint64)
    return (w & 0xFFFF).astype(np.int64), (w >> 16).astype(np.int64)


def rope_frequencies(head_dim, theta):
    """Angular frequency of each rotation pair: theta ** (-2 i / D), i < D/2."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / head_dim)


def rope(x, pos, theta):
    """Rotate vectors x[..., D] by position ``pos`` (rotate-half RoPE, fp64).

    Pair (x_i, x_{i+D/2}) is turned by the angle pos * theta_i:
      y_i       = x_i cos - x_{i+D/2} sin
      y_{i+D/2} = x_{i+D/2} cos + x_i sin
    ``pos`` broadcasts against x's leading axes.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    freqs = rope_frequencies(d, theta)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * freqs
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def softmax(scores):
    """Row softmax: subtract the row max, exponentiate, divide by the row sum."""
    s = np.asarray(scores, dtype=np.float64)
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def valid_slots(table_row, length, block_fill=None):
    """Table slots j < length that hold a token, in order.

    Slot j is slot j % 16 of block table_row[j // 16].  Without fill counts
    every slot does; with them (block_fill[block id] = tokens stored in that
    physical block, the rest of it unused, e.g. the end of a document whose
    length is not a multiple of 16) only slots below their block's count.
    """
    j = np.arange(int(length))
    if block_fill is None or j.size == 0:
        return j
    ids, _ = unpack_block_word(np.asarray(table_row)[j // BLOCK_TOKENS])
    return j[(j % BLOCK_TOKENS) < np.asarray(block_fill)[ids]]


def materialize_sequence(k_pool, v_pool, table_row, length, kv_head, theta, block_fill=None):
    """Eager position-adjusted copy of one sequence's keys and values.

    Logical token j of the sequence lives in block table_row[j // 16], slot
    j % 16 (slots past a block's fill count hold no token and are skipped).
    Its key is the stored key rotated by that block's offset (the copy that
    position-aware caching would keep, [LA] "Declaração do Problema"); its
    value is the stored value.  Returns (K_hat, V_hat), each [tokens, D]
    float64.
    """
    d = k_pool.shape[-1]
    j = valid_slots(table_row, length, block_fill)
    if j.size == 0:
        return np.zeros((0, d)), np.zeros((0, d))
    ids, offs = unpack_block_word(np.asarray(table_row)[j // BLOCK_TOKENS])
    slots = j % BLOCK_TOKENS
    k_stored = np.asarray(k_pool)[ids, kv_head, slots, :].astype(np.float64)
    v_stored = np.asarray(v_pool)[ids, kv_head, slots, :].astype(np.float64)
    return rope(k_stored, offs, theta), v_stored


def _attend(q_rot, k_hat, v_hat, scale, visible):
    """Standard attention on explicit matrices ([KVF] "Flash Attention").

    S = scale * Q K^T, masked where not visible, P = softmax(S), O = P V.
    q_rot [R, D]; k_hat, v_hat [N, D]; visible [R, N] bool.
    Rows with no visible key give zeros.
    """
    r = q_rot.shape[0]
    out = np.zeros((r, v_hat.shape[1]))
    if k_hat.shape[0] == 0:
        return out
    s = scale * (q_rot @ k_hat.T)
    s = np.where(visible, s, -np.inf)
    any_vis = visible.any(axis=1)
    if any_vis.any():
        p = softmax(s[any_vis])
        out[any_vis] = p @ v_hat
    return out


def decode_one(q_vec, q_pos, k_pool, v_pool, table_row, seq_len, kv_head, scale, theta, block_fill=None):
    """One decode row: a single query against all seq_len cached tokens.

    [WHY] "El remedio": the new query attends a 1 x (t+1) row of the cache,
    softmax, times V.  The query is rotated to its absolute position n and
    each key is the materialised position-adjusted copy ([LA] "Equivalência
    Matemática" states that deferring the rotation gives the same result).
    """
    k_hat, v_hat = materialize_sequence(k_pool, v_pool, table_row, seq_len, kv_head, theta, block_fill)
    q_rot = rope(np.asarray(q_vec, dtype=np.float64)[None, :], q_pos, theta)
    vis = np.ones((1, k_hat.shape[0]), dtype=bool)
    return _attend(q_rot, k_hat, v_hat, scale, vis)[0]


def decode(q, q_pos, k_pool, v_pool, block_table, seq_lens, scale, theta, block_fill=None):
    """Decode for a batch.  q [B, Hq, D] raw; returns out [B, Hq, D] float64.

    Query head h reads KV head h // (Hq / Hkv) (grouped-query attention).
    """
    q = np.asarray(q, dtype=np.float64)
    bsz, hq, d = q.shape
    hkv = k_pool.shape[1]
    group = hq // hkv
    out = np.zeros((bsz, hq, d))
    for b in range(bsz):
        for g in range(hkv):
            k_hat, v_hat = materialize_sequence(k_pool, v_pool, block_table[b], seq_lens[b], g, theta,
                                                block_fill)
            q_rot = rope(q[b, g * group:(g + 1) * group], q_pos[b], theta)
            vis = np.ones((group, k_hat.shape[0]), dtype=bool)
            out[b, g * group:(g + 1) * group] = _attend(q_rot, k_hat, v_hat, scale, vis)
    return out


def prefill_rows(q_rows, rows, q_len, q_pos_start, k_pool, v_pool, table_row, kv_len,
                 kv_head, scale, theta, block_fill=None):
    """Prefill output for selected prompt rows of one sequence and one head.

    The prompt's P = q_len tokens are the last P logical tokens of the table
    (their K/V were appended before the call).  Prompt row r sits at logical
    index t = kv_len - P + r and position n = q_pos_start + r; it sees the
    keys with logical index <= t ([KVF] "Flash Attention" tiles Q against
    K/V; causal within the prompt).  q_rows [R, D] raw, rows [R] ints.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    k_hat, v_hat = materialize_sequence(k_pool, v_pool, table_row, kv_len, kv_head, theta, block_fill)
    q_rot = rope(q_rows, q_pos_start + rows, theta)
    t = kv_len - q_len + rows     # the prompt fills the table's last slots
    vis = valid_slots(table_row, kv_len, block_fill)[None, :] <= t[:, None]
    return _attend(q_rot, k_hat, v_hat, scale, vis)


def prefill(q, cu_q_lens, q_pos_start, k_pool, v_pool, block_table, kv_lens, scale, theta, block_fill=None):
    """Prefill for a batch.  q [Tq, Hq, D] packed by cu_q_lens [B+1]."""
    q = np.asarray(q, dtype=np.float64)
    tq, hq, d = q.shape
    hkv = k_pool.shape[1]
    group = hq // hkv
    out = np.zeros((tq, hq, d))
    for b in range(len(cu_q_lens) - 1):
        s0, s1 = int(cu_q_lens[b]), int(cu_q_lens[b + 1])
        p = s1 - s0
        if p == 0:
            continue
        rows = np.arange(p)
        for h in range(hq):
            out[s0:s1, h] = prefill_rows(q[s0:s1, h], rows, p, int(q_pos_start[b]), k_pool, v_pool,
                                         block_table[b], int(kv_lens[b]), h // group, scale, theta,
                                         block_fill)
    return out


def append(k_pool, v_pool, k_new, v_new, slot_mapping):
    """Return copies of the pools with new rows written, unrotated.

    [KVF] "Construa", Passo 1 (append per layer/head) and [WHY] "El remedio"
    (add the new row to the cache).  Token t of k_new/v_new [T, Hkv, D] goes
    to block slot_mapping[t] // 16, slot slot_mapping[t] % 16, every head.
    Slots < 0 are padding and slots past the pool do not exist; both are
    skipped.  The copy is exact.
    """
    k_out, v_out = np.array(k_pool, copy=True), np.array(v_pool, copy=True)
    capacity = k_out.shape[0] * BLOCK_TOKENS
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0 or slot >= capacity:
            continue
        k_out[slot // BLOCK_TOKENS, :, slot % BLOCK_TOKENS, :] = k_new[t]
        v_out[slot // BLOCK_TOKENS, :, slot % BLOCK_TOKENS, :] = v_new[t]
    return k_out, v_out


def cache_bytes(layers, heads, head_dim, seq_len, batch, elem_bytes):
    """Bytes held by a KV cache: 2 * L * H * d_h * S * B * s ([WHY] "El precio")."""
    return 2 * layers * heads * head_dim * seq_len * batch * elem_bytes


def relative_rotation_overhead(m_rows, n_keys, head_dim):
    """Extra FLOPs of rotating one staged key tile once by the relative offset,
    as a fraction of the tile's attention FLOPs ([LA] "Implementação Técnica",
    Prefilling).  Each of the tile's N x D key elements takes 3 FLOPs in the
    rotate-half form (x cos - y sin: two products and a sum); Q K^T and P V
    take 2 * M * N * D FLOPs each for a query tile of M rows."""
    rotate = 3 * n_keys * head_dim
    attend = 2 * (2 * m_rows * n_keys * head_dim)
    return rotate / attend


def _tile_partial(q, keys, values):
    """Softmax statistics of one key tile on its own: (m, l, u) with
    m = max_j s_j, l = sum_j exp(s_j - m), u = sum_j exp(s_j - m) v_j, where
    s_j = q . k_j.  An empty tile has m = -inf, l = 0, u = 0."""
    if keys.shape[0] == 0:
        return -np.inf, 0.0, np.zeros(values.shape[1])
    scores = keys @ q
    m = float(np.max(scores))
    w = np.exp(scores - m)
    return m, float(np.sum(w)), w @ values


def merge_tile_partials(partials):
    """Log-sum-exp merge of per-tile (m, l, u) statistics.

    With M = max over tiles of m_t, every tile's terms are brought to the
    common reference by the factor exp(m_t - M):
      softmax(s) . V = sum_t exp(m_t - M) u_t / sum_t exp(m_t - M) l_t.
    Tiles with m_t = -inf (no keys) carry weight 0.
    """
    big = max(m for m, _, _ in partials)
    num = np.zeros_like(partials[0][2])
    den = 0.0
    for m, l, u in partials:
        f = 0.0 if m == -np.inf else float(np.exp(m - big))
        num = num + f * u
        den = den + f * l
    return num / den


def blockwise_softmax_dot(q, keys, values, tile):
    """softmax(q . K^T) V from independent key tiles ([KVF] "Construa",
    Passo 2, and "Flash Attention": the result of a softmax over all keys can
    be assembled from tiles seen one at a time).

    Each tile of ``tile`` keys is reduced to (max, sum, unnormalised output)
    by itself; the partials are then combined by one log-sum-exp merge.  No
    scale is applied, as on the page; callers pre-scale q.
    """
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    starts = range(0, keys.shape[0], tile)
    return merge_tile_partials([_tile_partial(q, keys[a:a + tile], values[a:a + tile]) for a in starts])

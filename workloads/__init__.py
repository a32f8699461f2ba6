"""Seeded synthetic inputs for the deferred-RoPE paged attention workloads.

Shared by the tests, ``bench.py`` and ``__graft_entry__.smoke()``: the only
code that both the CPU oracle and the HIP path are fed from.  It holds none of
the attention arithmetic -- it draws random values, builds documents, packs
block-table words, assigns pool slots, and converts between float32 and
bfloat16 bit patterns.

Workload shapes (documents of 256..2048 tokens, 8B / 70B head geometry,
Zipf-skewed document reuse, a ~1 GB KV budget) stand in for the RAG
benchmarks of the LazyAttention summary's "Resultados Experimentais", whose
datasets and model weights are not available; all values are synthetic.

Layout conventions (the same ones the library documents):
  * K/V pool: [num_blocks][num_kv_heads][16][head_dim], content-only keys.
  * Table word: block id in bits 0..15, position offset in bits 16..31.
  * Every block of a document carries the document's start position as its
    offset; a prompt's (or a new token's) blocks carry the prompt's first
    position.  Only a sequence's last block may be partly filled, except in
    ragged layouts, where every document's last block may be: there a
    per-block fill count (uint8 per physical block) says how many of its 16
    slots hold tokens, and lengths count table slots.
"""

from dataclasses import dataclass, field
from typing import List

import numpy as np

BLOCK = 16

F32 = "f32"
BF16 = "bf16"


# ----------------------------------------------------------------- bit helpers
def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (round to nearest even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b):
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def pack_words(block_ids, offsets):
    """Pack (block id, offset) pairs into uint32 table words (16 | 16 bits)."""
    ids = np.asarray(block_ids, dtype=np.int64)
    offs = np.asarray(offsets, dtype=np.int64)
    if ids.size and (ids.min() < 0 or ids.max() > 0xFFFF):
        raise ValueError("block id out of the 16-bit range")
    if offs.size and (offs.min() < 0 or offs.max() > 0xFFFF):
        raise ValueError("offset out of the 16-bit range")
    return (ids | (offs << 16)).astype(np.uint32)


def e4m3_codes(rng, shape, exp_lo=3, exp_hi=9, subnormal_frac=0.05):
    """Random contents of an 8-bit (E4M3) pool: byte patterns with a uniform
    sign, exponent field U{exp_lo..exp_hi} (magnitudes 2^-4 .. 7.5), mantissa
    U{0..7}, and a fraction of subnormal patterns (exponent field 0).  Never
    the NaN pattern.  Input data only: no value is quantised here."""
    n = int(np.prod(shape))
    sign = rng.integers(0, 2, size=n, dtype=np.uint8) << np.uint8(7)
    exp = rng.integers(exp_lo, exp_hi + 1, size=n).astype(np.uint8)
    exp[rng.random(n) < subnormal_frac] = 0
    man = rng.integers(0, 8, size=n, dtype=np.uint8)
    return (sign | (exp << np.uint8(3)) | man).reshape(shape)


def e4m3_codes_torch(shape, device, seed, exp_lo=3, exp_hi=9):
    """e4m3_codes drawn on the GPU with torch's seeded generator (full-size
    pools), without subnormal patterns."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    sign = torch.randint(0, 2, shape, dtype=torch.uint8, device=device, generator=gen) << 7
    exp = torch.randint(exp_lo, exp_hi + 1, shape, dtype=torch.uint8, device=device, generator=gen)
    man = torch.randint(0, 8, shape, dtype=torch.uint8, device=device, generator=gen)
    return sign | (exp << 3) | man


def int8_codes(rng, shape, spread=40.0):
    """Random contents of an int8 pool: rounded N(0, spread^2) integers,
    clipped to [-127, 127], as int8 bytes.  Input data only."""
    x = np.clip(np.rint(rng.standard_normal(size=shape) * spread), -127, 127)
    return x.astype(np.int8)


def int8_codes_torch(shape, device, seed, spread=40.0):
    """int8_codes drawn on the GPU with torch's seeded generator (full-size pools)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    x = torch.randn(shape, device=device, generator=gen) * spread
    return x.round().clamp(-127, 127).to(torch.int8)


def _fp8_lane_order():
    """For byte b of an 8-bit pool's (block, KV head) record (2048 bytes, the
    lane order the library documents), the logical index token * 128 + dim of
    the K code and of the V code stored there."""
    b = np.arange(2048)
    i, lane, x = b // 1024, (b % 1024) // 16, b % 16
    g, t = lane // 16, lane % 16
    k_src = t * 128 + 32 * g + 16 * i + x
    v_src = (4 * g + x % 4) * 128 + 16 * (4 * i + x // 4) + t
    return k_src, v_src


def fp8_pools_to_device_order(k_codes, v_codes):
    """Logical [NB, Hkv, 16, 128] E4M3 codes -> the library's byte order (same
    shape, bytes permuted within each (block, KV head))."""
    ks, vs = _fp8_lane_order()
    shp = k_codes.shape
    k = np.ascontiguousarray(k_codes).reshape(shp[0], shp[1], 2048)[..., ks].reshape(shp)
    v = np.ascontiguousarray(v_codes).reshape(shp[0], shp[1], 2048)[..., vs].reshape(shp)
    return k, v


def fp8_pools_from_device_order(k_dev, v_dev):
    """Inverse of fp8_pools_to_device_order."""
    ks, vs = _fp8_lane_order()
    shp = k_dev.shape
    k = np.empty((shp[0], shp[1], 2048), dtype=k_dev.dtype)
    v = np.empty_like(k)
    k[..., ks] = np.ascontiguousarray(k_dev).reshape(shp[0], shp[1], 2048)
    v[..., vs] = np.ascontiguousarray(v_dev).reshape(shp[0], shp[1], 2048)
    return k.reshape(shp), v.reshape(shp)


# ------------------------------------------------------------------- layouts
@dataclass
class Layout:
    """Block placement of a batch of sequences over one shared pool.

    table[b] lists the sequence's blocks in logical order; tail_* describe the
    region written by the step's append (a new decode token or a prompt).
    """
    num_blocks: int
    table: np.ndarray            # uint32 [B, max_blocks]
    cached_lens: np.ndarray      # int32 [B] tokens already in the cache
    tail_lens: np.ndarray        # int32 [B] tokens the step appends
    tail_pos: np.ndarray         # int32 [B] position of the first appended token
    slot_mapping: np.ndarray     # int32 [sum(tail_lens)] pool slot of each appended token
    doc_spans: List[list] = field(default_factory=list)  # per seq: (doc, length, offset)
    unique_doc_tokens: int = 0   # tokens physically stored for documents
    block_fill: np.ndarray = None  # ragged layouts: uint8 [num_blocks] tokens per block
    slot_lens: np.ndarray = None   # ragged layouts: int32 [B] table slots up to the last token

    @property
    def total_lens(self):
        return (self.cached_lens + self.tail_lens).astype(np.int32)

    @property
    def batch(self):
        return int(self.table.shape[0])


def build_layout(rng, seq_docs, doc_lens, tail_lens, offsets=None, tail_pos=None,
                 spare_blocks=0, shuffle=True, ragged=False):
    """Place documents and appended tails into a shuffled block pool.

    seq_docs[b]  : list of document indices making up sequence b (in order).
    doc_lens[d]  : length of document d; every document except a sequence's
                   last item must be a whole number of blocks.
    tail_lens[b] : tokens the step appends after the documents.
    offsets[b]   : optional explicit offset of each document of sequence b;
                   default is contiguous placement (prefix sums).
    tail_pos[b]  : position of the first appended token (default: right after
                   the documents).
    A document used by several sequences is stored once (zero-copy reuse).
    ragged=True lets any document end mid-block and records block_fill (the
    tokens of each physical block, 16 for spare blocks) and slot_lens.
    """
    bsz = len(seq_docs)
    doc_blocks = {}
    n_blocks = 0
    for docs in seq_docs:
        for d in docs:
            if d not in doc_blocks:
                nb = -(-int(doc_lens[d]) // BLOCK)
                doc_blocks[d] = (n_blocks, nb)
                n_blocks += nb
    unique_tokens = sum(int(doc_lens[d]) for d in doc_blocks)
    tail_first = []
    for b in range(bsz):
        tail_first.append(n_blocks)
        n_blocks += -(-int(tail_lens[b]) // BLOCK)
    n_blocks += spare_blocks
    if n_blocks > 0x10000:
        raise ValueError("pool needs more than 65536 blocks")
    perm = rng.permutation(n_blocks) if shuffle else np.arange(n_blocks)
    fill = None
    if ragged:
        fill = np.full(n_blocks, BLOCK, dtype=np.uint8)
        for d, (first, nb) in doc_blocks.items():
            fill[perm[first + nb - 1]] = int(doc_lens[d]) - BLOCK * (nb - 1)

    rows, cached, tpos, spans, slots, slot_lens = [], [], [], [], [], []
    for b, docs in enumerate(seq_docs):
        words = []
        pos = 0
        span = []
        for i, d in enumerate(docs):
            ln = int(doc_lens[d])
            if ln % BLOCK and not ragged and (i != len(docs) - 1 or tail_lens[b]):
                raise ValueError("only a sequence's last item may end mid-block")
            off = pos if offsets is None else int(offsets[b][i])
            first, nb = doc_blocks[d]
            words.extend(pack_words(perm[first:first + nb], [off] * nb).tolist())
            span.append((d, ln, off))
            pos += ln
        cached.append(pos)
        tp = pos if tail_pos is None else int(tail_pos[b])
        tpos.append(tp)
        nt = int(tail_lens[b])
        nbt = -(-nt // BLOCK)
        ids = perm[tail_first[b]:tail_first[b] + nbt]
        words.extend(pack_words(ids, [tp] * nbt).tolist())
        for t in range(nt):
            slots.append(int(ids[t // BLOCK]) * BLOCK + t % BLOCK)
        if ragged:
            for i in range(nbt):
                fill[ids[i]] = min(BLOCK, nt - BLOCK * i)
        slot_lens.append(BLOCK * (len(words) - nbt) + nt)
        rows.append(words)
        spans.append(span)
    width = max(1, max(len(r) for r in rows))
    table = np.zeros((bsz, width), dtype=np.uint32)
    for b, r in enumerate(rows):
        table[b, :len(r)] = r
    return Layout(num_blocks=n_blocks, table=table,
                  cached_lens=np.array(cached, dtype=np.int32),
                  tail_lens=np.array(tail_lens, dtype=np.int32),
                  tail_pos=np.array(tpos, dtype=np.int32),
                  slot_mapping=np.array(slots, dtype=np.int32),
                  doc_spans=spans, unique_doc_tokens=unique_tokens, block_fill=fill,
                  slot_lens=np.array(slot_lens, dtype=np.int32) if ragged else None)


def block_frame_table(layout):
    """The layout's table with every block carrying its own first token's
    position (frame start + 16 * block index within the frame) instead of the
    frame start: the rows ALiBi reads, where a key's position is its block's
    offset plus its slot."""
    table = layout.table.copy()
    for b in range(layout.batch):
        col = 0
        runs = [(ln, off) for _, ln, off in layout.doc_spans[b]]
        runs.append((int(layout.tail_lens[b]), int(layout.tail_pos[b])))
        for ln, off in runs:
            nb = -(-int(ln) // BLOCK)
            ids = table[b, col:col + nb] & np.uint32(0xFFFF)
            table[b, col:col + nb] = pack_words(ids, off + BLOCK * np.arange(nb))
            col += nb
    return table


def _docs_filling(rng, total, lo_blocks, hi_blocks):
    """Document lengths (multiples of 16, uniform in blocks) summing to total."""
    lens = []
    left = total
    while left > 0:
        ln = BLOCK * int(rng.integers(lo_blocks, hi_blocks + 1))
        ln = min(ln, left)
        lens.append(ln)
        left -= ln
    return lens


def _split_into(rng, total_blocks, parts):
    """Cut total_blocks into `parts` non-empty block counts at random points."""
    cuts = np.sort(rng.choice(np.arange(1, total_blocks), size=parts - 1, replace=False))
    edges = np.concatenate([[0], cuts, [total_blocks]])
    return (np.diff(edges) * BLOCK).tolist()


# -------------------------------------------------------------------- values
@dataclass
class Case:
    """One workload: geometry, layout and (once materialised) its values."""
    name: str
    kind: str                    # "decode" | "prefill"
    dtype: str                   # F32 | BF16
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    rope_theta: float
    layout: Layout
    q_std: float = 1.0
    kv_std: float = 0.5
    seed: int = 0
    # values: numpy arrays (float32, or uint16 bf16 bits) or torch tensors
    q: object = None             # decode [B, Hq, D]; prefill [Tq, Hq, D]
    k_pool: object = None        # [NB, Hkv, 16, D]
    v_pool: object = None
    k_new: object = None         # [T_new, Hkv, D]
    v_new: object = None

    @property
    def scale(self):
        return 1.0 / float(np.sqrt(self.head_dim))

    @property
    def batch(self):
        return self.layout.batch

    @property
    def q_pos(self):
        """Decode: position of the new query token."""
        return self.layout.tail_pos.astype(np.int32)

    @property
    def seq_lens(self):
        """Lengths the library takes: tokens attended by the step (cached +
        appended), counted in table slots for ragged layouts."""
        lay = self.layout
        return lay.total_lens if lay.slot_lens is None else lay.slot_lens

    @property
    def block_fill(self):
        return self.layout.block_fill

    @property
    def cu_q_lens(self):
        return np.concatenate([[0], np.cumsum(self.layout.tail_lens)]).astype(np.int32)

    @property
    def max_q_len(self):
        return int(self.layout.tail_lens.max()) if self.batch else 0

    def kv_bytes_read(self):
        """Logical K+V bytes a decode pass reads (every attended token once)."""
        esz = 4 if self.dtype == F32 else 2
        return int(self.layout.total_lens.sum()) * self.num_kv_heads * self.head_dim * 2 * esz

    def attention_flops(self):
        """4*D FLOPs per visible (query, key) pair per query head (QK^T and PV)."""
        if self.kind == "decode":
            pairs = int(self.seq_lens.sum())
        else:
            pairs = 0
            for c, p in zip(self.layout.cached_lens.tolist(), self.layout.tail_lens.tolist()):
                pairs += p * c + p * (p + 1) // 2
        return 4 * self.head_dim * pairs * self.num_q_heads


def _shape_of(case):
    lay = case.layout
    nq = lay.batch if case.kind == "decode" else int(lay.tail_lens.sum())
    nnew = int(lay.tail_lens.sum())
    return ((nq, case.num_q_heads, case.head_dim),
            (lay.num_blocks, case.num_kv_heads, BLOCK, case.head_dim),
            (nnew, case.num_kv_heads, case.head_dim))


def materialize_numpy(case):
    """Draw the case's values on the host with numpy (seeded)."""
    rng = np.random.default_rng(case.seed + 1000)
    qs, ps, ns = _shape_of(case)

    def draw(shape, std):
        x = rng.standard_normal(size=shape, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        return x if case.dtype == F32 else f32_to_bf16_bits(x)

    case.q = draw(qs, case.q_std)
    case.k_pool = draw(ps, case.kv_std)
    case.v_pool = draw(ps, case.kv_std)
    case.k_new = draw(ns, case.kv_std)
    case.v_new = draw(ns, case.kv_std)
    return case


def add_score_shift(case, q_amp, k_cached, k_new, seed=0):
    """Give every score of a query row a large common part (host arrays).

    The last rotary pair (dims D/2-1 and D-1, the lowest frequency) is
    overwritten: q gets x = U(-q_amp, q_amp), y = 0; cached keys x = k_cached
    and appended keys x = k_new, y = 0.  With rope_theta ~ 1e30 that pair turns
    by a negligible angle, so q.k gains q_x * k_x, equal for all keys of a
    kind: scores far outside exp's range while the softmax itself stays as
    well-conditioned as without the shift.  Call after materialize_numpy.
    """
    rng = np.random.default_rng(seed + 3000)
    d = case.head_dim
    xi, yi = d // 2 - 1, d - 1

    def edit(arr, fn):
        x = to_float(arr, case.dtype).copy()
        fn(x)
        return x if case.dtype == F32 else f32_to_bf16_bits(x)

    def q_fn(x):
        x[..., xi] = rng.uniform(-q_amp, q_amp, size=x.shape[:-1]).astype(np.float32)
        x[..., yi] = 0.0

    def k_fn(val):
        def fn(x):
            x[..., xi] = np.float32(val)
            x[..., yi] = 0.0
        return fn

    case.q = edit(case.q, q_fn)
    case.k_pool = edit(case.k_pool, k_fn(k_cached))
    case.k_new = edit(case.k_new, k_fn(k_new))
    return case


def set_score_spread(case, sigma, v_abs=2.0, seed=0):
    """Scores that spread widely across keys (host arrays).

    Keys (cached and appended) are redrawn as N(0, sigma^2) per element and
    values as U(-v_abs, v_abs); with q ~ N(0, 1) and the scale 1/sqrt(D), a
    query's scores then have standard deviation sigma (natural-log units)
    across keys.  Bounded values keep the output's own bf16 rounding small
    next to errors in the scores.  Call after materialize_numpy.
    """
    rng = np.random.default_rng(seed + 4000)

    def draw(arr, fn):
        x = fn(np.shape(arr)).astype(np.float32)
        return x if case.dtype == F32 else f32_to_bf16_bits(x)

    def k_fn(shape):
        return rng.standard_normal(shape) * sigma

    def v_fn(shape):
        return rng.uniform(-v_abs, v_abs, size=shape)

    case.k_pool = draw(case.k_pool, k_fn)
    case.k_new = draw(case.k_new, k_fn)
    case.v_pool = draw(case.v_pool, v_fn)
    case.v_new = draw(case.v_new, v_fn)
    return case


def materialize_torch(case, device):
    """Draw the case's values directly in device memory with torch (seeded).

    Used for the full-size workloads, whose pools are gigabytes.
    """
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(case.seed + 2000)
    qs, ps, ns = _shape_of(case)
    tdt = torch.float32 if case.dtype == F32 else torch.bfloat16

    def draw(shape, std):
        x = torch.empty(shape, dtype=torch.float32, device=device)
        x.normal_(0.0, std, generator=gen)
        return x if tdt == torch.float32 else x.to(tdt)

    case.q = draw(qs, case.q_std)
    case.k_pool = draw(ps, case.kv_std)
    case.v_pool = draw(ps, case.kv_std)
    case.k_new = draw(ns, case.kv_std)
    case.v_new = draw(ns, case.kv_std)
    return case


def to_float(arr, dtype):
    """Host float32 view of a case value (bf16 bits widened exactly)."""
    try:
        import torch
        if isinstance(arr, torch.Tensor):
            t = arr.detach()
            if t.dtype == torch.bfloat16:
                return bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16))
            return t.float().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.asarray(arr)
    return bf16_bits_to_f32(a) if dtype == BF16 else a.astype(np.float32)


# ------------------------------------------------------------ the workloads
def tiny_decode(seed=1, layer=0, swap_docs=False):
    """Tiny fp32 decode step, one layer of the 4-layer / 4-head / d_h=16 model.

    Two 16-token documents stored position-free and placed at positions 0 and
    16 (swapped order with swap_docs); 32 cached tokens; the new query at
    position 32 appends its own K/V and attends 33 tokens.  theta = 1e4,
    q, K, V ~ N(0, 1).  Each layer is an independent draw.
    """
    rng = np.random.default_rng(seed * 100 + layer)
    order = [1, 0] if swap_docs else [0, 1]
    lay = build_layout(rng, [order], [16, 16], [1], offsets=[[0, 16]])
    case = Case("tiny_fp32_decode", "decode", F32, 4, 4, 16, 1.0e4, lay,
                q_std=1.0, kv_std=1.0, seed=seed * 100 + layer)
    return case


def decode_case(seed, batch, num_q_heads, num_kv_heads, head_dim, ctx, doc_blocks=(16, 128),
                dtype=BF16, theta=5.0e5, offsets="contiguous", new_token=True, name="decode",
                kv_std=0.5):
    """Decode batch whose sequences are cached documents filling ctx tokens each.

    ctx may be an int or a per-sequence list; documents have lengths
    16 * U{doc_blocks}; only the last document of a sequence is truncated to
    hit ctx exactly (ctx not a multiple of 16 gives a ragged last block when
    new_token is False).  offsets="random" places documents at arbitrary,
    non-contiguous positions instead of prefix sums.
    """
    rng = np.random.default_rng(seed)
    ctxs = [ctx] * batch if np.isscalar(ctx) else list(ctx)
    seq_docs, doc_lens, offs = [], [], []
    for b in range(batch):
        c = int(ctxs[b])
        if new_token and c % BLOCK:
            raise ValueError("with a new token the cached context must fill whole blocks")
        lens = _docs_filling(rng, c, *doc_blocks) if c else []
        ids = list(range(len(doc_lens), len(doc_lens) + len(lens)))
        doc_lens.extend(lens)
        seq_docs.append(ids)
        if offsets == "random":
            offs.append([int(x) for x in rng.integers(0, 60000 - 2048, size=len(lens))])
    tails = [1 if new_token else 0] * batch
    tail_pos = None
    if offsets == "random":
        tail_pos = [int(x) for x in rng.integers(0, 60000, size=batch)]
    lay = build_layout(rng, seq_docs, doc_lens, tails,
                       offsets=offs if offsets == "random" else None, tail_pos=tail_pos)
    return Case(name, "decode", dtype, num_q_heads, num_kv_heads, head_dim, theta, lay,
                kv_std=kv_std, seed=seed)


def llama8b_decode(seed=2, batch=64, ctx=8192):
    """Llama-3.1-8B-shaped single-layer decode, bf16: 32 q / 8 KV heads, d_h=128.

    64 sequences of 8192 cached tokens built from documents of 256..2048
    tokens in 16-token blocks shuffled in a pool; the new token (position
    8192) is appended and attends 8193 tokens.  K, V ~ N(0,1)*0.5,
    theta = 5e5.
    """
    return decode_case(seed, batch, 32, 8, 128, ctx, (16, 128), name="llama8b_decode")


def llama70b_decode(seed=4, batch=16, ctx=32768, docs=(16, 64)):
    """Llama-3.1-70B-shaped single-layer decode, bf16: 64 q / 8 KV heads (GQA 8).

    16 sequences of 32768 cached tokens cut at block granularity into
    U{16..64} documents each; the new token at position 32768 is appended.
    """
    rng = np.random.default_rng(seed)
    seq_docs, doc_lens = [], []
    for _ in range(batch):
        parts = int(rng.integers(docs[0], docs[1] + 1))
        lens = _split_into(rng, ctx // BLOCK, parts)
        seq_docs.append(list(range(len(doc_lens), len(doc_lens) + len(lens))))
        doc_lens.extend(lens)
    lay = build_layout(rng, seq_docs, doc_lens, [1] * batch)
    return Case("llama70b_decode", "decode", BF16, 64, 8, 128, 5.0e5, lay, seed=seed)


def zipf_decode(seed=5, batch=128, catalogue=1000, zipf_s=1.2, docs_per_seq=(4, 8),
                doc_blocks=(16, 128), num_q_heads=32, num_kv_heads=8):
    """Zipf document-reuse decode mix, bf16, 8B shape.

    A catalogue of 1000 documents (16 * U{16..128} tokens); each of the 128
    sequences draws U{4..8} distinct documents with p(rank i) ~ i^-1.2 and
    places them contiguously in random order.  A document drawn by several
    sequences is stored once and its blocks are shared zero-copy.
    """
    rng = np.random.default_rng(seed)
    doc_lens = [BLOCK * int(x) for x in rng.integers(doc_blocks[0], doc_blocks[1] + 1, size=catalogue)]
    p = np.arange(1, catalogue + 1, dtype=np.float64) ** (-zipf_s)
    p /= p.sum()
    seq_docs = []
    for _ in range(batch):
        k = int(rng.integers(docs_per_seq[0], docs_per_seq[1] + 1))
        seq_docs.append([int(d) for d in rng.choice(catalogue, size=k, replace=False, p=p)])
    lay = build_layout(rng, seq_docs, doc_lens, [1] * batch)
    return Case("zipf_reuse_decode", "decode", BF16, num_q_heads, num_kv_heads, 128, 5.0e5, lay, seed=seed)


def prefill_case(seed, batch, num_q_heads, num_kv_heads, head_dim, cached, prompt,
                 doc_blocks=(16, 128), dtype=BF16, theta=5.0e5, offsets="contiguous",
                 name="prefill"):
    """Prefill batch: cached documents then a prompt that is appended and attends.

    cached / prompt may be ints or per-sequence lists.  The prompt's blocks
    carry the prompt's first position as offset (contiguous after the
    documents unless offsets="random").
    """
    rng = np.random.default_rng(seed)
    cs = [cached] * batch if np.isscalar(cached) else list(cached)
    ps = [prompt] * batch if np.isscalar(prompt) else list(prompt)
    seq_docs, doc_lens, offs, tpos = [], [], [], []
    for b in range(batch):
        if cs[b] % BLOCK:
            raise ValueError("cached documents must fill whole blocks")
        lens = _docs_filling(rng, int(cs[b]), *doc_blocks) if cs[b] else []
        seq_docs.append(list(range(len(doc_lens), len(doc_lens) + len(lens))))
        doc_lens.extend(lens)
        if offsets == "random":
            offs.append([int(x) for x in rng.integers(0, 30000, size=len(lens))])
            tpos.append(int(rng.integers(0, 30000)))
    lay = build_layout(rng, seq_docs, doc_lens, ps,
                       offsets=offs if offsets == "random" else None,
                       tail_pos=tpos if offsets == "random" else None)
    return Case(name, "prefill", dtype, num_q_heads, num_kv_heads, head_dim, theta, lay, seed=seed)


def ragged_case(seed, kind, batch, num_q_heads, num_kv_heads, head_dim, docs_per_seq=(2, 5),
                doc_len=(1, 700), prompt=(1, 300), catalogue=None, dtype=BF16, theta=5.0e5,
                offsets="contiguous", name="ragged"):
    """Documents of any token count (their last blocks partly filled).

    A catalogue of documents (default: enough that few are shared) with
    lengths U{doc_len}, whose first entries are forced to the edge lengths 1,
    15, 16, 17, 31 and 33; each sequence draws U{docs_per_seq} distinct ones.
    Decode appends one new token per sequence; prefill a prompt of U{prompt}
    tokens.  Layout is ragged: block_fill and table-slot lengths are set.
    """
    rng = np.random.default_rng(seed)
    ncat = catalogue or batch * docs_per_seq[1]
    lens = [int(x) for x in rng.integers(doc_len[0], doc_len[1] + 1, size=ncat)]
    edge = [1, 15, 16, 17, 31, 33]
    lens[:min(len(edge), ncat)] = edge[:ncat]
    seq_docs, offs, tpos = [], [], []
    for _ in range(batch):
        k = int(rng.integers(docs_per_seq[0], docs_per_seq[1] + 1))
        seq_docs.append([int(d) for d in rng.choice(ncat, size=min(k, ncat), replace=False)])
        if offsets == "random":
            offs.append([int(x) for x in rng.integers(0, 30000, size=len(seq_docs[-1]))])
            tpos.append(int(rng.integers(0, 30000)))
    if kind == "decode":
        tails = [1] * batch
    else:
        tails = [int(x) for x in rng.integers(prompt[0], prompt[1] + 1, size=batch)]
    lay = build_layout(rng, seq_docs, lens, tails, offsets=offs if offsets == "random" else None,
                       tail_pos=tpos if offsets == "random" else None, ragged=True)
    return Case(name, kind, dtype, num_q_heads, num_kv_heads, head_dim, theta, lay, seed=seed)


def _ragged_docs(rng, total, lo, hi):
    """Document lengths U{lo..hi} tokens (any count, not whole blocks) summing to total."""
    lens = []
    left = total
    while left > 0:
        ln = min(int(rng.integers(lo, hi + 1)), left)
        lens.append(ln)
        left -= ln
    return lens


def llama8b_decode_ragged(seed=6, batch=64, ctx=8192):
    """The 8B decode shape with documents of U{256..2048} tokens, any count:
    every document's last block is partly filled (on average 7.5 unused
    slots per document), lengths are table slots."""
    rng = np.random.default_rng(seed)
    seq_docs, doc_lens = [], []
    for _ in range(batch):
        lens = _ragged_docs(rng, ctx, 256, 2048)
        seq_docs.append(list(range(len(doc_lens), len(doc_lens) + len(lens))))
        doc_lens.extend(lens)
    lay = build_layout(rng, seq_docs, doc_lens, [1] * batch, ragged=True)
    return Case("llama8b_decode_ragged", "decode", BF16, 32, 8, 128, 5.0e5, lay, seed=seed)


def llama8b_prefill_ragged(seed=7, batch=4, cached=6144, prompt=2048):
    """The 8B prefill shape with cached documents of U{256..2048} tokens, any count."""
    rng = np.random.default_rng(seed)
    seq_docs, doc_lens = [], []
    for _ in range(batch):
        lens = _ragged_docs(rng, cached, 256, 2048)
        seq_docs.append(list(range(len(doc_lens), len(doc_lens) + len(lens))))
        doc_lens.extend(lens)
    lay = build_layout(rng, seq_docs, doc_lens, [prompt] * batch, ragged=True)
    return Case("llama8b_prefill_ragged", "prefill", BF16, 32, 8, 128, 5.0e5, lay, seed=seed)


def llama8b_prefill(seed=3, batch=4, cached=6144, prompt=2048):
    """Llama-3.1-8B-shaped single-layer prefill, bf16: 32 q / 8 KV heads, d_h=128.

    4 sequences; 6144 cached document tokens (documents of 256..2048 tokens)
    followed by a 2048-token prompt at position 6144 that is appended and
    attends causally (query tiles of 128).  theta = 5e5.
    """
    return prefill_case(seed, batch, 32, 8, 128, cached, prompt, name="llama8b_prefill")


def group_decode_equal_bytes(group, seed=8):
    """Decode shapes of equal K/V bytes (~0.5 GB) that differ only in how
    many query heads share a KV head: 15 sequences x 8 KV heads for GQA 4
    (32 query heads), 120 sequences x 1 KV head for multi-query groups of 32
    or 64 (a one-head pool holds at most 65536 blocks).  8192 cached tokens
    per sequence in documents of 16*U{16..128} tokens, plus the new token;
    bf16, d_h 128, theta 5e5."""
    if group == 4:
        batch, hq, hkv = 15, 32, 8
    else:
        batch, hq, hkv = 120, group, 1
    return decode_case(seed, batch, hq, hkv, 128, 8192, (16, 128), name=f"decode_g{group}_equal_bytes")


WORKLOADS = {
    "tiny_fp32_decode": tiny_decode,
    "llama8b_decode": llama8b_decode,
    "llama8b_prefill": llama8b_prefill,
    "llama70b_decode": llama70b_decode,
    "zipf_reuse_decode": zipf_decode,
    "llama8b_decode_ragged": llama8b_decode_ragged,
    "llama8b_prefill_ragged": llama8b_prefill_ragged,
    "decode_g4_equal_bytes": lambda **kw: group_decode_equal_bytes(4, **kw),
    "decode_g32_equal_bytes": lambda **kw: group_decode_equal_bytes(32, **kw),
    "decode_g64_equal_bytes": lambda **kw: group_decode_equal_bytes(64, **kw),
}


def make(name, **kw) -> Case:
    return WORKLOADS[name](**kw)


__all__ = [
    "BLOCK", "F32", "BF16", "Case", "Layout", "build_layout", "pack_words",
    "f32_to_bf16_bits", "bf16_bits_to_f32", "to_float", "materialize_numpy",
    "materialize_torch", "add_score_shift", "decode_case", "prefill_case", "tiny_decode",
    "llama8b_decode", "llama8b_prefill", "llama70b_decode", "zipf_decode", "ragged_case",
    "llama8b_decode_ragged", "llama8b_prefill_ragged", "group_decode_equal_bytes", "e4m3_codes", "e4m3_codes_torch",
    "int8_codes", "int8_codes_torch",
    "fp8_pools_to_device_order", "fp8_pools_from_device_order", "make",
    "WORKLOADS",
]

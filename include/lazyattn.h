/*
 * lazyattn.h -- position-agnostic paged KV attention (deferred RoPE) on gfx950.
 *
 * The cache stores keys and values by content only; the rotary position of a
 * cached document is applied inside the attention kernel, so one physical copy
 * of a document serves any position without re-encoding (LazyAttention summary
 * on gist.science, sections "Metodologia" and "Equivalência Matemática").
 *
 * Data layout (all device memory, row-major, owned by the caller):
 *   K/V pool   [num_blocks][num_kv_heads][16][head_dim]   element type `dtype`
 *   table word uint32: bits 0..15 = physical block id (< num_blocks <= 65536),
 *              bits 16..31 = the block's position offset (unsigned).
 *   block_table [batch][max_blocks_per_seq] table words; table slot j of a
 *              sequence is block word[j / 16], slot j % 16.
 *   block_fill uint8 [num_blocks rounded up to a multiple of 4] or NULL:
 *              tokens stored in each physical block (0..16; larger values
 *              count as 16), the rest of the block unused -- the end of a
 *              document whose length is not a multiple of 16.  NULL means
 *              every block is full.  Slots past their block's count hold no
 *              token and are skipped; lengths (seq_lens, kv_lens) still count
 *              table slots, and a prompt's rows sit in the table's last
 *              kv_lens - q_len .. kv_lens - 1 slots.  A query that sees no
 *              token gets zeros.  Read as 32-bit words, hence the rounding.
 *              Device memory, read only.
 *
 * Position convention.  A stored key carries the rotation of its place within
 * its own frame (a document encoded from position 0, or a prompt encoded from
 * its first position); the block's offset is where that frame starts in the
 * sequence.  The key a placed token really has is therefore
 * rot(stored, offset), and a query at absolute position n scores it as
 * rot(q, n - offset) . stored.  RoPE is the rotate-half form: pairs
 * (i, i + D/2) turned by the angle p * theta^(-2i/D).  Values never rotate.
 *
 * Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL is
 * the null stream), allocate nothing, keep no device state and are
 * re-entrant.  Argument errors are reported by a negative status before any
 * launch.  Device-side preconditions (block ids < num_blocks, offsets and
 * positions < 65536) are checked
 * by the kernels where cheap: a sequence whose length is negative or exceeds
 * 16 * max_blocks_per_seq, or whose table holds a block id >= num_blocks,
 * gets NaN output instead of touching memory outside the pool.
 */
#ifndef LAZYATTN_H
#define LAZYATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LAZYATTN_BLOCK_TOKENS 16
#define LAZYATTN_MAX_BLOCKS 65536
#define LAZYATTN_MAX_POSITION 65535
/* fixed device scratch of lazyattn_decode_noalloc, per GPU: 8 MiB */
#define LAZYATTN_NOALLOC_SCRATCH_BYTES (8u << 20)

/* Element type of q, K/V pools, new rows and outputs. */
enum { LAZYATTN_F32 = 0, LAZYATTN_BF16 = 1 };

/* Status codes. */
enum {
  LAZYATTN_OK = 0,
  LAZYATTN_ERR_NULL = -1,        /* a required pointer is NULL */
  LAZYATTN_ERR_DTYPE = -2,       /* unknown dtype, or dtype not offered by this call */
  LAZYATTN_ERR_SHAPE = -3,       /* bad size: head_dim, head counts, num_blocks, ... */
  LAZYATTN_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required */
  LAZYATTN_ERR_LAUNCH = -5,      /* the HIP launch failed (hipGetLastError) */
  LAZYATTN_ERR_SCRATCH = -6      /* lazyattn_decode_noalloc: partials exceed its fixed scratch */
};

/* Text for a status code (static storage). */
const char *lazyattn_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int lazyattn_version(void);

/*
 * kvcache_append -- write new content-only K/V rows into pool slots.
 *
 * Appending the new rows of K and V to the cache before attending is the
 * cache step of lynx-cortex "00 — Por qué existe un KV Cache", section
 * "El remedio"; the per-layer, per-head append of ai-engineering.academy
 * "KV Cache, Flash Attention & Otimização de Inferência", "Construa" Passo 1.
 *
 *   k_pool, v_pool  [num_blocks][num_kv_heads][16][head_dim]   (written)
 *   k_new, v_new    [num_tokens][num_kv_heads][head_dim]       (read)
 *   slot_mapping    int32 [num_tokens]: pool slot = block_id * 16 + slot;
 *                   a slot < 0 or >= 16 * num_blocks is skipped (padding).
 * Rows are copied bit-exactly, unrotated.  head_dim in {16, 32, 64, 128, 256}.
 * num_tokens == 0 is a no-op.
 */
int kvcache_append(void *k_pool, void *v_pool, int dtype, int num_blocks, int num_kv_heads,
                   int head_dim, const void *k_new, const void *v_new,
                   const int32_t *slot_mapping, int num_tokens, void *stream);

/*
 * Bytes of workspace lazyattn_decode needs for these sizes (split_blocks as
 * passed to lazyattn_decode; 0 = automatic).  The workspace holds the per-split
 * partial results (max, sum, unnormalised output) of sequences split over
 * several workgroups; it needs no initialisation and must be 16-byte aligned
 * (LAZYATTN_ERR_WORKSPACE otherwise).  0 means the call uses none (every
 * sequence fits one split) and workspace may be NULL.  Calls that share one
 * workspace must not overlap.
 */
size_t lazyattn_decode_workspace_size(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                      int max_blocks_per_seq, int split_blocks);

/*
 * lazyattn_decode -- one new query token per sequence against its paged,
 * position-free cache (LazyAttention summary, "Implementação Técnica",
 * Decoding: the query is rotated inside the kernel only when the offset
 * changes, and only K and V are read).
 *
 *   out         [batch][num_q_heads][head_dim]  dtype      (written)
 *   q           [batch][num_q_heads][head_dim]  dtype, raw (unrotated) query
 *   q_pos       int32 [batch]: absolute position n of each query
 *   k_pool, v_pool, block_table, max_blocks_per_seq, block_fill: see the layout above
 *   seq_lens    int32 [batch]: table slots the query attends (>= 0)
 *   num_q_heads a multiple of num_kv_heads; query head h reads KV head
 *               h / (num_q_heads / num_kv_heads); the group size is a power
 *               of two up to 64 (64 covers multi-query attention with
 *               num_kv_heads = 1 and up to 64 query heads).
 *   head_dim    f32: 16, 64 or 128; bf16: 64 or 128.
 *   scale       softmax scale (usually 1/sqrt(head_dim))
 *   rope_theta  RoPE base (> 1)
 *   split_blocks blocks per split-K partition (0 = automatic; else 4..1024).
 *               A sequence longer than one partition is split over several
 *               workgroups whose partial results a second kernel merges.
 *   workspace   see lazyattn_decode_workspace_size
 *
 * out[b][h] = sum_j softmax_j(scale * rot(q, n) . rot(k_j, off_j)) v_j over the
 * seq_lens[b] tokens, computed with fp32 accumulation; a sequence with
 * seq_lens[b] == 0 gets zeros.  batch == 0 is a no-op.
 */
int lazyattn_decode(void *out, const void *q, const int32_t *q_pos, const void *k_pool,
                    const void *v_pool, const uint32_t *block_table, int max_blocks_per_seq,
                    const uint8_t *block_fill, const int32_t *seq_lens, int batch, int num_q_heads, int num_kv_heads,
                    int head_dim, int num_blocks, int dtype, float scale, float rope_theta,
                    int split_blocks, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Planned decode: lazyattn_decode with its work cut at document boundaries,
 * and the sequences that share a cached document reading it together.  One
 * physical copy of a document serves every request that places it, at any
 * position (LazyAttention summary, "Metodologia"; the Zipf-skewed reuse of
 * "Resultados Experimentais"); per-sequence decode reads that copy once per
 * sequence.  A plan cuts each sequence's table into runs; the runs of up to
 * four sequences that hold the same blocks (and for 16 / G >= 2) become one
 * work item, whose workgroup reads the blocks once for all of them (its 16
 * matrix-core columns are (sequence, query head) pairs).  The items of one
 * (document, KV head) go to one XCD in consecutive places, so that XCD's L2
 * serves the document's further readers.
 *
 * lazyattn_decode_plan (host code, host memory, no GPU): builds the plan
 * from a host copy of block_table and seq_lens.  A run ends where the table
 * offset changes once it holds 4 blocks, at max_item_blocks blocks (0 = 128),
 * and at the sequence's end; runs are shared only if they are not their
 * sequence's last and keep one offset throughout.  plan receives
 * lazyattn_decode_plan_ints ints at most: int32 [batch] run counts (the
 * partial slots per sequence), padded to a multiple of 4, then *num_items
 * items of 12 ints: KV head | members << 16, first and end block (in the
 * first member's row), 0, up to 4 members as sequence | slot << 16, and the
 * run's first block in each member's row (a shared document may sit at a
 * different place in each).  *max_items_per_seq sizes
 * the workspace.  Returns LAZYATTN_ERR_WORKSPACE if plan_ints is too small.
 * The plan depends only on the table, the lengths and the head counts.  A
 * sequence's last run ends at max_blocks_per_seq and the kernel clips it to
 * the sequence's length, so the plan stays valid while sequences grow into
 * blocks appended to their rows; rebuild it when words already in a row
 * change.
 *
 * lazyattn_decode_planned: as lazyattn_decode, with plan a device copy of
 * the plan's first (padded batch + 12 * num_items) ints, 16-byte aligned,
 * read only.  bf16 pools, head_dim 128, group sizes 1..16 (LAZYATTN_ERR_SHAPE
 * otherwise); lazy RoPE only.  The workspace (16-byte aligned, no
 * initialisation) holds max_items_per_seq partials per (sequence, KV head);
 * lazyattn_decode_planned_workspace_size gives its size (0: none needed).
 * Results match lazyattn_decode up to the order in which partials are
 * summed.  A plan for other sizes never makes the kernels read outside the
 * table, pool or workspace (items naming sequences, heads or slots outside
 * the batch, the heads or a sequence's run count are skipped, block ranges
 * are clipped to the first member's sequence), but its output is then
 * undefined.
 */
size_t lazyattn_decode_plan_ints(int batch, int max_blocks_per_seq, int num_kv_heads);
int lazyattn_decode_plan(const uint32_t *block_table, const int32_t *seq_lens, int batch,
                         int max_blocks_per_seq, int num_q_heads, int num_kv_heads, int max_item_blocks,
                         int32_t *plan, size_t plan_ints, int *num_items, int *max_items_per_seq);
size_t lazyattn_decode_planned_workspace_size(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                              int max_items_per_seq);
int lazyattn_decode_planned(void *out, const void *q, const int32_t *q_pos, const void *k_pool,
                            const void *v_pool, const uint32_t *block_table, int max_blocks_per_seq,
                            const uint8_t *block_fill, const int32_t *seq_lens, int batch, int num_q_heads,
                            int num_kv_heads, int head_dim, int num_blocks, int dtype, float scale,
                            float rope_theta, const int32_t *plan, int num_items, int max_items_per_seq,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * lazyattn_prefill -- a prompt's queries against cached documents plus the
 * prompt itself, causal within the prompt (LazyAttention summary,
 * "Implementação Técnica", Prefilling: query tiles of M = 128 rows, one
 * relative rotation per tile and document instead of two).
 *
 *   out         [total_q][num_q_heads][head_dim]  bf16            (written)
 *   q           [total_q][num_q_heads][head_dim]  bf16, raw, packed by cu_q_lens
 *   cu_q_lens   int32 [batch + 1]: prompt b is rows cu_q_lens[b] .. cu_q_lens[b+1]-1
 *   total_q     rows of q and out; a prompt whose rows fall outside [0, total_q)
 *               (or with cu_q_lens decreasing) is left unwritten
 *   q_pos_start int32 [batch]: position of prompt b's first token
 *   kv_lens     int32 [batch]: table slots INCLUDING the prompt, whose K/V
 *               must already be appended in the table's last P_b slots (in
 *               blocks of their own, full except the last)
 *   max_q_len   >= every prompt length (sizes the launch grid)
 *   num_q_heads a multiple of num_kv_heads (group size 1..64)
 *   head_dim    64 or 128; dtype must be LAZYATTN_BF16.
 *
 * Prompt row r of sequence b sits at table slot kv_lens[b] - P_b + r and
 * position q_pos_start[b] + r, and sees the stored tokens in table slots <=
 * its own (masking uses table order, never positions).  bf16 MFMA with
 * fp32 accumulation; P is rounded to bf16 for the P.V product.
 */
int lazyattn_prefill(void *out, const void *q, int total_q, const int32_t *cu_q_lens,
                     const int32_t *q_pos_start, const void *k_pool, const void *v_pool,
                     const uint32_t *block_table, int max_blocks_per_seq, const uint8_t *block_fill,
                     const int32_t *kv_lens,
                     int batch, int max_q_len, int num_q_heads, int num_kv_heads, int head_dim,
                     int num_blocks, int dtype, float scale, float rope_theta, void *stream);

/*
 * lazyattn_prefill_precise -- lazyattn_prefill for score rows that spread
 * widely across keys.  The pages trace every quality difference of the method
 * to floating-point precision (LazyAttention summary, "Resultados
 * Experimentais"); lazyattn_prefill rounds the rotated, pre-scaled query to
 * bf16 once per row and document, so a score moves by up to ~|s| * 2^-9 and
 * rows whose scores differ by more than a few units lose accuracy.  Here the
 * query reaches the matrix cores as bf16 hi + lo (~2^-17), and K/V tiles end
 * where the document offset changes, so stored keys are used as they are
 * (never rotated and rounded).  The error then no longer grows with the score
 * spread; the price is twice the Q.K^T products.
 *
 * Same arguments, layout, ownership and error codes as lazyattn_prefill.
 */
int lazyattn_prefill_precise(void *out, const void *q, int total_q, const int32_t *cu_q_lens,
                             const int32_t *q_pos_start, const void *k_pool, const void *v_pool,
                             const uint32_t *block_table, int max_blocks_per_seq, const uint8_t *block_fill,
                             const int32_t *kv_lens, int batch, int max_q_len, int num_q_heads,
                             int num_kv_heads, int head_dim, int num_blocks, int dtype, float scale,
                             float rope_theta, void *stream);

/*
 * lazyattn_decode_noalloc -- lazyattn_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, layout, results and
 * error codes as lazyattn_decode, without the workspace: the split-K
 * partials live in a fixed array of LAZYATTN_NOALLOC_SCRATCH_BYTES in device
 * memory that the library holds on each GPU it runs on until the process
 * ends.  The call itself allocates nothing (no hipMalloc/hipFree).
 *
 *   Sizes whose partials need more than LAZYATTN_NOALLOC_SCRATCH_BYTES
 *   (lazyattn_decode_workspace_size with the same arguments) are rejected
 *   with LAZYATTN_ERR_SCRATCH before any launch; so is a device whose
 *   scratch address cannot be obtained.  The current HIP device must be the
 *   one the pointers and the stream belong to.
 *   All calls on one GPU share that GPU's scratch, which keeps the last
 *   call's partials (every partial is written before it is read, so nothing
 *   needs clearing): calls that overlap on one GPU (other streams, other
 *   threads) race and must be serialised by the caller.
 */
int lazyattn_decode_noalloc(void *out, const void *q, const int32_t *q_pos, const void *k_pool,
                            const void *v_pool, const uint32_t *block_table, int max_blocks_per_seq,
                            const uint8_t *block_fill, const int32_t *seq_lens, int batch, int num_q_heads,
                            int num_kv_heads, int head_dim, int num_blocks, int dtype, float scale,
                            float rope_theta, int split_blocks, void *stream);

/*
 * lazyattn_decode_eager, lazyattn_prefill_eager -- the non-lazy baseline that
 * the method's overhead is measured against (LazyAttention summary,
 * "Declaração do Problema": conventional caches hold keys already rotated to
 * their place in the sequence, and reuse at a new place means re-encoding or
 * re-rotating them).  Same arguments, layout, ownership and error codes as
 * lazyattn_decode / lazyattn_prefill, with one difference in meaning: the
 * pool's keys are taken as already rotated to their absolute positions, the
 * offset half of every table word is ignored, and each query is rotated once
 * by its own position.  Equivalently: the lazy call on a table whose offsets
 * are all 0.
 */
int lazyattn_decode_eager(void *out, const void *q, const int32_t *q_pos, const void *k_pool,
                          const void *v_pool, const uint32_t *block_table, int max_blocks_per_seq,
                          const uint8_t *block_fill, const int32_t *seq_lens, int batch, int num_q_heads, int num_kv_heads,
                          int head_dim, int num_blocks, int dtype, float scale, float rope_theta,
                          int split_blocks, void *workspace, size_t workspace_bytes, void *stream);

int lazyattn_prefill_eager(void *out, const void *q, int total_q, const int32_t *cu_q_lens,
                           const int32_t *q_pos_start, const void *k_pool, const void *v_pool,
                           const uint32_t *block_table, int max_blocks_per_seq, const uint8_t *block_fill,
                           const int32_t *kv_lens, int batch, int max_q_len, int num_q_heads,
                           int num_kv_heads, int head_dim, int num_blocks, int dtype, float scale,
                           float rope_theta, void *stream);

/*
 * lazyattn_decode_alibi, lazyattn_prefill_alibi -- the same attention with
 * ALiBi linear biases instead of RoPE (the LazyAttention summary on
 * gist.science, "Principais Contribuições" 4, names ALiBi among the position
 * schemes deferred lazily).  Nothing rotates: the score of query position n
 * against a key at position p is scale * q . k + slopes[h] * (p - n) for query
 * head h.  Keys and values are stored by content only, as for RoPE; since no
 * position is baked into a stored key, each block's table word carries the
 * absolute position of the block's first token in its offset half, and the
 * token in slot s sits at offset + s (a block frame).
 *   slopes  [num_q_heads] float32, device, read only; e.g. 2^(-8 (h+1) / Hq).
 * Every other argument, layout, ownership and status code is that of
 * lazyattn_decode / lazyattn_prefill (rope_theta is not taken); slopes NULL
 * gives LAZYATTN_ERR_NULL.
 */
int lazyattn_decode_alibi(void *out, const void *q, const int32_t *q_pos, const void *k_pool,
                          const void *v_pool, const uint32_t *block_table, int max_blocks_per_seq,
                          const uint8_t *block_fill, const int32_t *seq_lens, const float *slopes, int batch, int num_q_heads,
                          int num_kv_heads, int head_dim, int num_blocks, int dtype, float scale,
                          int split_blocks, void *workspace, size_t workspace_bytes, void *stream);

int lazyattn_prefill_alibi(void *out, const void *q, int total_q, const int32_t *cu_q_lens,
                           const int32_t *q_pos_start, const void *k_pool, const void *v_pool,
                           const uint32_t *block_table, int max_blocks_per_seq, const uint8_t *block_fill,
                           const int32_t *kv_lens,
                           const float *slopes, int batch, int max_q_len, int num_q_heads,
                           int num_kv_heads, int head_dim, int num_blocks, int dtype, float scale,
                           void *stream);

/*
 * 8-bit KV pools.  The pages name a one-byte KV cache without defining it
 * (ai-engineering.academy "KV Cache, Flash Attention & Otimização de
 * Inferência", section "Use-o": serving with an fp8 KV-cache dtype;
 * lynx-cortex "00 — Por qué existe un KV Cache", "El precio": one byte per
 * element).  Here a pool element is an OCP FP8 E4M3 code (1 sign, 4 exponent
 * bits with bias 7, 3 mantissa bits, subnormals, no infinities, S.1111.111 =
 * NaN, largest magnitude 448) with one float scale per tensor: the value a
 * code stands for is decode(code) * scale.  head_dim is 128.  Each
 * (block, KV head) record is 2048 bytes at [num_blocks][num_kv_heads] as in the
 * bf16 pool, with its codes in the lane order of the matrix-core decode: for
 * half i < 2, lane l = 16 g + t < 64 and x < 16, byte 1024 i + 16 l + x holds
 *   K: token t, dim 32 g + 16 i + x
 *   V: token 4 g + x % 4, dim 16 (4 i + x / 4) + t
 * so that every wave load reads 1 KiB contiguously and feeds the matrix cores
 * without exchanging data between lanes.  kvcache_append_fp8 writes this order.
 *
 * kvcache_append_fp8 -- kvcache_append into 8-bit pools.  k_new/v_new are
 * `dtype` rows (LAZYATTN_F32 or LAZYATTN_BF16).  Each element is stored as the
 * E4M3 code nearest to the float32 quotient x / scale (correctly rounded
 * division), ties to an even mantissa, magnitudes above 448 saturating to
 * +-448, NaN as 0x7F.  k_scale, v_scale must be finite and > 0, head_dim
 * 128 (LAZYATTN_ERR_SHAPE otherwise).  Other arguments as kvcache_append.
 */
int kvcache_append_fp8(void *k_pool, void *v_pool, int dtype, int num_blocks, int num_kv_heads,
                       int head_dim, const void *k_new, const void *v_new, const int32_t *slot_mapping,
                       int num_tokens, float k_scale, float v_scale, void *stream);

/*
 * lazyattn_decode_fp8 -- lazyattn_decode (lazy RoPE) against 8-bit pools:
 * keys are decode(code) * k_scale, values decode(code) * v_scale.  q and out
 * are bf16; head_dim must be 128; any power-of-two group up to 64 (up to 16
 * query heads per workgroup).  Reads one byte per K/V element, half of the
 * bf16 pool's traffic.  The workspace is sized by
 * lazyattn_decode_workspace_size with the same arguments.  Other arguments
 * and errors as lazyattn_decode.
 */
int lazyattn_decode_fp8(void *out, const void *q, const int32_t *q_pos, const void *k_pool,
                        const void *v_pool, const uint32_t *block_table, int max_blocks_per_seq,
                        const uint8_t *block_fill, const int32_t *seq_lens, int batch, int num_q_heads,
                        int num_kv_heads, int head_dim, int num_blocks, float scale, float rope_theta,
                        float k_scale, float v_scale, int split_blocks, void *workspace,
                        size_t workspace_bytes, void *stream);

/*
 * lazyattn_prefill_fp8_workspace_size -- bytes of workspace lazyattn_prefill_fp8
 * needs: a bf16 copy (K and V) of every block slot of the batch,
 * 2 * batch * max_blocks_per_seq * num_kv_heads * 16 * 128 * 2 bytes.  0 when
 * head_dim is not 128 or a count is not positive.
 */
size_t lazyattn_prefill_fp8_workspace_size(int batch, int max_blocks_per_seq, int num_kv_heads, int head_dim);

/*
 * lazyattn_prefill_fp8 -- lazyattn_prefill (lazy RoPE) against 8-bit pools
 * written by kvcache_append_fp8: keys are decode(code) * k_scale, values
 * decode(code) * v_scale.  This is the step that reuses cached documents for
 * a new prompt (LazyAttention summary on gist.science, "Implementação
 * Técnica", Prefilling) over the one-byte cache (ai-engineering.academy,
 * "Use-o"; lynx-cortex "00", "El precio").  A first pass widens each block
 * the batch can see, once and exactly, into the caller's workspace
 * (lazyattn_prefill_fp8_workspace_size bytes, device memory the call
 * overwrites; its previous contents are irrelevant), and the prefill then
 * reads that bf16 copy: each block is widened once instead of once per query
 * tile that reads it.  q and out are bf16 [total_q][num_q_heads][128];
 * head_dim must be 128; k_scale and v_scale finite and > 0
 * (LAZYATTN_ERR_SHAPE otherwise); a missing or short workspace gives
 * LAZYATTN_ERR_WORKSPACE before any launch.  Other arguments, layouts and
 * errors as lazyattn_prefill.
 */
int lazyattn_prefill_fp8(void *out, const void *q, int total_q, const int32_t *cu_q_lens,
                         const int32_t *q_pos_start, const void *k_pool, const void *v_pool,
                         const uint32_t *block_table, int max_blocks_per_seq, const uint8_t *block_fill,
                         const int32_t *kv_lens, int batch, int max_q_len, int num_q_heads, int num_kv_heads,
                         int head_dim, int num_blocks, float scale, float rope_theta, float k_scale,
                         float v_scale, void *workspace, size_t workspace_bytes, void *stream);

/*
 * int8 KV pools: the same one-byte cache (lynx-cortex "00 — Por qué existe un
 * KV Cache", "El precio": s = 1 for int8) with symmetric signed integer codes
 * and one float scale per tensor: the value a code stands for is
 * code * scale.  Same record layout and lane order as the 8-bit E4M3 pools
 * above, head_dim 128.
 *
 * kvcache_append_int8 -- each element is stored as the integer nearest to the
 * float32 quotient x / scale (correctly rounded division), ties to even,
 * clamped to [-127, 127] (-128 is never written; infinities clamp), NaN as 0.
 * Arguments and errors as kvcache_append_fp8.
 *
 * lazyattn_decode_int8, lazyattn_prefill_int8 -- lazyattn_decode_fp8 and
 * lazyattn_prefill_fp8 over int8 pools: keys are code * k_scale, values
 * code * v_scale (a code of -128, which the append never writes, reads as
 * -128).  The widening for the prefill is exact; its workspace is
 * lazyattn_prefill_fp8_workspace_size bytes.  Arguments, workspaces and errors
 * as the E4M3 calls.
 */
int kvcache_append_int8(void *k_pool, void *v_pool, int dtype, int num_blocks, int num_kv_heads,
                        int head_dim, const void *k_new, const void *v_new, const int32_t *slot_mapping,
                        int num_tokens, float k_scale, float v_scale, void *stream);
int lazyattn_decode_int8(void *out, const void *q, const int32_t *q_pos, const void *k_pool,
                         const void *v_pool, const uint32_t *block_table, int max_blocks_per_seq,
                         const uint8_t *block_fill, const int32_t *seq_lens, int batch, int num_q_heads,
                         int num_kv_heads, int head_dim, int num_blocks, float scale, float rope_theta,
                         float k_scale, float v_scale, int split_blocks, void *workspace,
                         size_t workspace_bytes, void *stream);
int lazyattn_prefill_int8(void *out, const void *q, int total_q, const int32_t *cu_q_lens,
                          const int32_t *q_pos_start, const void *k_pool, const void *v_pool,
                          const uint32_t *block_table, int max_blocks_per_seq, const uint8_t *block_fill,
                          const int32_t *kv_lens, int batch, int max_q_len, int num_q_heads, int num_kv_heads,
                          int head_dim, int num_blocks, float scale, float rope_theta, float k_scale,
                          float v_scale, void *workspace, size_t workspace_bytes, void *stream);

/*
 * lazyattn_prefill_fp8_precise, lazyattn_prefill_int8_precise -- the 8-bit
 * prefills with the rotated query carried as bf16 hi + lo and K/V tiles cut
 * where the document offset changes, as lazyattn_prefill_precise does for
 * bf16 pools (LazyAttention summary, "Resultados Experimentais": quality
 * differences come down to floating-point precision).  A large K scale
 * spreads a row's scores the way large keys do; these calls stay within
 * tolerance there.  Same arguments, workspace, layout and errors as
 * lazyattn_prefill_fp8 / lazyattn_prefill_int8.
 */
int lazyattn_prefill_fp8_precise(void *out, const void *q, int total_q, const int32_t *cu_q_lens,
                                 const int32_t *q_pos_start, const void *k_pool, const void *v_pool,
                                 const uint32_t *block_table, int max_blocks_per_seq, const uint8_t *block_fill,
                                 const int32_t *kv_lens, int batch, int max_q_len, int num_q_heads,
                                 int num_kv_heads, int head_dim, int num_blocks, float scale, float rope_theta,
                                 float k_scale, float v_scale, void *workspace, size_t workspace_bytes,
                                 void *stream);
int lazyattn_prefill_int8_precise(void *out, const void *q, int total_q, const int32_t *cu_q_lens,
                                  const int32_t *q_pos_start, const void *k_pool, const void *v_pool,
                                  const uint32_t *block_table, int max_blocks_per_seq, const uint8_t *block_fill,
                                  const int32_t *kv_lens, int batch, int max_q_len, int num_q_heads,
                                  int num_kv_heads, int head_dim, int num_blocks, float scale, float rope_theta,
                                  float k_scale, float v_scale, void *workspace, size_t workspace_bytes,
                                  void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LAZYATTN_H */

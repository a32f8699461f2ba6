// lazyattn_decode: one query token per sequence against a paged, position-free
// KV cache, split-K over 16-token blocks (flash-decoding).
//
// Method (LazyAttention summary on gist.science, "Implementação Técnica",
// Decoding): the cached keys carry no placement, so the rotation for a
// document's offset is applied to the *query*, and only when the offset
// changes (a new document); the kernel reads K and V exactly once and, per
// block, only the packed (block id, offset) word besides.  The scores
// rot(q, n - off) . k equal rot(q, n) . rot(k, off) ("Equivalência
// Matemática"), i.e. attention against the eager position-adjusted copy.
// Softmax is the running (max, sum) form of ai-engineering.academy
// "Flash Attention" (the numerical trick), kept per lane stream and merged at
// the end of each split, then across splits.
//
// Two kernels.  bf16 pools with head_dim 128 (and 8-bit pools) run on the
// matrix cores (decode_mma16_kernel, decode_mma8_kernel, described where they
// are defined); fp32 pools and head_dim 64 run on the VALU
// (decode_split_kernel).  Both walk a sequence's 16-token blocks split-K
// (flash-decoding); a sequence split over several workgroups writes per-split
// (max, sum, unnormalised output) to the workspace and a second, small kernel
// merges them (log-sum-exp).  The kernel boundary orders the two; no
// device-scope fence is used (on gfx950 one costs an L2 write-back).  A
// sequence with one split writes its output directly.
//
// VALU kernel, gfx950 mapping (wave64):
//   * A K (or V) block of one KV head is 16 rows x D contiguous elements.  A
//     lane loads 16-byte chunks; LPT = D / (16 B / elem) lanes cover one row,
//     so one dwordx4 load instruction reads 64 * 16 B = 1 KiB of the block
//     contiguously, and NI instructions cover the block.
//   * Each lane holds the rotated query slice for its chunk's dims for all G
//     query heads of the KV head (grouped-query attention).  For bf16 the
//     slice is kept as packed bf16 pairs and both products use
//     v_dot2_f32_bf16 (two multiply-adds per instruction, fp32 accumulate):
//     Q.K pairs along the head dimension, P.V pairs two token rows (P rounded
//     to bf16, as the MFMA prefill does).  Partial dot products are summed
//     over the LPT lanes of a row with DPP (quad perms, row mirrors).
//   * A lane keeps its own running max/sum per head over the rows it sees, so a
//     block needs no cross-lane max; the rows are merged once per split.  The
//     max is only raised when a block exceeds it by more than 2^8 (values stay
//     bounded by 256), which skips almost every rescale of the accumulators.
//   * The next block's K/V loads are issued before the current block is
//     computed.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace lazyattn {

constexpr int kDecodeWaves = 4;
constexpr int kXcds = 8;
constexpr float kRescaleSlack = 8.0f;  // in log2 units
constexpr float kMaxFloor = -0x1p127f;  // below any finite score that does not overflow

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kPerChunk = 4;
  static __device__ __forceinline__ float load(const float *p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float *p, size_t i, float x) { p[i] = x; }
};
template <>
struct Elem<bf16> {
  static constexpr int kPerChunk = 8;
  static __device__ __forceinline__ float load(const bf16 *p, size_t i) {
    return __uint_as_float((uint32_t)p[i].bits << 16);
  }
  static __device__ __forceinline__ void store(bf16 *p, size_t i, float x) {
    p[i].bits = to_bf16_bits(x);
  }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

struct DecodeKernelArgs {
  void *out;
  const void *q;
  const int32_t *q_pos;
  const uint4 *k_pool;
  const uint4 *v_pool;
  const uint32_t *table;
  const int32_t *seq_lens;
  const float *slopes;  // ALiBi: per query head
  const uint32_t *fill4;  // per-block fill counts, 4 per word (nullptr: all full)
  float *ws_o;    // [B][Hkv][S][G][D]
  float2 *ws_ml;  // [B][Hkv][S][G] (max, sum)
  int max_blocks;
  int num_kv_heads;  // work heads: KV heads x head split (each takes G query heads)
  int kv_shift;      // log2 of the head split
  int num_units;     // splits x KV heads x batch, or the plan's item count
  int num_blocks, split_blocks, max_splits;
  float scale_log2, rope_theta;
  float out_scale;   // V scale of an 8-bit pool (1 otherwise)
  // A work plan (planned decode): per-sequence slot counts, and the items
  // (kPlanInts ints each) that workgroup i takes; nullptr otherwise.
  const int4 *plan_items;
  const int32_t *plan_counts;
  int batch;
};

// The share of the decode a workgroup takes: sequence b, work head g, split
// `split` of `nsplit`, blocks [blk0, blk1) of the sequence's table (nblk of
// them in all).  Returns false for a workgroup past the last unit.
struct DecodeShare {
  int b, g, split, nsplit, blk0, blk1, nblk, seq_len;
  bool bad_len;
};
__device__ __forceinline__ bool decode_share(const DecodeKernelArgs &a, DecodeShare &w) {
  // Work item -> (split, KV head, sequence).  A KV head whose query heads are
  // split over 2^kv_shift workgroups gives them consecutive slots on one XCD
  // (workgroups go round-robin over the XCDs), so they run side by side and
  // the twin reads of each K/V block are served by that XCD's L2.
  const int hkv = a.num_kv_heads;
  const int slot = blockIdx.x / kXcds;
  const int hsub = slot & ((1 << a.kv_shift) - 1);
  const int unit = (slot >> a.kv_shift) * kXcds + (int)(blockIdx.x % kXcds);
  if (unit >= a.num_units) return false;
  const int hkv_pool = hkv >> a.kv_shift;
  w.split = unit % a.max_splits;
  const int gp = (unit / a.max_splits) % hkv_pool;  // KV head in the pool
  w.b = unit / a.max_splits / hkv_pool;
  w.g = (gp << a.kv_shift) | hsub;                  // work head: query heads g*G .. g*G+G-1
  w.seq_len = a.seq_lens[w.b];
  w.bad_len = w.seq_len < 0 || w.seq_len > a.max_blocks * kBlockTokens;
  w.nblk = w.bad_len ? 0 : (w.seq_len + kBlockTokens - 1) / kBlockTokens;
  w.nsplit = (w.nblk + a.split_blocks - 1) / a.split_blocks;
  w.blk0 = w.split * a.split_blocks;
  w.blk1 = min(w.blk0 + a.split_blocks, w.nblk);
  w.blk0 = min(w.blk0, w.blk1);
  return true;
}

// MODE kRopeEager: the non-lazy baseline the method is measured against.  The
// pool then holds keys already rotated to their absolute positions (the eager,
// position-adjusted copy), table offsets are ignored, and the query is rotated
// once by its own position.
// MODE kAlibi: no rotation at all; the score of a key at position p (block
// offset + slot) takes the bias slope_h * (p - n) of query head h.
template <typename T, int D, int G, int MODE>
__global__ void __launch_bounds__(kDecodeWaves * kWave)
decode_split_kernel(const DecodeKernelArgs a) {
  using E = Elem<T>;
  constexpr bool kBf16 = sizeof(T) == 2;
  constexpr bool EAGER = MODE == kRopeEager;
  constexpr bool ALIBI = MODE == kAlibi;
  constexpr int EPL = E::kPerChunk;  // pool elements per 16-byte chunk
  constexpr int LPT = D / EPL;             // lanes per token row
  constexpr int TPI = kWave / LPT;         // token rows per load instruction
  constexpr int NI = kBlockTokens / TPI;   // load instructions per block
  constexpr int HALF = D / 2;
  constexpr int NT = kDecodeWaves * kWave;
  static_assert(LPT >= 4 && LPT <= kWave && TPI <= kBlockTokens, "unsupported head geometry");
  static_assert(!kBf16 || NI % 2 == 0, "bf16 P.V pairs token rows");

  __shared__ float s_q[G][D];
  __shared__ float s_m[kDecodeWaves][G];
  __shared__ float s_l[kDecodeWaves][G];
  __shared__ float s_o[kDecodeWaves][G][D];
  __shared__ int s_bad;

  // Work item -> (split, KV head, sequence).  A KV head whose query heads are
  // split over 2^kv_shift workgroups gives them consecutive slots on one XCD
  // (workgroups go round-robin over the XCDs), so they run side by side and
  // the twin reads of each K/V block are served by that XCD's L2.
  const int hkv = a.num_kv_heads;
  const int slot = blockIdx.x / kXcds;
  const int hsub = slot & ((1 << a.kv_shift) - 1);
  const int unit = (slot >> a.kv_shift) * kXcds + (int)(blockIdx.x % kXcds);
  if (unit >= a.num_units) return;
  const int hkv_pool = hkv >> a.kv_shift;
  const int split = unit % a.max_splits;
  const int gp = (unit / a.max_splits) % hkv_pool;    // KV head in the pool
  const int b = unit / a.max_splits / hkv_pool;
  const int g = (gp << a.kv_shift) | hsub;            // work head: query heads g*G .. g*G+G-1
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform: SGPR
  const int hq = hkv * G;

  const int seq_len = a.seq_lens[b];
  const bool bad_len = seq_len < 0 || seq_len > a.max_blocks * kBlockTokens;
  const int nblk = bad_len ? 0 : (seq_len + kBlockTokens - 1) / kBlockTokens;
  const int nsplit = (nblk + a.split_blocks - 1) / a.split_blocks;
  T *out = (T *)a.out + ((size_t)b * hq + (size_t)g * G) * D;

  if (nsplit == 0) {  // empty sequence -> zeros; invalid length -> NaN
    if (split == 0)
      for (int i = tid; i < G * D; i += NT) E::store(out, i, bad_len ? __builtin_nanf("") : 0.f);
    return;
  }
  if (split >= nsplit) return;

  const T *qg = (const T *)a.q + ((size_t)b * hq + (size_t)g * G) * D;
  for (int i = tid; i < G * D; i += NT) s_q[i / D][i % D] = E::load(qg, i);
  if (tid == 0) s_bad = 0;
  __syncthreads();

  const int n_pos = a.q_pos[b];
  const int c = lane % LPT;
  const int r = lane / LPT;
  const int d0 = c * EPL;
  const bool upper = d0 >= HALF;
  const int pd0 = upper ? d0 - HALF : d0 + HALF;
  const double inv_freq = lane < HALF ? rope_inv_freq(lane, D, a.rope_theta) : 0.0;

  // rotated, pre-scaled query slice: packed bf16 pairs as hi + lo parts (bf16;
  // see split_bf16x2), or floats (f32)
  uint32_t qp[G][EPL / 2], ql[G][kBf16 ? EPL / 2 : 1];
  float qf[G][kBf16 ? 1 : EPL];
  float acc[G][EPL];
  float m[G], l[G];
  // Running maxima start at a finite floor far below any score: the first
  // block with a finite score always rescales (alpha = 2^(floor - max) = 0),
  // masked scores (-inf) give p = 0, and p needs no guard against -inf - -inf.
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kMaxFloor;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  const int blk0 = split * a.split_blocks;
  const int blk1 = min(nblk, blk0 + a.split_blocks);
  const uint32_t *trow = a.table + (size_t)b * a.max_blocks;
  constexpr size_t kChunksPerHeadBlock = (size_t)kBlockTokens * LPT;
  bool bad = false;
  int cur_off = -1;

  // Loads block bk's K/V and returns in w its table word with the block id
  // replaced by the block's fill count (the id is not needed afterwards; the
  // offset stays in the high half).
  auto issue = [&](int bk, uint32_t &w, uint4 (&kk)[NI], uint4 (&vv)[NI]) {
    w = trow[bk];
    uint32_t id = word_block(w);
    if (id >= (uint32_t)a.num_blocks) {  // table points outside the pool
      bad = true;
      id = 0;
    }
    const uint32_t fill = a.fill4 ? (a.fill4[id >> 2] >> ((id & 3u) * 8u)) & 0xffu : (uint32_t)kBlockTokens;
    w = (w & 0xffff0000u) | fill;
    // wave-uniform block base (scalar registers) + a 32-bit lane offset
    const size_t hb = ((size_t)id * hkv_pool + gp) * kChunksPerHeadBlock;
    const uint4 *kb = a.k_pool + hb;
    const uint4 *vb = a.v_pool + hb;
#pragma unroll
    for (int i = 0; i < NI; ++i) kk[i] = kb[lane + i * kWave];
#pragma unroll
    for (int i = 0; i < NI; ++i) vv[i] = vb[lane + i * kWave];
  };

  // q' = rot(q, n - off) * scale * log2(e), for this lane's dims and all G heads.
  // Lane i < D/2 evaluates frequency i once; the values are shuffled to the
  // lanes holding dims i and i + D/2.  bf16: the angle is reduced in double to
  // a fraction of a turn and evaluated with v_cos/v_sin (which take turns), light
  // on registers (this runs inside the block loop).  f32: double-precision
  // cos/sin.
  auto rotate = [&](int delta) {
    float cs = 1.f, sn = 0.f;
    if (lane < HALF) {
      if constexpr (kBf16) {
        const double t = (double)delta * (inv_freq * 0.15915494309189535);
        const float f = (float)(t - rint(t));
        cs = __builtin_amdgcn_cosf(f);
        sn = __builtin_amdgcn_sinf(f);
      } else {
        rope_cos_sin(delta, inv_freq, cs, sn);
      }
    }
    float ce[EPL], se[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int fi = (d0 + e) % HALF;
      ce[e] = __shfl(cs, fi);
      se[e] = __shfl(sn, fi);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float rot[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float x = s_q[h][d0 + e];
        const float y = s_q[h][pd0 + e];
        rot[e] = (upper ? fmaf(x, ce[e], y * se[e]) : fmaf(x, ce[e], -(y * se[e]))) * a.scale_log2;
      }
      if constexpr (kBf16) {
#pragma unroll
        for (int w = 0; w < EPL / 2; ++w) split_bf16x2(rot[2 * w], rot[2 * w + 1], qp[h][w], ql[h][w]);
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) qf[h][e] = rot[e];
      }
    }
  };

  // Two register sets for K/V take turns as "current" and "next" block: the
  // loop body runs twice per iteration with their roles swapped, so no
  // registers are copied between blocks.  The second pass of the last
  // iteration may find no block left (blk >= blk1); it then masks every row
  // (the partial-block path) and adds nothing.
  // Loads are issued unconditionally (a conditional load would make the
  // compiler copy the landed registers, i.e. wait for them, right after
  // issuing): past the split's last block they re-read that block (an L2 hit)
  // and the step that takes it masks every row.
  int blk = blk0 + wave;
  const int blast = blk1 - 1;  // >= blk0: a split has at least one block
  uint32_t wA = 0, wB = 0;
  uint4 kA[NI], vA[NI], kB[NI], vB[NI];
  issue(min(blk, blast), wA, kA, vA);
  if constexpr (EAGER) rotate(n_pos);
  if constexpr (ALIBI) rotate(0);  // the identity: q * scale * log2(e)
  // ALiBi: slopes of this workgroup's heads, in log2 units
  float slope2[ALIBI ? G : 1];
  if constexpr (ALIBI) {
#pragma unroll
    for (int h = 0; h < G; ++h) slope2[h] = a.slopes[g * G + h] * kLog2e;
  }
  auto step = [&](const uint32_t &wcur, uint4 (&kc)[NI], uint4 (&vc)[NI], uint32_t &wn, uint4 (&kn)[NI],
                  uint4 (&vn)[NI]) {
    // a new document: re-rotate the query (the lazy rotation).  Done before
    // the next block's loads are issued, so that the rotation's temporaries
    // never share registers with loads in flight.
    if constexpr (MODE == kRopeLazy) {
      const int off = word_offset(wcur);
      if (off != cur_off && blk < blk1) {
        rotate(n_pos - off);
        cur_off = off;
      }
    }
    const int nb = blk + kDecodeWaves;
    issue(min(nb, blast), wn, kn, vn);

    // scores (log2 units) of this lane's NI rows for every head
    float s[NI][G];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float t;
        if constexpr (kBf16) {
          t = dot2_bf16(qp[h][0], dw4(kc[i], 0), 0.f);
#pragma unroll
          for (int w = 1; w < EPL / 2; ++w) t = dot2_bf16(qp[h][w], dw4(kc[i], w), t);
#pragma unroll
          for (int w = 0; w < EPL / 2; ++w) t = dot2_bf16(ql[h][w], dw4(kc[i], w), t);
        } else {
          t = qf[h][0] * __uint_as_float(dw4(kc[i], 0));
#pragma unroll
          for (int w = 1; w < EPL; ++w) t = fmaf(qf[h][w], __uint_as_float(dw4(kc[i], w)), t);
        }
        s[i][h] = t;
      }
    }
    // sum the partial products over the LPT lanes of each row, one DPP step at
    // a time over all NI*G values (independent neighbours: no wait states)
    group_sum_all<LPT, NI * G>(&s[0][0]);
    if constexpr (ALIBI) {  // key position - query position, per row of this lane
      const float base = (float)(word_offset(wcur) + r - n_pos);
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int h = 0; h < G; ++h) s[i][h] = fmaf(slope2[h], base + (float)(i * TPI), s[i][h]);
    }
    // rows of this block that count: its fill count, the sequence's length in
    // its last block, none once the split is exhausted (blk >= blk1: a
    // re-read block)
    const int nvalid = blk < blk1 ? min(seq_len - blk * kBlockTokens, (int)(wcur & 0xffffu)) : 0;
    if (nvalid < kBlockTokens) {  // partly filled or exhausted
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        if (i * TPI + r >= nvalid) {
#pragma unroll
          for (int h = 0; h < G; ++h) s[i][h] = -INFINITY;
          vc[i] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
    }

    float bm[G];
    bool need = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if constexpr (NI == 4) {
        bm[h] = max4_nn(s[0][h], s[1][h], s[2][h], s[3][h]);
      } else {
        bm[h] = s[0][h];
#pragma unroll
        for (int i = 1; i < NI; ++i) bm[h] = fmaxf(bm[h], s[i][h]);
      }
      need |= bm[h] > m[h] + kRescaleSlack;
    }
    if (wave_any(need)) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mn = fmaxf(m[h], bm[h]);
        const float alpha = fast_exp2(m[h] - mn);  // 0 on the first rescale
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
        m[h] = mn;
      }
    }

    float p[NI][G];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < NI; ++i) p[i][h] = fast_exp2(s[i][h] - m[h]);
    if constexpr (kBf16) {
      // P.V pairs token rows i, i+1; the row sums take the same bf16-rounded
      // weights that P.V uses
#pragma unroll
      for (int i = 0; i < NI; i += 2) {
        uint32_t pp[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          pp[h] = pack_bf16x2(p[i][h], p[i + 1][h]);
          l[h] = dot2_bf16(pp[h], 0x3f803f80u, l[h]);
        }
#pragma unroll
          for (int w = 0; w < EPL / 2; ++w) {
            const uint32_t v0 = dw4(vc[i], w), v1 = dw4(vc[i + 1], w);
            const uint32_t lo = __builtin_amdgcn_perm(v1, v0, 0x05040100u);  // dim 2w of rows i, i+1
            const uint32_t hi = __builtin_amdgcn_perm(v1, v0, 0x07060302u);  // dim 2w+1
#pragma unroll
            for (int h = 0; h < G; ++h) {
              acc[h][2 * w] = dot2_bf16(pp[h], lo, acc[h][2 * w]);
              acc[h][2 * w + 1] = dot2_bf16(pp[h], hi, acc[h][2 * w + 1]);
            }
          }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int h = 0; h < G; ++h) {
          l[h] += p[i][h];
#pragma unroll
          for (int e = 0; e < EPL; ++e)
            acc[h][e] = fmaf(p[i][h], __uint_as_float(dw4(vc[i], e)), acc[h][e]);
        }
    }
    blk = nb;
  };
  while (blk < blk1) {
    step(wA, kA, vA, wB, kB, vB);
    step(wB, kB, vB, wA, kA, vA);
  }

  // merge the TPI row streams of this wave (lanes with equal c)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mx = m[h];
#pragma unroll
    for (int x = LPT; x < kWave; x <<= 1) mx = fmaxf(mx, __shfl_xor(mx, x));
    const float f = mx == -INFINITY ? 0.f : fast_exp2(m[h] - mx);
    float lw = l[h] * f;
#pragma unroll
    for (int x = LPT; x < kWave; x <<= 1) lw += __shfl_xor(lw, x);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float v = acc[h][e] * f;
#pragma unroll
      for (int x = LPT; x < kWave; x <<= 1) v += __shfl_xor(v, x);
      acc[h][e] = v;
    }
    m[h] = mx;
    l[h] = lw;
  }
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_o[wave][h][d0 + e] = acc[h][e];
      if (c == 0) {
        s_m[wave][h] = m[h];
        s_l[wave][h] = l[h];
      }
    }
  }
  if (bad) s_bad = 1;
  __syncthreads();

  // merge the waves; one split -> final output, else a partial for the combine kernel
  const bool single = nsplit == 1;
  const bool flagged = s_bad != 0;
  const size_t part = ((size_t)b * hkv + g) * a.max_splits + split;
  for (int i = tid; i < G * D; i += NT) {
    const int h = i / D, d = i % D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) mx = fmaxf(mx, s_m[w][h]);
    float o = 0.f, lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      const float f = s_m[w][h] == -INFINITY ? 0.f : fast_exp2(s_m[w][h] - mx);
      o = fmaf(s_o[w][h][d], f, o);
      lsum = fmaf(s_l[w][h], f, lsum);
    }
    if (flagged) {
      o = __builtin_nanf("");
      lsum = __builtin_nanf("");
    }
    if (single) {
      E::store(out, i, lsum != 0.f ? o / lsum * a.out_scale : 0.f);  // no visible token -> 0 (NaN stays NaN)
    } else {
      a.ws_o[part * G * D + i] = o;
      if (d == 0) a.ws_ml[part * G + h] = make_float2(mx, lsum);
    }
  }
}

// ---------------------------------------------------------------------------
// 8-bit pools on the matrix cores.  With one byte per element the VALU form
// above runs out of issue slots before HBM does (its dot products, row sums and
// conversions cost ~240 VALU instructions per block and wave, and the block
// arrives in half the time), so here the two contractions of a block go to
// MFMA: S = K.q'^T as 4 x v_mfma_f32_16x16x32_bf16 (16 tokens x up to 16 query
// heads, k = 32 dims each) and O += P.V as 8 x v_mfma_f32_16x16x16_bf16
// (16 heads x 16 dims, k = 16 tokens each).  The VALU keeps the code widening
// (exact), the exponentials and the running maximum.
//
// Lane l = 16 g + t (t = l % 16, g = l / 16):
//   * QK: A = K rows: token t, dims 32 g + 8 c .. + 8 of chunk c; B = q' with
//     the same dims for query head t (zero for t >= G).  Output S[token][head]:
//     lane l holds tokens 4g .. 4g+3 of head t.
//   * PV: A = P (rows = heads, k = tokens): exactly the lane's 4 weights of head
//     t at tokens 4g .. 4g+3, so P never moves between lanes.  B = V: tokens
//     4g .. 4g+3 of dim 16 c + t.  Output O[head 4g+j][dim 16 c + t].
//   * The 8-bit pool stores each (block, KV head) in that lane order, so that
//     every load instruction reads 1 KiB contiguously: byte
//     1024 i + 16 l + x holds K[t][32 g + 16 i + x] and
//     V[4 g + x % 4][16 (4 i + x / 4) + t].
//   * The four lane groups of a head share one running maximum (two permlane
//     swaps per block), since P.V sums their tokens in one accumulator.
constexpr int kMma8WorkgroupsPerCu = 2;  // occupancy the register allocation is held to

template <int G, int MODE, int FMT>
__device__ __forceinline__ void decode_mma8_body(const DecodeKernelArgs &a) {
  using E = Elem<bf16>;
  constexpr int D = 128;
  constexpr int NT = kDecodeWaves * kWave;
  static_assert(G >= 1 && G <= 16, "one workgroup takes up to 16 query heads");
  static_assert(MODE == kRopeLazy, "8-bit pools: lazy RoPE");
  typedef short s16x4_t __attribute__((ext_vector_type(4)));

  // rows padded by 16 bytes: the rotation reads 16 heads' rows at once (lane
  // = head) and the merge writes 4 heads' rows at once (lane group = head);
  // unpadded, those rows start in the same LDS bank
  __shared__ float s_q[G][D + 4];
  // a rotation's (cos, sin) per frequency; frequencies 32..63 sit 16 bytes
  // further on, so that the two lane groups reading them at once do not
  // share a bank slot
  __shared__ __attribute__((aligned(16))) float2 s_cs[kDecodeWaves][64 + 2];
  __shared__ float s_m[kDecodeWaves][G];
  __shared__ float s_l[kDecodeWaves][G];
  __shared__ float s_o[kDecodeWaves][G][D + 4];
  __shared__ int s_bad;

  const int hkv = a.num_kv_heads;
  const int slot = blockIdx.x / kXcds;
  const int hsub = slot & ((1 << a.kv_shift) - 1);
  const int unit = (slot >> a.kv_shift) * kXcds + (int)(blockIdx.x % kXcds);
  if (unit >= a.num_units) return;
  const int hkv_pool = hkv >> a.kv_shift;
  const int split = unit % a.max_splits;
  const int gp = (unit / a.max_splits) % hkv_pool;
  const int b = unit / a.max_splits / hkv_pool;
  const int g = (gp << a.kv_shift) | hsub;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int hq = hkv * G;

  const int seq_len = a.seq_lens[b];
  const bool bad_len = seq_len < 0 || seq_len > a.max_blocks * kBlockTokens;
  const int nblk = bad_len ? 0 : (seq_len + kBlockTokens - 1) / kBlockTokens;
  const int nsplit = (nblk + a.split_blocks - 1) / a.split_blocks;
  bf16 *out = (bf16 *)a.out + ((size_t)b * hq + (size_t)g * G) * D;
  if (nsplit == 0) {
    if (split == 0)
      for (int i = tid; i < G * D; i += NT) E::store(out, i, bad_len ? __builtin_nanf("") : 0.f);
    return;
  }
  if (split >= nsplit) return;

  const bf16 *qg = (const bf16 *)a.q + ((size_t)b * hq + (size_t)g * G) * D;
  for (int i = tid; i < G * D; i += NT) s_q[i / D][i % D] = E::load(qg, i);
  if (tid == 0) s_bad = 0;
  __syncthreads();

  const int n_pos = a.q_pos[b];
  const int t16 = lane & 15;  // token row of K, head column of S / P, dim of O
  const int g4 = lane >> 4;   // lane group
  const bool live = t16 < G;
  const double inv_freq = rope_inv_freq(lane, D, a.rope_theta);  // lane i: frequency i (64 of them)

  bf16x8_t qh[4], ql[4];  // q' as bf16 hi + lo parts (see split_bf16x2)
  f32x4_t O[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) O[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c) qh[c] = ql[c] = bf16x8_t{};
  float m = kMaxFloor, lsum = 0.f;

  const int blk0 = split * a.split_blocks;
  const int blk1 = min(nblk, blk0 + a.split_blocks);
  const uint32_t *trow = a.table + (size_t)b * a.max_blocks;
  bool bad = false;
  int cur_off = -1;

  // K and V of block bk (this lane's 32 bytes of each); w returns with the
  // block id replaced by the block's fill count
  auto issue = [&](int bk, uint32_t &w, uint4 (&kk)[2], uint4 (&vv)[2]) {
    w = trow[bk];
    uint32_t id = word_block(w);
    if (id >= (uint32_t)a.num_blocks) {
      bad = true;
      id = 0;
    }
    const uint32_t fill = a.fill4 ? (a.fill4[id >> 2] >> ((id & 3u) * 8u)) & 0xffu : (uint32_t)kBlockTokens;
    w = (w & 0xffff0000u) | fill;
    const size_t hb = ((size_t)id * hkv_pool + gp) * 128;  // 2 KiB = 128 chunks per (block, KV head)
    kk[0] = a.k_pool[hb + lane];
    kk[1] = a.k_pool[hb + 64 + lane];
    vv[0] = a.v_pool[hb + lane];
    vv[1] = a.v_pool[hb + 64 + lane];
  };

  // q' = rot(q, n - off) * scale * log2(e) * k_scale for head t16, dims
  // 32 g4 .. 32 g4 + 31 (frequency d % 64, the pair of dim d is d ^ 64), as
  // bf16 hi + lo parts: S takes one product against each
  // lane i evaluates frequency i into the wave's (cos, sin) table; a lane
  // then reads its 32 frequencies as 16-byte broadcasts
  auto rotate = [&](int delta) {
    const double tt = (double)delta * (inv_freq * 0.15915494309189535);
    const float f = (float)(tt - rint(tt));
    s_cs[wave][lane + (lane >= 32 ? 2 : 0)] = make_float2(__builtin_amdgcn_cosf(f), __builtin_amdgcn_sinf(f));
    __builtin_amdgcn_wave_barrier();
    const int hh = live ? t16 : 0;
    const int d0 = 32 * g4;
    const bool upper = d0 >= 64;
    const float4 *cs4 = (const float4 *)&s_cs[wave][(d0 & 63) + ((d0 & 63) >= 32 ? 2 : 0)];
    float r[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const float4 pr = cs4[k >> 1];  // frequencies d0 + (k & ~1), + 1
      const float c = (k & 1) ? pr.z : pr.x, sv = (k & 1) ? pr.w : pr.y;
      const float x = s_q[hh][d0 + k], y = s_q[hh][(d0 + k) ^ 64];
      const float v = (upper ? fmaf(x, c, y * sv) : fmaf(x, c, -(y * sv))) * a.scale_log2;
      r[k] = live ? v : 0.f;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint32_t wh[4], wl[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) split_bf16x2(r[8 * c + 2 * k], r[8 * c + 2 * k + 1], wh[k], wl[k]);
      qh[c] = __builtin_bit_cast(bf16x8_t, make_uint4(wh[0], wh[1], wh[2], wh[3]));
      ql[c] = __builtin_bit_cast(bf16x8_t, make_uint4(wl[0], wl[1], wl[2], wl[3]));
    }
  };

  // two register sets take turns as current and next block, as in the kernel
  // above (no copies; loads past the split's end re-read its last block and
  // are masked).  Loading further ahead was measured and gains nothing.
  int blk = blk0 + wave;
  const int blast = blk1 - 1;
  uint32_t wA = 0, wB = 0;
  uint4 kA[2], vA[2], kB[2], vB[2];
  issue(min(blk, blast), wA, kA, vA);
  auto step = [&](const uint32_t &wcur, uint4 (&kc)[2], uint4 (&vc)[2], uint32_t &wn, uint4 (&kn)[2],
                  uint4 (&vn)[2]) {
    const int off = word_offset(wcur);
    if (off != cur_off && blk < blk1) {
      rotate(n_pos - off);
      cur_off = off;
    }
    issue(min(blk + kDecodeWaves, blast), wn, kn, vn);

    // S[token 4 g4 + j][head t16], log2 units: K q_h^T + K q_l^T
    f32x4_t S = {0.f, 0.f, 0.f, 0.f}, Sl = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t w0 = dw4(kc[c >> 1], 2 * (c & 1)), w1 = dw4(kc[c >> 1], 2 * (c & 1) + 1);
      const uint4 ka = make_uint4(code8x2_to_bf16x2<FMT, false>(w0), code8x2_to_bf16x2<FMT, true>(w0),
                                  code8x2_to_bf16x2<FMT, false>(w1), code8x2_to_bf16x2<FMT, true>(w1));
      S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka), qh[c], S, 0, 0, 0);
      Sl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka), ql[c], Sl, 0, 0, 0);
    }
    float sv[4] = {S[0] + Sl[0], S[1] + Sl[1], S[2] + Sl[2], S[3] + Sl[3]};
    const int nvalid = blk < blk1 ? min(seq_len - blk * kBlockTokens, (int)(wcur & 0xffffu)) : 0;
    if (nvalid < kBlockTokens) {  // partly filled or exhausted: mask tokens, zero their V bytes
      const int nv = nvalid - 4 * g4;  // valid tokens among this lane's 4
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j >= nv) sv[j] = -INFINITY;
      const uint32_t keep = nv >= 4 ? 0xffffffffu : nv <= 0 ? 0u : (0xffffffffu >> (8 * (4 - nv)));
      vc[0] = make_uint4(vc[0].x & keep, vc[0].y & keep, vc[0].z & keep, vc[0].w & keep);
      vc[1] = make_uint4(vc[1].x & keep, vc[1].y & keep, vc[1].z & keep, vc[1].w & keep);
    }
    // block maximum of head t16 over the four lane groups
    float bm = max4_mfma(sv[0], sv[1], sv[2], sv[3]);
    {
      const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
      bm = fmaxf(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
      const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
      bm = fmaxf(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
    }
    if (wave_any(live && bm > m + kRescaleSlack)) {
      const float mn = fmaxf(m, bm);
      const float alpha = fast_exp2(m - mn);  // 0 on the first rescale
      lsum *= alpha;
      m = mn;
      // O rows are heads 4 g4 + j: their factors live in lanes 4 g4 + j
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float aj = __shfl(alpha, 4 * g4 + j);
#pragma unroll
        for (int c = 0; c < 8; ++c) O[c][j] *= aj;
      }
    }
    const float p0 = fast_exp2(sv[0] - m), p1 = fast_exp2(sv[1] - m);
    const float p2 = fast_exp2(sv[2] - m), p3 = fast_exp2(sv[3] - m);
    const uint32_t pa0 = pack_bf16x2(p0, p1), pa1 = pack_bf16x2(p2, p3);
    lsum = dot2_bf16(pa0, 0x3f803f80u, lsum);  // the bf16 weights P.V uses
    lsum = dot2_bf16(pa1, 0x3f803f80u, lsum);
    const s16x4_t pa = __builtin_bit_cast(s16x4_t, make_uint2(pa0, pa1));
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t vw = dw4(vc[c >> 2], c & 3);
      const s16x4_t vb =
          __builtin_bit_cast(s16x4_t, make_uint2(code8x2_to_bf16x2<FMT, false>(vw), code8x2_to_bf16x2<FMT, true>(vw)));
      O[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, O[c], 0, 0, 0);
    }
    blk += kDecodeWaves;
  };
  while (blk < blk1) {
    step(wA, kA, vA, wB, kB, vB);
    step(wB, kB, vB, wA, kA, vA);
  }

  // this wave's (max, sum, output) per head; sums over the four lane groups
  {
    const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
    lsum = __uint_as_float(x32[0]) + __uint_as_float(x32[1]);
    const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
    lsum = __uint_as_float(x16[0]) + __uint_as_float(x16[1]);
  }
  if (live && g4 == 0) {
    s_m[wave][t16] = m;
    s_l[wave][t16] = lsum;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = 4 * g4 + j;
    if (h < G) {
#pragma unroll
      for (int c = 0; c < 8; ++c) s_o[wave][h][16 * c + t16] = O[c][j];
    }
  }
  if (bad) s_bad = 1;
  __syncthreads();

  const bool single = nsplit == 1;
  const bool flagged = s_bad != 0;
  const size_t part = ((size_t)b * hkv + g) * a.max_splits + split;
  for (int i = tid; i < G * D; i += NT) {
    const int h = i / D, d = i % D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) mx = fmaxf(mx, s_m[w][h]);
    float o = 0.f, ls = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      const float f = s_m[w][h] == -INFINITY ? 0.f : fast_exp2(s_m[w][h] - mx);
      o = fmaf(s_o[w][h][d], f, o);
      ls = fmaf(s_l[w][h], f, ls);
    }
    if (flagged) {
      o = __builtin_nanf("");
      ls = __builtin_nanf("");
    }
    if (single) {
      E::store(out, i, ls != 0.f ? o / ls * a.out_scale : 0.f);
    } else {
      a.ws_o[part * G * D + i] = o;
      if (d == 0) a.ws_ml[part * G + h] = make_float2(mx, ls);
    }
  }
}

template <int G, int MODE>
__global__ void __launch_bounds__(kDecodeWaves * kWave, kMma8WorkgroupsPerCu)
decode_mma8_kernel(const DecodeKernelArgs a) {
  decode_mma8_body<G, MODE, kCodeE4M3>(a);
}

// the same over an int8 pool (same lane-order layout; codes widened exactly)
template <int G>
__global__ void __launch_bounds__(kDecodeWaves * kWave, kMma8WorkgroupsPerCu)
decode_int8_kernel(const DecodeKernelArgs a) {
  decode_mma8_body<G, kRopeLazy, kCodeInt8>(a);
}

// ---------------------------------------------------------------------------
// bf16 pools (head_dim 128) on the matrix cores.  The VALU form above runs out
// of issue slots before HBM does once the query group is large (its Q.K and
// P.V dot products grow with G), and it holds a register double buffer that
// limits the loads in flight; here, as for 8-bit pools, both contractions of a
// block go to MFMA:
// S = K.q'^T as 4 x v_mfma_f32_16x16x32_bf16 (16 tokens x up to 16 query heads)
// and O^T += V^T.P^T as 8 x v_mfma_f32_16x16x16_bf16 (16 dims x 16 heads,
// k = the block's 16 tokens).  The pool keeps its plain [block][head][16][D]
// layout; each wave streams its blocks straight into a two-slot LDS ring
// (global_load_lds_dwordx4, 1 KiB contiguous per instruction, chunks swizzled
// as in the prefill) and reads them back in operand order: K rows with
// ds_read_b128, V transposed with ds_read_b64_tr_b16.
//
// Lane l = 16 g + t (t = l % 16, g = l / 16):
//   * QK: A = K[token t][dims 32c + 8g .. + 8], B = q'[head t][same dims].
//     Output: lane l holds the scores of head t at tokens 4g .. 4g+3.
//   * PV: A = V^T[dim 16c + t][tokens 4g .. 4g+3] (one transposing read),
//     B = the lane's own four weights (head t, tokens 4g .. 4g+3), so P never
//     moves.  Output: lane l holds O^T[dims 16c + 4g .. + 4][head t], so a
//     head's rescale factor is the lane's own.
//   * The four lane groups of a head share one running maximum (two permlane
//     swaps per block), since P.V sums their tokens into one accumulator.
//   * A slot is refilled with the block two steps ahead as soon as its
//     contents are in registers, so about two blocks per wave stay in flight.
constexpr int kMmaSlots = 2;           // LDS ring slots per wave (K and V of one block each)
constexpr int kMma16WorkgroupsPerCu = 2;

// PLAN: the workgroup takes one item of a host-built plan (see
// decode_plan.cpp): a run of blocks of one KV head and up to kPlanMembers
// sequences that read the same blocks (one document they all hold).  Its 16
// MFMA columns are then (member, query head) pairs: member t16 / G, head
// t16 % G, each with its own query, position and offset; every member
// writes its own partial.
constexpr int kPlanMembers = 4;
constexpr int kPlanInts = 12;  // ints per plan item
static_assert(kPlanInts == 12, "the kernel reads an item as three int4");

template <int G, int MODE, bool PLAN>
__device__ __forceinline__ void decode_mma16_body(const DecodeKernelArgs &a) {
  using E = Elem<bf16>;
  constexpr int D = 128;
  constexpr int CPR = D / 8;               // 16-byte chunks per row
  constexpr int RPI = kWave / CPR;         // rows per DMA instruction
  constexpr int IPB = kBlockTokens / RPI;  // DMA instructions per block (K or V)
  constexpr int ROWB = D * 2;
  constexpr int BLKB = kBlockTokens * ROWB;  // 4 KiB: one block of one KV head
  constexpr int NT = kDecodeWaves * kWave;
  constexpr bool EAGER = MODE == kRopeEager;
  constexpr bool ALIBI = MODE == kAlibi;
  static_assert(G >= 1 && G <= 16, "one workgroup takes up to 16 query heads");
  static_assert(!PLAN || MODE == kRopeLazy, "plans: lazy RoPE");
  constexpr int NC = PLAN ? 16 : G;  // MFMA columns in use at most
  // a column's partial output row in the ring at the merge: with all 16
  // columns live, rows padded by 16 bytes keep the eight lanes of a
  // ds_write_b128 cycle (eight columns, same dims) out of one bank slot
  constexpr int OROW = PLAN ? D + 4 : D;
  static_assert(NC * OROW * sizeof(float) <= kMmaSlots * 2 * BLKB, "a wave's partial output fits its ring");

  // per wave: kMmaSlots x (K tile, V tile); after the loop a wave's ring holds
  // its partial output [NC][D] for the merge
  __shared__ __attribute__((aligned(1024))) char s_ring[kDecodeWaves][kMmaSlots][2][BLKB];
  __shared__ float s_m[kDecodeWaves][NC];
  __shared__ float s_l[kDecodeWaves][NC];
  __shared__ int s_bad[kDecodeWaves];  // per wave: a table word pointed outside the pool

  const int hkv = a.num_kv_heads;
  const int hkv_pool = hkv >> a.kv_shift;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int hq = hkv * G;
  const int t16 = lane & 15;  // K token row / query head column / V^T dim row
  const int g4 = lane >> 4;   // lane group

  int b, g, split, nsplit, nblk, seq_len, blk0, blk1;
  bool bad_len;
  int nmem = 1;                              // planned: members of the item
  uint32_t mem[kPlanMembers] = {0u, 0u, 0u, 0u};  // (sequence | slot << 16)
  int mstart[kPlanMembers] = {0, 0, 0, 0};        // the run's first block in each member's row
  if constexpr (PLAN) {
    // item: (KV head | members << 16, first block, end block (both in
    // member 0's row), 0, members 0..3, the run's start in each member's
    // row); an item naming a sequence, head, slot or row place outside the
    // batch, the heads, a sequence's slot count or the table is skipped,
    // block ranges are clipped to member 0's length
    if ((int)blockIdx.x >= a.num_units) return;
    const int4 *item = a.plan_items + (size_t)(kPlanInts / 4) * blockIdx.x;
    const int4 r0 = item[0], r1 = item[1], r2 = item[2];
    g = r0.x & 0xffff;
    nmem = (int)((uint32_t)r0.x >> 16);
    blk0 = r0.y;
    blk1 = r0.z;
    mem[0] = (uint32_t)r1.x;
    mem[1] = (uint32_t)r1.y;
    mem[2] = (uint32_t)r1.z;
    mem[3] = (uint32_t)r1.w;
    mstart[0] = r2.x;
    mstart[1] = r2.y;
    mstart[2] = r2.z;
    mstart[3] = r2.w;
    if (g >= hkv || nmem < 1 || nmem > kPlanMembers || nmem * G > 16) return;
    for (int k = 0; k < nmem; ++k) {
      const int mb = (int)(mem[k] & 0xffffu), ms = (int)(mem[k] >> 16);
      if (mb >= a.batch || mstart[k] < 0 || mstart[k] >= a.max_blocks) return;
      const int cnt = a.plan_counts[mb];
      if (cnt < 1 || cnt > a.max_splits || ms >= cnt) return;
    }
    b = (int)(mem[0] & 0xffffu);
    split = (int)(mem[0] >> 16);
    nsplit = a.plan_counts[b];
    seq_len = a.seq_lens[b];
    bad_len = seq_len < 0 || seq_len > a.max_blocks * kBlockTokens;
    nblk = bad_len ? 0 : (seq_len + kBlockTokens - 1) / kBlockTokens;
    blk1 = min(max(blk1, 0), nblk);
    blk0 = min(max(blk0, 0), blk1);
  } else {
    DecodeShare sh;
    if (!decode_share(a, sh)) return;
    b = sh.b;
    g = sh.g;
    split = sh.split;
    nsplit = sh.nsplit;
    nblk = sh.nblk;
    seq_len = sh.seq_len;
    bad_len = sh.bad_len;
    blk0 = sh.blk0;
    blk1 = sh.blk1;
  }
  const int gp = g >> a.kv_shift;

  bf16 *out = (bf16 *)a.out + ((size_t)b * hq + (size_t)g * G) * D;
  if (nblk == 0) {  // empty sequence -> zeros; invalid length -> NaN
    if (split == 0 && nmem == 1)
      for (int i = tid; i < G * D; i += NT) E::store(out, i, bad_len ? __builtin_nanf("") : 0.f);
    return;
  }
  if (split >= nsplit) return;

  const int n_pos = a.q_pos[b];
  // this lane's column: query head t16, or (planned) head t16 % G of member
  // t16 / G, whose sequence is bcol
  const int ncol = PLAN ? nmem * G : G;
  const bool live = t16 < ncol;
  const int mcol = PLAN ? t16 / G : 0;
  const int hcol = PLAN ? t16 % G : t16;
  const int bcol = !PLAN || !live ? b
                   : (int)((mcol == 0 ? mem[0] : mcol == 1 ? mem[1] : mcol == 2 ? mem[2] : mem[3]) & 0xffffu);

  // raw (bf16) query of the lane's column, dims 32c + 8 g4 .. + 8 (chunk 4c + g4)
  uint4 qraw[4];
  {
    const uint4 *qh =
        (const uint4 *)((const bf16 *)a.q + ((size_t)bcol * hq + (size_t)g * G + (live ? hcol : 0)) * D);
#pragma unroll
    for (int c = 0; c < 4; ++c) qraw[c] = live ? qh[4 * c + g4] : make_uint4(0u, 0u, 0u, 0u);
  }
  const double inv_freq = rope_inv_freq(lane, D, a.rope_theta);  // lane i: frequency i (D/2 = 64 of them)

  // q' = rot(q, delta) * scale * log2(e) for head t16, as two bf16 parts
  // (qh + ql, see split_bf16x2): S takes one product against each, so q' is
  // not rounded to bf16 (that rounding alone limits wide score spreads).
  // The lane's dims d (c = 0, 1) and d + 64 (c + 2) form rotate-half pairs,
  // so the rotation is lane-local; cos/sin of frequency i come from lane i
  // (angle reduced in double to a fraction of a turn, then v_cos/v_sin).
  bf16x8_t qh[4], ql[4];
  auto rotate = [&](int delta) {
    const double tt = (double)delta * (inv_freq * 0.15915494309189535);
    const float f = (float)(tt - rint(tt));
    const float cs = __builtin_amdgcn_cosf(f), sn = __builtin_amdgcn_sinf(f);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      uint32_t xh[4], xl[4], yh[4], yl[4];  // dims d (x) and d + 64 (y): hi and lo parts
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float r[4];
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
          const int e = 2 * k + e2;
          const int fi = 32 * c + 8 * g4 + e;
          const float cv = __shfl(cs, fi), sv = __shfl(sn, fi);
          const uint32_t wx = dw4(qraw[c], k), wy = dw4(qraw[c + 2], k);
          const float x = e2 ? bf16_hi(wx) : bf16_lo(wx);
          const float y = e2 ? bf16_hi(wy) : bf16_lo(wy);
          r[e2] = fmaf(x, cv, -(y * sv)) * a.scale_log2;
          r[2 + e2] = fmaf(y, cv, x * sv) * a.scale_log2;
        }
        split_bf16x2(r[0], r[1], xh[k], xl[k]);
        split_bf16x2(r[2], r[3], yh[k], yl[k]);
      }
      qh[c] = as_bf16x8(make_uint4(xh[0], xh[1], xh[2], xh[3]));
      ql[c] = as_bf16x8(make_uint4(xl[0], xl[1], xl[2], xl[3]));
      qh[c + 2] = as_bf16x8(make_uint4(yh[0], yh[1], yh[2], yh[3]));
      ql[c + 2] = as_bf16x8(make_uint4(yl[0], yl[1], yl[2], yl[3]));
    }
  };
  // the same rotation with a delta of the lane's own (planned items with
  // several members: each column has its sequence's position and offset):
  // the lane evaluates its 16 frequencies itself, from lane fi's inverse
  // frequency, by the same expression, so a delta gives the same q' either way
  auto rotate_own = [&](int delta) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      uint32_t xh[4], xl[4], yh[4], yl[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float r[4];
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
          const int e = 2 * k + e2;
          const int fi = 32 * c + 8 * g4 + e;
          const double tt = (double)delta * (__shfl(inv_freq, fi) * 0.15915494309189535);
          const float f = (float)(tt - rint(tt));
          const float cv = __builtin_amdgcn_cosf(f), sv = __builtin_amdgcn_sinf(f);
          const uint32_t wx = dw4(qraw[c], k), wy = dw4(qraw[c + 2], k);
          const float x = e2 ? bf16_hi(wx) : bf16_lo(wx);
          const float y = e2 ? bf16_hi(wy) : bf16_lo(wy);
          r[e2] = fmaf(x, cv, -(y * sv)) * a.scale_log2;
          r[2 + e2] = fmaf(y, cv, x * sv) * a.scale_log2;
        }
        split_bf16x2(r[0], r[1], xh[k], xl[k]);
        split_bf16x2(r[2], r[3], yh[k], yl[k]);
      }
      qh[c] = as_bf16x8(make_uint4(xh[0], xh[1], xh[2], xh[3]));
      ql[c] = as_bf16x8(make_uint4(xl[0], xl[1], xl[2], xl[3]));
      qh[c + 2] = as_bf16x8(make_uint4(yh[0], yh[1], yh[2], yh[3]));
      ql[c + 2] = as_bf16x8(make_uint4(yl[0], yl[1], yl[2], yl[3]));
    }
  };
  if constexpr (EAGER) rotate(n_pos);
  if constexpr (ALIBI) rotate(0);  // the identity: q * scale * log2(e)
  const float slope2 = ALIBI && live ? a.slopes[g * G + t16] * kLog2e : 0.f;

  // DMA source offsets (tile-independent): lane L of instruction i fills row
  // i * RPI + L / CPR, chunk slot L % CPR, from global chunk (L % CPR) ^ swz(row)
  uint32_t ld_off[IPB];
#pragma unroll
  for (int i = 0; i < IPB; ++i) {
    const int r = i * RPI + lane / CPR;
    ld_off[i] = (uint32_t)(r * ROWB + (((lane % CPR) ^ swz<CPR>(r)) * 16));
  }
  // operand read offsets: K row t16, chunk 4c + g4; V^T source row 4 g4 + t16 / 4, dims 16c + 4 (t16 % 4)
  uint32_t k_off[4], v_off[8];
#pragma unroll
  for (int c = 0; c < 4; ++c) k_off[c] = (uint32_t)(t16 * ROWB + (((4 * c + g4) ^ swz<CPR>(t16)) * 16));
  {
    const int vr = 4 * g4 + (t16 >> 2);
    const int tdim = (t16 & 3) * 4;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int dim = 16 * c + tdim;
      v_off[c] = (uint32_t)(vr * ROWB + (((dim / 8) ^ swz<CPR>(vr)) * 16) + (dim % 8) * 2);
    }
  }
  char *ring = &s_ring[wave][0][0][0];
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_ptr_t)ring;

  // table words and fill counts as scalar loads (see as_const_as)
  const auto trow = as_const_as(a.table + (size_t)b * a.max_blocks);
  const auto fill4 = a.fill4 ? as_const_as(a.fill4) : nullptr;
  bool bad = false;

  // K and V of the block whose table word is w into ring slot SL.  Returns the
  // block's offset << 16 | the bit position of its fill count in fw, the
  // 32-bit word of the fill array that holds it (all ones without an array).
  // The count is extracted when the block is computed, two steps later, so
  // its scalar load is never waited for here.
  auto issue = [&](uint32_t w, uint32_t &fw, auto slc) -> uint32_t {
    constexpr int SL = decltype(slc)::value;
    uint32_t id = word_block(w);
    if (id >= (uint32_t)a.num_blocks) {
      bad = true;
      id = 0;
    }
    const char *kg = (const char *)a.k_pool + ((size_t)id * hkv_pool + gp) * BLKB;
    const char *vg = (const char *)a.v_pool + ((size_t)id * hkv_pool + gp) * BLKB;
#pragma unroll
    for (int i = 0; i < IPB; ++i) {
      lds_dma16(kg, ld_off[i], ring_lds + (SL * 2) * BLKB + i * 1024);
      lds_dma16(vg, ld_off[i], ring_lds + (SL * 2 + 1) * BLKB + i * 1024);
    }
    fw = fill4 ? fill4[id >> 2] : 0xffffffffu;
    return (w & 0xffff0000u) | ((id & 3u) * 8u);
  };

  f32x4_t O[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) O[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = kMaxFloor, lsum = 0.f;
  int cur_off = -1;
  // several members: every column rotated once, by its own sequence's
  // position and offset (the plan takes such runs only where each member's
  // offset stays the same over the run)
  const bool multi = PLAN && nmem > 1;
  if constexpr (PLAN) {
    if (multi && blk0 < blk1) {
      const int scol = mcol == 0 ? mstart[0] : mcol == 1 ? mstart[1] : mcol == 2 ? mstart[2] : mstart[3];
      const int own_off = word_offset(a.table[(size_t)bcol * a.max_blocks + (live ? scol : blk0)]);
      rotate_own(live ? a.q_pos[bcol] - own_off : 0);
    }
  }

  // this wave takes blocks blk0 + wave, + 4, ...; slots alternate
  int blk = blk0 + wave;
  uint32_t meta0 = 0, meta1 = 0, fw0 = 0, fw1 = 0;
  if (blk < blk1) meta0 = issue(trow[blk], fw0, std::integral_constant<int, 0>{});
  if (blk + kDecodeWaves < blk1) meta1 = issue(trow[blk + kDecodeWaves], fw1, std::integral_constant<int, 1>{});
  // table word of the block two steps ahead, loaded one step before its DMA
  uint32_t wpre = blk + 2 * kDecodeWaves < blk1 ? trow[blk + 2 * kDecodeWaves] : 0u;

  auto step = [&](uint32_t &meta, uint32_t &fw, auto slc) {
    constexpr int SL = decltype(slc)::value;
    // this block's loads have landed (the next block's may still be in flight)
    if (blk + kDecodeWaves < blk1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * IPB) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const char *kb = ring + (SL * 2) * BLKB;
    const char *vb = ring + (SL * 2 + 1) * BLKB;
    uint4 ka[4];
    uint2 va[8];
#pragma unroll
    for (int c = 0; c < 4; ++c) ka[c] = *(const uint4 *)(kb + k_off[c]);
#pragma unroll
    for (int c = 0; c < 8; ++c) va[c] = lds_read_tr16((const uint16_t *)(vb + v_off[c]));
    const uint32_t mcur = meta;
    const uint32_t fcur = (fw >> (mcur & 31u)) & 0xffu;  // fill count (255: no array)
    // refill the slot with the block two steps ahead once the reads are done
    const int bfar = blk + 2 * kDecodeWaves;
    if (bfar < blk1) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      meta = issue(wpre, fw, slc);
      wpre = bfar + kDecodeWaves < blk1 ? trow[bfar + kDecodeWaves] : 0u;
    }

    if constexpr (MODE == kRopeLazy) {
      const int off = word_offset(mcur);
      if (!multi && off != cur_off) {
        rotate(n_pos - off);
        cur_off = off;
      }
    }
    // S[token 4 g4 + j][head t16], log2 units: K q_h^T + K q_l^T
    f32x4_t S = {0.f, 0.f, 0.f, 0.f}, Sl = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka[c]), qh[c], S, 0, 0, 0);
      Sl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka[c]), ql[c], Sl, 0, 0, 0);
    }
    float sv[4] = {S[0] + Sl[0], S[1] + Sl[1], S[2] + Sl[2], S[3] + Sl[3]};
    if constexpr (ALIBI) {  // key position (block offset + slot) - query position
      const float base = (float)(word_offset(mcur) + 4 * g4 - n_pos);
#pragma unroll
      for (int j = 0; j < 4; ++j) sv[j] = fmaf(slope2, base + (float)j, sv[j]);
    }
    const int nvalid = min(seq_len - blk * kBlockTokens, (int)fcur);
    if (nvalid < kBlockTokens) {  // partly filled: mask tokens, zero their V values
      const int nv = nvalid - 4 * g4;  // valid tokens among this lane's 4
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j >= nv) sv[j] = -INFINITY;
      const uint32_t kx = nv >= 2 ? 0xffffffffu : nv == 1 ? 0xffffu : 0u;
      const uint32_t ky = nv >= 4 ? 0xffffffffu : nv == 3 ? 0xffffu : 0u;
#pragma unroll
      for (int c = 0; c < 8; ++c) va[c] = make_uint2(va[c].x & kx, va[c].y & ky);
    }
    // block maximum of head t16 over the four lane groups
    const float bm = col_max4(max4_mfma(sv[0], sv[1], sv[2], sv[3]));
    if (wave_any(live && bm > m + kRescaleSlack)) {
      const float mn = fmaxf(m, bm);
      const float alpha = fast_exp2(m - mn);  // 0 on the first rescale
      lsum *= alpha;
      m = mn;
#pragma unroll
      for (int c = 0; c < 8; ++c) O[c] *= alpha;
    }
    const uint32_t pa0 = pack_bf16x2(fast_exp2(sv[0] - m), fast_exp2(sv[1] - m));
    const uint32_t pa1 = pack_bf16x2(fast_exp2(sv[2] - m), fast_exp2(sv[3] - m));
    lsum = dot2_bf16(pa0, 0x3f803f80u, lsum);  // the bf16 weights P.V uses
    lsum = dot2_bf16(pa1, 0x3f803f80u, lsum);
    const s16x4_t pb = __builtin_bit_cast(s16x4_t, make_uint2(pa0, pa1));
#pragma unroll
    for (int c = 0; c < 8; ++c)
      O[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, va[c]), pb, O[c], 0, 0, 0);
    blk += kDecodeWaves;
  };
  while (blk < blk1) {
    step(meta0, fw0, std::integral_constant<int, 0>{});
    if (blk >= blk1) break;
    step(meta1, fw1, std::integral_constant<int, 1>{});
  }

  // this wave's (max, sum, output): sums over the four lane groups; the
  // output goes to the wave's own ring (its loads have all landed)
  lsum = col_sum4(lsum);
  if (live && g4 == 0) {
    s_m[wave][t16] = m;
    s_l[wave][t16] = lsum;
  }
  if (live) {
    float *so = (float *)ring + t16 * OROW + 4 * g4;
#pragma unroll
    for (int c = 0; c < 8; ++c) *(f32x4_t *)(so + 16 * c) = O[c];
  }
  if (lane == 0) s_bad[wave] = bad;
  __syncthreads();

  const bool flagged = (s_bad[0] | s_bad[1] | s_bad[2] | s_bad[3]) != 0;
  for (int i = tid; i < ncol * D; i += NT) {
    const int h = i / D;  // column
    const int d = i % D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) mx = fmaxf(mx, s_m[w][h]);
    float o = 0.f, ls = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) {
      const float f = s_m[w][h] == -INFINITY ? 0.f : fast_exp2(s_m[w][h] - mx);
      o = fmaf(((const float *)&s_ring[w][0][0][0])[h * OROW + d], f, o);
      ls = fmaf(s_l[w][h], f, ls);
    }
    if (flagged) {
      o = __builtin_nanf("");
      ls = __builtin_nanf("");
    }
    // the column's sequence, query head (within the group) and partial slot
    int bs = b, hh = h, sp = split, ns = nsplit;
    if constexpr (PLAN) {
      const int k = h / G;
      const uint32_t mk = k == 0 ? mem[0] : k == 1 ? mem[1] : k == 2 ? mem[2] : mem[3];
      bs = (int)(mk & 0xffffu);
      sp = (int)(mk >> 16);
      hh = h % G;
      ns = a.plan_counts[bs];
    }
    if (ns == 1) {
      E::store((bf16 *)a.out + ((size_t)bs * hq + (size_t)g * G + hh) * D, d, ls != 0.f ? o / ls : 0.f);
    } else {
      const size_t part = ((size_t)bs * hkv + g) * a.max_splits + sp;
      a.ws_o[(part * G + hh) * D + d] = o;
      if (d == 0) a.ws_ml[part * G + hh] = make_float2(mx, ls);
    }
  }
}

// ---------------------------------------------------------------------------
// Query groups of 32 or 64 heads (multi-query attention) on the matrix cores.
// The kernel above takes up to 16 heads (one MFMA column tile); giving a larger
// group to G / 16 workgroups would make each of them walk every block again.
// Here one workgroup takes all G = 16 CT heads of a KV head, so each K/V block
// is read from memory once.  Its NW waves (4 for 32 heads; 8 for 64, one
// workgroup per CU, so that each wave takes one block per step) form
// BS = NW / CT = 2 block streams of CT waves: wave w takes column tile w % CT
// (heads 16 (w % CT) ..) and stream w / CT, and the CT waves of a stream share
// each block of that stream through LDS.  A stream owns R = 4 ring slots (the
// workgroup keeps 8 blocks, 64 KiB, in LDS, as the kernel above does): the
// block of step i goes to slot i % R, R - 1 steps ahead.  Each of the stream's waves issues
// IPW = 8 / CT of the block's 8 DMA instructions (1 KiB each, K then V), and
// one workgroup barrier per step both publishes the landed block to every
// reader and frees the slot all waves read one step before.  Streams that run
// out of blocks re-read their split's last block (never computed on), so
// every wave has the same number of loads in flight at each wait.  Per wave
// and block the products, the lazy rotation, the masking and the softmax are
// those of the kernel above, for the wave's 16 heads; the streams' partial
// results are merged in LDS at the end.
constexpr int wide_waves(int ct) { return ct == 4 ? 8 : kDecodeWaves; }

template <int CT, int MODE>
__global__ void __launch_bounds__(wide_waves(CT) * kWave, CT == 4 ? 1 : kMma16WorkgroupsPerCu)
decode_mma16_wide_kernel(const DecodeKernelArgs a) {
  using E = Elem<bf16>;
  constexpr int G = 16 * CT;               // query heads of the workgroup
  constexpr int NW = wide_waves(CT);       // waves of the workgroup
  constexpr int BS = NW / CT;              // block streams
  constexpr int R = 8 / BS;                // ring slots per stream (4)
  constexpr int P = 1;                     // blocks of a stream per step
  constexpr int RS = R / P;                // steps the ring holds
  constexpr int D = 128;
  constexpr int CPR = D / 8;               // 16-byte chunks per row
  constexpr int RPI = kWave / CPR;         // rows per DMA instruction
  constexpr int IPB = kBlockTokens / RPI;  // DMA instructions per block (K or V)
  constexpr int IPW = 2 * IPB / CT;        // DMA instructions per wave and block
  constexpr int ROWB = D * 2;
  constexpr int BLKB = kBlockTokens * ROWB;  // 4 KiB: one block of one KV head
  constexpr int NT = NW * kWave;
  constexpr bool EAGER = MODE == kRopeEager;
  constexpr bool ALIBI = MODE == kAlibi;
  static_assert(CT == 2 || CT == 4, "32 or 64 query heads");
  static_assert(RS >= 2 && RS * P == R, "at least one step of prefetch");
  constexpr int OROW = D + 4;  // merge rows padded by 16 bytes (else 16 lanes store into one bank)
  // the ring, and after the loop the waves' partial outputs [NW][16][OROW]
  constexpr int RINGB = BS * R * 2 * BLKB;
  constexpr int MERGEB = NW * 16 * OROW * (int)sizeof(float);
  __shared__ __attribute__((aligned(1024))) char s_ring[RINGB > MERGEB ? RINGB : MERGEB];
  __shared__ float s_m[NW][16];
  __shared__ float s_l[NW][16];
  __shared__ int s_bad[NW];

  const int hkv = a.num_kv_heads;
  const int unit = (int)blockIdx.x;
  if (unit >= a.num_units) return;
  const int split = unit % a.max_splits;
  const int g = (unit / a.max_splits) % hkv;
  const int b = unit / a.max_splits / hkv;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int ct = wave % CT;  // column tile: heads 16 ct .. 16 ct + 15 of the group
  const int st = wave / CT;  // block stream
  const int hq = hkv * G;

  const int seq_len = a.seq_lens[b];
  const bool bad_len = seq_len < 0 || seq_len > a.max_blocks * kBlockTokens;
  const int nblk = bad_len ? 0 : (seq_len + kBlockTokens - 1) / kBlockTokens;
  const int nsplit = (nblk + a.split_blocks - 1) / a.split_blocks;
  bf16 *out = (bf16 *)a.out + ((size_t)b * hq + (size_t)g * G) * D;
  if (nsplit == 0) {
    if (split == 0)
      for (int i = tid; i < G * D; i += NT) E::store(out, i, bad_len ? __builtin_nanf("") : 0.f);
    return;
  }
  if (split >= nsplit) return;

  const int n_pos = a.q_pos[b];
  const int t16 = lane & 15;  // K token row / query head column / V^T dim row
  const int g4 = lane >> 4;   // lane group
  const int head = 16 * ct + t16;

  uint4 qraw[4];
  {
    const uint4 *qh = (const uint4 *)((const bf16 *)a.q + ((size_t)b * hq + (size_t)g * G + head) * D);
#pragma unroll
    for (int c = 0; c < 4; ++c) qraw[c] = qh[4 * c + g4];
  }
  const double inv_freq = rope_inv_freq(lane, D, a.rope_theta);

  // q' = rot(q, delta) * scale * log2(e) as bf16 hi + lo parts, as above
  bf16x8_t qh[4], ql[4];
  auto rotate = [&](int delta) {
    const double tt = (double)delta * (inv_freq * 0.15915494309189535);
    const float f = (float)(tt - rint(tt));
    const float cs = __builtin_amdgcn_cosf(f), sn = __builtin_amdgcn_sinf(f);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      uint32_t xh[4], xl[4], yh[4], yl[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float r[4];
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
          const int fi = 32 * c + 8 * g4 + 2 * k + e2;
          const float cv = __shfl(cs, fi), sv = __shfl(sn, fi);
          const uint32_t wx = dw4(qraw[c], k), wy = dw4(qraw[c + 2], k);
          const float x = e2 ? bf16_hi(wx) : bf16_lo(wx);
          const float y = e2 ? bf16_hi(wy) : bf16_lo(wy);
          r[e2] = fmaf(x, cv, -(y * sv)) * a.scale_log2;
          r[2 + e2] = fmaf(y, cv, x * sv) * a.scale_log2;
        }
        split_bf16x2(r[0], r[1], xh[k], xl[k]);
        split_bf16x2(r[2], r[3], yh[k], yl[k]);
      }
      qh[c] = as_bf16x8(make_uint4(xh[0], xh[1], xh[2], xh[3]));
      ql[c] = as_bf16x8(make_uint4(xl[0], xl[1], xl[2], xl[3]));
      qh[c + 2] = as_bf16x8(make_uint4(yh[0], yh[1], yh[2], yh[3]));
      ql[c + 2] = as_bf16x8(make_uint4(yl[0], yl[1], yl[2], yl[3]));
    }
  };
  if constexpr (EAGER) rotate(n_pos);
  if constexpr (ALIBI) rotate(0);
  const float slope2 = ALIBI ? a.slopes[g * G + head] * kLog2e : 0.f;

  uint32_t ld_off[IPB];
#pragma unroll
  for (int i = 0; i < IPB; ++i) {
    const int r = i * RPI + lane / CPR;
    ld_off[i] = (uint32_t)(r * ROWB + (((lane % CPR) ^ swz<CPR>(r)) * 16));
  }
  uint32_t k_off[4], v_off[8];
#pragma unroll
  for (int c = 0; c < 4; ++c) k_off[c] = (uint32_t)(t16 * ROWB + (((4 * c + g4) ^ swz<CPR>(t16)) * 16));
  {
    const int vr = 4 * g4 + (t16 >> 2);
    const int tdim = (t16 & 3) * 4;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int dim = 16 * c + tdim;
      v_off[c] = (uint32_t)(vr * ROWB + (((dim / 8) ^ swz<CPR>(vr)) * 16) + (dim % 8) * 2);
    }
  }
  char *ring = s_ring + st * (R * 2 * BLKB);
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_ptr_t)ring;

  const int blk0 = split * a.split_blocks;
  const int blk1 = min(nblk, blk0 + a.split_blocks);
  const int steps = (blk1 - blk0 + BS * P - 1) / (BS * P);  // the same for every wave
  const auto trow = as_const_as(a.table + (size_t)b * a.max_blocks);
  const auto fill4 = a.fill4 ? as_const_as(a.fill4) : nullptr;
  bool bad = false;

  // this wave's share of the DMA of its stream's k-th block (past the
  // stream's end: the split's last block again, never computed on) into
  // slot k % R
  auto issue = [&](int kk) {
    const int bk = min(blk0 + st + BS * kk, blk1 - 1);
    uint32_t id = word_block(trow[bk]);
    if (id >= (uint32_t)a.num_blocks) {
      bad = true;
      id = 0;
    }
    const char *kg = (const char *)a.k_pool + ((size_t)id * hkv + g) * BLKB;
    const char *vg = (const char *)a.v_pool + ((size_t)id * hkv + g) * BLKB;
    const uint32_t sl = ring_lds + (uint32_t)((kk % R) * 2 * BLKB);
#pragma unroll
    for (int j = ct; j < 2 * IPB; j += CT) {
      if (j < IPB) lds_dma16(kg, ld_off[j], sl + j * 1024);
      else lds_dma16(vg, ld_off[j - IPB], sl + BLKB + (j - IPB) * 1024);
    }
  };

  f32x4_t O[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) O[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = kMaxFloor, lsum = 0.f;
  int cur_off = -1;

  // step i: this wave's 16 heads against the stream's blocks P i .. P i + P - 1
  // (ring slots kk % R).  The blocks' scores share one maximum update and one
  // set of exponentials; a block past the stream's end takes no part.
  auto consume = [&](int i) __attribute__((always_inline)) {
    int bk[P];
    bool has[P];
    uint4 ka[P][4];
    uint2 va[P][8];
    float sv[P][4];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int kk = i * P + p;
      bk[p] = blk0 + st + BS * kk;
      has[p] = bk[p] < blk1;  // wave-uniform
      if (!has[p]) continue;
      const char *kb = ring + (kk % R) * 2 * BLKB;
      const char *vb = kb + BLKB;
#pragma unroll
      for (int c = 0; c < 4; ++c) ka[p][c] = *(const uint4 *)(kb + k_off[c]);
#pragma unroll
      for (int c = 0; c < 8; ++c) va[p][c] = lds_read_tr16((const uint16_t *)(vb + v_off[c]));
    }
#pragma unroll
    for (int p = 0; p < P; ++p) {
      if (!has[p]) {
        sv[p][0] = sv[p][1] = sv[p][2] = sv[p][3] = -INFINITY;
        continue;
      }
      const uint32_t w = trow[bk[p]];
      if constexpr (MODE == kRopeLazy) {
        const int off = word_offset(w);
        if (off != cur_off) {
          rotate(n_pos - off);
          cur_off = off;
        }
      }
      f32x4_t S = {0.f, 0.f, 0.f, 0.f}, Sl = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka[p][c]), qh[c], S, 0, 0, 0);
        Sl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka[p][c]), ql[c], Sl, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) sv[p][j] = S[j] + Sl[j];
      if constexpr (ALIBI) {
        const float base = (float)(word_offset(w) + 4 * g4 - n_pos);
#pragma unroll
        for (int j = 0; j < 4; ++j) sv[p][j] = fmaf(slope2, base + (float)j, sv[p][j]);
      }
      const uint32_t fcur =
          a.fill4 ? (fill4[min(word_block(w), (uint32_t)a.num_blocks - 1) >> 2] >> ((word_block(w) & 3u) * 8u)) & 0xffu
                  : 0xffu;
      const int nvalid = min(seq_len - bk[p] * kBlockTokens, (int)fcur);
      if (nvalid < kBlockTokens) {
        const int nv = nvalid - 4 * g4;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (j >= nv) sv[p][j] = -INFINITY;
        const uint32_t kx = nv >= 2 ? 0xffffffffu : nv == 1 ? 0xffffu : 0u;
        const uint32_t ky = nv >= 4 ? 0xffffffffu : nv == 3 ? 0xffffu : 0u;
#pragma unroll
        for (int c = 0; c < 8; ++c) va[p][c] = make_uint2(va[p][c].x & kx, va[p][c].y & ky);
      }
    }
    float bm = max4_mfma(sv[0][0], sv[0][1], sv[0][2], sv[0][3]);
#pragma unroll
    for (int p = 1; p < P; ++p) bm = fmaxf(bm, max4_mfma(sv[p][0], sv[p][1], sv[p][2], sv[p][3]));
    bm = col_max4(bm);
    if (wave_any(bm > m + kRescaleSlack)) {
      const float mn = fmaxf(m, bm);
      const float alpha = fast_exp2(m - mn);
      lsum *= alpha;
      m = mn;
#pragma unroll
      for (int c = 0; c < 8; ++c) O[c] *= alpha;
    }
#pragma unroll
    for (int p = 0; p < P; ++p) {
      if (!has[p]) continue;
      const uint32_t pa0 = pack_bf16x2(fast_exp2(sv[p][0] - m), fast_exp2(sv[p][1] - m));
      const uint32_t pa1 = pack_bf16x2(fast_exp2(sv[p][2] - m), fast_exp2(sv[p][3] - m));
      lsum = dot2_bf16(pa0, 0x3f803f80u, lsum);
      lsum = dot2_bf16(pa1, 0x3f803f80u, lsum);
      const s16x4_t pb = __builtin_bit_cast(s16x4_t, make_uint2(pa0, pa1));
#pragma unroll
      for (int c = 0; c < 8; ++c)
        O[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, va[p][c]), pb, O[c], 0, 0, 0);
    }
  };

  // step i takes the stream's blocks P i .. P i + P - 1; the ring holds RS
  // steps, filled RS - 1 steps ahead
#pragma unroll
  for (int kk = 0; kk < (RS - 1) * P; ++kk) issue(kk);
  for (int i = 0; i < steps; ++i) {
    // this wave's loads of step i have landed (RS - 2 later steps may be in
    // flight); after the barrier so have the other waves' shares, and every
    // wave is done with the slots the next DMAs overwrite
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((RS - 2) * P * IPW) : "memory");
    __syncthreads();
#pragma unroll
    for (int p = 0; p < P; ++p) issue((i + RS - 1) * P + p);
    consume(i);
  }
  // the re-reads past the end must land before the ring is reused for the merge
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // merge the streams: wave w's partial output [16][D] at ring offset w * 8 KiB
  lsum = col_sum4(lsum);
  if (g4 == 0) {
    s_m[wave][t16] = m;
    s_l[wave][t16] = lsum;
  }
  {
    float *so = (float *)s_ring + (wave * 16 + t16) * OROW + 4 * g4;
#pragma unroll
    for (int c = 0; c < 8; ++c) *(f32x4_t *)(so + 16 * c) = O[c];
  }
  if (lane == 0) s_bad[wave] = bad;
  __syncthreads();

  const bool single = nsplit == 1;
  bool flagged = false;
#pragma unroll
  for (int w = 0; w < NW; ++w) flagged |= s_bad[w] != 0;
  const size_t part = ((size_t)b * hkv + g) * a.max_splits + split;
  const float *po = (const float *)s_ring;
  for (int i = tid; i < G * D; i += NT) {
    const int h = i / D, d = i % D;
    const int hc = h / 16, hh = h % 16;
    float mx = -INFINITY;
#pragma unroll
    for (int s2 = 0; s2 < BS; ++s2) mx = fmaxf(mx, s_m[s2 * CT + hc][hh]);
    float o = 0.f, ls = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < BS; ++s2) {
      const int w2 = s2 * CT + hc;
      const float f = s_m[w2][hh] == -INFINITY ? 0.f : fast_exp2(s_m[w2][hh] - mx);
      o = fmaf(po[(w2 * 16 + hh) * OROW + d], f, o);
      ls = fmaf(s_l[w2][hh], f, ls);
    }
    if (flagged) {
      o = __builtin_nanf("");
      ls = __builtin_nanf("");
    }
    if (single) {
      E::store(out, i, ls != 0.f ? o / ls : 0.f);
    } else {
      a.ws_o[part * G * D + i] = o;
      if (d == 0) a.ws_ml[part * G + h] = make_float2(mx, ls);
    }
  }
}

template <int G, int MODE>
__global__ void __launch_bounds__(kDecodeWaves * kWave, kMma16WorkgroupsPerCu)
decode_mma16_kernel(const DecodeKernelArgs a) {
  decode_mma16_body<G, MODE, false>(a);
}

// the planned decode: one plan item per workgroup
template <int G>
__global__ void __launch_bounds__(kDecodeWaves * kWave, kMma16WorkgroupsPerCu)
decode_planned_kernel(const DecodeKernelArgs a) {
  decode_mma16_body<G, kRopeLazy, true>(a);
}

// Merge the per-split partials of one (sequence, KV head): log-sum-exp weights.
// One workgroup per (sequence, KV head, group of up to 8 query heads); each
// thread merges 4 consecutive dims of one head with 16-byte loads, so that a
// 64-head group's partials (16 times those of a 4-head group) are read with
// few, wide, independent loads.
template <typename T, int D, int G>
__global__ void __launch_bounds__(256)
decode_combine_kernel(const DecodeKernelArgs a) {
  using E = Elem<T>;
  constexpr int GH = G < 8 ? G : 8;  // query heads per workgroup
  constexpr int TPH = D / 4;         // threads per head
  const int hg = blockIdx.x % (G / GH);
  const int g = blockIdx.x / (G / GH);
  const int b = blockIdx.y;
  const int h = hg * GH + threadIdx.x / TPH;
  const int d = 4 * (threadIdx.x % TPH);
  const int hkv = a.num_kv_heads;
  const int seq_len = a.seq_lens[b];
  if (seq_len < 0 || seq_len > a.max_blocks * kBlockTokens) return;  // written by the split kernel
  const int nblk = (seq_len + kBlockTokens - 1) / kBlockTokens;
  const int nsplit = a.plan_counts ? a.plan_counts[b] : (nblk + a.split_blocks - 1) / a.split_blocks;
  if (nblk == 0 || nsplit <= 1 || nsplit > a.max_splits) return;
  const size_t part = ((size_t)b * hkv + g) * a.max_splits;
  const float4 *po = (const float4 *)(a.ws_o + (part * G + h) * D + d);
  const float2 *pml = a.ws_ml + part * G + h;
  float mx = -INFINITY;
  for (int sp = 0; sp < nsplit; ++sp) mx = fmaxf(mx, pml[sp * G].x);
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  float lsum = 0.f;
#pragma unroll 4
  for (int sp = 0; sp < nsplit; ++sp) {
    const float2 ml = pml[sp * G];
    const float f = fast_exp2(ml.x - mx);
    const float4 v = po[(size_t)sp * (G * D / 4)];
    o.x = fmaf(v.x, f, o.x);
    o.y = fmaf(v.y, f, o.y);
    o.z = fmaf(v.z, f, o.z);
    o.w = fmaf(v.w, f, o.w);
    lsum = fmaf(ml.y, f, lsum);
  }
  T *out = (T *)a.out + (((size_t)b * hkv + g) * G + h) * D + d;
  const bool any = lsum != 0.f;  // no visible token -> 0 (NaN stays NaN)
  E::store(out, 0, any ? o.x / lsum * a.out_scale : 0.f);
  E::store(out, 1, any ? o.y / lsum * a.out_scale : 0.f);
  E::store(out, 2, any ? o.z / lsum * a.out_scale : 0.f);
  E::store(out, 3, any ? o.w / lsum * a.out_scale : 0.f);
}

// ------------------------------------------------------------------- host side
static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// bf16 pools with head_dim 128 always take the matrix-core kernels: measured
// against the VALU kernel on 8B-sized contexts they are as fast for query
// groups of 1 and 2 and faster from 4 on (GQA-8: 4.6 -> 5.5 TB/s).  The VALU
// kernel serves fp32 and head_dim 64.
int decode_impl(bool pool8, bool bf16, int head_dim) {
  if (pool8) return kDecodeMma8;
  return bf16 && head_dim == 128 ? kDecodeMma16 : kDecodeValu;
}

// Workgroups that share one KV head's query heads.  VALU kernel: G = 8 keeps
// 8 heads x 8 dims of output accumulators per lane and caps the kernel at one
// wave per SIMD, too few loads in flight to cover HBM latency; two workgroups
// of 4 heads each (sharing every K/V block through L2) run at two waves per
// SIMD, and larger groups (multi-query attention) take G / 4 workgroups of 4
// heads.  The 8-bit matrix-core kernel takes up to 16 query heads (one MFMA
// column each) per workgroup; the bf16 one takes every group up to 64 in one
// workgroup (decode_mma16_wide_kernel above 16).
int decode_head_split(int num_q_heads, int num_kv_heads, int impl) {
  const int group = num_q_heads / num_kv_heads;
  if (impl == kDecodeMma16) return 1;
  if (impl == kDecodeMma8) return group > 16 ? group / 16 : 1;
  return group >= 8 ? group / 4 : 1;  // MQA-like groups (16..64): 4..16 workgroups of 4 heads
}

int decode_split_blocks(int batch, int num_q_heads, int num_kv_heads, int max_blocks_per_seq,
                        int requested, int impl) {
  if (requested > 0) return requested;
  // Workgroups to aim at: one round of resident workgroups, as few as keep
  // the chip's HBM share busy.  The bf16 matrix-core kernels run one
  // workgroup per CU (256; a 64-head group runs 8 waves), the 8-bit kernel
  // two (512), the VALU kernel ~1024.  Measured with launches interleaved: at
  // ~0.5 GB of K/V and 120 (sequence, KV head) units, 2 splits instead of 4
  // took 8-9 % off bf16 GQA 4 and a 32-head group, and 2 % off the bf16 70B
  // shape (128 units); the 8-bit kernel (three workgroups fit a CU) was 34 %
  // slower at 2 splits than at 4 there, and 3, 5 or 6 were also slower.
  // Splits also cost their partials (written, then merged by a second kernel),
  // and a second, partial round of workgroups cost 9 % on the 70B shape.
  const long long units = (long long)batch * num_kv_heads * decode_head_split(num_q_heads, num_kv_heads, impl);
  const long long target = impl == kDecodeValu ? 1024 : impl == kDecodeMma16 ? 256 : 512;
  if (units >= target) return max_blocks_per_seq;  // one split each
  // splits per unit: as many as keep units x splits within the target (the
  // block count per split is rounded up, which never adds a split)
  const long long splits = target / units;
  long long sb = (max_blocks_per_seq + splits - 1) / splits;
  if (sb < 32) sb = 32;
  sb = (sb + kDecodeWaves - 1) / kDecodeWaves * kDecodeWaves;
  return (int)sb;
}

// Partials of `splits` slots per (sequence, work head): (max, sum) pairs, then
// the outputs at off_o (256-byte aligned).
static void workspace_layout(int batch, int num_q_heads, int num_kv_heads, int head_dim, size_t splits,
                             size_t *off_o, size_t *total) {
  const size_t units = (size_t)batch * num_kv_heads;
  const size_t group = (size_t)(num_q_heads / num_kv_heads);
  *off_o = align_up(units * splits * group * sizeof(float2), 256);
  *total = *off_o + units * splits * group * head_dim * sizeof(float);
}

// The partials' size depends only on the number of splits (units x heads per
// unit is the query head count); it covers every kernel's split choice.
size_t decode_workspace_size(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                             int max_blocks_per_seq, int split_blocks) {
  size_t need = 0;
  for (const int impl : {kDecodeValu, kDecodeMma8, kDecodeMma16}) {
    const int sb = decode_split_blocks(batch, num_q_heads, num_kv_heads, max_blocks_per_seq, split_blocks, impl);
    if ((max_blocks_per_seq + sb - 1) / sb <= 1) continue;  // one split: no partials
    size_t off_o, t;
    workspace_layout(batch, num_q_heads, num_kv_heads, head_dim, (size_t)((max_blocks_per_seq + sb - 1) / sb),
                     &off_o, &t);
    need = t > need ? t : need;
  }
  return need;
}

size_t decode_planned_workspace_size(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                     int max_items_per_seq) {
  if (max_items_per_seq <= 1) return 0;
  size_t off_o, t;
  workspace_layout(batch, num_q_heads, num_kv_heads, head_dim, (size_t)max_items_per_seq, &off_o, &t);
  return t;
}

size_t decode_plan_items_offset(int batch) { return ((size_t)batch + 3) / 4 * 4; }

// IMPL: kValu (decode_split_kernel), kMma8 (8-bit pools), kMma16 (bf16 pools,
// matrix cores, up to 16 heads), kMma16Wide (bf16 pools, 32 or 64 heads)
enum DecodeImplKernel { kValu = 0, kMma8 = 1, kMma16 = 2, kMma16Wide = 3, kMma8Int8 = 4 };

template <typename T, int D, int G, int MODE, bool F8 = false, int IMPL = kValu>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t stream) {
  if (a.plan) return hipErrorInvalidValue;  // plans go to launch_decode_planned
  DecodeKernelArgs k;
  k.out = a.out;
  k.q = a.q;
  k.q_pos = a.q_pos;
  k.k_pool = (const uint4 *)a.k_pool;
  k.v_pool = (const uint4 *)a.v_pool;
  k.table = a.table;
  k.seq_lens = a.seq_lens;
  k.slopes = a.slopes;
  k.fill4 = (const uint32_t *)a.block_fill;
  const int hsplit = a.num_q_heads / a.num_kv_heads / G;  // work heads per KV head
  const int work_heads = a.num_kv_heads * hsplit;
  k.max_blocks = a.max_blocks;
  k.num_kv_heads = work_heads;
  k.kv_shift = __builtin_ctz((unsigned)hsplit);  // hsplit is a power of two
  k.num_blocks = a.num_blocks;
  k.split_blocks = a.split_blocks;
  k.max_splits = (a.max_blocks + a.split_blocks - 1) / a.split_blocks;
  k.batch = a.batch;
  k.plan_counts = nullptr;
  k.plan_items = nullptr;
  k.scale_log2 = a.scale * kLog2e * (F8 ? a.k_scale : 1.f);
  k.out_scale = F8 ? a.v_scale : 1.f;
  k.rope_theta = a.rope_theta;
  const long long units = (long long)k.max_splits * a.num_kv_heads * a.batch;
  const long long grid = (units + kXcds - 1) / kXcds * kXcds * hsplit;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  k.num_units = (int)units;
  size_t off_o, total;
  workspace_layout(a.batch, a.num_q_heads, work_heads, a.head_dim, (size_t)k.max_splits, &off_o, &total);
  char *ws = (char *)a.workspace;
  k.ws_ml = ws ? (float2 *)ws : nullptr;
  k.ws_o = ws ? (float *)(ws + off_o) : nullptr;
  if constexpr (IMPL == kMma8)
    hipLaunchKernelGGL((decode_mma8_kernel<G, MODE>), dim3((unsigned)grid), dim3(kDecodeWaves * kWave), 0, stream,
                       k);
  else if constexpr (IMPL == kMma8Int8)
    hipLaunchKernelGGL((decode_int8_kernel<G>), dim3((unsigned)grid), dim3(kDecodeWaves * kWave), 0, stream, k);
  else if constexpr (IMPL == kMma16Wide)
    hipLaunchKernelGGL((decode_mma16_wide_kernel<G / 16, MODE>), dim3((unsigned)grid),
                       dim3(wide_waves(G / 16) * kWave), 0, stream, k);
  else if constexpr (IMPL == kMma16)
    hipLaunchKernelGGL((decode_mma16_kernel<G, MODE>), dim3((unsigned)grid), dim3(kDecodeWaves * kWave), 0, stream,
                       k);
  else
    hipLaunchKernelGGL((decode_split_kernel<T, D, G, MODE>), dim3((unsigned)grid), dim3(kDecodeWaves * kWave),
                       0, stream, k);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || k.max_splits <= 1) return e;
  constexpr int kGh = G < 8 ? G : 8;
  hipLaunchKernelGGL((decode_combine_kernel<T, D, G>), dim3((unsigned)(work_heads * (G / kGh)), (unsigned)a.batch),
                     dim3(kGh * D / 4), 0, stream, k);
  return hipGetLastError();
}

// Planned decode (bf16 pools, head_dim 128, lazy RoPE): one workgroup per
// plan item, then the combine over each sequence's slots.
template <int G>
static hipError_t launch_planned_t(const DecodeArgs &a, hipStream_t stream) {
  DecodeKernelArgs k;
  k.out = a.out;
  k.q = a.q;
  k.q_pos = a.q_pos;
  k.k_pool = (const uint4 *)a.k_pool;
  k.v_pool = (const uint4 *)a.v_pool;
  k.table = a.table;
  k.seq_lens = a.seq_lens;
  k.slopes = nullptr;
  k.fill4 = (const uint32_t *)a.block_fill;
  k.max_blocks = a.max_blocks;
  k.num_kv_heads = a.num_kv_heads;
  k.kv_shift = 0;
  k.num_units = a.plan_items;
  k.num_blocks = a.num_blocks;
  k.split_blocks = 0;  // unused: slots come from the plan
  k.max_splits = a.plan_max_items;
  k.scale_log2 = a.scale * kLog2e;
  k.rope_theta = a.rope_theta;
  k.out_scale = 1.f;
  k.batch = a.batch;
  k.plan_counts = a.plan;
  k.plan_items = (const int4 *)(a.plan + decode_plan_items_offset(a.batch));
  size_t off_o, total;
  workspace_layout(a.batch, a.num_q_heads, a.num_kv_heads, a.head_dim, (size_t)k.max_splits, &off_o, &total);
  char *ws = (char *)a.workspace;
  k.ws_ml = ws ? (float2 *)ws : nullptr;
  k.ws_o = ws ? (float *)(ws + off_o) : nullptr;
  hipLaunchKernelGGL((decode_planned_kernel<G>), dim3((unsigned)a.plan_items),
                     dim3(kDecodeWaves * kWave), 0, stream, k);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || k.max_splits <= 1) return e;
  constexpr int kGh = G < 8 ? G : 8;
  hipLaunchKernelGGL((decode_combine_kernel<bf16, 128, G>), dim3((unsigned)(a.num_kv_heads * (G / kGh)),
                     (unsigned)a.batch), dim3(kGh * 128 / 4), 0, stream, k);
  return hipGetLastError();
}

hipError_t launch_decode_planned(const DecodeArgs &a, hipStream_t s) {
  if (!a.plan || a.plan_items < 1 || a.plan_max_items < 1 || a.head_dim != 128 || a.mode != kRopeLazy)
    return hipErrorInvalidValue;
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_planned_t<1>(a, s);
    case 2: return launch_planned_t<2>(a, s);
    case 4: return launch_planned_t<4>(a, s);
    case 8: return launch_planned_t<8>(a, s);
    case 16: return launch_planned_t<16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <int MODE>
static hipError_t dispatch_mma16(const DecodeArgs &a, hipStream_t s) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_decode_t<bf16, 128, 1, MODE, false, kMma16>(a, s);
    case 2: return launch_decode_t<bf16, 128, 2, MODE, false, kMma16>(a, s);
    case 4: return launch_decode_t<bf16, 128, 4, MODE, false, kMma16>(a, s);
    case 8: return launch_decode_t<bf16, 128, 8, MODE, false, kMma16>(a, s);
    case 16: return launch_decode_t<bf16, 128, 16, MODE, false, kMma16>(a, s);
    case 32: return launch_decode_t<bf16, 128, 32, MODE, false, kMma16Wide>(a, s);
    case 64: return launch_decode_t<bf16, 128, 64, MODE, false, kMma16Wide>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int D, int MODE>
static hipError_t dispatch_group_e(const DecodeArgs &a, hipStream_t s) {
  if constexpr (sizeof(T) == 2 && D == 128) {
    if (decode_impl(false, true, D) == kDecodeMma16) return dispatch_mma16<MODE>(a, s);
  }
  switch (a.num_q_heads / a.num_kv_heads / decode_head_split(a.num_q_heads, a.num_kv_heads, kDecodeValu)) {
    case 1: return launch_decode_t<T, D, 1, MODE>(a, s);
    case 2: return launch_decode_t<T, D, 2, MODE>(a, s);
    case 4: return launch_decode_t<T, D, 4, MODE>(a, s);
    case 8: return launch_decode_t<T, D, 8, MODE>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int D>
static hipError_t dispatch_group(const DecodeArgs &a, hipStream_t s) {
  switch (a.mode) {
    case kRopeLazy: return dispatch_group_e<T, D, kRopeLazy>(a, s);
    case kRopeEager: return dispatch_group_e<T, D, kRopeEager>(a, s);
    case kAlibi: return dispatch_group_e<T, D, kAlibi>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// bf16 queries against an 8-bit (E4M3) pool, lazy RoPE, head_dim 128, on the
// matrix cores (the pool in the lane order decode_mma8_kernel reads).
hipError_t launch_decode_fp8(const DecodeArgs &a, hipStream_t s) {
  if (a.head_dim != 128 || a.mode != kRopeLazy) return hipErrorInvalidValue;
  if (a.int8) {
    switch (a.num_q_heads / a.num_kv_heads / decode_head_split(a.num_q_heads, a.num_kv_heads, kDecodeMma8)) {
      case 1: return launch_decode_t<bf16, 128, 1, kRopeLazy, true, kMma8Int8>(a, s);
      case 2: return launch_decode_t<bf16, 128, 2, kRopeLazy, true, kMma8Int8>(a, s);
      case 4: return launch_decode_t<bf16, 128, 4, kRopeLazy, true, kMma8Int8>(a, s);
      case 8: return launch_decode_t<bf16, 128, 8, kRopeLazy, true, kMma8Int8>(a, s);
      case 16: return launch_decode_t<bf16, 128, 16, kRopeLazy, true, kMma8Int8>(a, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (a.num_q_heads / a.num_kv_heads / decode_head_split(a.num_q_heads, a.num_kv_heads, kDecodeMma8)) {
    case 1: return launch_decode_t<bf16, 128, 1, kRopeLazy, true, kMma8>(a, s);
    case 2: return launch_decode_t<bf16, 128, 2, kRopeLazy, true, kMma8>(a, s);
    case 4: return launch_decode_t<bf16, 128, 4, kRopeLazy, true, kMma8>(a, s);
    case 8: return launch_decode_t<bf16, 128, 8, kRopeLazy, true, kMma8>(a, s);
    case 16: return launch_decode_t<bf16, 128, 16, kRopeLazy, true, kMma8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const DecodeArgs &a, bool is_bf16, hipStream_t s) {
  if (is_bf16) {
    switch (a.head_dim) {
      case 64: return dispatch_group<bf16, 64>(a, s);
      case 128: return dispatch_group<bf16, 128>(a, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (a.head_dim) {
    case 16: return dispatch_group<float, 16>(a, s);
    case 64: return dispatch_group<float, 64>(a, s);
    case 128: return dispatch_group<float, 128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lazyattn

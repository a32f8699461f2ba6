// lazyattn_prefill: a prompt's query tiles (M = 128 rows) against the cached
// documents plus the prompt itself, causal within the prompt, on bf16 MFMA.
//
// Method (LazyAttention summary on gist.science, "Implementação Técnica",
// Prefilling): instead of rotating cached keys twice (back to position 0, then
// to the target), one relative rotation per tile is applied.  Since
// rot(q, n) . rot(k, off) = rot(q, n - off) . k ("Equivalência Matemática"),
// the scores equal those against the eager position-adjusted keys.  On gfx950
// the VALU is the scarce unit next to the matrix cores, so the rotation is
// split between the two operands by cost:
//   * the query tile is rotated to one offset per K/V tile, and re-rotated
//     only when that offset changes, i.e. about once per document (3*M*D
//     FLOPs per document instead of 3*N*D per tile);
//   * a K/V tile is always four whole blocks, whether or not it straddles a
//     document boundary; a block whose offset differs from the query's is
//     rotated once in LDS by the difference (the relative rotation of a
//     staged key tile, "Implementação Técnica", Prefilling), by the wave that
//     loaded it.  Tiles are therefore never cut short at a document's end.
//
// Structure (FlashAttention tiling, ai-engineering.academy "Flash
// Attention"): the query tile stays in registers, K/V tiles are staged through
// LDS, S and the running (max, sum) softmax never leave the chip, and O is
// written once.
//
// gfx950 mapping: 4 waves x 32 query rows; v_mfma_f32_16x16x32_bf16.
//   S^T = K Q^T : A = K rows from LDS (row-major, as stored), B = rotated Q in
//                 registers.  The accumulator gives each lane one query column
//                 and 4 keys per 16-key m-tile, which is exactly a B-operand
//                 slice of P^T for the next product (the k-slots are permuted
//                 consistently on both operands), so P never goes through LDS.
//   O^T = V^T P^T : A = V^T, read from the row-major V tile with the
//                 transposing LDS read (ds_read_b64_tr_b16).
//   Weights are 2^(s - r) against a per-row reference r that moves only when
//   a row's running sum leaves [2^-64, 2^64], which skips almost every
//   rescale of the O accumulators.
//   Work items are ordered heaviest first and mapped so that the query heads
//   sharing a KV head run on the same XCD (shared L2 for their K/V tiles).
#include <math.h>

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace lazyattn {

constexpr int kPfWaves = 4;
constexpr int kPfRows = 128;      // query rows per workgroup (M)
constexpr int kPfTileBlocks = 4;  // K/V tile: up to 4 blocks = 64 keys
constexpr int kPfN = kPfTileBlocks * kBlockTokens;
constexpr int kXcds = 8;

struct PrefillKernelArgs {
  uint16_t *out;
  const uint16_t *q;
  const int32_t *cu_q_lens;
  const int32_t *q_pos_start;
  const uint16_t *k_pool;
  const uint16_t *v_pool;
  const uint32_t *table;
  const int32_t *kv_lens;
  const float *slopes;  // ALiBi: per query head
  const uint32_t *fill4;  // per-block fill counts, 4 per word (nullptr: all full)
  int total_q, batch, num_q_heads, num_kv_heads, num_blocks, max_blocks;
  int head_groups;  // workgroups per KV head (G / HP)
  int tok_tiles;    // token tiles per sequence
  int num_units;    // batch * num_kv_heads * head_groups
  float scale_log2, rope_theta;
  float out_scale;  // V scale of an 8-bit pool (1 otherwise)
  int staged;       // 8-bit pools: K/V come from the widened copy (block j of
                    // sequence b at index b * max_blocks + j), not the table
};

// HP query heads of one KV head share a workgroup: rows = HP heads x (128 / HP)
// tokens; wave w owns 32 consecutive rows (one head).
//
// K/V tiles go from HBM straight into LDS (global_load_lds_dwordx4, no
// registers), row-major as in the pool, with the 16-byte chunk index of each
// row XOR-swizzled by the row so that both operand reads are free of bank
// conflicts: K rows feed the A operand of S^T = K Q^T with ds_read_b128, V
// rows feed the A operand of O^T = V^T P^T through two transposing reads.
// Two buffers: the next tile streams in while the current one is computed.
//
// MODE kRopeEager: the non-lazy baseline the method is measured against.  The
// pool then holds keys already rotated to their absolute positions and table
// offsets are ignored, so the query rows are rotated once, by their own
// positions, before the first tile.
// MODE kAlibi: no rotation; a key at position p (block offset + slot) takes the
// bias slope_h * (p - n).  The tiles are
// walked from the last visible block back to the first, so that each row meets
// its largest biases first and the reference below rarely has to move.
//
// PRECISE (lazy RoPE only): the rotated, pre-scaled query is carried as two
// bf16 parts, hi = bf16(q') and lo = bf16(q' - hi), and every K fragment meets
// both (twice the QK products), so q' reaches the matrix cores to ~2^-17
// instead of 2^-9.  A score's error then no longer grows with the spread of
// the scores across keys.  Keys are never rotated either: a K/V tile ends
// where the block offset changes, so each tile's keys all take the query's
// rotation.  The raw query rows are reloaded from memory at each re-rotation to
// make room for the low parts in registers.
//
// 8-bit pools: a bandwidth-bound pass (widen_fp8_kernel) first widens every
// visible block of the batch once, exactly, into a bf16 copy laid out like a
// bf16 pool; this kernel then reads that copy (staged).  Widening inside the
// kernel would repeat it for every query tile that reads a block (64 times
// per block for a 2048-token prompt).  The K scale is folded into the
// rotated query, the V scale into the final normalisation.
template <int D, int HP, int MODE, bool PRECISE>
__global__ void __launch_bounds__(kPfWaves * kWave, 2)
prefill_kernel(const PrefillKernelArgs a) {
  constexpr int KC = D / 32;          // 32-dim k-chunks of the QK product
  constexpr int DT = D / 16;          // 16-dim m-tiles of O^T
  constexpr int HALF = D / 2;
  constexpr int CPR = D / 8;          // 16-byte chunks per key row (the swizzle period)
  constexpr int RPI = kWave / CPR;    // rows per 1 KiB load instruction
  constexpr int IPB = kBlockTokens / RPI;  // load instructions per block (K or V)
  constexpr int ROWB = D * 2;         // bytes per row
  constexpr int TILEB = kPfN * ROWB;  // bytes per K (or V) tile
  constexpr int TOK = kPfRows / HP;   // tokens per workgroup
  constexpr int WPH = kPfWaves / HP;  // waves per head
  static_assert(D == 64 || D == 128, "head_dim must be 64 or 128");
  static_assert(HP == 1 || HP == 2 || HP == 4, "1, 2 or 4 heads per workgroup");
  constexpr bool ALIBI = MODE == kAlibi;
  constexpr bool LAZY = MODE == kRopeLazy;  // table offsets rotate queries and keys
  static_assert(!PRECISE || LAZY, "the hi + lo query is built for lazy RoPE");

  __shared__ __attribute__((aligned(1024))) uint16_t sK[2][TILEB / 2];
  __shared__ __attribute__((aligned(1024))) uint16_t sV[2][TILEB / 2];
  __shared__ float s_turn[HALF];                // theta_i / (2 pi): turns per position
  __shared__ float s_frac[kPfWaves][HALF];       // frac((n0 - off) * turn_i) of the query offset
  __shared__ __attribute__((aligned(16))) float2 s_kcs[kPfWaves][HALF];  // (cos, sin) of a key block's relative rotation
  __shared__ int s_bad;

  // ---- work item: the token tiles of one (sequence, KV head, head group) run
  // consecutively on one XCD (their K/V tiles share its L2), heaviest first
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int unit = (slot / a.tok_tiles) * kXcds + xcd;
  if (unit >= a.num_units) return;
  const int tt = a.tok_tiles - 1 - slot % a.tok_tiles;
  const int hgrp = unit % a.head_groups;
  const int g = (unit / a.head_groups) % a.num_kv_heads;
  const int b = unit / (a.head_groups * a.num_kv_heads);
  const int G = a.num_q_heads / a.num_kv_heads;

  const int q0 = a.cu_q_lens[b];
  const int plen = a.cu_q_lens[b + 1] - q0;
  if (q0 < 0 || plen < 0 || q0 + plen > a.total_q) return;  // rows outside q/out: not written
  if (tt * TOK >= plen) return;
  const int kv_len = a.kv_lens[b];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform: SGPR
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  const int hq = g * G + hgrp * HP + wave / WPH;   // this wave's query head
  const int tw0 = (wave % WPH) * 32;               // this wave's first token in the tile

  const int tok_valid = min(TOK, plen - tt * TOK);
  uint16_t *out = a.out;
  if (plen > kv_len || kv_len > a.max_blocks * kBlockTokens) {  // inconsistent lengths: NaN
    for (int i = lane; i < 32 * D; i += kWave) {
      const int tk = tw0 + i / D;
      if (tk < tok_valid)
        out[((size_t)(q0 + tt * TOK + tk) * a.num_q_heads + hq) * D + i % D] = 0x7fc0;
    }
    return;
  }

  // zero both V buffers once: rows a tile does not load must hold finite values
  for (int i = tid; i < TILEB / 4; i += kPfWaves * kWave) {
    ((uint32_t *)sV[0])[i] = 0u;
    ((uint32_t *)sV[1])[i] = 0u;
  }
  double turn_d = 0.0;  // this lane's frequency in turns per position (lanes < HALF), double
  if (lane < HALF) turn_d = rope_inv_freq(lane, D, a.rope_theta) * 0.15915494309189535;
  if (tid < HALF) s_turn[tid] = (float)turn_d;
  if (tid == 0) s_bad = 0;
  __syncthreads();

  // ---- query rows: this lane holds tokens tw0 + nt*16 + l16 and the dims
  // kc*32 + lg*8 + e.  The raw (bf16, exact) rows stay in registers and are
  // rotated afresh whenever a new document starts.
  const uint4 *qsrc[2];
  bool qok[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int row = tt * TOK + tw0 + nt * 16 + l16;
    qok[nt] = row < plen;
    qsrc[nt] = (const uint4 *)(a.q + ((size_t)(q0 + (qok[nt] ? row : 0)) * a.num_q_heads + hq) * D);
  }

  const int n0 = a.q_pos_start[b] + tt * TOK;    // position of tile token 0
  const int t_lo = kv_len - plen + tt * TOK;     // logical index of tile token 0
  const int t_hi = t_lo + tok_valid - 1;
  const int t_wave = t_lo + tw0;                 // this wave's first token
  const int nblk_vis = t_hi / kBlockTokens + 1;
  const uint32_t *trow = a.table + (size_t)b * a.max_blocks;
  const int hkv = a.num_kv_heads;

  // ---- staging: wave w streams block w of the tile (K then V) into LDS.
  // Lane L of load instruction i fills LDS row r = i*RPI + L/CPR of the block,
  // chunk slot L % CPR, with global chunk (L % CPR) ^ swz(r).  The per-lane
  // source offsets do not depend on the tile; the block base is wave-uniform.
  uint32_t ld_off[IPB];
#pragma unroll
  for (int i = 0; i < IPB; ++i) {
    const int r = i * RPI + lane / CPR;
    ld_off[i] = (uint32_t)(r * ROWB + (((lane % CPR) ^ swz<CPR>(r)) * 16));
  }

  // Table words travel one tile ahead: lanes 0..3 of a VGPR hold the words of
  // blocks jw .. jw+3 (0 past the visible blocks).  A tile's start, length and
  // offset are wave-uniform (scalar registers).
  auto load_words = [&](int jw) -> uint32_t {
    return (lane < kPfTileBlocks && jw + lane < nblk_vis) ? trow[jw + lane] : 0u;
  };
  // the tile starting at block jw: its block count (1..4, never cut at a
  // document boundary) and the offset the query rows are rotated to for it,
  // that of its third block (or last, if shorter): a tile that straddles a
  // boundary takes the offset most of its blocks share, and its other
  // blocks' keys are rotated by the difference (rotate_keys)
  auto tile_of = [&](uint32_t wv, int jw, int &cnt, int &off) {
    cnt = min(kPfTileBlocks, nblk_vis - jw);
    if constexpr (PRECISE) {
      // the tile ends before the first block whose offset differs from its
      // first block's, so no key of it needs a rotation of its own
      off = word_offset((uint32_t)__builtin_amdgcn_readlane((int)wv, 0));
      const uint64_t diff = __ballot(lane < cnt && word_offset(wv) != off);
      if (diff) cnt = (int)__builtin_ctzll(diff);
    } else {
      off = !LAZY ? 0 : word_offset((uint32_t)__builtin_amdgcn_readlane((int)wv, min(2, cnt - 1)));
    }
  };
  // the tile [jw, jw + cnt): wave w < cnt streams block jw + w
  auto issue_tile = [&](uint32_t wv, int jw, int cnt, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    if (wave >= cnt) return;
    uint32_t id = word_block((uint32_t)__builtin_amdgcn_readlane((int)wv, wave));
    if (id >= (uint32_t)a.num_blocks) {
      s_bad = 1;
      id = 0;
    }
    const size_t src = a.staged ? (size_t)b * a.max_blocks + jw + wave : (size_t)id;
    const char *kg = (const char *)a.k_pool + (src * hkv + g) * (kBlockTokens * ROWB);
    const char *vg = (const char *)a.v_pool + (src * hkv + g) * (kBlockTokens * ROWB);
#pragma unroll
    for (int i = 0; i < IPB; ++i) {
      const int dst = (wave * kBlockTokens + i * RPI) * D;  // wave-uniform row base
      lds_dma16(kg, ld_off[i], (uint32_t)(uintptr_t)(lds_ptr_t)(&sK[BUF][dst]));
      lds_dma16(vg, ld_off[i], (uint32_t)(uintptr_t)(lds_ptr_t)(&sV[BUF][dst]));
    }
  };
  // [LA] "Implementação Técnica", Prefilling: one relative rotation of a
  // staged key block.  After this wave's block of the tile has landed, if
  // its offset differs from the offset
  // qoff the query rows are rotated to for this tile, its 16 keys are
  // rotated in place by (offset - qoff), so that rot(q, n - qoff) .
  // rot(k, offset - qoff) = rot(q, n - offset) . k ("Equivalência
  // Matemática").  Lane i < D/2 evaluates frequency i (angle reduced in
  // double to a fraction of a turn); lane (l16, lg) then takes row l16 and
  // the rotate-half chunk pairs (c, c + CPR/2), c = 4 t + lg, whose 16-byte
  // slots are swizzled alike (slot ^ CPR/2): the same lane-to-address map as
  // the K operand read, free of bank conflicts.  The rotated key is rounded
  // to bf16.  Only blocks at a document boundary take this path.
  auto rotate_keys = [&](int cnt, int qoff, uint32_t wv, auto bufc) __attribute__((always_inline)) {
    constexpr int BUF = decltype(bufc)::value;
    constexpr int PPL = CPR / 8;  // chunk pairs per lane
    if constexpr (LAZY && !PRECISE) {
      if (wave >= cnt) return;
      const int delta = word_offset((uint32_t)__builtin_amdgcn_readlane((int)wv, wave)) - qoff;
      if (delta == 0) return;
      if (lane < HALF) {
        const double t = (double)delta * turn_d;
        const float f = (float)(t - rint(t));
        s_kcs[wave][lane] = make_float2(__builtin_amdgcn_cosf(f), __builtin_amdgcn_sinf(f));
      }
      __builtin_amdgcn_wave_barrier();
      char *kb = (char *)sK[BUF] + wave * kBlockTokens * ROWB;
      const int r = l16;
      const int sw = swz<CPR>(r);
#pragma unroll
      for (int t = 0; t < PPL; ++t) {
        const int cp = 4 * t + lg;
        uint4 *px = (uint4 *)(kb + r * ROWB + ((cp ^ sw) * 16));
        uint4 *py = (uint4 *)(kb + r * ROWB + (((cp + CPR / 2) ^ sw) * 16));
        const uint4 x = *px, y = *py;
        const float4 *cs = (const float4 *)&s_kcs[wave][8 * cp];
        uint32_t xo[4], yo[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float4 c2 = cs[k];  // (cos, sin) of frequencies 8 cp + 2k, 8 cp + 2k + 1
          const uint32_t wx = dw4(x, k), wy = dw4(y, k);
          const float x0 = bf16_lo(wx), x1 = bf16_hi(wx), y0 = bf16_lo(wy), y1 = bf16_hi(wy);
          xo[k] = pack_bf16x2(fmaf(x0, c2.x, -(y0 * c2.y)), fmaf(x1, c2.z, -(y1 * c2.w)));
          yo[k] = pack_bf16x2(fmaf(y0, c2.x, x0 * c2.y), fmaf(y1, c2.z, x1 * c2.w));
        }
        *px = make_uint4(xo[0], xo[1], xo[2], xo[3]);
        *py = make_uint4(yo[0], yo[1], yo[2], yo[3]);
      }
    }
  };
  // per lane: the fill count of the block whose table word the lane holds
  auto load_fill = [&](uint32_t wv) -> uint32_t {
    if (!a.fill4) return (uint32_t)kBlockTokens;
    uint32_t id = word_block(wv);
    if (id >= (uint32_t)a.num_blocks) id = 0;
    return (a.fill4[id >> 2] >> ((id & 3u) * 8u)) & 0xffu;
  };
  // after the wave's own loads landed: zero V rows of its block past kv_len
  // or past the block's fill count (their weights are 0; whatever the pool
  // holds there must not turn 0 * x into NaN)
  // tokens of this wave's block of the tile starting at block j that hold data
  auto block_valid = [&](int j, uint32_t fv) -> int {
    return min(kv_len - (j + wave) * kBlockTokens, __builtin_amdgcn_readlane((int)fv, wave));
  };
  auto fix_tail = [&](int j, int cnt, uint32_t fv, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    if (wave >= cnt) return;
    const int valid = block_valid(j, fv);
    if (valid >= kBlockTokens) return;
    for (int i = lane; i < kBlockTokens * CPR; i += kWave) {
      const int r = i / CPR;
      if (r >= valid) *(uint4 *)(&sV[BUF][(wave * kBlockTokens + r) * D + (i % CPR) * 8]) = make_uint4(0u, 0u, 0u, 0u);
    }
  };

  // per-lane LDS read offsets (bytes), independent of the tile and the buffer:
  // K operand rows mt*16 + l16, chunk kc*4 + lg; V^T operand source rows
  // lg*4 + l16/4 (+16, +32ks), dims dt*16 + 4*(l16 % 4)
  uint32_t k_off[KC], v_off[DT];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) k_off[kc] = (uint32_t)(l16 * ROWB + (((kc * 4 + lg) ^ swz<CPR>(l16)) * 16));
  {
    const int vr = lg * 4 + (l16 >> 2);
    const int tdim = (l16 & 3) * 4;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int chunk = (dt * 16 + tdim) / 8;
      v_off[dt] = (uint32_t)(vr * ROWB + ((chunk ^ swz<CPR>(vr)) * 16) + ((dt * 16 + tdim) % 8) * 2);
    }
  }

  // ---- softmax bookkeeping.  Weights are p = 2^(s - r) with a per-row
  // reference r (0 to start), not the running maximum: the common factor 2^-r
  // cancels in O / l.  r moves only when a row's sum would leave
  // [2^-64, 2^64] -- checked per lane against the upper bound every tile, and
  // per row against the lower bound until every row holds a sum -- so no
  // per-tile maximum is needed.
  bf16x8_t bq[2][KC];
  bf16x8_t bql[2][KC];  // PRECISE: the low parts of the rotated query
  f32x4_t O[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) O[dt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float ref[2] = {0.f, 0.f};
  float lsum[2] = {0.f, 0.f};
  bool ref_nz = false;    // wave-uniform: some row's reference is not 0
  bool settled = false;   // wave-uniform: every row holds a sum (>= 2^-64)
  int cur_off = -1;
  constexpr float kHi = 0x1p64f, kLo = 0x1p-64f;

  // tile state (wave-uniform): current tile (cj, ccnt, coff; its words cw);
  // the next tile starts at block nj and its words nw are in flight.  ALiBi
  // walks backwards: tile [cj, cj + ccnt) is followed by [nj, cj).
  int cj = 0, ccnt, coff = 0;
  if constexpr (ALIBI) {
    ccnt = min(kPfTileBlocks, nblk_vis);
    cj = nblk_vis - ccnt;
  }
  // After a tile's loads have landed, before the barrier that publishes it:
  // rotate this wave's block if its offset differs from the query's (lazy
  // RoPE), zero its V rows past the data.  Done at the
  // end of the step before, behind that step's P.V products on the matrix
  // cores, instead of at the start of the tile's own step.
  auto prepare = [&](int j, int cnt, int off, uint32_t wv, uint32_t fv, auto bufc) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0);   // this wave's loads of the tile have landed
    rotate_keys(cnt, off, wv, bufc);
    fix_tail(j, cnt, fv, bufc);
  };

  uint32_t cw = load_words(cj);
  uint32_t cf = load_fill(cw);   // the current tile's fill counts (lanes 0..3)
  if constexpr (!ALIBI) tile_of(cw, 0, ccnt, coff);
  issue_tile(cw, cj, ccnt, std::integral_constant<int, 0>{});
  int nj = ALIBI ? cj - min(kPfTileBlocks, cj) : ccnt;
  uint32_t nw = (ALIBI ? cj > 0 : nj < nblk_vis) ? load_words(nj) : 0u;
  prepare(cj, ccnt, coff, cw, cf, std::integral_constant<int, 0>{});
  // ALiBi: this wave's slope in log2 units, and the workgroup's reference
  // position (its last query token): the bias is taken as slope * (p - nref),
  // which differs from slope * (p - n) by a constant per query row (softmax
  // ignores it) and is <= 0 for every key a row sees
  const float slope2 = ALIBI ? a.slopes[hq] * kLog2e : 0.f;
  const int nref = n0 + TOK - 1;
  // raw (bf16) query rows, loaded once and kept packed in registers for the
  // rotations at document changes
  uint4 qraw[2][KC];
  auto load_rows = [&](uint4 (&r)[2][KC]) __attribute__((always_inline)) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) r[nt][kc] = qok[nt] ? qsrc[nt][kc * 4 + lg] : make_uint4(0u, 0u, 0u, 0u);
  };
  if constexpr (!PRECISE) load_rows(qraw);
  if constexpr (ALIBI) {  // no rotation: q * scale * log2(e), once
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t wx = dw4(qraw[nt][kc], e >> 1);
          bq[nt][kc][e] = (__bf16)(((e & 1) ? bf16_hi(wx) : bf16_lo(wx)) * a.scale_log2);
        }
  }

  // q' = rot(q, rho + n0 - off) * scale * log2(e), rho = token index inside
  // the tile.  The angle in turns is rho * turn_i + frac((n0 - off) *
  // turn_i); the large part is reduced in double, the rest (< TOK turns)
  // evaluated with v_sin/v_cos.
  auto rotate_q = [&](int off) __attribute__((always_inline)) {
    uint4 qre[2][KC];  // PRECISE: the raw rows, reloaded for this rotation
    if constexpr (PRECISE) {
      load_rows(qre);
    } else {
      // opaque to the optimiser: otherwise it hoists the bf16 unpacking out of
      // the tile loop and keeps twice the registers live
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
          asm volatile("" : "+v"(qraw[nt][kc].x), "+v"(qraw[nt][kc].y), "+v"(qraw[nt][kc].z), "+v"(qraw[nt][kc].w));
    }
    auto row = [&](int nt, int kc) -> const uint4 & { return PRECISE ? qre[nt][kc] : qraw[nt][kc]; };
    if (lane < HALF) {
      const double t = (double)(n0 - off) * turn_d;
      s_frac[wave][lane] = (float)(t - rint(t));
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const float rho = (float)(tw0 + nt * 16 + l16);
#pragma unroll
      for (int kc = 0; kc < KC / 2; ++kc) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int fi = kc * 32 + lg * 8 + e;
          const float turns = fmaf(rho, s_turn[fi], s_frac[wave][fi]);
          const float c = __builtin_amdgcn_cosf(turns), s = __builtin_amdgcn_sinf(turns);
          const uint32_t wx = dw4(row(nt, kc), e >> 1), wy = dw4(row(nt, kc + KC / 2), e >> 1);
          const float x = (e & 1) ? bf16_hi(wx) : bf16_lo(wx);
          const float y = (e & 1) ? bf16_hi(wy) : bf16_lo(wy);
          const float fx = fmaf(x, c, -(y * s)) * a.scale_log2;
          const float fy = fmaf(y, c, x * s) * a.scale_log2;
          bq[nt][kc][e] = (__bf16)fx;
          bq[nt][kc + KC / 2][e] = (__bf16)fy;
          if constexpr (PRECISE) {
            bql[nt][kc][e] = (__bf16)(fx - (float)bq[nt][kc][e]);
            bql[nt][kc + KC / 2][e] = (__bf16)(fy - (float)bq[nt][kc + KC / 2][e]);
          }
        }
      }
    }
  };
  // the non-lazy baseline rotates the rows once, by their own positions
  if constexpr (MODE == kRopeEager) rotate_q(0);

  // One tile on LDS buffer BUF; returns false after the last tile.
  auto step = [&](auto bufc) -> bool {
    constexpr int BUF = decltype(bufc)::value;
    __builtin_amdgcn_s_waitcnt(0);   // this tile's K/V and the next tile's words have landed
    // the next tile's fill counts, used when it is prepared and current
    const uint32_t nf = load_fill(nw);
    __syncthreads();                 // every wave's block of this tile is prepared

    const bool more = ALIBI ? cj > 0 : nj < nblk_vis;
    int ncnt = 0, noff = 0, nnj = 0;
    uint32_t nnw = 0u;
    if (more) {
      if constexpr (ALIBI) {
        ncnt = cj - nj;
        nnj = nj - min(kPfTileBlocks, nj);
      } else {
        tile_of(nw, nj, ncnt, noff);
        nnj = nj + ncnt;
      }
      issue_tile(nw, nj, ncnt, std::integral_constant<int, BUF ^ 1>{});  // streams in during this tile
      nnw = (ALIBI ? nj > 0 : nnj < nblk_vis) ? load_words(nnj) : 0u;
    }

    // ---- a new document: re-rotate the query rows (lazy RoPE)
    if (LAZY && coff != cur_off) {
      cur_off = coff;
      rotate_q(coff);
    }

    // ---- S'^T = K Q^T - r  (per lane: keys mt*16 + lg*4 + i, token nt*16 + l16)
    const char *kb = (const char *)sK[BUF];
    f32x4_t S[kPfTileBlocks][2];
    if constexpr (ALIBI) {
      // per-key bias slope * (offset + slot - nref), minus the row reference
#pragma unroll
      for (int mt = 0; mt < kPfTileBlocks; ++mt) {
        const int offm = word_offset((uint32_t)__builtin_amdgcn_readlane((int)cw, mt));
        const float b0 = slope2 * (float)(offm + lg * 4 - nref);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float bias = fmaf(slope2, (float)i, b0);
          S[mt][0][i] = bias - ref[0];
          S[mt][1][i] = bias - ref[1];
        }
      }
    } else if (ref_nz) {
#pragma unroll
      for (int mt = 0; mt < kPfTileBlocks; ++mt) {
        S[mt][0] = f32x4_t{-ref[0], -ref[0], -ref[0], -ref[0]};
        S[mt][1] = f32x4_t{-ref[1], -ref[1], -ref[1], -ref[1]};
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < kPfTileBlocks; ++mt) S[mt][0] = S[mt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    // per 32-key half; a tile of at most 2 blocks (the end of the table)
    // skips the second half's products (its scores are masked below)
    auto qk_half = [&](int h) {
#pragma unroll
      for (int mt = 2 * h; mt < 2 * h + 2; ++mt) {
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          const bf16x8_t ka = as_bf16x8(*(const uint4 *)(kb + mt * 16 * ROWB + k_off[kc]));
          S[mt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, bq[0][kc], S[mt][0], 0, 0, 0);
          S[mt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, bq[1][kc], S[mt][1], 0, 0, 0);
          if constexpr (PRECISE) {
            S[mt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, bql[0][kc], S[mt][0], 0, 0, 0);
            S[mt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, bql[1][kc], S[mt][1], 0, 0, 0);
          }
        }
      }
    };
    qk_half(0);
    if (ccnt > kPfTileBlocks / 2) qk_half(1);

    // ---- mask: keys past the tile's blocks, past kv_len, or after the query token;
    // and slots past a block's fill count.  Per lane and query column, keys
    // mt*16 + lg*4 + i of the tile stay when mt*16 + i <= lim and
    // lg*4 + i < fill(mt).
    const int key0 = cj * kBlockTokens;
    if (ccnt < kPfTileBlocks || key0 + kPfN > kv_len || key0 + kPfN - 1 > t_wave) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int last = min(min(kv_len - 1, t_wave + nt * 16 + l16), key0 + ccnt * kBlockTokens - 1);
        const int lim = last - key0 - lg * 4;
#pragma unroll
        for (int mt = 0; mt < kPfTileBlocks; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (mt * 16 + i > lim) S[mt][nt][i] = -INFINITY;
      }
    }
    if (wave_any(lane < ccnt && cf < (uint32_t)kBlockTokens)) {
#pragma unroll
      for (int mt = 0; mt < kPfTileBlocks; ++mt) {
        const int flim = __builtin_amdgcn_readlane((int)cf, mt) - 1 - lg * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i > flim) S[mt][0][i] = S[mt][1][i] = -INFINITY;
      }
    }

    // ---- weights p = 2^S' (bf16, as P.V uses them) and the lane's row sums
    bf16x8_t bp[2][2];  // [ks][nt]: keys 32ks + {lg*4 + 0..3, 16 + lg*4 + 0..3}
    float ln[2];
    auto weights = [&]() {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
        for (int mt = 0; mt < kPfTileBlocks; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) bp[mt >> 1][nt][(mt & 1) * 4 + i] = (__bf16)__builtin_amdgcn_exp2f(S[mt][nt][i]);
        float l = lsum[nt];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const uint4 pw = __builtin_bit_cast(uint4, bp[ks][nt]);
          l = dot2_bf16(pw.x, 0x3f803f80u, l);
          l = dot2_bf16(pw.y, 0x3f803f80u, l);
          l = dot2_bf16(pw.z, 0x3f803f80u, l);
          l = dot2_bf16(pw.w, 0x3f803f80u, l);
        }
        ln[nt] = l;
      }
    };
    weights();
    bool bad = !(ln[0] <= kHi) || !(ln[1] <= kHi);   // NaN counts as bad
    if (!settled) bad |= !(col_sum4(ln[0]) >= kLo) || !(col_sum4(ln[1]) >= kLo);
    if (wave_any(bad)) {
      // Rare: move the reference of every row whose sum left the range to
      // max(tile maximum, log2 of the sum so far), rescale what the row holds,
      // and recompute its weights.  Afterwards such a row's sum is in [1, 65].
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        float x = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < kPfTileBlocks; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) x = fmaxf(x, S[mt][nt][i]);
        const float tmax = col_max4(x);
        const float t_old = col_sum4(lsum[nt]);
        const float t_new = col_sum4(ln[nt]);
        float sh = 0.f;
        if (!(t_new >= kLo && t_new <= kHi)) {
          sh = fmaxf(tmax, t_old > 0.f ? __builtin_amdgcn_logf(t_old) : -INFINITY);
          if (!(sh > -INFINITY && sh < INFINITY)) sh = 0.f;
        }
        // alpha = 2^-sh = half^2, applied in two steps: with a sum so far,
        // sh >= log2(sum) >= -149 keeps half <= 2^74.5; without one, the row
        // holds only zeros and alpha is irrelevant (0 avoids 0 * inf)
        const float half = t_old > 0.f ? __builtin_amdgcn_exp2f(-0.5f * sh) : 0.f;
        ref[nt] += sh;
        lsum[nt] = lsum[nt] * half * half;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) O[dt][nt] = O[dt][nt] * half * half;
#pragma unroll
        for (int mt = 0; mt < kPfTileBlocks; ++mt) S[mt][nt] -= sh;
      }
      weights();
      ref_nz = wave_any(ref[0] != 0.f || ref[1] != 0.f);
    }
    // A row's sum is now >= 2^-64 (after a rescale: >= 1) or 0 because no
    // key of the row has been visible yet (a later tile holds them: the first
    // tile need not reach every row when the walk starts at the far end).
    // Stop checking the lower bound once every row of the wave holds a sum.
    if (!settled) settled = !wave_any(!(col_sum4(ln[0]) > 0.f) || !(col_sum4(ln[1]) > 0.f));
    lsum[0] = ln[0];
    lsum[1] = ln[1];

    // ---- O^T += V^T P^T: A operand rows = dims, k-slots = keys
    // 32ks + lg*4 + 0..3 and 32ks + 16 + lg*4 + 0..3, read transposed.
    const char *vb = (const char *)sV[BUF];
    auto pv_half = [&](int ks) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint2 lo = lds_read_tr16((const uint16_t *)(vb + ks * 32 * ROWB + v_off[dt]));
        const uint2 up = lds_read_tr16((const uint16_t *)(vb + (ks * 32 + 16) * ROWB + v_off[dt]));
        const bf16x8_t va = as_bf16x8(make_uint4(lo.x, lo.y, up.x, up.y));
        O[dt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, bp[ks][0], O[dt][0], 0, 0, 0);
        O[dt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, bp[ks][1], O[dt][1], 0, 0, 0);
      }
    };
    pv_half(0);
    if (ccnt > kPfTileBlocks / 2) pv_half(1);   // a short tile has no keys there

    if (!more) return false;
    prepare(nj, ncnt, noff, nw, nf, std::integral_constant<int, BUF ^ 1>{});
    cj = nj;
    ccnt = ncnt;
    coff = noff;
    cw = nw;
    cf = nf;
    nj = nnj;
    nw = nnw;
    return true;
  };
  for (;;) {
    if (!step(std::integral_constant<int, 0>{})) break;
    if (!step(std::integral_constant<int, 1>{})) break;
  }

  // ---- normalise and write: lane holds O^T[dt*16 + lg*4 + i][token nt*16 + l16]
  __syncthreads();  // s_bad is final
  const bool flagged = s_bad != 0;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const float tot = col_sum4(lsum[nt]);
    // a row with no visible token (fill counts below its own slot) gives 0
    const float inv = flagged ? __builtin_nanf("") : tot != 0.f ? a.out_scale / tot : 0.f;
    const int tk = tw0 + nt * 16 + l16;
    if (tk < tok_valid) {
      uint16_t *dst = out + ((size_t)(q0 + tt * TOK + tk) * a.num_q_heads + hq) * D + lg * 4;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint2 pk = make_uint2(pack_bf16x2(O[dt][nt][0] * inv, O[dt][nt][1] * inv),
                                    pack_bf16x2(O[dt][nt][2] * inv, O[dt][nt][3] * inv));
        *(uint2 *)(dst + dt * 16) = pk;
      }
    }
  }
}

template <int D, int HP, int MODE, bool PRECISE = false>
static hipError_t launch_prefill_t(const PrefillArgs &a, hipStream_t stream) {
  PrefillKernelArgs k;
  k.out = (uint16_t *)a.out;
  k.q = (const uint16_t *)a.q;
  k.total_q = a.total_q;
  k.cu_q_lens = a.cu_q_lens;
  k.q_pos_start = a.q_pos_start;
  k.k_pool = (const uint16_t *)a.k_pool;
  k.v_pool = (const uint16_t *)a.v_pool;
  k.table = a.table;
  k.kv_lens = a.kv_lens;
  k.slopes = a.slopes;
  k.fill4 = (const uint32_t *)a.block_fill;
  k.batch = a.batch;
  k.num_q_heads = a.num_q_heads;
  k.num_kv_heads = a.num_kv_heads;
  k.num_blocks = a.num_blocks;
  k.max_blocks = a.max_blocks;
  k.head_groups = a.num_q_heads / a.num_kv_heads / HP;
  constexpr int tok = kPfRows / HP;
  k.tok_tiles = (a.max_q_len + tok - 1) / tok;
  k.num_units = a.batch * a.num_kv_heads * k.head_groups;
  k.scale_log2 = a.scale * kLog2e * a.k_scale;
  k.out_scale = a.v_scale;
  k.staged = a.staged;
  k.rope_theta = a.rope_theta;
  const long long grid = (long long)(k.num_units + kXcds - 1) / kXcds * kXcds * k.tok_tiles;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_kernel<D, HP, MODE, PRECISE>), dim3((unsigned)grid), dim3(kPfWaves * kWave), 0,
                     stream, k);
  return hipGetLastError();
}

template <int D, int MODE, bool PRECISE = false>
static hipError_t launch_prefill_e(const PrefillArgs &a, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  if (group % 4 == 0) return launch_prefill_t<D, 4, MODE, PRECISE>(a, stream);
  if (group % 2 == 0) return launch_prefill_t<D, 2, MODE, PRECISE>(a, stream);
  return launch_prefill_t<D, 1, MODE, PRECISE>(a, stream);
}

template <int D>
static hipError_t launch_prefill_d(const PrefillArgs &a, hipStream_t stream) {
  if (a.precise) return a.mode == kRopeLazy ? launch_prefill_e<D, kRopeLazy, true>(a, stream) : hipErrorInvalidValue;
  switch (a.mode) {
    case kRopeLazy: return launch_prefill_e<D, kRopeLazy>(a, stream);
    case kRopeEager: return launch_prefill_e<D, kRopeEager>(a, stream);
    case kAlibi: return launch_prefill_e<D, kAlibi>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

// ---- 8-bit pools: widen every visible block once into a bf16 copy
struct WidenArgs {
  const uint8_t *k_codes, *v_codes;  // the 8-bit pools, 2 KiB per (block, KV head)
  const uint32_t *table;
  const int32_t *kv_lens;
  uint16_t *k_out, *v_out;           // [batch][max_blocks][num_kv_heads][16][128] bf16
  int batch, max_blocks, num_kv_heads, num_blocks;
};

// One wave per (sequence, block slot, KV head), KV head fastest; a slot past
// the sequence's length, or whose table word names no block, is skipped (the
// prefill kernel never reads the former and flags the latter).  Codes are
// stored in the decode's lane order (byte 1024 i + 16 l + x, l = 16 g + t):
// K[t][32 g + 16 i + x] and V[4 g + x % 4][16 (4 i + x / 4) + t].  K goes
// straight to its row-major place (32 contiguous bytes per lane and chunk);
// V is transposed through LDS so that every store is a contiguous 1 KiB.
// Widening E4M3 or int8 codes to bf16 is exact.
template <int FMT>
__device__ __forceinline__ void widen8_body(const WidenArgs &a) {
  // V rows padded to 272 bytes: the transposing stores write 4 rows at once
  // (one per lane group), which unpadded start in the same LDS bank
  constexpr int VROW = 136;
  __shared__ __attribute__((aligned(16))) uint16_t s_v[4][kBlockTokens * VROW];
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const size_t item = (size_t)blockIdx.x * 4 + wave;
  const int hkv = a.num_kv_heads;
  if (item >= (size_t)a.batch * a.max_blocks * hkv) return;
  const int g = (int)(item % hkv);
  const size_t slot = item / hkv;
  const int j = (int)(slot % a.max_blocks);
  const int b = (int)(slot / a.max_blocks);
  const int kv_len = a.kv_lens[b];
  if (kv_len <= 0 || kv_len > a.max_blocks * kBlockTokens || j * kBlockTokens >= kv_len) return;
  const uint32_t id = word_block(a.table[slot]);
  if (id >= (uint32_t)a.num_blocks) return;
  const uint4 *kr = (const uint4 *)(a.k_codes + ((size_t)id * hkv + g) * 2048);
  const uint4 *vr = (const uint4 *)(a.v_codes + ((size_t)id * hkv + g) * 2048);
  uint16_t *ko = a.k_out + item * (kBlockTokens * 128);
  uint4 *vo = (uint4 *)(a.v_out + item * (kBlockTokens * 128));
  const int t = lane & 15, gq = lane >> 4;
  uint4 kc[2], vc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    kc[i] = kr[64 * i + lane];
    vc[i] = vr[64 * i + lane];
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    uint32_t w[8];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      w[2 * d] = code8x2_to_bf16x2<FMT, false>(dw4(kc[i], d));
      w[2 * d + 1] = code8x2_to_bf16x2<FMT, true>(dw4(kc[i], d));
    }
    uint4 *dst = (uint4 *)(ko + t * 128 + 32 * gq + 16 * i);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
  // Lanes t and t ^ 1 hold dims 2m and 2m + 1 (m = t / 2) of the same four
  // rows.  One swap gives each the other's values for two rows, so that each
  // writes whole 4-byte words (both dims): the even lane rows 4 gq and
  // 4 gq + 1, the odd lane rows 4 gq + 2 and 4 gq + 3.
  uint16_t *sv = s_v[wave];
  const bool odd = t & 1;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint32_t c = dw4(vc[i], jj);
      const uint32_t lo = code8x2_to_bf16x2<FMT, false>(c), hi = code8x2_to_bf16x2<FMT, true>(c);  // rows (0,1), (2,3)
      const uint32_t give = odd ? lo : hi;
      const uint32_t got = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)give, kDppQuadXor1, 0xf, 0xf, false);
      const uint32_t mine = odd ? hi : lo;
      // word of the first row: (even lane's value, odd lane's value) in dim order
      const uint32_t w0 = odd ? ((got & 0xffffu) | (mine << 16)) : ((mine & 0xffffu) | (got << 16));
      const uint32_t w1 = odd ? ((got >> 16) | (mine & 0xffff0000u)) : ((mine >> 16) | (got & 0xffff0000u));
      const int row = 4 * gq + (odd ? 2 : 0);
      const int dim = 16 * (4 * i + jj) + (t & ~1);
      *(uint32_t *)(sv + row * VROW + dim) = w0;
      *(uint32_t *)(sv + (row + 1) * VROW + dim) = w1;
    }
  }
  __builtin_amdgcn_wave_barrier();  // a wave's LDS accesses complete in order
#pragma unroll
  // read back row-major; the 16 lanes of a row take its chunks rotated by
  // the row, so that with the padded rows every 16-lane group of a 16-byte
  // read meets 16 different bank slots
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * r + lane / 16;
    const int c = (lane - lane / 16) & 15;
    vo[row * 16 + c] = *(const uint4 *)(sv + row * VROW + c * 8);
  }
}

__global__ void __launch_bounds__(4 * kWave) widen_fp8_kernel(const WidenArgs a) { widen8_body<kCodeE4M3>(a); }
__global__ void __launch_bounds__(4 * kWave) widen_int8_kernel(const WidenArgs a) { widen8_body<kCodeInt8>(a); }

size_t prefill_fp8_workspace_size(int batch, int max_blocks, int num_kv_heads) {
  if (batch <= 0 || max_blocks <= 0 || num_kv_heads <= 0) return 0;
  return 2 * (size_t)batch * max_blocks * num_kv_heads * (kBlockTokens * 128 * sizeof(uint16_t));
}

// bf16 queries against 8-bit (E4M3 or int8) pools in the decode's lane order,
// lazy RoPE, head_dim 128: widen, then the bf16 kernel on the widened copy.
hipError_t launch_prefill_fp8(const PrefillArgs &a, void *workspace, hipStream_t stream) {
  if (a.head_dim != 128 || a.mode != kRopeLazy || !workspace) return hipErrorInvalidValue;
  const size_t half = prefill_fp8_workspace_size(a.batch, a.max_blocks, a.num_kv_heads) / 2;
  WidenArgs w;
  w.k_codes = (const uint8_t *)a.k_pool;
  w.v_codes = (const uint8_t *)a.v_pool;
  w.table = a.table;
  w.kv_lens = a.kv_lens;
  w.k_out = (uint16_t *)workspace;
  w.v_out = (uint16_t *)((char *)workspace + half);
  w.batch = a.batch;
  w.max_blocks = a.max_blocks;
  w.num_kv_heads = a.num_kv_heads;
  w.num_blocks = a.num_blocks;
  const long long items = (long long)a.batch * a.max_blocks * a.num_kv_heads;
  const long long wgs = (items + 3) / 4;
  if (wgs <= 0) return hipSuccess;
  if (wgs > 0x7fffffffLL) return hipErrorInvalidValue;
  if (a.int8) hipLaunchKernelGGL(widen_int8_kernel, dim3((unsigned)wgs), dim3(4 * kWave), 0, stream, w);
  else hipLaunchKernelGGL(widen_fp8_kernel, dim3((unsigned)wgs), dim3(4 * kWave), 0, stream, w);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  PrefillArgs s = a;
  s.k_pool = w.k_out;
  s.v_pool = w.v_out;
  s.staged = 1;
  if (a.precise) return launch_prefill_e<128, kRopeLazy, true>(s, stream);
  return launch_prefill_e<128, kRopeLazy>(s, stream);
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream) {
  switch (a.head_dim) {
    case 64: return launch_prefill_d<64>(a, stream);
    case 128: return launch_prefill_d<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lazyattn

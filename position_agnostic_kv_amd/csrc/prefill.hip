// lazyattn_prefill: a prompt's query tiles (M = 128 rows) against the cached
// documents plus the prompt itself, causal within the prompt, on bf16 MFMA.
//
// Method (LazyAttention summary on gist.science, "Implementação Técnica",
// Prefilling): instead of rotating cached keys twice (back to position 0, then
// to the target), one relative rotation per tile is applied.  Here the rotation
// goes on the query tile: a K/V tile is a run of up to four blocks that share
// one offset, and the query tile is re-rotated by (tile start position - offset)
// only when that offset changes, i.e. once per document.  Since
// rot(q, n) . rot(k, off) = rot(q, n - off) . k ("Equivalência Matemática"),
// the scores equal those against the eager position-adjusted keys.  On gfx950
// the VALU is the scarce unit next to the matrix cores, and this costs
// 3*M*D FLOPs per document instead of 3*N*D per tile (rotating each staged
// key tile), with K never re-rounded.
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
//   O^T = V^T P^T : A = V^T, staged transposed into LDS.
//   The row max is raised only when a tile exceeds it by more than 2^8, which
//   skips almost every rescale of the O accumulators.
//   Work items are ordered heaviest first and mapped so that the query heads
//   sharing a KV head run on the same XCD (shared L2 for their K/V tiles).
#include <math.h>

#include "common.h"
#include "launch.h"

namespace lazyattn {

constexpr int kPfWaves = 4;
constexpr int kPfM = 128;         // query rows per workgroup
constexpr int kPfTileBlocks = 4;  // K/V tile: up to 4 blocks = 64 keys
constexpr int kPfN = kPfTileBlocks * kBlockTokens;
constexpr float kPfSlack = 8.0f;
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
  int total_q, batch, num_q_heads, num_kv_heads, num_blocks, max_blocks, q_tiles, num_units;
  float scale_log2, rope_theta;
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

template <int D>
__global__ void __launch_bounds__(kPfWaves * kWave)
prefill_kernel(const PrefillKernelArgs a) {
  constexpr int KC = D / 32;          // 32-dim k-chunks of the QK product
  constexpr int DT = D / 16;          // 16-dim m-tiles of O^T
  constexpr int HALF = D / 2;
  constexpr int KSTR = D + 8;         // sK row stride (bf16)
  constexpr int VSTR = kPfN + 4;      // sVt row stride (bf16)
  constexpr int CPR = D / 8;          // 16-byte chunks per key row
  constexpr int NT = kPfWaves * kWave;
  static_assert(D == 64 || D == 128, "head_dim must be 64 or 128");

  __shared__ __attribute__((aligned(16))) uint16_t sK[kPfN * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[D * VSTR];
  __shared__ double s_invf[HALF];
  __shared__ int s_bad;

  // ---- work item: heavy-first units of (q tile, sequence, KV head), the G
  // query heads of a unit consecutive on one XCD
  const int G = a.num_q_heads / a.num_kv_heads;
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int unit = (slot / G) * kXcds + xcd;
  if (unit >= a.num_units) return;
  const int hi = slot % G;
  const int g = unit % a.num_kv_heads;
  const int rest = unit / a.num_kv_heads;
  const int b = rest % a.batch;
  const int qt = a.q_tiles - 1 - rest / a.batch;
  const int hq = g * G + hi;

  const int q0 = a.cu_q_lens[b];
  const int plen = a.cu_q_lens[b + 1] - q0;
  if (q0 < 0 || plen < 0 || q0 + plen > a.total_q) return;  // rows outside q/out: not written
  if (qt * kPfM >= plen) return;
  const int kv_len = a.kv_lens[b];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int l16 = lane & 15;
  const int lg = lane >> 4;

  const int rows_valid = min(kPfM, plen - qt * kPfM);
  uint16_t *out = a.out;
  if (plen > kv_len || kv_len > a.max_blocks * kBlockTokens) {  // inconsistent lengths: NaN
    for (int i = tid; i < rows_valid * D; i += NT) {
      const int rr = i / D, d = i % D;
      out[((size_t)(q0 + qt * kPfM + rr) * a.num_q_heads + hq) * D + d] = 0x7fc0;
    }
    return;
  }

  if (tid < HALF) s_invf[tid] = rope_inv_freq(tid, D, a.rope_theta);
  if (tid == 0) s_bad = 0;
  __syncthreads();

  // ---- query tile: this lane holds rows (nt*16 + l16) of the wave's 32 and the
  // dims kc*32 + lg*8 + e; q_rho = rot(q, rho), rho = row index inside the tile.
  float qf[2][KC][8];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int rho = wave * 32 + nt * 16 + l16;
    const int row = qt * kPfM + rho;
    const bool ok = row < plen;
    const uint4 *src = (const uint4 *)(a.q + ((size_t)(q0 + (ok ? row : 0)) * a.num_q_heads + hq) * D);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const uint4 v = ok ? src[kc * 4 + lg] : make_uint4(0u, 0u, 0u, 0u);
      qf[nt][kc][0] = bf16_lo(v.x);
      qf[nt][kc][1] = bf16_hi(v.x);
      qf[nt][kc][2] = bf16_lo(v.y);
      qf[nt][kc][3] = bf16_hi(v.y);
      qf[nt][kc][4] = bf16_lo(v.z);
      qf[nt][kc][5] = bf16_hi(v.z);
      qf[nt][kc][6] = bf16_lo(v.w);
      qf[nt][kc][7] = bf16_hi(v.w);
    }
#pragma unroll
    for (int kc = 0; kc < KC / 2; ++kc) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float c, s;
        rope_cos_sin_small(rho, s_invf[kc * 32 + lg * 8 + e], c, s);
        const float x = qf[nt][kc][e], y = qf[nt][kc + KC / 2][e];
        qf[nt][kc][e] = fmaf(x, c, -(y * s));
        qf[nt][kc + KC / 2][e] = fmaf(y, c, x * s);
      }
    }
  }

  const int n0 = a.q_pos_start[b] + qt * kPfM;   // position of tile row 0
  const int t_lo = kv_len - plen + qt * kPfM;    // logical index of tile row 0
  const int t_hi = t_lo + rows_valid - 1;
  const int t_wave = t_lo + wave * 32;           // this wave's first row
  const int nblk_vis = t_hi / kBlockTokens + 1;
  const uint32_t *trow = a.table + (size_t)b * a.max_blocks;
  const int hkv = a.num_kv_heads;

  bf16x8_t bq[2][KC];
  f32x4_t O[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) O[dt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY};
  float lsum[2] = {0.f, 0.f};
  int cur_off = -1;

  for (int j = 0; j < nblk_vis;) {
    // ---- tile = run of up to 4 blocks sharing one offset
    uint32_t wt[kPfTileBlocks];
#pragma unroll
    for (int u = 0; u < kPfTileBlocks; ++u) wt[u] = (j + u < nblk_vis) ? trow[j + u] : 0u;
    const int off = word_offset(wt[0]);
    int cnt = 1;
#pragma unroll
    for (int u = 1; u < kPfTileBlocks; ++u)
      if (cnt == u && j + u < nblk_vis && word_offset(wt[u]) == off) cnt = u + 1;

    // ---- stage K (row-major) and V (transposed) into LDS; invalid keys -> 0
    __syncthreads();
    for (int p = tid; p < 16 * CPR; p += NT) {
      const int kg = p & 15;        // keys 4kg .. 4kg+3 (all in block kg/4)
      const int cc = p >> 4;        // dims cc*8 .. cc*8+7
      const int bt = kg >> 2;
      uint32_t w = wt[0];
#pragma unroll
      for (int u = 1; u < kPfTileBlocks; ++u)
        if (bt == u) w = wt[u];
      uint32_t id = word_block(w);
      const bool blk_ok = bt < cnt;
      if (blk_ok && id >= (uint32_t)a.num_blocks) {
        s_bad = 1;
        id = 0;
      }
      const int kbase = (j + bt) * kBlockTokens + (kg & 3) * 4;
      uint4 kv[4], vv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = blk_ok && kbase + i < kv_len;
        const size_t idx = (((size_t)id * hkv + g) * kBlockTokens + (kg & 3) * 4 + i) * D + cc * 8;
        kv[i] = ok ? *(const uint4 *)(a.k_pool + idx) : make_uint4(0u, 0u, 0u, 0u);
        vv[i] = ok ? *(const uint4 *)(a.v_pool + idx) : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) *(uint4 *)(sK + (kg * 4 + i) * KSTR + cc * 8) = kv[i];
      const uint32_t *v32[4] = {&vv[0].x, &vv[1].x, &vv[2].x, &vv[3].x};
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {  // dims cc*8 + 2*e2 (+1)
        const uint32_t x0 = v32[0][e2], x1 = v32[1][e2], x2 = v32[2][e2], x3 = v32[3][e2];
        const uint2 lo = make_uint2((x0 & 0xffffu) | (x1 << 16), (x2 & 0xffffu) | (x3 << 16));
        const uint2 hi2 = make_uint2((x0 >> 16) | (x1 & 0xffff0000u), (x2 >> 16) | (x3 & 0xffff0000u));
        *(uint2 *)(sVt + (cc * 8 + 2 * e2) * VSTR + kg * 4) = lo;
        *(uint2 *)(sVt + (cc * 8 + 2 * e2 + 1) * VSTR + kg * 4) = hi2;
      }
    }
    __syncthreads();

    // ---- re-rotate the query tile when the offset changes (a new document)
    if (off != cur_off) {
      cur_off = off;
      float cs = 0.f, sn = 0.f;
      if (lane < HALF) rope_cos_sin(n0 - off, s_invf[lane], cs, sn);
#pragma unroll
      for (int kc = 0; kc < KC / 2; ++kc) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int fi = kc * 32 + lg * 8 + e;
          const float c = __shfl(cs, fi), s = __shfl(sn, fi);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            const float x = qf[nt][kc][e], y = qf[nt][kc + KC / 2][e];
            const float lo = fmaf(x, c, -(y * s)) * a.scale_log2;
            const float up = fmaf(y, c, x * s) * a.scale_log2;
            bq[nt][kc][e] = (__bf16)lo;
            bq[nt][kc + KC / 2][e] = (__bf16)up;
          }
        }
      }
    }

    // ---- S^T = K Q^T  (per lane: keys mt*16 + lg*4 + i, query nt*16 + l16)
    f32x4_t S[kPfTileBlocks][2];
#pragma unroll
    for (int mt = 0; mt < kPfTileBlocks; ++mt) {
      S[mt][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      S[mt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const bf16x8_t ka = as_bf16x8(*(const uint4 *)(sK + (mt * 16 + l16) * KSTR + kc * 32 + lg * 8));
        S[mt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, bq[0][kc], S[mt][0], 0, 0, 0);
        S[mt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, bq[1][kc], S[mt][1], 0, 0, 0);
      }
    }

    // ---- mask: keys past the tile's run, past kv_len, or after the query
    const int key0 = j * kBlockTokens;
    const bool need_mask = cnt < kPfTileBlocks || key0 + kPfN > kv_len || key0 + kPfN - 1 > t_wave;
    if (need_mask) {
#pragma unroll
      for (int mt = 0; mt < kPfTileBlocks; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kidx = key0 + mt * 16 + lg * 4 + i;
            const int tq = t_wave + nt * 16 + l16;
            if (mt >= cnt || kidx >= kv_len || kidx > tq) S[mt][nt][i] = -INFINITY;
          }
    }

    // ---- online softmax per query column
    float bm[2];
    bool need = false;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float x = S[0][nt][0];
#pragma unroll
      for (int mt = 0; mt < kPfTileBlocks; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) x = fmaxf(x, S[mt][nt][i]);
      x = fmaxf(x, __shfl_xor(x, 16));
      x = fmaxf(x, __shfl_xor(x, 32));
      bm[nt] = x;
      need |= x > m[nt] + kPfSlack;
    }
    if (wave_any(need)) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const float mn = fmaxf(m[nt], bm[nt]);
        const float alpha = mn == -INFINITY ? 1.f : exp2f(m[nt] - mn);
        lsum[nt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) O[dt][nt] *= alpha;
        m[nt] = mn;
      }
    }
    bf16x8_t bp[2][2];  // [ks][nt]: keys 32ks + {lg*4 + 0..3, 16 + lg*4 + 0..3}
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const float ms = m[nt] == -INFINITY ? 0.f : m[nt];
#pragma unroll
      for (int mt = 0; mt < kPfTileBlocks; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = exp2f(S[mt][nt][i] - ms);
          lsum[nt] += p;
          bp[mt >> 1][nt][(mt & 1) * 4 + i] = (__bf16)p;
        }
      }
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint16_t *vrow = sVt + (dt * 16 + l16) * VSTR + ks * 32 + lg * 4;
        const uint2 lo = *(const uint2 *)vrow;
        const uint2 up = *(const uint2 *)(vrow + 16);
        const bf16x8_t va = as_bf16x8(make_uint4(lo.x, lo.y, up.x, up.y));
        O[dt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, bp[ks][0], O[dt][0], 0, 0, 0);
        O[dt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, bp[ks][1], O[dt][1], 0, 0, 0);
      }
    }
    j += cnt;
  }

  // ---- normalise and write: lane holds O^T[dt*16 + lg*4 + i][nt*16 + l16]
  const bool flagged = s_bad != 0;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    float tot = lsum[nt];
    tot += __shfl_xor(tot, 16);
    tot += __shfl_xor(tot, 32);
    const float inv = flagged ? __builtin_nanf("") : 1.f / tot;
    const int row = qt * kPfM + wave * 32 + nt * 16 + l16;
    if (row < plen) {
      uint16_t *dst = out + ((size_t)(q0 + row) * a.num_q_heads + hq) * D + lg * 4;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint2 pk = make_uint2(pack_bf16x2(O[dt][nt][0] * inv, O[dt][nt][1] * inv),
                                    pack_bf16x2(O[dt][nt][2] * inv, O[dt][nt][3] * inv));
        *(uint2 *)(dst + dt * 16) = pk;
      }
    }
  }
}

template <int D>
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
  k.batch = a.batch;
  k.num_q_heads = a.num_q_heads;
  k.num_kv_heads = a.num_kv_heads;
  k.num_blocks = a.num_blocks;
  k.max_blocks = a.max_blocks;
  k.q_tiles = (a.max_q_len + kPfM - 1) / kPfM;
  k.num_units = k.q_tiles * a.batch * a.num_kv_heads;
  k.scale_log2 = a.scale * kLog2e;
  k.rope_theta = a.rope_theta;
  const int group = a.num_q_heads / a.num_kv_heads;
  const long long slots = (long long)(k.num_units + kXcds - 1) / kXcds * group;
  const long long grid = slots * kXcds;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_kernel<D>), dim3((unsigned)grid), dim3(kPfWaves * kWave), 0, stream, k);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream) {
  switch (a.head_dim) {
    case 64: return launch_prefill_t<64>(a, stream);
    case 128: return launch_prefill_t<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lazyattn

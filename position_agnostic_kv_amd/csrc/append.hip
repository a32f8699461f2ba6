// kvcache_append: scatter new content-only K/V rows into 16-token pool blocks.
// The new rows of K and V are added to the cache unrotated (LazyAttention
// summary, "Metodologia": the cache keeps content only; lynx-cortex
// "El remedio": append the new row, then attend).
#include "common.h"
#include "launch.h"

namespace lazyattn {

// One thread moves one 16-byte chunk of K and the same chunk of V.
__global__ void __launch_bounds__(256)
append_kernel(uint4 *__restrict__ k_pool, uint4 *__restrict__ v_pool,
              const uint4 *__restrict__ k_new, const uint4 *__restrict__ v_new,
              const int32_t *__restrict__ slot_mapping, int num_tokens, int num_kv_heads,
              int chunks_per_row, long long num_slots) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)num_tokens * num_kv_heads * chunks_per_row;
  if (idx >= total) return;
  const int chunk = (int)(idx % chunks_per_row);
  const long long row = idx / chunks_per_row;      // token * heads + head
  const int head = (int)(row % num_kv_heads);
  const int tok = (int)(row / num_kv_heads);
  const long long slot = slot_mapping[tok];
  if (slot < 0 || slot >= num_slots) return;        // padding / out of the pool
  const long long blk = slot / kBlockTokens;
  const long long in_blk = slot % kBlockTokens;
  const long long dst = ((blk * num_kv_heads + head) * kBlockTokens + in_blk) * chunks_per_row + chunk;
  k_pool[dst] = k_new[idx];
  v_pool[dst] = v_new[idx];
}

hipError_t launch_append(void *k_pool, void *v_pool, int elem_bytes, int num_blocks,
                         int num_kv_heads, int head_dim, const void *k_new, const void *v_new,
                         const int32_t *slot_mapping, int num_tokens, hipStream_t stream) {
  const int cpr = head_dim * elem_bytes / 16;
  const long long total = (long long)num_tokens * num_kv_heads * cpr;
  const unsigned grid = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(append_kernel, dim3(grid), dim3(256), 0, stream, (uint4 *)k_pool,
                     (uint4 *)v_pool, (const uint4 *)k_new, (const uint4 *)v_new, slot_mapping,
                     num_tokens, num_kv_heads, cpr, (long long)num_blocks * kBlockTokens);
  return hipGetLastError();
}

// ---- 8-bit pools: quantise on the way in -------------------------------------
// A pool of OCP E4M3 codes with one scale per tensor: the stored code is the
// float32 quotient x / scale rounded to the nearest E4M3 value (ties to an even
// mantissa), magnitudes above 448 saturating, NaN stored as 0x7F.  The rounding
// works on the quotient's bits: a normal E4M3 value keeps the float's top three
// mantissa bits with the exponent rebiased from 127 to 7; below 2^-6 the codes
// are the multiples of 2^-9.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t mag = u & 0x7fffffffu;
  if (mag > 0x7f800000u) return 0x7fu;           // NaN
  if (mag > 0x43e00000u) return sign | 0x7eu;    // beyond 448, infinity included
  uint32_t code;
  if (mag >= 0x3c800000u) {                      // >= 2^-6
    // round away the low 20 mantissa bits, ties to even; a carry moves the
    // exponent up, which is the next E4M3 binade's first code
    const uint32_t r = (mag + 0x7ffffu + ((mag >> 20) & 1u)) >> 20;
    code = r - (120u << 3);                      // exponent bias 127 -> 7
  } else {
    code = (uint32_t)__builtin_rintf(__uint_as_float(mag) * 512.0f);  // 0..8, ties to even
  }
  return sign | code;
}

// An int8 pool (symmetric codes, one scale per tensor): the stored code is
// the float32 quotient x / scale rounded to the nearest integer (ties to
// even), clamped to [-127, 127], NaN stored as 0.
__device__ __forceinline__ uint32_t f32_to_i8(float x) {
  if (!(x == x)) return 0u;
  const float r = __builtin_rintf(fminf(fmaxf(x, -127.f), 127.f));
  return (uint32_t)(uint8_t)(int8_t)(int)r;
}

template <int FMT>
__device__ __forceinline__ uint32_t f32_to_code8(float x) {
  if constexpr (FMT == kCodeInt8) return f32_to_i8(x);
  else return f32_to_e4m3(x);
}

__device__ __forceinline__ void load8(const uint16_t *p, float (&x)[8]) {
  const uint4 c = *(const uint4 *)p;
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float *p, float (&x)[8]) {
  const float4 a = *(const float4 *)p, b = *(const float4 *)(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
template <int FMT>
__device__ __forceinline__ uint2 quant8(const float (&x)[8], float scale) {
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i >> 2] |= f32_to_code8<FMT>(__fdiv_rn(x[i], scale)) << (8 * (i & 3));
  return make_uint2(w[0], w[1]);
}

// One thread quantises 8 consecutive dims of one K row and of one V row.  The
// 8-bit pool keeps each (block, KV head) of 16 x 128 codes in the lane order of
// the matrix-core decode: byte 1024 i + 16 l + x (half i, lane l = 16 g + t,
// x < 16) holds K[token t][dim 32 g + 16 i + x] and
// V[token 4 g + x % 4][dim 16 (4 i + x / 4) + t].  The K codes of 8 dims are 8
// adjacent bytes; the V codes of 8 dims go to 8 lanes' bytes.
template <int FMT, typename TI>
__device__ __forceinline__ void append8_body(uint8_t *__restrict__ k_pool, uint8_t *__restrict__ v_pool,
                                             const TI *__restrict__ k_new, const TI *__restrict__ v_new,
                                             const int32_t *__restrict__ slot_mapping, int num_tokens,
                                             int num_kv_heads, long long num_slots, float k_scale,
                                             float v_scale) {
  constexpr int kGroups = 16;  // 128 dims / 8
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)num_tokens * num_kv_heads * kGroups;
  if (idx >= total) return;
  const int grp = (int)(idx % kGroups);
  const long long row = idx / kGroups;      // token * heads + head
  const int head = (int)(row % num_kv_heads);
  const int tok = (int)(row / num_kv_heads);
  const long long slot = slot_mapping[tok];
  if (slot < 0 || slot >= num_slots) return;  // padding / out of the pool
  const long long blk = slot / kBlockTokens;
  const int t = (int)(slot % kBlockTokens);
  uint8_t *kb = k_pool + (blk * num_kv_heads + head) * 2048;
  uint8_t *vb = v_pool + (blk * num_kv_heads + head) * 2048;
  const int d0 = grp * 8;
  float x[8];
  load8(k_new + idx * 8, x);
  *(uint2 *)(kb + ((d0 >> 4) & 1) * 1024 + (16 * (d0 >> 5) + t) * 16 + (d0 & 15)) = quant8<FMT>(x, k_scale);
  load8(v_new + idx * 8, x);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int d = d0 + e, c = d >> 4;
    vb[(c >> 2) * 1024 + (16 * (t >> 2) + (d & 15)) * 16 + (c & 3) * 4 + (t & 3)] =
        (uint8_t)f32_to_code8<FMT>(__fdiv_rn(x[e], v_scale));
  }
}

template <typename TI>
__global__ void __launch_bounds__(256)
append_fp8_kernel(uint8_t *__restrict__ k_pool, uint8_t *__restrict__ v_pool, const TI *__restrict__ k_new,
                  const TI *__restrict__ v_new, const int32_t *__restrict__ slot_mapping, int num_tokens,
                  int num_kv_heads, long long num_slots, float k_scale, float v_scale) {
  append8_body<kCodeE4M3>(k_pool, v_pool, k_new, v_new, slot_mapping, num_tokens, num_kv_heads, num_slots,
                          k_scale, v_scale);
}

// the same for an int8 pool (same lane-order layout)
template <typename TI>
__global__ void __launch_bounds__(256)
append_int8_kernel(uint8_t *__restrict__ k_pool, uint8_t *__restrict__ v_pool, const TI *__restrict__ k_new,
                   const TI *__restrict__ v_new, const int32_t *__restrict__ slot_mapping, int num_tokens,
                   int num_kv_heads, long long num_slots, float k_scale, float v_scale) {
  append8_body<kCodeInt8>(k_pool, v_pool, k_new, v_new, slot_mapping, num_tokens, num_kv_heads, num_slots,
                          k_scale, v_scale);
}

hipError_t launch_append_fp8(void *k_pool, void *v_pool, bool bf16_rows, int num_blocks,
                             int num_kv_heads, int head_dim, const void *k_new, const void *v_new,
                             const int32_t *slot_mapping, int num_tokens, float k_scale, float v_scale,
                             hipStream_t stream, bool int8) {
  if (head_dim != 128) return hipErrorInvalidValue;  // the lane-order layout is defined for 128 dims
  const long long total = (long long)num_tokens * num_kv_heads * 16;
  const unsigned grid = (unsigned)((total + 255) / 256);
  const long long slots = (long long)num_blocks * kBlockTokens;
  uint8_t *kp = (uint8_t *)k_pool, *vp = (uint8_t *)v_pool;
  if (bf16_rows) {
    const uint16_t *kn = (const uint16_t *)k_new, *vn = (const uint16_t *)v_new;
    if (int8)
      hipLaunchKernelGGL(append_int8_kernel<uint16_t>, dim3(grid), dim3(256), 0, stream, kp, vp, kn, vn,
                         slot_mapping, num_tokens, num_kv_heads, slots, k_scale, v_scale);
    else
      hipLaunchKernelGGL(append_fp8_kernel<uint16_t>, dim3(grid), dim3(256), 0, stream, kp, vp, kn, vn,
                         slot_mapping, num_tokens, num_kv_heads, slots, k_scale, v_scale);
  } else {
    const float *kn = (const float *)k_new, *vn = (const float *)v_new;
    if (int8)
      hipLaunchKernelGGL(append_int8_kernel<float>, dim3(grid), dim3(256), 0, stream, kp, vp, kn, vn,
                         slot_mapping, num_tokens, num_kv_heads, slots, k_scale, v_scale);
    else
      hipLaunchKernelGGL(append_fp8_kernel<float>, dim3(grid), dim3(256), 0, stream, kp, vp, kn, vn,
                         slot_mapping, num_tokens, num_kv_heads, slots, k_scale, v_scale);
  }
  return hipGetLastError();
}

}  // namespace lazyattn

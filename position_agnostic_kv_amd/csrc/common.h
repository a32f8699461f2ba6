// Device helpers shared by the lazyattn kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lazyattn {

constexpr int kBlockTokens = 16;
constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// bfloat16 storage is handled as raw 16-bit patterns.
struct bf16 {
  uint16_t bits;
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Widen the low / high bfloat16 halves of a dword (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two floats to bfloat16 (nearest even, the hardware conversion) and pack lo | hi << 16.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// x, y as bf16 pairs hi + lo: hi = bf16(x), lo = bf16(x - hi) (x - hi is
// exact in float).  hi + lo is within 2^-17 relative of x, against 2^-9 for
// hi alone, so a product against hi and lo on the matrix cores carries the
// float operand almost exactly.
__device__ __forceinline__ void split_bf16x2(float x, float y, uint32_t &hi, uint32_t &lo) {
  hi = pack_bf16x2(x, y);
  lo = pack_bf16x2(x - bf16_lo(hi), y - bf16_hi(hi));
}

__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// c + a.lo * b.lo + a.hi * b.hi on packed bf16 pairs, fp32 accumulate (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// max of four scores that are never NaN (v_max3_f32 + v_max_f32), without the
// canonicalising moves that fmaxf's NaN rules add.  Inline assembly: the
// compiler pads no hazard wait states in front of it, so its inputs must come
// from ordinary VALU instructions (which the hardware interlocks), never
// straight from a matrix-core (MFMA) result -- use max4_mfma for those.
__device__ __forceinline__ float max4_nn(float a, float b, float c, float d) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3\n\tv_max_f32 %0, %0, %4" : "=&v"(r) : "v"(a), "v"(b), "v"(c), "v"(d));
  return r;
}

// max of four MFMA results: plain builtins, so that the compiler inserts the
// wait states a VALU read of a matrix-core result needs on gfx950.
__device__ __forceinline__ float max4_mfma(float a, float b, float c, float d) {
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// Two OCP E4M3 codes (bytes 0-1, or 2-3 with HI) of a word -> a packed bf16
// pair (v_cvt_scalef32_pk_bf16_fp8 with scale 1: exact, every E4M3 value is
// a bf16 value).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// Two signed 8-bit integer codes (bytes 0-1, or 2-3 with HI) of a word -> a
// packed bf16 pair, byte 2 HI in the low half: exact (every integer of
// magnitude <= 256 is a bf16 value).
template <bool HI>
__device__ __forceinline__ uint32_t i8x2_to_bf16x2(uint32_t w) {
  const int sh = HI ? 16 : 0;
  return pack_bf16x2((float)(int)(int8_t)(w >> sh), (float)(int)(int8_t)(w >> (sh + 8)));
}

// 8-bit pool code formats
enum Code8 { kCodeE4M3 = 0, kCodeInt8 = 1 };
template <int FMT, bool HI>
__device__ __forceinline__ uint32_t code8x2_to_bf16x2(uint32_t w) {
  if constexpr (FMT == kCodeInt8) return i8x2_to_bf16x2<HI>(w);
  else return e4m3x2_to_bf16x2<HI>(w);
}

// Dword w (a compile-time constant after unrolling) of a 16-byte chunk.
__device__ __forceinline__ uint32_t dw4(const uint4 &v, int w) {
  return w == 0 ? v.x : w == 1 ? v.y : w == 2 ? v.z : v.w;
}

// Table word: block id in bits 0..15, position offset in bits 16..31.
__device__ __forceinline__ uint32_t word_block(uint32_t w) { return w & 0xffffu; }
__device__ __forceinline__ int word_offset(uint32_t w) { return (int)(w >> 16); }

// RoPE frequency theta^(-2i/D) in double precision.
__device__ __forceinline__ double rope_inv_freq(int i, int head_dim, float theta) {
  return pow((double)theta, -2.0 * (double)i / (double)head_dim);
}

// cos/sin of delta * inv_freq, with the angle formed and reduced in double
// precision (|delta| reaches 65535, where a float angle would be off by ~4e-3 rad).
__device__ __forceinline__ void rope_cos_sin(int delta, double inv_freq, float &c, float &s) {
  double sd, cd;
  sincos((double)delta * inv_freq, &sd, &cd);
  c = (float)cd;
  s = (float)sd;
}

// ------------------------------------------------------------ cross-lane sums
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppRowMirror = 0x140;     // lane i <-> 15-i within 16

// Sums over aligned groups of N consecutive lanes (N a power of two, <= 64)
// of the n values x[0..n).  Every lane of a group gets the bit-identical total
// (each step pairs lanes symmetrically and float addition is commutative).
// Each DPP step is applied to all values before the next step, so a value is
// never read by DPP right after the instruction that wrote it (no wait states
// between dependent DPP adds).
template <int N, int n>
__device__ __forceinline__ void group_sum_all(float *x) {
  if constexpr (N >= 2) {
#pragma unroll
    for (int j = 0; j < n; ++j) x[j] += dpp_f32<kDppQuadXor1>(x[j]);
  }
  if constexpr (N >= 4) {
#pragma unroll
    for (int j = 0; j < n; ++j) x[j] += dpp_f32<kDppQuadXor2>(x[j]);
  }
  if constexpr (N >= 8) {
#pragma unroll
    for (int j = 0; j < n; ++j) x[j] += dpp_f32<kDppRowHalfMirror>(x[j]);
  }
  if constexpr (N >= 16) {
#pragma unroll
    for (int j = 0; j < n; ++j) x[j] += dpp_f32<kDppRowMirror>(x[j]);
  }
  if constexpr (N >= 32) {
#pragma unroll
    for (int j = 0; j < n; ++j) x[j] += __shfl_xor(x[j], 16);
  }
  if constexpr (N >= 64) {
#pragma unroll
    for (int j = 0; j < n; ++j) x[j] += __shfl_xor(x[j], 32);
  }
}

// Reduce over lanes l, l^16, l^32, l^48 (the four lane groups holding one
// column of a 16x16 MFMA tile) with v_permlane16_swap / v_permlane32_swap.
__device__ __forceinline__ float col_max4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float col_sum4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ------------------------------------------ LDS staging of K/V tiles (DMA)
__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

typedef short s16x4_t __attribute__((ext_vector_type(4)));

// LDS chunk swizzle of a K/V tile row (16-byte chunks, CPR per row): slot =
// chunk ^ swz(row).  Measured on gfx950 (rocprofv3 SQ_LDS_BANK_CONFLICT over
// single-pattern kernels): LDS banks repeat every 256 bytes, and
// ds_read_b128 serves a wave in four groups of 16 lanes, each the four lane
// quads of one half-wave whose quad index has one bit parity (lanes 0-3,
// 12-15, 20-27 form one group).  For 16 chunks per row, swz(r) = 2 (r mod 8)
// gives every such group 16 distinct bank slots in the K operand read (row
// l16, chunk 4 kc + lg) and keeps the transposing V read (ds_read_b64_tr_b16,
// two rows x two chunks per lane quad) free of conflicts as well.
template <int CPR>
__device__ __forceinline__ int swz(int r) {
  if constexpr (CPR == 16) return (r & 7) << 1;
  else return (r >> 1) & (CPR - 1);
}
typedef __attribute__((address_space(3))) void *lds_ptr_t;

// 16 bytes per lane from global memory straight into LDS
// (global_load_lds_dwordx4, scalar base + per-lane 32-bit offset): lane L's
// bytes land at LDS address lds + 16 * L.  Issued as inline assembly so the
// compiler does not order every later LDS read behind it (it cannot tell the
// buffers apart); the kernel waits for these loads itself (s_waitcnt and a
// barrier at each tile start).  M0 holds the LDS address; one wait state
// separates its write from the load.  The compiler warns that M0 is reserved
// and will not save it around the statement: no other instruction of these
// kernels reads or writes M0 (checked in their assembly), so nothing live is
// lost.
__device__ __forceinline__ void lds_dma16(const void *base, uint32_t voff, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(base), "s"(lds)
      : "memory", "m0");
}

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, output
// lane i gets element (i % 4) of the 8-byte rows read by source lanes
// i / 4 + 4k, k = 0..3.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t *p) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t *)(p));
  return __builtin_bit_cast(uint2, v);
}

// Read-only kernel inputs seen through the constant address space: uniform
// loads from it are always scalar (s_load, counted by lgkmcnt), even next to
// inline assembly that clobbers memory, so they never wait on, or make the
// compiler wait for, vector loads in flight.
template <typename T>
using const_as_ptr = const __attribute__((address_space(4))) T *;
template <typename T>
__device__ __forceinline__ const_as_ptr<T> as_const_as(const T *p) {
  return (const_as_ptr<T>)(uintptr_t)p;
}

// Wave-uniform "any lane true".
__device__ __forceinline__ bool wave_any(bool p) { return __ballot(p) != 0ull; }

}  // namespace lazyattn

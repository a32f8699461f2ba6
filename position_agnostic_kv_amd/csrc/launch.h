// Internal launchers behind the C ABI (argument checks happen in abi.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lazyattn {

// Position scheme of a decode/prefill launch.
enum PosMode : int {
  kRopeLazy = 0,   // RoPE, keys in their own frames, offsets applied lazily
  kRopeEager = 1,  // RoPE, keys already at absolute positions, offsets ignored
  kAlibi = 2       // ALiBi: no rotation; key position = block offset + slot
};

hipError_t launch_append(void *k_pool, void *v_pool, int elem_bytes, int num_blocks,
                         int num_kv_heads, int head_dim, const void *k_new, const void *v_new,
                         const int32_t *slot_mapping, int num_tokens, hipStream_t stream);
hipError_t launch_append_fp8(void *k_pool, void *v_pool, bool bf16_rows, int num_blocks,
                             int num_kv_heads, int head_dim, const void *k_new, const void *v_new,
                             const int32_t *slot_mapping, int num_tokens, float k_scale, float v_scale,
                             hipStream_t stream, bool int8 = false);

// Which decode kernel family a launch runs on.
enum DecodeImpl : int {
  kDecodeValu = 0,   // fp32 pools and head_dim 64: VALU kernel
  kDecodeMma8 = 1,   // 8-bit pools: matrix cores
  kDecodeMma16 = 2   // bf16 pools with head_dim 128: matrix cores
};
int decode_impl(bool pool8, bool bf16, int head_dim);
// Workgroups that share one KV head's query heads in a decode launch.
int decode_head_split(int num_q_heads, int num_kv_heads, int impl);
// Blocks per split-K partition for a decode launch (requested == 0: automatic).
int decode_split_blocks(int batch, int num_q_heads, int num_kv_heads, int max_blocks_per_seq,
                        int requested, int impl);
size_t decode_workspace_size(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                             int max_blocks_per_seq, int split_blocks);

struct DecodeArgs {
  void *out;
  const void *q;
  const int32_t *q_pos;
  const void *k_pool;
  const void *v_pool;
  const uint32_t *table;
  const int32_t *seq_lens;
  void *workspace;
  int batch, num_q_heads, num_kv_heads, head_dim, num_blocks, max_blocks;
  int split_blocks;  // resolved (> 0)
  float scale, rope_theta;
  const float *slopes;  // ALiBi slopes [num_q_heads] (device), else unused
  const uint8_t *block_fill;  // per-block fill counts, or nullptr (all full)
  int mode;             // PosMode
  float k_scale = 1.f, v_scale = 1.f;  // 8-bit pools: value = code * scale
  bool int8 = false;    // 8-bit pools: int8 codes instead of E4M3
  // work plan (device): per-sequence slot counts [batch], then plan_items
  // items of 12 ints from decode_plan_items_offset(batch); nullptr: splits
  const int32_t *plan = nullptr;
  int plan_items = 0, plan_max_items = 0;
};
hipError_t launch_decode(const DecodeArgs &a, bool bf16, hipStream_t stream);
hipError_t launch_decode_planned(const DecodeArgs &a, hipStream_t stream);
size_t decode_planned_workspace_size(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                     int max_items_per_seq);
size_t decode_plan_items_offset(int batch);
hipError_t launch_decode_fp8(const DecodeArgs &a, hipStream_t stream);

struct PrefillArgs {
  void *out;
  const void *q;
  const int32_t *cu_q_lens;
  const int32_t *q_pos_start;
  const void *k_pool;
  const void *v_pool;
  const uint32_t *table;
  const int32_t *kv_lens;
  int total_q, batch, max_q_len, num_q_heads, num_kv_heads, head_dim, num_blocks, max_blocks;
  float scale, rope_theta;
  const float *slopes;  // ALiBi slopes [num_q_heads] (device), else unused
  const uint8_t *block_fill;  // per-block fill counts, or nullptr (all full)
  int mode;             // PosMode
  float k_scale = 1.f, v_scale = 1.f;  // 8-bit pools: value = code * scale
  bool int8 = false;    // 8-bit pools: int8 codes instead of E4M3
  int staged = 0;       // K/V pools are the widened copy of an 8-bit pool
  bool precise = false; // rotated query as bf16 hi + lo, tiles cut at offset changes (lazy RoPE)
};
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream);
// 8-bit pools: bytes of the bf16 copy of every block slot the batch can see
size_t prefill_fp8_workspace_size(int batch, int max_blocks, int num_kv_heads);
hipError_t launch_prefill_fp8(const PrefillArgs &a, void *workspace, hipStream_t stream);

}  // namespace lazyattn

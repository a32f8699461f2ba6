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

}  // namespace lazyattn

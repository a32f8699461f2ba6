// C ABI of the lazyattn library: argument checks, then launches on the caller's
// stream.  Nothing here allocates or synchronises.
#include "lazyattn.h"

#include <math.h>

#include <mutex>

#include "launch.h"

using namespace lazyattn;

namespace {

// Split-K partials of lazyattn_decode_noalloc: a fixed array in device memory
// (one copy per GPU the library runs on, held until the process ends).  Host
// code never passes the array's name to a kernel: its device address on the
// current GPU comes from hipGetSymbolAddress, looked up once per device.
constexpr size_t kScratchBytes = (size_t)LAZYATTN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void *scratch_ptr[kMaxDevices];

// The scratch address on the current device, or nullptr if it cannot be had.
void *scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    scratch_ptr[dev] = ptr;
  }
  return scratch_ptr[dev];
}

bool valid_dtype(int dtype) { return dtype == LAZYATTN_F32 || dtype == LAZYATTN_BF16; }
int elem_bytes(int dtype) { return dtype == LAZYATTN_F32 ? 4 : 2; }
bool pow2_group(int g) { return g >= 1 && g <= 64 && (g & (g - 1)) == 0; }
bool valid_kv_scale(float s) { return s > 0.f && isfinite(s); }

int from_hip(hipError_t e) { return e == hipSuccess ? LAZYATTN_OK : LAZYATTN_ERR_LAUNCH; }

}  // namespace

extern "C" {

const char *lazyattn_status_string(int status) {
  switch (status) {
    case LAZYATTN_OK: return "ok";
    case LAZYATTN_ERR_NULL: return "a required pointer is NULL";
    case LAZYATTN_ERR_DTYPE: return "unsupported dtype for this call";
    case LAZYATTN_ERR_SHAPE: return "unsupported or inconsistent size argument";
    case LAZYATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case LAZYATTN_ERR_LAUNCH: return "kernel launch failed";
    case LAZYATTN_ERR_SCRATCH:
      return "split-K partials exceed the fixed scratch of lazyattn_decode_noalloc (or its address is unavailable)";
    default: return "unknown status";
  }
}

int lazyattn_version(void) { return 100; }

int kvcache_append(void *k_pool, void *v_pool, int dtype, int num_blocks, int num_kv_heads,
                   int head_dim, const void *k_new, const void *v_new,
                   const int32_t *slot_mapping, int num_tokens, void *stream) {
  if (!valid_dtype(dtype)) return LAZYATTN_ERR_DTYPE;
  if (num_tokens < 0 || num_blocks < 1 || num_blocks > LAZYATTN_MAX_BLOCKS || num_kv_heads < 1 ||
      num_kv_heads > 1024)
    return LAZYATTN_ERR_SHAPE;
  if (!(head_dim == 16 || head_dim == 32 || head_dim == 64 || head_dim == 128 || head_dim == 256))
    return LAZYATTN_ERR_SHAPE;
  if (num_tokens == 0) return LAZYATTN_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !slot_mapping) return LAZYATTN_ERR_NULL;
  return from_hip(launch_append(k_pool, v_pool, elem_bytes(dtype), num_blocks, num_kv_heads,
                                head_dim, k_new, v_new, slot_mapping, num_tokens,
                                (hipStream_t)stream));
}

static int append8_common(void *k_pool, void *v_pool, int dtype, int num_blocks, int num_kv_heads,
                          int head_dim, const void *k_new, const void *v_new, const int32_t *slot_mapping,
                          int num_tokens, float k_scale, float v_scale, void *stream, bool int8) {
  if (!valid_dtype(dtype)) return LAZYATTN_ERR_DTYPE;
  if (num_tokens < 0 || num_blocks < 1 || num_blocks > LAZYATTN_MAX_BLOCKS || num_kv_heads < 1 ||
      num_kv_heads > 1024)
    return LAZYATTN_ERR_SHAPE;
  if (head_dim != 128) return LAZYATTN_ERR_SHAPE;  // the 8-bit pool layout is defined for 128 dims
  if (!valid_kv_scale(k_scale) || !valid_kv_scale(v_scale)) return LAZYATTN_ERR_SHAPE;
  if (num_tokens == 0) return LAZYATTN_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !slot_mapping) return LAZYATTN_ERR_NULL;
  return from_hip(launch_append_fp8(k_pool, v_pool, dtype == LAZYATTN_BF16, num_blocks, num_kv_heads,
                                    head_dim, k_new, v_new, slot_mapping, num_tokens, k_scale, v_scale,
                                    (hipStream_t)stream, int8));
}

int kvcache_append_fp8(void *k_pool, void *v_pool, int dtype, int num_blocks, int num_kv_heads,
                       int head_dim, const void *k_new, const void *v_new, const int32_t *slot_mapping,
                       int num_tokens, float k_scale, float v_scale, void *stream) {
  return append8_common(k_pool, v_pool, dtype, num_blocks, num_kv_heads, head_dim, k_new, v_new, slot_mapping,
                        num_tokens, k_scale, v_scale, stream, false);
}

int kvcache_append_int8(void *k_pool, void *v_pool, int dtype, int num_blocks, int num_kv_heads,
                        int head_dim, const void *k_new, const void *v_new, const int32_t *slot_mapping,
                        int num_tokens, float k_scale, float v_scale, void *stream) {
  return append8_common(k_pool, v_pool, dtype, num_blocks, num_kv_heads, head_dim, k_new, v_new, slot_mapping,
                        num_tokens, k_scale, v_scale, stream, true);
}

size_t lazyattn_decode_workspace_size(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                      int max_blocks_per_seq, int split_blocks) {
  if (batch <= 0 || num_kv_heads <= 0 || num_q_heads <= 0 || head_dim <= 0 ||
      max_blocks_per_seq <= 0 || split_blocks < 0 || num_q_heads % num_kv_heads)
    return 0;
  return decode_workspace_size(batch, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                               split_blocks);
}

static int decode_common(void *out, const void *q, const int32_t *q_pos, const void *k_pool,
                         const void *v_pool, const uint32_t *block_table, int max_blocks_per_seq,
                         const uint8_t *block_fill, const int32_t *seq_lens, int batch, int num_q_heads, int num_kv_heads,
                         int head_dim, int num_blocks, int dtype, float scale, float rope_theta,
                         int split_blocks, void *workspace, size_t workspace_bytes, void *stream,
                         int mode, const float *slopes, bool pool8 = false, float k_scale = 1.f,
                         float v_scale = 1.f, const int32_t *plan = nullptr, int plan_items = 0,
                         int plan_max_items = 0, bool int8 = false) {
  if (!valid_dtype(dtype)) return LAZYATTN_ERR_DTYPE;
  if (batch < 0 || batch > 65535 || num_kv_heads < 1 || num_kv_heads > 65535 || num_q_heads < 1 ||
      num_q_heads % num_kv_heads || !pow2_group(num_q_heads / num_kv_heads))
    return LAZYATTN_ERR_SHAPE;
  const bool bf16 = dtype == LAZYATTN_BF16;
  if (bf16 ? !(head_dim == 64 || head_dim == 128)
           : !(head_dim == 16 || head_dim == 64 || head_dim == 128))
    return LAZYATTN_ERR_SHAPE;
  if (num_blocks < 1 || num_blocks > LAZYATTN_MAX_BLOCKS || max_blocks_per_seq < 1 ||
      max_blocks_per_seq > LAZYATTN_MAX_POSITION / LAZYATTN_BLOCK_TOKENS + 1)
    return LAZYATTN_ERR_SHAPE;
  if (split_blocks != 0 && (split_blocks < 4 || split_blocks > 1024)) return LAZYATTN_ERR_SHAPE;
  if (!(rope_theta > 1.0f) || !isfinite(rope_theta) || !isfinite(scale)) return LAZYATTN_ERR_SHAPE;
  if (pool8 && (head_dim != 128 || !valid_kv_scale(k_scale) || !valid_kv_scale(v_scale)))
    return LAZYATTN_ERR_SHAPE;
  if (batch == 0) return LAZYATTN_OK;
  if (!out || !q || !q_pos || !k_pool || !v_pool || !block_table || !seq_lens)
    return LAZYATTN_ERR_NULL;
  if (mode == kAlibi && !slopes) return LAZYATTN_ERR_NULL;
  const size_t need = plan ? decode_planned_workspace_size(batch, num_q_heads, num_kv_heads, head_dim, plan_max_items)
                           : decode_workspace_size(batch, num_q_heads, num_kv_heads, head_dim,
                                                   max_blocks_per_seq, split_blocks);
  if (need && (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 15u)))
    return LAZYATTN_ERR_WORKSPACE;

  DecodeArgs a;
  a.out = out;
  a.q = q;
  a.q_pos = q_pos;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.table = block_table;
  a.seq_lens = seq_lens;
  a.workspace = need ? workspace : nullptr;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.split_blocks = decode_split_blocks(batch, num_q_heads, num_kv_heads, max_blocks_per_seq, split_blocks,
                                      decode_impl(pool8, bf16, head_dim));
  a.scale = scale;
  a.rope_theta = rope_theta;
  a.mode = mode;
  a.slopes = slopes;
  a.block_fill = block_fill;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.plan = plan;
  a.plan_items = plan_items;
  a.plan_max_items = plan_max_items;
  a.int8 = int8;
  if (pool8) return from_hip(launch_decode_fp8(a, (hipStream_t)stream));
  if (plan) return from_hip(launch_decode_planned(a, (hipStream_t)stream));
  return from_hip(launch_decode(a, bf16, (hipStream_t)stream));
}

int lazyattn_decode_noalloc(void *out, const void *q, const int32_t *q_pos, const void *k_pool,
                            const void *v_pool, const uint32_t *block_table, int max_blocks_per_seq,
                            const uint8_t *block_fill, const int32_t *seq_lens, int batch, int num_q_heads,
                            int num_kv_heads, int head_dim, int num_blocks, int dtype, float scale,
                            float rope_theta, int split_blocks, void *stream) {
  // the partials this call needs (0: every sequence fits one split)
  const size_t need = (batch > 0 && num_kv_heads > 0 && num_q_heads > 0 && num_q_heads % num_kv_heads == 0 &&
                       head_dim > 0 && max_blocks_per_seq > 0 && split_blocks >= 0)
                          ? decode_workspace_size(batch, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                                                  split_blocks)
                          : 0;
  if (need > kScratchBytes) return LAZYATTN_ERR_SCRATCH;
  void *ws = nullptr;
  if (need) {
    ws = scratch_for_current_device();
    if (!ws) return LAZYATTN_ERR_SCRATCH;
  }
  return decode_common(out, q, q_pos, k_pool, v_pool, block_table, max_blocks_per_seq, block_fill, seq_lens,
                       batch, num_q_heads, num_kv_heads, head_dim, num_blocks, dtype, scale, rope_theta,
                       split_blocks, ws, kScratchBytes, stream, kRopeLazy, nullptr);
}

int lazyattn_decode_fp8(void *out, const void *q, const int32_t *q_pos, const void *k_pool,
                        const void *v_pool, const uint32_t *block_table, int max_blocks_per_seq,
                        const uint8_t *block_fill, const int32_t *seq_lens, int batch, int num_q_heads,
                        int num_kv_heads, int head_dim, int num_blocks, float scale, float rope_theta,
                        float k_scale, float v_scale, int split_blocks, void *workspace,
                        size_t workspace_bytes, void *stream) {
  return decode_common(out, q, q_pos, k_pool, v_pool, block_table, max_blocks_per_seq, block_fill, seq_lens,
                       batch, num_q_heads, num_kv_heads, head_dim, num_blocks, LAZYATTN_BF16, scale,
                       rope_theta, split_blocks, workspace, workspace_bytes, stream, kRopeLazy, nullptr,
                       true, k_scale, v_scale);
}

int lazyattn_decode_int8(void *out, const void *q, const int32_t *q_pos, const void *k_pool,
                         const void *v_pool, const uint32_t *block_table, int max_blocks_per_seq,
                         const uint8_t *block_fill, const int32_t *seq_lens, int batch, int num_q_heads,
                         int num_kv_heads, int head_dim, int num_blocks, float scale, float rope_theta,
                         float k_scale, float v_scale, int split_blocks, void *workspace,
                         size_t workspace_bytes, void *stream) {
  return decode_common(out, q, q_pos, k_pool, v_pool, block_table, max_blocks_per_seq, block_fill, seq_lens,
                       batch, num_q_heads, num_kv_heads, head_dim, num_blocks, LAZYATTN_BF16, scale,
                       rope_theta, split_blocks, workspace, workspace_bytes, stream, kRopeLazy, nullptr,
                       true, k_scale, v_scale, nullptr, 0, 0, true);
}

int lazyattn_decode(void *out, const void *q, const int32_t *q_pos, const void *k_pool,
                    const void *v_pool, const uint32_t *block_table, int max_blocks_per_seq,
                    const uint8_t *block_fill, const int32_t *seq_lens, int batch, int num_q_heads, int num_kv_heads,
                    int head_dim, int num_blocks, int dtype, float scale, float rope_theta,
                    int split_blocks, void *workspace, size_t workspace_bytes, void *stream) {
  return decode_common(out, q, q_pos, k_pool, v_pool, block_table, max_blocks_per_seq, block_fill, seq_lens,
                       batch, num_q_heads, num_kv_heads, head_dim, num_blocks, dtype, scale,
                       rope_theta, split_blocks, workspace, workspace_bytes, stream, kRopeLazy, nullptr);
}

size_t lazyattn_decode_planned_workspace_size(int batch, int num_q_heads, int num_kv_heads, int head_dim,
                                              int max_items_per_seq) {
  if (batch <= 0 || num_kv_heads <= 0 || num_q_heads <= 0 || head_dim <= 0 || num_q_heads % num_kv_heads ||
      max_items_per_seq <= 0)
    return 0;
  return decode_planned_workspace_size(batch, num_q_heads, num_kv_heads, head_dim, max_items_per_seq);
}

int lazyattn_decode_planned(void *out, const void *q, const int32_t *q_pos, const void *k_pool,
                            const void *v_pool, const uint32_t *block_table, int max_blocks_per_seq,
                            const uint8_t *block_fill, const int32_t *seq_lens, int batch, int num_q_heads,
                            int num_kv_heads, int head_dim, int num_blocks, int dtype, float scale,
                            float rope_theta, const int32_t *plan, int num_items, int max_items_per_seq,
                            void *workspace, size_t workspace_bytes, void *stream) {
  if (!valid_dtype(dtype)) return LAZYATTN_ERR_DTYPE;
  if (dtype != LAZYATTN_BF16) return LAZYATTN_ERR_DTYPE;
  if (head_dim != 128 || num_kv_heads < 1 || num_q_heads < 1 || num_q_heads % num_kv_heads ||
      !pow2_group(num_q_heads / num_kv_heads) || num_q_heads / num_kv_heads > 16 || num_items < 1 ||
      max_items_per_seq < 1 || max_items_per_seq > 65535)
    return LAZYATTN_ERR_SHAPE;
  if (batch > 0 && !plan) return LAZYATTN_ERR_NULL;
  if ((uintptr_t)plan & 15u) return LAZYATTN_ERR_SHAPE;
  return decode_common(out, q, q_pos, k_pool, v_pool, block_table, max_blocks_per_seq, block_fill, seq_lens,
                       batch, num_q_heads, num_kv_heads, head_dim, num_blocks, dtype, scale, rope_theta, 0,
                       workspace, workspace_bytes, stream, kRopeLazy, nullptr, false, 1.f, 1.f, plan, num_items,
                       max_items_per_seq);
}

int lazyattn_decode_eager(void *out, const void *q, const int32_t *q_pos, const void *k_pool,
                          const void *v_pool, const uint32_t *block_table, int max_blocks_per_seq,
                          const uint8_t *block_fill, const int32_t *seq_lens, int batch, int num_q_heads, int num_kv_heads,
                          int head_dim, int num_blocks, int dtype, float scale, float rope_theta,
                          int split_blocks, void *workspace, size_t workspace_bytes, void *stream) {
  return decode_common(out, q, q_pos, k_pool, v_pool, block_table, max_blocks_per_seq, block_fill, seq_lens,
                       batch, num_q_heads, num_kv_heads, head_dim, num_blocks, dtype, scale,
                       rope_theta, split_blocks, workspace, workspace_bytes, stream, kRopeEager, nullptr);
}

int lazyattn_decode_alibi(void *out, const void *q, const int32_t *q_pos, const void *k_pool,
                          const void *v_pool, const uint32_t *block_table, int max_blocks_per_seq,
                          const uint8_t *block_fill, const int32_t *seq_lens, const float *slopes, int batch, int num_q_heads,
                          int num_kv_heads, int head_dim, int num_blocks, int dtype, float scale,
                          int split_blocks, void *workspace, size_t workspace_bytes, void *stream) {
  return decode_common(out, q, q_pos, k_pool, v_pool, block_table, max_blocks_per_seq, block_fill, seq_lens,
                       batch, num_q_heads, num_kv_heads, head_dim, num_blocks, dtype, scale,
                       10000.0f /* unused */, split_blocks, workspace, workspace_bytes, stream, kAlibi,
                       slopes);
}

static int prefill_common(void *out, const void *q, int total_q, const int32_t *cu_q_lens,
                          const int32_t *q_pos_start, const void *k_pool, const void *v_pool,
                          const uint32_t *block_table, int max_blocks_per_seq,
                          const uint8_t *block_fill, const int32_t *kv_lens,
                          int batch, int max_q_len, int num_q_heads, int num_kv_heads, int head_dim,
                          int num_blocks, int dtype, float scale, float rope_theta, void *stream,
                          int mode, const float *slopes, bool pool8 = false, float k_scale = 1.f,
                          float v_scale = 1.f, void *workspace = nullptr, size_t workspace_bytes = 0,
                          bool int8 = false, bool precise = false) {
  if (dtype != LAZYATTN_BF16) return LAZYATTN_ERR_DTYPE;
  if (pool8 && (head_dim != 128 || !valid_kv_scale(k_scale) || !valid_kv_scale(v_scale)))
    return LAZYATTN_ERR_SHAPE;
  if (batch < 0 || batch > 65535 || max_q_len < 0 || max_q_len > LAZYATTN_MAX_POSITION + 1 || total_q < 0 ||
      num_kv_heads < 1 || num_kv_heads > 65535 || num_q_heads < 1 || num_q_heads % num_kv_heads ||
      num_q_heads / num_kv_heads > 64)
    return LAZYATTN_ERR_SHAPE;
  if (!(head_dim == 64 || head_dim == 128)) return LAZYATTN_ERR_SHAPE;
  if (num_blocks < 1 || num_blocks > LAZYATTN_MAX_BLOCKS || max_blocks_per_seq < 1 ||
      max_blocks_per_seq > LAZYATTN_MAX_POSITION / LAZYATTN_BLOCK_TOKENS + 1)
    return LAZYATTN_ERR_SHAPE;
  if (!(rope_theta > 1.0f) || !isfinite(rope_theta) || !isfinite(scale)) return LAZYATTN_ERR_SHAPE;
  if (batch == 0 || max_q_len == 0 || total_q == 0) return LAZYATTN_OK;
  if (!out || !q || !cu_q_lens || !q_pos_start || !k_pool || !v_pool || !block_table || !kv_lens)
    return LAZYATTN_ERR_NULL;
  if (mode == kAlibi && !slopes) return LAZYATTN_ERR_NULL;
  if (pool8 && (!workspace || workspace_bytes < prefill_fp8_workspace_size(batch, max_blocks_per_seq, num_kv_heads)))
    return LAZYATTN_ERR_WORKSPACE;
  PrefillArgs a;
  a.out = out;
  a.q = q;
  a.total_q = total_q;
  a.cu_q_lens = cu_q_lens;
  a.q_pos_start = q_pos_start;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.table = block_table;
  a.kv_lens = kv_lens;
  a.batch = batch;
  a.max_q_len = max_q_len;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.scale = scale;
  a.rope_theta = rope_theta;
  a.mode = mode;
  a.slopes = slopes;
  a.block_fill = block_fill;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.int8 = int8;
  a.precise = precise;
  if (pool8) return from_hip(launch_prefill_fp8(a, workspace, (hipStream_t)stream));
  return from_hip(launch_prefill(a, (hipStream_t)stream));
}

int lazyattn_prefill(void *out, const void *q, int total_q, const int32_t *cu_q_lens,
                     const int32_t *q_pos_start, const void *k_pool, const void *v_pool,
                     const uint32_t *block_table, int max_blocks_per_seq, const uint8_t *block_fill, const int32_t *kv_lens,
                     int batch, int max_q_len, int num_q_heads, int num_kv_heads, int head_dim,
                     int num_blocks, int dtype, float scale, float rope_theta, void *stream) {
  return prefill_common(out, q, total_q, cu_q_lens, q_pos_start, k_pool, v_pool, block_table,
                        max_blocks_per_seq, block_fill, kv_lens, batch, max_q_len, num_q_heads, num_kv_heads,
                        head_dim, num_blocks, dtype, scale, rope_theta, stream, kRopeLazy, nullptr);
}

int lazyattn_prefill_precise(void *out, const void *q, int total_q, const int32_t *cu_q_lens,
                             const int32_t *q_pos_start, const void *k_pool, const void *v_pool,
                             const uint32_t *block_table, int max_blocks_per_seq, const uint8_t *block_fill,
                             const int32_t *kv_lens, int batch, int max_q_len, int num_q_heads,
                             int num_kv_heads, int head_dim, int num_blocks, int dtype, float scale,
                             float rope_theta, void *stream) {
  return prefill_common(out, q, total_q, cu_q_lens, q_pos_start, k_pool, v_pool, block_table,
                        max_blocks_per_seq, block_fill, kv_lens, batch, max_q_len, num_q_heads, num_kv_heads,
                        head_dim, num_blocks, dtype, scale, rope_theta, stream, kRopeLazy, nullptr, false, 1.f,
                        1.f, nullptr, 0, false, true);
}

int lazyattn_prefill_eager(void *out, const void *q, int total_q, const int32_t *cu_q_lens,
                           const int32_t *q_pos_start, const void *k_pool, const void *v_pool,
                           const uint32_t *block_table, int max_blocks_per_seq, const uint8_t *block_fill,
                           const int32_t *kv_lens, int batch, int max_q_len, int num_q_heads,
                           int num_kv_heads, int head_dim, int num_blocks, int dtype, float scale,
                           float rope_theta, void *stream) {
  return prefill_common(out, q, total_q, cu_q_lens, q_pos_start, k_pool, v_pool, block_table,
                        max_blocks_per_seq, block_fill, kv_lens, batch, max_q_len, num_q_heads, num_kv_heads,
                        head_dim, num_blocks, dtype, scale, rope_theta, stream, kRopeEager, nullptr);
}

int lazyattn_prefill_alibi(void *out, const void *q, int total_q, const int32_t *cu_q_lens,
                           const int32_t *q_pos_start, const void *k_pool, const void *v_pool,
                           const uint32_t *block_table, int max_blocks_per_seq, const uint8_t *block_fill, const int32_t *kv_lens,
                           const float *slopes, int batch, int max_q_len, int num_q_heads,
                           int num_kv_heads, int head_dim, int num_blocks, int dtype, float scale,
                           void *stream) {
  return prefill_common(out, q, total_q, cu_q_lens, q_pos_start, k_pool, v_pool, block_table,
                        max_blocks_per_seq, block_fill, kv_lens, batch, max_q_len, num_q_heads, num_kv_heads,
                        head_dim, num_blocks, dtype, scale, 10000.0f /* unused */, stream, kAlibi, slopes);
}

int lazyattn_prefill_fp8(void *out, const void *q, int total_q, const int32_t *cu_q_lens,
                         const int32_t *q_pos_start, const void *k_pool, const void *v_pool,
                         const uint32_t *block_table, int max_blocks_per_seq, const uint8_t *block_fill,
                         const int32_t *kv_lens, int batch, int max_q_len, int num_q_heads, int num_kv_heads,
                         int head_dim, int num_blocks, float scale, float rope_theta, float k_scale,
                         float v_scale, void *workspace, size_t workspace_bytes, void *stream) {
  return prefill_common(out, q, total_q, cu_q_lens, q_pos_start, k_pool, v_pool, block_table,
                        max_blocks_per_seq, block_fill, kv_lens, batch, max_q_len, num_q_heads, num_kv_heads,
                        head_dim, num_blocks, LAZYATTN_BF16, scale, rope_theta, stream, kRopeLazy, nullptr,
                        true, k_scale, v_scale, workspace, workspace_bytes);
}

int lazyattn_prefill_int8(void *out, const void *q, int total_q, const int32_t *cu_q_lens,
                          const int32_t *q_pos_start, const void *k_pool, const void *v_pool,
                          const uint32_t *block_table, int max_blocks_per_seq, const uint8_t *block_fill,
                          const int32_t *kv_lens, int batch, int max_q_len, int num_q_heads, int num_kv_heads,
                          int head_dim, int num_blocks, float scale, float rope_theta, float k_scale,
                          float v_scale, void *workspace, size_t workspace_bytes, void *stream) {
  return prefill_common(out, q, total_q, cu_q_lens, q_pos_start, k_pool, v_pool, block_table,
                        max_blocks_per_seq, block_fill, kv_lens, batch, max_q_len, num_q_heads, num_kv_heads,
                        head_dim, num_blocks, LAZYATTN_BF16, scale, rope_theta, stream, kRopeLazy, nullptr,
                        true, k_scale, v_scale, workspace, workspace_bytes, true);
}

int lazyattn_prefill_fp8_precise(void *out, const void *q, int total_q, const int32_t *cu_q_lens,
                                 const int32_t *q_pos_start, const void *k_pool, const void *v_pool,
                                 const uint32_t *block_table, int max_blocks_per_seq, const uint8_t *block_fill,
                                 const int32_t *kv_lens, int batch, int max_q_len, int num_q_heads,
                                 int num_kv_heads, int head_dim, int num_blocks, float scale, float rope_theta,
                                 float k_scale, float v_scale, void *workspace, size_t workspace_bytes,
                                 void *stream) {
  return prefill_common(out, q, total_q, cu_q_lens, q_pos_start, k_pool, v_pool, block_table,
                        max_blocks_per_seq, block_fill, kv_lens, batch, max_q_len, num_q_heads, num_kv_heads,
                        head_dim, num_blocks, LAZYATTN_BF16, scale, rope_theta, stream, kRopeLazy, nullptr,
                        true, k_scale, v_scale, workspace, workspace_bytes, false, true);
}

int lazyattn_prefill_int8_precise(void *out, const void *q, int total_q, const int32_t *cu_q_lens,
                                  const int32_t *q_pos_start, const void *k_pool, const void *v_pool,
                                  const uint32_t *block_table, int max_blocks_per_seq, const uint8_t *block_fill,
                                  const int32_t *kv_lens, int batch, int max_q_len, int num_q_heads,
                                  int num_kv_heads, int head_dim, int num_blocks, float scale, float rope_theta,
                                  float k_scale, float v_scale, void *workspace, size_t workspace_bytes,
                                  void *stream) {
  return prefill_common(out, q, total_q, cu_q_lens, q_pos_start, k_pool, v_pool, block_table,
                        max_blocks_per_seq, block_fill, kv_lens, batch, max_q_len, num_q_heads, num_kv_heads,
                        head_dim, num_blocks, LAZYATTN_BF16, scale, rope_theta, stream, kRopeLazy, nullptr,
                        true, k_scale, v_scale, workspace, workspace_bytes, true, true);
}

size_t lazyattn_prefill_fp8_workspace_size(int batch, int max_blocks_per_seq, int num_kv_heads, int head_dim) {
  if (head_dim != 128) return 0;
  return prefill_fp8_workspace_size(batch, max_blocks_per_seq, num_kv_heads);
}

}  // extern "C"

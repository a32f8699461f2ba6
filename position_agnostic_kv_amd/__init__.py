"""Position-agnostic paged KV attention (deferred RoPE) for MI355X / gfx950.

A thin ctypes binding over ``liblazyattn.so`` (C ABI in ``include/lazyattn.h``):
argument marshalling only.  PyTorch supplies device memory and the current
stream; every step of the attention runs in the library's HIP kernels.  If the
library has not been built, every entry point raises -- there is no fallback.

Entry points (same names as the C ABI):
  kvcache_append(k_pool, v_pool, k_new, v_new, slot_mapping)
  lazyattn_decode(q, q_pos, k_pool, v_pool, block_table, seq_lens, ...)
  lazyattn_prefill(q, cu_q_lens, q_pos_start, k_pool, v_pool, block_table, kv_lens, max_q_len, ...)
  lazyattn_decode_eager / lazyattn_prefill_eager: the non-lazy baseline (keys
  already rotated to absolute positions, table offsets ignored)
"""

import ctypes
import math
import os

import torch

__all__ = [
    "LazyAttnError", "lib_path", "load_library", "version", "kvcache_append",
    "decode_workspace_size", "lazyattn_decode", "lazyattn_prefill", "lazyattn_decode_eager",
    "lazyattn_prefill_eager", "lazyattn_prefill_precise", "lazyattn_decode_alibi", "lazyattn_prefill_alibi", "kvcache_append_fp8",
    "lazyattn_decode_fp8", "lazyattn_prefill_fp8", "prefill_fp8_workspace_size", "lazyattn_decode_noalloc",
    "kvcache_append_int8", "lazyattn_decode_int8", "lazyattn_prefill_int8", "lazyattn_prefill_fp8_precise",
    "lazyattn_prefill_int8_precise",
    "DecodePlan", "decode_plan", "decode_planned_workspace_size", "lazyattn_decode_planned", "BLOCK_TOKENS",
]

BLOCK_TOKENS = 16
_F32, _BF16 = 0, 1
_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblazyattn.so")
_lib = None

_vp, _i32, _sz, _f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
_SIGNATURES = {
    "lazyattn_status_string": (ctypes.c_char_p, [_i32]),
    "lazyattn_version": (_i32, []),
    "kvcache_append": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _i32, _vp]),
    "lazyattn_decode_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "lazyattn_decode": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                               _i32, _f32, _f32, _i32, _vp, _sz, _vp]),
    "lazyattn_prefill": (_i32, [_vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32,
                                _i32, _i32, _i32, _i32, _f32, _f32, _vp]),
}
_SIGNATURES.update({
    "lazyattn_cache_create": (_vp, [_i32, _i32]),
    "lazyattn_cache_destroy": (None, [_vp]),
    "lazyattn_cache_acquire": (_i32, [_vp, _vp, _vp, _i32, _i32, _vp, _i32, _vp, _vp]),
    "lazyattn_cache_release": (_i32, [_vp, _i32]),
    "lazyattn_cache_stats": (_i32, [_vp, _vp, _i32]),
})
_SIGNATURES["lazyattn_decode_eager"] = _SIGNATURES["lazyattn_decode"]
_SIGNATURES["lazyattn_decode_noalloc"] = (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32,
                                                 _i32, _i32, _f32, _f32, _i32, _vp])
_SIGNATURES["lazyattn_decode_alibi"] = (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _i32, _i32,
                                               _i32, _i32, _i32, _f32, _i32, _vp, _sz, _vp])
_SIGNATURES["lazyattn_prefill_alibi"] = (_i32, [_vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp,
                                                _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _vp])
_SIGNATURES["lazyattn_prefill_eager"] = _SIGNATURES["lazyattn_prefill"]
_SIGNATURES["lazyattn_prefill_precise"] = _SIGNATURES["lazyattn_prefill"]
_SIGNATURES["kvcache_append_fp8"] = (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _i32, _f32, _f32, _vp])
_SIGNATURES["lazyattn_decode_fp8"] = (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32,
                                             _i32, _f32, _f32, _f32, _f32, _i32, _vp, _sz, _vp])
_SIGNATURES["lazyattn_prefill_fp8"] = (_i32, [_vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32,
                                              _i32, _i32, _i32, _i32, _f32, _f32, _f32, _f32, _vp, _sz, _vp])
_SIGNATURES["lazyattn_prefill_fp8_workspace_size"] = (_sz, [_i32, _i32, _i32, _i32])
_SIGNATURES["kvcache_append_int8"] = _SIGNATURES["kvcache_append_fp8"]
_SIGNATURES["lazyattn_decode_int8"] = _SIGNATURES["lazyattn_decode_fp8"]
_SIGNATURES["lazyattn_prefill_int8"] = _SIGNATURES["lazyattn_prefill_fp8"]
_SIGNATURES["lazyattn_prefill_fp8_precise"] = _SIGNATURES["lazyattn_prefill_fp8"]
_SIGNATURES["lazyattn_prefill_int8_precise"] = _SIGNATURES["lazyattn_prefill_fp8"]
_SIGNATURES["lazyattn_decode_plan_ints"] = (_sz, [_i32, _i32, _i32])
_SIGNATURES["lazyattn_decode_plan"] = (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _sz, _vp, _vp])
_SIGNATURES["lazyattn_decode_planned_workspace_size"] = (_sz, [_i32, _i32, _i32, _i32, _i32])
_SIGNATURES["lazyattn_decode_planned"] = (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32,
                                                 _i32, _i32, _f32, _f32, _vp, _i32, _i32, _vp, _sz, _vp])


class LazyAttnError(RuntimeError):
    pass


def lib_path():
    return _LIB_PATH


def load_library():
    """Load liblazyattn.so (raises if it is missing: there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise LazyAttnError(
                f"{_LIB_PATH} is not built; run `python -m position_agnostic_kv_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _lib = lib
    return _lib


def version():
    return load_library().lazyattn_version()


def _check(status, what):
    if status != 0:
        msg = load_library().lazyattn_status_string(status).decode()
        raise LazyAttnError(f"{what} failed: {msg} (status {status})")


def _dtype_code(t):
    if t.dtype == torch.float32:
        return _F32
    if t.dtype == torch.bfloat16:
        return _BF16
    raise LazyAttnError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _dev(*tensors):
    dev = tensors[0].device
    for t in tensors:
        if t.device.type != "cuda":
            raise LazyAttnError("all tensors must be on the GPU")
        if t.device != dev:
            raise LazyAttnError("all tensors must be on the same GPU")
        if not t.is_contiguous():
            raise LazyAttnError("all tensors must be contiguous")
    return dev


def _int32(t, name):
    if t.dtype not in (torch.int32, torch.uint32):
        raise LazyAttnError(f"{name} must be int32 (uint32 bit patterns for the block table)")
    return t


def _stream_ptr(stream, device):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _hold_temporaries(stream, device, *temps):
    """Make temporaries safe for a launch on a stream other than torch's current one.

    The binding allocates (and fills) its temporaries -- output, workspace,
    padded fill counts -- on the current stream.  When the launch goes to
    another stream, that stream first waits for the current one (so the fills
    are complete and the memory's previous users are done), and each
    temporary is recorded as used by it, so that the caching allocator does
    not hand its memory to new work before the launch has finished."""
    temps = [t for t in temps if t is not None]
    if stream is None or not temps:
        return
    if stream.cuda_stream == torch.cuda.current_stream(device).cuda_stream:
        return
    stream.wait_stream(torch.cuda.current_stream(device))
    for t in temps:
        t.record_stream(stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def kvcache_append(k_pool, v_pool, k_new, v_new, slot_mapping, stream=None):
    """Write rows k_new/v_new [T, Hkv, D] into pool slots (block*16 + slot); < 0 skipped."""
    dev = _dev(k_pool, v_pool, k_new, v_new, slot_mapping)
    _int32(slot_mapping, "slot_mapping")
    nb, hkv, bt, d = k_pool.shape
    if bt != BLOCK_TOKENS or v_pool.shape != k_pool.shape:
        raise LazyAttnError("pools must be [num_blocks, num_kv_heads, 16, head_dim]")
    if k_new.shape != v_new.shape or k_new.shape[1:] != (hkv, d) or k_new.dtype != k_pool.dtype:
        raise LazyAttnError("k_new/v_new must be [T, num_kv_heads, head_dim] of the pool dtype")
    if slot_mapping.numel() != k_new.shape[0]:
        raise LazyAttnError("slot_mapping must have one entry per new row")
    lib = load_library()
    _check(lib.kvcache_append(_ptr(k_pool), _ptr(v_pool), _dtype_code(k_pool), nb, hkv, d,
                              _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), k_new.shape[0],
                              _stream_ptr(stream, dev)), "kvcache_append")


_POOL8 = (torch.uint8, torch.float8_e4m3fn)   # E4M3 code pools
_POOL_INT8 = (torch.int8, torch.uint8)         # int8 code pools (uint8: the same bytes)


def kvcache_append_fp8(k_pool, v_pool, k_new, v_new, slot_mapping, k_scale, v_scale, stream=None):
    """Quantise rows k_new/v_new [T, Hkv, D] (bf16 or f32) into an 8-bit pool
    (uint8 or float8_e4m3fn [NB, Hkv, 16, D] of E4M3 codes): code = nearest E4M3
    of the float32 x / scale, saturating at 448.  Slots < 0 are skipped."""
    return _append8("kvcache_append_fp8", _POOL8, k_pool, v_pool, k_new, v_new, slot_mapping, k_scale, v_scale,
                    stream)


def kvcache_append_int8(k_pool, v_pool, k_new, v_new, slot_mapping, k_scale, v_scale, stream=None):
    """Quantise rows k_new/v_new [T, Hkv, D] (bf16 or f32) into an int8 pool
    (int8 or uint8 [NB, Hkv, 16, D]): code = the float32 x / scale rounded to
    the nearest integer (ties to even), clamped to +-127, NaN as 0.  Slots < 0
    are skipped."""
    return _append8("kvcache_append_int8", _POOL_INT8, k_pool, v_pool, k_new, v_new, slot_mapping, k_scale,
                    v_scale, stream)


def _append8(fn, pool_types, k_pool, v_pool, k_new, v_new, slot_mapping, k_scale, v_scale, stream):
    dev = _dev(k_pool, v_pool, k_new, v_new, slot_mapping)
    _int32(slot_mapping, "slot_mapping")
    nb, hkv, bt, d = k_pool.shape
    if bt != BLOCK_TOKENS or v_pool.shape != k_pool.shape:
        raise LazyAttnError("pools must be [num_blocks, num_kv_heads, 16, head_dim]")
    if k_pool.dtype not in pool_types or v_pool.dtype != k_pool.dtype:
        raise LazyAttnError(f"{fn}: pools must be one of {pool_types}")
    if k_new.shape != v_new.shape or k_new.shape[1:] != (hkv, d) or k_new.dtype != v_new.dtype:
        raise LazyAttnError("k_new/v_new must be [T, num_kv_heads, head_dim] of one dtype")
    if slot_mapping.numel() != k_new.shape[0]:
        raise LazyAttnError("slot_mapping must have one entry per new row")
    lib = load_library()
    _check(getattr(lib, fn)(_ptr(k_pool), _ptr(v_pool), _dtype_code(k_new), nb, hkv, d,
                            _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), k_new.shape[0],
                            float(k_scale), float(v_scale), _stream_ptr(stream, dev)), fn)


def lazyattn_decode_fp8(q, q_pos, k_pool, v_pool, block_table, seq_lens, k_scale, v_scale, *, scale=None,
                        rope_theta=10000.0, split_blocks=0, out=None, workspace=None, stream=None,
                        block_fill=None):
    """lazyattn_decode over an 8-bit pool of E4M3 codes (uint8 or
    float8_e4m3fn): keys are decode(code) * k_scale, values decode(code) *
    v_scale.  q and out are bf16; head_dim 128."""
    return _decode("lazyattn_decode_fp8", q, q_pos, k_pool, v_pool, block_table, seq_lens, scale,
                   rope_theta, split_blocks, out, workspace, stream, block_fill=block_fill,
                   kv_scales=(float(k_scale), float(v_scale)), pool_types=_POOL8)


def lazyattn_decode_int8(q, q_pos, k_pool, v_pool, block_table, seq_lens, k_scale, v_scale, *, scale=None,
                         rope_theta=10000.0, split_blocks=0, out=None, workspace=None, stream=None,
                         block_fill=None):
    """lazyattn_decode over an int8 pool (int8 or uint8): keys are code *
    k_scale, values code * v_scale.  q and out are bf16; head_dim 128."""
    return _decode("lazyattn_decode_int8", q, q_pos, k_pool, v_pool, block_table, seq_lens, scale,
                   rope_theta, split_blocks, out, workspace, stream, block_fill=block_fill,
                   kv_scales=(float(k_scale), float(v_scale)), pool_types=_POOL_INT8)


def decode_workspace_size(batch, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                          split_blocks=0):
    return int(load_library().lazyattn_decode_workspace_size(
        batch, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, split_blocks))


def lazyattn_decode(q, q_pos, k_pool, v_pool, block_table, seq_lens, *, scale=None,
                    rope_theta=10000.0, split_blocks=0, out=None, workspace=None, stream=None,
                    block_fill=None):
    """Decode attention; q [B, Hq, D] raw queries at positions q_pos [B].

    block_table [B, max_blocks] int32/uint32 words (block id | offset << 16);
    seq_lens [B] table slots attended.  ``workspace`` (uint8, zero-filled once)
    is allocated zeroed when not given.  ``block_fill`` (uint8 [num_blocks],
    optional): tokens stored in each physical block; None = all full.
    Returns out [B, Hq, D] in q's dtype.
    """
    return _decode("lazyattn_decode", q, q_pos, k_pool, v_pool, block_table, seq_lens, scale,
                   rope_theta, split_blocks, out, workspace, stream, block_fill=block_fill)


def lazyattn_decode_eager(q, q_pos, k_pool, v_pool, block_table, seq_lens, *, scale=None,
                          rope_theta=10000.0, split_blocks=0, out=None, workspace=None, stream=None,
                          block_fill=None):
    """Non-lazy baseline of lazyattn_decode: the pool holds keys already rotated
    to their absolute positions, table offsets are ignored, q is rotated once."""
    return _decode("lazyattn_decode_eager", q, q_pos, k_pool, v_pool, block_table, seq_lens, scale,
                   rope_theta, split_blocks, out, workspace, stream, block_fill=block_fill)


def lazyattn_decode_alibi(q, q_pos, k_pool, v_pool, block_table, seq_lens, slopes, *, scale=None,
                          split_blocks=0, out=None, workspace=None, stream=None, block_fill=None):
    """Decode with ALiBi biases instead of RoPE: slopes [Hq] float32 on the
    device; each table word's offset is the absolute position of its block's
    first token.  Otherwise as lazyattn_decode."""
    return _decode("lazyattn_decode_alibi", q, q_pos, k_pool, v_pool, block_table, seq_lens, scale,
                   None, split_blocks, out, workspace, stream, slopes=slopes, block_fill=block_fill)


def lazyattn_decode_noalloc(q, q_pos, k_pool, v_pool, block_table, seq_lens, *, out, scale=None,
                            rope_theta=10000.0, split_blocks=0, stream=None, block_fill=None):
    """lazyattn_decode for callers that cannot allocate: the split-K partials
    live in the library's fixed per-GPU scratch (8 MiB; larger needs raise),
    and this wrapper allocates nothing either, so ``out`` must be given and
    ``block_fill`` (if any) must already hold a multiple of 4 entries.  Calls
    that overlap on one GPU race on the shared scratch."""
    dev = _dev(q, q_pos, k_pool, v_pool, block_table, seq_lens, out)
    for t, n in ((q_pos, "q_pos"), (block_table, "block_table"), (seq_lens, "seq_lens")):
        _int32(t, n)
    b, hq, d = q.shape
    nb, hkv, bt, dk = k_pool.shape
    if bt != BLOCK_TOKENS or dk != d or v_pool.shape != k_pool.shape:
        raise LazyAttnError("pools must be [num_blocks, num_kv_heads, 16, head_dim]")
    if q.dtype != k_pool.dtype or v_pool.dtype != k_pool.dtype:
        raise LazyAttnError("q and pools must share a dtype")
    if block_table.dim() != 2 or block_table.shape[0] != b or q_pos.numel() != b or seq_lens.numel() != b:
        raise LazyAttnError("block_table [B, max_blocks], q_pos [B], seq_lens [B]")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise LazyAttnError("out must match q")
    fill = ctypes.c_void_p(0)
    if block_fill is not None:
        _dev(block_fill)
        if block_fill.device != dev or block_fill.dtype != torch.uint8 or block_fill.dim() != 1 \
                or block_fill.numel() < (nb + 3) // 4 * 4:
            raise LazyAttnError("block_fill must be uint8 with num_blocks rounded up to 4 entries "
                                "(no padding copy is made here)")
        fill = _ptr(block_fill)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _check(load_library().lazyattn_decode_noalloc(
        _ptr(out), _ptr(q), _ptr(q_pos), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), block_table.shape[1], fill,
        _ptr(seq_lens), b, hq, hkv, d, nb, _dtype_code(q), scale, float(rope_theta), int(split_blocks),
        _stream_ptr(stream, dev)), "lazyattn_decode_noalloc")
    return out


class DecodePlan:
    """A work plan for lazyattn_decode_planned: ``ints`` (int32, host) as the
    library's planner wrote it, ``device`` its copy on the GPU, and the item
    count and largest per-sequence slot count the call needs."""

    def __init__(self, ints, device, num_items, max_items_per_seq, batch, num_q_heads, num_kv_heads):
        self.ints, self.device = ints, device
        self.num_items, self.max_items_per_seq = num_items, max_items_per_seq
        self.batch, self.num_q_heads, self.num_kv_heads = batch, num_q_heads, num_kv_heads


def decode_plan(block_table, seq_lens, num_q_heads, num_kv_heads, *, max_item_blocks=0, device=None):
    """Build a plan for lazyattn_decode_planned with the library's host-side
    planner (lazyattn_decode_plan) from copies of block_table [B, max_blocks]
    and seq_lens [B] in host memory; the plan goes to ``device`` (default: the
    table's device, if a GPU).  It stays valid while sequences grow into
    blocks appended to their rows; rebuild it when the words already in the
    table, or the head counts, change."""
    _int32(block_table, "block_table")
    _int32(seq_lens, "seq_lens")
    if block_table.dim() != 2 or seq_lens.numel() != block_table.shape[0]:
        raise LazyAttnError("block_table [B, max_blocks], seq_lens [B]")
    b, max_blocks = block_table.shape
    table = block_table.detach().to("cpu").view(torch.int32).contiguous()
    lens = seq_lens.detach().to("cpu").view(torch.int32).contiguous()
    lib = load_library()
    cap = int(lib.lazyattn_decode_plan_ints(b, max_blocks, num_kv_heads))
    if cap == 0:
        raise LazyAttnError("decode_plan: empty batch or bad sizes")
    buf = torch.empty(cap, dtype=torch.int32)
    n, m = ctypes.c_int(0), ctypes.c_int(0)
    _check(lib.lazyattn_decode_plan(_ptr(table), _ptr(lens), b, max_blocks, num_q_heads, num_kv_heads,
                                    int(max_item_blocks), _ptr(buf), cap, ctypes.byref(n), ctypes.byref(m)),
           "lazyattn_decode_plan")
    ints = buf[:(b + 3) // 4 * 4 + 12 * n.value].clone()
    if device is None:
        device = block_table.device if block_table.device.type == "cuda" else None
    dev_ints = ints.to(device) if device is not None else None
    return DecodePlan(ints, dev_ints, n.value, m.value, b, num_q_heads, num_kv_heads)


def decode_planned_workspace_size(batch, num_q_heads, num_kv_heads, head_dim, max_items_per_seq):
    return int(load_library().lazyattn_decode_planned_workspace_size(
        batch, num_q_heads, num_kv_heads, head_dim, max_items_per_seq))


def lazyattn_decode_planned(q, q_pos, k_pool, v_pool, block_table, seq_lens, plan, *, scale=None,
                            rope_theta=10000.0, out=None, workspace=None, stream=None, block_fill=None):
    """lazyattn_decode with the work of ``plan`` (decode_plan of the same
    table, lengths and KV head count): sequences that share a cached document
    read it together.  bf16, head_dim 128, group sizes up to 16."""
    dev = _dev(q, q_pos, k_pool, v_pool, block_table, seq_lens)
    for t, nm in ((q_pos, "q_pos"), (block_table, "block_table"), (seq_lens, "seq_lens")):
        _int32(t, nm)
    b, hq, d = q.shape
    nb, hkv, bt, dk = k_pool.shape
    if bt != BLOCK_TOKENS or dk != d or v_pool.shape != k_pool.shape:
        raise LazyAttnError("pools must be [num_blocks, num_kv_heads, 16, head_dim]")
    if q.dtype != k_pool.dtype or v_pool.dtype != k_pool.dtype:
        raise LazyAttnError("q and pools must share a dtype")
    if block_table.dim() != 2 or block_table.shape[0] != b or q_pos.numel() != b or seq_lens.numel() != b:
        raise LazyAttnError("block_table [B, max_blocks], q_pos [B], seq_lens [B]")
    if not isinstance(plan, DecodePlan) or plan.device is None or plan.batch != b or plan.num_kv_heads != hkv \
            or plan.num_q_heads != hq:
        raise LazyAttnError("plan must be decode_plan() of this batch's table and KV heads, on the GPU")
    _dev(plan.device, q)
    if out is None:
        out = torch.empty_like(q)
        new_out = True
    else:
        new_out = False
        _dev(out, q)
        if out.shape != q.shape or out.dtype != q.dtype:
            raise LazyAttnError("out must match q")
    need = decode_planned_workspace_size(b, hq, hkv, d, plan.max_items_per_seq) if b else 0
    new_ws = workspace is None
    if new_ws:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _dev(workspace, q)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    fill_keep, fill = _fill_arg(block_fill, nb, dev)
    _hold_temporaries(stream, dev, out if new_out else None, workspace if new_ws else None,
                      fill_keep if fill_keep is not block_fill else None)
    _check(load_library().lazyattn_decode_planned(
        _ptr(out), _ptr(q), _ptr(q_pos), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), block_table.shape[1], fill,
        _ptr(seq_lens), b, hq, hkv, d, nb, _dtype_code(q), scale, float(rope_theta), _ptr(plan.device),
        plan.num_items, plan.max_items_per_seq, _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream_ptr(stream, dev)), "lazyattn_decode_planned")
    return out


def _fill_arg(block_fill, num_blocks, dev):
    """The block_fill pointer (NULL for None); the library reads it in 4-byte
    words, so a tensor shorter than num_blocks rounded up to 4 is padded."""
    if block_fill is None:
        return None, ctypes.c_void_p(0)
    _dev(block_fill)
    if block_fill.device != dev or block_fill.dtype != torch.uint8 or block_fill.dim() != 1 \
            or block_fill.numel() < num_blocks:
        raise LazyAttnError("block_fill must be a uint8 tensor of num_blocks entries on the inputs' device")
    need = (num_blocks + 3) // 4 * 4
    if block_fill.numel() < need:
        block_fill = torch.cat([block_fill, block_fill.new_full((need - block_fill.numel(),), 16)])
    return block_fill, _ptr(block_fill)


def _decode(fn, q, q_pos, k_pool, v_pool, block_table, seq_lens, scale, rope_theta, split_blocks,
            out, workspace, stream, slopes=None, block_fill=None, kv_scales=None, pool_types=_POOL8):
    dev = _dev(q, q_pos, k_pool, v_pool, block_table, seq_lens)
    _int32(q_pos, "q_pos")
    _int32(block_table, "block_table")
    _int32(seq_lens, "seq_lens")
    b, hq, d = q.shape
    nb, hkv, bt, dk = k_pool.shape
    if bt != BLOCK_TOKENS or dk != d or v_pool.shape != k_pool.shape:
        raise LazyAttnError("pools must be [num_blocks, num_kv_heads, 16, head_dim]")
    if kv_scales is not None:
        if q.dtype != torch.bfloat16 or k_pool.dtype not in pool_types or v_pool.dtype != k_pool.dtype:
            raise LazyAttnError(f"{fn}: pools must be one of {pool_types}, queries bf16")
    elif q.dtype != k_pool.dtype or v_pool.dtype != k_pool.dtype:
        raise LazyAttnError("q and pools must share a dtype")
    if block_table.dim() != 2 or block_table.shape[0] != b or q_pos.numel() != b or seq_lens.numel() != b:
        raise LazyAttnError("block_table [B, max_blocks], q_pos [B], seq_lens [B]")
    max_blocks = block_table.shape[1]
    new_out = out is None
    if new_out:
        out = torch.empty_like(q)
    else:
        _dev(out, q)
        if out.shape != q.shape or out.dtype != q.dtype:
            raise LazyAttnError("out must match q")
    need = decode_workspace_size(b, hq, hkv, d, max_blocks, split_blocks) if b else 0
    new_ws = workspace is None
    if new_ws:
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _dev(workspace, q)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    fill_keep, fill = _fill_arg(block_fill, nb, dev)
    _hold_temporaries(stream, dev, out if new_out else None, workspace if new_ws else None,
                      fill_keep if fill_keep is not block_fill else None)
    lib = load_library()
    if slopes is not None:
        _slopes(slopes, hq, dev)
        _check(getattr(lib, fn)(_ptr(out), _ptr(q), _ptr(q_pos), _ptr(k_pool), _ptr(v_pool),
                                _ptr(block_table), max_blocks, fill, _ptr(seq_lens), _ptr(slopes), b, hq, hkv,
                                d, nb, _dtype_code(q), scale, int(split_blocks), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream_ptr(stream, dev)), fn)
        return out
    if kv_scales is not None:
        _check(getattr(lib, fn)(_ptr(out), _ptr(q), _ptr(q_pos), _ptr(k_pool), _ptr(v_pool),
                                _ptr(block_table), max_blocks, fill, _ptr(seq_lens), b, hq, hkv, d, nb,
                                scale, float(rope_theta), kv_scales[0], kv_scales[1], int(split_blocks),
                                _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream_ptr(stream, dev)), fn)
        return out
    _check(getattr(lib, fn)(_ptr(out), _ptr(q), _ptr(q_pos), _ptr(k_pool), _ptr(v_pool),
                            _ptr(block_table), max_blocks, fill, _ptr(seq_lens), b, hq, hkv, d, nb,
                            _dtype_code(q), scale, float(rope_theta), int(split_blocks),
                            _ptr(workspace), workspace.numel() * workspace.element_size(),
                            _stream_ptr(stream, dev)), fn)
    return out


def _slopes(slopes, hq, dev):
    _dev(slopes)
    if slopes.dtype != torch.float32 or slopes.numel() != hq or not slopes.is_contiguous():
        raise LazyAttnError("slopes must be a contiguous float32 tensor of num_q_heads entries")
    if slopes.device != dev:
        raise LazyAttnError("slopes must be on the inputs' device")


def lazyattn_prefill(q, cu_q_lens, q_pos_start, k_pool, v_pool, block_table, kv_lens, max_q_len,
                     *, scale=None, rope_theta=10000.0, out=None, stream=None, block_fill=None):
    """Prefill attention; q [Tq, Hq, D] bf16 packed by cu_q_lens [B+1].

    The prompts' K/V must already be appended as each table's last tokens;
    kv_lens [B] counts them.  Returns out [Tq, Hq, D] bf16.
    """
    return _prefill("lazyattn_prefill", q, cu_q_lens, q_pos_start, k_pool, v_pool, block_table,
                    kv_lens, max_q_len, scale, rope_theta, out, stream, block_fill=block_fill)


def lazyattn_prefill_eager(q, cu_q_lens, q_pos_start, k_pool, v_pool, block_table, kv_lens, max_q_len,
                           *, scale=None, rope_theta=10000.0, out=None, stream=None, block_fill=None):
    """Non-lazy baseline of lazyattn_prefill: keys already rotated to their
    absolute positions, table offsets ignored, each query row rotated once."""
    return _prefill("lazyattn_prefill_eager", q, cu_q_lens, q_pos_start, k_pool, v_pool, block_table,
                    kv_lens, max_q_len, scale, rope_theta, out, stream, block_fill=block_fill)


def lazyattn_prefill_precise(q, cu_q_lens, q_pos_start, k_pool, v_pool, block_table, kv_lens, max_q_len,
                             *, scale=None, rope_theta=10000.0, out=None, stream=None, block_fill=None):
    """lazyattn_prefill with the rotated query carried as bf16 hi + lo (twice
    the Q.K^T products): accurate however widely the scores spread."""
    return _prefill("lazyattn_prefill_precise", q, cu_q_lens, q_pos_start, k_pool, v_pool, block_table,
                    kv_lens, max_q_len, scale, rope_theta, out, stream, block_fill=block_fill)


def lazyattn_prefill_alibi(q, cu_q_lens, q_pos_start, k_pool, v_pool, block_table, kv_lens, max_q_len,
                           slopes, *, scale=None, out=None, stream=None, block_fill=None):
    """Prefill with ALiBi biases instead of RoPE (see lazyattn_decode_alibi)."""
    return _prefill("lazyattn_prefill_alibi", q, cu_q_lens, q_pos_start, k_pool, v_pool, block_table,
                    kv_lens, max_q_len, scale, None, out, stream, slopes=slopes, block_fill=block_fill)


def prefill_fp8_workspace_size(batch, max_blocks_per_seq, num_kv_heads, head_dim=128):
    return int(load_library().lazyattn_prefill_fp8_workspace_size(batch, max_blocks_per_seq, num_kv_heads,
                                                                  head_dim))


def lazyattn_prefill_fp8(q, cu_q_lens, q_pos_start, k_pool, v_pool, block_table, kv_lens, max_q_len,
                         k_scale, v_scale, *, scale=None, rope_theta=10000.0, out=None, workspace=None,
                         stream=None, block_fill=None):
    """lazyattn_prefill over an 8-bit pool of E4M3 codes (uint8 or
    float8_e4m3fn) written by kvcache_append_fp8: keys are decode(code) *
    k_scale, values decode(code) * v_scale.  q and out are bf16; head_dim 128.
    workspace: device bytes for the widened copy of the visible blocks
    (prefill_fp8_workspace_size); allocated here when not given."""
    return _prefill("lazyattn_prefill_fp8", q, cu_q_lens, q_pos_start, k_pool, v_pool, block_table,
                    kv_lens, max_q_len, scale, rope_theta, out, stream, block_fill=block_fill,
                    kv_scales=(float(k_scale), float(v_scale)), workspace=workspace, pool_types=_POOL8)


def lazyattn_prefill_int8(q, cu_q_lens, q_pos_start, k_pool, v_pool, block_table, kv_lens, max_q_len,
                          k_scale, v_scale, *, scale=None, rope_theta=10000.0, out=None, workspace=None,
                          stream=None, block_fill=None):
    """lazyattn_prefill over an int8 pool (int8 or uint8) written by
    kvcache_append_int8: keys are code * k_scale, values code * v_scale.
    workspace as lazyattn_prefill_fp8 (prefill_fp8_workspace_size bytes)."""
    return _prefill("lazyattn_prefill_int8", q, cu_q_lens, q_pos_start, k_pool, v_pool, block_table,
                    kv_lens, max_q_len, scale, rope_theta, out, stream, block_fill=block_fill,
                    kv_scales=(float(k_scale), float(v_scale)), workspace=workspace, pool_types=_POOL_INT8)


def lazyattn_prefill_fp8_precise(q, cu_q_lens, q_pos_start, k_pool, v_pool, block_table, kv_lens, max_q_len,
                                 k_scale, v_scale, *, scale=None, rope_theta=10000.0, out=None, workspace=None,
                                 stream=None, block_fill=None):
    """lazyattn_prefill_fp8 with the rotated query as bf16 hi + lo (see
    lazyattn_prefill_precise)."""
    return _prefill("lazyattn_prefill_fp8_precise", q, cu_q_lens, q_pos_start, k_pool, v_pool, block_table,
                    kv_lens, max_q_len, scale, rope_theta, out, stream, block_fill=block_fill,
                    kv_scales=(float(k_scale), float(v_scale)), workspace=workspace, pool_types=_POOL8)


def lazyattn_prefill_int8_precise(q, cu_q_lens, q_pos_start, k_pool, v_pool, block_table, kv_lens, max_q_len,
                                  k_scale, v_scale, *, scale=None, rope_theta=10000.0, out=None, workspace=None,
                                  stream=None, block_fill=None):
    """lazyattn_prefill_int8 with the rotated query as bf16 hi + lo (see
    lazyattn_prefill_precise)."""
    return _prefill("lazyattn_prefill_int8_precise", q, cu_q_lens, q_pos_start, k_pool, v_pool, block_table,
                    kv_lens, max_q_len, scale, rope_theta, out, stream, block_fill=block_fill,
                    kv_scales=(float(k_scale), float(v_scale)), workspace=workspace, pool_types=_POOL_INT8)


def _prefill(fn, q, cu_q_lens, q_pos_start, k_pool, v_pool, block_table, kv_lens, max_q_len, scale,
             rope_theta, out, stream, slopes=None, block_fill=None, kv_scales=None, workspace=None,
             pool_types=_POOL8):
    dev = _dev(q, cu_q_lens, q_pos_start, k_pool, v_pool, block_table, kv_lens)
    for t, n in ((cu_q_lens, "cu_q_lens"), (q_pos_start, "q_pos_start"), (kv_lens, "kv_lens"),
                 (block_table, "block_table")):
        _int32(t, n)
    tq, hq, d = q.shape
    nb, hkv, bt, dk = k_pool.shape
    b = kv_lens.numel()
    if bt != BLOCK_TOKENS or dk != d or v_pool.shape != k_pool.shape:
        raise LazyAttnError("pools must be [num_blocks, num_kv_heads, 16, head_dim]")
    if kv_scales is not None:
        if q.dtype != torch.bfloat16 or k_pool.dtype not in pool_types or v_pool.dtype != k_pool.dtype:
            raise LazyAttnError(f"{fn}: pools must be one of {pool_types}, queries bf16")
    elif q.dtype != k_pool.dtype or v_pool.dtype != k_pool.dtype:
        raise LazyAttnError("q and pools must share a dtype")
    if cu_q_lens.numel() != b + 1 or q_pos_start.numel() != b or block_table.dim() != 2 \
            or block_table.shape[0] != b:
        raise LazyAttnError("cu_q_lens [B+1], q_pos_start [B], block_table [B, max_blocks], kv_lens [B]")
    new_out = out is None
    if new_out:
        out = torch.empty_like(q)
    else:
        _dev(out, q)
        if out.shape != q.shape or out.dtype != q.dtype:
            raise LazyAttnError("out must match q")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    fill_keep, fill = _fill_arg(block_fill, nb, dev)
    new_ws = kv_scales is not None and workspace is None
    if new_ws:
        need = prefill_fp8_workspace_size(b, block_table.shape[1], hkv, d) if b else 0
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif workspace is not None:
        _dev(workspace, q)
    _hold_temporaries(stream, dev, out if new_out else None, workspace if new_ws else None,
                      fill_keep if fill_keep is not block_fill else None)
    lib = load_library()
    if slopes is not None:
        _slopes(slopes, hq, dev)
        _check(getattr(lib, fn)(_ptr(out), _ptr(q), tq, _ptr(cu_q_lens), _ptr(q_pos_start), _ptr(k_pool),
                                _ptr(v_pool), _ptr(block_table), block_table.shape[1], fill, _ptr(kv_lens),
                                _ptr(slopes), b, int(max_q_len), hq, hkv, d, nb, _dtype_code(q), scale,
                                _stream_ptr(stream, dev)), fn)
        return out
    if kv_scales is not None:
        _check(getattr(lib, fn)(_ptr(out), _ptr(q), tq, _ptr(cu_q_lens), _ptr(q_pos_start), _ptr(k_pool),
                                _ptr(v_pool), _ptr(block_table), block_table.shape[1], fill, _ptr(kv_lens),
                                b, int(max_q_len), hq, hkv, d, nb, scale, float(rope_theta), kv_scales[0],
                                kv_scales[1], _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream_ptr(stream, dev)), fn)
        return out
    _check(getattr(lib, fn)(_ptr(out), _ptr(q), tq, _ptr(cu_q_lens), _ptr(q_pos_start), _ptr(k_pool),
                            _ptr(v_pool), _ptr(block_table), block_table.shape[1], fill, _ptr(kv_lens),
                            b, int(max_q_len), hq, hkv, d, nb, _dtype_code(q), scale,
                            float(rope_theta), _stream_ptr(stream, dev)), fn)
    return out

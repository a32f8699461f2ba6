"""ctypes binding of the host-side KV pool manager (include/lazyattn_cache.h).

The manager hands out 16-token blocks from a free list, keeps cached documents
with reference counts, evicts unreferenced documents least-recently-used first,
and writes each request's block-table row in the (block id | frame start << 16)
format that lazyattn_decode / lazyattn_prefill read.  All bookkeeping runs in
native code; this module only marshals arguments.
"""

import ctypes

import numpy as np

from . import LazyAttnError, load_library

AGNOSTIC, AWARE, PREFIX = 0, 1, 2
MODES = {"agnostic": AGNOSTIC, "aware": AWARE, "prefix": PREFIX}
STATS = ("requests", "doc_hits", "doc_misses", "tokens_hit", "tokens_missed", "evicted",
         "free_blocks", "doc_blocks", "prompt_blocks", "cached_docs")
ERR_ARG, ERR_NOSPACE, ERR_POSITION = -1, -2, -3


class CacheError(LazyAttnError):
    def __init__(self, status, what):
        super().__init__(f"{what}: status {status}")
        self.status = status


class CacheManager:
    """A manager for a pool of `num_blocks` blocks under one cache-key `mode`
    ("agnostic", "aware" or "prefix", or the enum value)."""

    def __init__(self, num_blocks, mode="agnostic"):
        self._h = None
        self._lib = load_library()
        m = MODES[mode] if isinstance(mode, str) else int(mode)
        self._h = self._lib.lazyattn_cache_create(int(num_blocks), m)
        if not self._h:
            raise CacheError(ERR_ARG, f"lazyattn_cache_create({num_blocks}, {mode})")
        self.num_blocks = int(num_blocks)

    def close(self):
        if self._h:
            self._lib.lazyattn_cache_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def acquire(self, doc_ids, doc_lens, prompt_len=0, max_blocks=None):
        """Place one request; returns (table_row uint32[n], miss uint8[n_docs], request_id).
        Raises CacheError (status -2: no space, -3: positions past 65535, -1: bad argument)."""
        ids = np.ascontiguousarray(doc_ids, dtype=np.int32)
        lens = np.ascontiguousarray(doc_lens, dtype=np.int32)
        if ids.shape != lens.shape or ids.ndim != 1:
            raise CacheError(ERR_ARG, "doc_ids and doc_lens must be 1-D of one length")
        if max_blocks is None:
            max_blocks = int(np.sum(np.maximum(lens, 0)) // 16 + (int(prompt_len) + 15) // 16)
        row = np.zeros(max(int(max_blocks), 1), dtype=np.uint32)
        miss = np.zeros(max(len(ids), 1), dtype=np.uint8)
        rid = ctypes.c_int32(-1)
        n = self._lib.lazyattn_cache_acquire(self._h, ids.ctypes.data, lens.ctypes.data, len(ids),
                                             int(prompt_len), row.ctypes.data, int(max_blocks),
                                             miss.ctypes.data, ctypes.byref(rid))
        if n < 0:
            raise CacheError(n, "lazyattn_cache_acquire")
        return row[:n].copy(), miss[:len(ids)].copy(), int(rid.value)

    def release(self, request_id):
        st = self._lib.lazyattn_cache_release(self._h, int(request_id))
        if st != 0:
            raise CacheError(st, "lazyattn_cache_release")

    def stats(self):
        out = np.zeros(len(STATS), dtype=np.int64)
        n = self._lib.lazyattn_cache_stats(self._h, out.ctypes.data, len(STATS))
        return {k: int(v) for k, v in zip(STATS[:n], out[:n])}

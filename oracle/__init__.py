"""CPU oracle for position-agnostic (deferred-RoPE) paged attention.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain reference that the
HIP library is checked against.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it; the product path
(``position_agnostic_kv_amd``) never does, and the two share no code.

Everything here is numpy in float64 and follows the definitions on the pages
step by step, without blocking, fusion or reordering:

* [LA]  gist.science, "Resumo Técnico: LazyAttention" (summary of the
  LazyAttention paper): sections "Declaração do Problema", "Metodologia",
  "Implementação Técnica" (Prefilling, Decoding), "Equivalência Matemática".
* [KVF] ai-engineering.academy, "KV Cache, Flash Attention & Otimização de
  Inferência": sections "Flash Attention" (standard attention, running
  softmax), "PagedAttention", "Construa" (Passo 1 KVCache, Passo 2 tile-by-tile
  softmax).
* [WHY] lynx-cortex, "00 — Por qué existe un KV Cache": sections
  "Lo que hace el decoding autorregresivo", "El remedio", "El precio".

Modules: ``lazy_oracle`` (deferred-RoPE attention, append, cache bytes, the
tile-by-tile softmax), ``alibi_oracle`` (the ALiBi variant), ``quant_oracle`` (KV
pools of 8-bit E4M3 floats or int8 integers, one scale per tensor) and ``cache_policy``
(a plain model of the host pool manager's block and eviction policy).

Every function is pinned by a ``-m "not gpu"`` test in ``tests/`` against
something other than itself (closed forms, a complex-number formulation of
the rotation, brute force, torch's CPU scaled_dot_product_attention, values
the pages print).  No function here is "parity unpinned".
"""

from .lazy_oracle import (  # noqa: F401
    BLOCK_TOKENS,
    append,
    cache_bytes,
    decode,
    decode_one,
    materialize_sequence,
    prefill,
    prefill_rows,
    rope,
    rope_frequencies,
    softmax,
    relative_rotation_overhead,
    blockwise_softmax_dot,
    merge_tile_partials,
    unpack_block_word,
    valid_slots,
)
from .alibi_oracle import alibi_slopes, decode_alibi, key_positions, prefill_alibi  # noqa: F401
from .quant_oracle import (  # noqa: F401
    append_fp8,
    append_int8,
    decode_fp8,
    decode_int8,
    dequantize,
    dequantize_int8,
    e4m3_decode,
    e4m3_quantize,
    int8_decode,
    int8_quantize,
    prefill_fp8,
    prefill_int8,
    quantize_kv,
    quantize_kv_int8,
)

"""CPU pins of the algorithmic work that bench.py's roofline fractions divide
by, against closed forms of the workload shapes (not against bench.py's own
arithmetic): the 8B prefill's attention FLOPs, and the 8B and 70B decodes'
K+V bytes and the extra bytes of queries, outputs, table words and lengths."""

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402


def test_prefill_flops_closed_form():
    # 4 sequences x 32 query heads; each prompt row r (0..2047) sees the 6144
    # cached keys plus prompt keys 0..r: 2048 * 6144 + 2048 * 2049 / 2 pairs;
    # QK^T and PV take 2 * 128 FLOPs each per pair
    case = W.make("llama8b_prefill")
    pairs = 2048 * 6144 + 2048 * 2049 // 2
    assert case.attention_flops() == 4 * 128 * pairs * 32 * 4 == 962139783168


def test_decode_bytes_closed_form():
    for name, batch, ctx, hq, hkv in (("llama8b_decode", 64, 8193, 32, 8), ("llama70b_decode", 16, 32769, 64, 8)):
        case = W.make(name)
        assert case.batch == batch and case.num_q_heads == hq and case.num_kv_heads == hkv
        assert (case.seq_lens == ctx).all()
        kv, total = bench.decode_algorithmic_bytes(case)
        assert kv == batch * ctx * hkv * 128 * 2 * 2        # K and V, bf16, each token once per KV head
        blocks = batch * -(-ctx // 16)
        extra = batch * hq * 128 * 2 * 2 + blocks * 4 + batch * 8   # q in + out, table words, lengths
        assert total == kv + extra
    assert bench.decode_algorithmic_bytes(W.make("llama8b_decode"))[1] == 2148926208

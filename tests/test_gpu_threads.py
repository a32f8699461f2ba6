"""Calls from several host threads at once (the C ABI is re-entrant).

Four threads, each with its own stream, output buffers and decode workspace,
run decode and prefill on shared read-only inputs twenty times over, while
the others do the same.  ctypes releases the interpreter lock for the
duration of each foreign call, so the library's host code runs concurrently.
Every result must be bit-identical to the same call made alone on the
current stream (the kernels are deterministic for fixed inputs and
launch configuration).  lazyattn_decode_noalloc is left out: its fixed
scratch is shared by design, and overlapping calls to it race.
"""

import threading

import numpy as np
import pytest
import torch

import position_agnostic_kv_amd as pak
import workloads as W
from tests.gpu_helpers import DEV, DeviceCase, assert_parity, oracle_decode, oracle_prefill, say

pytestmark = pytest.mark.gpu

THREADS, REPEATS = 4, 20


def test_concurrent_host_threads_give_serial_results():
    dcase = W.materialize_numpy(W.decode_case(171, 4, 32, 8, 128, [640, 1024, 208, 96], (2, 12),
                                              offsets="random"))
    pcase = W.materialize_numpy(W.prefill_case(172, 2, 32, 8, 128, [512, 256], [200, 130], (2, 10),
                                               offsets="random"))
    dd, pd = DeviceCase(dcase), DeviceCase(pcase)
    dd.append()
    pd.append()
    split = 4
    wsb = pak.decode_workspace_size(dcase.batch, dcase.num_q_heads, dcase.num_kv_heads, dcase.head_dim,
                                    dd.table.shape[1], split)

    def decode(out, ws, stream=None):
        return pak.lazyattn_decode(dd.q, dd.q_pos, dd.k_pool, dd.v_pool, dd.table, dd.seq_lens,
                                   scale=dcase.scale, rope_theta=dcase.rope_theta, split_blocks=split,
                                   out=out, workspace=ws, stream=stream)

    def prefill(out, stream=None):
        return pak.lazyattn_prefill(pd.q, pd.cu, pd.q_pos_start, pd.k_pool, pd.v_pool, pd.table, pd.seq_lens,
                                    pcase.max_q_len, scale=pcase.scale, rope_theta=pcase.rope_theta, out=out,
                                    stream=stream)

    say("[threads] serial reference")
    ref_d = decode(torch.empty_like(dd.q), torch.zeros(max(wsb, 16), dtype=torch.uint8, device=DEV))
    ref_p = prefill(torch.empty_like(pd.q))
    torch.cuda.synchronize()
    assert_parity(W.to_float(ref_d, dcase.dtype), oracle_decode(dcase), dcase.dtype, "serial decode")
    assert_parity(W.to_float(ref_p, pcase.dtype), oracle_prefill(pcase), pcase.dtype, "serial prefill")

    streams = [torch.cuda.Stream() for _ in range(THREADS)]
    outs_d = [torch.empty_like(dd.q) for _ in range(THREADS)]
    outs_p = [torch.empty_like(pd.q) for _ in range(THREADS)]
    wss = [torch.zeros(max(wsb, 16), dtype=torch.uint8, device=DEV) for _ in range(THREADS)]
    torch.cuda.synchronize()
    mismatches, errors = [], []
    start = threading.Barrier(THREADS)

    def worker(t):
        try:
            start.wait()
            for i in range(REPEATS):
                decode(outs_d[t], wss[t], streams[t])
                prefill(outs_p[t], streams[t])
                streams[t].synchronize()
                if not torch.equal(outs_d[t], ref_d) or not torch.equal(outs_p[t], ref_p):
                    mismatches.append((t, i))
        except Exception as e:  # reported below, on the main thread
            errors.append((t, repr(e)))

    say(f"[threads] {THREADS} threads x {REPEATS} decode + prefill")
    threads = [threading.Thread(target=worker, args=(t,)) for t in range(THREADS)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a thread did not finish"
    assert not errors, errors
    assert not mismatches, f"results differing from the serial call: {mismatches[:8]}"
    assert np.isfinite(W.to_float(outs_p[0], pcase.dtype)).all()

"""Helpers for the GPU parity tests: move a workload to the device, run one
step through the C ABI (append, then attend), and compute the oracle on the
same values (bf16 inputs widened exactly)."""

import sys

import numpy as np
import torch

import oracle
import position_agnostic_kv_amd as pak
import workloads as W
from workloads.device import DeviceInputs

# tolerances, from the stated targets: fp32 inputs <= 1e-5 max-abs; bf16 inputs
# with fp32 accumulation <= 2e-2 max-abs and <= 5e-3 mean-abs
TOL_F32_MAX = 1e-5
TOL_BF16_MAX = 2e-2
TOL_BF16_MEAN = 5e-3

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class DeviceCase(DeviceInputs):
    """A workload on the GPU plus one step through the C ABI."""

    def __init__(self, case):
        super().__init__(case, DEV)

    def append(self):
        if self.k_new.shape[0]:
            pak.kvcache_append(self.k_pool, self.v_pool, self.k_new, self.v_new, self.slots)

    def decode(self, split_blocks=0, workspace=None, seq_lens=None, q_pos=None):
        c = self.case
        return pak.lazyattn_decode(self.q, self.q_pos if q_pos is None else q_pos, self.k_pool,
                                   self.v_pool, self.table,
                                   self.seq_lens if seq_lens is None else seq_lens,
                                   scale=c.scale, rope_theta=c.rope_theta,
                                   split_blocks=split_blocks, workspace=workspace, block_fill=self.fill)

    def prefill(self, precise=False):
        c = self.case
        fn = pak.lazyattn_prefill_precise if precise else pak.lazyattn_prefill
        return fn(self.q, self.cu, self.q_pos_start, self.k_pool, self.v_pool, self.table, self.seq_lens,
                  c.max_q_len, scale=c.scale, rope_theta=c.rope_theta, block_fill=self.fill)


def host_float(t_or_a, dtype):
    return W.to_float(t_or_a, dtype).astype(np.float64)


def host_pools_after_append(case):
    """Oracle-side pools: the case's pools with the step's new rows appended."""
    k = W.to_float(case.k_pool, case.dtype)
    v = W.to_float(case.v_pool, case.dtype)
    kn = W.to_float(case.k_new, case.dtype)
    vn = W.to_float(case.v_new, case.dtype)
    return oracle.append(k, v, kn, vn, case.layout.slot_mapping)


def oracle_decode(case, k_pool=None, v_pool=None):
    if k_pool is None:
        k_pool, v_pool = host_pools_after_append(case)
    q = W.to_float(case.q, case.dtype)
    return oracle.decode(q, case.q_pos, k_pool, v_pool, case.layout.table, case.seq_lens,
                         case.scale, case.rope_theta, block_fill=case.block_fill)


def oracle_prefill(case, k_pool=None, v_pool=None):
    if k_pool is None:
        k_pool, v_pool = host_pools_after_append(case)
    q = W.to_float(case.q, case.dtype)
    return oracle.prefill(q, case.cu_q_lens, case.layout.tail_pos, k_pool, v_pool, case.layout.table,
                          case.seq_lens, case.scale, case.rope_theta, block_fill=case.block_fill)


def errors(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    diff = np.abs(got - want)
    return float(diff.max()) if diff.size else 0.0, float(diff.mean()) if diff.size else 0.0


def assert_parity(got, want, dtype, what):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    mx, mean = errors(got, want)
    say(f"  {what}: max-abs {mx:.3e} mean-abs {mean:.3e}")
    if dtype == W.F32:
        assert mx <= TOL_F32_MAX, f"{what}: max-abs {mx:.3e} > {TOL_F32_MAX}"
    else:
        assert mx <= TOL_BF16_MAX, f"{what}: max-abs {mx:.3e} > {TOL_BF16_MAX}"
        assert mean <= TOL_BF16_MEAN, f"{what}: mean-abs {mean:.3e} > {TOL_BF16_MEAN}"

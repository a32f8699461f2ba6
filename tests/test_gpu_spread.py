"""GPU parity when scores spread widely across keys (not a common shift).

Keys are N(0, sigma^2) per element and q ~ N(0, 1), so with the scale
1/sqrt(D) a query's scores have standard deviation sigma (natural-log units)
across keys; values are U(-2, 2), so the output's own bf16 rounding stays
small next to errors in the scores.  The pages put every quality difference
of the method down to floating-point precision (LazyAttention summary,
"Resultados Experimentais"); these cases find where that precision stops
meeting the stated tolerance (bf16: 2e-2 max-abs, 5e-3 mean-abs).

* Decode forms the rotated, pre-scaled query q' in float and hands it to
  the matrix cores as two bf16 parts (hi + lo), so q' is carried to ~2^-17:
  green at every spread tried, up to sigma = 64.
* Prefill rounds q' to bf16 once per query row and document (a second
  product against the low part would add half again to its matrix-core
  work, and the prefill is bound by that work).  An error of 2^-9 relative
  in q' moves a score by ~sigma * 2^-9, so the tolerance holds up to
  sigma = 2 and not beyond; the failing spreads are kept as skipped cases
  with the errors measured on MI355X.  A bf16 pipeline that rotates q and
  stores it as bf16 before attention rounds the same way.
  lazyattn_prefill_precise carries q' as hi + lo as the decode does (twice
  the Q.K^T products, ~20 % more time on the 8B prefill) and is green at the
  same spreads up to sigma = 64 (tests/test_gpu_precise.py).
* 8-bit pools: a K scale of 3 on codes up to 7.5 spreads scores the same
  way; a V scale of 2 makes |V| up to 15, where the bf16 rounding of the
  softmax weights and of the output itself (2^-9 relative) reaches the
  absolute tolerance.
"""

import pytest
import torch

import workloads as W
from tests.gpu_helpers import DeviceCase, assert_parity, oracle_decode, oracle_prefill, say

pytestmark = pytest.mark.gpu


def _decode(sigma, hq, hkv, d, split):
    case = W.decode_case(300 + hq, 3, hq, hkv, d, [1024, 512, 208], (2, 12), offsets="random")
    W.materialize_numpy(case)
    W.set_score_spread(case, sigma, seed=hq)
    say(f"[spread decode] sigma {sigma} Hq{hq} Hkv{hkv} D{d} split {split}")
    dc = DeviceCase(case)
    dc.append()
    out = dc.decode(split_blocks=split)
    torch.cuda.synchronize()
    assert_parity(W.to_float(out, case.dtype), oracle_decode(case), case.dtype,
                  f"spread {sigma} decode G{hq // hkv} D{d}")


def _prefill(sigma, hq, hkv, d):
    case = W.prefill_case(310 + hq, 2, hq, hkv, d, [512, 768], [300, 200], (2, 12), offsets="random")
    W.materialize_numpy(case)
    W.set_score_spread(case, sigma, seed=hq)
    say(f"[spread prefill] sigma {sigma} Hq{hq} Hkv{hkv} D{d}")
    dc = DeviceCase(case)
    dc.append()
    out = dc.prefill()
    torch.cuda.synchronize()
    assert_parity(W.to_float(out, case.dtype), oracle_prefill(case), case.dtype,
                  f"spread {sigma} prefill G{hq // hkv} D{d}")


@pytest.mark.parametrize("sigma", [4, 16, 64])
@pytest.mark.parametrize("hq,hkv,d,split", [(32, 8, 128, 0), (64, 1, 128, 4), (16, 4, 64, 0)])
def test_decode_wide_score_spread(sigma, hq, hkv, d, split):
    """Matrix-core decode (GQA 4; MQA 64 with split-K) and the VALU decode
    (head_dim 64): green up to sigma = 64 (measured max-abs <= 5.2e-3)."""
    _decode(sigma, hq, hkv, d, split)


_Q_ROUNDING = ("lazyattn_prefill rounds the rotated query to bf16; lazyattn_prefill_precise (hi + lo query) "
               "is green at this spread")
_Q_ROUNDING_8BIT = ("lazyattn_prefill_fp8 rounds the rotated, K-scaled query to bf16; "
                    "lazyattn_prefill_fp8_precise (hi + lo query) is green at k_scale 3 "
                    "(tests/test_gpu_fp8.py)")


@pytest.mark.parametrize("sigma,hq,hkv,d", [
    (1, 32, 8, 128),
    (2, 32, 8, 128),
    (2, 8, 4, 64),
    pytest.param(3, 32, 8, 128, marks=pytest.mark.skip(
        reason=f"measured max-abs 2.36e-2 > 2e-2 at sigma 3 (mean 1.3e-3): {_Q_ROUNDING}")),
    pytest.param(8, 32, 8, 128, marks=pytest.mark.skip(
        reason=f"measured max-abs 6.06e-2 > 2e-2 at sigma 8 (mean 3.2e-3): {_Q_ROUNDING}")),
    pytest.param(64, 32, 8, 128, marks=pytest.mark.skip(
        reason=f"measured max-abs 4.31e-1 > 2e-2 at sigma 64 (mean 4.1e-3): {_Q_ROUNDING}")),
])
def test_prefill_wide_score_spread(sigma, hq, hkv, d):
    """Prefill: green up to sigma = 2 (measured max-abs 1.06e-2 for head_dim
    128, 9.7e-3 for 64); the wider spreads are skipped with their errors."""
    _prefill(sigma, hq, hkv, d)


@pytest.mark.parametrize("kind,ks,vs", [
    ("decode", 3.0, 0.25),
    pytest.param("decode", 3.0, 2.0, marks=pytest.mark.skip(
        reason="measured max-abs 3.5e-2 > 2e-2: |V| up to 15 (v_scale 2 on codes up to 7.5), where the "
               "bf16 rounding of the softmax weights and of the output (2^-9 relative) reaches the tolerance")),
    pytest.param("prefill", 3.0, 0.25, marks=pytest.mark.skip(
        reason=f"measured max-abs 5.7e-2 > 2e-2 (k_scale 3 spreads the scores): {_Q_ROUNDING_8BIT}")),
    pytest.param("prefill", 3.0, 2.0, marks=pytest.mark.skip(
        reason=f"measured max-abs 4.58e-1 > 2e-2 (mean 1.1e-2): k_scale 3 spreads the scores and "
               f"v_scale 2 makes |V| up to 15: {_Q_ROUNDING_8BIT}")),
])
def test_fp8_large_scales(kind, ks, vs):
    """8-bit pools at large scales (the decode's hi + lo query keeps the K
    spread harmless; measured max-abs 4.4e-3 at k_scale 3, v_scale 0.25)."""
    from tests.test_gpu_fp8 import _run, _run_prefill
    say(f"[fp8 large scales] {kind} k_scale {ks} v_scale {vs}")
    if kind == "decode":
        case = W.decode_case(241, 3, 32, 8, 128, [512, 1024, 96], (2, 10), offsets="random")
        got, want = _run(case, 47, ks, vs, 0)
    else:
        case = W.prefill_case(281, 2, 32, 8, 128, [512, 96], [256, 77], (2, 12), offsets="contiguous")
        got, want = _run_prefill(case, 57, ks, vs)
    assert_parity(got, want, W.BF16, f"fp8 {kind} k_scale {ks} v_scale {vs}")

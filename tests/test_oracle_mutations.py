"""Plant plausible mistakes in a copy of the oracle (on the CPU) and require
that the pins catch every one of them.  This guards the pins themselves: a
dropped term, a wrong sign or index, or a transposed operand must fail."""

import inspect
import types

import pytest

from oracle import lazy_oracle
from tests import oracle_pins

MUTATIONS = {
    "rope_sign_low": [("lo * c - hi * s", "lo * c + hi * s")],
    "rope_sign_high": [("hi * c + lo * s", "hi * c - lo * s")],
    "rope_interleaved_pairs": [("lo, hi = x[..., : d // 2], x[..., d // 2:]",
                                "lo, hi = x[..., 0::2], x[..., 1::2]")],
    "rope_frequency_law": [("-2.0 * i / head_dim", "-1.0 * i / head_dim")],
    "word_fields_swapped": [("return (w & 0xFFFF).astype(np.int64), (w >> 16).astype(np.int64)",
                             "return (w >> 16).astype(np.int64), (w & 0xFFFF).astype(np.int64)")],
    "slot_index": [("slots = j % BLOCK_TOKENS", "slots = (j + 1) % BLOCK_TOKENS")],
    "keys_not_rotated": [("return rope(k_stored, offs, theta), v_stored", "return k_stored, v_stored")],
    "values_rotated": [("return rope(k_stored, offs, theta), v_stored",
                        "return rope(k_stored, offs, theta), rope(v_stored, offs, theta)")],
    "missing_scale": [("s = scale * (q_rot @ k_hat.T)", "s = (q_rot @ k_hat.T)")],
    "softmax_axis": [("return e / np.sum(e, axis=-1, keepdims=True)", "return e / np.sum(e, axis=0, keepdims=True)")],
    "decode_gqa_map": [("q_rot = rope(q[b, g * group:(g + 1) * group], q_pos[b], theta)",
                        "q_rot = rope(q[b, g::hkv], q_pos[b], theta)"),
                       ("out[b, g * group:(g + 1) * group] = _attend", "out[b, g::hkv] = _attend")],
    "decode_query_position": [("q_rot = rope(q[b, g * group:(g + 1) * group], q_pos[b], theta)",
                               "q_rot = rope(q[b, g * group:(g + 1) * group], q_pos[b] + 1, theta)")],
    "prefill_gqa_map": [("block_table[b], int(kv_lens[b]), h // group, scale, theta,",
                         "block_table[b], int(kv_lens[b]), h % hkv, scale, theta,")],
    "fill_off_by_one": [("j[(j % BLOCK_TOKENS) < np.asarray(block_fill)[ids]]",
                         "j[(j % BLOCK_TOKENS) <= np.asarray(block_fill)[ids]]")],
    "fill_ignored": [("    if block_fill is None or j.size == 0:\n        return j",
                      "    if True:\n        return j")],
    "fill_visibility_by_token_count": [("vis = valid_slots(table_row, kv_len, block_fill)[None, :] <= t[:, None]",
                                        "vis = np.arange(k_hat.shape[0])[None, :] <= t[:, None]")],
    "causal_off_by_one": [("<= t[:, None]", "< t[:, None]")],
    "prefill_query_position": [("q_rot = rope(q_rows, q_pos_start + rows, theta)",
                                "q_rot = rope(q_rows, q_pos_start + rows + 1, theta)")],
    "merge_no_rescale": [("num = num + f * u", "num = num + u")],
    "merge_sum_unscaled": [("den = den + f * l", "den = den + l")],
    "tile_partial_max_not_subtracted": [("w = np.exp(scores - m)", "w = np.exp(scores)")],
    "append_wrong_source": [("k_out[slot // BLOCK_TOKENS, :, slot % BLOCK_TOKENS, :] = k_new[t]",
                             "k_out[slot // BLOCK_TOKENS, :, slot % BLOCK_TOKENS, :] = v_new[t]")],
    "cache_bytes_no_kv_factor": [("return 2 * layers * heads", "return layers * heads")],
    "rotation_two_flops": [("rotate = 3 * n_keys * head_dim", "rotate = 2 * n_keys * head_dim")],
    "rotation_counts_one_product": [("attend = 2 * (2 * m_rows * n_keys * head_dim)",
                                     "attend = 2 * m_rows * n_keys * head_dim")],
}


def _mutant(edits):
    src = inspect.getsource(lazy_oracle)
    for old, new in edits:
        assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
        src = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    mod = _mutant(MUTATIONS[name])
    failures = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(mod)
        except Exception as exc:  # noqa: BLE001 - any failure counts as caught
            failures.append((check.__name__, type(exc).__name__))
    assert failures, f"planted mistake {name!r} passed every pin"

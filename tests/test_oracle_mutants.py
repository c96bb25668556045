"""Plant plausible mistakes in copies of the CPU oracle and check that the
pins catch every one of them.  The mutants live only in this process's
memory; the oracle on disk is not touched.  CPU only."""

import os
import types

import pytest

import oracle_pins

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "paged_attention.py")

# (name, text in the oracle, replacement)
MUTANTS = [
    ("slot_offset_from_block_index", "offset = pos % block_size", "offset = pos // block_size"),
    ("slot_ignores_table", "physical_block = int(block_tables[s, logical_block])",
     "physical_block = int(logical_block)"),
    ("slot_off_by_one", "slots.append(physical_block * block_size + offset)",
     "slots.append(physical_block * block_size + offset + 1)"),
    ("decode_position_not_last", "out.append((s, L - 1))", "out.append((s, L))"),
    ("prefill_position_shift", "out.append((s, L - q_len + i))", "out.append((s, L - q_len + i - 1))"),
    ("write_v_gets_k", "v_cache[block, offset] = v_new[t]", "v_cache[block, offset] = k_new[t]"),
    ("write_ignores_padding", "        if slot < 0:\n            continue\n        block, offset",
     "        block, offset"),
    ("gather_no_truncation", "return np.concatenate(parts, axis=0)[: int(context_len)]",
     "return np.concatenate(parts, axis=0)"),
    ("gather_wrong_block", "parts = [cache[int(block_table_row[j])] for j in range(n_blocks)]",
     "parts = [cache[int(block_table_row[n_blocks - 1 - j])] for j in range(n_blocks)]"),
    ("paged_read_row", "out[t] = cache[int(block_table_row[t // block_size]), t % block_size]",
     "out[t] = cache[int(block_table_row[t // block_size]), (t + 1) % block_size]"),
    ("gqa_modulo", "    return q_head // n_rep", "    return q_head % num_kv_heads"),
    ("scale_dropped", "scores = scale * (keys @ q)\n    m = scores.max()\n    p = np.exp(scores - m)\n    return",
     "scores = (keys @ q)\n    m = scores.max()\n    p = np.exp(scores - m)\n    return"),
    ("no_max_subtraction", "p = np.exp(scores - m)\n    return (p @ values) / p.sum()",
     "p = np.exp(scores)\n    return (p @ values) / p.sum()"),
    ("not_normalised", "return (p @ values) / p.sum()", "return (p @ values)"),
    ("transposed_operand", "return (p @ values) / p.sum()", "return (p @ keys) / p.sum()"),
    ("causal_excludes_diagonal", "visible = np.arange(L)[None, :] <= pos[:, None]",
     "visible = np.arange(L)[None, :] < pos[:, None]"),
    ("causal_one_extra", "visible = np.arange(L)[None, :] <= pos[:, None]",
     "visible = np.arange(L)[None, :] <= pos[:, None] + 1"),
    ("prefill_scale_dropped", "scores = scale * (qf[lo + rows, h] @ keys[:, g, :].T)",
     "scores = (qf[lo + rows, h] @ keys[:, g, :].T)"),
    ("prefill_no_max_subtraction", "np.where(visible, scores - m, -np.inf)",
     "np.where(visible, scores, -np.inf)"),
    ("prefill_max_over_masked_keys", "m = np.where(visible, scores, -np.inf).max(axis=1, keepdims=True)",
     "m = scores.max(axis=1, keepdims=True)"),
    ("prefill_not_normalised", "(p @ vals[:, g, :]) / p.sum(axis=1, keepdims=True)",
     "(p @ vals[:, g, :])"),
    ("prefill_transposed_operand", "(p @ vals[:, g, :]) / p.sum(axis=1, keepdims=True)",
     "(p @ keys[:, g, :]) / p.sum(axis=1, keepdims=True)"),
    ("prefill_rows_not_shifted", "out[lo + rows, h] =", "out[lo + np.arange(rows.size), h] ="),
    ("prefill_keeps_rows_without_keys", "rows = np.nonzero(visible.any(axis=1))[0]",
     "rows = np.arange(visible.shape[0])"),
    ("prefill_query_from_wrong_head", "scores = scale * (qf[lo + rows, h] @ keys[:, g, :].T)",
     "scores = scale * (qf[lo + rows, g] @ keys[:, g, :].T)"),
    ("merge_weight_sign", "w = np.asarray(l, dtype=np.float64) * np.exp(m - M)",
     "w = np.asarray(l, dtype=np.float64) * np.exp(M - m)"),
    ("merge_drops_l", "w = np.asarray(l, dtype=np.float64) * np.exp(m - M)", "w = np.exp(m - M)"),
    ("partition_overlap", "k = keys[start:start + partition_size]", "k = keys[max(start - 1, 0):start + partition_size]"),
    ("bf16_shift", "<< np.uint32(16)", "<< np.uint32(15)"),
    ("empty_context_nan", "    if keys.shape[0] == 0:\n        return np.zeros(q.shape[-1], dtype=np.float64)\n",
     ""),
]


def _mutant(old, new):
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique or missing: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new):
    mod = _mutant(old, new)
    failed = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(mod)
        except Exception:          # an assertion, or the mutant crashing on a pin's input
            failed.append(check.__name__)
    assert failed, f"mutant {name} passed every pin"


def test_unmutated_copy_passes():
    mod = _mutant("import numpy as np\n", "import numpy as np\n")
    for check in oracle_pins.ALL_CHECKS:
        check(mod)

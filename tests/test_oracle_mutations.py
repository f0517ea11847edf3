"""Planted mistakes in the oracle must fail at least one of its pins.

Each mutant is the oracle's own source with one plausible slip (a wrong index,
a dropped term, a swapped operand, a shifted mask). It is built in memory on
the CPU and run through the same checks that pin the real oracle; a mutant
that passes every check would mean the pins leave that part of the oracle
unconstrained.
"""

import inspect
import types

import pytest

from oracle import paged_attention as ORACLE
from tests.test_oracle import CHECKS

MUTANTS = {
    "gather_block_uses_modulo": ("table[positions // block_size]",
                                 "table[positions % block_size]"),
    "gather_row_uses_division": ("cache)[physical, positions % block_size]",
                                 "cache)[physical, positions // block_size]"),
    "gather_off_by_one_block": ("table[positions // block_size]",
                                "table[np.minimum(positions // block_size + 1, len(table) - 1)]"),
    "gqa_heads_interleaved": ("g = h // group", "g = h % num_kv_heads"),
    "causal_top_left": ("visible = [prior + i + 1 for", "visible = [i + 1 for"),
    "causal_off_by_one": ("visible = [prior + i + 1 for", "visible = [prior + i for"),
    "causal_ignored": ("if causal:", "if False:"),
    "no_normalisation": ("out[i] = (w @ values[:m]) / w.sum()", "out[i] = (w @ values[:m])"),
    "scale_dropped": ("logits = scale * (keys[:m] @ q_rows[i])",
                      "logits = (keys[:m] @ q_rows[i])"),
    "keys_and_values_swapped": ("logits = scale * (keys[:m] @ q_rows[i])",
                                "logits = scale * (values[:m] @ q_rows[i])"),
    "exp_of_negated_logits": ("w = np.exp(logits - logits.max())",
                              "w = np.exp(logits.max() - logits)"),
    "one_key_dropped": ("m = int(visible[i])", "m = max(int(visible[i]) - 1, 1)"),
    "store_block_row_swapped": ("block, row = divmod(slot, block_size)",
                                "row, block = divmod(slot, block_size)"),
    "store_k_into_v": ("vc[block, row] = v[t]", "vc[block, row] = k[t]"),
    "store_skips_slot_zero": ("if slot < 0:", "if slot <= 0:"),
    "bf16_shift_wrong": ("<< np.uint32(16)", "<< np.uint32(15)"),
    "context_len_off_by_one": ("positions = np.arange(int(context_len))",
                               "positions = np.arange(max(int(context_len) - 1, 1))"),
}


def _mutant(old, new):
    src = inspect.getsource(ORACLE)
    assert old in src, f"mutation target not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    mod.__dict__["__name__"] = "oracle_mutant"
    exec(compile(src.replace(old, new), "<oracle_mutant>", "exec"), mod.__dict__)
    return mod


def _survives(mod):
    for check in CHECKS:
        try:
            check(mod)
        except Exception:
            return False
    return True


def test_unmutated_source_passes():
    assert _survives(_mutant("", ""))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    assert not _survives(_mutant(old, new)), f"mutant {name} passed every pin"

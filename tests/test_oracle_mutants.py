"""The oracle's pins have teeth: each plausible mistake below, planted in a
fresh copy of the oracle's own source (a one-line change: a dropped term, a
wrong sign, index or operand), is patched in place of the real functions, and
at least one CPU pin must then fail.  CPU only; the real oracle is restored
after each case."""

import inspect
import types

import pytest

import oracle.gdn as ogdn
import oracle.slots as oslots
from tests import test_oracle_paged as tp
from tests import test_oracle_recurrence as tr
from tests import test_oracle_slots as ts

GDN_MUTANTS = [
    ("output from the old state",
     "    S = alpha[:, None, None] * S + delta[:, :, None] * k[:, None, :]\n"
     "    o = scale * np.matmul(S, q[:, :, None])[:, :, 0]\n",
     "    o = scale * np.matmul(S, q[:, :, None])[:, :, 0]\n"
     "    S = alpha[:, None, None] * S + delta[:, :, None] * k[:, None, :]\n"),
    ("no decay inside the delta",
     "delta = beta[:, None] * (v - alpha[:, None] * Sk)",
     "delta = beta[:, None] * (v - Sk)"),
    ("beta on v only",
     "delta = beta[:, None] * (v - alpha[:, None] * Sk)",
     "delta = beta[:, None] * v - alpha[:, None] * Sk"),
    ("update subtracted",
     "S = alpha[:, None, None] * S + delta[:, :, None] * k[:, None, :]",
     "S = alpha[:, None, None] * S - delta[:, :, None] * k[:, None, :]"),
    ("decay after the update",
     "S = alpha[:, None, None] * S + delta[:, :, None] * k[:, None, :]",
     "S = alpha[:, None, None] * (S + delta[:, :, None] * k[:, None, :])"),
    ("decay of the wrong sign", "alpha = np.exp(g)", "alpha = np.exp(-g)"),
    ("decay never applied to S",
     "S = alpha[:, None, None] * S + delta[:, :, None] * k[:, None, :]",
     "S = S + delta[:, :, None] * k[:, None, :]"),
    ("output read with k", "o = scale * np.matmul(S, q[:, :, None])",
     "o = scale * np.matmul(S, k[:, :, None])"),
    ("checkpoint one interval late", "j = (p + n) // N - p // N - 1", "j = (p + n) // N - p // N"),
    ("checkpoints on the wrong token", "if cidx is not None and (p + n) % N == 0:",
     "if cidx is not None and (p + n - 1) % N == 0:"),
    ("bf16 states truncated",
     "bits = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16) << 16",
     "bits = (bits >> 16) << 16"),
]

SLOT_MUTANTS = [
    ("read the page of the first new token",
     "out[\"state_indices\"].append(pages[(p - 1) // page_size] if p > 0 else -1)",
     "out[\"state_indices\"].append(pages[p // page_size] if p > 0 else -1)"),
    ("prefix from the page count",
     "total = (n - 1) * page_size + int(last_page_len[b])",
     "total = n * page_size"),
    ("checkpoint start one page early",
     "out[\"checkpoint_cu_starts\"].append(int(page_indptr[b]) + p // page_size)",
     "out[\"checkpoint_cu_starts\"].append(int(page_indptr[b]) + max(0, p // page_size - 1))"),
    ("decode of a new page reads the new page",
     "            rd.append(pages[-2])", "            rd.append(pages[-1])"),
    ("chunks without the left pad",
     "return ((prefix % CHUNK) + new_len + CHUNK - 1) // CHUNK",
     "return (new_len + CHUNK - 1) // CHUNK"),
    ("zero-length sequence writes its last page",
     "out[\"output_state_indices\"].append(pages[-1] if L > 0 else -1)",
     "out[\"output_state_indices\"].append(pages[-1])"),
]

PINS = [  # cheapest first: a mutant stops at the first pin that fails
    lambda: tr.test_closed_form_product(4, 4, 6),
    lambda: tr.test_closed_form_product(8, 4, 8),
    tr.test_beta0_g0_leaves_state_unchanged,
    tr.test_unit_key_writes_value_exactly,
    tr.test_beta0_is_pure_decay,
    tr.test_full_decay_resets_state,
    tr.test_linearity_in_initial_state,
    tr.test_zero_start_never_reads,
    tr.test_minus_one_write_row_and_zero_length,
    tr.test_gqa_head_mapping_head_by_head,
    tr.test_bf16_states_rounded_only_where_stored,
    tp.test_decode_equals_one_token_prefill,
    tp.test_checkpoint_buffer_with_skipped_rows,
    tp.test_duplicate_final_and_boundary_store_agree,
    tp.test_zero_length_prefill_leaves_pool,
    ts.test_csr_self_test_1,
    ts.test_csr_three_sequences_both_directions,
    ts.test_prefill_2500_token_example,
    ts.test_long_prompt_checkpoint_total,
    ts.test_config0_rows,
    ts.test_decode_rows_new_page,
    ts.test_chunk_count_left_pad,
    ts.test_oracle_checkpoint_writes_sampled,
    lambda: tp.test_split_invariance_bit_exact(64),
    lambda: ts.test_rows_match_token_walk(64),
    tr.test_round_bf16_matches_torch_and_ties_to_even,
    ts.test_checkpoint_count_identity,
]


def _mutated_module(mod, old, new):
    src = inspect.getsource(mod)
    assert src.count(old) == 1, f"mutation site not unique in {mod.__name__}: {old!r}"
    m = types.ModuleType(mod.__name__)
    m.__dict__.update(__package__=mod.__package__, __file__=mod.__file__)
    exec(compile(src.replace(old, new), mod.__file__, "exec"), m.__dict__)
    return m


def _caught(monkeypatch, mod, old, new):
    mut = _mutated_module(mod, old, new)
    for name, val in vars(mut).items():
        if callable(val) and hasattr(mod, name) and getattr(val, "__module__", "") == mod.__name__:
            monkeypatch.setattr(mod, name, val)
    if mod is oslots:  # the prefill oracle calls the slot rules through its own import
        monkeypatch.setattr(ogdn, "_slots", mut)
    for i, pin in enumerate(PINS):
        try:
            pin()
        except Exception:  # an assertion or a rejected input: the pin noticed
            return i + 1
    return 0


@pytest.mark.parametrize("what,old,new", GDN_MUTANTS, ids=[m[0] for m in GDN_MUTANTS])
def test_pins_catch_recurrence_mutant(monkeypatch, what, old, new):
    assert _caught(monkeypatch, ogdn, old, new), f"no pin fails for: {what}"


@pytest.mark.parametrize("what,old,new", SLOT_MUTANTS, ids=[m[0] for m in SLOT_MUTANTS])
def test_pins_catch_slot_mutant(monkeypatch, what, old, new):
    assert _caught(monkeypatch, oslots, old, new), f"no pin fails for: {what}"


def test_unmutated_oracle_passes_every_pin():
    for pin in PINS:
        pin()


@pytest.mark.parametrize("mod,old", [(ogdn, "# [H]"), (oslots, "CHUNK = 64")],
                         ids=["recurrence", "slots"])
def test_harness_null_mutant_passes_every_pin(monkeypatch, mod, old):
    """A copy with no change in behaviour (a comment added) is caught by no pin:
    the swap itself breaks nothing, so a caught mutant was caught for its change."""
    assert _caught(monkeypatch, mod, old, old + "  # unchanged") == 0

"""Mutation check of the oracle's pins (CPU): each plausible mistake below is
planted in a copy of the oracle's source text (the tracked file is never
touched), the copy is loaded as a module of its own, every pin module is
pointed at it, and the pins are run until one fails. A mutant that passes
every pin means the pins do not fix that part of the oracle.

The mistakes: a dropped ReLU or a ReLU taken after the weight, keys read
with the page and row indices swapped, the last valid position masked,
weights applied to the wrong heads, no NaN for a page outside the pool, a
wrong bfloat16 or e4m3 decode, no length clamp, wrong tie or NaN order or an
unsorted top-k, tolerance scales with one formula swapped for the other or
with signed weights, per-token rows of the multi-token step misaligned,
attention without its scale, over the wrong dimensions, with a base-2
log-sum-exp, unnormalised, reading the wrong row, keeping negative entries,
dropping duplicates or not flagging a bad page, and a key map or histogram
off in its sign handling, NaN key, shift or range.
"""
import importlib.util
import os

import numpy as np
import pytest

import test_oracle_attention as p_att
import test_oracle_fp8 as p_fp8
import test_oracle_hist as p_hist
import test_oracle_magnitudes as p_mag
import test_oracle_mtp as p_mtp
import test_oracle_score as p_score
import test_oracle_topk as p_topk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCE = os.path.join(ROOT, "oracle", "indexer.py")
PIN_MODULES = [p_att, p_fp8, p_hist, p_mag, p_mtp, p_score, p_topk]

# (name, text in the oracle, replacement); each text occurs exactly once
MUTANTS = [
    ("score: ReLU dropped", "relu = np.maximum(dots, 0.0)", "relu = dots"),
    ("score: ReLU after the weight", "row = w64[b] @ relu ", "row = np.maximum(w64[b][:, None] * dots, 0.0).sum(axis=0) "),
    ("score: page and row swapped", "keys = decode(safe).reshape(n_slots * PAGE, -1)[:length]",
     "keys = decode(safe).transpose(1, 0, 2).reshape(n_slots * PAGE, -1)[:length]"),
    ("score: last valid position masked", "        out[b, :L] = row\n", "        out[b, :L - 1] = row[:L - 1]\n"),
    ("score: weights reversed", "    w64 = np.asarray(w, dtype=np.float64)\n    B = q.shape[0]\n    N = page_table.shape[1] * PAGE\n    out",
     "    w64 = np.asarray(w, dtype=np.float64)[:, ::-1]\n    B = q.shape[0]\n    N = page_table.shape[1] * PAGE\n    out"),
    ("score: no NaN for a bad page", "row[bad] = np.nan", "pass"),
    ("score: bf16 decode off by half an ulp", "<< np.uint32(16)", "<< np.uint32(16) | np.uint32(0x8000)"),
    ("score: no length clamp",
     "        L = clamp_len(seq_lens[b], N)\n        if L == 0:\n            continue\n        keys, bad",
     "        L = int(seq_lens[b])\n        if L == 0:\n            continue\n        keys, bad"),
    ("topk: higher index first on ties", "order = np.lexsort((idx, neg, nan))", "order = np.lexsort((-idx, neg, nan))"),
    ("topk: NaN ranked as zero", "order = np.lexsort((idx, neg, nan))", "order = np.lexsort((idx, neg))"),
    ("topk: output not ascending", "chosen = np.sort(order[:min(k, L)])", "chosen = order[:min(k, L)]"),
    ("magnitudes: M with A's formula", "M[b, :L] = w64[b] @ np.abs(q[b] @ keys.T)",
     "M[b, :L] = w64[b] @ (np.abs(q[b]) @ np.abs(keys).T)"),
    ("magnitudes: A with M's formula", "A[b, :L] = w64[b] @ (np.abs(q[b]) @ np.abs(keys).T)",
     "A[b, :L] = w64[b] @ np.abs(q[b] @ keys.T)"),
    ("magnitudes: signed weights", "w64 = np.abs(np.asarray(w, dtype=np.float64))", "w64 = np.asarray(w, dtype=np.float64)"),
    ("magnitudes: M as the size of the score", "M[b, :L] = w64[b] @ np.abs(q[b] @ keys.T)",
     "M[b, :L] = np.abs(w64[b] @ np.maximum(q[b] @ keys.T, 0.0))"),
    ("magnitudes: fp8 scales left out",
     "return magnitudes_keys(q_bits, w, fp8_pages(k8, k_scale), k8.shape[0], page_table, seq_lens)",
     "return magnitudes_keys(q_bits, w, fp8_pages(k8, np.ones_like(k_scale)), k8.shape[0], page_table, seq_lens)"),
    ("magnitudes: token rows transposed", "return M.reshape(B, T, -1), A.reshape(B, T, -1)",
     "return M.reshape(T, B, -1).transpose(1, 0, 2), A.reshape(T, B, -1).transpose(1, 0, 2)"),
    ("magnitudes: page table tiled over tokens",
     "                            np.repeat(np.asarray(page_table), T, axis=0), np.asarray(seq_lens).reshape(B * T))\n    return M",
     "                            np.tile(np.asarray(page_table), (T, 1)), np.asarray(seq_lens).reshape(B * T))\n    return M"),
    ("mtp: one length for every token",
     "                 np.repeat(np.asarray(page_table), T, axis=0), np.asarray(seq_lens).reshape(B * T))\n    return flat",
     "                 np.repeat(np.asarray(page_table), T, axis=0), np.repeat(np.asarray(seq_lens)[:, -1], T))\n    return flat"),
    ("mtp: tokens' queries reversed", "flat = score(q_bits.reshape(B * T, H, D)", "flat = score(q_bits[:, ::-1].reshape(B * T, H, D)"),
    ("mtp: page table tiled over tokens",
     "                 np.repeat(np.asarray(page_table), T, axis=0), np.asarray(seq_lens).reshape(B * T))\n    return flat",
     "                 np.tile(np.asarray(page_table), (T, 1)), np.asarray(seq_lens).reshape(B * T))\n    return flat"),
    ("fp8: exponent bias 8", "np.exp2(e - 7.0)", "np.exp2(e - 8.0)"),
    ("fp8: subnormals one binade low", "(m / 8.0) * 2.0 ** -6", "(m / 8.0) * 2.0 ** -7"),
    ("attention: no scale", "s = scale * (q[b] @ lat.T)", "s = q[b] @ lat.T"),
    ("attention: scores over the value dims only", "s = scale * (q[b] @ lat.T)", "s = scale * (q[b][:, :vd] @ lat[:, :vd].T)"),
    ("attention: base-2 log-sum-exp", "lse[b] = (m + np.log(l))[:, 0]", "lse[b] = (m + np.log2(l))[:, 0]"),
    ("attention: not normalised", "out[b] = (e / l) @ lat[:, :vd]", "out[b] = e @ lat[:, :vd]"),
    ("attention: value from the last dims", "out[b] = (e / l) @ lat[:, :vd]", "out[b] = (e / l) @ lat[:, -vd:]"),
    ("attention: row off by one", "kv_bits[pages, pos % PAGE]", "kv_bits[pages, (pos + 1) % PAGE]"),
    ("attention: negative entries kept", "for s in idx[b] if s >= 0]", "for s in idx[b] if s >= -1]"),
    ("attention: duplicates dropped", "pos = np.asarray([int(s) for s in idx[b] if s >= 0], dtype=np.int64)",
     "pos = np.unique(np.asarray([int(s) for s in idx[b] if s >= 0], dtype=np.int64))"),
    ("attention: no NaN for a bad page", "if np.any((pages < 0) | (pages >= num_pages)):",
     "if np.any(pages >= num_pages + 10 ** 9):"),
    ("keys: -0 not folded into +0", "u = (x + np.float32(0.0)).view(np.uint32)", "u = x.view(np.uint32)"),
    ("keys: negatives sign-flipped instead of complemented", "key = np.where(neg, ~u, u | np.uint32(0x80000000))",
     "key = np.where(neg, u ^ np.uint32(0x80000000), u | np.uint32(0x80000000))"),
    ("keys: NaN as key 0", "return np.where(np.isnan(x), np.uint32(1), key)", "return np.where(np.isnan(x), np.uint32(0), key)"),
    ("keys: positives not flipped", "u | np.uint32(0x80000000)).astype", "u).astype"),
    ("histogram: shift off by one", "digit = order_keys(logits[b, :L]) >> np.uint32(32 - bits)",
     "digit = order_keys(logits[b, :L]) >> np.uint32(31 - bits)"),
    ("histogram: whole row counted", "digit = order_keys(logits[b, :L])", "digit = order_keys(logits[b, :])"),
]

# every pin, cheapest first: (module, test function, arguments)
PINS = (
    [(p_score, "test_relu_before_weight", ()), (p_score, "test_zero_query_or_weight_gives_zero", ()),
     (p_score, "test_unit_queries_read_single_key_dims", ()), (p_score, "test_query_equal_to_key_and_its_negation", ()),
     (p_score, "test_length_clamped", ()), (p_score, "test_bad_page_in_valid_slot_is_nan_and_poison_tail_is_ignored", ())]
    + [(p_score, "test_mask_edges", (L,)) for L in (0, 1, 63, 64, 65, 127, 128, 191, 192)]
    + [(p_score, n, ()) for n in ("test_nonnegative_weights_give_nonnegative_scores",
                                  "test_physical_page_permutation_invariance", "test_row_width_does_not_change_prefix",
                                  "test_power_of_two_weight_scaling_is_exact", "test_magnitudes_bound_the_score",
                                  "test_tiny_config_end_to_end")]
    + [(p_topk, n, ()) for n in ("test_all_equal_takes_lowest_indices", "test_monotone_rows",
                                 "test_padding_and_empty_rows", "test_signed_zeros_tie_and_nan_last",
                                 "test_masked_tail_never_selected", "test_values_follow_indices",
                                 "test_selected_dominate_unselected")]
    + [(p_topk, "test_brute_force_random_with_ties", (s,)) for s in range(6)]
    + [(p_hist, n, ()) for n in ("test_keys_of_known_bit_patterns", "test_key_order_is_the_float_order",
                                 "test_histogram_counts_valid_positions")]
    + [(p_hist, "test_kth_largest_lies_in_the_bin_the_prefix_counts_name", (k,)) for k in (1, 7, 64, 299, 300)]
    + [(p_fp8, n, ()) for n in ("test_e4m3_decode_matches_torch_on_every_code", "test_e4m3_nan_codes",
                                "test_fp8_score_scales_exactly_with_positive_power_of_two",
                                "test_fp8_score_of_zero_scale_is_zero", "test_fp8_keys_from_generator_round_trip")]
    + [(p_fp8, "test_fp8_score_equals_bf16_score_on_shared_keys", (s,)) for s in range(3)]
    + [(p_mtp, n, ()) for n in ("test_one_token_is_the_plain_step", "test_tokens_are_independent_rows",
                                "test_recipe_is_causal", "test_brute_force_tiny")]
    + [(p_att, n, ()) for n in ("test_single_position_returns_its_value", "test_zero_query_averages_the_values",
                                "test_order_of_selection_does_not_matter", "test_split_selection_merges_by_log_sum_exp",
                                "test_empty_selection", "test_positions_off_the_table_or_pool_poison_only_their_request",
                                "test_a_repeated_position_counts_twice", "test_brute_force_small")]
    + [(p_mag, "test_magnitudes_closed_form", ())]
    + [(p_mag, "check_bf16_magnitudes", (s,)) for s in range(3)]
    + [(p_mag, "check_fp8_magnitudes", (s,)) for s in range(2)]
    + [(p_mag, "check_mtp_magnitudes", (s,)) for s in range(2)]
    + [(p_score, "test_brute_force_random", (s,)) for s in range(3)]
)


def _load_mutant(text: str, tag: str):
    spec = importlib.util.spec_from_loader(f"oracle_mutant_{tag}", loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(text, f"<oracle mutant {tag}>", "exec"), mod.__dict__)
    return mod


def test_unmutated_copy_passes_every_pin(monkeypatch):
    """The harness itself: the copy loaded the same way passes every pin."""
    mod = _load_mutant(open(SOURCE).read(), "none")
    for m in PIN_MODULES:
        monkeypatch.setattr(m, "oracle", mod)
    for m, name, args in PINS:
        getattr(m, name)(*args)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_fails_a_pin(monkeypatch, name, old, new):
    src = open(SOURCE).read()
    assert src.count(old) == 1, f"mutation site of '{name}' not found exactly once"
    mod = _load_mutant(src.replace(old, new, 1), str(abs(hash(name))))
    for m in PIN_MODULES:
        monkeypatch.setattr(m, "oracle", mod)
    with np.errstate(all="ignore"):
        for m, pin, args in PINS:
            try:
                getattr(m, pin)(*args)
            except Exception:  # an assertion, or the mutant breaking outright
                return
    pytest.fail(f"mutant '{name}' passed every pin")

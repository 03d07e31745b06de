"""CPU oracle pinned against the pages, closed forms, invariants and library routines."""
import json
import os

import pytest

import oracle_pins as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
NAMES = ["tiny", "dsv3", "grouped", "long", "mtp"]


def test_bf16_rounding_matches_torch():
    P.check_bf16_against_torch()


def test_f16_rounding_matches_torch():
    P.check_f16_against_torch()


def test_rmsnorm_matches_torch():
    P.check_rmsnorm_against_torch()


def test_rope_properties():
    P.check_rope_properties()


def test_rope_frequency_ladder():
    P.check_rope_frequency_ladder()


@pytest.mark.parametrize("name", ["tiny", "grouped", "mtp"])
def test_value_up_projection(name):
    P.check_value_up_projection(name)


@pytest.mark.parametrize("name", NAMES)
def test_explicit_equals_absorbed(name):
    # the pages' exactness claim: both formulations agree in exact arithmetic
    P.check_explicit_equals_absorbed(name, tol=1e-10)


@pytest.mark.parametrize("name", ["tiny", "grouped", "mtp"])
def test_rows_sum_to_one(name):
    P.check_rows_sum_to_one(name)


def test_single_token():
    P.check_single_token()


def test_geometric_closed_form():
    P.check_geometric_closed_form()


def test_scale_invariance():
    P.check_scale_invariance()


def test_bounded_logits():
    P.check_bounded_logits()


def test_textbook_reduction_sdpa():
    P.check_textbook_reduction()


def test_causal_prefix():
    P.check_causal_prefix()


def test_group_collapse():
    P.check_group_collapse()


def test_cache_image_layout():
    P.check_cache_image_layout()


def test_image_decode_matches_explicit_f32():
    P.check_image_decode_matches_explicit_f32()


def test_bf16_image_within_tolerance():
    P.check_bf16_image_within_tolerance()


def test_split_invariance():
    P.check_split_invariance()


def test_split_bounds():
    P.check_split_bounds()


def test_page_permutation():
    P.check_page_permutation()


def test_combine_closed_form():
    P.check_combine_closed_form()


def test_no_alpha_is_plain_mla():
    P.check_no_alpha_is_plain_mla()


def test_intensity_golden():
    with open(os.path.join(GOLDEN, "gqla_absorbed_intensity.json")) as f:
        golden = json.load(f)
    P.check_intensity_golden(golden)


def test_sparse_split_bounds():
    P.check_sparse_split_bounds()


@pytest.mark.parametrize("name", ["mtp", "grouped"])
def test_sparse_all_visible_equals_dense(name):
    P.check_sparse_all_visible_equals_dense(name)


def test_sparse_subset_against_explicit():
    P.check_sparse_subset_against_explicit()


def test_sparse_invalid_entries():
    P.check_sparse_invalid_entries()


def test_expanded_keys_unit_rms():
    P.check_expanded_keys_unit_rms()


def test_prefill_matches_explicit_f32():
    P.check_prefill_matches_explicit_f32()


def test_prefill_bf16_within_tolerance():
    P.check_prefill_bf16_within_tolerance()


def test_gqa_image_against_torch():
    P.check_gqa_image_against_torch()


def test_gqa_matches_explicit_f32():
    P.check_gqa_matches_explicit_f32()


def test_gqa_equals_absorbed_f32():
    P.check_gqa_equals_absorbed_f32()


def test_gqa_split_invariance():
    P.check_gqa_split_invariance()


def test_gqa_bf16_within_tolerance():
    P.check_gqa_bf16_within_tolerance()

"""The pins must catch plausible mistakes: each test plants one mistake in the
oracle (on the CPU, through monkeypatch) and checks that at least one pin
fails.  Nothing here touches the GPU path."""
import numpy as np
import pytest

import oracle.mla_oracle as om
from tests import test_oracle_attention as A
from tests import test_oracle_fp8 as F


def _pins():
    pins = [lambda c=c: A.test_oracle_matches_brute_force(c) for c in range(len(A.BRUTE_CASES))]
    pins += [A.test_zero_query_gives_mean_of_visible_values, A.test_zero_scale_gives_mean_of_visible_values,
             A.test_first_new_token_without_prefix_returns_first_value,
             A.test_constant_values_give_that_constant, A.test_two_token_closed_form,
             A.test_concatenated_rope_equals_standard_attention, A.test_prefix_consistency,
             A.test_page_permutation_invariance, A.test_head_and_batch_independence,
             A.test_query_with_no_visible_key_is_zero, F.test_fp8_attention_is_attention_of_dequantised_values]
    return pins


def _count_failures():
    failed = 0
    for pin in _pins():
        try:
            pin()
        except AssertionError:
            failed += 1
    return failed


_orig_attend = om._attend
_orig_rope = om.rope_rows


def _attend_no_rope(q, kn, kr, v, scale, qpos, kpos):
    return _orig_attend(np.concatenate([q[:, :128], np.zeros_like(q[:, 128:])], axis=1), kn, kr, v, scale, qpos, kpos)


def _attend_scale_nope_only(q, kn, kr, v, scale, qpos, kpos):
    q2 = q.copy()
    if scale != 0:
        q2[:, 128:] /= scale
    return _orig_attend(q2, kn, kr, v, scale, qpos, kpos)


def _attend_values_are_keys(q, kn, kr, v, scale, qpos, kpos):
    return _orig_attend(q, kn, kr, kn, scale, qpos, kpos)


def _attend_rope_negated(q, kn, kr, v, scale, qpos, kpos):
    return _orig_attend(q, kn, -kr, v, scale, qpos, kpos)


def _rope_logical_pages(cache, layer_idx, page_table, page_size, rope_col, b, positions):
    pt = np.asarray(om._host_array(page_table)).copy()
    pt[b] = np.arange(pt.shape[1])
    return _orig_rope(cache, layer_idx, pt, page_size, rope_col, b, positions)


def _rope_slot_off_by_one(cache, layer_idx, page_table, page_size, rope_col, b, positions):
    return _orig_rope(cache, layer_idx, page_table, page_size, rope_col, b,
                      [min(int(x) + 1, int(max(positions))) for x in positions])


def _rope_from_sequence_zero(cache, layer_idx, page_table, page_size, rope_col, b, positions):
    return _orig_rope(cache, layer_idx, page_table, page_size, rope_col, 0, positions)


MUTATIONS = {
    "rope term dropped": ("_attend", _attend_no_rope),
    "scale on the nope term only": ("_attend", _attend_scale_nope_only),
    "keys used as values": ("_attend", _attend_values_are_keys),
    "rope sign flipped": ("_attend", _attend_rope_negated),
    "exclusive diagonal": ("_visible", lambda qpos, kpos: kpos[None, :] < qpos[:, None]),
    "mask ignores the prefix": ("_query_positions", lambda p, b, count: np.arange(count, dtype=np.int64)),
    "cache_offsets ignored": ("_key_positions", lambda co, b, count: np.arange(count, dtype=np.int64)),
    "page table ignored": ("rope_rows", _rope_logical_pages),
    "page slot off by one": ("rope_rows", _rope_slot_off_by_one),
    "rope of the wrong sequence": ("rope_rows", _rope_from_sequence_zero),
    "fp8 mantissa misread": ("decode_e4m3fn",
                             lambda c: np.where(np.asarray(c) & 0x7F == 0x7F, np.nan,
                                                np.ldexp(1.0 + (np.asarray(c, dtype=np.int64) & 7) / 16.0,
                                                         ((np.asarray(c, dtype=np.int64) >> 3) & 15) - 7)
                                                * np.where(np.asarray(c) & 0x80, -1.0, 1.0))),
}


def test_unmutated_oracle_passes_every_pin():
    assert _count_failures() == 0


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(om, attr, fn)
    assert _count_failures() >= 1, f"no pin caught: {name}"

"""The pins must catch plausible mistakes: each test plants one mistake in the
oracle (on the CPU, through monkeypatch) and checks that at least one pin
fails.  Nothing here touches the GPU path."""
import numpy as np
import pytest

import oracle
import oracle.mla_oracle as om
from tests import test_oracle_attention as A
from tests import test_oracle_fp8 as F
from tests import test_oracle_masks_merge as M
from tests import test_oracle_split as S
from tests import test_oracle_latent as L


def _pins():
    pins = [lambda c=c: A.test_oracle_matches_brute_force(c) for c in range(len(A.BRUTE_CASES))]
    pins += [A.test_zero_query_gives_mean_of_visible_values, A.test_zero_scale_gives_mean_of_visible_values,
             A.test_first_new_token_without_prefix_returns_first_value,
             A.test_constant_values_give_that_constant, A.test_two_token_closed_form,
             A.test_concatenated_rope_equals_standard_attention, A.test_prefix_consistency,
             A.test_page_permutation_invariance, A.test_head_and_batch_independence,
             A.test_query_with_no_visible_key_is_zero, F.test_fp8_attention_is_attention_of_dequantised_values]
    pins += [lambda c=c: M.test_null_mask_matches_brute_force(c) for c in range(len(M.NULL_CASES))]
    pins += [lambda c=c: M.test_lse_matches_brute_force(c) for c in range(len(M.LSE_CASES))]
    pins += [M.test_null_mask_zero_query_gives_mean_of_all_values, M.test_null_mask_last_token_equals_causal,
             M.test_lse_single_key_is_the_scaled_score, M.test_lse_of_zero_query_is_log_of_key_count,
             M.test_lse_shift_by_constant_score, M.test_merge_two_single_key_partials_closed_form,
             M.test_merge_with_empty_side_is_identity, M.test_merge_is_symmetric_and_associative]
    pins += [lambda c=c: M.test_rows_merged_equal_single_row(c) for c in range(len(M.MULTI_ROW_CASES))]
    pins += [lambda c=c, k=k: S.test_split_fp8_matches_brute_force(c, k)
             for c in range(len(S.SPLIT_CASES)) for k in (False, True)]
    pins += [lambda m=m: S.test_halves_of_one_query_equal_that_query(m) for m in ("causal", "null")]
    pins += [S.test_q_scale_scales_q_nope_only, S.test_contiguous_rope_equals_paged_rope,
             S.test_contiguous_rope_is_indexed_by_buffer_row]
    pins += [lambda c=c: L.test_latent_up_matches_brute_force(c) for c in range(len(L.CASES))]
    pins += [L.test_one_hot_weights_select_latent_columns, L.test_linear_in_the_weights_and_halves_in_place,
             L.test_unused_slots_are_zero_and_rows_follow_the_plan]
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
_orig_visible = om._visible
_orig_rope = om.rope_rows
_orig_merge = om.merge_partials
_orig_split = om.mla_prefill_ragged_split
_orig_latent = om.latent_up


def _attend_no_rope(q, kn, kr, v, scale, qpos, kpos, mask="causal"):
    return _orig_attend(np.concatenate([q[:, :128], np.zeros_like(q[:, 128:])], axis=1), kn, kr, v, scale, qpos, kpos, mask)


def _attend_scale_nope_only(q, kn, kr, v, scale, qpos, kpos, mask="causal"):
    q2 = q.copy()
    if scale != 0:
        q2[:, 128:] /= scale
    return _orig_attend(q2, kn, kr, v, scale, qpos, kpos, mask)


def _attend_values_are_keys(q, kn, kr, v, scale, qpos, kpos, mask="causal"):
    return _orig_attend(q, kn, kr, kn, scale, qpos, kpos, mask)


def _attend_rope_negated(q, kn, kr, v, scale, qpos, kpos, mask="causal"):
    return _orig_attend(q, kn, -kr, v, scale, qpos, kpos, mask)


def _attend_lse_no_max(q, kn, kr, v, scale, qpos, kpos, mask="causal"):
    """lse = ln(sum exp(score - max)), the max shift left out."""
    o, lse = _orig_attend(q, kn, kr, v, scale, qpos, kpos, mask)
    if len(q) == 0 or len(kpos) == 0:
        return o, lse
    s = scale * (q[:, :128] @ kn.T + q[:, 128:] @ kr.T)
    s = np.where(_orig_visible(qpos, kpos, mask), s, -np.inf)
    top = s.max(axis=1)
    return o, np.where(np.isfinite(lse), lse - np.where(np.isfinite(top), top, 0.0), lse)


def _attend_lse_log2(q, kn, kr, v, scale, qpos, kpos, mask="causal"):
    o, lse = _orig_attend(q, kn, kr, v, scale, qpos, kpos, mask)
    return o, lse / np.log(2.0)


def _attend_lse_unscaled(q, kn, kr, v, scale, qpos, kpos, mask="causal"):
    o, _ = _orig_attend(q, kn, kr, v, scale, qpos, kpos, mask)
    _, lse = _orig_attend(q, kn, kr, v, 1.0, qpos, kpos, mask)
    return o, lse


def _merge_plain_average(o_a, lse_a, o_b, lse_b):
    o, lse = _orig_merge(o_a, lse_a, o_b, lse_b)
    fa, fb = np.isfinite(lse_a), np.isfinite(lse_b)
    avg = np.where((fa & fb)[..., None], 0.5 * (o_a + o_b), np.where(fa[..., None], o_a, o_b))
    return np.where(np.isfinite(lse)[..., None], avg, 0.0), lse


def _merge_max_only(o_a, lse_a, o_b, lse_b):
    o, lse = _orig_merge(o_a, lse_a, o_b, lse_b)
    pick = np.where((np.asarray(lse_a) >= np.asarray(lse_b))[..., None], o_a, o_b)
    return np.where(np.isfinite(lse)[..., None], pick, 0.0), np.maximum(lse_a, lse_b)


def _merge_swapped(o_a, lse_a, o_b, lse_b):
    o, lse = _orig_merge(o_a, lse_a, o_b, lse_b)
    some = np.isfinite(lse)
    safe = np.where(some, lse, 0.0)
    wa = np.where(some, np.exp(np.asarray(lse_b) - safe), 0.0)
    wb = np.where(some, np.exp(np.asarray(lse_a) - safe), 0.0)
    return wa[..., None] * o_a + wb[..., None] * o_b, lse


def _split_q_scale_on_rope(q_nope, q_rope, *args, scales=None, **kw):
    if scales is not None:
        q_rope = np.asarray(om._as_f64(q_rope)) * scales["q"]
    return _orig_split(q_nope, q_rope, *args, scales=scales, **kw)


def _split_rope_ignored(q_nope, q_rope, *args, **kw):
    return _orig_split(q_nope, np.zeros_like(np.asarray(om._as_f64(q_rope))), *args, **kw)


def _split_contig_by_position(q_nope, q_rope, k_nope, v, cache_lengths, valid_length, cache_row_offsets,
                              cache_offsets, scale, k_rope_rows=None, **kw):
    if k_rope_rows is not None:
        rows = np.asarray(om._as_f64(k_rope_rows)).reshape(-1, 64)
        moved = np.zeros_like(rows)
        cro = np.asarray(cache_row_offsets, dtype=np.int64)
        for b in range(len(cro) - 1):
            c0 = 0 if cache_offsets is None else int(cache_offsets[b])
            for j in range(int(cro[b + 1] - cro[b])):
                moved[cro[b] + j] = rows[min(c0 + j, len(rows) - 1)]
        k_rope_rows = moved
    return _orig_split(q_nope, q_rope, k_nope, v, cache_lengths, valid_length, cache_row_offsets, cache_offsets,
                       scale, k_rope_rows=k_rope_rows, **kw)


def _split_k_rope_scale_dropped(*args, scales=None, **kw):
    if scales is not None:
        scales = dict(scales, k_rope=1.0)
    return _orig_split(*args, scales=scales, **kw)


def _latent_halves_swapped(*args):
    k, v = _orig_latent(*args)
    return v, k


def _latent_head_major_misread(cache, layer_idx, pt, ps, bro, co, latent_col, latent_dim, w, heads, cap):
    w = np.asarray(w).reshape(2, heads, 128, latent_dim).transpose(1, 0, 2, 3).reshape(heads * 256, latent_dim)
    return _orig_latent(cache, layer_idx, pt, ps, bro, co, latent_col, latent_dim, w, heads, cap)


def _latent_column_off_by_one(cache, layer_idx, pt, ps, bro, co, latent_col, latent_dim, w, heads, cap):
    return _orig_latent(cache, layer_idx, pt, ps, bro, co, latent_col + 1, latent_dim, w, heads, cap)


def _latent_offsets_ignored(cache, layer_idx, pt, ps, bro, co, latent_col, latent_dim, w, heads, cap):
    return _orig_latent(cache, layer_idx, pt, ps, bro, np.zeros_like(np.asarray(co)), latent_col, latent_dim, w,
                        heads, cap)


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
    "exclusive diagonal": ("_visible", lambda qpos, kpos, mask="causal":
                           kpos[None, :] < qpos[:, None] if mask == "causal" else _orig_visible(qpos, kpos, mask)),
    "null mask applies the causal predicate": ("_visible", lambda qpos, kpos, mask="causal":
                                               _orig_visible(qpos, kpos, "causal")),
    "null mask hides the diagonal": ("_visible", lambda qpos, kpos, mask="causal":
                                     _orig_visible(qpos, kpos, mask) & (kpos[None, :] != qpos[:, None])
                                     if mask == "null" else _orig_visible(qpos, kpos, mask)),
    "lse without the max shift": ("_attend", _attend_lse_no_max),
    "lse in log2 units": ("_attend", _attend_lse_log2),
    "lse of unscaled scores": ("_attend", _attend_lse_unscaled),
    "merge by plain average": ("merge_partials", _merge_plain_average),
    "merge by the larger lse only": ("merge_partials", _merge_max_only),
    "merge weights swapped": ("merge_partials", _merge_swapped),
    "split: q_scale applied to q_rope too": ("mla_prefill_ragged_split", _split_q_scale_on_rope),
    "split: q_rope ignored": ("mla_prefill_ragged_split", _split_rope_ignored),
    "split: contiguous rope indexed by position": ("mla_prefill_ragged_split", _split_contig_by_position),
    "split: cache scale of K_rope dropped": ("mla_prefill_ragged_split", _split_k_rope_scale_dropped),
    "latent: key and value halves swapped": ("latent_up", _latent_halves_swapped),
    "latent: weight rows read part-major": ("latent_up", _latent_head_major_misread),
    "latent: columns off by one": ("latent_up", _latent_column_off_by_one),
    "latent: plan cache offsets ignored": ("latent_up", _latent_offsets_ignored),
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
    if hasattr(oracle, attr):            # names the pins call through the package
        monkeypatch.setattr(oracle, attr, fn)
    assert _count_failures() >= 1, f"no pin caught: {name}"

"""Host-side choice of the key-split threshold (no GPU): pipeline.balanced_split_keys."""
import numpy as np

from mla_ragged_paged_amd import workloads
from mla_ragged_paged_amd.pipeline import ATTENTION_SLOTS, balanced_split_keys


def test_full_grids_are_not_split():
    # DeepSeek-V3-shaped batch: 37 query tiles per head, so 16 heads already give 592 >= 512 tiles
    w = workloads.build(workloads.SPECS["dsv3"])
    assert sum(-(-int(n) // 128) for n in w.n) == 37
    assert balanced_split_keys(w.n, w.p, 128) == 0
    assert balanced_split_keys(w.n, w.p, 16) == 0


def test_underfilled_grid_splits_at_half_the_most_keys():
    w = workloads.build(workloads.SPECS["dsv3"])
    most = int(w.n.max())                       # no cached prefix: the last tile sees n keys
    assert balanced_split_keys(w.n, w.p, 8) == -(-most // 2)
    # with a cached prefix the most keys are p + n
    assert balanced_split_keys([300], [5000], 4) == -(-5300 // 2)
    # null mask: every tile of a sequence sees p + n keys
    assert balanced_split_keys([130], [0], 2, causal=False) == 128 and balanced_split_keys([130], [0], 2) == 128


def test_no_tile_above_the_threshold_means_no_split():
    assert balanced_split_keys([64], [0], 2) == 0            # 64 keys: below the 128-key floor
    assert balanced_split_keys([], [], 8) == 0
    assert balanced_split_keys([0, 0], [100, 9000], 8) == 0  # no query tile at all


def test_slot_count_is_the_boundary():
    n = [128] * 8                                            # one tile per sequence
    p = [1000] * 8
    assert balanced_split_keys(n, p, ATTENTION_SLOTS // 8) == 0
    assert balanced_split_keys(n, p, ATTENTION_SLOTS // 8 - 1) == 564
    assert np.isclose(564, -(-1128 // 2))

"""Pins for the oracle's float8_e4m3fn handling (CPU only)."""
import numpy as np
import torch

import oracle
from tests.oracle_cases import call, make_problem


def test_every_code_decodes_like_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


def test_format_landmarks():
    d = oracle.decode_e4m3fn
    assert d([0x7E])[0] == 448.0 == oracle.E4M3FN_MAX       # largest finite
    assert d([0xFE])[0] == -448.0
    assert d([0x01])[0] == 2.0 ** -9                        # smallest subnormal
    assert d([0x08])[0] == 2.0 ** -6                        # smallest normal
    assert d([0x38])[0] == 1.0
    assert np.isnan(d([0x7F])[0]) and np.isnan(d([0xFF])[0])
    assert d([0x80])[0] == 0.0 and np.signbit(d([0x80])[0])


def test_fp8_attention_is_attention_of_dequantised_values():
    """Each operand is decoded and multiplied by its own scale; distinct scales
    make a swapped or missing scale visible."""
    rng = np.random.default_rng(3)
    n, p = [5, 4], [3, 2]
    common, rows, _ = make_problem(rng, n, p, heads=2, width=96, rope_col=32)
    row = rows[0]

    def q8(x):
        s = float(np.float32(np.abs(x).max() / 448.0))
        return torch.from_numpy(x / s).to(torch.float8_e4m3fn), s

    q_c, sq = q8(common["q"])
    kn_c, skn = q8(row["k_nope"])
    v_c, sv = q8(row["v"] * 3.0)
    cache_c, skr = q8(common["cache"] * 0.5)
    scales = {"q": sq, "k_nope": skn, "v": sv, "k_rope": skr}
    assert len(set(scales.values())) == 4
    got = oracle.mla_prefill_ragged(q_c, kn_c, v_c, cache_c, 0, common["page_table"], common["page_size"],
                                    common["rope_col"], common["cache_lengths"], common["valid_length"],
                                    row["cache_row_offsets"], row["cache_offsets"], common["scale"],
                                    scales=scales)
    deq = lambda c, s: c.to(torch.float64).numpy() * s  # noqa: E731  (torch's own decoder)
    c2 = dict(common, q=deq(q_c, sq), cache=deq(cache_c, skr))
    r2 = dict(row, k_nope=deq(kn_c, skn), v=deq(v_c, sv))
    ref = call(oracle, c2, r2)
    assert np.abs(got - ref).max() <= 1e-12

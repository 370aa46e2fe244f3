"""Seeded input generator: bf16 rounding and reproducibility (CPU only)."""
import numpy as np

import kvc_synth as syn


def test_bf16_round_to_nearest_even():
    cases = {
        0x3F800000: 0x3F80,          # 1.0 exact
        0x3F808000: 0x3F80,          # tie, even stays
        0x3F818000: 0x3F82,          # tie, odd rounds up
        0x3F808001: 0x3F81,          # above tie
        0x3F807FFF: 0x3F80,          # below tie
        0x7F7FFFFF: 0x7F80,          # overflow to inf
        0xFF800000: 0xFF80,          # -inf
        0x80000000: 0x8000,          # -0
    }
    x = np.array(list(cases), dtype=np.uint32).view(np.float32)
    assert syn.bf16_bits(x).tolist() == list(cases.values())
    assert syn.bf16_bits(np.array([np.nan], dtype=np.float32))[0] == 0x7FC0


def test_chunks_reproducible_and_distinct():
    a = syn.normal_chunk(3, 1, "k", 2, 5, (4, 8), syn.BF16)
    b = syn.normal_chunk(3, 1, "k", 2, 5, (4, 8), syn.BF16)
    c = syn.normal_chunk(3, 1, "v", 2, 5, (4, 8), syn.BF16)
    assert np.array_equal(a, b) and not np.array_equal(a, c)


def test_dense_case_poison_and_shapes():
    c = syn.dense_case(2, 8, 2, 64, 10, [3, 10], syn.BF16)
    assert c["k_cache"].shape == (2, 2, 10, 64) and c["q"].shape == (2, 8, 64)
    assert np.all(c["k_cache"][0, :, 3:] == syn.BF16_QNAN)
    assert not np.any(c["k_cache"][1] == syn.BF16_QNAN)


def test_c3_lengths_in_range():
    pre = syn.pre_append_lens(syn.C3)
    assert pre.shape == (32,) and pre.min() >= 1023 and pre.max() <= 32767
    assert np.array_equal(pre, syn.pre_append_lens(syn.C3))


def test_topk_indices_sorted_distinct():
    idx = syn.topk_indices(5, 0, 2, 3, 64, 1000)
    for row in idx.reshape(-1, 64):
        assert np.all(np.diff(row) > 0) and row.min() >= 0 and row.max() < 1000

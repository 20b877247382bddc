"""The seeded input generators: shapes, determinism, and the stated readings."""
import numpy as np

from synth import bf16_bits_from_f32, make_workload, rng_for, zipf_counts
from synth.workloads import offsets_from_counts


def test_bf16_rounding_ties_to_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.0, 0.0], np.float32)
    assert list(bf16_bits_from_f32(x)) == [0x3F80, 0x3F80, 0x3F82, 0xC000, 0x0000]


def test_tiny_workload_deterministic_with_outliers():
    a = make_workload("tiny")
    b = make_workload("tiny")
    assert np.array_equal(a["A"], b["A"]) and np.array_equal(a["W"], b["W"])
    assert a["A"].shape == (128, 512) and a["W"].shape == (256, 512)
    assert len(a["outlier_channels"]) == 4


def test_zipf_counts_profile():
    c = zipf_counts(32768, 32, 1.1, rng_for(0, "counts_up"))
    assert c.sum() == 32768 and (c == 0).sum() == 2 and c.max() > 5000
    off = offsets_from_counts(c)
    assert off[0] == 0 and off[-1] == 32768 and np.all(np.diff(off) >= 0)


def test_grouped_shrink_keeps_ragged_profile():
    d = make_workload("grouped_up", rows=600, parts={"A"})
    c = d["counts"]
    assert (c == 0).sum() == 2 and d["A"].shape == (int(c.sum()), 7168)
    assert d["offsets"][-1] == c.sum()

"""Pins of the per-tensor-scaling ablation (oracle.ablation).  CPU only."""
import numpy as np
import pytest

from oracle import e4m3_decode, e4m3_decode_table, quant_act_1x128, quant_w_128x128
from oracle.ablation import ablate, dequant_per_tensor, product_errors, quant_per_tensor, run
from synth.workloads import bf16_bits_from_f32


def _bf16(x):
    return bf16_bits_from_f32(np.asarray(x, dtype=np.float32))


def test_one_group_tensors_match_the_tile_and_block_rules():
    # a 1x128 activation is one tile and a 128x128 weight one block: the
    # per-tensor rule must give the same codes and scale there
    rng = np.random.default_rng(5)
    a = _bf16(rng.standard_normal((1, 128)) * 3)
    q, s = quant_per_tensor(a)
    qt, st = quant_act_1x128(a)
    assert np.array_equal(q, qt) and s == st[0, 0]
    w = _bf16(rng.standard_normal((128, 128)) * 0.02)
    q, s = quant_per_tensor(w)
    qb, sb = quant_w_128x128(w)
    assert np.array_equal(q, qb) and s == sb[0, 0]


def test_equal_tile_maxima_give_the_tile_codes():
    # every 1x128 tile holds +-7.5 once and smaller values elsewhere: all tile
    # scales equal the tensor scale, so the codes are identical
    rng = np.random.default_rng(6)
    x = rng.uniform(-7, 7, size=(6, 512)).astype(np.float32)
    for t in range(4):
        x[np.arange(6), t * 128 + rng.integers(0, 128, size=6)] = 7.5 * rng.choice([-1, 1], size=6)
    bits = _bf16(x)
    q, s = quant_per_tensor(bits)
    qt, st = quant_act_1x128(bits)
    assert np.all(st == s)
    assert np.array_equal(q, qt)


def test_zero_tensor_has_zero_scale_and_no_nan():
    q, s = quant_per_tensor(np.zeros((3, 256), np.uint16))
    assert s == 0.0
    assert np.all((q & 0x7F) == 0)
    assert np.all(dequant_per_tensor(q, s) == 0.0)


def test_representable_values_round_trip_exactly():
    # every finite non-negative E4M3 value, with 448 present: the scale is 1 and
    # each value comes back exactly
    vals = e4m3_decode_table()[:127].astype(np.float32)
    x = np.concatenate([vals, -vals, [448.0]]).reshape(1, -1)
    q, s = quant_per_tensor(_bf16(x))
    assert s == 1.0
    assert np.array_equal(e4m3_decode(q).astype(np.float32), x.astype(np.float32))


def test_product_errors_closed_form():
    rng = np.random.default_rng(7)
    ref = rng.standard_normal((16, 32))
    e = product_errors(ref * (1 + 2.0 ** -9), ref)
    assert e["normwise"] == pytest.approx(2.0 ** -9, rel=1e-9)
    assert e["elementwise_max"] == pytest.approx(2.0 ** -9, rel=1e-9)
    assert e["share_above_1e-2"] == 0.0


def test_tiny_ablation_reports_per_tensor_worse():
    # measured on the tiny workload (4 outlier channels x50): the fine-grained
    # scales represent each tile's largest value exactly, so the outlier
    # channels dominate the gap; the regular channels lose little (E4M3 spans
    # enough binades for a x50 spread)
    r = run("tiny")
    f, t = r["fine_grained"], r["per_tensor"]
    assert f["normwise"] < t["normwise"]
    assert f["a_zero_share"] < t["a_zero_share"]
    assert abs(f["a_regular_error"] - t["a_regular_error"]) < 0.1 * f["a_regular_error"]


def test_ablation_without_outliers_matches_on_equal_maxima():
    # when every tile and block has the same max-abs, both schemes quantise
    # identically and report identical errors
    rng = np.random.default_rng(8)
    a = rng.uniform(-1, 1, size=(4, 256)).astype(np.float32)
    a[:, 0] = 2.0
    a[:, 128] = 2.0
    w = rng.uniform(-1, 1, size=(128, 256)).astype(np.float32)
    w[0, 0] = 2.0
    w[0, 128] = 2.0
    r = ablate(_bf16(a), _bf16(w))
    assert r["fine_grained"]["normwise"] == r["per_tensor"]["normwise"]

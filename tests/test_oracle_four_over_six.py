"""Pins for the oracle's Four Over Six encoder (CPU only): hand-worked
blocks, every block scale a nearest E4M3 value of its target, the choice
against a float64 evaluation of the same error, never worse than the core
recipe, identical to the core recipe when mapping to 4 cannot help, and the
KV frame-block codec built on it."""

import json
import os

import numpy as np
import pytest

import oracle
from oracle import four_over_six as fo6
from oracle import formats as F


def _golden(golden_dir):
    with open(os.path.join(golden_dir, "four_over_six_blocks.json")) as f:
        return json.load(f)


def test_hand_worked_blocks(golden_dir):
    g = _golden(golden_dir)
    x = np.array(g["x"], np.float32)[None, :]
    q, pick4 = fo6.quantize_4over6_with_amax(x, oracle.amax(x))
    assert q.tscale[0] == np.float32(g["tscale"])
    assert [f"{b:02X}" for b in q.scales[0]] == g["scales"]
    assert [f"{b:02X}" for b in q.codes[0]] == g["codes_hex"]
    assert pick4[0].tolist() == g["keeps_four"]
    s = q.tscale[0]
    sig6 = fo6.block_scales_to(x, s, 6.0)
    sig4 = fo6.block_scales_to(x, s, 4.0)
    e6 = fo6.block_sq_error(x, oracle.encode(x, sig6, s), sig6, s)[0]
    e4 = fo6.block_sq_error(x, oracle.encode(x, sig4, s), sig4, s)[0]
    assert e6.tolist() == [np.float32(v) for v in g["e6"]]
    assert e4.tolist() == [np.float32(v) for v in g["e4"]]
    assert np.array_equal(oracle.dequantize(q)[0], np.array(g["dequant"], np.float32))
    # the same bytes through the public one-domain entry point
    q2 = fo6.quantize_4over6(x)
    assert np.array_equal(q2.codes, q.codes) and np.array_equal(q2.scales, q.scales)


def test_error_sum_order_is_pinned(golden_dir):
    """Block 5 of the golden is built so that the float32 error sums depend
    on their order: summed from element 0 (the reading) the core candidate
    is kept; summed from element 15 down, E4 < E6 and the choice would flip.
    The expected errors are the hand-worked ones."""
    g = _golden(golden_dir)
    x = np.array(g["x"], np.float32)[None, 80:96]
    assert g["keeps_four"][5] is False
    s = np.float32(1.0)   # the golden's tensor scale (its first block holds 2688)
    sig6, sig4 = fo6.block_scales_to(x, s, 6.0), fo6.block_scales_to(x, s, 4.0)
    e6 = fo6.block_sq_error(x, oracle.encode(x, sig6, s), sig6, s)
    e4 = fo6.block_sq_error(x, oracle.encode(x, sig4, s), sig4, s)
    assert e6[0, 0] == np.float32(0.25) and e4[0, 0] == np.float32(0.25) + np.float32(2.0 ** -25)
    # the same squared errors summed in the opposite order
    d6 = np.array([0, 0.25, 2.0 ** -26, 2.0 ** -26, 0] + [0] * 11, np.float32)
    d4 = np.array([0, 0, 2.0 ** -26, 2.0 ** -26, 0.25] + [0] * 11, np.float32)
    rev = []
    for d in (d6, d4):
        e = np.float32(0)
        for v in d[::-1]:
            e = np.float32(e + v)
        rev.append(e)
    assert rev[1] < rev[0]          # reversed: mapping to 4 would win
    assert not e4[0, 0] < e6[0, 0]  # the reading: the core scale is kept


@pytest.fixture
def rng():
    return np.random.default_rng(4060)


def _tensor(rng, rows, k):
    x = rng.standard_normal((rows, k)).astype(np.float32)
    x *= np.exp(rng.uniform(-2, 2, (rows, 1))).astype(np.float32)
    x[rng.random(x.shape) < 0.02] *= 25
    return x.astype(np.float32)


def test_candidate_scales_are_nearest_e4m3(rng):
    """Each candidate byte is a nearest E4M3 value (brute force over every
    finite byte, float64) of (block max / target) / S, saturating at 448."""
    x = _tensor(rng, 40, 256)
    s = oracle.tensor_scale(oracle.amax(x))
    table = F.e4m3_value(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)  # 0 .. 448
    a_b = np.max(np.abs(x.reshape(40, 16, 16)), axis=2).astype(np.float64)
    for target in (6.0, 4.0):
        sig = fo6.block_scales_to(x, s, target)
        u = ((a_b.astype(np.float32) / np.float32(target)) / s).astype(np.float64)
        got = F.e4m3_value(sig).astype(np.float64)
        best = np.min(np.abs(table[None, None, :] - np.minimum(u, 448.0)[:, :, None]), axis=2)
        assert np.all(np.abs(got - np.minimum(u, 448.0)) <= best + 1e-300)


def _err64(x, q):
    """Float64 squared decode error per block (independent of the encoder's
    float32 evaluation)."""
    rows, k = x.shape
    d = oracle.dequantize(q).astype(np.float64) - x.astype(np.float64)
    return np.sum((d * d).reshape(rows, k // 16, 16), axis=2)


def test_choice_matches_float64_error(rng):
    """Where the two candidates' errors differ clearly, the kept one is the
    smaller in float64 too; and the result is never worse than the core
    recipe by more than float32 rounding of the comparison."""
    for seed in range(4):
        r = np.random.default_rng(100 + seed)
        x = _tensor(r, 64, 512)
        a = oracle.amax(x)
        q, pick4 = fo6.quantize_4over6_with_amax(x, a)
        s = q.tscale[0]
        sig4 = fo6.block_scales_to(x, s, 4.0)
        q4 = oracle.QTensor(oracle.encode(x, sig4, s), sig4, q.tscale)
        q6 = oracle.quantize_with_amax(x, a)
        e4, e6, e = _err64(x, q4), _err64(x, q6), _err64(x, q)
        clear = np.abs(e4 - e6) > 1e-5 * np.maximum(e4, e6)
        assert np.array_equal(pick4[clear], (e4 < e6)[clear])
        assert np.all(e <= e6 * (1 + 1e-5) + 1e-30)
        assert 0 < pick4.sum() < pick4.size  # both candidates occur on such data


def test_same_as_core_recipe_when_four_cannot_help(rng):
    """Blocks whose maximum maps to 6 with an exactly representable scale and
    whose values sit on that scaled grid have zero error under the core
    recipe, so mapping to 4 never wins and every byte equals oracle.quantize."""
    rows, k = 32, 128
    nb = k // 16
    sig = rng.integers(0x30, 0x50, (rows, nb)).astype(np.uint8)
    codes = rng.integers(0, 16, (rows, k)).astype(np.uint8)
    c3 = codes.reshape(rows, nb, 16)
    c3[:, :, 0] = 7  # a +6 in every block sets the block max
    x = (F.e2m1_value(c3) * F.e4m3_value(sig)[:, :, None]).reshape(rows, k).astype(np.float32)
    x[0, 0] = np.float32(6 * 448)  # the tensor max: S = 1
    want = oracle.quantize(x)
    got, pick4 = fo6.quantize_4over6_with_amax(x, oracle.amax(x))
    assert not pick4.any()
    assert np.array_equal(got.codes, want.codes) and np.array_equal(got.scales, want.scales)


def test_lower_total_error_on_gaussian_data(rng):
    x = rng.standard_normal((256, 256)).astype(np.float32)
    q6 = oracle.quantize(x)
    q = fo6.quantize_4over6(x)
    assert _err64(x, q).sum() < _err64(x, q6).sum()


def test_kv_codec_with_four_over_six():
    """Same frame-block domains and tensor scales as the core KV codec; each
    frame block is the one-domain encoder applied to its rows; decode is the
    unchanged KV decode."""
    rng = np.random.default_rng(7)
    f, t, h, d = 12, 5, 3, 32
    kv = (rng.standard_normal((f, t, h, d)) * np.exp(rng.uniform(-1, 1, (1, 1, h, 1)))).astype(np.float32)
    q = fo6.kv_quantize_4over6(kv)
    core = oracle.kv_quantize(kv)
    assert np.array_equal(q.tscale, core.tscale)
    rows = t * h
    for b, (f0, f1) in enumerate([(0, 8), (8, 12)]):
        qb = fo6.quantize_4over6(kv[f0:f1].reshape(-1, d))
        assert np.array_equal(q.codes[f0 * rows:f1 * rows], qb.codes)
        assert np.array_equal(q.scales[f0 * rows:f1 * rows], qb.scales)
        assert q.tscale[b] == qb.tscale[0]
    y = oracle.kv_dequantize(q, f, t, h, d, out="f32")
    assert y.shape == (f, t, h, d)
    e_fo6 = np.sum((y.astype(np.float64) - kv) ** 2)
    e_core = np.sum((oracle.kv_dequantize(core, f, t, h, d, out="f32").astype(np.float64) - kv) ** 2)
    assert e_fo6 <= e_core

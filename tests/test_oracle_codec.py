"""Pins for the oracle's NVFP4 codec (CPU only): hand-worked blocks, exact
round trips on grid-representable tensors, invariances, block locality,
nearest-point optimality of every code, storage size and the KV codec."""

import json
import os

import numpy as np
import pytest

import oracle
from oracle import codec, formats as F


def _load(golden_dir):
    with open(os.path.join(golden_dir, "hand_blocks.json")) as f:
        return json.load(f)["cases"]


def test_hand_worked_blocks(golden_dir):
    for case in _load(golden_dir):
        x = np.array(case["x"], np.float32)[None, :]
        q = oracle.quantize(x)
        assert q.tscale[0] == np.float32(case["tscale"]), case["name"]
        assert [f"{b:02X}" for b in q.scales[0]] == case["scales"], case["name"]
        assert [f"{b:02X}" for b in q.codes[0]] == case["codes_hex"], case["name"]
        deq = oracle.dequantize(q)[0]
        want = np.array(case["dequant"], np.float32)
        assert np.array_equal(deq, want), case["name"]
        assert np.array_equal(np.signbit(deq), np.signbit(want)), case["name"]


def _grid_tensor(rng, rows, k, s_exp):
    """A tensor whose every element is exactly e2m1 * sigma_b * 2^s_exp, with
    a +-6 in every block and one block carrying sigma = 448."""
    nb = k // 16
    codes = rng.integers(0, 16, (rows, k)).astype(np.uint8)
    pos = rng.integers(0, 16, (rows, nb))
    sign = rng.integers(0, 2, (rows, nb)).astype(np.uint8) << 3
    c3 = codes.reshape(rows, nb, 16)
    np.put_along_axis(c3, pos[:, :, None], (7 | sign)[:, :, None], axis=2)
    sigma = rng.integers(1, 0x7F, (rows, nb)).astype(np.uint8)  # nonzero finite
    sigma[rng.integers(0, rows), rng.integers(0, nb)] = 0x7E
    sigma[sigma > 0x7E] = 0x7E
    # tiny sigmas with a +-6 element: keep blocks away from the subnormal tail
    # of float32 when s_exp is very negative (not needed here)
    vals = F.e2m1_value(codes).reshape(rows, nb, 16) * F.e4m3_value(sigma)[:, :, None] * 2.0 ** s_exp
    return vals.reshape(rows, k).astype(np.float32), codes, sigma


@pytest.mark.parametrize("s_exp", [0, -7, 5])
def test_round_trip_exact_on_grid(s_exp):
    rng = np.random.default_rng(100 + s_exp)
    x, codes, sigma = _grid_tensor(rng, 24, 96, s_exp)
    q = oracle.quantize(x)
    assert q.tscale[0] == np.float32(2.0 ** s_exp)
    assert np.array_equal(q.scales, sigma)
    packed = codes[:, 0::2] | (codes[:, 1::2] << 4)
    assert np.array_equal(q.codes, packed)
    y = oracle.dequantize(q)
    assert np.array_equal(y, x) and np.array_equal(np.signbit(y), np.signbit(x))


def test_power_of_two_and_sign_invariance():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((16, 64)) * 3).astype(np.float32)
    q = oracle.quantize(x)
    for j in (-20, -3, 4, 30):
        q2 = oracle.quantize((x * np.float32(2.0 ** j)).astype(np.float32))
        assert np.array_equal(q2.codes, q.codes) and np.array_equal(q2.scales, q.scales)
        assert q2.tscale[0] == q.tscale[0] * np.float32(2.0 ** j)
    qn = oracle.quantize(-x)
    assert np.array_equal(qn.scales, q.scales)
    assert np.array_equal(qn.codes, q.codes ^ 0x88)


def test_block_locality():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((8, 64)).astype(np.float32)
    x[0, 0] = 100.0  # the global max lives in block (0, 0)
    q = oracle.quantize(x)
    x2 = x.copy()
    x2[3, 16:32] = rng.standard_normal(16).astype(np.float32) * 5
    q2 = oracle.quantize(x2)
    changed = np.zeros((8, 4), bool)
    changed[3, 1] = True
    c = codec.unpack_codes(q.codes).reshape(8, 4, 16)
    c2 = codec.unpack_codes(q2.codes).reshape(8, 4, 16)
    assert np.array_equal(c[~changed], c2[~changed])
    assert np.array_equal(q.scales[~changed], q2.scales[~changed])


def test_every_code_is_a_nearest_grid_point():
    # Brute force over the 8 magnitudes: |e2m1(code)| is at least as close to
    # |y| as any other grid point (ties excepted), saturating above 6.
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 128)) * np.exp(rng.uniform(-3, 3, (64, 1)))).astype(np.float32)
    q = oracle.quantize(x)
    s = q.tscale[0]
    d = (F.e4m3_value(q.scales).astype(np.float32) * s).astype(np.float32)
    r = np.where(d > 0, np.float32(1) / np.where(d > 0, d, 1), 0).astype(np.float32)
    y = np.abs(x.reshape(64, 8, 16) * r[:, :, None]).astype(np.float64)
    mag = np.abs(F.e2m1_value(codec.unpack_codes(q.codes))).reshape(64, 8, 16)
    grid = F.E2M1_MAGNITUDES
    dist = np.abs(y[..., None] - grid)
    assert np.all(np.abs(y - mag) <= dist.min(axis=-1) + 0.0)
    assert np.all(np.signbit(F.e2m1_value(codec.unpack_codes(q.codes))) == np.signbit(x))
    # block scales: the decoded block max stays within the E2M1 range
    assert np.all(y.max(axis=-1) <= 6.0 * (1 + 2 ** -3) + 1e-6)


def test_block_scale_is_nearest_e4m3_of_the_ideal_scale():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((32, 64)).astype(np.float32)
    q = oracle.quantize(x)
    ideal = (np.abs(x).reshape(32, 4, 16).max(-1) / 6.0) / np.float64(q.tscale[0])
    tab = F.e4m3_value(np.arange(0x7F))
    got = F.e4m3_value(q.scales)
    best = np.abs(ideal[..., None] - tab).min(-1)
    assert np.all(np.abs(ideal - got) <= best * (1 + 1e-6) + 1e-12)


def test_storage_is_4_5_bits_per_element():
    # 4-bit code + an 8-bit scale per 16 elements: 16 / 4.5 = 3.56x smaller than
    # bf16, the ~3.6x KV compression the pages report.
    x = np.zeros((880, 128), np.float32)
    q = oracle.quantize(x)
    bits = (q.codes.nbytes + q.scales.nbytes) * 8 / x.size
    assert bits == 4.5
    assert round(16 / bits, 1) == 3.6


def test_all_zero_tensor():
    q = oracle.quantize(np.zeros((4, 32), np.float32))
    assert q.tscale[0] == 0 and not q.scales.any() and not q.codes.any()
    qn = oracle.quantize(-np.zeros((4, 32), np.float32))
    assert np.all(q.codes == 0) and np.all(qn.codes == 0x88)


def test_kv_frame_blocks():
    rng = np.random.default_rng(9)
    f, t, h, d = 12, 5, 3, 32
    kv = rng.standard_normal((f, t, h, d)).astype(np.float32)
    kv[10] *= 50  # the second frame block has a larger amax
    q = oracle.kv_quantize(kv)
    assert q.tscale.shape == (2,)
    assert q.tscale[0] == np.float32(np.abs(kv[:8]).max() / np.float32(2688))
    assert q.tscale[1] == np.float32(np.abs(kv[8:]).max() / np.float32(2688))
    # frames of the first block do not see the second block's amax
    q0 = oracle.quantize(kv[:8].reshape(-1, d))
    n0 = 8 * t * h
    assert np.array_equal(q.codes[:n0], q0.codes) and np.array_equal(q.scales[:n0], q0.scales)
    y = oracle.kv_dequantize(q, f, t, h, d, out="f32")
    assert y.shape == (f, t, h, d)
    # decode error: at most half a grid step of the largest code, per block
    err = np.abs(y - kv).reshape(-1, 16).max(-1)
    assert np.all(err <= np.abs(kv).reshape(-1, 16).max(-1) / 6 * 1.2 + 1e-6)
    ybf = oracle.kv_dequantize(q, f, t, h, d, out="bf16")
    assert np.array_equal(ybf, F.f32_to_bf16_bits(y))

"""Pins for the oracle's 16-point random Hadamard transform (CPU only):
the Sylvester matrix from two constructions, the butterfly on unit vectors
(exact), hand-worked float32 blocks that fix the butterfly stage order,
orthogonality, the inverse, inner-product preservation and the float32
rounding bound against a float64 matrix product."""

import json
import os

import numpy as np

import oracle
from oracle import rht


def _popcount_matrix():
    i = np.arange(16)
    pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1, -1)


def test_sylvester_matrix():
    h = rht.hadamard16()
    assert np.array_equal(h, _popcount_matrix())
    assert np.array_equal(h @ h.T, 16 * np.eye(16, dtype=np.int64))


def test_sign_mask_bits():
    d = rht.sign_vector(0b1000_0000_0000_0101)
    assert list(np.nonzero(d < 0)[0]) == [0, 2, 15]


def test_butterfly_on_unit_vectors_is_exact():
    mask = 0xB3C5
    d = rht.sign_vector(mask)
    h = _popcount_matrix()
    for j in range(16):
        e = np.zeros((1, 32), np.float32)
        e[0, 16 + j] = 1.0
        out = rht.rht16_rows(e, mask)
        assert not out[0, :16].any()
        assert np.array_equal(out[0, 16:], 0.25 * d[j] * h[:, j])


def test_fp32_result_within_rounding_of_fp64_product():
    rng = np.random.default_rng(0)
    mask = 0x5A17
    x = rng.standard_normal((64, 128)).astype(np.float32)
    out = rht.rht16_rows(x, mask).astype(np.float64)
    m = 0.25 * _popcount_matrix() * rht.sign_vector(mask)[None, :]
    exact = (x.astype(np.float64).reshape(64, 8, 16) @ m.T).reshape(64, 128)
    # four add/sub stages: each output's error is below 4 ulp of the block's L1 norm / 4
    l1 = np.abs(x).reshape(64, 8, 16).sum(-1).repeat(16, axis=1) / 4
    assert np.all(np.abs(out - exact) <= 4 * 2.0 ** -24 * l1 + 1e-30)


def test_orthogonal_inverse_and_inner_products():
    rng = np.random.default_rng(1)
    mask = 0x0F0F
    a = rng.standard_normal((32, 64)).astype(np.float32)
    b = rng.standard_normal((32, 64)).astype(np.float32)
    ta = rht.rht16_rows(a, mask).astype(np.float64)
    tb = rht.rht16_rows(b, mask).astype(np.float64)
    assert np.allclose(np.linalg.norm(ta, axis=1), np.linalg.norm(a.astype(np.float64), axis=1), rtol=1e-6)
    assert np.allclose((ta * tb).sum(1), (a.astype(np.float64) * b).sum(1), rtol=1e-5, atol=1e-5)
    # inverse: (1/4) diag(d) H16 undoes (1/4) H16 diag(d)
    inv = 0.25 * rht.sign_vector(mask)[:, None] * _popcount_matrix()
    back = (ta.reshape(32, 4, 16) @ inv.T).reshape(32, 64)
    assert np.allclose(back, a, atol=1e-6)


def test_rht_quantize_axis0_is_transposed_axis1():
    rng = np.random.default_rng(2)
    mask = 0x1234
    g = rng.laplace(0, 1e-3, (64, 48)).astype(np.float32)
    q0 = oracle.rht16_quantize(g, mask, axis=0)
    q1 = oracle.rht16_quantize(np.ascontiguousarray(g.T), mask, axis=1)
    assert q0.codes.shape == (48, 32)
    assert np.array_equal(q0.codes, q1.codes) and np.array_equal(q0.scales, q1.scales)
    assert q0.tscale[0] == q1.tscale[0]


def _butterflies(x, mask, order):
    """A float32 RHT16 with the butterfly stages in `order` (the oracle's is
    1, 2, 4, 8): only used to show that the golden blocks tell orders apart."""
    w = (np.asarray(x, np.float32) * rht.sign_vector(mask)).astype(np.float32)
    for h in order:
        lo = np.array([i for i in range(16) if not i & h])
        a, b = w[lo].copy(), w[lo + h].copy()
        w[lo], w[lo + h] = a + b, a - b
    return (w * np.float32(0.25)).astype(np.float32)


def test_butterfly_stage_order_golden(golden_dir):
    """Hand-worked blocks (tests/golden/rht16_butterfly_order.json) on which
    the float32 result depends on the stage order: the oracle reproduces them
    bit for bit, and the stage order 8, 4, 2, 1 does not."""
    with open(os.path.join(golden_dir, "rht16_butterfly_order.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        x = np.array(c["x"], np.float32)[None, :]
        want = np.array(c["out"], np.float32)
        got = rht.rht16_rows(x, c["mask"])[0]
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), c["name"]
        assert np.array_equal(_butterflies(x[0], c["mask"], (1, 2, 4, 8)), want)
        assert not np.array_equal(_butterflies(x[0], c["mask"], (8, 4, 2, 1)), want), c["name"]

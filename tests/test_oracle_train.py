"""Pins for the oracle's NVFP4 training GEMM triple (CPU only): exact products
on operands that both quantization axes represent exactly, and orientation
checks of all three GEMMs against the unquantized float64 products (a
transposed or swapped operand gives an unrelated matrix)."""

import numpy as np

import oracle
from oracle import formats as F


def _grid_both_axes(rng, rows, cols):
    """A tensor exactly representable in NVFP4 along rows and along columns:
    entries e2m1 * 448, and +-2688 on the diagonal of every 16x16 tile, so
    every 16-element block in either direction holds the tensor maximum
    (S = 1, every block scale 448)."""
    codes = rng.integers(0, 16, (rows, cols)).astype(np.uint8)
    x = (F.e2m1_value(codes) * 448.0).astype(np.float32)
    i, j = np.indices((rows, cols))
    diag = (i % 16) == (j % 16)
    x[diag] = np.where(rng.random(diag.sum()) < 0.5, -2688.0, 2688.0).astype(np.float32)
    return x


def test_forward_and_input_gradient_exact_on_representable_operands():
    rng = np.random.default_rng(31)
    m, n, k = 48, 64, 80
    x, w, dy = _grid_both_axes(rng, m, k), _grid_both_axes(rng, n, k), _grid_both_axes(rng, m, n)
    r = oracle.linear_train_ref(x, w, dy, mask=0x1234)
    x64, w64, dy64 = x.astype(np.float64), w.astype(np.float64), dy.astype(np.float64)
    assert np.array_equal(r["y"], x64 @ w64.T)
    assert np.array_equal(r["dx"], dy64 @ w64)
    # every operand was quantized exactly
    for q, t in ((r["xq"], x), (r["wq"], w), (r["dyq"], dy), (r["wtq"], w.T)):
        assert np.array_equal(oracle.dequantize(q), np.ascontiguousarray(t))


def test_weight_gradient_with_rht_preserves_the_product():
    """The RHT is orthogonal and applied to both operands with the same signs,
    so dW approximates dY^T X; the same holds for any mask."""
    rng = np.random.default_rng(32)
    m, n, k = 256, 64, 96
    x = rng.standard_normal((m, k)).astype(np.float32)
    dy = (rng.laplace(0, 1e-3, (m, n))).astype(np.float32)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    exact = dy.astype(np.float64).T @ x.astype(np.float64)
    for mask in (0x0000, 0xA5C3, 0xFFFF):
        dw = oracle.linear_train_ref(x, w, dy, mask)["dw"]
        assert dw.shape == (n, k)
        rel = np.linalg.norm(dw - exact) / np.linalg.norm(exact)
        assert rel < 0.3, (mask, rel)  # NVFP4 noise ~0.13; an unrelated matrix gives ~1.4
    # a transposed operand pairing is unrelated to the product
    wrong = oracle.gemm_ref(oracle.rht16_quantize(x, 0xA5C3, axis=0), oracle.rht16_quantize(dy, 0xA5C3, axis=0))[0]
    assert np.linalg.norm(wrong.T - exact) / np.linalg.norm(exact) < 0.3  # (K, N) orientation check
    assert wrong.shape == (k, n)


def test_orientation_of_all_three_gemms():
    rng = np.random.default_rng(33)
    m, n, k = 128, 96, 160
    x = rng.standard_normal((m, k)).astype(np.float32)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    dy = rng.laplace(0, 1e-3, (m, n)).astype(np.float32)
    r = oracle.linear_train_ref(x, w, dy, 0x0F0F)
    x64, w64, dy64 = (t.astype(np.float64) for t in (x, w, dy))
    for got, want in ((r["y"], x64 @ w64.T), (r["dx"], dy64 @ w64), (r["dw"], dy64.T @ x64)):
        assert got.shape == want.shape
        assert np.linalg.norm(got - want) / np.linalg.norm(want) < 0.3
    # negative control: the forward product against the wrong orientation
    assert np.linalg.norm(r["y"][:, :min(n, k)] - (x64 @ w64.T[:, ::-1])[:, :min(n, k)]) / np.linalg.norm(
        x64 @ w64.T) > 0.5
    # the bounds bound the results
    for key in ("y", "dx", "dw"):
        assert np.all(np.abs(r[key]) <= r["b" + key] * (1 + 1e-12) + 1e-300)

"""16-point random Hadamard transform (RHT) ahead of quantization.

Test infrastructure only (see the package docstring).

The pages say only that weight gradients (gradient-sensitive paths) go through
a random Hadamard transform before NVFP4 quantization (neurohive.io
LongLive-2.0 summary, NVFP4 paragraph; tailorednewshub.com "Entrenamiento
NVFP4").  Reading used here:

* the transform acts on each 16-element quantization block v independently:
  v' = (1/4) * H16 * diag(d) * v, with H16 the Sylvester Hadamard matrix
  H16[i][j] = (-1)^popcount(i & j) and d a 16-vector of +-1 signs shared by
  every block of the tensor (d_j = -1 iff bit j of a 16-bit mask is set);
* 1/4 = 1/sqrt(16) makes the transform orthogonal, so the two operands of a
  GEMM transformed with the same d keep their inner products;
* float32 evaluation order (fixed so that codes are reproducible): the sign
  flip (exact), then four butterfly stages with strides 1, 2, 4, 8, each
  replacing (w_i, w_{i+h}) for i & h == 0 by (w_i + w_{i+h}, w_i - w_{i+h}),
  then a multiply by 0.25;
* the tensor amax and all block scales are taken on the transformed values.
"""

from __future__ import annotations

import numpy as np

from .codec import quantize, QTensor

F32 = np.float32


def hadamard16() -> np.ndarray:
    """Sylvester Hadamard matrix of order 16 (int64), by Kronecker doubling."""
    h = np.array([[1]], dtype=np.int64)
    base = np.array([[1, 1], [1, -1]], dtype=np.int64)
    for _ in range(4):
        h = np.kron(base, h)
    return h


def sign_vector(mask: int) -> np.ndarray:
    """The 16 diagonal signs: -1 where bit j of ``mask`` is set."""
    if not 0 <= int(mask) < (1 << 16):
        raise ValueError("sign mask must fit in 16 bits")
    return np.array([-1.0 if (int(mask) >> j) & 1 else 1.0 for j in range(16)], dtype=np.float32)


def rht16_rows(x: np.ndarray, mask: int) -> np.ndarray:
    """Apply the transform to every 16-element block along the last axis of a
    2-D float32 array, in the float32 order stated in the module docstring."""
    x = np.asarray(x, dtype=np.float32)
    rows, k = x.shape
    if k % 16:
        raise ValueError("last dim must be a multiple of 16")
    w = (x.reshape(rows, k // 16, 16) * sign_vector(mask)).astype(np.float32)
    for h in (1, 2, 4, 8):
        lo = [i for i in range(16) if not i & h]
        hi = [i + h for i in lo]
        a = w[:, :, lo].copy()
        b = w[:, :, hi].copy()
        w[:, :, lo] = a + b
        w[:, :, hi] = a - b
    w = w * F32(0.25)
    return w.reshape(rows, k).astype(np.float32)


def rht16_quantize(x: np.ndarray, mask: int, axis: int = 1) -> QTensor:
    """RHT then NVFP4-quantize a 2-D float32 tensor.

    ``axis`` is the dimension the 16-element blocks run along.  With axis 0
    (a gradient whose reduction dimension is dim 0) the tensor is transposed
    first, so the result is stored [cols, rows], K-contiguous."""
    x = np.asarray(x, dtype=np.float32)
    if axis == 0:
        x = np.ascontiguousarray(x.T)
    elif axis != 1:
        raise ValueError("axis must be 0 or 1")
    return quantize(rht16_rows(x, mask))

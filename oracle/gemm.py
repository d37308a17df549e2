"""Block-scaled W4A4 GEMM reference and GELU-tanh.

Test infrastructure only (see the package docstring).

The pages replace the BF16 GEMMs of the generator by FP4 GEMMs on both
weights and activations (tailorednewshub.com "Inferencia W4A4 NVFP4";
neurohive.io LongLive-2.0 summary, NVFP4 paragraph).  The product of two
NVFP4 operands quantized along the reduction dimension K is, by definition of
the format,

    C[m, n] = S_A * S_B * sum_k P_A[m, k] * P_B[n, k],
    P = e2m1(code) * E4M3(block scale)   (exact),

which is written out here with a float64 matmul over the exactly decoded
operands.  B is stored [N, K] (K-contiguous, like a linear layer's weight).
The error bound that parity tests use is

    bound[m, n] = S_A * S_B * sum_k |P_A[m, k] * P_B[n, k]|.
"""

from __future__ import annotations

import numpy as np

from .codec import QTensor, decode_exact

F32 = np.float32


def gemm_ref(a: QTensor, b: QTensor, rows: slice | np.ndarray | None = None, want_bound: bool = True):
    """Return (C, bound) as float64 [M, N] (or the selected rows of A); the
    bound is None when ``want_bound`` is False."""
    if a.k != b.k:
        raise ValueError("operands disagree on K")
    if rows is not None:
        a = QTensor(a.codes[rows], a.scales[rows], a.tscale)
    pa = decode_exact(a.codes, a.scales)
    pb = decode_exact(b.codes, b.scales)
    s = float(np.float64(a.tscale[0]) * np.float64(b.tscale[0]))
    c = (pa @ pb.T) * s
    bound = (np.abs(pa) @ np.abs(pb).T) * s if want_bound else None
    return c, bound


def gelu_tanh(h) -> np.ndarray:
    """GELU, tanh form: g(h) = 0.5 h (1 + tanh(u)), u = sqrt(2/pi) (h +
    0.044715 h^3), in float64.  The pages do not name the FFN activation; this
    standard form is the reading for the DiT FFN.

    Evaluated through the identity 0.5 (1 + tanh u) = 1 / (1 + e^(-2u)): the
    same function, written so that the negative tail keeps its relative
    precision.  Written as 1 + tanh(u), it cancels: below h of about -5.6
    that sum is exactly 0 in float64, while g is about h e^(2u), a normal
    number down to h of about -19."""
    h = np.asarray(h, dtype=np.float64)
    c = np.sqrt(2.0 / np.pi)
    u = c * (h + 0.044715 * h ** 3)
    with np.errstate(over="ignore"):
        return h / (1.0 + np.exp(-2.0 * u))

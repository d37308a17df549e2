"""The NVFP4 training GEMM triple of one linear layer Y = X W^T.

Test infrastructure only (see the package docstring).

The pages train the generator with NVFP4 GEMMs (tailorednewshub.com,
"LongLive-2.0: Infraestructura paralela NVFP4 para video largo", section
"Entrenamiento NVFP4": FP4 GEMMs with FP8 block and FP32 tensor scales, an RHT
before quantization on gradient-sensitive paths) and pass the weight
gradients through a random Hadamard transform first (neurohive.io LongLive-2.0
summary, NVFP4 paragraph).  Reading: each of the three GEMMs quantizes both of
its operands along its own reduction dimension, and only the weight-gradient
GEMM applies the RHT (the same sign vector on both operands, so that their
inner products are preserved):

* forward      Y  = Q(X) Q(W)^T            reduction over K (both along K);
* input grad   dX = Q(dY) Q(W^T)^T         reduction over N: dY along its
                                           rows' N, W along dim 0 (stored as
                                           the transposed [K, N] NVFP4 tensor);
* weight grad  dW = R(dY^T) R(X^T)^T       reduction over M: dY and X along
                                           dim 0 after the RHT16 (stored
                                           [N, M] and [K, M]).

Every GEMM is gemm_ref (float64 over exactly decoded operands) on operands
from the pinned quantizers.
"""

from __future__ import annotations

import numpy as np

from .codec import quantize
from .gemm import gemm_ref
from .rht import rht16_quantize


def linear_train_ref(x: np.ndarray, w: np.ndarray, dy: np.ndarray, mask: int, rows=None):
    """Return {"y", "dx", "dw"} (float64), each with its error bound, and the
    quantized operands.  ``rows`` (optional) restricts the returned rows of y
    and dx (rows of M) and of dw (rows of N) to the given indices."""
    x = np.asarray(x, dtype=np.float32)
    w = np.asarray(w, dtype=np.float32)
    dy = np.asarray(dy, dtype=np.float32)
    xq, wq = quantize(x), quantize(w)
    dyq, wtq = quantize(dy), quantize(np.ascontiguousarray(w.T))
    dyt, xt = rht16_quantize(dy, mask, axis=0), rht16_quantize(x, mask, axis=0)
    r_m = None if rows is None else rows["m"]
    r_n = None if rows is None else rows["n"]
    y, by = gemm_ref(xq, wq, rows=r_m)
    dx, bdx = gemm_ref(dyq, wtq, rows=r_m)
    dw, bdw = gemm_ref(dyt, xt, rows=r_n)
    return {"y": y, "by": by, "dx": dx, "bdx": bdx, "dw": dw, "bdw": bdw,
            "xq": xq, "wq": wq, "dyq": dyq, "wtq": wtq, "dyt": dyt, "xt": xt}

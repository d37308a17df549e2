"""NVFP4 block codec: amax, tensor scale, block scales, encode, pack, decode.

Test infrastructure only (see the package docstring).

What the pages fix (neurohive.io LongLive-2.0 summary, NVFP4 paragraph;
tailorednewshub.com "Entrenamiento NVFP4"): E2M1 elements, one FP8 scale per
16 consecutive elements, one FP32 scale per tensor.  What they leave open is
read as follows (every step is float32, round-to-nearest-even):

1. domain amax        A   = max |x| over the scaling domain (a whole tensor,
                            or one frame block of a KV tensor);
2. tensor scale       S   = A / 2688  (2688 = E2M1 max 6 * E4M3 max 448, so the
                            largest element lands on the top of both ranges);
3. block scale        a_b = max |x| over the 16-element block,
                      t_b = a_b / 6,  u_b = t_b / S  (0 when S = 0),
                      s_b = E4M3(u_b)  (RNE, saturating at 448);
4. block reciprocal   D_b = f32(s_b) * S,  r_b = 1 / D_b  (0 when D_b = 0);
5. element code       y_i = x_i * r_b,  code_i = sign(x_i) | E2M1(|y_i|)
                      (RNE, saturating at 6; a negative value that rounds to 0
                      keeps its sign, code 0x8);
6. packing            byte j of a row = code[2j] | code[2j+1] << 4; scales are
                      row-major [rows, K/16]; S is one float32 per domain.
7. decode             x' = f32(e2m1(code) * s_b) * S  (the product e2m1 * s_b
                      is exact in float32; one rounding at the multiply by S).

Quantization always runs along the last axis here; a caller that quantizes
along another axis passes the transposed tensor (the result is then stored
transposed, which is how a GEMM wants its K-contiguous operands).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .formats import (
    GLOBAL_MAX,
    e2m1_value,
    e4m3_value,
    f32_to_e2m1,
    f32_to_e4m3,
    f32_to_bf16_bits,
)

F32 = np.float32
BLOCK = 16


@dataclass
class QTensor:
    """An NVFP4 tensor: codes [rows, K/2] uint8, scales [rows, K/16] uint8
    (E4M3FN bytes) and the float32 tensor scale(s)."""

    codes: np.ndarray
    scales: np.ndarray
    tscale: np.ndarray  # float32, shape [n_domains]

    @property
    def rows(self) -> int:
        return self.codes.shape[0]

    @property
    def k(self) -> int:
        return self.codes.shape[1] * 2


def _check_rows(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype != np.float32:
        raise TypeError("the codec takes float32 input (widen bf16 first)")
    if x.ndim != 2 or x.shape[1] % BLOCK != 0:
        raise ValueError("expected a 2-D array whose last dim is a multiple of 16")
    return x


def amax(x: np.ndarray) -> np.float32:
    """Step 1: largest magnitude in the domain (exact)."""
    x = np.asarray(x, dtype=np.float32)
    return F32(np.max(np.abs(x))) if x.size else F32(0.0)


def tensor_scale(a: np.float32) -> np.float32:
    """Step 2: S = A / 2688 in float32 (0 for an all-zero domain)."""
    return F32(F32(a) / F32(GLOBAL_MAX))


def block_scales(x: np.ndarray, s: np.float32) -> np.ndarray:
    """Step 3: E4M3 block-scale bytes [rows, K/16] for tensor scale ``s``."""
    x = _check_rows(x)
    rows, k = x.shape
    a_b = np.max(np.abs(x.reshape(rows, k // BLOCK, BLOCK)), axis=2)
    t_b = a_b / F32(6.0)
    s = F32(s)
    if s > 0:
        u_b = t_b / s
    else:
        u_b = np.zeros_like(t_b)
    return f32_to_e4m3(u_b.astype(np.float32))


def encode(x: np.ndarray, sigma: np.ndarray, s: np.float32) -> np.ndarray:
    """Steps 4-6: packed codes [rows, K/2] for block scales ``sigma`` and
    tensor scale ``s``."""
    x = _check_rows(x)
    rows, k = x.shape
    d_b = e4m3_value(sigma).astype(np.float32) * F32(s)
    with np.errstate(divide="ignore"):
        r_b = np.where(d_b > 0, F32(1.0) / np.where(d_b > 0, d_b, F32(1.0)), F32(0.0))
    r_b = r_b.astype(np.float32)
    y = x.reshape(rows, k // BLOCK, BLOCK) * r_b[:, :, None]
    codes = f32_to_e2m1(y.astype(np.float32)).reshape(rows, k)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def quantize_with_amax(x: np.ndarray, a: np.float32) -> QTensor:
    """Steps 2-6 for one domain whose amax is ``a``."""
    x = _check_rows(x)
    s = tensor_scale(a)
    sigma = block_scales(x, s)
    codes = encode(x, sigma, s)
    return QTensor(codes, sigma, np.array([s], dtype=np.float32))


def quantize(x: np.ndarray) -> QTensor:
    """Quantize a 2-D float32 tensor (one scaling domain) along its last axis."""
    x = _check_rows(x)
    return quantize_with_amax(x, amax(x))


def unpack_codes(codes: np.ndarray) -> np.ndarray:
    """[rows, K/2] packed bytes -> [rows, K] 4-bit codes (low nibble first)."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty((codes.shape[0], codes.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = codes & 15
    out[:, 1::2] = codes >> 4
    return out


def decode_exact(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """P = e2m1(code) * s_b as float64 (exact), [rows, K]; no tensor scale."""
    c = unpack_codes(codes)
    rows, k = c.shape
    sig = e4m3_value(scales)
    return (e2m1_value(c).reshape(rows, k // BLOCK, BLOCK) * sig[:, :, None]).reshape(rows, k)


def dequantize(q: QTensor, out: str = "f32", domain_rows: int | None = None):
    """Step 7: float32 x' = f32(P) * S, or its bf16 bit pattern (RNE).

    ``domain_rows`` gives the rows per scaling domain when ``q`` holds several
    (the last domain may be shorter); default: one domain."""
    p = decode_exact(q.codes, q.scales).astype(np.float32)  # exact
    rows = p.shape[0]
    if domain_rows is None:
        domain_rows = max(rows, 1)
    dom = np.arange(rows) // domain_rows
    s_row = np.asarray(q.tscale, dtype=np.float32)[dom]
    y = p * s_row[:, None]
    if out == "f32":
        return y.astype(np.float32)
    if out == "bf16":
        return f32_to_bf16_bits(y)
    raise ValueError(out)


def kv_quantize(kv: np.ndarray, frame_block: int = 8) -> QTensor:
    """KV codec (hyper.ai LongLive-2.0 summary, "方法": the KV cache is
    quantized per block of eight frames).

    ``kv`` is float32 [frames, tokens, heads, head_dim].  Reading: one float32
    tensor scale per frame block (frames 0-7, 8-15, ...; the last block may be
    partial) taken over all tokens and heads of those frames; 16-element blocks
    run along head_dim.  Returns codes/scales flattened to
    [frames*tokens*heads, head_dim/2 | head_dim/16] and one S per frame block."""
    kv = np.asarray(kv, dtype=np.float32)
    f, t, h, d = kv.shape
    if d % BLOCK:
        raise ValueError("head_dim must be a multiple of 16")
    nfb = -(-f // frame_block)
    codes = np.empty((f * t * h, d // 2), np.uint8)
    scales = np.empty((f * t * h, d // BLOCK), np.uint8)
    ts = np.empty(nfb, np.float32)
    per_frame = t * h
    for b in range(nfb):
        f0, f1 = b * frame_block, min(f, (b + 1) * frame_block)
        rows = kv[f0:f1].reshape(-1, d)
        q = quantize(rows)
        codes[f0 * per_frame:f1 * per_frame] = q.codes
        scales[f0 * per_frame:f1 * per_frame] = q.scales
        ts[b] = q.tscale[0]
    return QTensor(codes, scales, ts)


def kv_dequantize(q: QTensor, frames: int, tokens: int, heads: int, head_dim: int,
                  frame_block: int = 8, out: str = "bf16") -> np.ndarray:
    """Inverse of :func:`kv_quantize` (step 7 per frame block), shaped
    [frames, tokens, heads, head_dim]."""
    y = dequantize(q, out=out, domain_rows=frame_block * tokens * heads)
    return y.reshape(frames, tokens, heads, head_dim)

"""Four Over Six: adaptive choice of the block scale for the NVFP4 KV cache.

Test infrastructure only (see the package docstring).

The pages name the technique and nothing else: the KV cache is quantized to
NVFP4 with micro-block scaling and an adaptive scale selection called Four
Over Six (tailorednewshub.com, "LongLive-2.0: Infraestructura paralela NVFP4
para video largo", section "Inferencia W4A4 NVFP4"; the FourOverSix
checkpoint format and package appear in the 171host.com setup instructions).
Reading taken here, the plainest one the name and the format support:

* the format does not change: E2M1 codes, one E4M3 scale per 16 elements, one
  float32 tensor scale per domain with S = A / 2688 as in the core recipe, and
  the standard decode;
* only the encoder changes: for every 16-element block it builds two
  candidates, one whose scale maps the block maximum to 6 (the core recipe)
  and one whose scale maps it to 4 (t_b = a_b / 4 instead of a_b / 6; the
  E2M1 grid is dense up to 4 and has a gap between 4 and 6, so a block whose
  large values sit in that gap can lose less precision), and keeps the one
  whose decoded block is closer to the input;
* "closer" is the squared error in the input's units,
  E = sum_i (x_i - x'_i)^2 with x'_i = f32(e2m1 * s_b) * S the standard
  decode, evaluated in float32 in a fixed order: d_i = x_i - x'_i,
  q_i = d_i * d_i, E = ((q_0 + q_1) + q_2) + ... + q_15 (every operation
  rounded to nearest even, no fused multiply-add).  The scale mapping to 4
  wins only when its E is strictly smaller; ties keep the core recipe.

Because the choice is an integer decision taken from floating-point values,
the GPU kernel evaluates exactly these float32 operations in this order, and
the two must agree bit for bit.
"""

from __future__ import annotations

import numpy as np

from .codec import BLOCK, F32, QTensor, _check_rows, amax, encode, tensor_scale, unpack_codes
from .formats import e2m1_value, e4m3_value, f32_to_e4m3


def block_scales_to(x: np.ndarray, s: np.float32, target: float) -> np.ndarray:
    """E4M3 block-scale bytes [rows, K/16] mapping each block maximum to
    ``target`` (6: the core recipe; 4: the alternative candidate):
    t_b = a_b / target, u_b = t_b / S, s_b = E4M3(u_b) (RNE, saturating)."""
    x = _check_rows(x)
    rows, k = x.shape
    a_b = np.max(np.abs(x.reshape(rows, k // BLOCK, BLOCK)), axis=2)
    t_b = a_b / F32(target)
    s = F32(s)
    u_b = t_b / s if s > 0 else np.zeros_like(t_b)
    return f32_to_e4m3(u_b.astype(np.float32))


def block_sq_error(x: np.ndarray, codes: np.ndarray, sigma: np.ndarray, s: np.float32) -> np.ndarray:
    """Float32 squared decode error of every block, [rows, K/16], in the
    fixed order of the module docstring."""
    x = _check_rows(x)
    rows, k = x.shape
    c = unpack_codes(codes).reshape(rows, k // BLOCK, BLOCK)
    p = (e2m1_value(c) * e4m3_value(sigma)[:, :, None]).astype(np.float32)  # exact
    xd = p * F32(s)                                                       # decode
    d = x.reshape(rows, k // BLOCK, BLOCK) - xd
    q = d * d
    e = np.zeros((rows, k // BLOCK), np.float32)
    for i in range(BLOCK):  # sequential float32 sum, element 0 first
        e = e + q[:, :, i]
    return e


def quantize_4over6_with_amax(x: np.ndarray, a: np.float32):
    """Four Over Six encode of one domain with amax ``a``.  Returns the
    QTensor and the per-block choice (True where the scale mapping the block
    maximum to 4 was kept)."""
    x = _check_rows(x)
    rows, k = x.shape
    s = tensor_scale(a)
    sig6 = block_scales_to(x, s, 6.0)
    sig4 = block_scales_to(x, s, 4.0)
    c6 = encode(x, sig6, s)
    c4 = encode(x, sig4, s)
    e6 = block_sq_error(x, c6, sig6, s)
    e4 = block_sq_error(x, c4, sig4, s)
    pick4 = e4 < e6
    sigma = np.where(pick4, sig4, sig6).astype(np.uint8)
    # codes: 8 bytes per block
    sel = np.repeat(pick4, BLOCK // 2, axis=1)
    codes = np.where(sel, c4, c6).astype(np.uint8)
    return QTensor(codes, sigma, np.array([s], dtype=np.float32)), pick4


def quantize_4over6(x: np.ndarray) -> QTensor:
    """Four Over Six quantization of a 2-D float32 tensor (one domain)."""
    x = _check_rows(x)
    return quantize_4over6_with_amax(x, amax(x))[0]


def kv_quantize_4over6(kv: np.ndarray, frame_block: int = 8) -> QTensor:
    """The KV codec of :func:`oracle.kv_quantize` (one tensor scale per block
    of ``frame_block`` frames, 16-element blocks along head_dim) with the
    Four Over Six encoder.  Decode with :func:`oracle.kv_dequantize`."""
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
        q = quantize_4over6(kv[f0:f1].reshape(-1, d))
        codes[f0 * per_frame:f1 * per_frame] = q.codes
        scales[f0 * per_frame:f1 * per_frame] = q.scales
        ts[b] = q.tscale[0]
    return QTensor(codes, scales, ts)

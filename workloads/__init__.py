"""Seeded synthetic inputs for the five DiT-shaped workloads.

This module only draws random numbers and casts them to the storage dtype; it
holds none of the quantization arithmetic, so both the HIP path (tests,
bench) and the CPU oracle can take their inputs from here without sharing any
of the method's code.

Shapes follow the LongLive-2.0 5B DiT as the pages describe it: 880 tokens per
latent frame at 1280x720, a model width of 3072, an FFN width of 14336, 24
heads of 128, a KV window of 3 sink + 9 local latent frames (171host.com
"LongLive 2.0 技术拆解", section 2.2) and 8-frame KV blocks (hyper.ai summary,
"方法").  No dataset, checkpoint or evaluation suite is used; random inputs
with the stated distributions stand in for activations, weights, gradients
and KV.

Workload 6 is not one of the five quoted configurations: it is the
training slice of one linear layer (forward, input gradient, weight
gradient) at the attention-projection shape, the input of the NVFP4
training GEMM triple.

Seeds: data ``1000 + workload number``, RHT sign mask ``2000 + workload
number``; robustness reruns add 100 or 200 to the data seed.  bf16 tensors are
returned as uint16 bit patterns (round-to-nearest-even cast done by torch on
the CPU); float32 tensors as float32.
"""

from __future__ import annotations

import numpy as np

WORKLOADS = {
    1: "tiny_linear_256x512x512",
    2: "dit_attn_proj_2640x3072x3072",
    3: "dit_ffn_10560x3072x14336",
    4: "kv_codec_12x880x24x128",
    5: "rht_wgrad_16384x3072",
    6: "train_linear_2640x3072x3072",
    7: "kv_window_attention_2640q_12x880x24x128",
}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (torch CPU cast, RNE) and return the bit patterns."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _outliers(rng, x: np.ndarray, p: float, factor: float) -> np.ndarray:
    mask = rng.random(x.shape) < p
    x[mask] *= np.float32(factor)
    return x


def tiny_linear(m=256, n=512, k=512, seed=1001):
    """Workload 1: A fp32 [m, k] and W fp32 [n, k] ~ N(0, 1), 1% of entries x20."""
    rng = np.random.default_rng(seed)
    a = _outliers(rng, rng.standard_normal((m, k), dtype=np.float32), 0.01, 20.0)
    w = _outliers(rng, rng.standard_normal((n, k), dtype=np.float32), 0.01, 20.0)
    return {"a": a, "w": w}


def attn_proj(m=2640, n=3072, k=3072, seed=1002):
    """Workload 2: X bf16 [m, k] ~ N(0, 1) times a per-channel factor drawn
    log-uniform in [0.1, 10]; W fp32 [n, k] ~ N(0, 0.02^2) (quantized offline)."""
    rng = np.random.default_rng(seed)
    c = np.exp(rng.uniform(np.log(0.1), np.log(10.0), size=k)).astype(np.float32)
    x = rng.standard_normal((m, k), dtype=np.float32) * c[None, :]
    w = (rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    return {"x": to_bf16_bits(x), "w": w}


def ffn(m=10560, d=3072, f=14336, seed=1003):
    """Workload 3: X bf16 [m, d] ~ N(0, 1) with 0.5% of entries x50;
    W1 fp32 [f, d] and W2 fp32 [d, f] ~ N(0, 0.02^2)."""
    rng = np.random.default_rng(seed)
    x = _outliers(rng, rng.standard_normal((m, d), dtype=np.float32), 0.005, 50.0)
    w1 = (rng.standard_normal((f, d), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    w2 = (rng.standard_normal((d, f), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    return {"x": to_bf16_bits(x), "w1": w1, "w2": w2}


def kv_cache(frames=12, tokens=880, heads=24, head_dim=128, seed=1004):
    """Workload 4: K and V bf16 [frames, tokens, heads, head_dim]; per head a
    std drawn log-uniform in [0.5, 4] (separately for K and V)."""
    rng = np.random.default_rng(seed)
    out = {}
    for name in ("k", "v"):
        std = np.exp(rng.uniform(np.log(0.5), np.log(4.0), size=heads)).astype(np.float32)
        x = rng.standard_normal((frames, tokens, heads, head_dim), dtype=np.float32)
        x *= std[None, None, :, None]
        out[name] = to_bf16_bits(x)
    return out


def rht_wgrad(rows=16384, cols=3072, seed=1005, mask_seed=2005):
    """Workload 5: gradient G bf16 [rows, cols] ~ Laplace(0, 1e-3) with 0.1% of
    entries x100, activations X bf16 [rows, cols] ~ N(0, 1), and the 16-bit
    RHT sign mask.  The reduction dimension of the weight-gradient GEMM is
    dim 0 (rows)."""
    rng = np.random.default_rng(seed)
    g = _outliers(rng, rng.laplace(0.0, 1e-3, size=(rows, cols)).astype(np.float32), 0.001, 100.0)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    mask = int(np.random.default_rng(mask_seed).integers(0, 2 ** 16))
    return {"g": to_bf16_bits(g), "x": to_bf16_bits(x), "mask": mask}


def train_linear(m=2640, n=3072, k=3072, seed=1006, mask_seed=2006):
    """Workload 6: one linear layer Y = X W^T in training at the attention-
    projection shape: X bf16 [m, k] as in workload 2, master weight W fp32
    [n, k] ~ N(0, 0.02^2), output gradient dY bf16 [m, n] ~ Laplace(0, 1e-3)
    with 0.1% of entries x100 (as the gradient of workload 5), and the RHT sign
    mask of the weight-gradient operands."""
    rng = np.random.default_rng(seed)
    c = np.exp(rng.uniform(np.log(0.1), np.log(10.0), size=k)).astype(np.float32)
    x = rng.standard_normal((m, k), dtype=np.float32) * c[None, :]
    w = (rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    dy = _outliers(rng, rng.laplace(0.0, 1e-3, size=(m, n)).astype(np.float32), 0.001, 100.0)
    mask = int(np.random.default_rng(mask_seed).integers(0, 2 ** 16))
    return {"x": to_bf16_bits(x), "w": w, "dy": to_bf16_bits(dy), "mask": mask}


def window_attention(frames=12, tokens=880, heads=24, head_dim=128, q_frames=3, seed=1007):
    """Workload 7: the K/V cache of workload 4 (3 sink + 9 window frames)
    plus the queries of the chunk being denoised: bf16 [q_frames * tokens,
    heads, head_dim] ~N(0,1) with a per-head std log-uniform in [0.5, 2]."""
    out = kv_cache(frames, tokens, heads, head_dim, seed=seed + 1)
    rng = np.random.default_rng(seed)
    std = np.exp(rng.uniform(np.log(0.5), np.log(2.0), size=heads)).astype(np.float32)
    q = rng.standard_normal((q_frames * tokens, heads, head_dim), dtype=np.float32)
    q *= std[None, :, None]
    out["q"] = to_bf16_bits(q)
    return out

"""Window attention over the NVFP4 KV cache.

Test infrastructure only (see the package docstring).

What the pages fix: generation is causal and frame-level autoregressive, a
chunk of latent frames at a time, with a causal mask hiding future frames
(171host.com "LongLive 2.0 技术拆解：KV Recache 与 NVFP4 推理", section on the
causal AR architecture); attention runs over a short window of 9 local latent
frames plus 3 sink frames kept permanently in the KV cache (same page,
section 2.2); the KV cache is held in NVFP4 (neurohive.io LongLive-2.0
summary, inference section; tailorednewshub.com "Inferencia W4A4 NVFP4") and
quantized per block of 8 frames (hyper.ai summary, "方法").

Reading implemented (the pages give no formula):

* the window is the cache's F frames (3 sink + 9 local = 12), stored as the
  NVFP4 KV codec stores them: rows (frame, token, head), 16-element blocks
  along head_dim, one tensor scale per 8-frame block;
* the queries are the tokens of the last ``q_frames`` frames of the window
  (the chunk being denoised, 3 frames), layout [q_frames * tokens, heads,
  head_dim];
* a query in window frame f sees every key of the frames 0..f (frame-level
  causal: the whole of its own frame, no future frame);
* per head, O = softmax(Q K^T / sqrt(head_dim)) V with K and V the exactly
  decoded cache values e2m1(code) * s_b * S (no rounding to bf16: the
  attention consumes the NVFP4 cache directly, which is the point of fusing
  the decode into it).

Everything is float64.  ``window_attention_ref`` also returns, per output
element, the quantity sum_j p_j |V_j| / sum_j p_j that the GPU tolerance is
expressed in (the error of rounding the probabilities scales with it).
"""

from __future__ import annotations

import numpy as np

from .codec import QTensor, decode_exact


def decode_kv(q: QTensor, frames: int, tokens: int, heads: int, head_dim: int, frame_block: int = 8) -> np.ndarray:
    """Exact float64 values e2m1 * s_b * S of a KV-codec tensor,
    [frames, tokens, heads, head_dim]."""
    p = decode_exact(q.codes, q.scales).reshape(frames, tokens, heads, head_dim)
    s = np.asarray(q.tscale, dtype=np.float64)[np.arange(frames) // frame_block]
    return p * s[:, None, None, None]


def key_visibility(frames: int, tokens: int, q_frames: int) -> np.ndarray:
    """Boolean [q_frames * tokens, frames * tokens]: query i (window frame
    frames - q_frames + i // tokens) sees key j (frame j // tokens) iff the
    key's frame is not later than the query's."""
    qf = frames - q_frames + np.arange(q_frames * tokens) // tokens
    kf = np.arange(frames * tokens) // tokens
    return kf[None, :] <= qf[:, None]


def window_attention_ref(q: np.ndarray, kq: QTensor, vq: QTensor, frames: int, tokens: int, heads: int,
                         head_dim: int, q_frames: int, frame_block: int = 8, query_rows=None):
    """O [q_frames * tokens, heads, head_dim] (float64) and the tolerance
    scale sum_j p_j |V_j| / sum_j p_j of the same shape.  ``q`` is float
    [q_frames * tokens, heads, head_dim]; ``query_rows`` optionally restricts
    the computed queries (the returned arrays then have that many rows)."""
    q = np.asarray(q, dtype=np.float64)
    k = decode_kv(kq, frames, tokens, heads, head_dim, frame_block).reshape(frames * tokens, heads, head_dim)
    v = decode_kv(vq, frames, tokens, heads, head_dim, frame_block).reshape(frames * tokens, heads, head_dim)
    vis = key_visibility(frames, tokens, q_frames)
    rows = np.arange(q.shape[0]) if query_rows is None else np.asarray(query_rows)
    out = np.empty((len(rows), heads, head_dim))
    scale = np.empty_like(out)
    for h in range(heads):
        s = (q[rows, h, :] @ k[:, h, :].T) / np.sqrt(head_dim)
        s = np.where(vis[rows], s, -np.inf)
        s = s - np.max(s, axis=1, keepdims=True)
        p = np.exp(s)
        l = np.sum(p, axis=1, keepdims=True)
        out[:, h, :] = (p @ v[:, h, :]) / l
        scale[:, h, :] = (p @ np.abs(v[:, h, :])) / l
    return out, scale

"""Pins for the oracle's window attention over the NVFP4 KV cache (CPU only).

Each pin comes from outside the oracle's own formula: a softmax over one key
returns that key's value; a zero query weights every visible key equally; on a
cache the codec represents exactly, the result equals PyTorch's
scaled_dot_product_attention on the unquantized tensors with a frame mask built
independently; a pure-Python loop on a tiny case; and the frame-causal
structure (a frame's keys reach exactly the queries of that frame and later).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as A
from oracle import formats as F


def _exact_kv(rng, frames, tokens, heads, d, frame_block, mags):
    """[frames, tokens, heads, d] float32 that the KV codec stores exactly:
    entries e2m1 * 448 * c with c = mags[frame block] (a power of two) and
    +-6 * 448 * c somewhere in every 16-element block, so S = c and every
    block scale is 448."""
    codes = rng.integers(0, 16, (frames, tokens, heads, d)).astype(np.uint8)
    x = F.e2m1_value(codes).astype(np.float64) * 448.0
    blk = x.reshape(frames, tokens, heads, d // 16, 16)
    pos = rng.integers(0, 16, blk.shape[:-1])
    sign = np.where(rng.random(blk.shape[:-1]) < 0.5, -1.0, 1.0)
    np.put_along_axis(blk, pos[..., None], (sign * 6.0 * 448.0)[..., None], axis=-1)
    c = np.asarray(mags, np.float64)[np.arange(frames) // frame_block]
    return (blk.reshape(x.shape) * c[:, None, None, None]).astype(np.float32)


@pytest.fixture
def rng():
    return np.random.default_rng(41)


def test_single_key_returns_its_value(rng):
    kv = rng.standard_normal((1, 1, 2, 32)).astype(np.float32)
    kq, vq = oracle.kv_quantize(kv), oracle.kv_quantize(kv * 3)
    q = rng.standard_normal((1, 2, 32))
    out, scale = A.window_attention_ref(q, kq, vq, 1, 1, 2, 32, 1)
    # the exact value e2m1 * s_b * S of every element (float64, no rounding)
    v = oracle.decode_exact(vq.codes, vq.scales) * np.float64(vq.tscale[0])
    assert np.array_equal(out[0], v)
    assert np.array_equal(scale[0], np.abs(v))


def test_zero_query_averages_the_visible_frames(rng):
    frames, tokens, heads, d, qf = 6, 3, 2, 16, 2
    k = rng.standard_normal((frames, tokens, heads, d)).astype(np.float32)
    v = rng.standard_normal((frames, tokens, heads, d)).astype(np.float32)
    kq, vq = oracle.kv_quantize(k, 4), oracle.kv_quantize(v, 4)
    vd = oracle.kv_dequantize(vq, frames, tokens, heads, d, 4, out="f32").astype(np.float64)
    out, _ = A.window_attention_ref(np.zeros((qf * tokens, heads, d)), kq, vq, frames, tokens, heads, d, qf, 4)
    for i in range(qf * tokens):
        last = frames - qf + i // tokens          # the query's own frame
        vis = vd[: last + 1].reshape(-1, heads, d)
        want = vis.mean(axis=0)
        # kv_dequantize rounds each decoded value to float32 (half an ulp)
        assert np.all(np.abs(out[i] - want) <= 2.0 ** -24 * np.abs(vis).mean(axis=0) + 1e-15)


def test_matches_sdpa_on_an_exactly_stored_cache(rng):
    frames, tokens, heads, d, qf, fb = 10, 5, 3, 32, 3, 8
    k = _exact_kv(rng, frames, tokens, heads, d, fb, [2.0 ** -5, 2.0 ** -2])
    v = _exact_kv(rng, frames, tokens, heads, d, fb, [2.0 ** 3, 2.0 ** -1])
    kq, vq = oracle.kv_quantize(k, fb), oracle.kv_quantize(v, fb)
    # the codec is exact on these tensors, with two distinct tensor scales
    assert np.array_equal(oracle.kv_dequantize(kq, frames, tokens, heads, d, fb, out="f32"), k)
    assert np.array_equal(oracle.kv_dequantize(vq, frames, tokens, heads, d, fb, out="f32"), v)
    assert kq.tscale[0] != kq.tscale[1] and vq.tscale[0] != vq.tscale[1]
    q = (rng.standard_normal((qf * tokens, heads, d)) * 0.05).astype(np.float32)
    out, _ = A.window_attention_ref(q, kq, vq, frames, tokens, heads, d, qf, fb)

    qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)               # [H, Lq, D]
    kt = torch.from_numpy(k.astype(np.float64)).reshape(-1, heads, d).permute(1, 0, 2)
    vt = torch.from_numpy(v.astype(np.float64)).reshape(-1, heads, d).permute(1, 0, 2)
    q_frame = torch.arange(frames - qf, frames).repeat_interleave(tokens)
    k_frame = torch.arange(frames).repeat_interleave(tokens)
    mask = k_frame[None, :] <= q_frame[:, None]
    want = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    want = want.permute(1, 0, 2).numpy()
    assert np.allclose(out, want, rtol=1e-12, atol=1e-12 * np.abs(v).max())


def test_pure_python_loop_on_a_tiny_cache(rng):
    frames, tokens, heads, d, qf = 3, 2, 2, 16, 2
    k = rng.standard_normal((frames, tokens, heads, d)).astype(np.float32)
    v = rng.standard_normal((frames, tokens, heads, d)).astype(np.float32)
    kq, vq = oracle.kv_quantize(k, 2), oracle.kv_quantize(v, 2)
    # float32 decode: each value within half an ulp of the exact one
    kd = oracle.kv_dequantize(kq, frames, tokens, heads, d, 2, out="f32").tolist()
    vd = oracle.kv_dequantize(vq, frames, tokens, heads, d, 2, out="f32").tolist()
    q = rng.standard_normal((qf * tokens, heads, d))
    out, _ = A.window_attention_ref(q, kq, vq, frames, tokens, heads, d, qf, 2)
    for i in range(qf * tokens):
        fq = frames - qf + i // tokens
        for h in range(heads):
            logits = []
            for f in range(fq + 1):
                for t in range(tokens):
                    dot = sum(float(q[i, h, e]) * kd[f][t][h][e] for e in range(d))
                    logits.append((dot / math.sqrt(d), f, t))
            top = max(s for s, _, _ in logits)
            w = [(math.exp(s - top), f, t) for s, f, t in logits]
            tot = sum(x for x, _, _ in w)
            for e in range(d):
                o = sum(x * vd[f][t][h][e] for x, f, t in w) / tot
                assert abs(out[i, h, e] - o) <= 1e-6 * (1 + abs(o))


def test_frame_causality(rng):
    frames, tokens, heads, d, qf = 7, 4, 2, 16, 3
    k = rng.standard_normal((frames, tokens, heads, d)).astype(np.float32)
    v = rng.standard_normal((frames, tokens, heads, d)).astype(np.float32)
    q = rng.standard_normal((qf * tokens, heads, d))
    kq, vq = oracle.kv_quantize(k), oracle.kv_quantize(v)
    base, _ = A.window_attention_ref(q, kq, vq, frames, tokens, heads, d, qf)
    per_frame = tokens * heads
    for f in range(frames):
        # flip the sign bit of every code of frame f (its values change sign)
        codes = vq.codes.copy()
        codes[f * per_frame:(f + 1) * per_frame] ^= 0x88
        vq2 = oracle.QTensor(codes, vq.scales, vq.tscale)
        out, _ = A.window_attention_ref(q, kq, vq2, frames, tokens, heads, d, qf)
        changed = np.any(out != base, axis=(1, 2))
        q_frame = frames - qf + np.arange(qf * tokens) // tokens
        assert np.array_equal(changed, q_frame >= f), f


def test_query_subset_and_scale_bound(rng):
    frames, tokens, heads, d, qf = 12, 6, 3, 32, 3
    k = rng.standard_normal((frames, tokens, heads, d)).astype(np.float32)
    v = rng.standard_normal((frames, tokens, heads, d)).astype(np.float32)
    q = rng.standard_normal((qf * tokens, heads, d))
    kq, vq = oracle.kv_quantize(k), oracle.kv_quantize(v)
    full, scale = A.window_attention_ref(q, kq, vq, frames, tokens, heads, d, qf)
    rows = np.array([0, 5, 6, 17])
    part, pscale = A.window_attention_ref(q, kq, vq, frames, tokens, heads, d, qf, query_rows=rows)
    # same values up to the summation order the matrix product picks
    assert np.allclose(part, full[rows], rtol=1e-13, atol=1e-15)
    assert np.allclose(pscale, scale[rows], rtol=1e-13, atol=1e-15)
    assert np.all(np.abs(full) <= scale * (1 + 1e-12))


def test_visibility_mask_shape():
    vis = A.key_visibility(frames=4, tokens=2, q_frames=2)
    # queries 0-1 sit in window frame 2 (keys 0-5), queries 2-3 in frame 3 (all 8)
    assert vis.sum(axis=1).tolist() == [6, 6, 8, 8]
    assert not vis[0, 6] and vis[0, 5]

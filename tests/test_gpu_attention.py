"""GPU parity of nvfp4_kv_attention (frame-causal window attention over the
NVFP4 KV cache) against the float64 oracle.

The caches are quantized by the oracle on the host and uploaded, so every
oracle input is the oracle's own.  Tolerance, per output element, derived from
the kernel's arithmetic (probabilities rounded to fp16: 2^-11 relative in
fp16's normal range, counted for numerator and denominator; score
accumulation in float32 over head_dim exact products: 2^-17 * A relative, A
the largest sum_d |q_d k_d| / sqrt(head_dim) over the visible keys, counted
twice; float32 accumulation of O and of the row sum over at most a few
hundred steps per lane: below 2^-15):

    |gpu - ref| <= scale * (2^-10 + 2^-15 * A) + U

with scale = sum_j p_j |V_j| / sum_j p_j (>= |ref|), plus half a bf16 ulp for
bf16 outputs.  U covers probabilities below fp16's normal range: the kernel's
probabilities are exp2(s_j - m) with m at most the largest score, so a key
with exp(score_j - max score) >= 2^-13 stays above 2^-14, in the normal
range; the others (set T) may be subnormal, where fp16 rounds with an
absolute error of at most 2^-25.  Numerator and denominator then move by at
most 2^-25 sum_T |V_j| and 2^-25 |T|, against a row sum of at least
L = sum_j exp(score_j - max score) over the visible keys:

    U = 2^-24 * (sum_T |V_j| + |T| |ref|) / L

(2^-25 doubled to cover the score error in L and in the split).  U matters
only where the output is carried by keys weighted below about 2^-24 of the
largest (e.g. dominant keys whose V is zero).  Observed errors are reported and sit far
below the bound."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import bf16_half_ulp, dev_bf16, host_bf16_bits, log, require_gpu, widen
from oracle import attention as A

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    return require_gpu()


def _upload(nv, q):
    return nv.NVFP4Tensor(torch.from_numpy(np.ascontiguousarray(q.codes)).cuda(),
                          torch.from_numpy(np.ascontiguousarray(q.scales)).cuda(),
                          torch.from_numpy(np.ascontiguousarray(q.tscale, dtype=np.float32)).cuda())


def _score_bound(qf, kq, frames, tokens, heads, d, q_frames, fb, rows):
    """A[row, head] = max over visible keys of sum_d |q_d k_d| / sqrt(d)."""
    k = A.decode_kv(kq, frames, tokens, heads, d, fb).reshape(frames * tokens, heads, d)
    vis = A.key_visibility(frames, tokens, q_frames)[rows]
    out = np.empty((len(rows), heads))
    for h in range(heads):
        s = np.abs(qf[rows, h, :]) @ np.abs(k[:, h, :]).T / np.sqrt(d)
        out[:, h] = np.max(np.where(vis, s, 0.0), axis=1)
    return out


def _underflow_term(qf, kq, vq, frames, tokens, heads, d, q_frames, fb, rows, ref):
    """U[row, head, :] = 2^-24 (sum_T |V_j| + |T| |ref|) / L, T the visible
    keys with exp(score_j - max score) < 2^-13, L = sum_j exp(score_j - max
    score) over the visible keys (module docstring)."""
    k = A.decode_kv(kq, frames, tokens, heads, d, fb).reshape(frames * tokens, heads, d)
    v = A.decode_kv(vq, frames, tokens, heads, d, fb).reshape(frames * tokens, heads, d)
    vis = A.key_visibility(frames, tokens, q_frames)[rows]
    out = np.empty((len(rows), heads, d))
    for h in range(heads):
        s = np.where(vis, qf[rows, h, :] @ k[:, h, :].T / np.sqrt(d), -np.inf)
        w = np.exp(s - s.max(axis=1, keepdims=True))       # 0 for keys not visible
        small = vis & (w < 2.0 ** -13)
        sum_v = small.astype(np.float64) @ np.abs(v[:, h, :])
        n = small.sum(axis=1).astype(np.float64)
        out[:, h, :] = 2.0 ** -24 * (sum_v + n[:, None] * np.abs(ref[:, h, :])) / w.sum(axis=1)[:, None]
    return out


def _check(gpu, ref, scale, bound, out_bf16, tag, under=0.0):
    tol = scale * (2.0 ** -10 + 2.0 ** -15 * bound[:, :, None]) + under
    if out_bf16:
        tol = tol + bf16_half_ulp(np.abs(ref) + tol)
    err = np.abs(np.asarray(gpu, np.float64) - ref)
    bad = np.argwhere(err > tol)
    rel = float((err / np.maximum(scale, 1e-300)).max())
    share = float(np.max(under / tol)) if np.ndim(under) else 0.0
    log(f"  {tag}: max err/scale {rel:.3e}, max A {bound.max():.1f}, largest share of U in a tolerance {share:.2f}")
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError(f"{tag}: {len(bad)} of {err.size} outside tolerance; first {i}: gpu {gpu[i]!r} "
                             f"ref {ref[i]!r} scale {scale[i]!r} tol {tol[i]!r}")
    return rel


def _run(nv, qbits, kq, vq, shape, q_frames, fb, out_dtype):
    f, t, h, d = shape
    qd = dev_bf16(qbits.reshape(q_frames * t, h, d))
    out = nv.kv_attention(qd, _upload(nv, kq), _upload(nv, vq), shape, fb, out_dtype=out_dtype)
    torch.cuda.synchronize()
    if out_dtype == torch.float32:
        return out.cpu().numpy().astype(np.float64)
    return widen(host_bf16_bits(out)).astype(np.float64)


def _case(rng, frames, tokens, heads, q_frames, q_std=1.0, k_std=1.0, v_std=1.0, d=128):
    k = (rng.standard_normal((frames, tokens, heads, d)) * k_std).astype(np.float32)
    v = (rng.standard_normal((frames, tokens, heads, d)) * v_std).astype(np.float32)
    q = (rng.standard_normal((q_frames * tokens, heads, d)) * q_std).astype(np.float32)
    return workloads.to_bf16_bits(q), k, v


CASES = [
    # frames, tokens, heads, q_frames, frame_block
    (12, 40, 3, 3, 8),     # two frame blocks, ragged last key tile, one query tile
    (12, 96, 2, 3, 8),     # three query tiles, frame boundaries inside tiles
    (5, 13, 2, 2, 8),      # one frame block, tokens not a multiple of 32
    (1, 7, 1, 1, 8),       # a single frame: every key visible
    (9, 32, 4, 1, 2),      # five frame blocks of 64 keys
    (4, 96, 2, 4, 2),      # all frames are queries; frame blocks of 192 keys (3 tiles)
    # frame blocks that are not a whole number of 64-key tiles: the tile
    # holding a block boundary mixes two tensor scales
    (12, 100, 2, 3, 8),    # 800-key blocks (boundary inside key tile 12)
    (4, 96, 2, 4, 3),      # 288-key blocks; all frames are queries
    (10, 9, 2, 3, 2),      # 18-key blocks: up to five blocks inside one tile
    (7, 50, 3, 2, 3),      # 150-key blocks, partial last block, ragged last tile
]


# head dimension 64 (the kernel's second instance) on the shapes that
# exercise ragged tiles and frame blocks that are not whole tiles
CASES_D64 = [c + (64,) for c in (CASES[0], CASES[3], CASES[4], CASES[6], CASES[8], CASES[9])]


@pytest.mark.parametrize("frames,tokens,heads,q_frames,fb,d", [c + (128,) for c in CASES] + CASES_D64)
def test_attention_matches_oracle(nv, frames, tokens, heads, q_frames, fb, d):
    log(f"kv_attention {frames}x{tokens}x{heads}x{d} q_frames={q_frames} fb={fb}")
    rng = np.random.default_rng(frames * 1000 + tokens * 10 + heads + (d != 128))
    qbits, k, v = _case(rng, frames, tokens, heads, q_frames, k_std=1.5, d=d)
    kq, vq = oracle.kv_quantize(k, fb), oracle.kv_quantize(v, fb)
    shape = (frames, tokens, heads, d)
    qf = widen(qbits).reshape(q_frames * tokens, heads, d)
    ref, scale = A.window_attention_ref(qf, kq, vq, frames, tokens, heads, d, q_frames, fb)
    rows = np.arange(q_frames * tokens)
    bound = _score_bound(qf, kq, frames, tokens, heads, d, q_frames, fb, rows)
    under = _underflow_term(qf, kq, vq, frames, tokens, heads, d, q_frames, fb, rows, ref)
    g32 = _run(nv, qbits, kq, vq, shape, q_frames, fb, torch.float32)
    _check(g32, ref, scale, bound, False, "f32 out", under)
    g16 = _run(nv, qbits, kq, vq, shape, q_frames, fb, torch.bfloat16)
    _check(g16, ref, scale, bound, True, "bf16 out", under)
    # the bf16 output is the float32 result rounded to nearest even
    assert np.array_equal(workloads.to_bf16_bits(g32.astype(np.float32)), workloads.to_bf16_bits(g16.astype(np.float32)))


def test_frame_block_beyond_window_is_one_block(nv):
    """frame_block >= frames means one block over the whole window: the
    result equals frame_block == frames bit for bit (the cache, quantized
    with one tensor scale, is the same)."""
    frames, tokens, heads, q_frames = 6, 40, 2, 2
    log("kv_attention frame_block beyond the window")
    rng = np.random.default_rng(91)
    qbits, k, v = _case(rng, frames, tokens, heads, q_frames)
    kq, vq = oracle.kv_quantize(k, frames), oracle.kv_quantize(v, frames)
    assert np.array_equal(oracle.kv_quantize(k, 1 << 20).codes, kq.codes)
    shape = (frames, tokens, heads, 128)
    ref = _run(nv, qbits, kq, vq, shape, q_frames, frames, torch.float32)
    for fb in (frames + 1, 64, 1 << 30):
        got = _run(nv, qbits, kq, vq, shape, q_frames, fb, torch.float32)
        assert np.array_equal(got.view(np.uint64), ref.view(np.uint64)), fb


@pytest.mark.parametrize("d", [128, 64])
def test_extreme_query_rows_and_scales(nv, d):
    """Query rows from 2^-60 to 2^18 (the per-row fp16 scaling on both ends),
    an all-zero row, K frame blocks with tensor scales 2^12 apart, a V frame
    block that is all zero (tensor scale 0).  Rows with moderate scores are
    held to the full tolerance; rows whose scores are so large that the
    softmax is one-hot (gap to the runner-up > 40 and far above the float32
    score error) must return the top key's value."""
    frames, tokens, heads, q_frames, fb = 10, 32, 2, 3, 4
    log(f"kv_attention extreme rows/scales d={d}")
    rng = np.random.default_rng(77)
    qbits, k, v = _case(rng, frames, tokens, heads, q_frames, d=d)
    q = widen(qbits).reshape(q_frames * tokens, heads, d)
    row_mag = 2.0 ** rng.integers(-60, 3, q.shape[0]).astype(np.float64)
    row_mag[:4] = [2.0 ** -60, 2.0 ** -20, 2.0 ** 18, 4.0]
    row_mag[5] = 0.0                               # an all-zero query row: uniform weights
    qbits = workloads.to_bf16_bits((q * row_mag[:, None, None]).astype(np.float32))
    k[4:8] *= 4096.0
    k[8:] /= 4096.0
    v[4:8] = 0.0
    kq, vq = oracle.kv_quantize(k, fb), oracle.kv_quantize(v, fb)
    assert vq.tscale[1] == 0.0 and kq.tscale[1] > 1000 * kq.tscale[0]
    shape = (frames, tokens, heads, d)
    qf = widen(qbits).reshape(q_frames * tokens, heads, d)
    ref, scale = A.window_attention_ref(qf, kq, vq, frames, tokens, heads, d, q_frames, fb)
    rows = np.arange(q_frames * tokens)
    bound = _score_bound(qf, kq, frames, tokens, heads, d, q_frames, fb, rows)
    under = _underflow_term(qf, kq, vq, frames, tokens, heads, d, q_frames, fb, rows, ref)
    g32 = _run(nv, qbits, kq, vq, shape, q_frames, fb, torch.float32)
    assert np.all(np.isfinite(g32))
    moderate = bound <= 64.0
    sel = moderate.all(axis=1)
    assert sel.sum() >= 20
    _check(g32[sel], ref[sel], scale[sel], bound[sel], False, "moderate rows", under[sel])
    # one-hot rows: exact float64 scores from the decoded cache
    kd = A.decode_kv(kq, frames, tokens, heads, d, fb).reshape(frames * tokens, heads, d)
    vd = A.decode_kv(vq, frames, tokens, heads, d, fb).reshape(frames * tokens, heads, d)
    vis = A.key_visibility(frames, tokens, q_frames)
    checked = 0
    for r in np.argwhere(~moderate):
        i, h = int(r[0]), int(r[1])
        sc = np.where(vis[i], kd[:, h, :] @ qf[i, h, :].astype(np.float64) / np.sqrt(d), -np.inf)
        top2 = np.sort(sc)[-2:]
        if top2[1] - top2[0] > max(40.0, 2.0 ** -14 * bound[i, h]):
            j = int(np.argmax(sc))
            want = vd[j, h, :]
            assert np.all(np.abs(g32[i, h] - want) <= 2.0 ** -10 * np.abs(want) + 1e-30), (i, h)
            checked += 1
    log(f"  one-hot rows checked: {checked} of {int((~moderate).sum())}")
    assert checked >= 4


def test_all_zero_key_block(nv):
    """A K frame block that is all zero (tensor scale 0): its keys score 0 for
    every query, so they take part in the softmax with weight exp(-max)."""
    frames, tokens, heads, q_frames, fb = 12, 32, 2, 3, 4
    log("kv_attention all-zero K frame block")
    rng = np.random.default_rng(79)
    qbits, k, v = _case(rng, frames, tokens, heads, q_frames)
    k[4:8] = 0.0
    kq, vq = oracle.kv_quantize(k, fb), oracle.kv_quantize(v, fb)
    assert kq.tscale[1] == 0.0
    shape = (frames, tokens, heads, 128)
    qf = widen(qbits).reshape(q_frames * tokens, heads, 128)
    ref, scale = A.window_attention_ref(qf, kq, vq, frames, tokens, heads, 128, q_frames, fb)
    rows = np.arange(q_frames * tokens)
    bound = _score_bound(qf, kq, frames, tokens, heads, 128, q_frames, fb, rows)
    under = _underflow_term(qf, kq, vq, frames, tokens, heads, 128, q_frames, fb, rows, ref)
    _check(_run(nv, qbits, kq, vq, shape, q_frames, fb, torch.float32), ref, scale, bound, False, "zero K block",
           under)


def test_four_over_six_cache(nv):
    """The attention reads a cache written by the Four Over Six encoder
    unchanged (same format)."""
    frames, tokens, heads, q_frames, fb = 12, 40, 2, 3, 8
    log("kv_attention four-over-six cache")
    rng = np.random.default_rng(78)
    qbits, k, v = _case(rng, frames, tokens, heads, q_frames)
    kq, vq = oracle.kv_quantize_4over6(k, fb), oracle.kv_quantize_4over6(v, fb)
    shape = (frames, tokens, heads, 128)
    qf = widen(qbits).reshape(q_frames * tokens, heads, 128)
    ref, scale = A.window_attention_ref(qf, kq, vq, frames, tokens, heads, 128, q_frames, fb)
    rows = np.arange(q_frames * tokens)
    bound = _score_bound(qf, kq, frames, tokens, heads, 128, q_frames, fb, rows)
    under = _underflow_term(qf, kq, vq, frames, tokens, heads, 128, q_frames, fb, rows, ref)
    _check(_run(nv, qbits, kq, vq, shape, q_frames, fb, torch.float32), ref, scale, bound, False, "4/6 cache",
           under)


@pytest.mark.timeout(600)
def test_attention_full_workload(nv):
    """Workload 7 at full size (2640 queries x 24 heads over 12 x 880 keys),
    bf16 output as timed: every query row of every head against the float64
    oracle."""
    log("kv_attention full workload")
    w = workloads.window_attention()
    frames, tokens, heads, d, q_frames, fb = 12, 880, 24, 128, 3, 8
    k, v = widen(w["k"]).reshape(frames, tokens, heads, d), widen(w["v"]).reshape(frames, tokens, heads, d)
    kq, vq = oracle.kv_quantize(k, fb), oracle.kv_quantize(v, fb)
    g16 = _run(nv, w["q"], kq, vq, (frames, tokens, heads, d), q_frames, fb, torch.bfloat16)
    assert g16.shape == (q_frames * tokens, heads, d)
    assert np.all(np.isfinite(g16))
    qf = widen(w["q"]).reshape(q_frames * tokens, heads, d)
    rows = np.arange(q_frames * tokens)
    ref, scale = A.window_attention_ref(qf, kq, vq, frames, tokens, heads, d, q_frames, fb)
    bound = _score_bound(qf, kq, frames, tokens, heads, d, q_frames, fb, rows)
    under = _underflow_term(qf, kq, vq, frames, tokens, heads, d, q_frames, fb, rows, ref)
    _check(g16, ref, scale, bound, True, "full workload, every row", under)


def test_attention_head_dim_64_window(nv):
    """head_dim 64 over a full-size window (12 frames of 880 tokens, 8-frame
    blocks, 2640 queries) and 4 heads, bf16 output: the first two query
    tiles, the last rows and a random sample against the float64 oracle."""
    frames, tokens, heads, d, q_frames, fb = 12, 880, 4, 64, 3, 8
    log("kv_attention head_dim 64 window")
    rng = np.random.default_rng(64)
    qbits, k, v = _case(rng, frames, tokens, heads, q_frames, d=d)
    kq, vq = oracle.kv_quantize(k, fb), oracle.kv_quantize(v, fb)
    g16 = _run(nv, qbits, kq, vq, (frames, tokens, heads, d), q_frames, fb, torch.bfloat16)
    nq = q_frames * tokens
    rows = np.unique(np.concatenate([np.arange(256), rng.choice(nq, 256, replace=False), np.arange(nq - 80, nq)]))
    qf = widen(qbits).reshape(nq, heads, d)
    ref, scale = A.window_attention_ref(qf, kq, vq, frames, tokens, heads, d, q_frames, fb, query_rows=rows)
    bound = _score_bound(qf, kq, frames, tokens, heads, d, q_frames, fb, rows)
    under = _underflow_term(qf, kq, vq, frames, tokens, heads, d, q_frames, fb, rows, ref)
    _check(g16[rows], ref, scale, bound, True, f"head_dim 64, {len(rows)} rows", under)

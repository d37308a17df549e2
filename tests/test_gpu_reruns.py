"""Robustness reruns: the full-size workloads again with the data seed moved by
+100 and +200, each against the oracle to the same bar as the default seed
(codes, scale bytes and tensor scales bit-exact; dequant bit-exact; GEMM and
attention within their parity bounds).  Different draws move block maxima
across E4M3 rounding boundaries and put different elements on E2M1 ties,
which a single seed exercises only once."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import (assert_gemm_close, assert_q_exact, dev_bf16, dev_f32, host_bf16_bits, log, require_gpu,
                         widen)
from oracle import attention as A
from test_gpu_attention import _check, _run, _score_bound, _underflow_term

pytestmark = pytest.mark.gpu

SHIFTS = [100, 200]


@pytest.fixture(scope="module")
def nv():
    return require_gpu()


@pytest.mark.parametrize("shift", SHIFTS)
def test_attn_proj_reruns(nv, shift):
    d = workloads.attn_proj(seed=1002 + shift)
    log(f"attention projection 2640x3072x3072, seed {1002 + shift}")
    gx = nv.quantize(dev_bf16(d["x"]))
    gw = nv.quantize(dev_f32(d["w"]))
    ox, ow = oracle.quantize(widen(d["x"])), oracle.quantize(d["w"])
    torch.cuda.synchronize()
    assert_q_exact(gx, ox, "X")
    assert_q_exact(gw, ow, "W")
    y = nv.gemm(gx, gw, out_dtype=torch.bfloat16)
    cref, bound = oracle.gemm_ref(ox, ow)
    assert_gemm_close(y.float().cpu().numpy(), cref, bound, True, f"seed +{shift}")


@pytest.mark.parametrize("shift", SHIFTS)
def test_kv_codec_reruns(nv, shift):
    d = workloads.kv_cache(seed=1004 + shift)
    shape = (12, 880, 24, 128)
    for name, fo6 in (("k", False), ("v", True)):
        log(f"KV codec {name} {shape}, seed {1004 + shift}, four_over_six={fo6}")
        x = widen(d[name]).reshape(shape)
        gq = nv.kv_quant(dev_bf16(d[name]), four_over_six=fo6)
        oq = oracle.kv_quantize_4over6(x) if fo6 else oracle.kv_quantize(x)
        torch.cuda.synchronize()
        assert_q_exact(gq, oq, f"kv {name}")
        y = host_bf16_bits(nv.kv_dequant(gq, shape))
        assert np.array_equal(y, oracle.kv_dequantize(oq, *shape))


@pytest.mark.parametrize("shift", SHIFTS)
def test_rht_gradient_reruns(nv, shift):
    """RHT16 + quantize along dim 0 of the first 4096 gradient rows (the
    transform and the column blocks do not couple rows across 16-row groups,
    so a row slice is an instance of the same computation)."""
    d = workloads.rht_wgrad(seed=1005 + shift, mask_seed=2005 + shift)
    g = np.ascontiguousarray(d["g"][:4096])
    log(f"RHT16 + quantize G[:4096] bf16 along dim 0, seed {1005 + shift}, mask {d['mask']:#06x}")
    gq = nv.rht16_quantize(dev_bf16(g), d["mask"], axis=0)
    oq = oracle.rht16_quantize(widen(g), d["mask"], axis=0)
    torch.cuda.synchronize()
    assert_q_exact(gq, oq, "rht G")


@pytest.mark.parametrize("shift", SHIFTS)
def test_window_attention_reruns(nv, shift):
    w = workloads.window_attention(seed=1007 + shift)
    frames, tokens, heads, d, q_frames, fb = 12, 880, 24, 128, 3, 8
    log(f"window attention 2640 queries x 24 heads, seed {1007 + shift}")
    k, v = widen(w["k"]).reshape(frames, tokens, heads, d), widen(w["v"]).reshape(frames, tokens, heads, d)
    kq, vq = oracle.kv_quantize(k, fb), oracle.kv_quantize(v, fb)
    g16 = _run(nv, w["q"], kq, vq, (frames, tokens, heads, d), q_frames, fb, torch.bfloat16)
    assert np.all(np.isfinite(g16))
    rows = np.union1d([0, 879, 880, 1759, 1760, 2639], np.random.default_rng(shift).integers(0, 2640, 16))
    qf = widen(w["q"]).reshape(q_frames * tokens, heads, d)
    ref, scale = A.window_attention_ref(qf, kq, vq, frames, tokens, heads, d, q_frames, fb, query_rows=rows)
    bound = _score_bound(qf, kq, frames, tokens, heads, d, q_frames, fb, rows)
    under = _underflow_term(qf, kq, vq, frames, tokens, heads, d, q_frames, fb, rows, ref)
    _check(g16[rows], ref, scale, bound, True, f"seed +{shift}", under)

"""GPU parity of the block-scaled W4A4 GEMM against the float64 oracle:
|gpu - C| <= 1e-5 * sum_k |P_A P_B| per element (plus half a bf16 ulp for bf16
outputs).  Operand codes are first checked bit-exact against the oracle's own
quantization, so both sides multiply the same NVFP4 numbers.  Covers ragged
M/N/K tails (the K-checked path and the K % 128 fast path), fp32/bf16
outputs, the GELU epilogue with its amax reduction, and the workload shapes
(tiny linear, attention projection, FFN pair stage by stage, weight-gradient
GEMM after the RHT) at full size."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import (assert_gemm_close, assert_q_exact, dev_bf16, dev_f32, log, require_gpu, widen)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    return require_gpu()


def _operands(nv, rng, m, n, k):
    a = (rng.standard_normal((m, k)) * np.exp(rng.uniform(-2, 2, (m, 1)))).astype(np.float32)
    a[rng.random(a.shape) < 0.01] *= 20
    b = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    ga, gb = nv.quantize(dev_f32(a)), nv.quantize(dev_f32(b))
    oa, ob = oracle.quantize(a), oracle.quantize(b)
    torch.cuda.synchronize()
    assert_q_exact(ga, oa, "A")
    assert_q_exact(gb, ob, "B")
    return ga, gb, oa, ob


SHAPES = [(1, 1, 16), (17, 33, 48), (64, 256, 128), (255, 130, 512), (200, 300, 1024), (33, 65, 2064),
          (129, 257, 384), (512, 512, 256)]


@pytest.mark.parametrize("m,n,k", SHAPES)
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemm_matches_oracle(nv, m, n, k, out):
    log(f"gemm {m}x{n}x{k} -> {out}")
    rng = np.random.default_rng(m * 1000003 + n * 101 + k)
    ga, gb, oa, ob = _operands(nv, rng, m, n, k)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    c = nv.gemm(ga, gb, out_dtype=dt)
    cref, bound = oracle.gemm_ref(oa, ob)
    assert_gemm_close(c.float().cpu().numpy(), cref, bound, out == "bf16", f"{m}x{n}x{k} {out}")


@pytest.mark.parametrize("tiles", [(2, 4), (4, 2), (3, 3), (4, 4)])
@pytest.mark.parametrize("m,n,k", [(300, 520, 384), (97, 1100, 1280), (1030, 70, 256), (200, 330, 192),
                                   (65, 300, 1344)])
def test_gemm_every_tile_shape(nv, tiles, m, n, k):
    log(f"gemm tiles {tiles} {m}x{n}x{k}")
    rng = np.random.default_rng(m + n + k + 10 * tiles[0])
    ga, gb, oa, ob = _operands(nv, rng, m, n, k)
    cref, bound = oracle.gemm_ref(oa, ob)
    c = nv.gemm(ga, gb, out_dtype=torch.float32, tiles=tiles)
    assert_gemm_close(c.cpu().numpy(), cref, bound, False, f"tiles {tiles}")
    amax = torch.empty(1, device="cuda")
    h = nv.gemm(ga, gb, out_dtype=torch.bfloat16, epilogue=nv.EPI_GELU_TANH, amax_out=amax, tiles=tiles)
    hh = h.float().cpu().numpy().astype(np.float64)
    g = oracle.gelu_tanh(cref)
    tol = 1.13 * 1e-5 * bound + np.abs(g) * 2.0 ** -8 + 8 * np.spacing(np.abs(g).astype(np.float32)) + 1e-37
    assert np.all(np.abs(hh - g) <= tol)
    assert amax.item() == float(np.abs(hh).max())


@pytest.mark.parametrize("m,n,k", [(300, 520, 384), (65, 300, 1344), (512, 512, 3072)])
def test_tile_shapes_are_bit_identical(nv, m, n, k):
    """Every tile shape (and the automatic choice) accumulates an output
    element in the same order: float32 results are bit-identical.  The data
    span a wide range, so the float32 sums do round (checked against the
    float64 oracle), which makes the identity a property of the order."""
    log(f"gemm tile-shape identity {m}x{n}x{k}")
    rng = np.random.default_rng(m * 7 + k)
    a = (rng.standard_normal((m, k)) * np.exp(rng.uniform(-4, 4, (m, 1)))).astype(np.float32)
    a[rng.random(a.shape) < 0.02] *= 50
    b = (rng.standard_normal((n, k)) * np.exp(rng.uniform(-3, 3, (1, k)))).astype(np.float32)
    ga, gb = nv.quantize(dev_f32(a)), nv.quantize(dev_f32(b))
    outs = [nv.gemm(ga, gb, out_dtype=torch.float32, tiles=t).cpu().numpy() for t in (None, (2, 4), (4, 2), (3, 3), (4, 4))]
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))
    cref, bound = oracle.gemm_ref(oracle.quantize(a), oracle.quantize(b))
    assert_gemm_close(outs[0], cref, bound, False, "tile identity")
    assert np.any(outs[0] != cref.astype(np.float32))  # the float32 accumulation rounded somewhere


def test_gemm_with_an_all_zero_operand(nv):
    """A zero activation tensor quantizes to S = 0; the product is exactly 0
    everywhere (no NaN from 0 * scale paths) and the output amax is 0."""
    rng = np.random.default_rng(11)
    b = (rng.standard_normal((300, 256)) * 0.02).astype(np.float32)
    ga, gb = nv.quantize(dev_f32(np.zeros((200, 256), np.float32))), nv.quantize(dev_f32(b))
    amax = torch.full((1,), 5.0, device="cuda")
    for out_dtype in (torch.float32, torch.bfloat16):
        c = nv.gemm(ga, gb, out_dtype=out_dtype, epilogue=nv.EPI_GELU_TANH, amax_out=amax)
        torch.cuda.synchronize()
        assert float(ga.tscale.cpu()[0]) == 0.0
        assert torch.all(c.float().cpu() == 0.0)
        assert amax.item() == 0.0


def test_gemm_into_strided_output(nv):
    rng = np.random.default_rng(3)
    ga, gb, oa, ob = _operands(nv, rng, 70, 90, 256)
    big = torch.full((70, 128), 7.0, device="cuda")
    nv.gemm(ga, gb, out=big[:, :90], out_dtype=torch.float32)
    h = big.cpu().numpy()
    cref, bound = oracle.gemm_ref(oa, ob)
    assert_gemm_close(h[:, :90], cref, bound, False, "strided")
    assert np.all(h[:, 90:] == 7.0)  # nothing written past N


@pytest.mark.parametrize("width", [312, 301])
@pytest.mark.parametrize("tiles", [(2, 4), (4, 2), (4, 4)])
def test_gemm_bf16_into_strided_output(nv, width, tiles):
    """bf16 output rows `width` elements apart: whole wavefront sub-tiles go
    through the LDS-staged 16-byte stores when rows are 16-byte aligned
    (width 312), the per-element stores otherwise (width 301); edge sub-tiles
    always take the per-element stores.  Nothing is written past N."""
    log(f"gemm bf16 strided width {width} tiles {tiles}")
    rng = np.random.default_rng(width + 7 * tiles[0])
    ga, gb, oa, ob = _operands(nv, rng, 200, 300, 256)
    fill = torch.tensor(3.0, dtype=torch.bfloat16)
    big = torch.full((200, width), 3.0, dtype=torch.bfloat16, device="cuda")
    amax = torch.empty(1, device="cuda")
    nv.gemm(ga, gb, out=big[:, :300], epilogue=nv.EPI_GELU_TANH, amax_out=amax, tiles=tiles)
    h = big.float().cpu().numpy().astype(np.float64)
    cref, bound = oracle.gemm_ref(oa, ob)
    g = oracle.gelu_tanh(cref)
    tol = 1.13 * 1e-5 * bound + np.abs(g) * 2.0 ** -8 + 8 * np.spacing(np.abs(g).astype(np.float32)) + 1e-37
    assert np.all(np.abs(h[:, :300] - g) <= tol)
    assert np.all(h[:, 300:] == float(fill))  # nothing written past N
    assert amax.item() == float(np.abs(h[:, :300]).max())


@pytest.mark.parametrize("m,n,k", [(64, 128, 256), (100, 70, 528), (256, 512, 3072)])
def test_gelu_epilogue_and_amax(nv, m, n, k):
    log(f"gemm gelu {m}x{n}x{k}")
    rng = np.random.default_rng(k + m)
    ga, gb, oa, ob = _operands(nv, rng, m, n, k)
    amax = torch.empty(1, device="cuda")
    h = nv.gemm(ga, gb, out_dtype=torch.float32, epilogue=nv.EPI_GELU_TANH, amax_out=amax)
    hh = h.cpu().numpy().astype(np.float64)
    cref, bound = oracle.gemm_ref(oa, ob)
    g = oracle.gelu_tanh(cref)
    # |g'| <= 1.13 carries the GEMM tolerance through GELU; float32 GELU adds a
    # few ulp of its own (tanhf, products).
    tol = 1.13 * 1e-5 * bound + 8 * np.spacing(np.abs(g).astype(np.float32)).astype(np.float64) + 1e-37
    err = np.abs(hh - g)
    assert np.all(err <= tol), f"max err/tol {np.max(err / tol)}"
    assert amax.item() == float(np.abs(h.cpu().numpy()).max())


# ---------------------------------------------------------------- workloads
def test_tiny_linear_full(nv):
    d = workloads.tiny_linear()
    log("workload 1: 256x512 @ 512x512 -> f32")
    ga, gb = nv.quantize(dev_f32(d["a"])), nv.quantize(dev_f32(d["w"]))
    oa, ob = oracle.quantize(d["a"]), oracle.quantize(d["w"])
    torch.cuda.synchronize()
    assert_q_exact(ga, oa, "A")
    assert_q_exact(gb, ob, "W")
    c = nv.gemm(ga, gb, out_dtype=torch.float32).cpu().numpy()
    cref, bound = oracle.gemm_ref(oa, ob)
    assert_gemm_close(c, cref, bound, False, "workload 1")


def test_attn_proj_full(nv):
    d = workloads.attn_proj()
    log("workload 2: X bf16 2640x3072 (act-quant) @ W 3072x3072 -> bf16")
    gw = nv.quantize(dev_f32(d["w"]))
    y = nv.linear(dev_bf16(d["x"]), gw)
    ox, ow = oracle.quantize(widen(d["x"])), oracle.quantize(d["w"])
    cref, bound = oracle.gemm_ref(ox, ow)
    assert_gemm_close(y.float().cpu().numpy(), cref, bound, True, "workload 2")


def _ffn_stagewise(nv, m, dmodel, f, seed):
    """FFN pair stage by stage; every expected value is the oracle's own."""
    d = workloads.ffn(m=m, d=dmodel, f=f, seed=seed)
    xd = dev_bf16(d["x"])
    gw1, gw2 = nv.quantize(dev_f32(d["w1"])), nv.quantize(dev_f32(d["w2"]))
    ox = oracle.quantize(widen(d["x"]))
    ow1, ow2 = oracle.quantize(d["w1"]), oracle.quantize(d["w2"])
    gx = nv.quantize(xd)
    torch.cuda.synchronize()
    assert_q_exact(gx, ox, "X")
    assert_q_exact(gw1, ow1, "W1")
    assert_q_exact(gw2, ow2, "W2")
    rows = np.unique(np.concatenate([[0, m - 1], np.random.default_rng(seed).integers(0, m, 48)]))
    c1, _ = oracle.gemm_ref(ox, ow1, want_bound=False)     # all rows: H needs them
    _, b1 = oracle.gemm_ref(ox, ow1, rows=rows)
    # (i) GEMM1 alone, float32 out
    g1 = nv.gemm(gx, gw1, out_dtype=torch.float32)
    assert_gemm_close(g1.cpu().numpy()[rows], c1[rows], b1, False, "GEMM1")
    del g1
    # (ii) GEMM1 with the GELU epilogue and its amax
    hmax = torch.empty(1, device="cuda")
    h = nv.gemm(gx, gw1, out_dtype=torch.float32, epilogue=nv.EPI_GELU_TANH, amax_out=hmax)
    g = oracle.gelu_tanh(c1[rows])
    hh = h.cpu().numpy()
    tol = 1.13 * 1e-5 * b1 + 8 * np.spacing(np.abs(g).astype(np.float32)).astype(np.float64) + 1e-37
    assert np.all(np.abs(hh[rows] - g) <= tol)
    assert hmax.item() == float(np.abs(hh).max())
    # (iii) re-quantization of H: the GPU encoder on the oracle's float32 H
    # must reproduce the oracle's codes exactly
    h32 = oracle.gelu_tanh(c1).astype(np.float32)
    oh = oracle.quantize(h32)
    gh = nv.quantize(dev_f32(h32))
    torch.cuda.synchronize()
    assert_q_exact(gh, oh, "H requant")
    # (iv) GEMM2 on the oracle's H codes
    c2, b2 = oracle.gemm_ref(oh, ow2, rows=rows)
    y2 = nv.gemm(gh, gw2, out_dtype=torch.bfloat16)
    assert_gemm_close(y2.float().cpu().numpy()[rows], c2, b2, True, "GEMM2")
    # (v) the fused GPU chain against the full-oracle chain (reported; code
    # flips at rounding boundaries are expected, so only a loose bound)
    y = nv.ffn(xd, gw1, gw2).float().cpu().numpy()
    rel = np.linalg.norm(y[rows] - c2) / np.linalg.norm(c2)
    log(f"FFN chain relative Frobenius error vs full oracle: {rel:.3e}")
    assert rel < 1e-2
    # the GPU amax drives the same tensor scale the oracle derives from its H
    ts_gpu = np.float32(hmax.item()) / np.float32(2688.0)
    assert abs(float(ts_gpu) - float(oh.tscale[0])) <= 1e-5 * float(oh.tscale[0])


def test_ffn_pair_reduced(nv):
    log("workload 3 (reduced M): FFN 1056 x 3072 -> 14336 -> 3072")
    _ffn_stagewise(nv, 1056, 3072, 14336, 1103)


@pytest.mark.timeout(900)
def test_ffn_pair_full(nv):
    log("workload 3 (full): FFN 10560 x 3072 -> 14336 -> 3072")
    _ffn_stagewise(nv, 10560, 3072, 14336, 1003)


@pytest.mark.timeout(600)
def test_wgrad_after_rht_full(nv):
    d = workloads.rht_wgrad()
    log("workload 5: RHT16 both operands along dim 0, GEMM 3072x3072x16384 -> f32")
    gg = nv.rht16_quantize(dev_bf16(d["g"]), d["mask"], axis=0)
    gx = nv.rht16_quantize(dev_bf16(d["x"]), d["mask"], axis=0)
    og = oracle.rht16_quantize(widen(d["g"]), d["mask"], axis=0)
    ox = oracle.rht16_quantize(widen(d["x"]), d["mask"], axis=0)
    torch.cuda.synchronize()
    assert_q_exact(gg, og, "G")
    assert_q_exact(gx, ox, "X")
    c = nv.gemm(gg, gx, out_dtype=torch.float32).cpu().numpy()
    rows = np.unique(np.concatenate([[0, 3071], np.random.default_rng(5).integers(0, 3072, 64)]))
    cref, bound = oracle.gemm_ref(og, ox, rows=rows)
    assert_gemm_close(c[rows], cref, bound, False, "workload 5")


@pytest.mark.timeout(600)
def test_train_linear_triple_full(nv):
    """Workload 6 (the training slice of the attention projection): forward,
    input gradient and weight gradient, every operand bit-exact against the
    oracle's quantizers and every GEMM within the parity bound on sampled rows."""
    d = workloads.train_linear()
    log("workload 6: training triple of a 2640x3072x3072 linear layer")
    x, w, dy = dev_bf16(d["x"]), dev_f32(d["w"]), dev_bf16(d["dy"])
    y, dx, dw = nv.linear_train(x, w, dy, d["mask"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    rows = {"m": np.unique(np.concatenate([[0, 2639], rng.integers(0, 2640, 40)])),
            "n": np.unique(np.concatenate([[0, 3071], rng.integers(0, 3072, 40)]))}
    r = oracle.linear_train_ref(widen(d["x"]), d["w"], widen(d["dy"]), d["mask"], rows=rows)
    # the quantized operands, recomputed through the same entry points
    assert_q_exact(nv.quantize(x), r["xq"], "X")
    assert_q_exact(nv.quantize(w), r["wq"], "W")
    assert_q_exact(nv.quantize(dy), r["dyq"], "dY")
    assert_q_exact(nv.quantize(w, axis=0), r["wtq"], "W along dim 0")
    assert_q_exact(nv.rht16_quantize(dy, d["mask"], axis=0), r["dyt"], "RHT dY along dim 0")
    assert_q_exact(nv.rht16_quantize(x, d["mask"], axis=0), r["xt"], "RHT X along dim 0")
    # the padded operands linear_train feeds the weight-gradient GEMM (M = 2640
    # padded to 2688): the oracle's bytes, then zero codes and zero scales
    for src, want, tag in ((dy, r["dyt"], "dY"), (x, r["xt"], "X")):
        gp = nv.rht16_quantize(src, d["mask"], axis=0, k_pad=2688)
        codes, scales = gp.codes.cpu().numpy(), gp.scales.cpu().numpy()
        assert np.array_equal(codes[:, :1320], want.codes) and not codes[:, 1320:].any(), tag
        assert np.array_equal(scales[:, :165], want.scales) and not scales[:, 165:].any(), tag
        assert gp.tscale.cpu().numpy()[0] == want.tscale[0], tag
    assert_gemm_close(y.float().cpu().numpy()[rows["m"]], r["y"], r["by"], True, "forward")
    assert_gemm_close(dx.float().cpu().numpy()[rows["m"]], r["dx"], r["bdx"], True, "input gradient")
    assert_gemm_close(dw.cpu().numpy()[rows["n"]], r["dw"], r["bdw"], False, "weight gradient")

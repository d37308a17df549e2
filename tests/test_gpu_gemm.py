"""GPU parity of the block-scaled W4A4 GEMM against the float64 oracle:
|gpu - C| <= 1e-5 * sum_k |P_A P_B| per element (plus half a bf16 ulp for bf16
outputs).  Operand codes are first checked bit-exact against the oracle's own
quantization, so both sides multiply the same NVFP4 numbers.  Covers ragged
M/N/K tails (the K-checked path and the pipelined path for K >= 512,
K % 256 == 0, with K / 128 both a multiple of 4 and not), fp32/bf16
outputs, the GELU epilogue with its amax reduction, and the workload shapes
(tiny linear, attention projection, FFN pair stage by stage, weight-gradient
GEMM after the RHT, the training triple) at full size, where every output row
is compared (the float64 bound is computed in row chunks to cap host
memory)."""

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


@pytest.mark.parametrize("tiles", [(2, 4), (4, 2), (3, 3), (4, 4), (1, 1)])
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
    outs = [nv.gemm(ga, gb, out_dtype=torch.float32, tiles=t).cpu().numpy()
            for t in (None, (2, 4), (4, 2), (3, 3), (4, 4), (1, 1))]
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))
    cref, bound = oracle.gemm_ref(oracle.quantize(a), oracle.quantize(b))
    assert_gemm_close(outs[0], cref, bound, False, "tile identity")
    assert np.any(outs[0] != cref.astype(np.float32))  # the float32 accumulation rounded somewhere


def test_split_last_tile_row(nv):
    """2144 x 8192 (K = 512): the automatic choice (128 x 256 tiles) would leave a last
    tile row of 96 rows that costs a third round of workgroups, so the 2048
    full tile rows and the 96 remaining rows run as two launches (the second
    with 64 x 64 tiles).  The result is bit-identical to one launch with
    pinned tiles, float32 and the bf16 GELU epilogue with its amax alike, and
    the rows on both sides of the seam match the float64 oracle."""
    m, n, k = 2144, 8192, 512
    log(f"gemm split of the last tile row {m}x{n}x{k}")
    rng = np.random.default_rng(2144)
    ga, gb, oa, ob = _operands(nv, rng, m, n, k)
    auto = nv.gemm(ga, gb, out_dtype=torch.float32).cpu().numpy()
    pinned = nv.gemm(ga, gb, out_dtype=torch.float32, tiles=(2, 4)).cpu().numpy()
    assert np.array_equal(auto.view(np.uint32), pinned.view(np.uint32))
    amax_a, amax_p = torch.empty(1, device="cuda"), torch.empty(1, device="cuda")
    ha = nv.gemm(ga, gb, out_dtype=torch.bfloat16, epilogue=nv.EPI_GELU_TANH, amax_out=amax_a)
    hp = nv.gemm(ga, gb, out_dtype=torch.bfloat16, epilogue=nv.EPI_GELU_TANH, amax_out=amax_p, tiles=(2, 4))
    assert torch.equal(ha.view(torch.int16), hp.view(torch.int16))
    assert amax_a.item() == amax_p.item() == float(ha.float().abs().max().item())
    rows = slice(1984, m)
    cref, bound = oracle.gemm_ref(oa, ob, rows=rows)
    assert_gemm_close(auto[rows], cref, bound, False, "rows at the seam")


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
@pytest.mark.parametrize("tiles", [(2, 4), (4, 2), (4, 4), (1, 1)])
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


@pytest.mark.parametrize("tiles", [(4, 4), (2, 4)])
def test_whole_tile_instances_match_edge_instances(nv, tiles):
    """Kernel instances without the branch between two epilogue paths: the
    4x4 float32-output kernels for launches of whole tiles, and the staged
    bf16 kernels (2x4, 4x4) for whole tiles and, with row and column checks,
    for edge tiles when ldc % 8 == 0 and N % 8 == 0.  Each is bit-identical
    to the general instance on the same rows (plain and with the GELU
    epilogue and its amax): a launch with one extra A row has a ragged tile
    row, and a bf16 output with a row pitch of n + 4 takes the general
    instance.  The whole-tile result also meets the float64 oracle."""
    m, n, k = 512, 768, 1024
    log(f"gemm whole-tile and edge instances {m}x{n}x{k}, tiles {tiles}")
    rng = np.random.default_rng(512768)
    ga, gb, oa, ob = _operands(nv, rng, m + 1, n, k)   # one extra A row: the ragged launch
    whole = nv.NVFP4Tensor(ga.codes[:m], ga.scales[:m], ga.tscale)
    for epi in (nv.EPI_NONE, nv.EPI_GELU_TANH):
        amax_w, amax_r = torch.empty(1, device="cuda"), torch.empty(1, device="cuda")
        cw = nv.gemm(whole, gb, out_dtype=torch.float32, epilogue=epi, amax_out=amax_w, tiles=tiles)
        cr = nv.gemm(ga, gb, out_dtype=torch.float32, epilogue=epi, amax_out=amax_r, tiles=tiles)
        assert torch.equal(cw.view(torch.int32), cr[:m].view(torch.int32)), epi
        assert amax_w.item() == float(cw.abs().max().item())
        # bf16: whole tiles (no checks), edge tiles (checked staged stores),
        # and the general instance through a row pitch that is not a multiple of 8
        amax_s = torch.empty(1, device="cuda")
        hw = nv.gemm(whole, gb, out_dtype=torch.bfloat16, epilogue=epi, amax_out=amax_w, tiles=tiles)
        hr = nv.gemm(ga, gb, out_dtype=torch.bfloat16, epilogue=epi, amax_out=amax_r, tiles=tiles)
        big = torch.full((m + 1, n + 4), 7.0, dtype=torch.bfloat16, device="cuda")
        nv.gemm(ga, gb, out=big[:, :n], epilogue=epi, amax_out=amax_s, tiles=tiles)
        assert torch.equal(hr.view(torch.int16), big[:, :n].view(torch.int16)), epi
        assert torch.equal(hw.view(torch.int16), hr[:m].view(torch.int16)), epi
        assert bool((big[:, n:] == 7.0).all())
        assert amax_r.item() == amax_s.item() == float(hr.float().abs().max().item())
    cref, bound = oracle.gemm_ref(oa, ob, rows=slice(0, m))
    cw = nv.gemm(whole, gb, out_dtype=torch.float32, tiles=tiles)
    assert_gemm_close(cw.cpu().numpy(), cref, bound, False, "whole tiles")


# ---------------------------------------------------------------- workloads
def _all_rows_close(gpu, oa, ob, out_bf16, tag, chunk=2048, keep=False):
    """Every row of a GPU GEMM result against gemm_ref, the float64 result
    and its bound computed `chunk` rows at a time.  Returns the largest
    err / bound and, with ``keep``, the float64 oracle result."""
    m = gpu.shape[0]
    worst, parts = 0.0, []
    for r0 in range(0, m, chunk):
        rows = slice(r0, min(m, r0 + chunk))
        cref, bound = oracle.gemm_ref(oa, ob, rows=rows)
        worst = max(worst, assert_gemm_close(gpu[rows], cref, bound, out_bf16, f"{tag} rows {r0}+"))
        if keep:
            parts.append(cref)
    log(f"  {tag}: all {m} rows within bound, max err/bound {worst:.3e}")
    return worst, (np.concatenate(parts) if keep else None)


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
    # the one-call linear layer leaves the same activation codes and output
    xq = nv.NVFP4Tensor.empty(256, 512, 1, "cuda")
    c1 = nv.linear(dev_f32(d["a"]), gb, out_dtype=torch.float32, xq=xq).cpu().numpy()
    assert_q_exact(xq, oa, "A (nvfp4_linear)")
    assert np.array_equal(c1.view(np.uint32), c.view(np.uint32))


@pytest.mark.parametrize("m,n,k,xdt,odt,epi", [(17, 33, 48, "bf16", "f32", 0), (255, 130, 512, "f32", "bf16", 1),
                                                (129, 257, 384, "bf16", "bf16", 1), (300, 520, 1024, "f32", "f32", 1)])
def test_linear_equals_quantize_then_gemm(nv, m, n, k, xdt, odt, epi):
    """nvfp4_linear (one call) gives bit for bit the codes, output and
    output amax of nvfp4_quantize followed by nvfp4_gemm; the second call
    reuses the same buffers, so stale contents would show."""
    log(f"linear {m}x{n}x{k} x {xdt} -> {odt} epilogue {epi}")
    rng = np.random.default_rng(m + 7 * n + 11 * k)
    x = (rng.standard_normal((m, k)) * 3).astype(np.float32)
    gx = dev_f32(x) if xdt == "f32" else dev_f32(x).to(torch.bfloat16)
    gw = nv.quantize(dev_f32((rng.standard_normal((n, k)) * 0.05).astype(np.float32)))
    dt = torch.float32 if odt == "f32" else torch.bfloat16
    want_q = nv.quantize(gx)
    want_amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    want = nv.gemm(want_q, gw, out_dtype=dt, epilogue=epi, amax_out=want_amax)
    xq = nv.NVFP4Tensor.empty(m, k, 1, "cuda")
    out = torch.empty((m, n), dtype=dt, device="cuda")
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    for _ in range(2):
        nv.linear(gx, gw, xq=xq, out=out, epilogue=epi, amax_out=amax)
        torch.cuda.synchronize()
        assert torch.equal(xq.codes, want_q.codes) and torch.equal(xq.scales, want_q.scales)
        assert torch.equal(xq.tscale, want_q.tscale)
        assert torch.equal(out.view(torch.int16 if odt == "bf16" else torch.int32),
                           want.view(torch.int16 if odt == "bf16" else torch.int32))
        assert torch.equal(amax, want_amax)


def test_attn_proj_full(nv):
    d = workloads.attn_proj()
    log("workload 2: X bf16 2640x3072 (act-quant) @ W 3072x3072 -> bf16")
    gw = nv.quantize(dev_f32(d["w"]))
    xq = nv.NVFP4Tensor.empty(2640, 3072, 1, "cuda")
    y = nv.linear(dev_bf16(d["x"]), gw, xq=xq)
    ox, ow = oracle.quantize(widen(d["x"])), oracle.quantize(d["w"])
    torch.cuda.synchronize()
    assert_q_exact(xq, ox, "X (the linear layer's own activation operand)")
    assert_q_exact(gw, ow, "W")
    _all_rows_close(y.float().cpu().numpy(), ox, ow, True, "workload 2")


def _gelu_check(h, pre, tag):
    """Stage (ii) of the FFN chain: the GELU-tanh epilogue (float32 H of the
    fused GEMM1) against the float64 GELU of the GPU's own float32 GEMM1
    output `pre` (same accumulation, same tensor scales; no epilogue), all
    elements, in row chunks.

    Tolerance in float32 ulps of the result: 4, plus the conditioning of the
    float32 exponent argument.  The kernel evaluates
    g = h / (1 + 2^w), w = -2 sqrt(2/pi) log2(e) (h + 0.044715 h^3), in
    float32: w carries a relative rounding error of a few 2^-24 (constants,
    cube, sum, product), which moves 2^w by ln2 |w| times that and g by the
    share e/(1+e) of it (e = 2^w).  For h > 0 (e small) this vanishes; in the
    negative tail, where g ~ h 2^-w underflows towards 0, it grows with |w|
    for any float32 evaluation of the argument.  So the bound is
    (4 + 5 |w| e/(1+e)) ulp(g), plus |h| 2^-126: where 1 + e exceeds 2^126
    the hardware reciprocal flushes its would-be-subnormal result, so the
    epilogue returns -0 for |g| < |h| 2^-126 (err/tol then approaches 1 at
    that boundary, by construction).  Observed: at most ~2.5 ulp where the
    argument's conditioning is negligible."""
    kw = -2.0 * np.sqrt(2.0 / np.pi) * np.log2(np.e)
    worst_flat, worst = 0.0, 0.0
    for r0 in range(0, h.shape[0], 1024):
        hh = h[r0:r0 + 1024].astype(np.float64)
        x = pre[r0:r0 + 1024].astype(np.float64)
        g = oracle.gelu_tanh(x)
        w = kw * (x + 0.044715 * x ** 3)
        with np.errstate(over="ignore"):
            share = 1.0 / (1.0 + np.exp2(-w))   # e / (1 + e), e = 2^w
        ulp = np.spacing(np.abs(g).astype(np.float32)).astype(np.float64)
        err = np.abs(hh - g) / ulp
        tol = 4.0 + 5.0 * np.abs(w) * share + np.abs(x) * 2.0 ** -126 / ulp
        bad = np.argwhere(err > tol)
        if bad.size:
            i = tuple(bad[0])
            raise AssertionError(f"{tag}: {len(bad)} GELU outputs outside tolerance; first row {r0 + i[0]}: "
                                 f"pre {x[i]!r} gpu {hh[i]!r} ref {g[i]!r} err {err[i]:.2f} ulp tol {tol[i]:.2f}")
        flat = np.abs(w) * share < 0.05      # well-conditioned part
        if flat.any():
            worst_flat = max(worst_flat, float(err[flat].max()))
        worst = max(worst, float((err / tol).max()))
    log(f"  {tag}: max GELU error {worst_flat:.2f} ulp where well conditioned; max err/tol {worst:.3f}")


def _ffn_stagewise(nv, m, dmodel, f, seed):
    """FFN pair stage by stage, every output compared; every expected value
    is the oracle's own, fed the GPU's intermediate where the stage says so:
    (i) GEMM1 (float32) within the GEMM bound; (ii) the GELU epilogue against
    float64 GELU of the GPU's GEMM1 output, and its amax equal to max|H|;
    (iii) the re-quantization of the GPU's own H with the epilogue's amax,
    bit-exact against the oracle quantizer fed that H and amax; (iv) GEMM2
    on those codes within the GEMM bound; (v) the fused ffn() equal to the
    staged result bit for bit, and its distance to the full-oracle chain
    reported (rounding-boundary code flips are expected there).
    (i) and (ii) together bound |H - gelu(C1_oracle)| by the stage-(ii)
    tolerance plus 1.13 (max |gelu'|) times the GEMM bound."""
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
    # (i) GEMM1 alone, float32 out, every row
    g1 = nv.gemm(gx, gw1, out_dtype=torch.float32).cpu().numpy()
    _, c1 = _all_rows_close(g1, ox, ow1, False, "GEMM1", keep=True)
    # (ii) GEMM1 with the GELU epilogue and its amax
    hmax = torch.empty(1, device="cuda")
    h = nv.gemm(gx, gw1, out_dtype=torch.float32, epilogue=nv.EPI_GELU_TANH, amax_out=hmax)
    hh = h.cpu().numpy()
    _gelu_check(hh, g1, "GELU epilogue")
    del g1
    hm = np.float32(hmax.item())
    assert hm == oracle.amax(hh)
    # (iii) re-quantization of the GPU's own H with the epilogue's amax
    gh = nv.encode(h, hmax)
    oh = oracle.quantize_with_amax(hh, hm)
    torch.cuda.synchronize()
    assert_q_exact(gh, oh, "H requant (GPU H, GPU amax)")
    # (iv) GEMM2 on those codes, every row
    y2 = nv.gemm(gh, gw2, out_dtype=torch.bfloat16)
    y2h = y2.float().cpu().numpy()
    _all_rows_close(y2h, oh, ow2, True, "GEMM2")
    del oh, hh
    # (v) the fused chain is the staged chain; distance to the full oracle
    y = nv.ffn(xd, gw1, gw2)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "fused ffn() differs from its stages"
    rows = np.unique(np.concatenate([[0, m - 1], np.random.default_rng(seed).integers(0, m, 48)]))
    oh_chain = oracle.quantize(oracle.gelu_tanh(c1).astype(np.float32))
    c2, _ = oracle.gemm_ref(oh_chain, ow2, rows=rows, want_bound=False)
    rel = np.linalg.norm(y2h[rows] - c2) / np.linalg.norm(c2)
    log(f"  FFN chain relative Frobenius error vs full oracle chain: {rel:.3e}")
    assert rel < 1e-2


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
    _all_rows_close(c, og, ox, False, "workload 5", chunk=1024)


def _padded_equal(gq, want, k_pad, tag):
    """An axis-0 operand zero-padded along K to k_pad: the oracle's bytes,
    then zero codes and zero scales."""
    codes, scales = gq.codes.cpu().numpy(), gq.scales.cpu().numpy()
    kc, ks = want.codes.shape[1], want.scales.shape[1]
    assert codes.shape == (want.codes.shape[0], k_pad // 2), tag
    assert np.array_equal(codes[:, :kc], want.codes) and not codes[:, kc:].any(), tag
    assert np.array_equal(scales[:, :ks], want.scales) and not scales[:, ks:].any(), tag
    assert gq.tscale.cpu().numpy()[0] == want.tscale[0], tag


@pytest.mark.timeout(600)
def test_linear_train_streams_match_one_stream(nv):
    """linear_train issues its three chains on three streams; three calls on
    different inputs, back to back into the same buffers with no
    synchronization between them, give results bit-identical to the same
    C-ABI calls issued one after another on one stream."""
    m, n, k, mask = 640, 512, 768, 0x5A3C
    log(f"linear_train on three streams {m}x{n}x{k}, three calls back to back")
    mp = -(-m // 256) * 256
    bufs = {"xq": nv.NVFP4Tensor.empty(m, k), "wq": nv.NVFP4Tensor.empty(n, k), "dyq": nv.NVFP4Tensor.empty(m, n),
            "wtq": nv.NVFP4Tensor.empty(k, n), "dyt": nv.NVFP4Tensor.empty(n, mp), "xt": nv.NVFP4Tensor.empty(k, mp),
            "y": torch.empty((m, n), dtype=torch.bfloat16, device="cuda"),
            "dx": torch.empty((m, k), dtype=torch.bfloat16, device="cuda"),
            "dw": torch.empty((n, k), dtype=torch.float32, device="cuda"),
            "wamax": torch.empty(1, dtype=torch.float32, device="cuda")}
    for nm in ("ws", "ws1", "ws2"):
        bufs[nm] = nv._workspace(nv.OP_RHT16, m, max(k, n), "cuda")
    inputs, outs = [], []
    for i in range(3):
        d = workloads.train_linear(m=m, n=n, k=k, seed=300 + i)
        x, w, dy = dev_bf16(d["x"]), dev_f32(d["w"]), dev_bf16(d["dy"])
        inputs.append((x, w, dy))
        y, dx, dw = nv.linear_train(x, w, dy, mask, bufs=bufs)
        outs.append((y.clone(), dx.clone(), dw.clone(), bufs["dyt"].codes.clone(), bufs["xt"].codes.clone()))
    torch.cuda.synchronize()
    for i, (x, w, dy) in enumerate(inputs):
        xq = nv.quantize(x)
        wamax = nv.amax(w)
        wq, wtq = nv.encode(w, wamax, axis=1), nv.encode(w, wamax, axis=0)
        dyq = nv.quantize(dy)
        dyt = nv.rht16_quantize(dy, mask, axis=0, k_pad=mp)
        xt = nv.rht16_quantize(x, mask, axis=0, k_pad=mp)
        ref = (nv.gemm(xq, wq), nv.gemm(dyq, wtq), nv.gemm(dyt, xt, out_dtype=torch.float32), dyt.codes, xt.codes)
        torch.cuda.synchronize()
        for got, want, nm in zip(outs[i], ref, ("y", "dx", "dw", "dyt codes", "xt codes")):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), (i, nm)


def test_train_linear_triple_full(nv):
    """Workload 6 (the training slice of the attention projection): forward,
    input gradient and weight gradient.  The six operands linear_train
    itself built (passed in as buffers) are compared with the oracle's
    quantizers byte for byte (the two RHT16 operands with their zero padding
    from M = 2640 to 2816), and every row of the three GEMMs is within the
    parity bound."""
    d = workloads.train_linear()
    log("workload 6: training triple of a 2640x3072x3072 linear layer")
    x, w, dy = dev_bf16(d["x"]), dev_f32(d["w"]), dev_bf16(d["dy"])
    m, k, n, mp = 2640, 3072, 3072, 2816
    bufs = {"xq": nv.NVFP4Tensor.empty(m, k), "wq": nv.NVFP4Tensor.empty(n, k), "dyq": nv.NVFP4Tensor.empty(m, n),
            "wtq": nv.NVFP4Tensor.empty(k, n), "dyt": nv.NVFP4Tensor.empty(n, mp), "xt": nv.NVFP4Tensor.empty(k, mp)}
    y, dx, dw = nv.linear_train(x, w, dy, d["mask"], bufs=bufs)
    torch.cuda.synchronize()
    r = oracle.linear_train_ref(widen(d["x"]), d["w"], widen(d["dy"]), d["mask"])
    assert_q_exact(bufs["xq"], r["xq"], "X")
    assert_q_exact(bufs["wq"], r["wq"], "W")
    assert_q_exact(bufs["dyq"], r["dyq"], "dY")
    assert_q_exact(bufs["wtq"], r["wtq"], "W along dim 0")
    _padded_equal(bufs["dyt"], r["dyt"], mp, "RHT dY along dim 0, padded")
    _padded_equal(bufs["xt"], r["xt"], mp, "RHT X along dim 0, padded")
    for gpu, c, b, bf, tag in ((y, r["y"], r["by"], True, "forward"), (dx, r["dx"], r["bdx"], True, "input gradient"),
                               (dw, r["dw"], r["bdw"], False, "weight gradient")):
        worst = assert_gemm_close(gpu.float().cpu().numpy(), c, b, bf, tag)
        log(f"  {tag}: all rows within bound, max err/bound {worst:.3e}")


@pytest.mark.parametrize("m,n,k,xdt,stride", [(1, 40, 16, "f32", 0), (1, 256, 512, "bf16", 0), (7, 33, 48, "bf16", 64),
                                              (130, 96, 272, "f32", 288)])
def test_linear_edges_against_oracle(nv, m, n, k, xdt, stride):
    """nvfp4_linear on a single row (its leading dimension is taken from the
    row length), K = 16 and other K below 512 (the bounds-checked GEMM path),
    and activations given as a strided view (ld > K): codes bit-exact and
    every output within the GEMM bound of the oracle."""
    log(f"linear edge {m}x{n}x{k} {xdt} ld {stride or k}")
    rng = np.random.default_rng(31 * m + n + k)
    a = (rng.standard_normal((m, k)) * 2).astype(np.float32)
    b = (rng.standard_normal((n, k)) * 0.05).astype(np.float32)
    full = np.zeros((m, stride), np.float32) if stride else a
    if stride:
        full[:, :k] = a
    xd = dev_f32(full)[:, :k] if stride else dev_f32(a)
    if xdt == "bf16":
        a = widen(workloads.to_bf16_bits(a))
        xd = xd.to(torch.bfloat16)
    gw = nv.quantize(dev_f32(b))
    xq = nv.NVFP4Tensor.empty(m, k, 1, "cuda")
    y = nv.linear(xd, gw, out_dtype=torch.float32, xq=xq)
    oa, ob = oracle.quantize(a), oracle.quantize(b)
    torch.cuda.synchronize()
    assert_q_exact(xq, oa, "linear's activation operand")
    assert_q_exact(gw, ob, "W")
    cref, bound = oracle.gemm_ref(oa, ob)
    assert_gemm_close(y.cpu().numpy(), cref, bound, False, f"linear {m}x{n}x{k}")

"""GPU parity of the codec entry points against the CPU oracle: codes, scale
bytes and tensor scales bit-exact; decode bit-exact.  Covers several tiles
and ragged tails, every dtype/axis, the hand-worked blocks, rounding ties,
zero/negative-zero/subnormal-scale edge cases, the KV frame-block codec and
the RHT, plus the full-size workload tensors."""

import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import (assert_q_exact, dev_bf16, dev_f32, host_bf16_bits, log, require_gpu, widen)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    return require_gpu()


def _rand(rng, rows, cols, spread=3.0, outlier=0.01):
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp(rng.uniform(-spread, spread, (rows, 1))).astype(np.float32)
    m = rng.random((rows, cols)) < outlier
    x[m] *= 30
    return x.astype(np.float32)


SHAPES = [(1, 16), (3, 48), (17, 256), (255, 512), (64, 3072), (130, 1040)]


@pytest.mark.parametrize("rows,cols", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_rows_matches_oracle(nv, rows, cols, dtype):
    log(f"quantize axis1 {dtype} {rows}x{cols}")
    rng = np.random.default_rng(rows * 7919 + cols)
    x = _rand(rng, rows, cols)
    if dtype == "bf16":
        bits = workloads.to_bf16_bits(x)
        xd, xh = dev_bf16(bits), widen(bits)
    else:
        xd, xh = dev_f32(x), x
    gq = nv.quantize(xd)
    torch.cuda.synchronize()
    assert_q_exact(gq, oracle.quantize(xh), f"{dtype} {rows}x{cols}")


@pytest.mark.parametrize("rows,cols,ld", [(37, 96, 120), (300, 1040, 1056), (1, 16, 24)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_rows_strided_input(nv, rows, cols, ld, dtype):
    """Axis 1 (blocks along the rows) from a view whose rows are ld > cols
    elements apart: quantize, the RHT16 variant and the separate amax/encode
    pair all read only the first cols of every row."""
    log(f"quantize axis1 strided {dtype} {rows}x{cols} ld {ld}")
    rng = np.random.default_rng(rows * 13 + ld)
    xp = _rand(rng, rows, ld)
    xp[:, cols:] = 1e30  # padding that would dominate any amax that read it
    if dtype == "bf16":
        bits = workloads.to_bf16_bits(xp)
        xd, xh = dev_bf16(bits)[:, :cols], np.ascontiguousarray(widen(bits)[:, :cols])
    else:
        xd, xh = dev_f32(xp)[:, :cols], np.ascontiguousarray(xp[:, :cols])
    assert rows == 1 or not xd.is_contiguous()
    gq = nv.quantize(xd)
    gr = nv.rht16_quantize(xd, 0x3C5A)
    a = nv.amax(xd)
    ge = nv.encode(xd, a)
    torch.cuda.synchronize()
    want = oracle.quantize(xh)
    assert_q_exact(gq, want, f"strided {dtype}")
    assert_q_exact(ge, want, f"strided amax+encode {dtype}")
    assert_q_exact(gr, oracle.rht16_quantize(xh, 0x3C5A), f"strided rht {dtype}")


@pytest.mark.parametrize("rows,cols", [(16, 16), (48, 33), (256, 130), (1040, 64)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_cols_matches_oracle(nv, rows, cols, dtype):
    log(f"quantize axis0 {dtype} {rows}x{cols}")
    rng = np.random.default_rng(rows * 31 + cols)
    x = _rand(rng, rows, cols)
    # keep rows 16-byte aligned: pad the leading dimension
    ld = -(-cols // 8) * 8
    xp = np.zeros((rows, ld), np.float32)
    xp[:, :cols] = x
    if dtype == "bf16":
        bits = workloads.to_bf16_bits(xp)
        xd, xh = dev_bf16(bits)[:, :cols], widen(bits)[:, :cols]
    else:
        xd, xh = dev_f32(xp)[:, :cols], xp[:, :cols]
    gq = nv.quantize(xd, axis=0)
    torch.cuda.synchronize()
    assert_q_exact(gq, oracle.quantize(np.ascontiguousarray(xh.T)), f"axis0 {dtype} {rows}x{cols}")


@pytest.mark.parametrize("rows,cols,ld,dtype", [(48, 8, 8, "bf16"), (32, 12, 12, "f32"), (64, 24, 24, "bf16"),
                                                (256, 130, 136, "f32"), (48, 33, 40, "bf16"), (16, 4, 4, "f32")])
def test_quantize_cols_amax_in_tail_column(nv, rows, cols, ld, dtype):
    """Axis 0 takes any column count, so the tensor amax must cover the
    columns past the last multiple of 16: the largest magnitude sits in the
    last column (also with fewer than 16 columns, and with rows stored
    contiguously, ld == cols)."""
    log(f"quantize axis0 tail-column amax {dtype} {rows}x{cols} ld {ld}")
    rng = np.random.default_rng(rows * 17 + cols)
    x = _rand(rng, rows, cols, spread=1.0, outlier=0.0)
    x[rows // 3, cols - 1] = -40.0 * np.abs(x).max()
    xp = np.zeros((rows, ld), np.float32)
    xp[:, :cols] = x
    if dtype == "bf16":
        bits = workloads.to_bf16_bits(xp)
        xd, xh = dev_bf16(bits)[:, :cols], widen(bits)[:, :cols]
    else:
        xd, xh = dev_f32(xp)[:, :cols], xp[:, :cols]
    assert (ld == cols) == xd.is_contiguous()
    gq = nv.quantize(xd, axis=0)
    torch.cuda.synchronize()
    want = oracle.quantize(np.ascontiguousarray(xh.T))
    assert want.tscale[0] == np.float32(np.abs(xh).max()) / np.float32(2688.0)
    assert_q_exact(gq, want, f"axis0 tail {dtype} {rows}x{cols}")


def test_hand_worked_blocks_on_gpu(nv, golden_dir):
    with open(os.path.join(golden_dir, "hand_blocks.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        x = np.array(case["x"], np.float32)[None, :]
        gq = nv.quantize(dev_f32(x))
        torch.cuda.synchronize()
        assert [f"{b:02X}" for b in gq.scales.cpu().numpy()[0]] == case["scales"], case["name"]
        assert [f"{b:02X}" for b in gq.codes.cpu().numpy()[0]] == case["codes_hex"], case["name"]
        assert gq.tscale.cpu().numpy()[0] == np.float32(case["tscale"])
        y = nv.dequantize(gq).cpu().numpy()[0]
        want = np.array(case["dequant"], np.float32)
        assert np.array_equal(y, want) and np.array_equal(np.signbit(y), np.signbit(want)), case["name"]


def test_rounding_ties_and_neighbours(nv):
    # S = 1 (amax 2688) and a 6.0 in every block make sigma = 1.0 and r = 1,
    # so every other element is encoded as itself: exercise each E2M1
    # threshold, its float32 neighbours and both signs.
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 6.0, 7.0], np.float32)
    vals = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(10))])
    vals = np.concatenate([vals, -vals, [0.0, -0.0, 1e-30, -1e-30]]).astype(np.float32)
    nblk = -(-vals.size // 15)
    x = np.zeros((nblk + 1, 16), np.float32)
    x[0, 0] = 2688.0
    x[1:, 0] = 6.0
    flat = x[1:, 1:].reshape(-1)
    flat[: vals.size] = vals
    x[1:, 1:] = flat.reshape(nblk, 15)
    x = x.reshape(1, -1)
    gq = nv.quantize(dev_f32(x))
    torch.cuda.synchronize()
    assert_q_exact(gq, oracle.quantize(x), "ties")


def test_edge_cases(nv):
    cases = {
        "zeros": np.zeros((4, 64), np.float32),
        "neg_zeros": -np.zeros((4, 64), np.float32),
        "one_outlier": np.where(np.arange(64 * 8).reshape(8, 64) == 77, 1e4, 1e-3).astype(np.float32),
        # blocks far below the amax get subnormal or zero E4M3 scales
        "subnormal_scales": (np.geomspace(1e-9, 1.0, 32 * 16, dtype=np.float64)
                             .reshape(32, 16) * np.where(np.arange(16) % 2, -1, 1)).astype(np.float32).reshape(2, 256),
        "huge_range": np.array([[1e30] + [1e-10] * 15 + [-3e29] + [2e-20] * 15], np.float32),
    }
    for name, x in cases.items():
        gq = nv.quantize(dev_f32(x))
        torch.cuda.synchronize()
        assert_q_exact(gq, oracle.quantize(x), name)
        y = nv.dequantize(gq).cpu().numpy()
        want = oracle.dequantize(oracle.quantize(x))
        assert np.array_equal(y.view(np.uint32), want.view(np.uint32)), name


def test_amax_and_encode_with_given_amax(nv):
    rng = np.random.default_rng(5)
    x = _rand(rng, 96, 160)
    xd = dev_f32(x)
    a = nv.amax(xd)
    torch.cuda.synchronize()
    assert a.cpu().numpy()[0] == oracle.amax(x)
    # a caller-supplied amax larger than the true one (e.g. carried over from
    # a previous step) is honoured as is
    big = torch.tensor([np.float32(oracle.amax(x)) * np.float32(3.5)], device="cuda")
    gq = nv.encode(xd, big)
    torch.cuda.synchronize()
    assert_q_exact(gq, oracle.codec.quantize_with_amax(x, np.float32(big.item())), "given amax")
    # per-domain amax over row groups
    a3 = nv.amax(xd, rows_per_domain=40)
    torch.cuda.synchronize()
    want = [oracle.amax(x[0:40]), oracle.amax(x[40:80]), oracle.amax(x[80:96])]
    assert np.array_equal(a3.cpu().numpy(), np.array(want, np.float32))


def test_row_domains_encode_and_dequantize(nv):
    """Row domains outside the KV layout: amax per 40-row group, encode with
    those maxima (one tensor scale per group), decode with the same groups;
    each group equals the oracle's quantization of that group on its own."""
    rng = np.random.default_rng(12)
    x = _rand(rng, 96, 160)
    xd = dev_f32(x)
    a3 = nv.amax(xd, rows_per_domain=40)
    gq = nv.encode(xd, a3, rows_per_domain=40)
    y = nv.dequantize(gq, torch.float32, rows_per_domain=40).cpu().numpy()
    torch.cuda.synchronize()
    codes, scales, ts = gq.codes.cpu().numpy(), gq.scales.cpu().numpy(), gq.tscale.cpu().numpy()
    for d, (r0, r1) in enumerate([(0, 40), (40, 80), (80, 96)]):
        oq = oracle.quantize(x[r0:r1])
        assert np.array_equal(codes[r0:r1], oq.codes) and np.array_equal(scales[r0:r1], oq.scales), d
        assert ts[d] == oq.tscale[0], d
        want = oracle.dequantize(oq, "f32")
        assert np.array_equal(y[r0:r1].view(np.uint32), want.view(np.uint32)), d


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dequantize_matches_oracle(nv, dtype):
    rng = np.random.default_rng(8)
    x = _rand(rng, 77, 320)
    gq = nv.quantize(dev_f32(x))
    oq = oracle.quantize(x)
    if dtype == "f32":
        y = nv.dequantize(gq, torch.float32).cpu().numpy()
        want = oracle.dequantize(oq, "f32")
        assert np.array_equal(y.view(np.uint32), want.view(np.uint32))
    else:
        y = host_bf16_bits(nv.dequantize(gq, torch.bfloat16))
        assert np.array_equal(y, oracle.dequantize(oq, "bf16"))


def test_repeat_runs_are_bit_identical(nv):
    rng = np.random.default_rng(9)
    xd = dev_f32(_rand(rng, 513, 1024))
    q1 = nv.quantize(xd)
    q2 = nv.quantize(xd)
    torch.cuda.synchronize()
    assert torch.equal(q1.codes, q2.codes) and torch.equal(q1.scales, q2.scales) and torch.equal(q1.tscale, q2.tscale)


@pytest.mark.parametrize("shape", [(12, 5, 3, 32), (9, 7, 2, 128), (3, 11, 4, 64), (17, 2, 1, 16)])
def test_kv_codec_small(nv, shape):
    f, t, h, d = shape
    log(f"kv codec {shape}")
    kv = workloads.kv_cache(frames=f, tokens=t, heads=h, head_dim=d, seed=40 + f)["k"]
    kd = dev_bf16(kv)
    gq = nv.kv_quant(kd)
    oq = oracle.kv_quantize(widen(kv))
    torch.cuda.synchronize()
    assert_q_exact(gq, oq, f"kv {shape}")
    y = host_bf16_bits(nv.kv_dequant(gq, shape))
    assert np.array_equal(y, oracle.kv_dequantize(oq, f, t, h, d))


@pytest.mark.parametrize("shape", [(12, 5, 3, 32), (9, 7, 2, 128), (17, 2, 1, 16), (3, 40, 4, 64)])
def test_kv_codec_four_over_six(nv, shape):
    f, t, h, d = shape
    log(f"kv codec Four Over Six {shape}")
    kv = workloads.kv_cache(frames=f, tokens=t, heads=h, head_dim=d, seed=90 + f)["v"]
    gq = nv.kv_quant(dev_bf16(kv), four_over_six=True)
    oq = oracle.kv_quantize_4over6(widen(kv))
    torch.cuda.synchronize()
    assert_q_exact(gq, oq, f"kv 4/6 {shape}")
    y = host_bf16_bits(nv.kv_dequant(gq, shape))
    assert np.array_equal(y, oracle.kv_dequantize(oq, f, t, h, d))


def test_four_over_six_hand_worked_blocks_on_gpu(nv, golden_dir):
    """The hand-worked Four Over Six blocks (tests/golden) through the KV
    entry point as one frame of one token and one head (head_dim 80)."""
    with open(os.path.join(golden_dir, "four_over_six_blocks.json")) as fh:
        g = json.load(fh)
    x = np.array(g["x"], np.float32)
    bits = host_bf16_bits(torch.from_numpy(x).to(torch.bfloat16))
    assert np.array_equal(widen(bits), x)  # every value is exact in bf16
    gq = nv.kv_quant(dev_bf16(bits.reshape(1, 1, 1, -1)), four_over_six=True)
    torch.cuda.synchronize()
    assert gq.tscale.cpu().numpy()[0] == np.float32(g["tscale"])
    assert [f"{b:02X}" for b in gq.scales.cpu().numpy()[0]] == g["scales"]
    assert [f"{b:02X}" for b in gq.codes.cpu().numpy()[0]] == g["codes_hex"]


@pytest.mark.parametrize("rows,cols", [(16, 16), (64, 48), (255, 512), (48, 1040)])
@pytest.mark.parametrize("axis", [1, 0])
def test_rht16_quantize_matches_oracle(nv, rows, cols, axis):
    if axis == 0:
        rows = -(-rows // 16) * 16
    log(f"rht16 axis{axis} {rows}x{cols}")
    rng = np.random.default_rng(rows + 3 * cols + axis)
    g = rng.laplace(0, 1e-3, (rows, cols)).astype(np.float32)
    g[rng.random(g.shape) < 0.01] *= 100
    ld = -(-cols // 8) * 8
    gp = np.zeros((rows, ld), np.float32)
    gp[:, :cols] = g
    bits = workloads.to_bf16_bits(gp)
    mask = int(np.random.default_rng(rows).integers(0, 2 ** 16))
    gq = nv.rht16_quantize(dev_bf16(bits)[:, :cols], mask, axis=axis)
    oq = oracle.rht16_quantize(widen(bits)[:, :cols], mask, axis=axis)
    torch.cuda.synchronize()
    assert_q_exact(gq, oq, f"rht axis{axis} {rows}x{cols}")


# ---------------------------------------------------------------- full size
def test_full_attn_proj_operands(nv):
    d = workloads.attn_proj()
    log("full-size workload 2 operands: X bf16 2640x3072, W f32 3072x3072")
    gx = nv.quantize(dev_bf16(d["x"]))
    gw = nv.quantize(dev_f32(d["w"]))
    torch.cuda.synchronize()
    assert_q_exact(gx, oracle.quantize(widen(d["x"])), "X")
    assert_q_exact(gw, oracle.quantize(d["w"]), "W")


@pytest.mark.parametrize("shape,fb", [((12, 5, 3, 32), 8), ((9, 7, 2, 128), 4), ((3, 11, 4, 64), 8),
                                      ((17, 2, 1, 16), 5), ((4, 40, 3, 128), 1), ((5, 1, 1, 16), 2)])
@pytest.mark.parametrize("fo6", [False, True])
def test_kv_quant_pair_small(nv, shape, fb, fo6):
    """K and V through nvfp4_kv_quant_pair (one amax and one encode launch for
    both) against the oracle: frame blocks with a partial last block, one
    block over the whole window (fb 8 > 3 frames), one frame per block."""
    f, t, h, d = shape
    log(f"kv quant pair {shape} frame_block {fb} four_over_six {fo6}")
    kv = workloads.kv_cache(frames=f, tokens=t, heads=h, head_dim=d, seed=140 + f)
    gk, gv = nv.kv_quant_pair(dev_bf16(kv["k"]), dev_bf16(kv["v"]), frame_block=fb, four_over_six=fo6)
    ref = oracle.kv_quantize_4over6 if fo6 else oracle.kv_quantize
    ok, ov = ref(widen(kv["k"]), frame_block=fb), ref(widen(kv["v"]), frame_block=fb)
    torch.cuda.synchronize()
    assert_q_exact(gk, ok, f"pair K {shape}")
    assert_q_exact(gv, ov, f"pair V {shape}")
    yk, yv = nv.kv_dequant_pair(gk, gv, shape, frame_block=fb)
    assert np.array_equal(host_bf16_bits(yk), oracle.kv_dequantize(ok, f, t, h, d, frame_block=fb))
    assert np.array_equal(host_bf16_bits(yv), oracle.kv_dequantize(ov, f, t, h, d, frame_block=fb))


def _full_kv(nv, fo6):
    d = workloads.kv_cache()
    shape = (12, 880, 24, 128)
    ref = oracle.kv_quantize_4over6 if fo6 else oracle.kv_quantize
    oq = {name: ref(widen(d[name]).reshape(shape)) for name in ("k", "v")}
    for name in ("k", "v"):
        log(f"full-size KV codec {name} {shape} four_over_six {fo6}")
        gq = nv.kv_quant(dev_bf16(d[name]), four_over_six=fo6)
        torch.cuda.synchronize()
        assert_q_exact(gq, oq[name], f"kv {name}")
        y = host_bf16_bits(nv.kv_dequant(gq, shape))
        assert np.array_equal(y, oracle.kv_dequantize(oq[name], *shape))
    # the pair entry point, as the bench times it
    log(f"full-size KV codec, K and V in one call, four_over_six {fo6}")
    gk, gv = nv.kv_quant_pair(dev_bf16(d["k"]), dev_bf16(d["v"]), four_over_six=fo6)
    torch.cuda.synchronize()
    assert_q_exact(gk, oq["k"], "pair K")
    assert_q_exact(gv, oq["v"], "pair V")
    yk, yv = nv.kv_dequant_pair(gk, gv, shape)
    assert np.array_equal(host_bf16_bits(yk), oracle.kv_dequantize(oq["k"], *shape))
    assert np.array_equal(host_bf16_bits(yv), oracle.kv_dequantize(oq["v"], *shape))


def test_full_kv_codec(nv):
    _full_kv(nv, False)


def test_full_kv_codec_four_over_six(nv):
    _full_kv(nv, True)


def test_full_rht_gradient(nv):
    d = workloads.rht_wgrad()
    log("full-size workload 5: RHT16 + quantize G bf16 16384x3072 along dim 0")
    gq = nv.rht16_quantize(dev_bf16(d["g"]), d["mask"], axis=0)
    oq = oracle.rht16_quantize(widen(d["g"]), d["mask"], axis=0)
    torch.cuda.synchronize()
    assert_q_exact(gq, oq, "rht G")



@pytest.mark.parametrize("rht", [False, True])
def test_workspace_shared_by_consecutive_calls(nv, rht):
    """Calls that reuse one workspace (stream-ordered) each see only their
    own partial maxima: the second call on different data is still exact."""
    rng = np.random.default_rng(61 + rht)
    mask = 0xA5C3
    ws = torch.empty((nv.workspace_bytes(nv.OP_QUANTIZE, 700, 3072) // 4,), dtype=torch.float32, device="cuda")
    for scale in (1.0, 1e-3):
        x = (_rand(rng, 700, 3072) * np.float32(scale)).astype(np.float32)
        bits = host_bf16_bits(torch.from_numpy(x).to(torch.bfloat16))
        want = oracle.rht16_quantize(widen(bits), mask) if rht else oracle.quantize(widen(bits))
        xd = dev_bf16(bits)
        log(f"shared workspace rht={rht} scale={scale}")
        gq = nv.rht16_quantize(xd, mask, ws=ws) if rht else nv.quantize(xd, ws=ws)
        torch.cuda.synchronize()
        assert_q_exact(gq, want, f"rht={rht} scale={scale}")

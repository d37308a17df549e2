"""nvfp4_quantize_noalloc (no workspace argument: the amax partials live in
the library's per-GPU scratch array) against nvfp4_quantize (caller-owned
workspace) on the same inputs, through the C ABI: codes, scale bytes and
tensor scale bit-identical, on consecutive calls where each later call is
smaller than the one before (the array keeps the previous call's partials),
for both block axes and both input dtypes, the column-pass amax included."""

import ctypes

import numpy as np
import pytest
import torch

import workloads
from gpu_helpers import assert_q_exact, dev_bf16, dev_f32, log, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    return require_gpu()


def _noalloc(nv, x, axis):
    rows, cols = x.shape
    r, k = (rows, cols) if axis == 1 else (cols, rows)
    out = nv.NVFP4Tensor.empty(r, k, 1, x.device)
    ct = out.c()
    st = nv.lib.nvfp4_quantize_noalloc(ctypes.c_void_p(x.data_ptr()), nv._dtype_code(x), rows, cols, nv._ld(x),
                                       axis, ctypes.byref(ct), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, nv.lib.nvfp4_status_string(st)
    return out


def _input(rng, rows, cols, dtype):
    x = (rng.standard_normal((rows, cols)) * np.exp(rng.uniform(-2, 2, (1, cols)))).astype(np.float32)
    x[rng.random(x.shape) < 0.005] *= 50
    return dev_bf16(workloads.to_bf16_bits(x)) if dtype == "bf16" else dev_f32(x)


# (rows, cols) of consecutive calls, each smaller than the last
SEQUENCES = [
    ("bf16", 1, [(2640, 3072), (96, 512), (16, 16)]),
    ("f32", 1, [(1040, 1040), (33, 48)]),
    ("f32", 0, [(512, 200), (64, 40)]),      # cols % 16 != 0: the column pass takes the amax
    ("bf16", 0, [(2688, 3072), (128, 64)]),
]


@pytest.mark.parametrize("dtype,axis,shapes", SEQUENCES)
def test_noalloc_matches_workspace_quantize(nv, dtype, axis, shapes):
    rng = np.random.default_rng(len(shapes) * 100 + axis * 10 + (dtype == "bf16"))
    for rows, cols in shapes:
        log(f"quantize_noalloc {dtype} axis {axis} {rows}x{cols}")
        x = _input(rng, rows, cols, dtype)
        got = _noalloc(nv, x, axis)
        want = nv.quantize(x, axis=axis)
        torch.cuda.synchronize()
        want_np = type("Q", (), {"codes": want.codes.cpu().numpy(), "scales": want.scales.cpu().numpy(),
                                 "tscale": want.tscale.cpu().numpy()})
        assert_q_exact(got, want_np, f"{dtype} axis {axis} {rows}x{cols}")


def test_noalloc_binding_into_given_output(nv):
    """The binding's quantize_noalloc writes into a caller-owned output (the
    allocation-free use) and matches nvfp4_quantize."""
    rng = np.random.default_rng(5)
    x = _input(rng, 300, 1024, "bf16")
    out = nv.NVFP4Tensor.empty(300, 1024, 1, "cuda")
    got = nv.quantize_noalloc(x, out=out)
    assert got is out
    want = nv.quantize(x)
    torch.cuda.synchronize()
    assert torch.equal(out.codes, want.codes) and torch.equal(out.scales, want.scales)
    assert torch.equal(out.tscale.view(torch.int32), want.tscale.view(torch.int32))

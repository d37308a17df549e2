"""Shared helpers of the GPU parity tests: host<->device transfer of seeded
inputs, NVFP4 result comparison and the GEMM tolerance of the parity bar.

Nothing here computes the method: expected values always come from
``oracle`` on the host; the GPU side always runs through the C ABI."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import nvfp4_w4a4_block_02_amd as nv  # raises if the HIP library is missing

    return nv


def dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).cuda()


def host_bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def widen(bits: np.ndarray) -> np.ndarray:
    """Exact bf16 -> float32 of an input (data plumbing, not the codec)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def assert_q_exact(gq, oq, tag: str = ""):
    """Codes, scale bytes and tensor scales bit-identical."""
    codes = gq.codes.cpu().numpy()
    scales = gq.scales.cpu().numpy()
    ts = gq.tscale.cpu().numpy()
    assert codes.shape == oq.codes.shape, (tag, codes.shape, oq.codes.shape)
    assert scales.shape == oq.scales.shape, (tag, scales.shape, oq.scales.shape)
    ts_o = np.asarray(oq.tscale, np.float32)
    assert np.array_equal(ts[: ts_o.size].view(np.uint32), ts_o.view(np.uint32)), (tag, ts, ts_o)
    bad_s = np.argwhere(scales != oq.scales)
    assert bad_s.size == 0, f"{tag}: {len(bad_s)} scale bytes differ, first {bad_s[:3].tolist()}"
    bad_c = np.argwhere(codes != oq.codes)
    assert bad_c.size == 0, f"{tag}: {len(bad_c)} code bytes differ, first {bad_c[:3].tolist()}"


def bf16_half_ulp(v: np.ndarray) -> np.ndarray:
    """Half a bf16 ulp at |v| (float64), for outputs rounded to bf16."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 8), 0.0)


def gemm_tolerance(bound: np.ndarray, c_ref: np.ndarray, out_bf16: bool) -> np.ndarray:
    """|gpu - C| <= 1e-5 * sum_k |a_k b_k| (fp64 oracle), plus half a bf16 ulp
    of the result when the output is rounded to bf16."""
    tol = 1e-5 * bound
    if out_bf16:
        tol = tol + bf16_half_ulp(np.abs(c_ref) + tol)
    return tol


def assert_gemm_close(gpu: np.ndarray, c_ref: np.ndarray, bound: np.ndarray, out_bf16: bool, tag: str = ""):
    gpu = np.asarray(gpu, np.float64)
    tol = gemm_tolerance(bound, c_ref, out_bf16)
    err = np.abs(gpu - c_ref)
    bad = np.argwhere(err > tol)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError(f"{tag}: {len(bad)} of {gpu.size} outside tolerance; first {i}: gpu {gpu[i]!r} "
                             f"ref {c_ref[i]!r} bound {bound[i]!r} err {err[i]!r} tol {tol[i]!r}")
    return float((err / np.maximum(bound, 1e-300)).max())

"""The C ABI library loads on a CPU-only machine, exports every entry point
include/nvfp4.h declares, and rejects bad arguments on the host before any
HIP call (no compute call is made here)."""

import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def nv():
    from nvfp4_w4a4_block_02_amd import build as b

    if not os.path.exists(b.LIB):
        b.build()
    import nvfp4_w4a4_block_02_amd as nv

    return nv


def _declared():
    with open(os.path.join(ROOT, "include", "nvfp4.h")) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char)\s*\*?\s*([a-z0-9_]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_exports_every_declared_symbol(nv):
    declared = _declared()
    assert len(declared) >= 11
    assert sorted(nv.EXPORTED) == declared
    for name in declared:
        assert hasattr(nv.lib, name), name


def test_missing_library_fails_loudly(nv, monkeypatch, tmp_path):
    monkeypatch.setattr(nv, "LIB_PATH", str(tmp_path / "libnvfp4.so"))
    with pytest.raises(ImportError, match="no non-HIP fallback"):
        nv._load()


def test_version_and_status_strings(nv):
    assert nv.lib.nvfp4_version() == 10000
    for code, text in [(0, b"ok"), (-1, b"invalid argument"), (-3, b"workspace too small"), (-4, b"HIP launch failed")]:
        assert nv.lib.nvfp4_status_string(code) == text
    assert nv.lib.nvfp4_status_string(123) == b"unknown status"


def test_workspace_sizes(nv):
    # 1024 partial maxima (4 KiB) per scaling domain
    assert nv.workspace_bytes(nv.OP_QUANTIZE, 10, 32) == 4096
    assert nv.workspace_bytes(nv.OP_RHT16, 10, 32) == 4096
    assert nv.workspace_bytes(nv.OP_GEMM, 10, 32) == 0
    assert nv.workspace_bytes(nv.OP_KV_QUANT, 12, 8) == 8192    # two frame blocks
    assert nv.workspace_bytes(nv.OP_KV_QUANT, 40, 8) == 20480   # five frame blocks
    assert nv.workspace_bytes(nv.OP_AMAX, 96, 40) == 12288      # three row domains


FAKE = 0x10000  # a 16-byte aligned address that is never dereferenced


def _t(nv, rows, k, codes=FAKE, scales=FAKE, tscale=FAKE):
    return nv._CTensor(codes, scales, tscale, rows, k)


def _stream():
    return ctypes.c_void_p(0)


def test_quantize_rejects_bad_arguments(nv):
    q = nv.lib.nvfp4_quantize
    ws = ctypes.c_void_p(FAKE)
    good = _t(nv, 4, 32)
    EINVAL, EWS = -1, -3
    # null input, bad dtype, k % 16, ld < cols, misaligned x, bad axis, shape mismatch
    assert q(None, 1, 4, 32, 32, 1, ctypes.byref(good), ws, 4096, _stream()) == EINVAL
    assert q(ctypes.c_void_p(FAKE), 7, 4, 32, 32, 1, ctypes.byref(good), ws, 4096, _stream()) == EINVAL
    assert q(ctypes.c_void_p(FAKE), 1, 4, 40, 40, 1, ctypes.byref(_t(nv, 4, 40)), ws, 4096, _stream()) == EINVAL
    assert q(ctypes.c_void_p(FAKE), 1, 4, 32, 16, 1, ctypes.byref(good), ws, 4096, _stream()) == EINVAL
    assert q(ctypes.c_void_p(FAKE + 2), 1, 4, 32, 32, 1, ctypes.byref(good), ws, 4096, _stream()) == EINVAL
    assert q(ctypes.c_void_p(FAKE), 1, 4, 32, 36, 1, ctypes.byref(good), ws, 4096, _stream()) == EINVAL  # row pitch
    assert q(ctypes.c_void_p(FAKE), 1, 4, 32, 32, 2, ctypes.byref(good), ws, 4096, _stream()) == EINVAL
    assert q(ctypes.c_void_p(FAKE), 1, 4, 32, 32, 1, ctypes.byref(_t(nv, 5, 32)), ws, 4096, _stream()) == EINVAL
    # axis 0 needs rows % 16 and a transposed output
    assert q(ctypes.c_void_p(FAKE), 1, 20, 32, 32, 0, ctypes.byref(_t(nv, 32, 20)), ws, 4096, _stream()) == EINVAL
    assert q(ctypes.c_void_p(FAKE), 1, 32, 48, 48, 0, ctypes.byref(_t(nv, 32, 48)), ws, 4096, _stream()) == EINVAL
    # null / misaligned output pointers
    assert q(ctypes.c_void_p(FAKE), 1, 4, 32, 32, 1, ctypes.byref(_t(nv, 4, 32, codes=0)), ws, 4096, _stream()) == EINVAL
    assert q(ctypes.c_void_p(FAKE), 1, 4, 32, 32, 1, ctypes.byref(_t(nv, 4, 32, scales=FAKE + 1)), ws, 4096, _stream()) == EINVAL
    # workspace
    assert q(ctypes.c_void_p(FAKE), 1, 4, 32, 32, 1, ctypes.byref(good), None, 16, _stream()) == EINVAL
    assert q(ctypes.c_void_p(FAKE), 1, 4, 32, 32, 1, ctypes.byref(good), ws, 8, _stream()) == EWS
    # zero-sized problems are a no-op (no launch)
    assert q(ctypes.c_void_p(FAKE), 1, 0, 32, 32, 1, ctypes.byref(_t(nv, 0, 32)), ws, 4096, _stream()) == 0
    assert q(ctypes.c_void_p(FAKE), 1, 4, 0, 0, 1, ctypes.byref(_t(nv, 4, 0)), ws, 4096, _stream()) == 0


def test_quantize_noalloc_rejects_bad_arguments(nv):
    """The no-workspace quantizer checks its arguments like nvfp4_quantize,
    on the host, before it touches HIP (no device needed here)."""
    q = nv.lib.nvfp4_quantize_noalloc
    good = _t(nv, 4, 32)
    EINVAL = -1
    assert q(None, 1, 4, 32, 32, 1, ctypes.byref(good), _stream()) == EINVAL
    assert q(ctypes.c_void_p(FAKE), 7, 4, 32, 32, 1, ctypes.byref(good), _stream()) == EINVAL
    assert q(ctypes.c_void_p(FAKE + 2), 1, 4, 32, 32, 1, ctypes.byref(good), _stream()) == EINVAL
    assert q(ctypes.c_void_p(FAKE), 1, 4, 32, 32, 2, ctypes.byref(good), _stream()) == EINVAL
    assert q(ctypes.c_void_p(FAKE), 1, 4, 32, 32, 1, ctypes.byref(_t(nv, 5, 32)), _stream()) == EINVAL
    assert q(ctypes.c_void_p(FAKE), 1, 20, 32, 32, 0, ctypes.byref(_t(nv, 32, 20)), _stream()) == EINVAL
    assert q(ctypes.c_void_p(FAKE), 1, 1 << 40, 1 << 40, 1 << 40, 1, ctypes.byref(_t(nv, 1 << 40, 1 << 40)),
             _stream()) == -2
    # zero-sized problems are a no-op
    assert q(ctypes.c_void_p(FAKE), 1, 0, 32, 32, 1, ctypes.byref(_t(nv, 0, 32)), _stream()) == 0


def test_rht_rejects_wide_mask(nv):
    good = _t(nv, 4, 32)
    st = nv.lib.rht16_quantize(ctypes.c_void_p(FAKE), 1, 4, 32, 32, 1, 1 << 16, ctypes.byref(good),
                               ctypes.c_void_p(FAKE), 4096, _stream())
    assert st == -1


def test_gemm_rejects_bad_arguments(nv):
    g = nv.lib.nvfp4_gemm
    a, b = _t(nv, 8, 64), _t(nv, 16, 64)
    c = ctypes.c_void_p(FAKE)
    assert g(ctypes.byref(a), ctypes.byref(_t(nv, 16, 48)), c, 0, 16, 0, None, None, 0, _stream()) == -1  # K mismatch
    assert g(ctypes.byref(a), ctypes.byref(b), c, 0, 8, 0, None, None, 0, _stream()) == -1  # ldc < N
    assert g(ctypes.byref(a), ctypes.byref(b), c, 5, 16, 0, None, None, 0, _stream()) == -1  # dtype
    assert g(ctypes.byref(a), ctypes.byref(b), c, 0, 16, 7, None, None, 0, _stream()) == -1  # epilogue
    assert g(ctypes.byref(a), ctypes.byref(b), None, 0, 16, 0, None, None, 0, _stream()) == -1
    assert g(ctypes.byref(a), ctypes.byref(b), c, 0, 16, 0, ctypes.c_void_p(FAKE + 2), None, 0, _stream()) == -1
    assert g(ctypes.byref(_t(nv, 8, 40)), ctypes.byref(_t(nv, 16, 40)), c, 0, 16, 0, None, None, 0, _stream()) == -1
    assert g(ctypes.byref(_t(nv, 0, 64)), ctypes.byref(b), c, 0, 16, 0, None, None, 0, _stream()) == 0
    gt = nv.lib.nvfp4_gemm_tiled
    assert gt(ctypes.byref(a), ctypes.byref(b), c, 0, 16, 0, None, 3, 4, _stream()) == -1  # unsupported tiles
    assert gt(ctypes.byref(a), ctypes.byref(b), c, 0, 8, 0, None, 2, 4, _stream()) == -1   # ldc < N
    assert gt(ctypes.byref(_t(nv, 0, 64)), ctypes.byref(b), c, 0, 16, 0, None, 4, 4, _stream()) == 0


def test_linear_rejects_bad_arguments_of_either_step(nv):
    """nvfp4_linear checks the quantize's and the GEMM's arguments before it
    launches anything: a bad GEMM argument is refused even though the
    quantize's are good (every call here would otherwise launch on memory
    that does not exist)."""
    lin = nv.lib.nvfp4_linear
    x, c, ws = ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE)
    xq, w = _t(nv, 8, 64), _t(nv, 16, 64)
    EINVAL, EWS = -1, -3

    def call(x=x, dt=1, rows=8, cols=64, ld=64, w=w, xq=xq, c=c, cdt=0, ldc=16, epi=0, amax=None, ws=ws,
             wsb=4096):
        return lin(x, dt, rows, cols, ld, ctypes.byref(w), ctypes.byref(xq), c, cdt, ldc, epi, amax, ws, wsb,
                   _stream())

    # quantize side
    assert call(x=None) == EINVAL
    assert call(dt=5) == EINVAL
    assert call(ld=32) == EINVAL
    assert call(xq=_t(nv, 9, 64)) == EINVAL        # xq rows != rows
    assert call(ws=None) == EINVAL
    assert call(wsb=8) == EWS
    # GEMM side, with a good quantize
    assert call(w=_t(nv, 16, 48)) == EINVAL        # K mismatch
    assert call(ldc=8) == EINVAL                   # ldc < N
    assert call(cdt=3) == EINVAL
    assert call(epi=9) == EINVAL
    assert call(c=None) == EINVAL
    assert call(amax=ctypes.c_void_p(FAKE + 2)) == EINVAL
    assert call(w=_t(nv, 16, 64, codes=FAKE + 1)) == EINVAL
    # zero rows: nothing to do (no amax_out to clear)
    assert call(rows=0, xq=_t(nv, 0, 64)) == 0


@pytest.mark.parametrize("entry", ["nvfp4_kv_quant", "nvfp4_kv_quant_4over6"])
def test_kv_rejects_bad_arguments(nv, entry):
    kq = getattr(nv.lib, entry)
    out = _t(nv, 12 * 4 * 2, 32)
    ws = ctypes.c_void_p(FAKE)
    assert kq(ctypes.c_void_p(FAKE), 12, 4, 2, 32, 0, ctypes.byref(out), ws, 8192, _stream()) == -1  # frame_block
    assert kq(ctypes.c_void_p(FAKE), 12, 4, 2, 24, 8, ctypes.byref(_t(nv, 96, 24)), ws, 8192, _stream()) == -1
    assert kq(ctypes.c_void_p(FAKE), 12, 4, 2, 32, 8, ctypes.byref(_t(nv, 95, 32)), ws, 8192, _stream()) == -1
    assert kq(None, 12, 4, 2, 32, 8, ctypes.byref(out), ws, 8192, _stream()) == -1
    assert kq(ctypes.c_void_p(FAKE), 12, 4, 2, 32, 8, ctypes.byref(out), None, 8192, _stream()) == -1
    assert kq(ctypes.c_void_p(FAKE), 12, 4, 2, 32, 8, ctypes.byref(out), ws, 4096, _stream()) == -3  # 2 domains
    assert kq(ctypes.c_void_p(FAKE), 40, 4, 2, 32, 8, ctypes.byref(_t(nv, 320, 32)), ws, 4096, _stream()) == -3
    assert kq(ctypes.c_void_p(FAKE), 0, 4, 2, 32, 8, ctypes.byref(_t(nv, 0, 32)), ws, 4096, _stream()) == 0
    kd = nv.lib.nvfp4_kv_dequant
    assert kd(ctypes.byref(out), 12, 4, 2, 32, 8, None, _stream()) == -1
    assert kd(ctypes.byref(out), 12, 4, 2, 32, 8, ctypes.c_void_p(FAKE + 8), _stream()) == -1
    assert kd(ctypes.byref(_t(nv, 96, 16)), 12, 4, 2, 32, 8, ctypes.c_void_p(FAKE), _stream()) == -1


def test_kv_quant_pair_rejects_bad_arguments(nv):
    kq = nv.lib.nvfp4_kv_quant_pair
    ko, vo = _t(nv, 12 * 4 * 2, 32), _t(nv, 12 * 4 * 2, 32)
    ws = ctypes.c_void_p(FAKE)
    x = ctypes.c_void_p(FAKE)

    def call(k=x, v=x, f=12, fb=8, fo6=0, ko=ko, vo=vo, ws=ws, wsb=16384):
        return kq(k, v, f, 4, 2, 32, fb, fo6, ctypes.byref(ko), ctypes.byref(vo), ws, wsb, _stream())

    assert nv.workspace_bytes(nv.OP_KV_QUANT_PAIR, 12, 8) == 16384  # two tensors x two frame blocks
    assert call(k=None) == -1
    assert call(v=ctypes.c_void_p(FAKE + 4)) == -1
    assert call(fb=0) == -1
    assert call(fo6=2) == -1
    assert call(ko=_t(nv, 95, 32)) == -1
    assert call(vo=_t(nv, 96, 16)) == -1
    assert call(vo=_t(nv, 96, 32, tscale=0)) == -1
    assert call(ws=None) == -1
    assert call(wsb=8192) == -3  # one tensor's workspace is not enough
    assert call(f=0, ko=_t(nv, 0, 32), vo=_t(nv, 0, 32)) == 0
    kd = nv.lib.nvfp4_kv_dequant_pair
    o = ctypes.c_void_p(FAKE)
    assert kd(ctypes.byref(ko), ctypes.byref(vo), 12, 4, 2, 32, 8, o, None, _stream()) == -1
    assert kd(ctypes.byref(ko), ctypes.byref(vo), 12, 4, 2, 32, 8, ctypes.c_void_p(FAKE + 8), o, _stream()) == -1
    assert kd(ctypes.byref(ko), ctypes.byref(_t(nv, 96, 16)), 12, 4, 2, 32, 8, o, o, _stream()) == -1
    assert kd(ctypes.byref(ko), ctypes.byref(vo), 12, 4, 2, 32, 0, o, o, _stream()) == -1
    assert kd(ctypes.byref(_t(nv, 0, 32)), ctypes.byref(_t(nv, 0, 32)), 0, 4, 2, 32, 8, o, o, _stream()) == 0


def test_amax_encode_dequant_reject_bad_arguments(nv):
    am = nv.lib.nvfp4_amax
    W = ctypes.c_void_p(FAKE)
    assert am(W, 1, 4, 32, 32, 0, None, W, 4096, _stream()) == -1
    assert am(W, 1, 4, 30, 32, 0, W, W, 4096, _stream()) == -1
    assert am(W, 1, 4, 32, 32, 0, W, None, 4096, _stream()) == -1
    assert am(W, 1, 8, 32, 32, 4, W, W, 4096, _stream()) == -3    # two domains need 8 KiB
    assert am(W, 1, 0, 32, 32, 0, W, W, 4096, _stream()) == 0
    good = _t(nv, 64, 32)
    enc = nv.lib.nvfp4_encode
    assert enc(ctypes.c_void_p(FAKE), 1, 64, 32, 32, 1, 0, None, ctypes.byref(good), _stream()) == -1
    assert enc(ctypes.c_void_p(FAKE), 1, 32, 64, 64, 0, 8, ctypes.c_void_p(FAKE), ctypes.byref(good), _stream()) == -1
    assert enc(ctypes.c_void_p(FAKE), 1, 64, 32, 32, 1, -1, ctypes.c_void_p(FAKE), ctypes.byref(good), _stream()) == -1
    dq = nv.lib.nvfp4_dequantize
    assert dq(ctypes.byref(good), 0, None, 0, _stream()) == -1
    assert dq(ctypes.byref(good), 0, ctypes.c_void_p(FAKE), 3, _stream()) == -1
    assert dq(ctypes.byref(_t(nv, 0, 32)), 0, ctypes.c_void_p(FAKE), 0, _stream()) == 0


def test_kv_attention_rejects_bad_arguments(nv):
    at = nv.lib.nvfp4_kv_attention
    F, W = FAKE, ctypes.c_void_p(FAKE)
    k = _t(nv, 12 * 40 * 2, 128)
    ok = dict(q=W, qf=3, k=k, v=k, frames=12, tokens=40, heads=2, d=128, fb=8, out=W, dt=0)

    def call(**kw):
        a = dict(ok, **kw)
        return at(a["q"], a["qf"], ctypes.byref(a["k"]), ctypes.byref(a["v"]), a["frames"], a["tokens"],
                  a["heads"], a["d"], a["fb"], a["out"], a["dt"], _stream())

    EINVAL, EUNS = -1, -2
    assert call(q=None) == EINVAL
    assert call(q=ctypes.c_void_p(F + 2)) == EINVAL
    assert call(out=None) == EINVAL
    assert call(dt=4) == EINVAL
    assert call(qf=13) == EINVAL                              # more query frames than the window
    assert call(fb=0) == EINVAL
    assert call(k=_t(nv, 12 * 40 * 2 - 1, 128)) == EINVAL     # cache rows
    assert call(v=_t(nv, 12 * 40 * 2, 64)) == EINVAL          # head_dim mismatch
    # head dimensions other than 64 and 128 are refused before any launch
    for d in (32, 96, 256):
        assert call(k=_t(nv, 12 * 40 * 2, d), v=_t(nv, 12 * 40 * 2, d), d=d) == EUNS, d
    # zero queries is a no-op, whatever the frame-block size (frame blocks of
    # any key count are supported; GPU tests cover them)
    k13 = _t(nv, 12 * 13 * 2, 128)
    assert call(k=k13, v=k13, tokens=13, qf=0) == 0
    assert call(qf=0) == 0
    assert call(qf=0, fb=1 << 40) == 0


def test_absurd_sizes_are_rejected_without_overflow(nv):
    """Sizes whose products overflow 64 bits are rejected on the host
    (unsupported size or a shape mismatch), never wrapped into a launch."""
    W = ctypes.c_void_p(FAKE)
    huge = 1 << 40
    ws = ctypes.c_void_p(FAKE)
    kq = nv.lib.nvfp4_kv_quant
    assert kq(W, huge, huge, 2, 32, 8, ctypes.byref(_t(nv, 64, 32)), ws, 8192, _stream()) == -2
    assert kq(W, 2, huge, huge, 32, 8, ctypes.byref(_t(nv, 64, 32)), ws, 8192, _stream()) == -2
    kd = nv.lib.nvfp4_kv_dequant
    assert kd(ctypes.byref(_t(nv, 64, 32)), huge, huge, 2, 32, 8, W, _stream()) == -2
    at = nv.lib.nvfp4_kv_attention
    k = _t(nv, 64, 128)
    assert at(W, 1, ctypes.byref(k), ctypes.byref(k), huge, huge, 2, 128, 8, W, 0, _stream()) == -2
    q = nv.lib.nvfp4_quantize
    big = (1 << 62) - 16
    assert q(W, 1, big, big, big, 1, ctypes.byref(_t(nv, big, big)), ws, 4096, _stream()) == -2
    assert nv.lib.nvfp4_workspace_bytes(nv.OP_KV_QUANT, 1 << 62, 1) >= 1 << 62
    dq = nv.lib.nvfp4_dequantize
    assert dq(ctypes.byref(_t(nv, big, big)), 0, W, 0, _stream()) == -2


def test_binding_refuses_host_tensors_and_mismatched_buffers(nv):
    """The binding checks tensors before any C-ABI call: a host tensor (whose
    pointer a kernel would dereference on the GPU) and NVFP4 buffers that do
    not match each other are refused with an exception (CPU-only test)."""
    x = torch.zeros((4, 32), dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="CUDA"):
        nv.quantize(x)
    with pytest.raises(TypeError, match="CUDA"):
        nv.amax(x)
    good = nv.NVFP4Tensor(torch.zeros((4, 16), dtype=torch.uint8), torch.zeros((4, 2), dtype=torch.uint8),
                          torch.zeros((1,), dtype=torch.float32))
    with pytest.raises(TypeError, match="CUDA"):
        good.c()
    short_scales = nv.NVFP4Tensor(good.codes, torch.zeros((4, 1), dtype=torch.uint8), good.tscale)
    with pytest.raises(ValueError, match="scales"):
        short_scales.c()
    with pytest.raises(ValueError, match="tscale"):
        good.c(n_domains=2)
    wrong_dtype = nv.NVFP4Tensor(good.codes, good.scales, torch.zeros((1,), dtype=torch.float16))
    with pytest.raises(TypeError, match="tscale"):
        wrong_dtype.c()
    with pytest.raises(ValueError, match="out must have shape"):
        nv.gemm(good, good, out=torch.zeros((3, 4)))


def test_product_and_oracle_share_no_code():
    """The product path (binding, HIP sources, header, bench's timed code path
    through the binding) names nothing under oracle/, and the oracle names
    nothing of the product; only workloads/ (seeded inputs) serves both."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    pkg = os.path.join(root, "nvfp4_w4a4_block_02_amd")
    product = [os.path.join(pkg, "__init__.py"), os.path.join(pkg, "build.py"),
               os.path.join(root, "include", "nvfp4.h")]
    product += [os.path.join(pkg, "csrc", f) for f in os.listdir(os.path.join(pkg, "csrc"))]
    for path in product:
        text = open(path, encoding="utf-8").read()
        assert not re.search(r"\boracle\b", text), path
    for f in os.listdir(os.path.join(root, "oracle")):
        if f.endswith(".py"):
            text = open(os.path.join(root, "oracle", f), encoding="utf-8").read()
            assert not re.search(r"^\s*(import|from)\s+nvfp4_w4a4_block_02_amd", text, re.M), f
            assert "csrc" not in text and "libnvfp4" not in text, f
    wl = open(os.path.join(root, "workloads", "__init__.py"), encoding="utf-8").read()
    assert not re.search(r"^\s*(import|from)\s+(oracle|nvfp4_w4a4_block_02_amd)", wl, re.M)


def test_checked_view_is_checked_again_when_a_buffer_changes(nv, monkeypatch):
    """NVFP4Tensor.c() keeps its checked C view only while the same three
    tensors sit on the same memory: a replaced buffer is checked again (and a
    mismatching one refused), a moved storage gives new pointers, and a
    larger domain count than the checked one is checked again (CPU-only: the
    device check is switched off for host tensors here)."""
    monkeypatch.setattr(nv, "_on_gpu", lambda t, name: None)
    q = nv.NVFP4Tensor(torch.zeros((4, 16), dtype=torch.uint8), torch.zeros((4, 2), dtype=torch.uint8),
                       torch.zeros((1,), dtype=torch.float32))
    v1 = q.c()
    assert q.c() is v1
    assert (v1.rows, v1.k, v1.codes) == (4, 32, q.codes.data_ptr())
    q.scales = torch.zeros((4, 1), dtype=torch.uint8)
    with pytest.raises(ValueError, match="scales"):
        q.c()
    q.scales = torch.zeros((4, 2), dtype=torch.uint8)
    v2 = q.c()
    assert v2 is not v1 and v2.scales == q.scales.data_ptr()
    with pytest.raises(ValueError, match="tscale"):
        q.c(n_domains=2)
    q.codes.set_(torch.zeros((4, 16), dtype=torch.uint8))
    v3 = q.c()
    assert v3 is not v2 and v3.codes == q.codes.data_ptr()

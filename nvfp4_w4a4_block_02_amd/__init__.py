"""Thin Python binding of libnvfp4.so (MI355X / gfx950 NVFP4 W4A4 path).

Every function here only marshals arguments: it allocates the output tensors
with torch (device memory is torch's), passes raw device pointers and the
current HIP stream to the C ABI declared in ``include/nvfp4.h``, and turns a
non-zero status into an exception.  All arithmetic runs in the HIP kernels.

The library must have been built (``python -m nvfp4_w4a4_block_02_amd.build``).
It is loaded on first use (so that the build module itself can be imported
before it exists); every entry point raises if it is missing — there is no
fallback path.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libnvfp4.so")

F32, BF16 = 0, 1
EPI_NONE, EPI_GELU_TANH = 0, 1
OP_QUANTIZE, OP_RHT16, OP_GEMM, OP_KV_QUANT, OP_AMAX, OP_KV_QUANT_PAIR = 0, 1, 2, 3, 4, 5


class NVFP4Error(RuntimeError):
    pass


class _CTensor(ctypes.Structure):
    _fields_ = [
        ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("tscale", ctypes.c_void_p),
        ("rows", ctypes.c_int64),
        ("k", ctypes.c_int64),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m nvfp4_w4a4_block_02_amd.build` "
            "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I64, SZ, U32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_uint32
    TP = ctypes.POINTER(_CTensor)
    sigs = {
        "nvfp4_version": (I, []),
        "nvfp4_status_string": (ctypes.c_char_p, [I]),
        "nvfp4_workspace_bytes": (SZ, [I, I64, I64]),
        "nvfp4_amax": (I, [P, I, I64, I64, I64, I64, P, P, SZ, P]),
        "nvfp4_encode": (I, [P, I, I64, I64, I64, I, I64, P, TP, P]),
        "nvfp4_quantize": (I, [P, I, I64, I64, I64, I, TP, P, SZ, P]),
        "nvfp4_quantize_noalloc": (I, [P, I, I64, I64, I64, I, TP, P]),
        "rht16_quantize": (I, [P, I, I64, I64, I64, I, U32, TP, P, SZ, P]),
        "nvfp4_gemm": (I, [TP, TP, P, I, I64, I, P, P, SZ, P]),
        "nvfp4_gemm_tiled": (I, [TP, TP, P, I, I64, I, P, I, I, P]),
        "nvfp4_linear": (I, [P, I, I64, I64, I64, TP, TP, P, I, I64, I, P, P, SZ, P]),
        "nvfp4_kv_quant": (I, [P, I64, I64, I64, I64, I64, TP, P, SZ, P]),
        "nvfp4_kv_quant_4over6": (I, [P, I64, I64, I64, I64, I64, TP, P, SZ, P]),
        "nvfp4_kv_quant_pair": (I, [P, P, I64, I64, I64, I64, I64, I, TP, TP, P, SZ, P]),
        "nvfp4_kv_dequant": (I, [TP, I64, I64, I64, I64, I64, P, P]),
        "nvfp4_kv_dequant_pair": (I, [TP, TP, I64, I64, I64, I64, I64, P, P, P]),
        "nvfp4_dequantize": (I, [TP, I64, P, I, P]),
        "nvfp4_kv_attention": (I, [P, I64, TP, TP, I64, I64, I64, I64, I64, P, I, P]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        _LIB = _load()
    return _LIB


def __getattr__(name):  # module attribute `lib` loads the library on first access
    if name == "lib":
        return _lib()
    raise AttributeError(name)


EXPORTED = ("nvfp4_version", "nvfp4_status_string", "nvfp4_workspace_bytes", "nvfp4_amax",
            "nvfp4_encode", "nvfp4_quantize", "nvfp4_quantize_noalloc", "rht16_quantize", "nvfp4_gemm", "nvfp4_gemm_tiled", "nvfp4_linear", "nvfp4_kv_quant",
            "nvfp4_kv_quant_4over6", "nvfp4_kv_quant_pair", "nvfp4_kv_dequant", "nvfp4_kv_dequant_pair", "nvfp4_dequantize", "nvfp4_kv_attention")


def _check(status: int, what: str):
    if status != 0:
        raise NVFP4Error(f"{what}: {_lib().nvfp4_status_string(status).decode()} ({status})")


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t: torch.Tensor | None):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _on_gpu(t: torch.Tensor, name: str):
    """The C ABI takes device pointers: a host tensor handed to a kernel would
    fault the GPU, so it is refused here."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA tensor")


def _need(t: torch.Tensor, name: str, shape=None, dtype=None, min_numel: int = 0, gpu: bool = True):
    """An output or auxiliary buffer the kernels write or read in full: right
    dtype, contiguous, of the required shape or size, and (unless `gpu` is
    False, for a caller that checks the device last) on the GPU."""
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.numel() < min_numel:
        raise ValueError(f"{name} needs at least {min_numel} elements, has {t.numel()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if gpu:
        _on_gpu(t, name)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


@dataclass
class NVFP4Tensor:
    """Device NVFP4 tensor: codes [rows, k/2] uint8, scales [rows, k/16] uint8
    (E4M3FN), tscale [n_domains] float32."""

    codes: torch.Tensor
    scales: torch.Tensor
    tscale: torch.Tensor
    # (codes, scales, tscale, their data pointers, tscale.numel(), C view) of
    # the last successful check; not part of the value.
    _cview: tuple | None = field(default=None, init=False, repr=False, compare=False)

    @property
    def rows(self) -> int:
        return self.codes.shape[0]

    @property
    def k(self) -> int:
        return self.codes.shape[1] * 2

    def c(self, n_domains: int = 1) -> _CTensor:
        """The C view; checks first that the three buffers match each other
        (codes [rows, k/2] and scales [rows, k/16] uint8, at least
        `n_domains` float32 tensor scales), so that no kernel reads or writes
        past them.  The checked view is kept and handed out again while the
        same three tensors still sit on the same device memory (a buffer that
        is replaced, or whose storage moves, is checked again); the C calls
        only read it."""
        cv = self._cview
        if (cv is not None and cv[0] is self.codes and cv[1] is self.scales and cv[2] is self.tscale
                and n_domains <= cv[4]
                and cv[3] == (self.codes.data_ptr(), self.scales.data_ptr(), self.tscale.data_ptr())):
            return cv[5]
        if self.codes.dim() != 2:
            raise ValueError("codes must be 2-D [rows, k/2]")
        _need(self.codes, "codes", dtype=torch.uint8, gpu=False)
        _need(self.scales, "scales", shape=(self.rows, self.k // 16), dtype=torch.uint8, gpu=False)
        _need(self.tscale, "tscale", dtype=torch.float32, min_numel=max(n_domains, 1), gpu=False)
        for name, t in (("codes", self.codes), ("scales", self.scales), ("tscale", self.tscale)):
            _on_gpu(t, name)
        ptrs = (self.codes.data_ptr(), self.scales.data_ptr(), self.tscale.data_ptr())
        view = _CTensor(ptrs[0], ptrs[1], ptrs[2], self.rows, self.k)
        self._cview = (self.codes, self.scales, self.tscale, ptrs, self.tscale.numel(), view)
        return view

    @staticmethod
    def empty(rows: int, k: int, n_domains: int = 1, device="cuda") -> "NVFP4Tensor":
        return NVFP4Tensor(
            torch.empty((rows, k // 2), dtype=torch.uint8, device=device),
            torch.empty((rows, k // 16), dtype=torch.uint8, device=device),
            torch.empty((max(n_domains, 1),), dtype=torch.float32, device=device),
        )


def workspace_bytes(op: int, rows: int, cols: int) -> int:
    """Device workspace bytes an entry point needs (nvfp4_workspace_bytes)."""
    return int(_lib().nvfp4_workspace_bytes(op, rows, cols))


def _workspace(op, rows, cols, device):
    n = max(workspace_bytes(op, rows, cols), 16)
    return torch.empty((n // 4,), dtype=torch.float32, device=device)


def _ld(x: torch.Tensor) -> int:
    """Leading dimension of a row-major 2-D tensor on the GPU (a single row may
    carry any stride in torch; it is then reported as the row length)."""
    _on_gpu(x, "tensor")
    if x.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    if x.shape[1] > 1 and x.stride(1) != 1:
        raise ValueError("rows must be contiguous (stride 1 along the last dim)")
    return x.stride(0) if x.shape[0] > 1 else x.shape[1]


def _out_shape(x: torch.Tensor, axis: int):
    rows, cols = x.shape
    return (rows, cols) if axis == 1 else (cols, rows)


def amax(x: torch.Tensor, rows_per_domain: int = 0, out: torch.Tensor | None = None,
         ws: torch.Tensor | None = None, stream=None):
    """max |x| per domain of `rows_per_domain` rows (0: the whole tensor) into a
    float32 tensor of one value per domain (nvfp4_amax)."""
    rows, cols = x.shape
    nd = 1 if rows_per_domain <= 0 or rows_per_domain >= rows else -(-rows // rows_per_domain)
    if out is None:
        out = torch.empty((nd,), dtype=torch.float32, device=x.device)
    _need(out, "out", dtype=torch.float32, min_numel=nd)
    if ws is None:
        ws = _workspace(OP_AMAX, rows, rows_per_domain, x.device)
    _need(ws, "ws")
    _check(_lib().nvfp4_amax(_ptr(x), _dtype_code(x), rows, cols, _ld(x), rows_per_domain, _ptr(out),
                          _ptr(ws), ws.numel() * 4, _stream(stream)), "nvfp4_amax")
    return out


def encode(x: torch.Tensor, amax_t: torch.Tensor, axis: int = 1, rows_per_domain: int = 0,
           out: NVFP4Tensor | None = None, stream=None) -> NVFP4Tensor:
    """Encode x with given per-domain maxima `amax_t` (nvfp4_encode): codes,
    block scales and tscale = amax / 2688; axis 0 stores the transpose."""
    rows, cols = x.shape
    nd = 1 if rows_per_domain <= 0 or rows_per_domain >= rows else -(-rows // rows_per_domain)
    _need(amax_t, "amax", dtype=torch.float32, min_numel=nd)
    if out is None:
        r, k = _out_shape(x, axis)
        out = NVFP4Tensor.empty(r, k, nd, x.device)
    ct = out.c(nd)
    _check(_lib().nvfp4_encode(_ptr(x), _dtype_code(x), rows, cols, _ld(x), axis, rows_per_domain,
                            _ptr(amax_t), ctypes.byref(ct), _stream(stream)), "nvfp4_encode")
    return out


def quantize(x: torch.Tensor, axis: int = 1, out: NVFP4Tensor | None = None, ws: torch.Tensor | None = None,
             stream=None) -> NVFP4Tensor:
    """Quantize a float32/bf16 matrix to NVFP4 with one tensor scale
    (nvfp4_quantize): blocks along the rows' elements (axis 1) or down the
    columns (axis 0, output stored transposed)."""
    rows, cols = x.shape
    if out is None:
        r, k = _out_shape(x, axis)
        out = NVFP4Tensor.empty(r, k, 1, x.device)
    if ws is None:
        ws = _workspace(OP_QUANTIZE, rows, cols, x.device)
    _need(ws, "ws")
    ct = out.c()
    _check(_lib().nvfp4_quantize(_ptr(x), _dtype_code(x), rows, cols, _ld(x), axis, ctypes.byref(ct),
                              _ptr(ws), ws.numel() * 4, _stream(stream)), "nvfp4_quantize")
    return out


def quantize_noalloc(x: torch.Tensor, axis: int = 1, out: NVFP4Tensor | None = None, stream=None) -> NVFP4Tensor:
    """nvfp4_quantize without a workspace (nvfp4_quantize_noalloc): the
    library keeps the partial maxima in its own per-GPU scratch array, so the
    call allocates nothing when ``out`` is given.  Calls that overlap in time
    on one GPU race on that array."""
    rows, cols = x.shape
    if out is None:
        r, k = _out_shape(x, axis)
        out = NVFP4Tensor.empty(r, k, 1, x.device)
    ct = out.c()
    _check(_lib().nvfp4_quantize_noalloc(_ptr(x), _dtype_code(x), rows, cols, _ld(x), axis, ctypes.byref(ct),
                                         _stream(stream)), "nvfp4_quantize_noalloc")
    return out


def rht16_quantize(x: torch.Tensor, sign_mask: int, axis: int = 1, out: NVFP4Tensor | None = None,
                   ws: torch.Tensor | None = None, stream=None, k_pad: int = 0) -> NVFP4Tensor:
    """RHT16 then quantize; for axis 0, ``k_pad`` > rows zero-pads the output's
    reduction dimension to that length (zero codes and scales)."""
    rows, cols = x.shape
    if out is None:
        r, k = _out_shape(x, axis)
        out = NVFP4Tensor.empty(r, max(k, k_pad) if axis == 0 else k, 1, x.device)
    if ws is None:
        ws = _workspace(OP_RHT16, rows, cols, x.device)
    _need(ws, "ws")
    ct = out.c()
    _check(_lib().rht16_quantize(_ptr(x), _dtype_code(x), rows, cols, _ld(x), axis, sign_mask,
                              ctypes.byref(ct), _ptr(ws), ws.numel() * 4, _stream(stream)), "rht16_quantize")
    return out


def gemm(a: NVFP4Tensor, b: NVFP4Tensor, out_dtype=torch.bfloat16, epilogue: int = EPI_NONE,
         amax_out: torch.Tensor | None = None, out: torch.Tensor | None = None, stream=None,
         tiles: tuple[int, int] | None = None) -> torch.Tensor:
    """C = A @ B^T on NVFP4 operands (B is [N, K]).  ``tiles`` pins the
    (fragments along M, fragments along N) per wavefront; default: automatic."""
    if out is None:
        out = torch.empty((a.rows, b.rows), dtype=out_dtype, device=a.codes.device)
    if tuple(out.shape) != (a.rows, b.rows):
        raise ValueError(f"out must have shape {(a.rows, b.rows)}, got {tuple(out.shape)}")
    if amax_out is not None:
        _need(amax_out, "amax_out", dtype=torch.float32, min_numel=1)
    ca, cb = a.c(), b.c()
    if tiles is None:
        _check(_lib().nvfp4_gemm(ctypes.byref(ca), ctypes.byref(cb), _ptr(out), _dtype_code(out), _ld(out),
                              epilogue, _ptr(amax_out), None, 0, _stream(stream)), "nvfp4_gemm")
    else:
        _check(_lib().nvfp4_gemm_tiled(ctypes.byref(ca), ctypes.byref(cb), _ptr(out), _dtype_code(out), _ld(out),
                                    epilogue, _ptr(amax_out), tiles[0], tiles[1], _stream(stream)),
               "nvfp4_gemm_tiled")
    return out


def kv_quant(kv: torch.Tensor, frame_block: int = 8, out: NVFP4Tensor | None = None,
             ws: torch.Tensor | None = None, stream=None, four_over_six: bool = False) -> NVFP4Tensor:
    """KV-cache quantization in frame blocks; ``four_over_six`` selects the
    Four Over Six encoder (nvfp4_kv_quant_4over6)."""
    f, t, h, d = kv.shape
    if kv.dtype != torch.bfloat16 or not kv.is_contiguous():
        raise TypeError("kv must be a contiguous bfloat16 tensor [frames, tokens, heads, head_dim]")
    _on_gpu(kv, "kv")
    nd = -(-f // frame_block) if frame_block > 0 else 1
    if out is None:
        out = NVFP4Tensor.empty(f * t * h, d, nd, kv.device)
    if ws is None:
        ws = _workspace(OP_KV_QUANT, f, frame_block, kv.device)
    _need(ws, "ws")
    ct = out.c(nd)
    fn = _lib().nvfp4_kv_quant_4over6 if four_over_six else _lib().nvfp4_kv_quant
    _check(fn(_ptr(kv), f, t, h, d, frame_block, ctypes.byref(ct), _ptr(ws), ws.numel() * 4, _stream(stream)),
           "nvfp4_kv_quant_4over6" if four_over_six else "nvfp4_kv_quant")
    return out


def kv_quant_pair(k: torch.Tensor, v: torch.Tensor, frame_block: int = 8, k_out: NVFP4Tensor | None = None,
                  v_out: NVFP4Tensor | None = None, ws: torch.Tensor | None = None, stream=None,
                  four_over_six: bool = False) -> tuple[NVFP4Tensor, NVFP4Tensor]:
    """K and V of one cache in one call (nvfp4_kv_quant_pair): the same results
    as kv_quant on each, in two launches instead of four."""
    for name, t in (("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or t.dim() != 4:
            raise TypeError(f"{name} must be a contiguous bfloat16 tensor [frames, tokens, heads, head_dim]")
        _on_gpu(t, name)
    if k.shape != v.shape:
        raise ValueError(f"k and v must have the same shape, got {tuple(k.shape)} and {tuple(v.shape)}")
    f, t, h, d = k.shape
    nd = -(-f // frame_block) if frame_block > 0 else 1
    if k_out is None:
        k_out = NVFP4Tensor.empty(f * t * h, d, nd, k.device)
    if v_out is None:
        v_out = NVFP4Tensor.empty(f * t * h, d, nd, k.device)
    if ws is None:
        ws = _workspace(OP_KV_QUANT_PAIR, f, frame_block, k.device)
    _need(ws, "ws")
    ck, cv = k_out.c(nd), v_out.c(nd)
    _check(_lib().nvfp4_kv_quant_pair(_ptr(k), _ptr(v), f, t, h, d, frame_block, int(four_over_six),
                                      ctypes.byref(ck), ctypes.byref(cv), _ptr(ws), ws.numel() * 4,
                                      _stream(stream)), "nvfp4_kv_quant_pair")
    return k_out, v_out


def kv_dequant(q: NVFP4Tensor, shape, frame_block: int = 8, out: torch.Tensor | None = None,
               stream=None) -> torch.Tensor:
    """Decode an NVFP4 KV cache of `shape` = (frames, tokens, heads, head_dim)
    to bf16 with its per-frame-block tensor scales (nvfp4_kv_dequant)."""
    f, t, h, d = shape
    if out is None:
        out = torch.empty((f, t, h, d), dtype=torch.bfloat16, device=q.codes.device)
    _need(out, "out", shape=(f, t, h, d), dtype=torch.bfloat16)
    ct = q.c(-(-f // frame_block) if frame_block > 0 else 1)
    _check(_lib().nvfp4_kv_dequant(ctypes.byref(ct), f, t, h, d, frame_block, _ptr(out), _stream(stream)),
           "nvfp4_kv_dequant")
    return out


def kv_dequant_pair(kq: NVFP4Tensor, vq: NVFP4Tensor, shape, frame_block: int = 8,
                    k_out: torch.Tensor | None = None, v_out: torch.Tensor | None = None,
                    stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """K and V of one cache decoded to bf16 in one launch (nvfp4_kv_dequant_pair)."""
    f, t, h, d = shape
    outs = []
    for o in (k_out, v_out):
        if o is None:
            o = torch.empty((f, t, h, d), dtype=torch.bfloat16, device=kq.codes.device)
        _need(o, "out", shape=(f, t, h, d), dtype=torch.bfloat16)
        outs.append(o)
    nd = -(-f // frame_block) if frame_block > 0 else 1
    ck, cv = kq.c(nd), vq.c(nd)
    _check(_lib().nvfp4_kv_dequant_pair(ctypes.byref(ck), ctypes.byref(cv), f, t, h, d, frame_block, _ptr(outs[0]),
                                        _ptr(outs[1]), _stream(stream)), "nvfp4_kv_dequant_pair")
    return outs[0], outs[1]


def kv_attention(q: torch.Tensor, k: NVFP4Tensor, v: NVFP4Tensor, shape, frame_block: int = 8,
                 out_dtype=torch.bfloat16, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Frame-causal window attention of ``q`` (bf16 [q_frames * tokens, heads,
    head_dim]) over the NVFP4 caches ``k``/``v`` of ``shape`` = (frames, tokens,
    heads, head_dim) (nvfp4_kv_attention)."""
    f, t, h, d = shape
    if q.dtype != torch.bfloat16 or not q.is_contiguous() or q.dim() != 3 or q.shape[1:] != (h, d) \
            or t == 0 or q.shape[0] % t:
        raise TypeError("q must be a contiguous bfloat16 tensor [q_frames * tokens, heads, head_dim]")
    _on_gpu(q, "q")
    qf = q.shape[0] // t
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    _need(out, "out", shape=q.shape)
    nfb = -(-f // frame_block) if frame_block > 0 else 1
    ck, cv = k.c(nfb), v.c(nfb)
    _check(_lib().nvfp4_kv_attention(_ptr(q), qf, ctypes.byref(ck), ctypes.byref(cv), f, t, h, d, frame_block,
                                     _ptr(out), _dtype_code(out), _stream(stream)), "nvfp4_kv_attention")
    return out


def dequantize(q: NVFP4Tensor, dtype=torch.float32, rows_per_domain: int = 0, out: torch.Tensor | None = None,
               stream=None) -> torch.Tensor:
    """Decode an NVFP4 tensor to float32 or bf16, one tensor scale per domain
    of `rows_per_domain` rows (nvfp4_dequantize)."""
    if out is None:
        out = torch.empty((q.rows, q.k), dtype=dtype, device=q.codes.device)
    _need(out, "out", shape=(q.rows, q.k))
    nd = 1 if rows_per_domain <= 0 or rows_per_domain >= q.rows else -(-q.rows // rows_per_domain)
    ct = q.c(nd)
    _check(_lib().nvfp4_dequantize(ctypes.byref(ct), rows_per_domain, _ptr(out), _dtype_code(out), _stream(stream)),
           "nvfp4_dequantize")
    return out


def linear(x: torch.Tensor, w: NVFP4Tensor, out_dtype=torch.bfloat16, xq: NVFP4Tensor | None = None,
           ws: torch.Tensor | None = None, out: torch.Tensor | None = None, stream=None,
           epilogue: int = EPI_NONE, amax_out: torch.Tensor | None = None) -> torch.Tensor:
    """W4A4 linear layer in one C call (nvfp4_linear): quantize the
    activations x [M, K] into ``xq``, then the block-scaled GEMM against the
    pre-quantized weights w [N, K] into ``out`` [M, N].

    This is the latency path of small layers, so its checks are the ones the
    C ABI cannot make from raw pointers, written out inline: every tensor on
    the GPU, rows of x and out contiguous, out of shape [M, N], a contiguous
    workspace (its byte count goes to the C side, which checks it, the
    dtypes, alignment and sizes)."""
    rows, cols = x.shape
    if xq is None:
        xq = NVFP4Tensor.empty(rows, cols, 1, x.device)
    if out is None:
        out = torch.empty((rows, w.rows), dtype=out_dtype, device=x.device)
    if ws is None:
        ws = _workspace(OP_QUANTIZE, rows, cols, x.device)
    osh = out.shape
    if len(osh) != 2 or osh[0] != rows or osh[1] != w.codes.shape[0]:
        raise ValueError(f"out must have shape {(rows, w.rows)}, got {tuple(osh)}")
    if not (x.is_cuda and out.is_cuda and ws.is_cuda):
        raise TypeError("x, out and ws must be CUDA tensors")
    if not ws.is_contiguous():
        raise ValueError("ws must be contiguous")
    xs, os_ = x.stride(), out.stride()
    if (cols > 1 and xs[1] != 1) or (osh[1] > 1 and os_[1] != 1):
        raise ValueError("rows of x and out must be contiguous (stride 1 along the last dim)")
    amax_p = 0
    if amax_out is not None:
        _need(amax_out, "amax_out", dtype=torch.float32, min_numel=1)
        amax_p = amax_out.data_ptr()
    cx, cw = xq.c(), w.c()
    st = (stream if stream is not None else torch.cuda.current_stream()).cuda_stream
    status = _lib().nvfp4_linear(x.data_ptr(), _dtype_code(x), rows, cols, xs[0] if rows > 1 else cols,
                                 ctypes.byref(cw), ctypes.byref(cx), out.data_ptr(), _dtype_code(out),
                                 os_[0] if rows > 1 else osh[1], epilogue, amax_p, ws.data_ptr(),
                                 ws.numel() * ws.element_size(), st)
    if status:
        _check(status, "nvfp4_linear")
    return out


def ffn(x: torch.Tensor, w1: NVFP4Tensor, w2: NVFP4Tensor, out_dtype=torch.bfloat16, bufs: dict | None = None,
        stream=None) -> torch.Tensor:
    """DiT FFN pair on NVFP4: quantize x -> GEMM1 with GELU-tanh epilogue into
    float32 H (the epilogue also reduces max|H|) -> re-quantize H with that
    amax -> GEMM2."""
    m = x.shape[0]
    dev = x.device
    if bufs is None:
        bufs = {}
    xq = quantize(x, out=bufs.get("xq"), ws=bufs.get("ws"), stream=stream)
    h = bufs.get("h")
    if h is None:
        h = torch.empty((m, w1.rows), dtype=torch.float32, device=dev)
    hmax = bufs.get("hmax")
    if hmax is None:
        hmax = torch.empty((1,), dtype=torch.float32, device=dev)
    gemm(xq, w1, epilogue=EPI_GELU_TANH, amax_out=hmax, out=h, stream=stream)
    hq = encode(h, hmax, out=bufs.get("hq"), stream=stream)
    return gemm(hq, w2, out_dtype=out_dtype, out=bufs.get("y"), stream=stream)


_SIDE_STREAMS: dict = {}


def _side_streams(device: torch.device):
    """Two streams per device for linear_train's independent chains (default
    priority, created once)."""
    idx = device.index if device.index is not None else torch.cuda.current_device()
    if idx not in _SIDE_STREAMS:
        with torch.cuda.device(idx):
            _SIDE_STREAMS[idx] = (torch.cuda.Stream(), torch.cuda.Stream())
    return _SIDE_STREAMS[idx]


def linear_train(x: torch.Tensor, w: torch.Tensor, dy: torch.Tensor, sign_mask: int, bufs: dict | None = None,
                 stream=None):
    """The NVFP4 GEMM triple of one linear layer Y = X W^T in training; each
    GEMM quantizes both operands along its own reduction dimension, and the
    weight-gradient operands go through the RHT16 first (one sign mask for
    both):

      y  = Q(X) Q(W)^T          (bf16)   x [M, K], w [N, K] (master weight)
      dx = Q(dY) Q(W^T)^T       (bf16)   dy [M, N]; W quantized along dim 0
      dw = R(dY^T) R(X^T)^T     (f32)    dY and X quantized along dim 0

    Returns (y, dx, dw).  Only sequences C-ABI calls: the three chains are
    independent but for W's amax, which both of W's encodings use, so they
    are issued on the caller's stream and two side streams (forked from and
    joined back into the caller's stream with events), letting the small
    quantization launches run side by side and beside the GEMMs' tails;
    results are the same as one stream's.
    Preallocated ``bufs`` must give "dyt" / "xt" a K of M rounded up to 256;
    workspaces "ws", "ws1", "ws2" serve the three streams (each large enough
    for the RHT16 of the larger operand)."""
    b = bufs if bufs is not None else {}
    s0 = stream if stream is not None else torch.cuda.current_stream()
    s1, s2 = _side_streams(x.device)
    fork = torch.cuda.Event()
    fork.record(s0)
    s1.wait_event(fork)
    s2.wait_event(fork)
    # Chain 1 (caller's stream): W's amax (one tensor scale for both of its
    # encodings: the amax does not depend on the block direction), W along
    # K, X along K, then Y.
    wamax = amax(w, out=b.get("wamax"), ws=b.get("ws"), stream=s0)
    w_amax_done = torch.cuda.Event()
    w_amax_done.record(s0)
    wq = encode(w, wamax, axis=1, out=b.get("wq"), stream=s0)
    xq = quantize(x, axis=1, out=b.get("xq"), ws=b.get("ws"), stream=s0)
    y = gemm(xq, wq, out_dtype=torch.bfloat16, out=b.get("y"), stream=s0)
    # Chain 2: dY along N; W along N once its amax is known; then dX.
    dyq = quantize(dy, axis=1, out=b.get("dyq"), ws=b.get("ws1"), stream=s1)
    s1.wait_event(w_amax_done)
    wtq = encode(w, wamax, axis=0, out=b.get("wtq"), stream=s1)
    dx = gemm(dyq, wtq, out_dtype=torch.bfloat16, out=b.get("dx"), stream=s1)
    # Chain 3: the weight gradient reduces over M; its operands are
    # zero-padded to a multiple of 256 along M (exact: zero blocks add
    # nothing) so that the GEMM runs its pipelined path for any token count.
    mp = -(-x.shape[0] // 256) * 256
    dyt = rht16_quantize(dy, sign_mask, axis=0, out=b.get("dyt"), ws=b.get("ws2"), stream=s2, k_pad=mp)
    xt = rht16_quantize(x, sign_mask, axis=0, out=b.get("xt"), ws=b.get("ws2"), stream=s2, k_pad=mp)
    dw = gemm(dyt, xt, out_dtype=torch.float32, out=b.get("dw"), stream=s2)
    for side in (s1, s2):
        done = torch.cuda.Event()
        done.record(side)
        s0.wait_event(done)
    return y, dx, dw

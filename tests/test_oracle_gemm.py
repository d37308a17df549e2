"""Pins for the oracle's block-scaled GEMM and GELU (CPU only): exact
rational dot products on tiny shapes, the unit-scale special case (a plain
integer matmul), a single 16-element block, operand orientation, and GELU
against torch's tanh-approximate GELU (a library routine)."""

from fractions import Fraction

from decimal import Decimal, localcontext

import numpy as np
import torch

import oracle
from oracle import codec, formats as F


def _frac_decode(codes_row, scales_row):
    """Fraction-valued decode straight from the bit fields, one row."""
    out = []
    for byte in (int(v) for v in codes_row):
        for nib in (byte & 15, byte >> 4):
            s, e, m = nib >> 3, (nib >> 1) & 3, nib & 1
            mag = Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
            out.append(-mag if s else mag)
    res = []
    for i, v in enumerate(out):
        b = int(scales_row[i // 16])
        be, bm = (b >> 3) & 15, b & 7
        sig = Fraction(bm, 512) if be == 0 else Fraction(2) ** (be - 7) * (1 + Fraction(bm, 8))
        res.append(v * sig)
    return res


def test_tiny_gemm_against_exact_fractions():
    rng = np.random.default_rng(0)
    for (m, n, k) in [(1, 1, 16), (3, 5, 32), (8, 8, 64), (7, 2, 48)]:
        a = (rng.standard_normal((m, k)) * rng.uniform(0.1, 10)).astype(np.float32)
        b = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
        qa, qb = oracle.quantize(a), oracle.quantize(b)
        c, bound = oracle.gemm_ref(qa, qb)
        sa, sb = Fraction(float(qa.tscale[0])), Fraction(float(qb.tscale[0]))
        for i in range(m):
            pa = _frac_decode(qa.codes[i], qa.scales[i])
            for j in range(n):
                pb = _frac_decode(qb.codes[j], qb.scales[j])
                exact = sa * sb * sum(x * y for x, y in zip(pa, pb))
                babs = sa * sb * sum(abs(x * y) for x, y in zip(pa, pb))
                assert abs(Fraction(c[i, j]) - exact) <= Fraction(1, 2 ** 50) * babs
                assert abs(Fraction(bound[i, j]) - babs) <= Fraction(1, 2 ** 50) * babs


def test_unit_scales_reduce_to_integer_matmul():
    # All block scales 1.0 (0x38) and S = 1: the product is the plain matmul
    # of the E2M1 values, i.e. (integer matmul of 2*e2m1) / 4.
    rng = np.random.default_rng(1)
    m, n, k = 6, 9, 80
    ca = rng.integers(0, 16, (m, k)).astype(np.uint8)
    cb = rng.integers(0, 16, (n, k)).astype(np.uint8)
    pack = lambda c: (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    one = np.full((m, k // 16), 0x38, np.uint8)
    qa = codec.QTensor(pack(ca), one, np.array([1.0], np.float32))
    qb = codec.QTensor(pack(cb), np.full((n, k // 16), 0x38, np.uint8), np.array([1.0], np.float32))
    ia = (2 * F.e2m1_value(ca)).astype(np.int64)
    ib = (2 * F.e2m1_value(cb)).astype(np.int64)
    c, _ = oracle.gemm_ref(qa, qb)
    assert np.array_equal(c, (ia @ ib.T) / 4.0)


def test_single_block_and_orientation():
    rng = np.random.default_rng(2)
    a = rng.standard_normal((4, 16)).astype(np.float32)
    b = rng.standard_normal((3, 16)).astype(np.float32)
    qa, qb = oracle.quantize(a), oracle.quantize(b)
    c, _ = oracle.gemm_ref(qa, qb)
    da = oracle.dequantize(qa).astype(np.float64)
    db = oracle.dequantize(qb).astype(np.float64)
    # C[m, n] = <row m of A, row n of B> (B stored [N, K])
    assert np.allclose(c, da @ db.T, rtol=1e-6, atol=1e-9)
    # and the row selection matches the full product
    c1, _ = oracle.gemm_ref(qa, qb, rows=np.array([2]))
    assert np.array_equal(c1[0], c[2])


def test_gelu_against_torch():
    """torch's gelu(approximate="tanh") (a library routine) where its own
    1 + tanh(u) does not cancel (h >= -2; below that torch loses relative
    precision, about 3e-10 at h = -5, and the decimal pin takes over)."""
    h = np.concatenate([np.linspace(-2, 12, 1401), [0.0, 1.0, -1.0, 1e-8, 40.0]])
    ours = oracle.gelu_tanh(h)
    lib = torch.nn.functional.gelu(torch.from_numpy(h), approximate="tanh").numpy()
    assert np.allclose(ours, lib, rtol=1e-13, atol=1e-300)
    assert oracle.gelu_tanh(0.0) == 0.0
    # the tanh part is odd: g(h) - g(-h) = h
    assert np.allclose(oracle.gelu_tanh(h) - oracle.gelu_tanh(-h), h, rtol=1e-12, atol=1e-12)


_PI = "3.14159265358979323846264338327950288419716939937510582097494459230781640628620899862803482534211706798"


def _gelu_decimal(h: float) -> float:
    """The definition 0.5 h (1 + tanh(u)), tanh(u) = (e^(2u) - 1) / (e^(2u) + 1),
    in 420-digit decimal arithmetic from the exact float64 input: enough
    digits that 1 + tanh(u) keeps its value down to e^(2u) ~ 1e-310."""
    with localcontext() as ctx:
        ctx.prec = 420
        x = Decimal(h)
        c = (Decimal(2) / Decimal(_PI)).sqrt()
        u = c * (x + Decimal("0.044715") * x ** 3)
        e = (2 * u).exp()
        t = (e - 1) / (e + 1)
        return float(Decimal("0.5") * x * (1 + t))


def test_gelu_against_high_precision_definition():
    """Every float64 result, the far negative tail included, within the
    rounding of its float64 evaluation of the definition computed to 420
    digits: the exponent argument 2u carries a relative error of a few
    2^-53, which moves e^(-2u) by |2u| times that."""
    rng = np.random.default_rng(15)
    h = np.concatenate([np.linspace(-19, 20, 391), rng.uniform(-19, 20, 200), [-1e-3, 1e-3, -0.5, 2.5]])
    ours = oracle.gelu_tanh(h)
    ref = np.array([_gelu_decimal(float(v)) for v in h])
    u = np.sqrt(2 / np.pi) * (h + 0.044715 * h ** 3)
    assert np.all(ours[h < -6] != 0.0) and np.all(ref[h < -6] != 0.0)   # the tail is not flushed
    rtol = 2.0 ** -52 * (8 + 4 * np.abs(u))
    assert np.all(np.abs(ours - ref) <= rtol * np.abs(ref) + 1e-320)

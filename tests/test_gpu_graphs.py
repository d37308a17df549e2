"""HIP graph capture of the library's call sequences.

The library allocates nothing when its outputs and workspaces are given and
clears memory (the GEMM epilogue's amax) with a fill kernel rather than
memset, so a sequence of its calls can be captured into a HIP graph and
replayed.  Each test captures a sequence once, then replays it several times
on new input data (written into the captured input buffer with eager work in
between) and requires every replay to equal an eager run of the same calls
on the same data bit for bit; the eager runs themselves are checked against
the oracle elsewhere (test_gpu_gemm.py)."""

import numpy as np
import pytest
import torch

import workloads
from gpu_helpers import dev_bf16, log, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    return require_gpu()


def _q_equal(a, b):
    return (torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)
            and torch.equal(a.tscale.view(torch.int32), b.tscale.view(torch.int32)))


def test_linear_graph_replays_match_eager(nv):
    """Activation quantize + GEMM (the 256 x 512 x 512 linear, float32 out)
    captured once and replayed on three inputs."""
    m, n, k = 256, 512, 512
    log(f"graph replay: linear {m}x{n}x{k}")
    d = workloads.tiny_linear(m=m, n=n, k=k)
    wq = nv.quantize(torch.from_numpy(d["w"]).cuda())
    a = torch.empty((m, k), dtype=torch.float32, device="cuda")
    aq = nv.NVFP4Tensor.empty(m, k, 1, "cuda")
    ws = nv._workspace(nv.OP_QUANTIZE, m, k, "cuda")
    c = torch.empty((m, n), dtype=torch.float32, device="cuda")
    a.copy_(torch.from_numpy(d["a"]))
    nv.quantize(a, out=aq, ws=ws)          # warm the calls up outside the capture
    nv.gemm(aq, wq, out=c)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        nv.quantize(a, out=aq, ws=ws)
        nv.gemm(aq, wq, out=c)
    rng = np.random.default_rng(7)
    for rep in range(3):
        x = (rng.standard_normal((m, k)) * (1.0 + 10.0 * rep)).astype(np.float32)
        a.copy_(torch.from_numpy(x))
        g.replay()
        torch.cuda.synchronize()
        got_c, got_q = c.clone(), nv.NVFP4Tensor(aq.codes.clone(), aq.scales.clone(), aq.tscale.clone())
        ref_q = nv.quantize(a)                # eager, fresh buffers
        ref_c = nv.gemm(ref_q, wq, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert _q_equal(got_q, ref_q), rep
        assert torch.equal(got_c.view(torch.int32), ref_c.view(torch.int32)), rep


def test_ffn_graph_replays_match_eager(nv):
    """The FFN chain (quantize, GEMM1 with the GELU epilogue and its amax,
    which clears the amax with a fill kernel, re-quantization of H, GEMM2)
    captured once and replayed on three inputs."""
    m, dm, f = 512, 512, 1024
    log(f"graph replay: ffn {m}x{dm}->{f}->{dm}")
    d = workloads.ffn(m=m, d=dm, f=f, seed=11)
    w1 = nv.quantize(torch.from_numpy(d["w1"]).cuda())
    w2 = nv.quantize(torch.from_numpy(d["w2"]).cuda())
    x = dev_bf16(d["x"])
    bufs = {"xq": nv.NVFP4Tensor.empty(m, dm, 1, "cuda"), "ws": nv._workspace(nv.OP_QUANTIZE, m, dm, "cuda"),
            "h": torch.empty((m, f), dtype=torch.float32, device="cuda"),
            "hmax": torch.empty((1,), dtype=torch.float32, device="cuda"),
            "hq": nv.NVFP4Tensor.empty(m, f, 1, "cuda"),
            "y": torch.empty((m, dm), dtype=torch.bfloat16, device="cuda")}
    nv.ffn(x, w1, w2, bufs=bufs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        nv.ffn(x, w1, w2, bufs=bufs)
    for rep in range(3):
        xn = workloads.ffn(m=m, d=dm, f=f, seed=100 + rep)["x"]
        x.copy_(dev_bf16(xn))
        g.replay()
        torch.cuda.synchronize()
        got_y, got_hmax = bufs["y"].clone(), bufs["hmax"].clone()
        got_hq = nv.NVFP4Tensor(bufs["hq"].codes.clone(), bufs["hq"].scales.clone(), bufs["hq"].tscale.clone())
        ref = {"h": torch.empty((m, f), dtype=torch.float32, device="cuda"),
               "hmax": torch.empty((1,), dtype=torch.float32, device="cuda"),
               "hq": nv.NVFP4Tensor.empty(m, f, 1, "cuda")}
        ref_y = nv.ffn(x, w1, w2, bufs=ref)    # eager
        torch.cuda.synchronize()
        assert torch.equal(got_hmax.view(torch.int32), ref["hmax"].view(torch.int32)), rep
        assert _q_equal(got_hq, ref["hq"]), rep
        assert torch.equal(got_y.view(torch.int16), ref_y.view(torch.int16)), rep


def test_one_call_linear_and_kv_pair_graph_replays_match_eager(nv):
    """nvfp4_linear (as the bench's graph figure captures it) and the K+V
    pair quantize + dequantize captured once and replayed on three inputs;
    every replay equals eager calls of the same entry points bit for bit."""
    m, n, k = 256, 512, 512
    shape = (3, 40, 4, 64)
    log(f"graph replay: nvfp4_linear {m}x{n}x{k}, K+V pair codec {shape}")
    d = workloads.tiny_linear(m=m, n=n, k=k)
    wq = nv.quantize(torch.from_numpy(d["w"]).cuda())
    a = torch.empty((m, k), dtype=torch.float32, device="cuda")
    aq = nv.NVFP4Tensor.empty(m, k, 1, "cuda")
    ws = nv._workspace(nv.OP_QUANTIZE, m, k, "cuda")
    c = torch.empty((m, n), dtype=torch.float32, device="cuda")
    kk = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    vv = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    rows = shape[0] * shape[1] * shape[2]
    kq, vq = nv.NVFP4Tensor.empty(rows, shape[3], 1, "cuda"), nv.NVFP4Tensor.empty(rows, shape[3], 1, "cuda")
    kws = nv._workspace(nv.OP_KV_QUANT_PAIR, shape[0], 8, "cuda")
    ko = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    vo = torch.empty(shape, dtype=torch.bfloat16, device="cuda")

    def calls():
        nv.linear(a, wq, xq=aq, ws=ws, out=c)
        nv.kv_quant_pair(kk, vv, k_out=kq, v_out=vq, ws=kws)
        nv.kv_dequant_pair(kq, vq, shape, k_out=ko, v_out=vo)

    rng = np.random.default_rng(11)
    a.copy_(torch.from_numpy(d["a"]))
    kk.normal_()
    vv.normal_()
    calls()                               # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep in range(3):
        a.copy_(torch.from_numpy((rng.standard_normal((m, k)) * (1.0 + 10.0 * rep)).astype(np.float32)))
        kk.copy_(torch.from_numpy((rng.standard_normal(shape) * (0.5 + rep)).astype(np.float32)).to(torch.bfloat16))
        vv.copy_(torch.from_numpy((rng.standard_normal(shape) * 3.0).astype(np.float32)).to(torch.bfloat16))
        g.replay()
        torch.cuda.synchronize()
        got = [c.clone(), ko.clone(), vo.clone()]
        got_q = [nv.NVFP4Tensor(t.codes.clone(), t.scales.clone(), t.tscale.clone()) for t in (aq, kq, vq)]
        ref_c = nv.linear(a, wq, out_dtype=torch.float32)
        ref_k, ref_v = nv.kv_quant_pair(kk, vv)
        ref_ko, ref_vo = nv.kv_dequant_pair(ref_k, ref_v, shape)
        ref_a = nv.quantize(a)
        torch.cuda.synchronize()
        assert torch.equal(got[0].view(torch.int32), ref_c.view(torch.int32)), f"replay {rep}: linear output"
        assert torch.equal(got[1].view(torch.int16), ref_ko.view(torch.int16)), f"replay {rep}: K dequant"
        assert torch.equal(got[2].view(torch.int16), ref_vo.view(torch.int16)), f"replay {rep}: V dequant"
        for gq, rq, nm in zip(got_q, (ref_a, ref_k, ref_v), ("A", "K", "V")):
            assert _q_equal(gq, rq), f"replay {rep}: {nm} codes"

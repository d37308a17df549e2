"""Benchmark of the NVFP4 W4A4 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-rows] [--no-cpu]
                    [--only ROW,ROW] [--no-headline] [--settle-ms MS]

One step = one pass of the attention-projection workload of the 5B DiT
(2640 tokens = 3 latent frames x 880, width 3072): amax of the bf16
activations, their NVFP4 encode, and the block-scaled W4A4 GEMM against
pre-quantized 3072x3072 NVFP4 weights into bf16.  The timed region starts
with every input resident in HBM; buffers rotate over 13 independent sets
(> 512 MB) so the 256 MB Infinity Cache cannot serve a step from the last
one.  Before the timed steps, W warmup steps and then further untimed steps
until the GPU has run this workload for at least --settle-ms (the clocks take
a few milliseconds to settle after a change of load).  The timed steps run
back to back with nothing between them (a HIP event recorded between two
kernels idles the GPU for ~10 us on this part, so per-kernel events would
distort the step time); per-kernel durations come from separate back-to-back
passes over the same buffers, each after the same settle, each timed by one
pair of HIP events on the launch stream.  Prints ONE JSON line.

Besides the headline value the line carries:
  roofline      the GEMM kernel (the dominant kernel): its algorithmic
                flops per launch / its mean duration over back-to-back
                launches on the launch stream;
  cpu_baseline  the CPU oracle timed on bounded samples of every workload
                on this host (element-wise work over row chunks on a thread
                pool, float64 GEMMs on the BLAS threads); `value` is the
                attention-projection workload, `per_config` all five;
  device_copy   a 256 MiB device-to-device copy (read + write bytes per
                second): the practical HBM rate that the HBM-bound rows are
                also quoted against (frac_copy), beside the 8 TB/s datasheet
                peak (frac_hbm);
  rows          the other rows of the path, each timed back to back the same
                way in five batches (ms = mean over all calls; ms_median and
                ms_min of the batch means): the tiny W4A4 linear (256x512 by
                512x512, latency); KV codec quantize (core recipe and Four
                Over Six) and dequantize (12x880x24x128 bf16, K and V); the
                frame-causal window attention of 2640 queries (3 latent
                frames) x 24 heads over that 12-frame NVFP4 KV cache, read
                directly (flops counted over the visible query-key pairs);
                RHT16 + quantize of a 16384x3072 gradient along dim 0 and the
                3072x3072x16384 weight-gradient GEMM; the FFN pair
                (10560x3072 -> 14336 -> 3072); the NVFP4 training triple
                (forward, input and weight gradient, with the six operand
                quantizations) of a 2640x3072x3072 linear layer.

--only restricts the rows to the named ones and --no-headline skips the
headline step (its keys are then absent): a profiler run of one row then
covers exactly one shape per kernel.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import re
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A4 NVFP4 GEMM TFLOPS (incl. act quant) at DiT shapes; quant/KV codec GB/s"
HBM_PEAK_GBS = 8000.0
PEAK_TFLOPS = {"f16": 2500.0, "fp8": 5000.0, "fp4": 10100.0}


def _args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=500,
                   help="untimed steps before the timed ones (500 steps, ~30 ms, let the GPU clocks settle)")
    p.add_argument("--no-rows", action="store_true", help="skip the per-row extra measurements")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--only", default="", help="comma-separated row names to run (default: all rows)")
    p.add_argument("--no-headline", action="store_true", help="skip the headline step (profiling a row alone)")
    p.add_argument("--settle-ms", type=float, default=30.0,
                   help="untimed run time after the warmup steps before any timed pass (clock settle)")
    p.add_argument("--sets", type=int, default=13, help="rotating buffer sets")
    p.add_argument("--calibrate", action="store_true",
                   help="only time the vendor's dense GEMMs (torch.matmul in bf16, torch._scaled_mm in fp8) "
                        "at the four W4A4 GEMM shapes, as the practical MFMA ceiling on this part, and exit")
    p.add_argument("--copy-probe", action="store_true",
                   help="only run three 256 MiB device-to-device copies (calibrates the rocprofv3 "
                        "FETCH_SIZE / WRITE_SIZE counters against a known byte count) and exit")
    return p.parse_args()


def copy_probe():
    import torch

    x = torch.ones(1 << 26, device="cuda")  # 256 MiB of float32
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_each_way": x.numel() * 4, "copies": 3}), flush=True)


# The W4A4 GEMM shapes of the timed rows: C[M, N] = A[M, K] . B[N, K]^T.
GEMM_SHAPES = (("attn_proj", 2640, 3072, 3072), ("ffn_gemm1", 10560, 14336, 3072),
               ("ffn_gemm2", 10560, 3072, 14336), ("wgrad", 3072, 3072, 16384))


def calibrate(steps):
    """Dense GEMMs of the library PyTorch dispatches to (hipBLASLt on this
    part) at the W4A4 GEMM shapes, same "TN" operand layout, bf16 in and out,
    and fp8 (e4m3, per-tensor scales) in with bf16 out.  These have no decode
    at all; their rates say what the MFMAs sustain on these shapes at the
    clocks the part runs under such load, beside the datasheet peaks."""
    import torch

    torch.cuda.init()
    stream = torch.cuda.current_stream()
    out = {"blas_library": str(torch.backends.cuda.preferred_blas_library()), "shapes": {}}
    for name, m, n, k in GEMM_SHAPES:
        flops = 2.0 * m * n * k
        nsets = max(2, min(8, int(1.2e9 // ((m + n) * k * 2 + m * n * 2))))
        g = torch.Generator(device="cuda").manual_seed(11)
        sets = [(torch.randn(m, k, device="cuda", generator=g).to(torch.bfloat16),
                 torch.randn(n, k, device="cuda", generator=g).mul_(0.02).to(torch.bfloat16),
                 torch.empty(m, n, device="cuda", dtype=torch.bfloat16)) for _ in range(nsets)]
        rec = {"M": m, "N": n, "K": k}

        def bf16(i):
            a, b, c = sets[i % nsets]
            torch.matmul(a, b.t(), out=c)

        _settle(torch, bf16, 30.0)
        ms = _b2b_ms(torch, stream, bf16, steps)
        rec["bf16_ms"] = round(ms, 5)
        rec["bf16_TFLOP/s"] = round(flops / ms / 1e9, 1)
        rec["bf16_frac_f16_peak"] = round(flops / ms / 1e9 / PEAK_TFLOPS["f16"], 4)
        try:
            f8 = [(a.to(torch.float8_e4m3fn), b.to(torch.float8_e4m3fn)) for a, b, _ in sets]
            one = torch.ones((), device="cuda")

            def fp8(i):
                a, b = f8[i % nsets]
                torch._scaled_mm(a, b.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)

            _settle(torch, fp8, 30.0)
            ms8 = _b2b_ms(torch, stream, fp8, steps)
            rec["fp8_ms"] = round(ms8, 5)
            rec["fp8_TFLOP/s"] = round(flops / ms8 / 1e9, 1)
            rec["fp8_frac_fp8_peak"] = round(flops / ms8 / 1e9 / PEAK_TFLOPS["fp8"], 4)
            del f8
        except (RuntimeError, TypeError) as e:  # no fp8 GEMM for this shape or build
            rec["fp8_error"] = str(e).splitlines()[0][:160]
        out["shapes"][name] = rec
        print(json.dumps({name: rec}), flush=True)
        del sets
        torch.cuda.empty_cache()
    print(json.dumps({"calibration": out}), flush=True)


def _b2b_ms(torch, stream, fn, n):
    """Mean duration of `n` back-to-back calls of `fn(i)` on `stream`, from
    one pair of HIP events around all of them (events between the calls would
    stall the queue and add their own gaps)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def _profiled_traffic():
    """HBM bytes per launch of the GEMM kernel from the committed rocprofv3
    counter summary, or None if the GEMM sources changed since it was taken."""
    prof = os.path.join(ROOT, "profiles", "gemm_attn_proj_2640x3072x3072.md")
    try:
        text = open(prof).read()
        rec = json.loads(re.findall(r"^\{.*\"traffic_bytes_per_launch\".*\}$", text, re.M)[-1])
        csrc = os.path.join(ROOT, "nvfp4_w4a4_block_02_amd", "csrc")
        src = b"".join(open(os.path.join(csrc, f), "rb").read() for f in ("gemm.hip", "device.h"))
        if hashlib.sha256(src).hexdigest()[:16] != rec["source_sha256_16"]:
            return None
        return int(rec["traffic_bytes_per_launch"])
    except (OSError, IndexError, ValueError, KeyError):
        return None


def _dev_bf16(torch, bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def _settle(torch, fn, settle_ms, start=0):
    """Untimed calls fn(i) until the GPU has run them for at least settle_ms
    (synchronizing after each call, so the time is GPU time); returns the
    next call index."""
    t0, i = time.perf_counter(), start
    while (time.perf_counter() - t0) * 1e3 < settle_ms:
        fn(i)
        i += 1
        torch.cuda.synchronize()
    return i


def bench_attn_proj(nv, torch, wl, steps, warmup, nsets, settle_ms):
    d = wl.attn_proj()
    m, k = d["x"].shape
    n = d["w"].shape[0]
    x0 = _dev_bf16(torch, d["x"])
    w0 = torch.from_numpy(d["w"]).cuda()
    sets = []
    for i in range(nsets):
        x = x0.clone()
        wq = nv.quantize(w0.clone())  # offline weight quantization (untimed)
        sets.append({
            "x": x, "wq": wq,
            "xq": nv.NVFP4Tensor.empty(m, k, 1, "cuda"),
            "ws": nv._workspace(nv.OP_QUANTIZE, m, k, "cuda"),
            "y": torch.empty((m, n), dtype=torch.bfloat16, device="cuda"),
        })
    stream = torch.cuda.current_stream()

    def quant(s):
        nv.quantize(s["x"], out=s["xq"], ws=s["ws"], stream=stream)

    def gemm(s):
        nv.gemm(s["xq"], s["wq"], out=s["y"], stream=stream)

    def step(s):
        quant(s)
        gemm(s)

    for i in range(warmup):
        step(sets[i % nsets])
    torch.cuda.synchronize()
    nxt = _settle(torch, lambda i: step(sets[i % nsets]), settle_ms, warmup)
    # The timed region: `steps` steps back to back, nothing else on the
    # stream; wall clock, and one event pair on the stream as a cross-check.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        step(sets[(nxt + i) % nsets])
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_event_ms = e0.elapsed_time(e1) / steps
    # Per-kernel durations, from back-to-back passes over the same rotating
    # buffer sets, each after the same settle: the activation quantize (amax +
    # encode) and the GEMM.
    _settle(torch, lambda i: quant(sets[i % nsets]), settle_ms)
    quant_ms = _b2b_ms(torch, stream, lambda i: quant(sets[i % nsets]), steps)
    _settle(torch, lambda i: gemm(sets[i % nsets]), settle_ms)
    gemm_b2b_ms = _b2b_ms(torch, stream, lambda i: gemm(sets[i % nsets]), steps)
    flops = 2.0 * m * n * k
    quant_bytes = m * k * 2 + m * k // 2 + m * k // 16 + 4
    return {
        "m": m, "n": n, "k": k, "wall_s": wall, "ms_per_step": wall * 1e3 / steps, "step_event_ms": step_event_ms,
        "gemm_ms": gemm_b2b_ms, "quant_ms": quant_ms, "flops": flops, "quant_bytes": quant_bytes,
    }


def _time_loop(torch, fn, sets, steps, warmup, settle_ms=30.0, batches=5):
    """Time of one call of `fn(set)` over `steps` back-to-back calls that
    rotate through `sets` (after `warmup` untimed calls and then at least
    settle_ms of further untimed calls), run as up to `batches` back-to-back
    batches with one event pair each.  Returns the mean over all calls ("ms")
    and the median and minimum of the batch means ("ms_median", "ms_min")."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        fn(sets[i % len(sets)])
    torch.cuda.synchronize()
    _settle(torch, lambda i: fn(sets[i % len(sets)]), settle_ms, warmup)
    nb = max(1, min(batches, steps))
    means, total, i0 = [], 0.0, 0
    for b in range(nb):
        size = steps // nb + (1 if b < steps % nb else 0)
        ms = _b2b_ms(torch, stream, lambda i, i0=i0: fn(sets[(i0 + i) % len(sets)]), size)
        means.append(ms)
        total += ms * size
        i0 += size
    return {"ms": total / steps, "ms_median": float(np.median(means)), "ms_min": float(min(means))}


def copy_rate(torch):
    """Reference rate for the HBM-bound rows: a 256 MiB device-to-device copy
    (torch's copy kernel), read + write bytes over its back-to-back time."""
    src = torch.ones(1 << 26, device="cuda")
    dst = torch.empty_like(src)
    ms = _time_loop(torch, lambda s: dst.copy_(src), [None], 10, 3)["ms"]
    nbytes = 2 * src.numel() * 4
    return {"ms": ms, "GB/s": nbytes / ms / 1e6, "frac_hbm": nbytes / ms / 1e6 / HBM_PEAK_GBS, "bytes": nbytes}


ROWS = ("tiny_linear", "kv_quant", "kv_quant_4over6", "kv_dequant", "kv_window_attention", "rht16_quantize",
        "wgrad_gemm", "ffn_pair", "train_linear_triple")


def bench_rows(nv, torch, wl, steps, warmup, copy_gbs, only, settle_ms):
    """Every row gets its warmup calls and then at least settle_ms of further
    untimed calls: the GPU's clocks take that long to settle after a change
    of load (the window attention measured ~500 us right after the KV codec
    rows and ~430 us once settled)."""
    out = {}
    stream = torch.cuda.current_stream()

    def want(*names):
        return any(nm in only for nm in names)

    def timed(fn, sets, st, wu):
        return _time_loop(torch, fn, sets, st, wu, settle_ms)

    def hbm_row(t, nbytes):
        gbs = nbytes / t["ms"] / 1e6
        return {**t, "GB/s": gbs, "frac_hbm": gbs / HBM_PEAK_GBS, "frac_copy": gbs / copy_gbs, "bytes": nbytes}

    def flop_row(t, flops):
        tf = flops / t["ms"] / 1e9
        return {**t, "TFLOP/s": tf, "frac_f16_peak": tf / PEAK_TFLOPS["f16"]}
    # Tiny W4A4 linear (workload 1): activation quantize of A fp32 256x512 +
    # GEMM against the pre-quantized 512x512 weight, float32 out; latency.
    if want("tiny_linear"):
        d = wl.tiny_linear()
        m, k = d["a"].shape
        n = d["w"].shape[0]
        tsets = []
        for i in range(4):
            tsets.append({"a": torch.from_numpy(d["a"]).cuda(), "wq": nv.quantize(torch.from_numpy(d["w"]).cuda()),
                          "aq": nv.NVFP4Tensor.empty(m, k, 1, "cuda"), "ws": nv._workspace(nv.OP_QUANTIZE, m, k, "cuda"),
                          "c": torch.empty((m, n), dtype=torch.float32, device="cuda")})

        def tiny(s):  # one C call: activation quantize + GEMM (nvfp4_linear)
            nv.linear(s["a"], s["wq"], xq=s["aq"], ws=s["ws"], out=s["c"], stream=stream)

        t = timed(tiny, tsets, max(steps, 20), warmup)
        out["tiny_linear"] = {**flop_row(t, 2.0 * m * n * k), "us": t["ms"] * 1e3}
        # The same call captured GC times (rotating over the buffer sets)
        # into one HIP graph and replayed: the per-call time of the GPU work
        # and its launch-to-launch gaps, without the host's per-call cost
        # (Python and ctypes take longer per call than the kernels here).  The
        # library allocates nothing and clears no memory with memset, so the
        # captured sequence is the eager one.
        GC = 32

        def graph_us(fn):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(GC):
                    fn(tsets[i % len(tsets)])
            return timed(lambda g: g.replay(), [g], max(steps // 4, 5), max(warmup // 8, 2))["ms"] * 1e3 / GC

        out["tiny_linear"]["graph_us"] = graph_us(
            lambda s: nv.linear(s["a"], s["wq"], xq=s["aq"], ws=s["ws"], out=s["c"]))
        del tsets
    # KV codec: K and V [12, 880, 24, 128] bf16, 8-frame blocks.
    shape = (12, 880, 24, 128)
    elems = 2 * 12 * 880 * 24 * 128
    kv_bytes = elems * 2 + elems // 2 + elems // 16 + 2 * 2 * 4
    if want("kv_quant", "kv_quant_4over6", "kv_dequant"):
        d = wl.kv_cache()
        kvsets = []
        for i in range(4):  # 4 sets x (2 x 65 MB in + 2 x 18 MB codes + 2 x 65 MB out) > 256 MB
            s = {}
            for nm in ("k", "v"):
                s[nm] = _dev_bf16(torch, d[nm]).reshape(shape)
                s[nm + "q"] = nv.NVFP4Tensor.empty(12 * 880 * 24, 128, 2, "cuda")
                s[nm + "o"] = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
            s["ws"] = nv._workspace(nv.OP_KV_QUANT_PAIR, 12, 8, "cuda")
            kvsets.append(s)

        # K and V in one call (nvfp4_kv_quant_pair: one amax and one encode
        # launch for both); the rows also carry the time of two one-tensor
        # calls (four launches) for comparison.
        def kvq(s, fo6=False):
            nv.kv_quant_pair(s["k"], s["v"], k_out=s["kq"], v_out=s["vq"], ws=s["ws"], stream=stream,
                             four_over_six=fo6)

        def kvq6(s):
            kvq(s, True)

        def kvq_two(s, fo6=False):
            nv.kv_quant(s["k"], out=s["kq"], ws=s["ws"], stream=stream, four_over_six=fo6)
            nv.kv_quant(s["v"], out=s["vq"], ws=s["ws"], stream=stream, four_over_six=fo6)

        def kvd(s):  # K and V in one launch (nvfp4_kv_dequant_pair)
            nv.kv_dequant_pair(s["kq"], s["vq"], shape, k_out=s["ko"], v_out=s["vo"], stream=stream)

        def kvd_two(s):
            nv.kv_dequant(s["kq"], shape, out=s["ko"], stream=stream)
            nv.kv_dequant(s["vq"], shape, out=s["vo"], stream=stream)

        if want("kv_quant"):
            out["kv_quant"] = hbm_row(timed(kvq, kvsets, steps, warmup), kv_bytes)
            out["kv_quant"]["ms_two_calls"] = timed(kvq_two, kvsets, steps, warmup)["ms"]
        if want("kv_quant_4over6"):
            out["kv_quant_4over6"] = hbm_row(timed(kvq6, kvsets, steps, warmup), kv_bytes)
            out["kv_quant_4over6"]["ms_two_calls"] = timed(lambda s: kvq_two(s, True), kvsets, steps, warmup)["ms"]
        if want("kv_dequant"):
            kvq(kvsets[0]), kvq(kvsets[1]), kvq(kvsets[2]), kvq(kvsets[3])
            out["kv_dequant"] = hbm_row(timed(kvd, kvsets, steps, warmup), kv_bytes)
            out["kv_dequant"]["ms_two_calls"] = timed(kvd_two, kvsets, steps, warmup)["ms"]
        del kvsets
    # Window attention reading the NVFP4 KV cache directly: the chunk's 3
    # latent frames of queries against the 12-frame cache (frame-causal).
    if want("kv_window_attention"):
        d = wl.window_attention()
        fr, tk, hd, dd = 12, 880, 24, 128
        asets = []
        for i in range(3):
            kk = _dev_bf16(torch, d["k"]).reshape(fr, tk, hd, dd)
            vv = _dev_bf16(torch, d["v"]).reshape(fr, tk, hd, dd)
            s = {"q": _dev_bf16(torch, d["q"]).reshape(3 * tk, hd, dd), "k": nv.kv_quant(kk), "v": nv.kv_quant(vv)}
            s["o"] = torch.empty_like(s["q"])
            asets.append(s)
            del kk, vv

        def attn(s):
            nv.kv_attention(s["q"], s["k"], s["v"], (fr, tk, hd, dd), 8, out=s["o"], stream=stream)

        pairs = sum((fr - 3 + f + 1) * tk for f in range(3)) * tk      # visible (query, key) pairs per head
        out["kv_window_attention"] = flop_row(timed(attn, asets, max(steps // 2, 5), 20), 4.0 * pairs * dd * hd)
        del asets
    # RHT16 + quantize along dim 0, and the weight-gradient GEMM.
    if want("rht16_quantize", "wgrad_gemm"):
        d = wl.rht_wgrad()
        rows, cols = d["g"].shape
        rsets = []
        for i in range(3):
            s = {"g": _dev_bf16(torch, d["g"]), "x": _dev_bf16(torch, d["x"]),
                 "gq": nv.NVFP4Tensor.empty(cols, rows, 1, "cuda"), "ws": nv._workspace(nv.OP_RHT16, rows, cols, "cuda")}
            s["xq"] = nv.rht16_quantize(s["x"], d["mask"], axis=0)
            nv.rht16_quantize(s["g"], d["mask"], axis=0, out=s["gq"], ws=s["ws"])
            s["c"] = torch.empty((cols, cols), dtype=torch.float32, device="cuda")
            rsets.append(s)

        def rq(s):
            nv.rht16_quantize(s["g"], d["mask"], axis=0, out=s["gq"], ws=s["ws"], stream=stream)

        def wg(s):
            nv.gemm(s["gq"], s["xq"], out=s["c"], stream=stream)

        rbytes = rows * cols * 2 + rows * cols // 2 + rows * cols // 16 + 4
        if want("rht16_quantize"):
            out["rht16_quantize"] = hbm_row(timed(rq, rsets, steps, warmup), rbytes)
        if want("wgrad_gemm"):
            out["wgrad_gemm"] = flop_row(timed(wg, rsets, max(steps // 2, 5), 20), 2.0 * cols * cols * rows)
        del rsets
    # FFN pair.
    if want("ffn_pair"):
        d = wl.ffn()
        m, dm = d["x"].shape
        f = d["w1"].shape[0]
        x = _dev_bf16(torch, d["x"])
        w1 = nv.quantize(torch.from_numpy(d["w1"]).cuda())
        w2 = nv.quantize(torch.from_numpy(d["w2"]).cuda())
        bufs = {"xq": nv.NVFP4Tensor.empty(m, dm, 1, "cuda"), "ws": nv._workspace(nv.OP_QUANTIZE, m, dm, "cuda"),
                "h": torch.empty((m, f), dtype=torch.float32, device="cuda"),
                "hmax": torch.empty(1, device="cuda"), "hq": nv.NVFP4Tensor.empty(m, f, 1, "cuda"),
                "y": torch.empty((m, dm), dtype=torch.bfloat16, device="cuda")}

        def ffn(s):
            nv.ffn(x, w1, w2, bufs=bufs, stream=stream)

        out["ffn_pair"] = flop_row(timed(ffn, [None], max(steps // 5, 3), 5), 2.0 * m * dm * f * 2)
        del bufs, x, w1, w2
    # Training triple of one linear layer at the attention-projection shape:
    # six quantizations (two with the RHT16) and three GEMMs per step.
    if want("train_linear_triple"):
        d = wl.train_linear()
        m, k = d["x"].shape
        n = d["w"].shape[0]
        tsets = []
        for i in range(3):
            s = {"x": _dev_bf16(torch, d["x"]), "w": torch.from_numpy(d["w"]).cuda(), "dy": _dev_bf16(torch, d["dy"])}
            s["bufs"] = {"xq": nv.NVFP4Tensor.empty(m, k, 1, "cuda"), "wq": nv.NVFP4Tensor.empty(n, k, 1, "cuda"),
                         "dyq": nv.NVFP4Tensor.empty(m, n, 1, "cuda"), "wtq": nv.NVFP4Tensor.empty(k, n, 1, "cuda"),
                         "dyt": nv.NVFP4Tensor.empty(n, -(-m // 256) * 256, 1, "cuda"),
                         "xt": nv.NVFP4Tensor.empty(k, -(-m // 256) * 256, 1, "cuda"),
                         "y": torch.empty((m, n), dtype=torch.bfloat16, device="cuda"),
                         "dx": torch.empty((m, k), dtype=torch.bfloat16, device="cuda"),
                         "dw": torch.empty((n, k), dtype=torch.float32, device="cuda"),
                         "ws": nv._workspace(nv.OP_RHT16, m, max(k, n), "cuda"),
                         "ws1": nv._workspace(nv.OP_RHT16, m, max(k, n), "cuda"),
                         "ws2": nv._workspace(nv.OP_RHT16, m, max(k, n), "cuda"),
                         "wamax": torch.empty(1, dtype=torch.float32, device="cuda")}
            tsets.append(s)

        def train(s):
            nv.linear_train(s["x"], s["w"], s["dy"], d["mask"], bufs=s["bufs"], stream=stream)

        out["train_linear_triple"] = flop_row(timed(train, tsets, max(steps // 2, 5), 30), 3 * 2.0 * m * n * k)
        del tsets
    return out


# ---------------------------------------------------------------- CPU oracle
def _host_threads():
    """Host thread counts: os.cpu_count(), the CPUs this process may run on,
    and the BLAS threads NumPy's dgemm uses."""
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    return os.cpu_count() or 1, len(os.sched_getaffinity(0)), int(blas)


def _chunks(n, parts):
    step = -(-n // parts)
    return [slice(i, min(n, i + step)) for i in range(0, n, step)]


def _pool_quantize(pool, oracle, x, workers):
    """oracle.quantize of a float32 matrix with the element-wise work spread
    over row chunks on the pool: the tensor amax first (max of the chunk
    maxima, exact), then quantize_with_amax of every chunk with it."""
    ch = _chunks(x.shape[0], workers)
    a = np.float32(max(pool.map(lambda c: float(oracle.amax(x[c])), ch)))
    qs = list(pool.map(lambda c: oracle.quantize_with_amax(np.ascontiguousarray(x[c]), a), ch))
    return oracle.QTensor(np.concatenate([q.codes for q in qs]), np.concatenate([q.scales for q in qs]), qs[0].tscale)


def _timed_reps(fn, budget_s, max_reps=50):
    """Run fn() until budget_s has passed (at least once); (reps, seconds)."""
    t0, reps = time.perf_counter(), 0
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= max_reps:
            return reps, el


def cpu_baselines(wl, budget_s=4.0):
    """The oracle, as it stands, on a bounded sample of each workload, on this
    host: element-wise codec work over row chunks on a thread pool (one
    worker per CPU this process may use), float64 GEMMs on the BLAS threads.
    Each config runs for about budget_s."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    ncpu, naff, blas = _host_threads()
    workers = max(1, naff)
    res = {}
    with ThreadPoolExecutor(workers) as pool:
        # 1: tiny linear, whole (quantize A + GEMM against the pre-quantized W)
        d = wl.tiny_linear()
        wq = oracle.quantize(d["w"])
        reps, el = _timed_reps(lambda: oracle.gemm_ref(_pool_quantize(pool, oracle, d["a"], workers), wq,
                                                       want_bound=False), budget_s)
        fl = 2.0 * 256 * 512 * 512
        res["1_tiny_linear"] = {"value": el / reps * 1e6, "unit": "us", "TFLOP/s": fl * reps / el / 1e12,
                                "sample": f"whole workload, {reps} reps"}
        # 2: attention projection, a quarter of the tokens per rep
        d = wl.attn_proj()
        x = (d["x"].astype(np.uint32) << 16).view(np.float32)
        wq = oracle.quantize(d["w"])
        rows = 660
        reps, el = _timed_reps(lambda: oracle.gemm_ref(_pool_quantize(pool, oracle, x[:rows], workers), wq,
                                                       want_bound=False), budget_s)
        res["2_attn_proj"] = {"value": 2.0 * rows * 3072 * 3072 * reps / el / 1e12, "unit": "TFLOP/s",
                              "sample": f"{rows} of 2640 token rows (act quantize + float64 GEMM), {reps} reps"}
        del x, wq
        # 3: FFN pair on 264 token rows (its own X and H tensor scales)
        d = wl.ffn(m=264)
        x = (d["x"].astype(np.uint32) << 16).view(np.float32)
        w1, w2 = oracle.quantize(d["w1"]), oracle.quantize(d["w2"])

        def ffn():
            c1, _ = oracle.gemm_ref(_pool_quantize(pool, oracle, x, workers), w1, want_bound=False)
            h = oracle.gelu_tanh(c1).astype(np.float32)
            oracle.gemm_ref(_pool_quantize(pool, oracle, h, workers), w2, want_bound=False)

        reps, el = _timed_reps(ffn, budget_s)
        res["3_ffn_pair"] = {"value": 4.0 * 264 * 3072 * 14336 * reps / el / 1e12, "unit": "TFLOP/s",
                             "sample": f"264 of 10560 token rows through the whole chain, {reps} reps"}
        del x, w1, w2
        # 4: KV codec on one frame of K (quantize, then bf16 dequantize)
        d = wl.kv_cache(frames=1)
        k1 = (d["k"].astype(np.uint32) << 16).view(np.float32).reshape(-1, 128)
        nb = k1.size * 2 + k1.size // 2 + k1.size // 16 + 4
        qk = _pool_quantize(pool, oracle, k1, workers)
        reps, el = _timed_reps(lambda: _pool_quantize(pool, oracle, k1, workers), budget_s / 2)
        res["4_kv_quant"] = {"value": nb * reps / el / 1e9, "unit": "GB/s",
                             "sample": f"1 of 12 frames of K (880x24x128), {reps} reps"}
        ch = _chunks(qk.rows, workers)
        deq = lambda: list(pool.map(lambda c: oracle.dequantize(oracle.QTensor(qk.codes[c], qk.scales[c], qk.tscale),
                                                                out="bf16"), ch))
        reps, el = _timed_reps(deq, budget_s / 2)
        res["4_kv_dequant"] = {"value": nb * reps / el / 1e9, "unit": "GB/s",
                               "sample": f"1 of 12 frames of K (880x24x128), {reps} reps"}
        del k1, qk
        # 5: RHT16 + quantize along dim 0 of 1024 gradient rows; the wgrad
        # GEMM over a 1024-long slice of its 16384-long reduction
        d = wl.rht_wgrad(rows=1024)
        g = (d["g"].astype(np.uint32) << 16).view(np.float32)
        xs = (d["x"].astype(np.uint32) << 16).view(np.float32)
        nb = g.size * 2 + g.size // 2 + g.size // 16 + 4

        def rht_q(a):
            t = np.ascontiguousarray(a.T)
            parts = list(pool.map(lambda c: oracle.rht16_rows(t[c], d["mask"]), _chunks(t.shape[0], workers)))
            return _pool_quantize(pool, oracle, np.concatenate(parts), workers)

        reps, el = _timed_reps(lambda: rht_q(g), budget_s / 2)
        res["5_rht16_quantize"] = {"value": nb * reps / el / 1e9, "unit": "GB/s",
                                   "sample": f"1024 of 16384 gradient rows, {reps} reps"}
        gq, xq = rht_q(g), rht_q(xs)
        reps, el = _timed_reps(lambda: oracle.gemm_ref(gq, xq, want_bound=False), budget_s / 2)
        res["5_wgrad_gemm"] = {"value": 2.0 * 3072 * 3072 * 1024 * reps / el / 1e12, "unit": "TFLOP/s",
                               "sample": f"reduction slice of 1024 of 16384, {reps} reps"}
    return res, {"os_cpu_count": ncpu, "affinity_cpus": naff, "blas_threads": blas, "pool_workers": workers}


def main():
    a = _args()
    if a.calibrate:
        calibrate(max(a.steps, 20))
        return
    if a.copy_probe:
        copy_probe()
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {a.gpus} is not supported by this build "
              "(the NVFP4 path here has no multi-GPU component)", file=sys.stderr)
        sys.exit(2)
    only = set(x for x in a.only.split(",") if x) or set(ROWS)
    unknown = only - set(ROWS)
    if unknown:
        print(f"unknown rows {sorted(unknown)}; rows are {list(ROWS)}", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads as wl
    import nvfp4_w4a4_block_02_amd as nv

    torch.cuda.init()
    copy = copy_rate(torch)
    line = {"metric": METRIC}
    r = None
    if not a.no_headline:
        r = bench_attn_proj(nv, torch, wl, a.steps, a.warmup, a.sets, a.settle_ms)
        tf = r["flops"] / (r["ms_per_step"] * 1e-3) / 1e12
        gemm_tf = r["flops"] / (r["gemm_ms"] * 1e-3) / 1e12
        line.update({
            "value": round(tf, 2),
            "unit": "TFLOP/s",
            "n_gpus": 1,
            "steps": a.steps,
            "warmup": a.warmup,
            "settle_ms": a.settle_ms,
            "ms_per_step": round(r["ms_per_step"], 5),
            "ms_per_step_events": round(r["step_event_ms"], 5),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "f16",
            "data": "synthetic",
            "config": {"workload": "dit_attn_proj_2640x3072x3072", "M": r["m"], "N": r["n"], "K": r["k"],
                       "act_in": "bf16", "weights": "nvfp4 (pre-quantized)", "out": "bf16",
                       "parallelism": "none (1 GPU)"},
            "roofline": {"bound": "mfma", "achieved": round(gemm_tf, 2), "peak": PEAK_TFLOPS["f16"],
                         "unit": "TFLOP/s", "frac": round(gemm_tf / PEAK_TFLOPS["f16"], 4),
                         "traffic": _profiled_traffic(), "kernel": "gemm_lds_kernel (nvfp4_gemm)",
                         "kernel_ms": round(r["gemm_ms"], 5),
                         "frac_fp8_peak": round(gemm_tf / PEAK_TFLOPS["fp8"], 4),
                         "frac_fp4_peak": round(gemm_tf / PEAK_TFLOPS["fp4"], 4)},
            "act_quant": {"ms": round(r["quant_ms"], 5), "GB/s": round(r["quant_bytes"] / r["quant_ms"] / 1e6, 1),
                          "frac_hbm": round(r["quant_bytes"] / r["quant_ms"] / 1e6 / HBM_PEAK_GBS, 4),
                          "frac_copy": round(r["quant_bytes"] / r["quant_ms"] / 1e6 / copy["GB/s"], 4),
                          "plus_gemm_ms": round(r["quant_ms"] + r["gemm_ms"], 5)},
        })
    line["device_copy"] = {k: (round(v, 5) if isinstance(v, float) else v) for k, v in copy.items()}
    rows = {}
    if not a.no_rows:
        rows = bench_rows(nv, torch, wl, max(a.steps // 2, 5), max(a.warmup // 2, 2), copy["GB/s"], only,
                          a.settle_ms)
        line["rows"] = {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                        for k, v in rows.items()}
    if not a.no_cpu and r is not None:
        per, threads = cpu_baselines(wl)
        gpu = {"1_tiny_linear": rows.get("tiny_linear", {}).get("us"),
               "2_attn_proj": line["value"],
               "3_ffn_pair": rows.get("ffn_pair", {}).get("TFLOP/s"),
               "4_kv_quant": (rows.get("kv_quant", {}).get("GB/s")),
               "4_kv_dequant": (rows.get("kv_dequant", {}).get("GB/s")),
               "5_rht16_quantize": rows.get("rht16_quantize", {}).get("GB/s"),
               "5_wgrad_gemm": rows.get("wgrad_gemm", {}).get("TFLOP/s")}
        for key, v in per.items():
            g = gpu.get(key)
            if g:
                v["gpu"] = round(g, 4)
                v["gpu_speedup"] = round(v["value"] / g if v["unit"] == "us" else g / v["value"], 1)
            v["value"] = round(v["value"], 6)
        c2 = per["2_attn_proj"]
        line["cpu_baseline"] = {"value": c2["value"], "unit": "TFLOP/s",
                                "cores": max(threads["pool_workers"], threads["blas_threads"]), "kind": "oracle",
                                "sample": c2["sample"] + "; codec element-wise on " + str(threads["pool_workers"])
                                          + " pool threads, float64 GEMM on " + str(threads["blas_threads"])
                                          + " BLAS threads",
                                **threads, "per_config": per}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

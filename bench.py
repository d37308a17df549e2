"""Benchmark of the NVFP4 W4A4 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-rows] [--no-cpu]

One step = one pass of the attention-projection workload of the 5B DiT
(2640 tokens = 3 latent frames x 880, width 3072): amax of the bf16
activations, their NVFP4 encode, and the block-scaled W4A4 GEMM against
pre-quantized 3072x3072 NVFP4 weights into bf16.  The timed region starts
with every input resident in HBM; buffers rotate over 13 independent sets
(> 512 MB) so the 256 MB Infinity Cache cannot serve a step from the last
one.  The timed steps run back to back with nothing between them (a HIP
event recorded between two kernels idles the GPU for ~10 us on this part, so
per-kernel events would distort the step time); per-kernel durations come
from separate back-to-back passes over the same buffers, each timed by one
pair of HIP events on the launch stream.  Prints ONE JSON line.

Besides the headline value the line carries:
  roofline      the GEMM kernel (the dominant kernel): its algorithmic
                flops per launch / its mean duration over back-to-back
                launches on the launch stream;
  cpu_baseline  the CPU oracle timed on a bounded sample of the same
                workload on this host;
  device_copy   a 256 MiB device-to-device copy (read + write bytes per
                second): the practical HBM rate that the HBM-bound rows are
                also quoted against (frac_copy), beside the 8 TB/s datasheet
                peak (frac_hbm);
  rows          the other rows of the path, each timed back to back the same
                way in five batches (ms = mean over all calls; ms_median and
                ms_min of the batch means), in this order: KV codec quantize (core recipe and Four
                Over Six) and dequantize (12x880x24x128 bf16, K and V); the
                frame-causal window attention of 2640 queries (3 latent
                frames) x 24 heads over that 12-frame NVFP4 KV cache, read
                directly (flops counted over the visible query-key pairs);
                RHT16 + quantize of a 16384x3072 gradient along dim 0 and the
                3072x3072x16384 weight-gradient GEMM; the FFN pair
                (10560x3072 -> 14336 -> 3072); the NVFP4 training triple
                (forward, input and weight gradient, with the six operand
                quantizations) of a 2640x3072x3072 linear layer.
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
    p.add_argument("--sets", type=int, default=13, help="rotating buffer sets")
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


def bench_attn_proj(nv, torch, wl, steps, warmup, nsets):
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

    def step(s):
        nv.quantize(s["x"], out=s["xq"], ws=s["ws"], stream=stream)
        nv.gemm(s["xq"], s["wq"], out=s["y"], stream=stream)

    for i in range(warmup):
        step(sets[i % nsets])
    torch.cuda.synchronize()
    # The timed region: `steps` steps back to back, nothing else on the
    # stream; wall clock, and one event pair on the stream as a cross-check.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        step(sets[i % nsets])
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_event_ms = e0.elapsed_time(e1) / steps
    # Per-kernel durations, from back-to-back passes over the same rotating
    # buffer sets: the activation quantize (amax + encode) and the GEMM.
    quant_ms = _b2b_ms(torch, stream, lambda i: nv.quantize(sets[i % nsets]["x"], out=sets[i % nsets]["xq"],
                                                           ws=sets[i % nsets]["ws"], stream=stream), steps)
    gemm_b2b_ms = _b2b_ms(torch, stream, lambda i: nv.gemm(sets[i % nsets]["xq"], sets[i % nsets]["wq"],
                                                          out=sets[i % nsets]["y"], stream=stream), steps)
    flops = 2.0 * m * n * k
    quant_bytes = m * k * 2 + m * k // 2 + m * k // 16 + 4
    return {
        "m": m, "n": n, "k": k, "wall_s": wall, "ms_per_step": wall * 1e3 / steps, "step_event_ms": step_event_ms,
        "gemm_ms": gemm_b2b_ms, "quant_ms": quant_ms, "flops": flops, "quant_bytes": quant_bytes,
    }


def _time_loop(torch, fn, sets, steps, warmup, batches=5):
    """Time of one call of `fn(set)` over `steps` back-to-back calls that
    rotate through `sets` (after `warmup` untimed calls), run as up to
    `batches` back-to-back batches with one event pair each.  Returns the
    mean over all calls ("ms") and the median and minimum of the batch means
    ("ms_median", "ms_min")."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        fn(sets[i % len(sets)])
    torch.cuda.synchronize()
    # then untimed calls until the row has run for at least 30 ms: the clocks
    # take that long to settle after a change of load
    t0, i = time.perf_counter(), warmup
    while time.perf_counter() - t0 < 0.03:
        fn(sets[i % len(sets)])
        i += 1
        torch.cuda.synchronize()
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


def bench_rows(nv, torch, wl, steps, warmup, copy_gbs):
    """Every row gets its warmup calls and then at least 30 ms of further
    untimed calls: the GPU's clocks take that long to settle after a change
    of load (the window attention measured ~500 us right after the KV codec
    rows and ~430 us once settled)."""
    out = {}
    stream = torch.cuda.current_stream()

    def hbm_row(t, nbytes):
        gbs = nbytes / t["ms"] / 1e6
        return {**t, "GB/s": gbs, "frac_hbm": gbs / HBM_PEAK_GBS, "frac_copy": gbs / copy_gbs, "bytes": nbytes}

    def flop_row(t, flops):
        tf = flops / t["ms"] / 1e9
        return {**t, "TFLOP/s": tf, "frac_f16_peak": tf / PEAK_TFLOPS["f16"]}
    # KV codec: K and V [12, 880, 24, 128] bf16, 8-frame blocks.
    d = wl.kv_cache()
    shape = (12, 880, 24, 128)
    kvsets = []
    for i in range(4):  # 4 sets x (2 x 65 MB in + 2 x 18 MB codes + 2 x 65 MB out) > 256 MB
        s = {}
        for nm in ("k", "v"):
            s[nm] = _dev_bf16(torch, d[nm]).reshape(shape)
            s[nm + "q"] = nv.NVFP4Tensor.empty(12 * 880 * 24, 128, 2, "cuda")
            s[nm + "o"] = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        s["ws"] = nv._workspace(nv.OP_KV_QUANT, 12, 8, "cuda")
        kvsets.append(s)

    def kvq(s):
        nv.kv_quant(s["k"], out=s["kq"], ws=s["ws"], stream=stream)
        nv.kv_quant(s["v"], out=s["vq"], ws=s["ws"], stream=stream)

    def kvq6(s):
        nv.kv_quant(s["k"], out=s["kq"], ws=s["ws"], stream=stream, four_over_six=True)
        nv.kv_quant(s["v"], out=s["vq"], ws=s["ws"], stream=stream, four_over_six=True)

    def kvd(s):
        nv.kv_dequant(s["kq"], shape, out=s["ko"], stream=stream)
        nv.kv_dequant(s["vq"], shape, out=s["vo"], stream=stream)

    elems = 2 * 12 * 880 * 24 * 128
    kv_bytes = elems * 2 + elems // 2 + elems // 16 + 2 * 2 * 4
    out["kv_quant"] = hbm_row(_time_loop(torch, kvq, kvsets, steps, warmup), kv_bytes)
    out["kv_quant_4over6"] = hbm_row(_time_loop(torch, kvq6, kvsets, steps, warmup), kv_bytes)
    out["kv_dequant"] = hbm_row(_time_loop(torch, kvd, kvsets, steps, warmup), kv_bytes)
    del kvsets
    # Window attention reading the NVFP4 KV cache directly: the chunk's 3
    # latent frames of queries against the 12-frame cache (frame-causal).
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
    out["kv_window_attention"] = flop_row(_time_loop(torch, attn, asets, max(steps // 2, 5), 20),
                                          4.0 * pairs * dd * hd)
    del asets
    # RHT16 + quantize along dim 0, and the weight-gradient GEMM.
    d = wl.rht_wgrad()
    rows, cols = d["g"].shape
    rsets = []
    for i in range(3):
        s = {"g": _dev_bf16(torch, d["g"]), "x": _dev_bf16(torch, d["x"]),
             "gq": nv.NVFP4Tensor.empty(cols, rows, 1, "cuda"), "ws": nv._workspace(nv.OP_RHT16, rows, cols, "cuda")}
        s["xq"] = nv.rht16_quantize(s["x"], d["mask"], axis=0)
        s["c"] = torch.empty((cols, cols), dtype=torch.float32, device="cuda")
        rsets.append(s)

    def rq(s):
        nv.rht16_quantize(s["g"], d["mask"], axis=0, out=s["gq"], ws=s["ws"], stream=stream)

    def wg(s):
        nv.gemm(s["gq"], s["xq"], out=s["c"], stream=stream)

    rbytes = rows * cols * 2 + rows * cols // 2 + rows * cols // 16 + 4
    out["rht16_quantize"] = hbm_row(_time_loop(torch, rq, rsets, steps, warmup), rbytes)
    out["wgrad_gemm"] = flop_row(_time_loop(torch, wg, rsets, max(steps // 2, 5), 20), 2.0 * cols * cols * rows)
    del rsets
    # FFN pair.
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

    out["ffn_pair"] = flop_row(_time_loop(torch, ffn, [None], max(steps // 5, 3), 5), 2.0 * m * dm * f * 2)
    del bufs, x, w1, w2
    # Training triple of one linear layer at the attention-projection shape:
    # six quantizations (two with the RHT16) and three GEMMs per step.
    d = wl.train_linear()
    m, k = d["x"].shape
    n = d["w"].shape[0]
    tsets = []
    for i in range(3):
        s = {"x": _dev_bf16(torch, d["x"]), "w": torch.from_numpy(d["w"]).cuda(), "dy": _dev_bf16(torch, d["dy"])}
        s["bufs"] = {"xq": nv.NVFP4Tensor.empty(m, k, 1, "cuda"), "wq": nv.NVFP4Tensor.empty(n, k, 1, "cuda"),
                     "dyq": nv.NVFP4Tensor.empty(m, n, 1, "cuda"), "wtq": nv.NVFP4Tensor.empty(k, n, 1, "cuda"),
                     "dyt": nv.NVFP4Tensor.empty(n, -(-m // 128) * 128, 1, "cuda"),
                     "xt": nv.NVFP4Tensor.empty(k, -(-m // 128) * 128, 1, "cuda"),
                     "y": torch.empty((m, n), dtype=torch.bfloat16, device="cuda"),
                     "dx": torch.empty((m, k), dtype=torch.bfloat16, device="cuda"),
                     "dw": torch.empty((n, k), dtype=torch.float32, device="cuda"),
                     "ws": nv._workspace(nv.OP_RHT16, m, max(k, n), "cuda"),
                     "wamax": torch.empty(1, dtype=torch.float32, device="cuda")}
        tsets.append(s)

    def train(s):
        nv.linear_train(s["x"], s["w"], s["dy"], d["mask"], bufs=s["bufs"], stream=stream)

    out["train_linear_triple"] = flop_row(_time_loop(torch, train, tsets, max(steps // 2, 5), 30), 3 * 2.0 * m * n * k)
    del tsets
    return out


def cpu_baseline(wl):
    """The oracle, as it stands, on the attention-projection workload: act
    quantize of the sampled rows + float64 GEMM against the (untimed,
    pre-quantized) weights."""
    import oracle

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    d = wl.attn_proj()
    x = (d["x"].astype(np.uint32) << 16).view(np.float32)
    wq = oracle.quantize(d["w"])
    rows = 660  # a quarter of the 2640 tokens
    t0 = time.perf_counter()
    reps = 0
    while True:
        xq = oracle.quantize(x[:rows] if reps % 2 == 0 else x[rows:2 * rows])
        oracle.gemm_ref(xq, wq, want_bound=False)
        reps += 1
        el = time.perf_counter() - t0
        if el > 10.0 or reps >= 40:
            break
    fl = 2.0 * rows * d["w"].shape[0] * d["w"].shape[1] * reps
    return {"value": fl / el / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"{reps} x (quantize {rows}x3072 bf16 rows + float64 GEMM against 3072x3072 NVFP4 weights), "
                      f"{el:.1f} s; element-wise codec single-threaded NumPy, GEMM on {blas_threads} BLAS threads"}


def main():
    a = _args()
    if a.copy_probe:
        copy_probe()
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {a.gpus} is not supported by this build "
              "(the NVFP4 path here has no multi-GPU component)", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads as wl
    import nvfp4_w4a4_block_02_amd as nv

    torch.cuda.init()
    r = bench_attn_proj(nv, torch, wl, a.steps, a.warmup, a.sets)
    copy = copy_rate(torch)
    tf = r["flops"] / (r["ms_per_step"] * 1e-3) / 1e12
    gemm_tf = r["flops"] / (r["gemm_ms"] * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(tf, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
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
                     "unit": "TFLOP/s", "frac": round(gemm_tf / PEAK_TFLOPS["f16"], 4), "traffic": _profiled_traffic(),
                     "kernel": "gemm_lds_kernel (nvfp4_gemm)", "kernel_ms": round(r["gemm_ms"], 5),
                     "frac_fp8_peak": round(gemm_tf / PEAK_TFLOPS["fp8"], 4),
                     "frac_fp4_peak": round(gemm_tf / PEAK_TFLOPS["fp4"], 4)},
        "act_quant": {"ms": round(r["quant_ms"], 5), "GB/s": round(r["quant_bytes"] / r["quant_ms"] / 1e6, 1),
                      "frac_hbm": round(r["quant_bytes"] / r["quant_ms"] / 1e6 / HBM_PEAK_GBS, 4),
                      "frac_copy": round(r["quant_bytes"] / r["quant_ms"] / 1e6 / copy["GB/s"], 4)},
        "device_copy": {k: (round(v, 5) if isinstance(v, float) else v) for k, v in copy.items()},
    }
    if not a.no_rows:
        rows = bench_rows(nv, torch, wl, max(a.steps // 2, 5), max(a.warmup // 2, 2), copy["GB/s"])
        line["rows"] = {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                        for k, v in rows.items()}
    if not a.no_cpu:
        cb = cpu_baseline(wl)
        cb["value"] = round(cb["value"], 6)
        line["cpu_baseline"] = cb
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the W4A16 group-wise INT4 hot path on one MI355X.

Metric: W4A16 GEMV achieved HBM GB/s at M=1 on the 7B-like decode projections
(4096x4096 and 11008x4096, group 128, asymmetric), with the prefill GEMM TFLOP/s (70B-like
28672x8192, M=2048) and the quantize/pack GB/s of the 32-layer 7B-like checkpoint in the
same JSON line.

A timed step is one decode pass: the W4A16 GEMV over both projections at M=1, issued as
one grouped call (q4_w4a16_gemm_grouped: both problems in one launch of the decode
kernel).  The same projections issued as two single-problem calls are measured too and
reported under "single_launches".  Each step reads a different copy of the packed
weights (the copies together are four times the 256 MB Infinity Cache), so every step
streams its weights from HBM.  The steps are replayed from captured HIP graphs (the
launches themselves are identical to direct calls; the graph removes the Python/ctypes
launch cost of ~7 us per call, which would otherwise dominate the ~10 us kernels).
Inputs are resident in HBM before the timed region starts.

Algorithmic bytes (what the method must move, nothing else):
  GEMV   per launch: n*k/2 (codes) + 2*n*k/g (fp16 scales) + 4*n*ceil(k/g/8) (zeros)
                     + 2*m*k (x, bf16) + 4*m*n (y, fp32)
  GEMM   2*m*n*k flop against the bf16 dense MFMA peak
  quantize per weight: 2 (bf16 read) + 0.5 (codes); per group 2 (scale) + 0.5 (zero)
  GPTQ     fp32 work: k^2 * tokens (Hessian) + k^3/3 (Cholesky) + n * k^2 (updates), against the
           fp32 matrix peak (157.3 TFLOP/s: the tile products run on v_mfma_f32_32x32x2_f32)
  MSE clip search: 110 vector operations per weight (10 per candidate ratio, 11 ratios)
           against the vector ALU (39.3e12 lane operations per second)
  KV attention per layer: both INT4 caches over the context (per token and head
                     d/2 codes + 2*d/g scale bytes + 4*ceil(d/g/8) zero-word bytes, each),
                     q (bf16), out (fp32)

Prints one JSON line.  ``--gpus`` above 1 is refused: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix (v_mfma_f32_*_f32), TFLOP/s
# The clip search is bound by the vector ALU: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz =
# 39.3e12 lane operations per second (fp32 and fp64 adds and multiplies issue at the same
# rate; no packed math).  Its algorithmic work per weight and candidate ratio: the
# quotient w/S, its rounding, the zero point added and the two clamps (5), the
# reconstruction S(q - z) (2), and the squared error accumulated in fp64 (a conversion, a
# subtraction and a fused multiply-add: 3) -- 10 operations, 11 candidates, so 110
# operations per weight (the per-group statistics and scale arithmetic, 1/g of that, are
# left out).
VALU_LANE_OPS = 256 * 4 * 16 * 2.4e9
MSE_OPS_PER_WEIGHT = 10 * 11
MSE_ALU_PEAK_GWEIGHTS = round(VALU_LANE_OPS / MSE_OPS_PER_WEIGHT / 1e9, 1)
MALL_BYTES = 256 * 2 ** 20
METRIC = "W4A16 GEMV achieved HBM GB/s (% peak) at M=1; GEMM TFLOP/s (% MFMA peak)"


def gemv_bytes(m, n, k, g, sym):
    zeros = 0 if sym else 4 * n * ((k // g + 7) // 8)
    return n * k // 2 + 2 * n * (k // g) + zeros + 2 * m * k + 4 * m * n


def quant_bytes(n, k, g, sym, in_bytes=2):
    zeros = 0 if sym else 4 * n * ((k // g + 7) // 8)
    return n * k * in_bytes + n * k // 2 + 2 * n * (k // g) + zeros


def source_digest(*names):
    h = hashlib.sha256()
    for nm in names:
        with open(os.path.join(ROOT, "w4a16_group_wise_q4_amd", "csrc", nm), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profiled_traffic(summary_name, digest):
    """Measured HBM bytes per launch from a committed rocprofv3 PMC summary, if it was
    taken on the current kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", summary_name)
    if not os.path.exists(path):
        return None
    text = open(path, encoding="utf-8").read()
    src = re.search(r"source_digest:\s*([0-9a-f]+)", text)
    val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not src or not val or src.group(1) != digest:
        return None
    return float(val.group(1))


def capture(fns):
    """A HIP graph of the given launches, in order (captured on a side stream)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):          # warm the launch path on the capture stream
        for f in fns[:2]:
            f()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    torch.cuda.synchronize()
    return g


def graph_ms(graph, reps, warm=3):
    """Mean duration in ms of one replay: HIP events on the launch stream, after `warm`
    untimed replays (the first replays after the device was idle run slow)."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warm):
        graph.replay()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(reps):
        graph.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / reps


def read_ceiling(torch, dev, sizes):
    """A plain streaming read (the probe kernels of libq4probe.so: 16-byte loads, every byte
    read once, one launch per buffer) at each size, graph-replayed over distinct buffers
    that together exceed the Infinity Cache four times; the fastest of the probe's
    workgroup shapes at each size is the practical ceiling of a bandwidth-bound kernel that
    reads that many bytes in one launch."""
    import ctypes
    from w4a16_group_wise_q4_amd import _build
    lib = ctypes.CDLL(_build.PROBE_LIBRARY)
    lib.q4probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                 ctypes.c_void_p]
    lib.q4probe_read.restype = ctypes.c_int
    lib.q4probe_sink_words.argtypes = [ctypes.c_int64, ctypes.c_int]
    lib.q4probe_sink_words.restype = ctypes.c_int64
    lib.q4probe_shape.argtypes = [ctypes.c_int] + [ctypes.POINTER(ctypes.c_int)] * 3
    shapes = []
    for s in range(lib.q4probe_shapes()):
        th, ld, ax = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
        lib.q4probe_shape(s, ctypes.byref(th), ctypes.byref(ld), ctypes.byref(ax))
        shapes.append((s, th.value, ld.value, ax.value))
    res = {}
    for label, nbytes in sizes:
        copies = max(2, -(-4 * MALL_BYTES // nbytes))
        bufs = [torch.full((nbytes,), 1, dtype=torch.uint8, device=dev) for _ in range(copies)]
        sink = torch.empty(max(lib.q4probe_sink_words(nbytes, s[0]) for s in shapes), dtype=torch.int32,
                           device=dev)
        best = None
        for s, th, ld, ax in shapes:
            def read(b, s=s):
                st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
                if lib.q4probe_read(ctypes.c_void_p(b.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()), s, st):
                    raise RuntimeError("read probe launch failed")
            t = graph_ms(capture([lambda b=b: read(b) for b in bufs]), 10) / copies * 1e-3
            if best is None or t < best[0]:
                best = (t, th, ld, ax)
        t, th, ld, ax = best
        res[label] = {"bytes": nbytes, "us": round(t * 1e6, 3), "gbs": round(nbytes / t / 1e9, 1),
                      "frac_hbm": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4),
                      "probe_shape": f"{th} threads x {ld} loads of 16 B"
                                     + (", non-temporal" if ax == 2 else "")}
        del bufs, sink
    return res


def join_cost(torch, dev, launches=10):
    """What joining partial sums across the workgroups of one launch costs (the probe
    kernels of libq4probe.so, join_probe.hip): launches of row blocks x splits workgroups
    of 512 threads, 688 in all as in a 11008-row decode GEMV, each writing 512 partial sums;
    the last arriver of each row block adds them.  Per launch, graph-replayed: the partial
    stores alone, the join through device-scope release/acquire fences, and the join
    through device-scope relaxed atomics; every launch's sums are checked."""
    import ctypes
    from w4a16_group_wise_q4_amd import _build
    lib = ctypes.CDLL(_build.PROBE_LIBRARY)
    vp = ctypes.c_void_p
    lib.q4probe_join.argtypes = [vp, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    lib.q4probe_join.restype = ctypes.c_int
    lib.q4probe_join_part_floats.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.q4probe_join_part_floats.restype = ctypes.c_int64
    res = {}
    for rb, s in ((172, 4), (86, 8), (688, 1)):
        part = torch.zeros(lib.q4probe_join_part_floats(rb, s), dtype=torch.float32, device=dev)
        cnt = torch.zeros(rb, dtype=torch.int32, device=dev)
        y = torch.zeros((launches + 1, rb, 512), dtype=torch.float32, device=dev)
        row = {}
        for mode, key in ((0, "partials_only_us"), (1, "fence_join_us"), (2, "atomic_join_us")):
            def one(it, mode=mode):
                st = vp(torch.cuda.current_stream().cuda_stream)
                if lib.q4probe_join(vp(part.data_ptr()), vp(cnt.data_ptr()), vp(y.data_ptr()), rb, s, mode, it, st):
                    raise RuntimeError("join probe launch failed")
            y.zero_()
            g = capture([lambda it=it: one(it) for it in range(1, launches + 1)])
            y.zero_()
            row[key] = round(graph_ms(g, 5) / launches * 1e3, 3)
            if mode:
                want = torch.arange(1, launches + 1, device=dev, dtype=torch.float32) * (s * (s + 1) / 2)
                ok = bool(torch.equal(y[1:], want[:, None, None].expand(launches, rb, 512)))
                ok = ok and int(cnt.abs().sum().item()) == 0
                row[key.replace("_us", "_sums_ok")] = ok
        res[f"{rb}x{s}"] = row
        del part, cnt, y
    return {"what": "one launch of row blocks x splits workgroups (688 in all), 512 partial sums "
                    "each, joined by the last arriver of each row block; per launch, graph-replayed",
            "results": res}


def kv_cache_bytes(heads, t, d, g, sym=False):
    """Bytes of one INT4 cache (K or V) holding t tokens: codes, scales, zero words."""
    zeros = 0 if sym else 4 * ((d // g + 7) // 8)
    return heads * t * (d // 2 + 2 * (d // g) + zeros)


def kv_leg(q4, synthetic, torch, dev, layers=32):
    """One decode step of 7B-shaped attention over every layer's INT4 K and V caches
    (4096-token context), plus the quantize calls that fill and extend the caches."""
    ck = synthetic.KV_7B
    H, D, g, T = ck["heads"], ck["head_dim"], ck["group_size"], ck["t"]
    k = synthetic.kv_tokens(T, H, D, ck["k_seed"], "k").to(dev)
    v = synthetic.kv_tokens(T, H, D, ck["v_seed"], "v").to(dev)
    q = synthetic.query(H, D, ck["q_seed"]).to(dev)
    scale = 1.0 / math.sqrt(D)
    kcs = [q4.empty_kv_cache(H, ck["t_cap"], D, g, False, dev) for _ in range(layers)]
    vcs = [q4.empty_kv_cache(H, ck["t_cap"], D, g, False, dev) for _ in range(layers)]
    fill = ([lambda c=c: q4.q4_kv_quantize(k, c, 0) for c in kcs] +
            [lambda c=c: q4.q4_kv_quantize(v, c, 0) for c in vcs])
    for f in fill:
        f()
    torch.cuda.synchronize()
    qname = q4.q4_last_kernel()
    t_fill = graph_ms(capture(fill), 3) / len(fill) * 1e-3
    k1, v1 = k[T - 1:].contiguous(), v[T - 1:].contiguous()
    app = ([lambda c=c: q4.q4_kv_quantize(k1, c, T - 1) for c in kcs] +
           [lambda c=c: q4.q4_kv_quantize(v1, c, T - 1) for c in vcs])
    t_app = graph_ms(capture(app), 5) / len(app) * 1e-3
    ws_bytes = q4.q4_kv_attention_workspace(H, D, T)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    outs = torch.empty((layers, H, D), dtype=torch.float32, device=dev)
    att = [lambda i=i: q4.q4_kv_attention(q, kcs[i], vcs[i], T, scale, out=outs[i], workspace=ws)
           for i in range(layers)]
    att[0]()
    torch.cuda.synchronize()
    aname = q4.q4_last_kernel()
    t_att = graph_ms(capture(att), 5) / layers * 1e-3
    cache = kv_cache_bytes(H, T, D, g)
    att_bytes = 2 * cache + H * D * 2 + H * D * 4
    del kcs, vcs, outs, ws
    # batched decode: 16 sequences of the same length, their heads side by side (512 heads),
    # 4 layers (1.3 GB of caches, past the Infinity Cache)
    B, LB = 16, 4
    kb = synthetic.kv_tokens(T, B * H, D, ck["k_seed"] + 10, "k").to(dev)
    vb = synthetic.kv_tokens(T, B * H, D, ck["v_seed"] + 10, "v").to(dev)
    qb = synthetic.query(B * H, D, ck["q_seed"] + 10).to(dev)
    kbs = [q4.empty_kv_cache(B * H, T, D, g, False, dev) for _ in range(LB)]
    vbs = [q4.empty_kv_cache(B * H, T, D, g, False, dev) for _ in range(LB)]
    for c in kbs:
        q4.q4_kv_quantize(kb, c, 0)
    for c in vbs:
        q4.q4_kv_quantize(vb, c, 0)
    del kb, vb
    wsb = torch.empty(q4.q4_kv_attention_workspace(B * H, D, T), dtype=torch.uint8, device=dev)
    ob = torch.empty((LB, B * H, D), dtype=torch.float32, device=dev)
    attb = [lambda i=i: q4.q4_kv_attention(qb, kbs[i], vbs[i], T, scale, out=ob[i], workspace=wsb)
            for i in range(LB)]
    attb[0]()
    torch.cuda.synchronize()
    t_attb = graph_ms(capture(attb), 3) / LB * 1e-3
    att_bytes_b = 2 * kv_cache_bytes(B * H, T, D, g) + B * H * D * 6
    del kbs, vbs, ob, wsb
    fill_bytes = H * T * D * 2 + cache
    bf16_cache = 2 * H * T * D * 2
    return {
        "workload": f"7B-shaped decode attention, {H} heads x head_dim {D}, {T}-token context, "
                    f"INT4 K and V caches g{g} asym, one step over {layers} layers",
        "attention": {"kernel": aname, "us_per_layer": round(t_att * 1e6, 3),
                      "bytes_per_layer": att_bytes,
                      "gbs": round(att_bytes / t_att / 1e9, 1),
                      "frac_hbm": round(att_bytes / t_att / 1e9 / HBM_PEAK_GBS, 4),
                      "cache_bytes_vs_bf16": round(2 * cache / bf16_cache, 4)},
        "attention_batch16": {"heads": B * H, "us_per_layer": round(t_attb * 1e6, 2),
                              "bytes_per_layer": att_bytes_b, "gbs": round(att_bytes_b / t_attb / 1e9, 1),
                              "frac_hbm": round(att_bytes_b / t_attb / 1e9 / HBM_PEAK_GBS, 4)},
        "prefill_quantize": {"kernel": qname, "tokens": T, "us": round(t_fill * 1e6, 2),
                             "gbs": round(fill_bytes / t_fill / 1e9, 1),
                             "frac_hbm": round(fill_bytes / t_fill / 1e9 / HBM_PEAK_GBS, 4)},
        "decode_append": {"tokens": 1, "us": round(t_app * 1e6, 3)},
    }


def gptq_leg(q4, synthetic, torch, dev, tokens=2048):
    """GPTQ of the 7B-like up projection [11008 x 4096] against 2048 synthetic calibration
    tokens (N(0,1) plus 8 shared factors), g128 sym (the pages' GPTQ setting)."""
    mat = synthetic.MLP_SWEEP["mats"][0]
    n, k, g = mat.n, mat.k, 128
    w = mat.make().to(dev)
    gen = torch.Generator().manual_seed(300)
    f = torch.randn((tokens, 8), generator=gen)
    b = torch.randn((k, 8), generator=gen) / 8 ** 0.5
    x = (torch.randn((tokens, k), generator=gen) + 1.5 * f @ b.T).to(torch.bfloat16).to(dev)
    ws = torch.empty(q4.q4_gptq_act_order_workspace(n, k, g), dtype=torch.uint8, device=dev)
    # fp32 work: Hessian lower triangle, Cholesky, error-feedback updates
    flops = k * k * tokens + k ** 3 / 3 + n * k * k
    r = q4.q4_quantize_pack(w, g, True)
    xf = x.float()
    wf = w.float()
    err = lambda pk: float(((xf @ (wf - q4.q4_dequant(pk)).t()) ** 2).sum())
    res = {"workload": f"GPTQ of W [{n}x{k}] bf16, {tokens} calibration tokens, g{g} sym"}
    for key, act in (("natural_order", False), ("act_order", True)):
        p = q4.q4_gptq_quantize(w, x, g, True, workspace=ws, act_order=act)
        torch.cuda.synchronize()
        kname = q4.q4_last_kernel()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 3
        e0.record()
        for _ in range(reps):
            q4.q4_gptq_quantize(w, x, g, True, out=p, workspace=ws, act_order=act)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[key] = {"kernel": kname, "ms": round(ms, 3),
                    "tflops_fp32": round(flops / (ms * 1e-3) / 1e12, 2),
                    "frac_fp32_mfma": round(flops / (ms * 1e-3) / 1e12 / FP32_MFMA_PEAK_TFLOPS, 4),
                    "layer_error_vs_rtn": round(err(p) / err(r), 4)}
    return res


def cpu_model():
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(seconds=6.0, max_threads=16):
    """The CPU oracle as it stands (plain scalar C, fp64 linear) timed on this host, on
    bounded samples of the same workloads:
    - the decode GEMV (both 7B projections, M=1, g128 asym), full passes for about
      ``seconds`` on one thread, then row-sharded (disjoint output rows, the same scalar
      code, one thread each, the GIL released inside the C calls) across the affinity cores
      up to ``max_threads``; ``value`` is the sharded rate in the metric's unit;
    - the quantize oracle on the full tensors of the tiny, 7B decode and MLP-sweep
      configurations and on one layer of the 32-layer checkpoint (extrapolated to 32);
    - the fp64 linear of the 70B prefill on 16 seeded rows of x against all 28672 output
      rows (3.8e9 multiply-adds), extrapolated to the 2048 rows of the workload."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import torch

    import oracle
    import synthetic
    aff = len(os.sched_getaffinity(0))
    threads = max(1, min(aff, max_threads))
    pool = ThreadPoolExecutor(threads)

    def shard(n):
        return [s for s in np.array_split(np.arange(n, dtype=np.int64), threads) if len(s)]

    def quant(w, g, sym):  # row blocks in parallel, concatenated as one call would give
        bits = synthetic.as_u16(w) if w.dtype != torch.float32 else None
        blocks = shard(w.shape[0])
        def one(r):
            if bits is not None:
                return oracle.quantize_pack((bits[r[0]:r[-1] + 1], oracle.BF16), g, sym)
            return oracle.quantize_pack(w[r[0]:r[-1] + 1].numpy(), g, sym)
        parts = list(pool.map(one, blocks))
        return (np.concatenate([p_[0] for p_ in parts]), np.concatenate([p_[1] for p_ in parts]),
                None if sym else np.concatenate([p_[2] for p_ in parts]))

    # ---- decode GEMV oracle
    cfg = synthetic.DECODE_7B
    x = synthetic.activations(1, 4096, cfg["x_seed"])
    xb = (synthetic.as_u16(x), oracle.BF16)
    t0 = time.perf_counter()
    packs, qweights = [], 0
    for mat in cfg["mats"]:
        q, s, z = quant(mat.make(), 128, False)
        packs.append((q, s, z, mat.n, mat.k))
        qweights += mat.n * mat.k
    t_q2 = time.perf_counter() - t0
    per_pass = sum(gemv_bytes(1, n, k, 128, False) for _, _, _, n, k in packs)

    def gemv_pass(sharded):
        for q, s, z, n, k in packs:
            if sharded:
                list(pool.map(lambda c: oracle.linear(xb, q, s, z, n, k, 128, False, cols=c), shard(n)))
            else:
                oracle.linear(xb, q, s, z, n, k, 128, False)

    def timed(sharded, budget):
        passes, t0_ = 0, time.perf_counter()
        while True:
            gemv_pass(sharded)
            passes += 1
            el_ = time.perf_counter() - t0_
            if el_ >= budget:
                return passes, el_
    p1, e1 = timed(False, seconds)
    pn, en = timed(True, seconds / 2)
    single = {"value": round(per_pass * p1 / e1 / 1e9, 4), "unit": "GB/s", "cores": 1,
              "sample": f"{p1} fp64 passes, {e1:.1f} s"}

    # ---- quantize oracle (row blocks across the same threads)
    quant_res = {}
    def qtime(label, mats, g, sym, scale=1):
        nonlocal quant_res
        t0_ = time.perf_counter()
        nbytes = 0
        for w in mats:
            quant(w, g, sym)
            nbytes += quant_bytes(w.shape[0], w.shape[1], g, sym, in_bytes=w.element_size())
        el_ = time.perf_counter() - t0_
        quant_res[label] = {"seconds": round(el_ * scale, 3), "gbs": round(nbytes / el_ / 1e9, 4)}
        if scale != 1:
            quant_res[label]["extrapolated"] = f"one layer timed, x{scale}"
    tiny = synthetic.TINY["w"].make()
    qtime("tiny_256x512_fp32_asym", [tiny], 128, False)
    qtime("tiny_256x512_fp32_sym", [tiny], 128, True)
    quant_res["decode_7b_g128_asym"] = {"seconds": round(t_q2, 3),
                                        "gbs": round(sum(quant_bytes(n, k, 128, False) for _, _, _, n, k in packs)
                                                     / t_q2 / 1e9, 4)}
    mlp = [m_.make() for m_ in synthetic.MLP_SWEEP["mats"]]
    for g in synthetic.MLP_SWEEP["group_sizes"]:
        for sym in synthetic.MLP_SWEEP["symmetric"]:
            qtime(f"mlp_g{g}_{'sym' if sym else 'asym'}", mlp, g, sym)
    del mlp
    layer = [m_.make(device="cpu") for m_ in synthetic.checkpoint_7b(1)]
    qtime("checkpoint_32_layers_g128_asym", layer, 128, False, scale=32)
    del layer

    # ---- fp64 linear of the 70B prefill on 16 seeded rows
    c4 = synthetic.PREFILL_70B
    wm = c4["w"]
    t0 = time.perf_counter()
    q4_, s4_, z4_ = quant(wm.make(), 128, False)
    t_q4 = time.perf_counter() - t0
    rows = synthetic.sample_rows(c4["m"], 16, c4["x_seed"]).numpy()
    x4 = synthetic.activations(c4["m"], wm.k, c4["x_seed"], outlier_seed=wm.seed,
                               outlier_factor=c4["x_outlier_factor"])[torch.as_tensor(rows)]
    x4b = (synthetic.as_u16(x4), oracle.BF16)
    t0 = time.perf_counter()
    list(pool.map(lambda c: oracle.linear(x4b, q4_, s4_, z4_, wm.n, wm.k, 128, False, cols=c), shard(wm.n)))
    t_l4 = time.perf_counter() - t0
    fl = 2.0 * 16 * wm.n * wm.k
    gemm = {"rows": 16, "seconds": round(t_l4, 3), "gflops": round(fl / t_l4 / 1e9, 3),
            "full_2048_rows_seconds_extrapolated": round(t_l4 * c4["m"] / 16, 1),
            "quantize_70b_seconds": round(t_q4, 3)}
    pool.shutdown()
    return {"value": round(per_pass * pn / en / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{pn} fp64 oracle passes of y = x.W_hat^T over the 4096x4096 and 11008x4096 "
                      f"g128 asym projections at M=1, output rows sharded over {threads} threads "
                      f"({en:.1f} s); single-core and quantize/70B-prefill samples beside it",
            "cores_available": os.cpu_count(), "affinity": aff, "cpu_model": cpu_model(),
            "single_core": single, "quantize": quant_res, "gemm_70b_16_rows": gemm}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1020)
    # the device needs about 40 replays of the decode graph (1360 launches, about 12 ms)
    # after idle before its launches reach their steady duration
    ap.add_argument("--warmup", type=int, default=1360)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--legs", default="gemm,quant,sweep,mlp,mse,dequant,kv,midm,gptq,join",
                    help="comma list of legs besides the headline decode GEMV")
    ap.add_argument("--mlp-n", default="", help="mlp leg: only these weight row counts (comma list)")
    ap.add_argument("--mlp-g", default="", help="mlp leg: only these group sizes (comma list)")
    ap.add_argument("--mlp-sym", default="", choices=["", "sym", "asym"], help="mlp leg: only this mode")
    ap.add_argument("--mlp-m", default="", help="mlp leg: only these batch sizes (comma list)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 512 MiB device-to-device copy 5 times (the "
                         "reference kernel for scaling HBM byte counters) and exit")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        nbytes = 512 * 2 ** 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "launches": 5}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import synthetic
    import w4a16_group_wise_q4_amd as q4

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    legs = set(args.legs.split(",")) if args.legs else set()
    out = {}

    # ------------------------------------------------------------ decode GEMV (the metric)
    cfg = synthetic.DECODE_7B
    base = [q4.q4_quantize_pack(mat.make().to(dev), 128, False) for mat in cfg["mats"]]
    step_bytes = sum(gemv_bytes(1, p.n, p.k, 128, False) for p in base)
    copies = max(2, -(-4 * MALL_BYTES // step_bytes))  # 4x the Infinity Cache
    packs = [[q4.PackedWeight(p.qweight.clone(), p.scales.clone(), p.zeros.clone(), p.n, p.k,
                              128, False) for p in base] for _ in range(copies)]
    x = synthetic.activations(1, 4096, cfg["x_seed"]).to(dev)
    ys = [torch.empty((1, p.n), dtype=torch.float32, device=dev) for p in base]

    def step_fns(c):  # one grouped launch: both projections
        return [lambda c=c: q4.q4_w4a16_gemm_grouped(x, packs[c], outs=ys)]

    def single_fns(c):  # the same step as one launch per projection
        return [lambda c=c, i=i: q4.q4_w4a16_gemm(x, packs[c][i], out=ys[i]) for i in range(len(base))]

    for f in step_fns(0):
        f()
    torch.cuda.synchronize()
    gemv_kernel = q4.q4_last_kernel()
    full = capture([f for c in range(copies) for f in step_fns(c)])
    tail_n = args.steps % copies
    tail = capture([f for c in range(tail_n) for f in step_fns(c)]) if tail_n else None
    # W untimed warmup steps: whole replays of the copies, then single steps for the rest
    for _ in range(args.warmup // copies):
        full.replay()
    for c in range(args.warmup % copies):
        for f in step_fns(c):
            f()
    torch.cuda.synchronize()
    # the timed region: exactly K steps, synchronized on both sides, nothing else inside;
    # HIP events on the stream the graphs replay on bracket the same K launches (one
    # grouped GEMV launch per step), which gives the kernel's average launch duration
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev0.record()
    for _ in range(args.steps // copies):
        full.replay()
    if tail is not None:
        tail.replay()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_step = wall * 1e3 / args.steps
    value = step_bytes * args.steps / wall / 1e9
    launch_ms = ev0.elapsed_time(ev1) / args.steps
    achieved = step_bytes / (launch_ms * 1e-3) / 1e9

    # for comparison: the same projections as one launch each (HIP events around graph
    # replays of every copy, a pass of its own)
    single_ms = []
    for i in range(len(base)):
        g = capture([lambda c=c: q4.q4_w4a16_gemm(x, packs[c][i], out=ys[i]) for c in range(copies)])
        single_ms.append(graph_ms(g, 10) / copies)
    single_step_ms = graph_ms(capture([f for c in range(copies) for f in single_fns(c)]), 10) / copies
    digest = source_digest("gemv.hip", "gemv_tile.h", "gemv_tile_g128.hip", "q4_device.h")
    traffic = profiled_traffic("q4_gemv_decode_7b_m1_pmc.md", digest)
    del packs
    # the streaming-read ceiling at the sizes of the decode matrices and step, the prefill
    # GEMM's weights and 1 GB
    ceiling = read_ceiling(torch, dev, [("4096x4096", gemv_bytes(1, 4096, 4096, 128, False)),
                                        ("11008x4096", gemv_bytes(1, 11008, 4096, 128, False)),
                                        ("decode_step", step_bytes),
                                        ("70b_weights", gemv_bytes(0, 28672, 8192, 128, False)),
                                        ("1GB", 1 << 30)])
    ceil_gbs = ceiling["decode_step"]["gbs"]
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "kernel": gemv_kernel,
                "per_launch_us": round(launch_ms * 1e3, 3), "bytes_per_launch": step_bytes,
                "ceiling_read_gbs": ceil_gbs, "frac_vs_ceiling": round(achieved / ceil_gbs, 4),
                "source_digest": digest}
    single = {"kernel": gemv_kernel,
              "per_launch_us": {f"{p.n}x{p.k}": round(t * 1e3, 3) for p, t in zip(base, single_ms)},
              "bytes_per_launch": {f"{p.n}x{p.k}": gemv_bytes(1, p.n, p.k, 128, False) for p in base},
              "achieved_gbs": {f"{p.n}x{p.k}": round(gemv_bytes(1, p.n, p.k, 128, False) / (t * 1e-3) / 1e9, 1)
                               for p, t in zip(base, single_ms)},
              "step_us": round(single_step_ms * 1e3, 3),
              "step_gbs": round(step_bytes / (single_step_ms * 1e-3) / 1e9, 1)}
    out["read_ceiling"] = {"what": "plain streaming read, one launch per buffer, graph-replayed over "
                                   "distinct buffers (4x the Infinity Cache)", "results": ceiling}

    # ------------------------------------------------------------ prefill GEMM
    gemm_roof = None
    if "gemm" in legs:
        c4 = synthetic.PREFILL_70B
        mat = c4["w"]
        pw0 = q4.q4_quantize_pack(mat.make().to(dev), 128, False)
        # distinct weight copies, 5 x 122 MB, so no launch finds its weights in the
        # 256 MB Infinity Cache
        gcopies = 5
        pws = [q4.PackedWeight(pw0.qweight.clone(), pw0.scales.clone(), pw0.zeros.clone(), mat.n, mat.k,
                               128, False) for _ in range(gcopies)]
        del pw0
        xg = synthetic.activations(c4["m"], mat.k, c4["x_seed"], outlier_seed=mat.seed,
                                   outlier_factor=c4["x_outlier_factor"]).to(dev)
        yg = torch.empty((c4["m"], mat.n), dtype=torch.float32, device=dev)
        q4.q4_w4a16_gemm(xg, pws[0], out=yg)
        torch.cuda.synchronize()
        kname = q4.q4_last_kernel()
        g = capture([lambda pp=pp: q4.q4_w4a16_gemm(xg, pp, out=yg) for pp in pws])
        t = graph_ms(g, 4) / gcopies * 1e-3
        flops = 2.0 * c4["m"] * mat.n * mat.k
        wbytes = gemv_bytes(0, mat.n, mat.k, 128, False)
        # the dense bf16 GEMM of the same shape (hipBLASLt through torch), as a ceiling
        wd = torch.empty((mat.n, mat.k), dtype=torch.bfloat16, device=dev).normal_(0, 0.015)
        xb = xg.to(torch.bfloat16)
        torch.nn.functional.linear(xb, wd)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(5):
            torch.nn.functional.linear(xb, wd)
        e1.record()
        torch.cuda.synchronize()
        t_dense = e0.elapsed_time(e1) / 5 * 1e-3
        del wd, xb
        tf, tf_dense = flops / t / 1e12, flops / t_dense / 1e12
        out["gemm"] = {"workload": f"70B-like prefill x[{c4['m']}x{mat.k}] . W[{mat.n}x{mat.k}]^T "
                                   "g128 asym", "kernel": kname, "ms": round(t * 1e3, 4),
                       "tflops": round(tf, 2), "frac_mfma_bf16": round(tf / BF16_PEAK_TFLOPS, 4),
                       "weight_copies": gcopies, "weight_bytes_per_copy": wbytes,
                       "dense_bf16_gemm_tflops": round(tf_dense, 1)}
        gemm_roof = {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4), "kernel": kname,
                     "per_launch_us": round(t * 1e6, 1), "flop_per_launch": flops,
                     "ceiling_dense_bf16_tflops": round(tf_dense, 1),
                     "frac_vs_ceiling": round(tf / tf_dense, 4)}
        del pws, xg, yg

    # ------------------------------------------------------------ MSE clip search (quantize)
    if "mse" in legs:
        res = {}
        for mat in cfg["mats"]:
            w = mat.make().to(dev)
            wf = w.float()
            for sym in (False, True):
                pm = q4.q4_quantize_pack_mse(w, 128, sym)
                kname = q4.q4_last_kernel()
                pr = q4.q4_quantize_pack(w, 128, sym)
                torch.cuda.synchronize()
                t = graph_ms(capture([lambda: q4.q4_quantize_pack_mse(w, 128, sym, out=pm)] * 3), 3) / 3 * 1e-3
                e_m = (q4.q4_dequant(pm) - wf).double().pow(2).sum().item()
                e_r = (q4.q4_dequant(pr) - wf).double().pow(2).sum().item()
                qb = quant_bytes(mat.n, mat.k, 128, sym)
                gw = mat.n * mat.k / t / 1e9
                res[f"{mat.n}x{mat.k} {'sym' if sym else 'asym'}"] = {
                    "kernel": kname, "us": round(t * 1e6, 1), "gbs": round(qb / t / 1e9, 1),
                    "gweights_per_s": round(gw, 1), "frac_alu": round(gw / MSE_ALU_PEAK_GWEIGHTS, 4),
                    "sq_error_vs_rtn": round(e_m / e_r, 4)}
                del pm, pr
            del w, wf
        out["mse_clip"] = {"workload": "7B-like decode matrices, bf16, g128, clip ratios (20-i)/20, "
                                       "i = 0..10, per group", "bound": "alu",
                           "alu_peak_gweights_per_s": MSE_ALU_PEAK_GWEIGHTS,
                           "alu_peak": "vector ALU 39.3e12 lane operations/s over 110 algorithmic "
                                       "operations per weight (10 per candidate ratio x 11)",
                           "results": res}

    # ------------------------------------------------------------ full dequantization
    if "dequant" in legs:
        res = {}
        for i, mat in enumerate(cfg["mats"]):
            p = base[i]
            for odt, ob in ((torch.bfloat16, 2), (torch.float32, 4)):
                db = quant_bytes(p.n, p.k, 128, False, in_bytes=0) + p.n * p.k * ob
                dcopies = max(2, -(-4 * MALL_BYTES // db))  # packed inputs and outputs rotate
                ps = [q4.PackedWeight(p.qweight.clone(), p.scales.clone(), p.zeros.clone(), p.n, p.k, 128, False)
                      for _ in range(dcopies)]
                os_ = [torch.empty((p.n, p.k), dtype=odt, device=dev) for _ in range(dcopies)]
                q4.q4_dequant(ps[0], out=os_[0])
                kname = q4.q4_last_kernel()
                torch.cuda.synchronize()
                t = graph_ms(capture([lambda pp=pp, oo=oo: q4.q4_dequant(pp, out=oo)
                                      for pp, oo in zip(ps, os_)]), 5) / dcopies * 1e-3
                del ps, os_
                res[f"{p.n}x{p.k} -> {str(odt).split('.')[-1]}"] = {
                    "kernel": kname, "us": round(t * 1e6, 2), "bytes": db, "copies": dcopies,
                    "gbs": round(db / t / 1e9, 1), "frac_hbm": round(db / t / 1e9 / HBM_PEAK_GBS, 4)}
        out["dequant"] = {"workload": "7B-like decode matrices, g128 asym packed, to bf16 and fp32",
                          "bytes": "codes n*k/2 + scales 2*n*k/g + zero words read, n*k*out "
                                   "written", "results": res}

    # ------------------------------------------------------------ split-K join cost (probe)
    if "join" in legs:
        out["split_k_join"] = join_cost(torch, dev)

    # ------------------------------------------------------------ INT4 KV cache (decode attention)
    if "kv" in legs:
        out["kv_cache"] = kv_leg(q4, synthetic, torch, dev)

    # ------------------------------------------------------------ GPTQ (one 7B-shaped layer)
    if "gptq" in legs:
        out["gptq"] = gptq_leg(q4, synthetic, torch, dev)

    # ------------------------------------------------------------ mid-M (17..256) products
    if "midm" in legs:
        res = {}
        shapes = [("up_11008x4096", 11008, 4096, 5), ("down_4096x11008", 4096, 11008, 6),
                  ("mlp70b_28672x8192", 28672, 8192, 8)]
        for nm, n_, k_, seed in shapes:
            w = synthetic.weight(n_, k_, 0.02, seed).to(dev)
            p0 = q4.q4_quantize_pack(w, 128, False)
            del w
            nb = gemv_bytes(1, n_, k_, 128, False)
            cps = max(2, -(-4 * MALL_BYTES // nb))
            pks = [q4.PackedWeight(p0.qweight.clone(), p0.scales.clone(), p0.zeros.clone(), n_, k_, 128, False)
                   for _ in range(cps)]
            x256 = synthetic.activations(256, k_, 7).to(dev)
            row = {}
            for m in (17, 32, 64, 128, 256):
                xm = x256[:m].contiguous()
                ym = torch.empty((m, n_), dtype=torch.float32, device=dev)
                need = q4.q4_w4a16_gemm_workspace(m, n_, k_, 128)
                ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
                byt = gemv_bytes(m, n_, k_, 128, False)
                entry = {}
                # the default (K split into the workspace where that fills the device), then
                # the product unsplit
                for key, split in (("split", True), ("unsplit", False)):
                    if key == "split" and need == 0:
                        continue
                    q4.q4_w4a16_gemm(xm, pks[0], out=ym, workspace=ws, split=split)
                    torch.cuda.synchronize()
                    kname = "+".join(q4.q4_last_kernels())
                    t = graph_ms(capture([lambda pp=pp: q4.q4_w4a16_gemm(xm, pp, out=ym, workspace=ws, split=split)
                                          for pp in pks]), 3) / cps * 1e-3
                    entry[key] = {"us": round(t * 1e6, 2), "gbs": round(byt / t / 1e9, 1),
                                  "frac_hbm": round(byt / t / 1e9 / HBM_PEAK_GBS, 4),
                                  "tflops": round(2.0 * m * n_ * k_ / t / 1e12, 1), "kernel": kname}
                row[f"m{m}"] = entry
                del ws
            res[nm] = row
            del pks, p0, x256
        out["midm"] = {"workload": "W4A16 products at m = 17..256 (decode batches of the pages' "
                                   "concurrency grid, short prompts), g128 asym, bf16 x", "results": res}

    # ------------------------------------------------------------ MLP batch sweep (GEMV, m <= 16)
    if "mlp" in legs:
        c3 = synthetic.MLP_SWEEP
        pick = lambda arg, vals: [v for v in vals if not arg or str(v) in arg.split(",")]
        res = {}
        for mat in c3["mats"]:
            if args.mlp_n and str(mat.n) not in args.mlp_n.split(","):
                continue
            w = mat.make().to(dev)
            x16 = synthetic.activations(16, mat.k, c3["x_seed"]).to(dev)
            for g in pick(args.mlp_g, c3["group_sizes"]):
                for sym in c3["symmetric"]:
                    if args.mlp_sym and args.mlp_sym != ("sym" if sym else "asym"):
                        continue
                    p0 = q4.q4_quantize_pack(w, g, sym)
                    nb = gemv_bytes(1, mat.n, mat.k, g, sym)
                    cps = max(2, -(-4 * MALL_BYTES // nb))
                    pks = [q4.PackedWeight(p0.qweight.clone(), p0.scales.clone(),
                                           None if sym else p0.zeros.clone(), mat.n, mat.k, g, sym)
                           for _ in range(cps)]
                    row = {}
                    for m in pick(args.mlp_m, c3["ms"]):
                        xm = x16[:m].contiguous()
                        ym = torch.empty((m, mat.n), dtype=torch.float32, device=dev)
                        q4.q4_w4a16_gemm(xm, pks[0], out=ym)
                        torch.cuda.synchronize()
                        kname = q4.q4_last_kernel()
                        t = graph_ms(capture([lambda pp=pp: q4.q4_w4a16_gemm(xm, pp, out=ym)
                                              for pp in pks]), 5) / cps * 1e-3
                        byt = gemv_bytes(m, mat.n, mat.k, g, sym)
                        row[f"m{m}"] = {"us": round(t * 1e6, 3), "gbs": round(byt / t / 1e9, 1),
                                        "frac_hbm": round(byt / t / 1e9 / HBM_PEAK_GBS, 4),
                                        "kernel": kname}
                    res[f"{mat.n}x{mat.k} g{g} {'sym' if sym else 'asym'}"] = row
                    del pks, p0
            del w
        # the gate and up projections of one layer (two 11008x4096 matrices sharing x) as
        # one grouped launch, g128 asym: the form a decoder layer runs them in
        grouped = {}
        mat = c3["mats"][0]
        if not args.mlp_n or str(mat.n) in args.mlp_n.split(","):
            w = mat.make().to(dev)
            x16 = synthetic.activations(16, mat.k, c3["x_seed"]).to(dev)
            p0 = q4.q4_quantize_pack(w, 128, False)
            del w
            nb = 2 * gemv_bytes(1, mat.n, mat.k, 128, False)
            cps = max(2, -(-4 * MALL_BYTES // nb))
            pks = [[q4.PackedWeight(p0.qweight.clone(), p0.scales.clone(), p0.zeros.clone(), mat.n, mat.k,
                                    128, False) for _ in range(2)] for _ in range(cps)]
            for m in pick(args.mlp_m, c3["ms"]):
                xm = x16[:m].contiguous()
                ys = [torch.empty((m, mat.n), dtype=torch.float32, device=dev) for _ in range(2)]
                q4.q4_w4a16_gemm_grouped(xm, pks[0], outs=ys)
                torch.cuda.synchronize()
                kname = q4.q4_last_kernel()
                t = graph_ms(capture([lambda pp=pp: q4.q4_w4a16_gemm_grouped(xm, pp, outs=ys)
                                      for pp in pks]), 5) / cps * 1e-3
                byt = 2 * gemv_bytes(m, mat.n, mat.k, 128, False) - 2 * m * mat.k  # x read once
                grouped[f"m{m}"] = {"us": round(t * 1e6, 3), "gbs": round(byt / t / 1e9, 1),
                                    "frac_hbm": round(byt / t / 1e9 / HBM_PEAK_GBS, 4), "kernel": kname}
            del pks, p0
        out["mlp_sweep"] = {"workload": "7B-like MLP GEMV, W [11008x4096] and [4096x11008], "
                                        "m in 1..16, one launch per product", "results": res,
                            "gate_up_grouped": {"workload": "two 11008x4096 g128 asym matrices "
                                                            "sharing x, one grouped launch",
                                                "results": grouped}}

    # ------------------------------------------------------------ checkpoint quantize + GEMV sweep
    if "quant" in legs or "sweep" in legs:
        mats = synthetic.checkpoint_7b(32)
        ws = [m_.make(device="cuda") for m_ in mats]
        torch.cuda.synchronize()
        res = {}
        for sym in (False, True):
            pk = [q4.empty_packed(m_.n, m_.k, 128, sym, dev) for m_ in mats]
            fq = [(lambda i=i: q4.q4_quantize_pack(ws[i], 128, sym, out=pk[i])) for i in range(len(mats))]
            for f in fq:
                f()
            torch.cuda.synchronize()
            kname = q4.q4_last_kernel()
            t_q = graph_ms(capture(fq), 3) * 1e-3
            qb = sum(quant_bytes(m_.n, m_.k, 128, sym) for m_ in mats)
            res["asym" if not sym else "sym"] = {
                "kernel": kname, "bytes": qb, "sweep_ms": round(t_q * 1e3, 3),
                "gbs": round(qb / t_q / 1e9, 1), "frac_hbm": round(qb / t_q / 1e9 / HBM_PEAK_GBS, 4),
                "launch": "one launch per matrix (224)"}
            # the same conversion one layer (seven matrices) per grouped launch
            fqg = [(lambda b=b: q4.q4_quantize_pack_grouped(ws[b:b + 7], 128, sym, outs=pk[b:b + 7]))
                   for b in range(0, len(mats), 7)]
            for f in fqg:
                f()
            torch.cuda.synchronize()
            t_qg = graph_ms(capture(fqg), 3) * 1e-3
            res[("asym" if not sym else "sym") + "_grouped"] = {
                "kernel": q4.q4_last_kernel(), "bytes": qb, "sweep_ms": round(t_qg * 1e3, 3),
                "gbs": round(qb / t_qg / 1e9, 1), "frac_hbm": round(qb / t_qg / 1e9 / HBM_PEAK_GBS, 4),
                "launch": "one grouped launch per layer (32)"}
            if not sym and "sweep" in legs:
                xs = {4096: synthetic.activations(1, 4096, 10).to(dev),
                      11008: synthetic.activations(1, 11008, 10).to(dev)}
                yy = {n_: torch.empty((1, n_), dtype=torch.float32, device=dev) for n_ in (4096, 11008)}
                fg = [(lambda i=i: q4.q4_w4a16_gemm(xs[mats[i].k], pk[i], out=yy[mats[i].n]))
                      for i in range(len(mats))]
                for f in fg:
                    f()
                t_g = graph_ms(capture(fg), 3) * 1e-3
                gb = sum(gemv_bytes(1, m_.n, m_.k, 128, False) for m_ in mats)
                res["gemv_sweep_m1"] = {"bytes": gb, "sweep_ms": round(t_g * 1e3, 3),
                                        "gbs": round(gb / t_g / 1e9, 1),
                                        "frac_hbm": round(gb / t_g / 1e9 / HBM_PEAK_GBS, 4),
                                        "launch": "one launch per matrix (224)"}
                # as a decode step issues them: q/k/v share their input and so do gate/up,
                # so each layer is four launches (q+k+v grouped, o, gate+up grouped, down)
                ys_ = {i: torch.empty((1, mats[i].n), dtype=torch.float32, device=dev)
                       for i in range(len(mats))}
                fgg = []
                for base_i in range(0, len(mats), 7):
                    for idx in ([0, 1, 2], [3], [4, 5], [6]):
                        ii = [base_i + j for j in idx]
                        kk = mats[ii[0]].k
                        if len(ii) == 1:
                            fgg.append(lambda i=ii[0], kk=kk: q4.q4_w4a16_gemm(xs[kk], pk[i], out=ys_[i]))
                        else:
                            fgg.append(lambda ii=ii, kk=kk: q4.q4_w4a16_gemm_grouped(
                                xs[kk], [pk[i] for i in ii], outs=[ys_[i] for i in ii]))
                for f in fgg:
                    f()
                t_gg = graph_ms(capture(fgg), 3) * 1e-3
                res["gemv_sweep_m1_grouped"] = {
                    "bytes": gb, "sweep_ms": round(t_gg * 1e3, 3), "gbs": round(gb / t_gg / 1e9, 1),
                    "frac_hbm": round(gb / t_gg / 1e9 / HBM_PEAK_GBS, 4),
                    "launch": "four launches per layer (q+k+v grouped, o, gate+up grouped, down)"}
            del pk
        res["workload"] = "32-layer 7B-like checkpoint, 224 bf16 matrices, 6.48e9 weights, g128"
        out["checkpoint"] = res
        del ws

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights with 0.1% outlier input channels x20, "
                "N(0,1) activations)",
        "config": {"workload": "7B-like decode GEMV, W [4096x4096] and [11008x4096], g=128 asym "
                               "uint4, x bf16 [1x4096], M=1", "group_size": 128, "m": 1,
                   "weight_copies": copies, "bytes_per_step": step_bytes,
                   "launch": "one grouped GEMV launch per step (both projections), replayed "
                             "from HIP graphs"},
        "roofline": roofline,
        "single_launches": single,
    }
    if gemm_roof is not None:
        # the metric's second half (prefill GEMM TFLOP/s and fraction of the bf16 MFMA peak),
        # inside roofline so a reader of the headline fields sees it too
        roofline["gemm"] = gemm_roof
        line["roofline_gemm"] = gemm_roof
    line.update(out)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line))


if __name__ == "__main__":
    main()

"""Benchmark of the Q4_K x Q8_1 decode GEMV at 4096 -> 14336, batch 1.

One step = the whole hot path for one token: quantize the fp32 activation to
Q8_1 and compute y = W x with W a 14336 x 4096 Q4_K matrix (33,030,144
bytes), as one rz_q4k_q8_gemv_f32 launch (bit-identical to rz_q8_1_quantize
followed by rz_q4k_q8_gemv, which is also timed).  Every step reads the next of R weight copies
(R * 33 MB >= 1 GiB), so no step finds its weights in the 256 MB Infinity
Cache or an L2; inputs are resident in HBM before the timed region.

Printed (one JSON line): the whole-step weight-stream rate in GB/s (`value`,
K steps captured in one HIP graph and replayed between HIP events, right after
W untimed warm-up steps), the fused kernel's rate against the 8 TB/s HBM peak
(`roofline`), a plain streaming read of the same bytes as the practical
ceiling (`read_ceiling`), the CPU oracle timed on the host (`cpu_baseline`:
the step's workload, and every configuration's oracle as the median of 3
runs), and under `rows` every other kernel of the path at its own workload,
timed the same way with its own weight rotation (the rows run first, so the
GPU clocks have settled when the step is timed): Q8_1 quantize, the GEMV
alone, the four attention projections on one shared activation (one
multi-matrix launch, and four launches), the SwiGLU chain and its down
projection, the Q4_0 LM head (fp32 and Q8_1 activation), 8 tokens sharing one
weight pass, and the small 896 x 1024 case; a row of a measured configuration
carries that configuration's oracle time, and every row the time of a plain
streaming read of its own byte count (`read_ceiling_us`, `frac_of_ceiling`).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-rows]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Q4_K×Q8_1 GEMV weight-stream GB/s and % HBM peak at 4096→14336, batch 1"
HBM_PEAK_GBS = 8000.0
OUT_DIM, IN_DIM = 14336, 4096
W_BYTES = OUT_DIM * (IN_DIM // 256) * 144            # 33,030,144
XQ_BYTES = (IN_DIM // 32) * 40                        # 5,120
Y_BYTES = OUT_DIM * 4                                 # 57,344
X_BYTES = IN_DIM * 4                                  # 16,384
GEMV_ALGO_BYTES = W_BYTES + XQ_BYTES + Y_BYTES        # 33,092,608 per GEMV launch
STEP_ALGO_BYTES = W_BYTES + X_BYTES + Y_BYTES         # 33,103,872 per fused launch
ROTATE_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "q4k_gemv_f32_4096x14336_traffic.txt")
KERNEL_SOURCES = ["q4k_gemv.h", "q4k_gemv_f32.hip", "rz_device.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "q4_q8_integer_quantize_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per GEMV launch from the committed rocprofv3 counter summary,
    or None when that summary was taken on different kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    fields = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_threads():
    """BLAS libraries numpy uses and their thread counts (threadpoolctl)."""
    try:
        import threadpoolctl
        return [{"api": d.get("internal_api"), "threads": d.get("num_threads")}
                for d in threadpoolctl.threadpool_info() if d.get("user_api") == "blas"]
    except Exception as e:   # threadpoolctl missing or failing: say so
        return [{"error": type(e).__name__}]


def _median_run(fn, runs: int = 3):
    """Median wall seconds and CPU seconds of `runs` calls of fn."""
    wall, cpu = [], []
    for _ in range(runs):
        c0, t0 = time.process_time(), time.perf_counter()
        fn()
        wall.append(time.perf_counter() - t0)
        cpu.append(time.process_time() - c0)
    order = sorted(range(runs), key=lambda i: wall[i])
    mid = order[runs // 2]
    return wall[mid], cpu[mid]


def cpu_baseline(target_seconds: float):
    """The oracle as it stands, on the host cores.

    Headline (`value`): Q8_1 quantize of the activation plus the integer form of
    the 4096 -> 14336 GEMV over all rows, repeated until target_seconds of wall
    time; rate = weight bytes per second.  `cores` = CPU time / wall time of that
    loop (the threads it actually kept busy).

    Per configuration (`per_config`), the median of 3 runs of the oracle's whole
    workload: the 896 x 1024 GEMV; the attention projections Q, K, V, O on one
    quantized activation; the SwiGLU chain (gate, up, silu * up, requantize,
    down); the Q4_0 LM head over an fp32 and over a Q8_1 activation; 8 tokens
    through the 4096 -> 14336 GEMV.  Reported with the weight rate and the
    threads kept busy (numpy's integer paths run on one core; the fp32 LM head
    is a BLAS matrix-vector product on the BLAS threads listed)."""
    import numpy as np
    import oracle
    import synth
    w = synth.q4k_weights(synth.rng(2, synth.T_W0), OUT_DIM, IN_DIM)
    x = synth.activation(synth.rng(2, synth.T_ACT), IN_DIM)
    reps, wall, cpu = 0, 0.0, 0.0
    while wall < target_seconds or reps < 1:
        c0, t0 = time.process_time(), time.perf_counter()
        xq = oracle.quantize_q8_1(x)
        oracle.gemv_q4k_q8_int(w, xq)
        wall += time.perf_counter() - t0
        cpu += time.process_time() - c0
        reps += 1
    rate = reps * W_BYTES / wall / 1e9

    per = {}

    def record(name, fn, weight_bytes):
        sec, cpus = _median_run(fn)
        per[name] = {"ms": round(sec * 1e3, 2), "weight_gbs": round(weight_bytes / sec / 1e9, 4),
                     "threads_busy": round(cpus / sec, 2)}

    # config 0: 896 x (896 -> 1024)
    w0 = synth.q4k_weights(synth.rng(0, 1), 896, 1024)
    x0 = np.zeros(1024, np.float32)
    x0[:896] = synth.activation(synth.rng(0, synth.T_ACT), 896)
    record("q4k_896x1024", lambda: oracle.gemv_q4k_q8_int(w0, oracle.quantize_q8_1(x0)),
           q4k_bytes(896, 1024))
    del w0
    # config 1: attention projections on one activation
    shapes = [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096)]
    wa = [synth.q4k_weights(synth.rng(1, 1 + k), o, i) for k, (o, i) in enumerate(shapes)]
    x1 = synth.activation(synth.rng(1, synth.T_ACT), IN_DIM)

    def attn():
        xq1 = oracle.quantize_q8_1(x1)
        for wk in wa:
            oracle.gemv_q4k_q8_int(wk, xq1)
    record("attn_qkvo_4096", attn, sum(q4k_bytes(o, i) for o, i in shapes))
    del wa
    # config 2: the SwiGLU chain
    INTER = 14336
    wg = synth.q4k_weights(synth.rng(2, 1), INTER, IN_DIM)
    wu = synth.q4k_weights(synth.rng(2, 2), INTER, IN_DIM)
    wd = synth.q4k_weights(synth.rng(2, 3), IN_DIM, INTER)
    record("swiglu_ffn_4096_14336",
           lambda: oracle.ffn_swiglu_q4k(wg, wu, wd, oracle.quantize_q8_1(x)), 3 * W_BYTES)
    del wu, wd
    # config 4: 8 tokens, one weight matrix
    x4 = synth.activation(synth.rng(4, synth.T_ACT), IN_DIM, 8)

    def batch8():
        xq4 = oracle.quantize_q8_1(x4)
        for t in range(8):
            oracle.gemv_q4k_q8_int(wg, xq4.token(t))
    record("q4k_batch8_4096x14336", batch8, W_BYTES)
    del wg
    # config 3: the Q4_0 LM head, fp32 and Q8_1 activation
    VOCAB, HID, HID_P = 151936, 896, 1024
    wl = synth.q4_0_weights(synth.rng(3, 1), VOCAB, HID_P)
    xl = np.zeros(HID_P, np.float32)
    xl[:HID] = synth.activation(synth.rng(3, synth.T_ACT), HID)
    record("q4_0_lm_head_151936x1024_fp32", lambda: oracle.gemv_q4_0_f32(wl, xl),
           q4_0_bytes(VOCAB, HID_P))
    record("q4_0_lm_head_151936x1024_q8_1",
           lambda: oracle.gemv_q4_0_q8_int(wl, oracle.quantize_q8_1(xl)), q4_0_bytes(VOCAB, HID_P))
    del wl
    return {"value": round(rate, 4), "unit": "GB/s", "cores": max(1, round(cpu / wall)),
            "kind": "oracle", "cpu_model": _cpu_model(),
            "host_cores": len(os.sched_getaffinity(0)), "blas": _blas_threads(),
            "sample": "%d full passes (quantize 4096 + integer-form GEMV 14336x4096, numpy), "
                      "%.1f s wall; per_config: median of 3 runs of each workload's oracle"
                      % (reps, wall),
            "per_config": per}


def q4k_bytes(out_dim: int, in_dim: int) -> int:
    return out_dim * (in_dim // 256) * 144


def q4_0_bytes(out_dim: int, in_dim: int) -> int:
    return out_dim * (in_dim // 32) * 18


def q8_bytes(n: int) -> int:
    return (n // 32) * 40


def row_entry(seconds: float, algo_bytes: int, weight_bytes: int, launches: str) -> dict:
    gbs = algo_bytes / seconds / 1e9
    return {"us": round(seconds * 1e6, 3), "launches": launches, "algo_bytes": algo_bytes,
            "weight_gbs": round(weight_bytes / seconds / 1e9, 2), "algo_gbs": round(gbs, 2),
            "frac": round(gbs / HBM_PEAK_GBS, 4)}


def time_rows(lib, rz, torch, dev, graph_time, copies, x, xq, y) -> dict:
    """Every kernel of the path at its own workload.  Each row rotates over its
    own weight copies (>= 1 GiB in all), so every call streams its weights from
    HBM; times are graph-replay means per call, as for the step."""
    import synth

    def rotated(blobs):
        reps = max(1, -(-ROTATE_BYTES // sum(b.size for b in blobs)))
        first = [torch.from_numpy(b.reshape(-1).copy()).to(dev) for b in blobs]
        return [first] + [[t.clone() for t in first] for _ in range(reps - 1)]

    def check(rc):
        if rc:
            raise RuntimeError(rz.rz_last_error())

    rows = {}
    x_p, xq_p, y_p = x.data_ptr(), xq.data_ptr(), y.data_ptr()
    n_copies = len(copies)
    w_p = [c.data_ptr() for c in copies]

    # a1: Q8_1 quantize of one 4096-value activation (launch-latency bound)
    rows["q8_1_quantize_4096"] = row_entry(
        graph_time(lambda i, s: check(lib.rz_q8_1_quantize(x_p, IN_DIM, IN_DIM, 1, xq_p, s))),
        X_BYTES + XQ_BYTES, 0, "rz_q8_1_quantize")
    check(lib.rz_q8_1_quantize(x_p, IN_DIM, IN_DIM, 1, xq_p, torch.cuda.current_stream().cuda_stream))

    # RMSNorm fused with the Q8_1 quantize (the attention and FFN inputs)
    gam = torch.from_numpy(synth.norm_weights(synth.rng(1, synth.T_GAMMA), IN_DIM)).to(dev)
    xq_n = torch.empty(XQ_BYTES, dtype=torch.uint8, device=dev)
    rows["rmsnorm_q8_1_4096"] = row_entry(
        graph_time(lambda i, s: check(lib.rz_rmsnorm_q8_1(x_p, gam.data_ptr(), 1e-5, IN_DIM,
                                                          IN_DIM, 1, None, xq_n.data_ptr(), s))),
        2 * X_BYTES + XQ_BYTES, 0, "rz_rmsnorm_q8_1")

    # a2+a3: the GEMV alone over the shared Q8_1 activation
    rows["q4k_gemv_4096x14336"] = row_entry(
        graph_time(lambda i, s: check(lib.rz_q4k_q8_gemv(w_p[i % n_copies], xq_p, y_p, OUT_DIM,
                                                         IN_DIM, 1, s))),
        GEMV_ALGO_BYTES, W_BYTES, "rz_q4k_q8_gemv")

    # the same GEMV on the fp32 activation, no Q8_1 (the non-quantized path)
    rows["q4k_gemv_xf32_4096x14336"] = row_entry(
        graph_time(lambda i, s: check(lib.rz_q4k_gemv(w_p[i % n_copies], x_p, IN_DIM, y_p,
                                                      OUT_DIM, IN_DIM, s))),
        W_BYTES + X_BYTES + Y_BYTES, W_BYTES, "rz_q4k_gemv (fp32 x)")

    # a8: 8 tokens, one weight pass
    x8 = torch.from_numpy(synth.activation(synth.rng(4, synth.T_ACT), IN_DIM, 8)).to(dev)
    xq8 = torch.empty(8 * XQ_BYTES, dtype=torch.uint8, device=dev)
    y8 = torch.empty(8 * OUT_DIM, dtype=torch.float32, device=dev)
    check(lib.rz_q8_1_quantize(x8.data_ptr(), IN_DIM, IN_DIM, 8, xq8.data_ptr(),
                               torch.cuda.current_stream().cuda_stream))
    rows["q4k_gemv_batch8_4096x14336"] = row_entry(
        graph_time(lambda i, s: check(lib.rz_q4k_q8_gemv(w_p[i % n_copies], xq8.data_ptr(),
                                                         y8.data_ptr(), OUT_DIM, IN_DIM, 8, s))),
        W_BYTES + 8 * XQ_BYTES + 8 * Y_BYTES, W_BYTES, "rz_q4k_q8_gemv n_tokens=8")

    # attention projections of one layer: Q 4096x4096, K and V 1024x4096, O 4096x4096
    shapes = [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096)]
    attn = rotated([synth.q4k_weights(synth.rng(1, 1 + k), o, i) for k, (o, i) in enumerate(shapes)])
    ya = torch.empty(4096, dtype=torch.float32, device=dev)
    attn_p = [[t.data_ptr() for t in c] for c in attn]

    def attn_body(i, s):
        ws = attn_p[i % len(attn_p)]
        for w, (o, n) in zip(ws, shapes):
            check(lib.rz_q4k_q8_gemv(w, xq_p, ya.data_ptr(), o, n, 1, s))

    import ctypes
    outs = [torch.empty(o, dtype=torch.float32, device=dev) for o, _ in shapes]
    ods = (ctypes.c_int * 4)(*[o for o, _ in shapes])
    yarr = (ctypes.c_void_p * 4)(*[t.data_ptr() for t in outs])
    warrs = [(ctypes.c_void_p * 4)(*c) for c in attn_p]

    def attn_multi(i, s):
        check(lib.rz_q4k_q8_gemv_multi(4, warrs[i % len(warrs)], yarr, ods, xq_p, 4096, 1, s))

    attn_w = sum(q4k_bytes(o, n) for o, n in shapes)
    attn_bytes = attn_w + XQ_BYTES + 4 * (4096 + 1024 + 1024 + 4096)
    rows["attn_qkvo_4096"] = row_entry(
        graph_time(attn_multi), attn_bytes, attn_w,
        "rz_q4k_q8_gemv_multi: Q, K, V, O in one launch on one Q8_1 activation")
    rows["attn_qkvo_4096_separate"] = row_entry(
        graph_time(attn_body), attn_w + 4 * XQ_BYTES + 4 * (4096 + 1024 + 1024 + 4096), attn_w,
        "4 x rz_q4k_q8_gemv (Q, K, V, O) on one Q8_1 activation")

    # the O projection alone, and with the residual add in its store (in place)
    o_w = q4k_bytes(4096, 4096)
    hid = torch.zeros(4096, dtype=torch.float32, device=dev)
    rows["o_proj_4096"] = row_entry(
        graph_time(lambda i, s: check(lib.rz_q4k_q8_gemv(attn_p[i % len(attn_p)][3], xq_p,
                                                         ya.data_ptr(), 4096, 4096, 1, s))),
        o_w + XQ_BYTES + 4 * 4096, o_w, "rz_q4k_q8_gemv")
    rows["o_proj_add_4096"] = row_entry(
        graph_time(lambda i, s: check(lib.rz_q4k_q8_gemv_add(attn_p[i % len(attn_p)][3], xq_p,
                                                             hid.data_ptr(), hid.data_ptr(),
                                                             4096, 4096, 1, s))),
        o_w + XQ_BYTES + 8 * 4096, o_w, "rz_q4k_q8_gemv_add (hidden += O x, in place)")
    # the attention output as fp32: quantize + O + residual in one launch, and as two
    ao = torch.from_numpy(synth.activation(synth.rng(1, 5), 4096)).to(dev)
    xq_o = torch.empty(XQ_BYTES, dtype=torch.uint8, device=dev)

    def o_f32_add(i, s, hp=None):
        hp = hp or hid.data_ptr()
        check(lib.rz_q4k_q8_gemv_f32_add(attn_p[i % len(attn_p)][3], ao.data_ptr(), 4096, None, hp,
                                         hp, 4096, 4096, s))

    def o_two_launch(i, s):
        check(lib.rz_q8_1_quantize(ao.data_ptr(), 4096, 4096, 1, xq_o.data_ptr(), s))
        check(lib.rz_q4k_q8_gemv_add(attn_p[i % len(attn_p)][3], xq_o.data_ptr(), hid.data_ptr(),
                                     hid.data_ptr(), 4096, 4096, 1, s))

    rows["o_proj_f32_add_4096"] = row_entry(
        graph_time(o_f32_add), o_w + 4 * 4096 + 8 * 4096, o_w,
        "rz_q4k_q8_gemv_f32_add (Q8_1 of the fp32 attention output, O, hidden += in place)")
    rows["o_proj_f32_add_4096_two_launch"] = row_entry(
        graph_time(o_two_launch), o_w + 4 * 4096 + 2 * XQ_BYTES + 8 * 4096, o_w,
        "rz_q8_1_quantize, then rz_q4k_q8_gemv_add")

    # SwiGLU chain 4096 -> 14336 -> 4096, and its down projection alone
    INTER = 14336
    ffn = rotated([synth.q4k_weights(synth.rng(2, 1), INTER, IN_DIM),
                   synth.q4k_weights(synth.rng(2, 2), INTER, IN_DIM),
                   synth.q4k_weights(synth.rng(2, 3), IN_DIM, INTER)])
    ffn_p = [[t.data_ptr() for t in c] for c in ffn]
    h = torch.empty(INTER, dtype=torch.float32, device=dev)
    hq = torch.empty(q8_bytes(INTER), dtype=torch.uint8, device=dev)
    yf = torch.empty(IN_DIM, dtype=torch.float32, device=dev)

    def ffn_body(i, s):
        wg, wu, wd = ffn_p[i % len(ffn_p)]
        check(lib.rz_swiglu_ffn_q4k(wg, wu, wd, xq_p, h.data_ptr(), hq.data_ptr(), yf.data_ptr(),
                                    None, IN_DIM, INTER, s))

    ffn_w = 3 * W_BYTES
    rows["swiglu_ffn_4096_14336"] = row_entry(
        graph_time(ffn_body),
        ffn_w + XQ_BYTES + 4 * INTER + 2 * q8_bytes(INTER) + 4 * IN_DIM, ffn_w,
        "rz_swiglu_ffn_q4k (gate/up + silu*up + requantize, then down)")
    hid_f = torch.zeros(IN_DIM, dtype=torch.float32, device=dev)

    def ffn_add_body(i, s):
        wg, wu, wd = ffn_p[i % len(ffn_p)]
        check(lib.rz_swiglu_ffn_q4k_add(wg, wu, wd, xq_p, h.data_ptr(), hq.data_ptr(),
                                        hid_f.data_ptr(), hid_f.data_ptr(), None, IN_DIM, INTER,
                                        s))

    rows["swiglu_ffn_add_4096_14336"] = row_entry(
        graph_time(ffn_add_body),
        ffn_w + XQ_BYTES + 4 * INTER + 2 * q8_bytes(INTER) + 8 * IN_DIM, ffn_w,
        "rz_swiglu_ffn_q4k_add (the chain, then hidden += y in the down store)")
    xf = torch.from_numpy(synth.activation(synth.rng(2, synth.T_ACT), IN_DIM)).to(dev)

    def ffn_f32_body(i, s):
        wg, wu, wd = ffn_p[i % len(ffn_p)]
        check(lib.rz_swiglu_ffn_q4k_f32(wg, wu, wd, xf.data_ptr(), h.data_ptr(), yf.data_ptr(),
                                        None, IN_DIM, INTER, s))

    rows["swiglu_ffn_f32_4096_14336"] = row_entry(
        graph_time(ffn_f32_body), ffn_w + 4 * IN_DIM + 2 * 4 * INTER + 4 * IN_DIM, ffn_w,
        "rz_swiglu_ffn_q4k_f32 (fp32 x and h, no Q8_1)")
    rows["q4k_gemv_xf32_down_14336x4096"] = row_entry(
        graph_time(lambda i, s: check(lib.rz_q4k_gemv(ffn_p[i % len(ffn_p)][2], h.data_ptr(),
                                                      INTER, yf.data_ptr(), IN_DIM, INTER, s))),
        W_BYTES + 4 * INTER + 4 * IN_DIM, W_BYTES, "rz_q4k_gemv (fp32 x, in_dim 14336)")
    rows["q4k_gemv_down_14336x4096"] = row_entry(
        graph_time(lambda i, s: check(lib.rz_q4k_q8_gemv(ffn_p[i % len(ffn_p)][2], hq.data_ptr(),
                                                         yf.data_ptr(), IN_DIM, INTER, 1, s))),
        W_BYTES + q8_bytes(INTER) + 4 * IN_DIM, W_BYTES, "rz_q4k_q8_gemv")

    # RMSNorm + Q8_1 + the Q, K, V projections, in one launch and as two; then
    # one decode layer's projections in sequence, as a model would chain them:
    # RMSNorm + Q8_1 + Q/K/V in one launch, the attention output (stood in for
    # by q) quantized for O and O with the residual in one launch, then
    # RMSNorm + Q8_1 + the SwiGLU chain with the residual; weights of both
    # halves rotated
    gam_l = torch.from_numpy(synth.norm_weights(synth.rng(1, synth.T_GAMMA), IN_DIM)).to(dev)
    hid_l = torch.from_numpy(synth.activation(synth.rng(1, synth.T_ACT), IN_DIM)).to(dev)
    xq_l = torch.empty(XQ_BYTES, dtype=torch.uint8, device=dev)
    qkv = [torch.empty(o, dtype=torch.float32, device=dev) for o, _ in shapes[:3]]
    qkv_y = (ctypes.c_void_p * 3)(*[t.data_ptr() for t in qkv])
    qkv_od = (ctypes.c_int * 3)(*[o for o, _ in shapes[:3]])
    qkv_w = [(ctypes.c_void_p * 3)(*c[:3]) for c in attn_p]

    def qkv_separate(i, s):
        check(lib.rz_rmsnorm_q8_1(hid_l.data_ptr(), gam_l.data_ptr(), 1e-5, IN_DIM, IN_DIM, 1,
                                  None, xq_l.data_ptr(), s))
        check(lib.rz_q4k_q8_gemv_multi(3, qkv_w[i % len(qkv_w)], qkv_y, qkv_od, xq_l.data_ptr(),
                                       IN_DIM, 1, s))

    def qkv_fused(i, s):
        check(lib.rz_rmsnorm_q4k_q8_gemv_multi(3, qkv_w[i % len(qkv_w)], qkv_y, qkv_od,
                                               hid_l.data_ptr(), gam_l.data_ptr(), 1e-5, IN_DIM,
                                               None, IN_DIM, s))

    qkv_wb = sum(q4k_bytes(o, n) for o, n in shapes[:3])
    qkv_bytes = qkv_wb + 2 * X_BYTES + 4 * (4096 + 1024 + 1024)
    rows["rmsnorm_qkv_4096"] = row_entry(
        graph_time(qkv_fused), qkv_bytes, qkv_wb,
        "rz_rmsnorm_q4k_q8_gemv_multi: RMSNorm + Q8_1 + Q, K, V in one launch")
    rows["rmsnorm_qkv_4096_two_launch"] = row_entry(
        graph_time(qkv_separate), qkv_bytes + 2 * XQ_BYTES, qkv_wb,
        "rz_rmsnorm_q8_1, then rz_q4k_q8_gemv_multi (Q, K, V)")

    hid_n = torch.from_numpy(synth.activation(synth.rng(2, synth.T_ACT), IN_DIM)).to(dev)

    def ffn_norm_separate(i, s):
        wg, wu, wd = ffn_p[i % len(ffn_p)]
        hp, xp = hid_n.data_ptr(), xq_l.data_ptr()
        check(lib.rz_rmsnorm_q8_1(hp, gam_l.data_ptr(), 1e-5, IN_DIM, IN_DIM, 1, None, xp, s))
        check(lib.rz_swiglu_ffn_q4k_add(wg, wu, wd, xp, h.data_ptr(), hq.data_ptr(), hp, hp, None,
                                        IN_DIM, INTER, s))

    def ffn_norm_fused(i, s, hp=None):
        wg, wu, wd = ffn_p[i % len(ffn_p)]
        hp = hp or hid_n.data_ptr()
        check(lib.rz_rmsnorm_swiglu_ffn_q4k_add(wg, wu, wd, hp, gam_l.data_ptr(), 1e-5,
                                                h.data_ptr(), hq.data_ptr(), hp, None, IN_DIM,
                                                INTER, s))

    ffn_norm_bytes = ffn_w + 4 * X_BYTES + 4 * INTER + 2 * q8_bytes(INTER)
    rows["rmsnorm_swiglu_ffn_add_4096_14336"] = row_entry(
        graph_time(ffn_norm_fused), ffn_norm_bytes, ffn_w,
        "rz_rmsnorm_swiglu_ffn_q4k_add: RMSNorm + Q8_1 in every gate/up workgroup, then down "
        "+ residual (2 kernels)")
    rows["rmsnorm_swiglu_ffn_add_4096_14336_three_launch"] = row_entry(
        graph_time(ffn_norm_separate), ffn_norm_bytes + 2 * XQ_BYTES, ffn_w,
        "rz_rmsnorm_q8_1, then rz_swiglu_ffn_q4k_add")

    def layer_body(i, s):
        a_w = attn_p[i % len(attn_p)]
        hp = hid_l.data_ptr()
        qkv_fused(i, s)
        check(lib.rz_q4k_q8_gemv_f32_add(a_w[3], qkv[0].data_ptr(), IN_DIM, None, hp, hp, IN_DIM,
                                         IN_DIM, s))
        ffn_norm_fused(i, s, hp)

    layer_w = attn_w + ffn_w
    rows["decode_layer_4096_14336"] = row_entry(
        graph_time(layer_body), layer_w + 9 * X_BYTES + 4 * 6144
        + 4 * INTER + 2 * q8_bytes(INTER), layer_w,
        "one layer's projections: RMSNorm+Q8_1+Q/K/V (one launch), Q8_1+O+residual (one launch), "
        "RMSNorm+Q8_1+SwiGLU gate/up (one launch), down+residual (4 kernels)")
    del ffn, attn

    # Q4_0 LM head 151936 x (896 -> 1024), fp32 and Q8_1 activation
    VOCAB, HID, HID_P = 151936, 896, 1024
    lm = rotated([synth.q4_0_weights(synth.rng(3, 1), VOCAB, HID_P)])
    lm_p = [c[0].data_ptr() for c in lm]
    xl = torch.zeros(HID_P, dtype=torch.float32, device=dev)
    xl[:HID] = torch.from_numpy(synth.activation(synth.rng(3, synth.T_ACT), HID)).to(dev)
    xlq = torch.empty(q8_bytes(HID_P), dtype=torch.uint8, device=dev)
    check(lib.rz_q8_1_quantize(xl.data_ptr(), HID, HID_P, 1, xlq.data_ptr(),
                               torch.cuda.current_stream().cuda_stream))
    logits = torch.empty(VOCAB, dtype=torch.float32, device=dev)
    lm_w = q4_0_bytes(VOCAB, HID_P)
    for fmt, xp, xbytes, name in ((0, xl.data_ptr(), 4 * HID_P, "fp32"),
                                  (1, xlq.data_ptr(), q8_bytes(HID_P), "q8_1")):
        rows["q4_0_lm_head_151936x1024_%s" % name] = row_entry(
            graph_time(lambda i, s: check(lib.rz_q4_0_gemv(lm_p[i % len(lm_p)], xp, fmt,
                                                           logits.data_ptr(), VOCAB, HID_P, s))),
            lm_w + xbytes + 4 * VOCAB, lm_w, "rz_q4_0_gemv x_format=%d" % fmt)
    # the same with the output bias and the greedy token (two kernels: the GEMV
    # with its epilogue, then the merge of the per-workgroup pairs)
    lm_bias = torch.from_numpy(synth.activation(synth.rng(3, 8), VOCAB)).to(dev)
    am_idx = torch.zeros(1, dtype=torch.int32, device=dev)
    am_val = torch.zeros(1, dtype=torch.float32, device=dev)
    for fmt, xp, xbytes, name in ((0, xl.data_ptr(), 4 * HID_P, "fp32"),
                                  (1, xlq.data_ptr(), q8_bytes(HID_P), "q8_1")):
        ws_bytes = lib.rz_lm_head_q4_0_workspace_bytes(VOCAB, HID_P, fmt)
        ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
        rows["q4_0_lm_head_bias_argmax_151936x1024_%s" % name] = row_entry(
            graph_time(lambda i, s: check(lib.rz_lm_head_q4_0(
                lm_p[i % len(lm_p)], xp, fmt, lm_bias.data_ptr(), logits.data_ptr(), VOCAB,
                HID_P, am_idx.data_ptr(), am_val.data_ptr(), ws.data_ptr(), ws_bytes, s))),
            lm_w + xbytes + 8 * VOCAB, lm_w,
            "rz_lm_head_q4_0 x_format=%d (bias + argmax epilogue, merge kernel)" % fmt)
    # the same with the top 40 instead of the greedy token (GEMV + bias, then
    # the slice and merge kernels of the selection)
    tk_idx = torch.zeros(128, dtype=torch.int32, device=dev)
    tk_val = torch.zeros(128, dtype=torch.float32, device=dev)
    tk_ws = torch.zeros(lib.rz_topk_f32_workspace_bytes(VOCAB, 128), dtype=torch.uint8,
                        device=dev)
    rows["q4_0_lm_head_bias_topk40_151936x1024_fp32"] = row_entry(
        graph_time(lambda i, s: check(lib.rz_lm_head_q4_0_topk(
            lm_p[i % len(lm_p)], xl.data_ptr(), 0, lm_bias.data_ptr(), logits.data_ptr(), VOCAB,
            HID_P, 40, tk_idx.data_ptr(), tk_val.data_ptr(), tk_ws.data_ptr(),
            lib.rz_topk_f32_workspace_bytes(VOCAB, 40), s))),
        lm_w + 4 * HID_P + 8 * VOCAB + 8 * 40, lm_w,
        "rz_lm_head_q4_0_topk x_format=0, k=40 (GEMV + bias, top-k slice and merge kernels)")
    # the selection alone over the 151936 logits
    for k in (1, 40, 128):
        rows["topk%d_151936" % k] = row_entry(
            graph_time(lambda i, s, k=k: check(lib.rz_topk_f32(
                logits.data_ptr(), VOCAB, k, tk_idx.data_ptr(), tk_val.data_ptr(),
                tk_ws.data_ptr(), lib.rz_topk_f32_workspace_bytes(VOCAB, k), s))),
            4 * VOCAB + 8 * k, 0, "rz_topk_f32 k=%d (slice kernel, merge kernel)" % k)
    del lm

    # GELU FFN of a phi-2-sized layer on Q4_0 weights, 2560 -> 10240 -> 2560, with biases
    GH, GI = 2560, 10240
    gelu_w = rotated([synth.q4_0_weights(synth.rng(5, 1), GI, GH),
                      synth.q4_0_weights(synth.rng(5, 2), GH, GI)])
    gelu_p = [[t.data_ptr() for t in c] for c in gelu_w]
    gx = torch.from_numpy(synth.activation(synth.rng(5, synth.T_ACT), GH)).to(dev)
    gub = torch.from_numpy(synth.activation(synth.rng(5, 7), GI)).to(dev)
    gdb = torch.from_numpy(synth.activation(synth.rng(5, 8), GH)).to(dev)
    gh = torch.empty(GI, dtype=torch.float32, device=dev)
    gy = torch.empty(GH, dtype=torch.float32, device=dev)

    def gelu_body(i, s):
        wu, wd = gelu_p[i % len(gelu_p)]
        check(lib.rz_gelu_ffn_q4_0(wu, wd, gx.data_ptr(), gub.data_ptr(), gdb.data_ptr(),
                                   gh.data_ptr(), gy.data_ptr(), GH, GI, s))

    gelu_wb = 2 * q4_0_bytes(GI, GH)
    rows["gelu_ffn_q4_0_2560_10240"] = row_entry(
        graph_time(gelu_body), gelu_wb + 4 * GH + 4 * GI + 2 * 4 * GI + 4 * GH + 4 * GH, gelu_wb,
        "rz_gelu_ffn_q4_0 (up + bias + GELU, then down + bias)")
    del gelu_w

    # the small case: 896 x (896 -> 1024), launch-bound
    small = rotated([synth.q4k_weights(synth.rng(0, 1), 896, 1024)])
    small_p = [c[0].data_ptr() for c in small]
    xs = torch.zeros(1024, dtype=torch.float32, device=dev)
    xs[:896] = torch.from_numpy(synth.activation(synth.rng(0, synth.T_ACT), 896)).to(dev)
    ys = torch.empty(896, dtype=torch.float32, device=dev)
    rows["q4k_fused_896x1024"] = row_entry(
        graph_time(lambda i, s: check(lib.rz_q4k_q8_gemv_f32(small_p[i % len(small_p)],
                                                             xs.data_ptr(), 896, None,
                                                             ys.data_ptr(), 896, 1024, s))),
        q4k_bytes(896, 1024) + 4 * 896 + 4 * 896, q4k_bytes(896, 1024), "rz_q4k_q8_gemv_f32")
    del small
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rows


def _stream_read_lib():
    import ctypes
    path = os.path.join(ROOT, "q4_q8_integer_quantize_amd", "librz_stream_read.so")
    rd = ctypes.CDLL(path)
    for fn in (rd.rz_stream_read, rd.rz_stream_read_once):
        fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                       ctypes.c_void_p]
        fn.restype = ctypes.c_int
    return rd


# read shapes tried for a ceiling: ("stride", grid) = grid-stride loop over `grid`
# workgroups; ("once", u) = one-shot grid, u 16-byte chunks a thread
READ_SHAPES = (("stride", 256), ("stride", 512), ("stride", 1024), ("stride", 2048),
               ("stride", 4096), ("once", 1), ("once", 2), ("once", 4))


def _read_call(rd, shape, ptr, nbytes, sink, strm) -> int:
    kind, k = shape
    if kind == "stride":
        return rd.rz_stream_read(ptr, nbytes, sink, k, strm)
    return rd.rz_stream_read_once(ptr, nbytes, sink, k, strm)


def read_ceiling(torch, dev, graph_time, w_p, n_copies) -> dict:
    """A plain streaming read of the same 33 MB weight copies, rotated the same
    way (librz_stream_read.so, not part of the path): what a kernel that only
    reads these bytes reaches on this part.  The best of several read shapes."""
    rd = _stream_read_lib()
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    best = None
    for shape in READ_SHAPES:
        def body(i, strm, shape=shape):
            if _read_call(rd, shape, w_p[i % n_copies], W_BYTES, sink.data_ptr(), strm):
                raise RuntimeError("rz_stream_read failed")
        sec = graph_time(body)
        if best is None or sec < best[0]:
            best = (sec, shape)
    return {"what": "plain non-temporal read of the step's weight bytes, same rotation, "
                    "best of grid-stride and one-shot shapes",
            "bytes": W_BYTES, "us": round(best[0] * 1e6, 3),
            "gbs": round(W_BYTES / best[0] / 1e9, 2),
            "shape": "%s %d" % best[1],
            "frac": round(W_BYTES / best[0] / 1e9 / HBM_PEAK_GBS, 4)}


def add_row_ceilings(rows: dict, torch, dev, graph_time) -> None:
    """Next to every row, a plain streaming read of the row's algorithmic bytes
    (rotated through 1 GiB, so every call reads from HBM, the best of four read
    shapes): a launch that moves a few MB pays the same fixed launch and ramp
    cost as this read, and `frac_of_ceiling` says how close the row comes to
    the read of its own size."""
    rd = _stream_read_lib()
    buf = torch.zeros(ROTATE_BYTES + (128 << 20), dtype=torch.uint8, device=dev)
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    base = buf.data_ptr()
    cache = {}
    for row in rows.values():
        nb = -(-row["algo_bytes"] // 256) * 256
        if nb > (128 << 20):
            continue
        if nb not in cache:
            span = max(1, ROTATE_BYTES // nb)
            best = None
            for shape in (("stride", 1024), ("stride", 2048), ("once", 1), ("once", 2)):
                def body(i, strm, shape=shape, nb=nb, span=span):
                    if _read_call(rd, shape, base + (i % span) * nb, nb, sink.data_ptr(), strm):
                        raise RuntimeError("rz_stream_read failed")
                sec = graph_time(body)
                best = sec if best is None else min(best, sec)
            cache[nb] = best
        row["read_ceiling_us"] = round(cache[nb] * 1e6, 3)
        row["frac_of_ceiling"] = round(cache[nb] * 1e6 / row["us"], 4)
    del buf
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


ONLY = {
    "step": "rz_q4k_q8_gemv_f32 4096 -> 14336",
    "gemv": "rz_q4k_q8_gemv 4096 -> 14336, 1 token",
    "batch8": "rz_q4k_q8_gemv 4096 -> 14336, 8 tokens",
    "lm_head_fp32": "rz_q4_0_gemv 151936 x 1024, fp32 x",
    "lm_head_q8": "rz_q4_0_gemv 151936 x 1024, Q8_1 x",
    "rmsnorm": "rz_rmsnorm_q8_1 4096, 1 token",
}


def rotated_copies(torch, dev, blob):
    """Device copies of a weight blob, >= 1 GiB in all, so that consecutive
    launches find none of their weights in a cache."""
    first = torch.from_numpy(blob.reshape(-1).copy()).to(dev)
    return [first] + [first.clone() for _ in range(-(-ROTATE_BYTES // blob.size) - 1)]


def run_only(name: str, launches: int) -> int:
    """Run one kernel `launches` times over >= 1 GiB of weight copies, untimed."""
    import numpy as np
    import torch
    import synth
    import q4_q8_integer_quantize_amd as rz
    dev = torch.device("cuda:0")
    if name == "rmsnorm":
        x = torch.from_numpy(synth.activation(synth.rng(1, synth.T_ACT), IN_DIM)).to(dev)
        gam = torch.from_numpy(synth.norm_weights(synth.rng(1, synth.T_GAMMA), IN_DIM)).to(dev)
        xq = torch.empty(XQ_BYTES, dtype=torch.uint8, device=dev)
        for i in range(launches):
            rz.rz_rmsnorm_q8_1(x, gam, 1e-5, IN_DIM, IN_DIM, 1, None, xq)
    elif name.startswith("lm_head"):
        V, H = 151936, 1024
        blob = synth.q4_0_weights(synth.rng(3, 1), V, H)
        x = np.zeros(H, np.float32)
        x[:896] = synth.activation(synth.rng(3, synth.T_ACT), 896)
        xd = torch.from_numpy(x).to(dev)
        xq = torch.empty((H // 32) * 40, dtype=torch.uint8, device=dev)
        rz.rz_q8_1_quantize(xd, 896, H, 1, xq)
        y = torch.empty(V, dtype=torch.float32, device=dev)
        ws = rotated_copies(torch, dev, blob)
        fmt = 0 if name == "lm_head_fp32" else 1
        for i in range(launches):
            rz.rz_q4_0_gemv(ws[i % len(ws)], xd if fmt == 0 else xq, fmt, y, V, H)
    else:
        nt = 8 if name == "batch8" else 1
        blob = synth.q4k_weights(synth.rng(2, synth.T_W0), OUT_DIM, IN_DIM)
        ws = rotated_copies(torch, dev, blob)
        x = torch.from_numpy(synth.activation(synth.rng(4, synth.T_ACT), IN_DIM, nt)).to(dev)
        xq = torch.empty(nt * XQ_BYTES, dtype=torch.uint8, device=dev)
        rz.rz_q8_1_quantize(x, IN_DIM, IN_DIM, nt, xq)
        y = torch.empty(nt * OUT_DIM, dtype=torch.float32, device=dev)
        for i in range(launches):
            if name == "step":
                rz.rz_q4k_q8_gemv_f32(ws[i % len(ws)], x, IN_DIM, None, y, OUT_DIM, IN_DIM)
            else:
                rz.rz_q4k_q8_gemv(ws[i % len(ws)], xq, y, OUT_DIM, IN_DIM, nt)
    torch.cuda.synchronize()
    print("ran %s x %d" % (ONLY[name], launches), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--only", choices=sorted(ONLY), default=None,
                    help="run one kernel of the path --launches times, untimed (for counter "
                         "collection under rocprofv3), then exit")
    ap.add_argument("--launches", type=int, default=12)
    ap.add_argument("--no-rows", action="store_true",
                    help="time only the step, not the other kernels of the path")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after timing, run 4 plain device copies of MIB MiB (a reference "
                         "for the HBM byte counters of a profiling run)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this path runs on one GPU; --gpus %d is not supported "
              "(output rows shard across GPUs without communication, so one GPU's share is "
              "what is measured)" % args.gpus,
              file=sys.stderr)
        return 2

    if args.only:
        return run_only(args.only, args.launches)

    import numpy as np
    import torch
    import synth
    import q4_q8_integer_quantize_amd as rz

    rz.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    w0 = synth.q4k_weights(synth.rng(2, synth.T_W0), OUT_DIM, IN_DIM)
    w0_dev = torch.from_numpy(w0.reshape(-1).copy()).to(dev)
    n_copies = -(-ROTATE_BYTES // W_BYTES)
    copies = [w0_dev] + [w0_dev.clone() for _ in range(n_copies - 1)]
    x = torch.from_numpy(synth.activation(synth.rng(2, synth.T_ACT), IN_DIM)).to(dev)
    xq = torch.empty(XQ_BYTES, dtype=torch.uint8, device=dev)
    y = torch.empty(OUT_DIM, dtype=torch.float32, device=dev)
    s = stream.cuda_stream

    lib = rz.load_library()
    x_p, xq_p, y_p = x.data_ptr(), xq.data_ptr(), y.data_ptr()
    w_p = [c.data_ptr() for c in copies]

    def fused(i, strm):
        # the step: Q8_1 quantize + Q4_K x Q8_1 GEMV in one launch
        if lib.rz_q4k_q8_gemv_f32(w_p[i % n_copies], x_p, IN_DIM, None, y_p, OUT_DIM, IN_DIM, strm):
            raise RuntimeError(rz.rz_last_error())

    def two_launch(i, strm):
        if (lib.rz_q8_1_quantize(x_p, IN_DIM, IN_DIM, 1, xq_p, strm)
                or lib.rz_q4k_q8_gemv(w_p[i % n_copies], xq_p, y_p, OUT_DIM, IN_DIM, 1, strm)):
            raise RuntimeError(rz.rz_last_error())

    def gemv_only(i, strm):
        if lib.rz_q4k_q8_gemv(w_p[i % n_copies], xq_p, y_p, OUT_DIM, IN_DIM, 1, strm):
            raise RuntimeError(rz.rz_last_error())

    # argument checks of the binding, once
    rz.rz_q4k_q8_gemv_f32(copies[0], x, IN_DIM, None, y, OUT_DIM, IN_DIM, s)
    rz.rz_q8_1_quantize(x, IN_DIM, IN_DIM, 1, xq, s)
    rz.rz_q4k_q8_gemv(copies[0], xq, y, OUT_DIM, IN_DIM, 1, s)
    torch.cuda.synchronize()
    K = args.steps
    W = max(1, args.warmup)

    def capture(body, first, count):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cs = torch.cuda.current_stream().cuda_stream
            for i in range(count):
                body(first + i, cs)
        return g

    def graph_time(body):
        """K calls of body, each on the next weight copy, captured in one HIP
        graph; the mean seconds per call over one replay bracketed by HIP events
        on the launch stream.  First both graphs run once untimed and the GPU is
        synchronized; then W untimed warm-up calls (the W copies before the
        timed ones, so the rotation runs on) are replayed back to back with
        the timed replay: the GPU is busy while the timed replay is queued, so
        the events bracket the K calls and not the host's graph launch."""
        g = capture(body, W, K)
        wg = capture(body, 0, W)
        wg.replay()
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        wg.replay()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / K

    # every other kernel first: seconds of back-to-back kernels bring the GPU
    # clocks to their sustained state before the step is timed
    rows = None if args.no_rows else time_rows(lib, rz, torch, dev, graph_time, copies, x, xq, y)
    if rows:
        add_row_ceilings(rows, torch, dev, graph_time)
    step_s = graph_time(fused)            # the timed steps (whole hot path)
    ceiling = read_ceiling(torch, dev, graph_time, w_p, n_copies)
    ms_step = step_s * 1e3
    two_s = graph_time(two_launch)        # same work as two launches
    gemv_s = graph_time(gemv_only)        # the GEMV kernel alone
    achieved = STEP_ALGO_BYTES / step_s / 1e9
    traffic = measured_traffic()

    if args.copy_calibration > 0:
        nbytes = args.copy_calibration << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    value = W_BYTES / (ms_step * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": "Q8_1 quantize + Q4_K x Q8_1 GEMV, 4096 -> 14336, batch 1 "
                        "(one launch, rz_q4k_q8_gemv_f32)",
            "out_dim": OUT_DIM, "in_dim": IN_DIM, "n_tokens": 1,
            "weight_bytes": W_BYTES, "weight_copies_rotated": n_copies,
            "pct_hbm_peak_step": round(100 * value / HBM_PEAK_GBS, 2),
        },
        "us_per_step": round(step_s * 1e6, 3),
        "two_launch_us_per_step": round(two_s * 1e6, 3),
        "gemv_kernel_us": round(gemv_s * 1e6, 3),
        "gemv_kernel_gbs": round(GEMV_ALGO_BYTES / gemv_s / 1e9, 2),
        "kernel_source_sha256_16": kernel_source_hash(),
        "rows": rows,
        "read_ceiling": dict(ceiling, step_frac_of_ceiling=round(achieved / ceiling["gbs"], 4)),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
        # each configuration's oracle time next to its GPU row
        if rows:
            for cfg, row in (("q4k_896x1024", "q4k_fused_896x1024"),
                             ("attn_qkvo_4096", "attn_qkvo_4096"),
                             ("swiglu_ffn_4096_14336", "swiglu_ffn_4096_14336"),
                             ("q4k_batch8_4096x14336", "q4k_gemv_batch8_4096x14336"),
                             ("q4_0_lm_head_151936x1024_fp32", "q4_0_lm_head_151936x1024_fp32"),
                             ("q4_0_lm_head_151936x1024_q8_1", "q4_0_lm_head_151936x1024_q8_1")):
                per = out["cpu_baseline"]["per_config"].get(cfg)
                if per and row in rows:
                    rows[row]["oracle_ms"] = per["ms"]
                    rows[row]["oracle_over_gpu"] = round(per["ms"] * 1e3 / rows[row]["us"], 1)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

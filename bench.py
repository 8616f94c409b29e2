"""Benchmark of the O-projection front half on one MI355X.

One step = one pass of the hot path over one batch of synthetic input: one
oproj_fused call -- inverse RoPE + 1x128 FP8 quantisation, then the grouped
wo_a GEMM, plus the dense wo_b GEMM for the workload that has one.  The kernels are also timed
one by one (oproj_inv_rope_quant, oproj_grouped_wo_a, oproj_dense_bf16_gemm).  The default workload
is the decode batch (T=64, 16 groups x 8 heads, D=4096, R=1024).

Inputs are resident in HBM before timing starts.  The steps rotate through
several copies of the inputs, weights and workspaces (more bytes than the
256 MB last-level cache) so weights are streamed from HBM every step.  The
rotation of C steps is captured once in a HIP graph and replayed (a decode
step is a few microseconds of GPU work, shorter than a Python launch).

Printed: one JSON line with the throughput, the roofline of the dominant
kernel (algorithmic bytes or FLOPs per launch / its average launch time from
HIP events around back-to-back replays) and the oracle's CPU baseline on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0   # dense FP8 MFMA
BF16_PEAK_TFLOPS = 2500.0  # dense BF16 MFMA


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def device_info() -> dict:
    """CU count and peak engine clock of device 0, read from the HIP runtime
    the library links, and the dense matrix-core peaks they imply (gfx950:
    8192 FP8 and 4096 BF16 FLOP per clock per CU).  The roofline fractions use
    the published peaks above; these are printed beside them as a check."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so.7")
    except OSError:
        return {}
    v = ctypes.c_int(0)
    info = {}
    for key, attr in (("cus", 63), ("clock_khz", 5)):  # hipDeviceAttributeMultiprocessorCount, ...ClockRate
        if hip.hipDeviceGetAttribute(ctypes.byref(v), attr, 0) != 0:
            return {}
        info[key] = v.value
    ghz = info["clock_khz"] / 1e6
    info["fp8_peak_tflops"] = info["cus"] * ghz * 8192 / 1e3
    info["bf16_peak_tflops"] = info["cus"] * ghz * 4096 / 1e3
    log(f"device: {info['cus']} CUs at {ghz:.2f} GHz peak -> dense FP8 {info['fp8_peak_tflops']:.0f} TFLOP/s, "
        f"BF16 {info['bf16_peak_tflops']:.0f} TFLOP/s")
    return info


def kernel_bytes_quant(w) -> int:
    """Algorithmic HBM bytes of a1+a2: read bf16 o, positions and the table
    rows; write FP8 codes and fp32 scales."""
    return w.T * w.H * 512 * 2 + w.T * 8 + w.T * 64 * 4 + w.T * w.n_groups * w.D + w.T * w.n_groups * w.KB * 4


def kernel_bytes_gemm(w) -> int:
    """Algorithmic HBM bytes of a3: FP8 weight + weight scales + live FP8
    activations + activation scales + bf16 z."""
    G, R, D, KB, T = w.n_groups, w.o_lora_rank, w.D, w.KB, w.T
    wrows = G * R
    wscales = (wrows if w.w_block_rows == 1 else (wrows + 127) // 128) * KB * 4
    return wrows * D + wscales + T * G * D + T * G * KB * 4 + T * G * R * 2


def kernel_flops_gemm(w) -> int:
    return 2 * w.T * w.n_groups * w.o_lora_rank * w.D


# the source files each kernel is built from (the counters are tied to them)
KERNEL_SOURCES = {
    "inv_rope_quant": ("rope_quant.hip", "rq_item.hpp", "device_common.hpp"),
    "grouped_wo_a": ("gemm_fp8.hip", "lds_dma.hpp", "device_common.hpp"),
    "wo_b": ("gemm_bf16.hip", "lds_dma.hpp", "device_common.hpp"),
    "fused_decode": ("gemm_fp8.hip", "rq_item.hpp", "lds_dma.hpp", "device_common.hpp"),
}


def source_sha(*names: str) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "attention_output_projection_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str, sha: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None when
    absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_sha") != sha:
        return None
    return int(d["bytes_per_launch"])


def cpu_baseline(w, o, pos, tab, wmat, max_tokens: int, reps: int = 3):
    """The oracle as it stands, on the first tokens of the same batch; the
    median of `reps` runs."""
    import oracle

    S = min(w.T, max_tokens)
    qw, sw = oracle.quant_weight(wmat, w.w_block_rows, w.pow2)  # offline weight prep, untimed
    threads = oracle.default_threads()
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        qa, sa = oracle.inv_rope_quant(o[:S], pos[:S], tab, w.n_groups, w.heads_per_group, pow2=w.pow2)
        oracle.grouped_gemm(qa, sa, qw, sw, w.n_groups, w.o_lora_rank, w.w_block_rows)
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    return {"value": S / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {S} of {w.T} tokens of the {w.name} batch: inverse RoPE + quant + "
                      f"grouped wo_a in fp64, median of {reps} runs of {dt:.2f} s "
                      f"({sum(times):.1f} s of CPU work)"}


def copy_calibration(torch, dev, mib: int) -> int:
    """A plain copy of a known size: each launch reads and writes mib MiB.
    Its FETCH_SIZE / WRITE_SIZE counters calibrate the HBM byte counts taken
    on the path's kernels."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(8):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"8 copies of {n} bytes")
    return 0


def bench_bf16(args, w, torch, ap, wl, dev) -> int:
    """The unquantised variant: oproj_inv_rope_bf16 then oproj_grouped_wo_a_bf16
    (bf16 weights), timed the same way as the quantised path."""
    if w.prequantised:
        log("the pre-quantised workload has no unquantised form")
        return 2
    log(f"unquantised path, workload {w.name}: T={w.T} G={w.n_groups} hpg={w.heads_per_group} D={w.D} "
        f"R={w.o_lora_rank}")
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    wq = wl.wo_a_bf16(w)
    per_copy = wq.nbytes + 2 * o.nbytes
    copies = args.copies or max(2, min(16, int(np.ceil(768e6 / per_copy))))
    log(f"{copies} rotating copies of {per_copy / 1e6:.1f} MB")
    shp = ap.Shape(T=w.T, n_groups=w.n_groups, heads_per_group=w.heads_per_group,
                   o_lora_rank=w.o_lora_rank, max_pos=w.max_pos)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    d_tab, d_pos = t(tab), t(pos)
    C = []
    for _ in range(copies):
        C.append({"o": t(o.view(np.int16)), "w": t(wq.view(np.int16)),
                  "x": torch.empty((w.T, w.n_groups, w.D), dtype=torch.int16, device=dev),
                  "z": torch.empty((w.T, w.n_groups, w.o_lora_rank), dtype=torch.int16, device=dev)})
    torch.cuda.synchronize()

    def rope(c):
        ap.oproj_inv_rope_bf16(shp, c["o"], d_pos, d_tab, c["x"])

    def gemm(c):
        ap.oproj_grouped_wo_a_bf16(shp, c["x"], None, c["w"], c["z"])

    def step(c):
        rope(c)
        gemm(c)

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for c in C:
                fn(c)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for c in C:
                fn(c)
        torch.cuda.synchronize()
        return g

    step(C[0])
    torch.cuda.synchronize()
    eager = C[0]["z"].clone()
    g_step, g_rope, g_gemm = capture(step), capture(rope), capture(gemm)
    g_step.replay()
    torch.cuda.synchronize()
    if not torch.equal(C[0]["z"], eager):
        log("graph replay differs from the eager result")
        return 1
    reps = max(1, args.steps // copies)
    K = reps * copies
    for _ in range(max(1, args.warmup // copies)):
        g_step.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        g_step.replay()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / K

    def kernel_time_us(g):
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.kernel_reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (args.kernel_reps * copies)

    t_rope, t_gemm = kernel_time_us(g_rope), kernel_time_us(g_gemm)
    log(f"{K} steps: {ms_per_step * 1e3:.2f} us/step; kernel averages: rope {t_rope:.2f} us, "
        f"grouped bf16 gemm {t_gemm:.2f} us")
    G, R, D, T = w.n_groups, w.o_lora_rank, w.D, w.T
    rope_bytes = 2 * T * w.H * 512 * 2 + T * 8 + T * 64 * 4
    gemm_bytes = G * R * D * 2 + T * G * D * 2 + T * G * R * 2
    gemm_flops = 2 * T * G * R * D
    hbm_bound = gemm_flops / gemm_bytes < BF16_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3
    kernels = {"inv_rope_bf16": {"us": t_rope, "bound": "hbm", "bytes": rope_bytes,
                                 "GB/s": rope_bytes / (t_rope * 1e3)},
               "grouped_wo_a_bf16": {"us": t_gemm, "bound": "hbm" if hbm_bound else "mfma",
                                     "bytes": gemm_bytes, "flops": gemm_flops,
                                     "GB/s": gemm_bytes / (t_gemm * 1e3), "TFLOP/s": gemm_flops / (t_gemm * 1e6)}}
    dom = max(kernels, key=lambda k: kernels[k]["us"])
    kd = kernels[dom]
    if kd["bound"] == "hbm":
        achieved, peak, unit = kd["GB/s"], HBM_PEAK_GBS, "GB/s"
    else:
        achieved, peak, unit = kd["TFLOP/s"], BF16_PEAK_TFLOPS, "TFLOP/s"
    result = {
        "metric": "tokens/s of the unquantised path (bf16 inverse RoPE + grouped bf16 wo_a)",
        "value": T / (ms_per_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": max(1, args.warmup // copies) * copies, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64 normals; random-init weights)",
        "config": {"workload": f"{w.name} unquantised: T={T} n_groups={G} heads_per_group={w.heads_per_group} "
                               f"D={D} o_lora_rank={R}", "global_batch": T, "parallelism": "single GPU",
                   "copies_rotated": copies},
        "device": device_info(),
        "roofline": {"bound": kd["bound"], "kernel": dom, "achieved": achieved, "peak": peak, "unit": unit,
                     "frac": achieved / peak, "traffic": None},
        "cpu_baseline": None,
        "kernels": kernels,
    }
    print(json.dumps(result), flush=True)
    return 0


def bench_epilogue(args, w, torch, ap, wl, dev) -> int:
    """The attention-epilogue producer alone (oproj_inv_rope_quant_f32: inverse
    RoPE + FP8 quantisation from fp32 attention output), timed like the path."""
    if w.prequantised:
        log("the pre-quantised workload has no attention output")
        return 2
    T, H, G = w.T, w.H, w.n_groups
    log(f"epilogue producer, workload {w.name}: T={T} H={H} G={G} D={w.D}")
    x = wl.normal_f32_bulk(wl.seed_of(900, 1), T * H * 512).reshape(T, H, 512)
    pos, tab = wl.positions(w), wl.table(w)
    copies = args.copies or max(2, min(16, int(np.ceil(768e6 / x.nbytes))))
    log(f"{copies} rotating copies of {x.nbytes / 1e6:.1f} MB")
    shp = ap.Shape(T=T, n_groups=G, heads_per_group=w.heads_per_group, o_lora_rank=w.o_lora_rank,
                   max_pos=w.max_pos)
    d_pos = torch.from_numpy(pos).to(dev)
    d_tab = torch.from_numpy(tab).to(dev)
    C = []
    for _ in range(copies):
        C.append({"x": torch.from_numpy(x).to(dev),
                  "codes": torch.empty((G, T, w.D), dtype=torch.uint8, device=dev),
                  "scales": torch.empty((G, w.KB, T), dtype=torch.float32, device=dev)})
    del x
    torch.cuda.synchronize()

    def run(c):
        ap.oproj_inv_rope_quant_f32(shp, 0, c["x"], d_pos, d_tab, c["codes"], c["scales"])

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in C:
            run(c)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for c in C:
            run(c)
    torch.cuda.synchronize()
    reps = max(1, args.steps // copies)
    K = reps * copies
    for _ in range(max(1, args.warmup // copies)):
        g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    ms_host = (time.perf_counter() - t0) * 1e3 / K
    us = a.elapsed_time(b) * 1e3 / K
    nb = T * H * 512 * 4 + T * G * w.D + T * G * w.KB * 4 + T * 8 + T * 64 * 4
    log(f"{K} launches: {ms_host * 1e3:.2f} us each (host clock), {us:.2f} us (events)")
    result = {
        "metric": "tokens/s of the attention-epilogue producer (fp32 in: inverse RoPE + FP8 quant)",
        "value": T / (ms_host * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": max(1, args.warmup // copies) * copies, "ms_per_step": ms_host,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32->fp8e4m3",
        "data": "synthetic (seeded SplitMix64 normals)",
        "config": {"workload": f"{w.name} epilogue producer: T={T} heads={H} n_groups={G} D={w.D}",
                   "global_batch": T, "parallelism": "single GPU", "copies_rotated": copies},
        "device": device_info(),
        "roofline": {"bound": "hbm", "kernel": "inv_rope_quant_f32", "achieved": nb / (us * 1e3),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": nb / (us * 1e3) / HBM_PEAK_GBS,
                     "traffic": None},
        "cpu_baseline": None,
        "kernels": {"inv_rope_quant_f32": {"us": us, "bound": "hbm", "bytes": nb, "GB/s": nb / (us * 1e3)}},
    }
    print(json.dumps(result), flush=True)
    return 0


def main() -> int:
    ap_ = argparse.ArgumentParser()
    ap_.add_argument("--gpus", type=int, default=1)
    ap_.add_argument("--steps", type=int, default=2000)
    ap_.add_argument("--warmup", type=int, default=200)
    ap_.add_argument("--workload", default="decode", choices=["decode", "prefill", "pow2", "full", "tiny"])
    ap_.add_argument("--copies", type=int, default=0, help="input/weight copies rotated (0: auto)")
    ap_.add_argument("--kernel-reps", type=int, default=50, help="graph replays per kernel timing")
    ap_.add_argument("--pct-reps", type=int, default=50,
                     help="individually timed graph replays for the p10/p50/p90 figures")
    ap_.add_argument("--cpu-tokens", type=int, default=64, help="oracle sample size (tokens)")
    ap_.add_argument("--no-cpu-baseline", action="store_true")
    ap_.add_argument("--path", default="fp8", choices=["fp8", "bf16", "one-launch", "epilogue"],
                     help="fp8: the quantised path (default); bf16: the unquantised variant; one-launch: "
                          "the quantised path as one kernel (oproj_fused_decode; decode-sized batches); "
                          "epilogue: the fp32-input producer oproj_inv_rope_quant_f32 alone")
    ap_.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                     help="only run plain device copies of MIB MiB (HBM counter calibration) and exit")
    args = ap_.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards over tokens or groups, see the design notes).", file=sys.stderr)
        return 2

    import torch

    import attention_output_projection_amd as ap
    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        return copy_calibration(torch, dev, args.copy_calibration)
    ap.load_library()
    w = wl.WORKLOADS[args.workload]
    if args.path == "bf16":
        return bench_bf16(args, w, torch, ap, wl, dev)
    if args.path == "epilogue":
        return bench_epilogue(args, w, torch, ap, wl, dev)
    log(f"workload {w.name}: T={w.T} G={w.n_groups} hpg={w.heads_per_group} D={w.D} R={w.o_lora_rank}")
    one_launch = args.path == "one-launch"
    if one_launch and (w.T > 64 or w.hidden):
        print("--path one-launch takes a decode-sized workload without wo_b (T <= 64)", file=sys.stderr)
        return 2

    # ---------------------------------------------------------------- inputs
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    wmat = wl.wo_a_f32(w)
    wob = wl.wo_b_bf16(w) if w.hidden else None
    per_copy = w.n_groups * w.o_lora_rank * w.D + o.nbytes + (wob.nbytes if wob is not None else 0)
    copies = args.copies or max(2, min(16, int(np.ceil(768e6 / per_copy))))
    log(f"{copies} rotating copies of {per_copy / 1e6:.1f} MB")

    shp = ap.Shape(T=w.T, n_groups=w.n_groups, heads_per_group=w.heads_per_group,
                   o_lora_rank=w.o_lora_rank, max_pos=w.max_pos)
    mode = ap.OPROJ_SCALE_POW2 if w.pow2 else ap.OPROJ_SCALE_FP32
    wblock = ap.OPROJ_WBLOCK_1x128 if w.w_block_rows == 1 else ap.OPROJ_WBLOCK_128x128
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    d_tab = t(tab)
    d_pos = t(pos)
    d_w32 = t(wmat)
    wrows = w.n_groups * w.o_lora_rank
    srows = wrows if w.w_block_rows == 1 else (wrows + 127) // 128
    hidden = w.hidden if wob is not None else 0
    ws_bytes = ap.oproj_fused_workspace_bytes(shp, hidden)
    C = []
    for i in range(copies):
        c = {}
        c["o"] = t(o.view(np.int16))
        c["wq"] = torch.empty((wrows, w.D), dtype=torch.uint8, device=dev)
        c["ws"] = torch.empty((srows, w.KB), dtype=torch.float32, device=dev)
        ap.oproj_quantize_weight(wrows, w.D, wblock, mode, d_w32, c["wq"], c["ws"])
        c["codes"] = torch.empty((w.n_groups, w.T, w.D), dtype=torch.uint8, device=dev)
        c["scales"] = torch.empty((w.n_groups, w.KB, w.T), dtype=torch.float32, device=dev)
        c["z"] = torch.empty((w.T, w.n_groups, w.o_lora_rank), dtype=torch.int16, device=dev)
        if wob is not None:
            c["wob"] = t(wob.view(np.int16))
            c["y"] = torch.empty((w.T, w.hidden), dtype=torch.int16, device=dev)
        c["work"] = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        C.append(c)
    del d_w32
    torch.cuda.synchronize()

    def quant(c):
        ap.oproj_inv_rope_quant(shp, mode, c["o"], d_pos, d_tab, c["codes"], c["scales"])

    def gemm(c):
        ap.oproj_grouped_wo_a(shp, mode, c["codes"], c["scales"], None, c["wq"], c["ws"], wblock, c["z"])

    def wo_b(c):
        ap.oproj_dense_bf16_gemm(w.T, w.hidden, wrows, c["z"], c["wob"], c["y"])

    def step(c):  # the whole path: one oproj_fused (or oproj_fused_decode) call
        if one_launch:
            ap.oproj_fused_decode(shp, mode, c["o"], d_pos, d_tab, c["wq"], c["ws"], wblock, c["work"],
                                  ws_bytes, c["z"])
            return
        out = c["y"] if wob is not None else c["z"]
        ap.oproj_fused(shp, mode, c["o"], d_pos, d_tab, c["wq"], c["ws"], wblock,
                       c.get("wob"), hidden, c["work"], ws_bytes, out)

    # eager reference result of copy 0
    step(C[0])
    torch.cuda.synchronize()
    eager_out = (C[0]["y"] if wob is not None else C[0]["z"]).clone()

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for c in C:  # one eager pass on the capture stream first
                fn(c)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for c in C:
                fn(c)
        torch.cuda.synchronize()
        return g

    g_step = capture(step)
    g_quant = capture(quant)
    g_gemm = capture(gemm)
    g_wob = capture(wo_b) if wob is not None else None

    # replays must reproduce the eager result
    for _ in range(3):
        g_step.replay()
        torch.cuda.synchronize()
        out = C[0]["y"] if wob is not None else C[0]["z"]
        if not torch.equal(out, eager_out):
            log("graph replay differs from the eager result")
            return 1
        step(C[0])  # eager work between replays
        torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed steps
    reps = max(1, args.steps // copies)
    K = reps * copies
    wreps = max(1, args.warmup // copies)
    for _ in range(wreps):
        g_step.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(reps):
        g_step.replay()
    ev1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    ms_per_step_ev = ev0.elapsed_time(ev1) / K
    log(f"{K} steps: {ms_per_step * 1e3:.2f} us/step (host clock), {ms_per_step_ev * 1e3:.2f} us/step (events)")

    # ---------------------------------------------------------------- per-kernel launch times
    def kernel_time_us(g):
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.kernel_reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (args.kernel_reps * copies)

    def percentiles_us(g):
        """p10/p50/p90 of the per-launch time over individually timed replays
        (each replay runs the rotation of `copies` launches)."""
        g.replay()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.pct_reps)]
        for a, b in evs:
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        v = np.array([a.elapsed_time(b) * 1e3 / copies for a, b in evs])
        return [float(np.percentile(v, q)) for q in (10, 50, 90)]

    pct = {"step": percentiles_us(g_step), "inv_rope_quant": percentiles_us(g_quant),
           "grouped_wo_a": percentiles_us(g_gemm)}
    if g_wob is not None:
        pct["wo_b"] = percentiles_us(g_wob)
    log("p10/p50/p90 us: " + ", ".join(f"{k} {a:.2f}/{b:.2f}/{c:.2f}" for k, (a, b, c) in pct.items()))

    t_quant = kernel_time_us(g_quant)
    t_gemm = kernel_time_us(g_gemm)
    t_wob = kernel_time_us(g_wob) if g_wob is not None else None
    log(f"kernel averages: quant {t_quant:.2f} us, grouped gemm {t_gemm:.2f} us"
        + (f", wo_b {t_wob:.2f} us" if t_wob else ""))

    kernels = {
        "inv_rope_quant": {"us": t_quant, "bound": "hbm", "bytes": kernel_bytes_quant(w),
                           "GB/s": kernel_bytes_quant(w) / (t_quant * 1e3)},
        "grouped_wo_a": {"us": t_gemm, "bytes": kernel_bytes_gemm(w), "flops": kernel_flops_gemm(w),
                         "GB/s": kernel_bytes_gemm(w) / (t_gemm * 1e3),
                         "TFLOP/s": kernel_flops_gemm(w) / (t_gemm * 1e6)},
    }
    ai = kernel_flops_gemm(w) / kernel_bytes_gemm(w)
    gemm_bound = "hbm" if ai < FP8_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3 else "mfma"
    kernels["grouped_wo_a"]["bound"] = gemm_bound
    if t_wob is not None:
        fl = 2 * w.T * w.hidden * wrows
        kernels["wo_b"] = {"us": t_wob, "bound": "mfma", "flops": fl, "TFLOP/s": fl / (t_wob * 1e6)}
    if one_launch:
        # the one kernel of the step; its bytes are both steps' (the codes and
        # scales still go through the workspace)
        t_one = kernel_time_us(g_step)
        nb = kernel_bytes_quant(w) + kernel_bytes_gemm(w)
        kernels["fused_decode"] = {"us": t_one, "bound": "hbm", "bytes": nb, "GB/s": nb / (t_one * 1e3)}
        log(f"one-launch kernel: {t_one:.2f} us")

    dominant = "fused_decode" if one_launch else max(kernels, key=lambda k: kernels[k]["us"])
    kd = kernels[dominant]
    sha = source_sha(*KERNEL_SOURCES[dominant])
    if dominant in ("inv_rope_quant", "fused_decode"):
        achieved, peak, unit, bound = kd["GB/s"], HBM_PEAK_GBS, "GB/s", "hbm"
    elif dominant == "grouped_wo_a":
        if gemm_bound == "hbm":
            achieved, peak, unit, bound = kd["GB/s"], HBM_PEAK_GBS, "GB/s", "hbm"
        else:
            achieved, peak, unit, bound = kd["TFLOP/s"], FP8_PEAK_TFLOPS, "TFLOP/s", "mfma"
    else:
        achieved, peak, unit, bound = kd["TFLOP/s"], BF16_PEAK_TFLOPS, "TFLOP/s", "mfma"
    traffic = load_traffic(dominant, w.name, sha)

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on the host ...")
        cpu = cpu_baseline(w, o, pos, tab, wmat, args.cpu_tokens)
        log(f"oracle: {cpu['value']:.1f} tokens/s on {cpu['cores']} threads")

    tokens_per_s = w.T / (ms_per_step * 1e-3)
    gemm_tflops = kernel_flops_gemm(w) / (ms_per_step * 1e9)
    result = {
        "metric": "tokens/s and TFLOP/s of inv-RoPE+FP8 quant+grouped wo_a; % of HBM/FP8 roofline",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": wreps * copies,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3",
        "data": "synthetic (seeded SplitMix64 normals; random-init weights)",
        "config": {"workload": f"{w.name}: T={w.T} n_groups={w.n_groups} heads_per_group={w.heads_per_group} "
                               f"head_dim=512 D={w.D} o_lora_rank={w.o_lora_rank} max_pos={w.max_pos}"
                               + (f" hidden={w.hidden}" if w.hidden else "")
                               + f" scales={'pow2' if w.pow2 else 'fp32'}",
                   "global_batch": w.T, "parallelism": "single GPU",
                   "path": "one kernel (oproj_fused_decode)" if one_launch else "oproj_fused",
                   "step_TFLOP/s": gemm_tflops, "copies_rotated": copies},
        "device": device_info(),
        "roofline": {"bound": bound, "kernel": dominant, "achieved": achieved, "peak": peak, "unit": unit,
                     "frac": achieved / peak, "traffic": traffic},
        "cpu_baseline": cpu,
        "kernels": kernels,
        "p10_p50_p90_us": pct,
    }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

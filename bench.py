"""Benchmark of the O-projection front half on one MI355X.

One step = one pass of the hot path over one batch of synthetic input: one
oproj_fused call -- inverse RoPE + 1x128 FP8 quantisation, then the grouped
wo_a GEMM, plus the dense wo_b GEMM for the workload that has one.  On the
pre-quantised pow2 workload the step is the grouped GEMM alone, reading the
live groups of a [T, 10, D] token-major input whose two padding groups hold
NaN codes and scales.  The default workload is the prefill batch (T=8192,
16 groups x 8 heads, D=4096, R=1024).

Inputs are resident in HBM before timing starts.  The steps rotate through
several copies of the inputs, weights and workspaces (more bytes than the
256 MB last-level cache) so weights are streamed from HBM every step.  Each
copy's step is captured once in a HIP graph; the timed region replays exactly
--steps graphs (after exactly --warmup untimed ones), each bracketed by HIP
events on the stream the kernels run on.  `value` is the batch's tokens over
the median per-step event time.

The kernels are also timed one by one (oproj_inv_rope_quant,
oproj_grouped_wo_a, oproj_dense_bf16_gemm): a graph holding one launch per
copy is replayed between HIP events, giving each kernel's average launch
duration; the roofline of the dominant kernel divides its algorithmic bytes
or FLOPs per launch by that average.  The decode batch (T=64) is measured the
same way and reported under "other_workloads".

Printed: one JSON line with the throughput, the roofline of the dominant
kernel and the oracle's CPU baseline on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import gc
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


def kernel_bytes_wo_b(w) -> int:
    """Algorithmic HBM bytes of a4: bf16 z, bf16 wo_b, bf16 y."""
    K = w.n_groups * w.o_lora_rank
    return (w.T * K + w.hidden * K + w.T * w.hidden) * 2


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


def pcts(v) -> list:
    return [float(np.percentile(v, q)) for q in (10, 50, 90)]


def cpu_baseline(w, o, pos, tab, wmat, wob, max_tokens: int, reps: int = 3):
    """The oracle as it stands, on the first tokens of the same batch, doing
    the work the step does (a1 + a2 + a3, + a4 with wo_b; a3 alone on the
    pre-quantised workload, whose codes the oracle makes untimed); the median
    of `reps` runs."""
    import oracle

    S = min(w.T, max_tokens)
    qw, sw = oracle.quant_weight(wmat, w.w_block_rows, w.pow2)  # offline weight prep, untimed
    threads = oracle.default_threads()
    pre = None
    if w.prequantised:
        pre = oracle.inv_rope_quant(o[:S], pos[:S], tab, w.n_groups, w.heads_per_group, pow2=w.pow2)
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        if pre is None:
            qa, sa = oracle.inv_rope_quant(o[:S], pos[:S], tab, w.n_groups, w.heads_per_group, pow2=w.pow2)
        else:
            qa, sa = pre
        z = oracle.grouped_gemm(qa, sa, qw, sw, w.n_groups, w.o_lora_rank, w.w_block_rows)
        if wob is not None:
            oracle.dense_gemm_bf16(oracle.f64_to_bf16(z).reshape(S, -1), wob)
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    work = ("grouped wo_a on the pre-quantised codes" if pre is not None else
            "inverse RoPE + quant + grouped wo_a" + (" + wo_b" if wob is not None else ""))
    return {"value": S / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {S} of {w.T} tokens of the {w.name} batch: {work}, fp64 accumulation, "
                      f"median of {reps} runs of {dt:.2f} s ({sum(times):.1f} s of CPU work)"}


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


# ---------------------------------------------------------------- graphs and timing
class Graphs:
    """HIP graphs of the benchmark, released explicitly (synchronised first)
    before the process tears the runtime down."""

    def __init__(self, torch):
        self.torch = torch
        self.all = []

    def capture(self, fns):
        """One graph holding fns() in order, after one eager pass on the
        capture stream."""
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for fn in fns:
                fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for fn in fns:
                fn()
        torch.cuda.synchronize()
        self.all.append(g)
        return g

    def release(self):
        self.torch.cuda.synchronize()
        for g in self.all:
            g.reset()
        self.all = []
        self.torch.cuda.synchronize()


def timed_steps(torch, graphs, steps: int, warmup: int):
    """Replay graphs[i % len(graphs)]: exactly `warmup` untimed, then exactly
    `steps` timed, each bracketed by HIP events; synchronised on both sides.
    Returns (per-step us array, host-clock us per step)."""
    n = len(graphs)
    for i in range(warmup):
        graphs[i % n].replay()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for i, (a, b) in enumerate(evs):
        a.record()
        graphs[(warmup + i) % n].replay()
        b.record()
    torch.cuda.synchronize()
    host = (time.perf_counter() - t0) * 1e6 / max(1, steps)
    return np.array([a.elapsed_time(b) * 1e3 for a, b in evs]), host


def launch_average_us(torch, g, launches_per_replay: int, replays: int):
    """Average launch duration of a kernel: a graph of `launches_per_replay`
    back-to-back launches replayed `replays` times back to back between two
    HIP events (after one untimed replay).  Also the per-launch p10/p50/p90
    over `replays` individually timed replays (each one pays its own ramp)."""
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    mean = a.elapsed_time(b) * 1e3 / (replays * launches_per_replay)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(replays)]
    for a, b in evs:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    v = np.array([a.elapsed_time(b) * 1e3 / launches_per_replay for a, b in evs])
    return float(mean), pcts(v)


def roofline_of(kd: dict, bound: str, peak_mfma: float):
    if bound == "hbm":
        return kd["GB/s"], HBM_PEAK_GBS, "GB/s"
    return kd["TFLOP/s"], peak_mfma, "TFLOP/s"


# ---------------------------------------------------------------- the quantised path
def run_fp8(args, w, torch, ap, wl, dev, steps: int, warmup: int, one_launch: bool = False,
            want_cpu: bool = True) -> dict:
    """Set up, check and time the quantised path on workload w; returns the
    result record (value = tokens per second from the median step time)."""
    log(f"workload {w.name}: T={w.T} G={w.n_groups} hpg={w.heads_per_group} D={w.D} R={w.o_lora_rank}"
        + (" (pre-quantised [T, %d, D] input)" % (w.n_groups + w.pad_groups) if w.prequantised else ""))
    o, pos, tab = wl.attn_out(w), wl.positions(w), wl.table(w)
    wmat = wl.wo_a_f32(w)
    wob = wl.wo_b_bf16(w) if w.hidden else None
    Gp = w.n_groups + w.pad_groups
    act_bytes = w.T * Gp * w.D if w.prequantised else o.nbytes
    per_copy = w.n_groups * w.o_lora_rank * w.D + act_bytes + (wob.nbytes if wob is not None else 0)
    copies = args.copies or max(2, min(16, int(np.ceil(768e6 / per_copy))))
    log(f"{copies} rotating copies of {per_copy / 1e6:.1f} MB")

    shp = ap.Shape(T=w.T, n_groups=w.n_groups, heads_per_group=w.heads_per_group,
                   o_lora_rank=w.o_lora_rank, max_pos=w.max_pos)
    mode = ap.OPROJ_SCALE_POW2 if w.pow2 else ap.OPROJ_SCALE_FP32
    wblock = ap.OPROJ_WBLOCK_1x128 if w.w_block_rows == 1 else ap.OPROJ_WBLOCK_128x128
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    d_tab, d_pos, d_w32 = t(tab), t(pos), t(wmat)
    wrows = w.n_groups * w.o_lora_rank
    srows = wrows if w.w_block_rows == 1 else (wrows + 127) // 128
    hidden = w.hidden if wob is not None else 0
    ws_bytes = ap.oproj_fused_workspace_bytes(shp, hidden)
    if one_launch:  # the codes and scales, then the groups' barrier words (zeroed once below)
        ws_bytes = ap.oproj_fused_decode_workspace_bytes(shp)
    # the padded token-major layout of a pre-quantised input: [T, Gp, D] codes, [T, Gp, KB] scales
    pad_lay = ap.ActLayout(Gp * w.D, w.D, Gp * w.KB, w.KB, 1) if w.prequantised else None
    C = []
    for _ in range(copies):
        c = {"wq": torch.empty((wrows, w.D), dtype=torch.uint8, device=dev),
             "ws": torch.empty((srows, w.KB), dtype=torch.float32, device=dev),
             "z": torch.empty((w.T, w.n_groups, w.o_lora_rank), dtype=torch.int16, device=dev)}
        ap.oproj_quantize_weight(wrows, w.D, wblock, mode, d_w32, c["wq"], c["ws"])
        if w.prequantised:
            # untimed input preparation: the live groups quantised on the GPU
            # into the padded layout, the padding groups NaN (code 0x7F)
            d_o = t(o.view(np.int16))
            c["codes"] = torch.full((w.T, Gp, w.D), 0x7F, dtype=torch.uint8, device=dev)
            c["scales"] = torch.full((w.T, Gp, w.KB), float("nan"), dtype=torch.float32, device=dev)
            ap.oproj_inv_rope_quant(shp, mode, d_o, d_pos, d_tab, c["codes"], c["scales"], pad_lay)
            del d_o
        else:
            c["o"] = t(o.view(np.int16))
            c["codes"] = torch.empty((w.n_groups, w.T, w.D), dtype=torch.uint8, device=dev)
            c["scales"] = torch.empty((w.n_groups, w.KB, w.T), dtype=torch.float32, device=dev)
            c["work"] = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
        if wob is not None:
            c["wob"] = t(wob.view(np.int16))
            c["y"] = torch.empty((w.T, w.hidden), dtype=torch.int16, device=dev)
        C.append(c)
    del d_w32
    torch.cuda.synchronize()

    def quant(c):
        ap.oproj_inv_rope_quant(shp, mode, c["o"], d_pos, d_tab, c["codes"], c["scales"])

    def gemm(c):
        ap.oproj_grouped_wo_a(shp, mode, c["codes"], c["scales"], pad_lay, c["wq"], c["ws"], wblock, c["z"])

    def wo_b(c):
        ap.oproj_dense_bf16_gemm(w.T, w.hidden, wrows, c["z"], c["wob"], c["y"])

    def step(c):  # the whole path: one oproj_fused (or oproj_fused_decode) call
        if w.prequantised:
            gemm(c)
        elif one_launch:
            ap.oproj_fused_decode(shp, mode, c["o"], d_pos, d_tab, c["wq"], c["ws"], wblock, c["work"],
                                  ws_bytes, c["z"])
        else:
            out = c["y"] if wob is not None else c["z"]
            ap.oproj_fused(shp, mode, c["o"], d_pos, d_tab, c["wq"], c["ws"], wblock,
                           c.get("wob"), hidden, c["work"], ws_bytes, out)

    out_of = lambda c: c["y"] if wob is not None else c["z"]
    step(C[0])
    torch.cuda.synchronize()
    eager_out = out_of(C[0]).clone()

    G = Graphs(torch)
    try:
        g_steps = [G.capture([lambda c=c: step(c)]) for c in C]
        g_gemm = G.capture([lambda c=c: gemm(c) for c in C])
        g_quant = None if w.prequantised else G.capture([lambda c=c: quant(c) for c in C])
        g_wob = G.capture([lambda c=c: wo_b(c) for c in C]) if wob is not None else None

        # replays must reproduce the eager result (eager work between replays)
        for _ in range(3):
            g_steps[0].replay()
            torch.cuda.synchronize()
            if not torch.equal(out_of(C[0]), eager_out):
                raise RuntimeError("graph replay differs from the eager result")
            step(C[0])
            torch.cuda.synchronize()

        # ------------------------------------------------------------ timed steps
        st_us, host_us = timed_steps(torch, g_steps, steps, warmup)
        med = float(np.median(st_us))
        log(f"{steps} steps after {warmup} warm-up: median {med:.2f} us/step by events "
            f"(p10/p90 {np.percentile(st_us, 10):.2f}/{np.percentile(st_us, 90):.2f}), "
            f"{host_us:.2f} us/step by host clock")

        # ------------------------------------------------------------ per-kernel launch times
        reps = max(args.kernel_reps, 1)
        kernels = {}
        pct = {"step": pcts(st_us)}
        # the steps back to back (one graph of the whole rotation): what a
        # stream of batches sustains when the host keeps ahead of the GPU
        g_rot = G.capture([lambda c=c: step(c) for c in C])
        rot_us, _ = launch_average_us(torch, g_rot, copies, reps)
        log(f"steps back to back: {rot_us:.2f} us/step")
        gemm_bound = "hbm" if kernel_flops_gemm(w) / kernel_bytes_gemm(w) < \
            FP8_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3 else "mfma"
        t_gemm, pct["grouped_wo_a"] = launch_average_us(torch, g_gemm, copies, reps)
        kernels["grouped_wo_a"] = {"us": t_gemm, "bound": gemm_bound, "bytes": kernel_bytes_gemm(w),
                                   "flops": kernel_flops_gemm(w),
                                   "GB/s": kernel_bytes_gemm(w) / (t_gemm * 1e3),
                                   "TFLOP/s": kernel_flops_gemm(w) / (t_gemm * 1e6)}
        if g_quant is not None:
            t_quant, pct["inv_rope_quant"] = launch_average_us(torch, g_quant, copies, reps)
            kernels["inv_rope_quant"] = {"us": t_quant, "bound": "hbm", "bytes": kernel_bytes_quant(w),
                                         "GB/s": kernel_bytes_quant(w) / (t_quant * 1e3)}
        if g_wob is not None:
            t_wob, pct["wo_b"] = launch_average_us(torch, g_wob, copies, reps)
            fl = 2 * w.T * w.hidden * wrows
            kernels["wo_b"] = {"us": t_wob, "bound": "mfma", "flops": fl, "bytes": kernel_bytes_wo_b(w),
                               "TFLOP/s": fl / (t_wob * 1e6), "GB/s": kernel_bytes_wo_b(w) / (t_wob * 1e3)}
        if one_launch:
            # the one kernel of the step; its bytes are both steps' (the codes
            # and scales still go through the workspace)
            t_one, pct["fused_decode"] = rot_us, pcts(st_us)
            nb = kernel_bytes_quant(w) + kernel_bytes_gemm(w)
            kernels["fused_decode"] = {"us": t_one, "bound": "hbm", "bytes": nb, "GB/s": nb / (t_one * 1e3)}
        log("kernel averages: " + ", ".join(f"{k} {v['us']:.2f} us" for k, v in kernels.items()))
    finally:
        G.release()

    dominant = "fused_decode" if one_launch else max(kernels, key=lambda k: kernels[k]["us"])
    kd = kernels[dominant]
    peak_mfma = BF16_PEAK_TFLOPS if dominant == "wo_b" else FP8_PEAK_TFLOPS
    achieved, peak, unit = roofline_of(kd, kd["bound"], peak_mfma)
    traffic = load_traffic(dominant, w.name, source_sha(*KERNEL_SOURCES[dominant]))

    cpu = None
    if want_cpu and not args.no_cpu_baseline:
        log("timing the oracle on the host ...")
        cpu = cpu_baseline(w, o, pos, tab, wmat, wob, args.cpu_tokens)
        log(f"oracle: {cpu['value']:.1f} tokens/s on {cpu['cores']} threads")

    step_desc = ("oproj_grouped_wo_a on the padded pre-quantised input" if w.prequantised else
                 "one kernel (oproj_fused_decode)" if one_launch else "oproj_fused")
    return {
        "metric": "tokens/s and TFLOP/s of inv-RoPE+FP8 quant+grouped wo_a; % of HBM/FP8 roofline",
        "value": w.T / (med * 1e-6),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": med * 1e-3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3",
        "data": "synthetic (seeded SplitMix64 normals; random-init weights)",
        "config": {"workload": f"{w.name}: T={w.T} n_groups={w.n_groups} heads_per_group={w.heads_per_group} "
                               f"head_dim=512 D={w.D} o_lora_rank={w.o_lora_rank} max_pos={w.max_pos}"
                               + (f" hidden={w.hidden}" if w.hidden else "")
                               + (f" input=[T,{Gp},D] pre-quantised" if w.prequantised else "")
                               + f" scales={'pow2' if w.pow2 else 'fp32'}"
                               + f" weight_blocks={'1x128' if w.w_block_rows == 1 else '128x128'}",
                   "global_batch": w.T, "parallelism": "single GPU", "path": step_desc,
                   "step_TFLOP/s": kernel_flops_gemm(w) / (med * 1e6), "copies_rotated": copies,
                   "host_clock_us_per_step": host_us, "back_to_back_us_per_step": rot_us},
        "roofline": {"bound": kd["bound"], "kernel": dominant, "achieved": achieved, "peak": peak, "unit": unit,
                     "frac": achieved / peak, "traffic": traffic},
        "cpu_baseline": cpu,
        "kernels": kernels,
        "p10_p50_p90_us": pct,
    }


# ---------------------------------------------------------------- other paths
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

    step(C[0])
    torch.cuda.synchronize()
    eager = C[0]["z"].clone()
    G = Graphs(torch)
    try:
        g_steps = [G.capture([lambda c=c: step(c)]) for c in C]
        g_rope = G.capture([lambda c=c: rope(c) for c in C])
        g_gemm = G.capture([lambda c=c: gemm(c) for c in C])
        g_steps[0].replay()
        torch.cuda.synchronize()
        if not torch.equal(C[0]["z"], eager):
            log("graph replay differs from the eager result")
            return 1
        st_us, host_us = timed_steps(torch, g_steps, args.steps, args.warmup)
        med = float(np.median(st_us))
        t_rope, _ = launch_average_us(torch, g_rope, copies, args.kernel_reps)
        t_gemm, _ = launch_average_us(torch, g_gemm, copies, args.kernel_reps)
    finally:
        G.release()
    log(f"{args.steps} steps: median {med:.2f} us/step; kernel averages: rope {t_rope:.2f} us, "
        f"grouped bf16 gemm {t_gemm:.2f} us")
    Gn, R, D, T = w.n_groups, w.o_lora_rank, w.D, w.T
    rope_bytes = 2 * T * w.H * 512 * 2 + T * 8 + T * 64 * 4
    gemm_bytes = Gn * R * D * 2 + T * Gn * D * 2 + T * Gn * R * 2
    gemm_flops = 2 * T * Gn * R * D
    hbm_bound = gemm_flops / gemm_bytes < BF16_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3
    kernels = {"inv_rope_bf16": {"us": t_rope, "bound": "hbm", "bytes": rope_bytes,
                                 "GB/s": rope_bytes / (t_rope * 1e3)},
               "grouped_wo_a_bf16": {"us": t_gemm, "bound": "hbm" if hbm_bound else "mfma",
                                     "bytes": gemm_bytes, "flops": gemm_flops,
                                     "GB/s": gemm_bytes / (t_gemm * 1e3), "TFLOP/s": gemm_flops / (t_gemm * 1e6)}}
    dom = max(kernels, key=lambda k: kernels[k]["us"])
    kd = kernels[dom]
    achieved, peak, unit = roofline_of(kd, kd["bound"], BF16_PEAK_TFLOPS)
    result = {
        "metric": "tokens/s of the unquantised path (bf16 inverse RoPE + grouped bf16 wo_a)",
        "value": T / (med * 1e-6), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": med * 1e-3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64 normals; random-init weights)",
        "config": {"workload": f"{w.name} unquantised: T={T} n_groups={Gn} heads_per_group={w.heads_per_group} "
                               f"D={D} o_lora_rank={R}", "global_batch": T, "parallelism": "single GPU",
                   "copies_rotated": copies, "host_clock_us_per_step": host_us},
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
    T, H, Gn = w.T, w.H, w.n_groups
    log(f"epilogue producer, workload {w.name}: T={T} H={H} G={Gn} D={w.D}")
    x = wl.normal_f32_bulk(wl.seed_of(900, 1), T * H * 512).reshape(T, H, 512)
    pos, tab = wl.positions(w), wl.table(w)
    copies = args.copies or max(2, min(16, int(np.ceil(768e6 / x.nbytes))))
    log(f"{copies} rotating copies of {x.nbytes / 1e6:.1f} MB")
    shp = ap.Shape(T=T, n_groups=Gn, heads_per_group=w.heads_per_group, o_lora_rank=w.o_lora_rank,
                   max_pos=w.max_pos)
    d_pos = torch.from_numpy(pos).to(dev)
    d_tab = torch.from_numpy(tab).to(dev)
    C = []
    for _ in range(copies):
        C.append({"x": torch.from_numpy(x).to(dev),
                  "codes": torch.empty((Gn, T, w.D), dtype=torch.uint8, device=dev),
                  "scales": torch.empty((Gn, w.KB, T), dtype=torch.float32, device=dev)})
    del x
    torch.cuda.synchronize()

    def run(c):
        ap.oproj_inv_rope_quant_f32(shp, 0, c["x"], d_pos, d_tab, c["codes"], c["scales"])

    G = Graphs(torch)
    try:
        g_steps = [G.capture([lambda c=c: run(c)]) for c in C]
        g_all = G.capture([lambda c=c: run(c) for c in C])
        st_us, host_us = timed_steps(torch, g_steps, args.steps, args.warmup)
        us, _ = launch_average_us(torch, g_all, copies, args.kernel_reps)
    finally:
        G.release()
    med = float(np.median(st_us))
    nb = T * H * 512 * 4 + T * Gn * w.D + T * Gn * w.KB * 4 + T * 8 + T * 64 * 4
    log(f"{args.steps} launches: median {med:.2f} us each, launch average {us:.2f} us (events)")
    result = {
        "metric": "tokens/s of the attention-epilogue producer (fp32 in: inverse RoPE + FP8 quant)",
        "value": T / (med * 1e-6), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": med * 1e-3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32->fp8e4m3",
        "data": "synthetic (seeded SplitMix64 normals)",
        "config": {"workload": f"{w.name} epilogue producer: T={T} heads={H} n_groups={Gn} D={w.D}",
                   "global_batch": T, "parallelism": "single GPU", "copies_rotated": copies,
                   "host_clock_us_per_step": host_us},
        "device": device_info(),
        "roofline": {"bound": "hbm", "kernel": "inv_rope_quant_f32", "achieved": nb / (us * 1e3),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": nb / (us * 1e3) / HBM_PEAK_GBS,
                     "traffic": None},
        "cpu_baseline": None,
        "kernels": {"inv_rope_quant_f32": {"us": us, "bound": "hbm", "bytes": nb, "GB/s": nb / (us * 1e3)}},
    }
    print(json.dumps(result), flush=True)
    return 0


def summary(r: dict) -> dict:
    """The figures of a secondary workload kept in the headline line."""
    return {"config": r["config"]["workload"], "value": r["value"], "unit": r["unit"],
            "ms_per_step": r["ms_per_step"],
            "back_to_back_us_per_step": r["config"]["back_to_back_us_per_step"],
            "roofline": r["roofline"], "kernels": r["kernels"],
            "p10_p50_p90_us": r["p10_p50_p90_us"]}


def main() -> int:
    ap_ = argparse.ArgumentParser()
    ap_.add_argument("--gpus", type=int, default=1)
    ap_.add_argument("--steps", type=int, default=50, help="timed steps (exactly this many)")
    ap_.add_argument("--warmup", type=int, default=5, help="untimed steps before them (exactly this many)")
    ap_.add_argument("--workload", default="prefill", choices=["decode", "prefill", "pow2", "full", "tiny"])
    ap_.add_argument("--also", default="decode",
                     help="comma-separated extra workloads measured after the headline one and reported "
                          "under other_workloads ('' for none)")
    ap_.add_argument("--copies", type=int, default=0, help="input/weight copies rotated (0: auto)")
    ap_.add_argument("--kernel-reps", type=int, default=50, help="graph replays per kernel timing")
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
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
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
    one_launch = args.path == "one-launch"
    if one_launch and (w.T > 64 or w.hidden or w.prequantised):
        print("--path one-launch takes a decode-sized workload without wo_b (T <= 64)", file=sys.stderr)
        return 2

    result = run_fp8(args, w, torch, ap, wl, dev, args.steps, args.warmup, one_launch=one_launch)
    result["device"] = device_info()
    others = {}
    for name in [s for s in args.also.split(",") if s and s != w.name and not one_launch]:
        # each workload starts from a released allocator cache, as in a process of its own: decode
        # buffers carved out of the prefill run's cached gigabyte segments measured ~1.4 us slower
        # per GEMM than freshly allocated ones (16.3 vs 17.8 us, same box, same kernel)
        gc.collect()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        r = run_fp8(args, wl.WORKLOADS[name], torch, ap, wl, dev, max(args.steps, 50), max(args.warmup, 5),
                    want_cpu=False)
        others[name] = summary(r)
    if others:
        result["other_workloads"] = others
    print(json.dumps(result), flush=True)
    torch.cuda.synchronize()
    return 0


if __name__ == "__main__":
    sys.exit(main())

#!/usr/bin/env python3
"""Benchmark of the dynamically quantized int8 linear layer on one MI355X.

One step = one pass of the whole layer over one batch of synthetic input:
w8a8_quantize_rows (per-row absmax/127 int8 quantization of X) followed by
w8a8_gemm (int8 MFMA GEMM with the fused dequant -> bf16 epilogue), on the
M=2048, K=N=4096 workload with 1% outlier channels. `value` is the effective
int8 rate of the step, 2*M*N*K / step time.

The line also carries:
  roofline     the GEMM kernel alone (the dominant kernel): algorithmic int8
               ops per launch / average launch time, against the int8 dense
               MFMA peak; traffic from the committed rocprofv3 PMC record when
               it was taken on the current kernel source, else null;
  cpu_baseline the CPU oracle timed on this host on a bounded sample (threads,
               CPU model), and its `parity`: the oracle's rows of that sample
               against the timed path's output for the same inputs (Xq and sx
               bit for bit, bf16 ulps);
  library_int_mm  the vendor library's int8 GEMM (torch._int_mm, hipBLASLt,
               int32 out, no dequant) on the same inputs, for dense M > 16;
  decode_m16   the M=16 weight-streaming path (K=N=4096): GB/s of the GEMM
               kernel against HBM peak, with rotated weight copies so the
               256 MB Infinity Cache cannot serve them; the two-launch layer
               (quantize + GEMM) and the single-launch w8a8_fused_linear, both
               priced at the layer's bytes (X bf16 + Wq + sw + out).

  peaks        reference rates measured on the same GPU in the same run
               (libpeaks.so): the int8 MFMA issue rate of back-to-back
               v_mfma_i32_32x32x32_i8 (and the bf16 rate of
               v_mfma_f32_32x32x16_bf16) with the shader clock it ran at
               (s_memtime against the 100 MHz reference), HBM streaming read
               and write rates over 1 GiB, and the time to stream-read 16.8 MB
               (the M=16 weight matrix) with the buffers rotated past the
               Infinity Cache, grid-stride and in the M-small GEMM's own
               row-slice pattern (decode_m16.vs_measured_read_floor takes the
               faster of the two), and the prefill GEMM's operand stream alone
               (its tiles, tile order, direct-to-LDS ring and barriers, no
               arithmetic) over operand sets rotated past the Infinity Cache
               (roofline.operand_stream_us and frac_of_operand_stream on the
               prefill line), and over one set that stays in the cache.
               roofline.frac_measured is the kernel's rate
               against these (for HBM-bound kernels: the time its read and
               write bytes take at the measured rates, over its time);
  clocks       amd-smi's gfx and memory clocks sampled while the step's HIP
               graph replays for about two seconds, and at idle.

Inputs are resident in HBM before the timed region; input sets are rotated
(copies at distinct addresses, more than twice the Infinity Cache in total).
Launches are captured into HIP graphs and replayed, so the timing is the GPU's
and not the Python binding's per-call host overhead. ms_per_step is one timed
region of exactly --steps steps; the kernel-alone figures (gemm_only, the
roofline's avg_launch_us, quantize_rows) are the median of five regions of
--steps calls each. Other workloads: --config (the roofline is HBM-bound for
the BSR kernel and for M <= 64); --config w4a16 / w4a16_decode time the W4A16
fused dequant GEMM (bf16 TFLOP/s) with the pages' M = 16 .. 1024 sweep.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective int8 TOPS (+% of MFMA peak) at M=2048,K=N=4096; GB/s at M=16"
PEAK_INT8_TOPS = 5000.0     # MI355X dense int8 MFMA, TOP/s
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, GB/s
MALL_BYTES = 256 << 20      # Infinity Cache
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "gemm_tiled_prefill_traffic.json")
GEMM_SOURCES = ["gemm_tiled.hip", "common.hpp"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default="prefill_outliers",
                    choices=["tiny", "decode", "prefill_outliers", "large_m", "bsr", "bsr_fc2",
                             "sparse24", "sparse24_decode", "w4a16", "w4a16_decode"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="launch every timed call directly instead of replaying HIP graphs "
                         "(for profilers that count per dispatch)")
    ap.add_argument("--peaks", action="store_true",
                    help="only measure the on-device reference rates (libpeaks.so) and exit")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the reference rates and the clock sampling")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy five times (the "
                         "reference for scaling HBM byte counters) and exit")
    return ap.parse_args()


def source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "quantized_gemm_quantize_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def rotation(bytes_per_set: int) -> int:
    """Copies needed for the rotated sets to exceed twice the Infinity Cache (at most 256:
    sets of a few kilobytes cannot leave the caches anyway)."""
    return min(256, max(2, -(-2 * MALL_BYTES // max(bytes_per_set, 1)) + 1))


def time_loop(fn, n: int, torch, period: int = 1, eager: bool = False) -> float:
    """Average ms per call of fn(i) over exactly n calls, replayed from HIP graphs.

    The calls are captured into a graph of `period` consecutive calls (one per
    rotated input set) plus one graph of n % period calls, so the timed region
    holds exactly n calls and the GPU runs them back to back without waiting on
    Python (an eager call costs several microseconds of host time). HIP events
    bracket the replays on the stream they run on; the region is bracketed by
    device synchronization on both sides. With eager=True the n calls are
    launched directly (host launch overhead included).
    """
    if eager:
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(n):
            fn(i)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / n

    def capture(count):
        if count == 0:
            return None
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(count):
                fn(i)
        return g
    full, rest = capture(period), capture(n % period)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(n // period):
        full.replay()
    if rest is not None:
        rest.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / n


def time_median(fn, n: int, torch, period: int, eager: bool, repeats: int = 5) -> float:
    """Median over `repeats` timed regions of time_loop (each of exactly n calls): a single
    region of a few milliseconds catches the GPU's clock changes."""
    runs = sorted(time_loop(fn, n, torch, period=period, eager=eager) for _ in range(repeats))
    return runs[len(runs) // 2]


def prepare(name: str, torch, np, b, dev):
    """Device-resident inputs for one workload (weights quantized by the library)."""
    from quantized_gemm_quantize_amd.inputs import bsr_from_dense, make_inputs
    inp = make_inputs(name, seed=0)
    x = torch.from_numpy(inp.x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    wq, sw = b.w8a8_quantize_rows_f32(torch.from_numpy(inp.w).to(dev))
    d = dict(inp=inp, x=x, wq=wq, sw=sw)
    if inp.meta.get("sparse24"):
        d["values24"], d["meta24"] = b.w8a8_compress24(wq)
    if inp.bs:
        crow, col, values = bsr_from_dense(wq.cpu().numpy(), inp.block_mask, inp.bs)
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        d.update(crow=t(crow), col=t(col), values=t(values))
    return d


def cpu_model() -> str:
    """The host CPU's model name (first `model name` line of /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def bf16_ulps(a, b, np):
    """Distance in bf16 ulps between two arrays of bf16 bit patterns (sign-magnitude mapped
    to ordered integers; +0 and -0 coincide)."""
    def ordered(u):
        u = u.astype(np.int32) & 0xFFFF
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(ordered(a) - ordered(b))


def cpu_baseline(name: str, np, gpu_rows=None):
    """The CPU oracle (untuned) on a bounded sample of the same workload. gpu_rows(r), when
    given, returns the timed path's Xq, sx and bf16 output bits for rows 0..r-1 of the same
    inputs: the oracle's rows are then compared with them (the `parity` entry)."""
    import oracle
    from quantized_gemm_quantize_amd.inputs import bsr_from_dense, make_inputs
    inp = make_inputs(name, seed=0)
    wq, sw = oracle.quantize_rows_f32(inp.w)
    M, N, K = inp.M, inp.N, inp.K
    bsr = bsr_from_dense(wq, inp.block_mask, inp.bs) if inp.bs else None

    sparse24 = oracle.compress24(wq) if inp.meta.get("sparse24") else None

    def run(rows):
        t0 = time.perf_counter()
        xq, sx = oracle.quantize_rows_bf16(inp.x_bits[:rows])
        if sparse24 is not None:
            acc = oracle.gemm_i32(xq, oracle.decompress24(*sparse24))
        elif bsr is None:
            acc = oracle.gemm_i32(xq, wq)
        else:
            acc = oracle.bsr_gemm_i32(xq, *bsr, N)
        out = oracle.epilogue_bf16(acc, sx, sw)
        return time.perf_counter() - t0, xq, sx, out

    probe = min(M, 64)
    t_probe = run(probe)[0]
    rows = int(min(M, max(probe, probe * 15.0 / max(t_probe, 1e-6))))
    t, xq, sx, out = run(rows)
    ops = 2.0 * rows * N * K
    if sparse24 is not None:
        ops /= 2          # the kept products only, as the GPU line counts them
    parity = None
    if gpu_rows is not None:
        g_xq, g_sx, g_out = gpu_rows(rows)
        ulps = bf16_ulps(g_out, out, np)
        parity = {"rows": rows, "xq_bit_exact": bool(np.array_equal(g_xq, xq)),
                  "sx_bit_exact": bool(np.array_equal(g_sx.view(np.uint32), sx.view(np.uint32))),
                  "max_ulp": int(ulps.max()), "frac_beyond_1ulp": float((ulps > 1).mean()),
                  "bar": "Xq and sx bit-exact, bf16 within 1 ulp"}
    return {"value": round(ops / t / 1e12, 6), "unit": "TOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"rows 0..{rows - 1} of the {name} workload (M={M}, N={N}, K={K}): "
                      f"quantize + exact int GEMM + float64 epilogue"
                      + (" (2:4 weight decompressed inside the timed region)" if sparse24 else "")
                      + f", {t:.2f} s wall", "parity": parity}


MFMA_RECORD = os.path.join(ROOT, "profiles", "gemm_tiled_prefill_mfma.json")


def measure_peaks(torch, eager=False):
    """Reference rates on this GPU, in this run (see the module docstring)."""
    import ctypes
    from quantized_gemm_quantize_amd.build import PEAKS_LIB
    if not os.path.exists(PEAKS_LIB):
        raise RuntimeError(f"{PEAKS_LIB} is not built: run __graft_entry__.build() first")
    lib = ctypes.CDLL(PEAKS_LIB)
    p, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.peaks_mfma_i8.argtypes = [i32, i32, p, p, p]
    lib.peaks_mfma_bf16.argtypes = [i32, i32, p, p, p]
    lib.peaks_read.argtypes = [p, i64, i32, p, p]
    lib.peaks_write.argtypes = [p, i64, i32, p]
    lib.peaks_read_rows.argtypes = [p, i32, p, p]
    lib.peaks_operand_stream.argtypes = [p, p, i32, i32, i32, p, p]
    for f in (lib.peaks_mfma_i8, lib.peaks_mfma_bf16, lib.peaks_read, lib.peaks_write,
              lib.peaks_read_rows, lib.peaks_operand_stream):
        f.restype = i32
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = lambda: torch.cuda.current_stream().cuda_stream

    def call(rc):
        if rc != 0:
            raise RuntimeError(f"peaks launch failed ({rc})")

    wgs, iters = 2 * cus, 2000
    sink = torch.zeros(4 * cus * 256, dtype=torch.int32, device=dev)
    clk = torch.zeros(2, dtype=torch.int64, device=dev)
    mf = lambda i: call(lib.peaks_mfma_i8(wgs, iters, sink.data_ptr(), clk.data_ptr(), stream()))
    mf(0)
    ms = time_median(mf, 20, torch, 1, eager)
    c = clk.cpu().tolist()
    mfma_tops = wgs * 4 * iters * 8 * 65536 / (ms * 1e-3) / 1e12
    shader_mhz = c[0] / (c[1] / 100e6) / 1e6 if c[1] else None
    mb = lambda i: call(lib.peaks_mfma_bf16(wgs, iters, sink.data_ptr(), clk.data_ptr(), stream()))
    mb(0)
    ms_bf16 = time_median(mb, 20, torch, 1, eager)
    cb = clk.cpu().tolist()
    bf16_tflops = wgs * 4 * iters * 8 * 32768 / (ms_bf16 * 1e-3) / 1e12
    bf16_mhz = cb[0] / (cb[1] / 100e6) / 1e6 if cb[1] else None

    nbytes = 1 << 30
    big = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    call(lib.peaks_write(big.data_ptr(), nbytes, 8 * cus, stream()))
    rd = lambda i: call(lib.peaks_read(big.data_ptr(), nbytes, 8 * cus, sink.data_ptr(), stream()))
    wr = lambda i: call(lib.peaks_write(big.data_ptr(), nbytes, 8 * cus, stream()))
    read_gbs = nbytes / (time_median(rd, 5, torch, 1, eager) * 1e-3) / 1e9
    write_gbs = nbytes / (time_median(wr, 5, torch, 1, eager) * 1e-3) / 1e9
    del big
    # a decode-sized read: the 4096 x 4096 int8 weight, buffers rotated past the MALL
    small = 4096 * 4096
    R = rotation(small)
    bufs = [torch.empty(small, dtype=torch.uint8, device=dev) for _ in range(R)]
    for t in bufs:
        call(lib.peaks_write(t.data_ptr(), small, 8 * cus, stream()))
    rs = lambda i: call(lib.peaks_read(bufs[i % R].data_ptr(), small, 4 * cus, sink.data_ptr(),
                                       stream()))
    read_small_us = time_median(rs, 20 * R, torch, R, eager) * 1e3
    # the same bytes read the way the M-small GEMM reads its weight (16 rows per workgroup,
    # every load in flight at once): the floor that kernel is rated against
    rr = lambda i: call(lib.peaks_read_rows(bufs[i % R].data_ptr(), 4096, sink.data_ptr(), stream()))
    read_rows_us = time_median(rr, 20 * R, torch, R, eager) * 1e3
    del bufs
    # the prefill GEMM's operand stream alone (M = 2048, N = K = 4096), operand sets rotated
    Mp, Np, Kp = 2048, 4096, 4096
    Ro = rotation((Mp + Np) * Kp)
    ops = [(torch.empty(Mp * Kp, dtype=torch.uint8, device=dev),
            torch.empty(Np * Kp, dtype=torch.uint8, device=dev)) for _ in range(Ro)]
    for a, bb in ops:
        call(lib.peaks_write(a.data_ptr(), Mp * Kp, 8 * cus, stream()))
        call(lib.peaks_write(bb.data_ptr(), Np * Kp, 8 * cus, stream()))
    osink = torch.zeros((Mp // 256) * (Np // 128) * 256, dtype=torch.int32, device=dev)
    os_ = lambda i: call(lib.peaks_operand_stream(ops[i % Ro][0].data_ptr(), ops[i % Ro][1].data_ptr(),
                                                  Mp, Np, Kp, osink.data_ptr(), stream()))
    operand_us = time_median(os_, 10 * Ro, torch, Ro, eager) * 1e3
    # the same stream over one operand set, which then stays in the Infinity Cache: the
    # difference is the cost of filling the L2s from HBM
    oc = lambda i: call(lib.peaks_operand_stream(ops[0][0].data_ptr(), ops[0][1].data_ptr(),
                                                 Mp, Np, Kp, osink.data_ptr(), stream()))
    operand_cached_us = time_median(oc, 10 * Ro, torch, 1, eager) * 1e3
    del ops
    torch.cuda.synchronize()
    return {"mfma_int8_TOPs": round(mfma_tops, 1), "mfma_loop_shader_MHz": round(shader_mhz, 1),
            "mfma_bf16_TFLOPs": round(bf16_tflops, 1), "mfma_bf16_loop_shader_MHz": round(bf16_mhz, 1),
            "hbm_read_GBps": round(read_gbs, 1), "hbm_write_GBps": round(write_gbs, 1),
            "read_16_8MB_us": round(read_small_us, 3),
            "read_16_8MB_GBps": round(small / (read_small_us * 1e-6) / 1e9, 1),
            "read_16_8MB_rows_us": round(read_rows_us, 3),
            "read_16_8MB_rows_GBps": round(small / (read_rows_us * 1e-6) / 1e9, 1),
            "prefill_operand_stream_us": round(operand_us, 3),
            "prefill_operand_stream_GBps_per_CU": round((256 + 128) * Kp / (operand_us * 1e-6) / 1e9, 1),
            "prefill_operand_stream_cached_us": round(operand_cached_us, 3),
            "method": "libpeaks.so: 8 independent v_mfma_i32_32x32x32_i8 (and, separately, "
                      "v_mfma_f32_32x32x16_bf16) chains per wavefront, "
                      f"{wgs} workgroups of 4 wavefronts; 16-byte loads / streaming stores over "
                      "1 GiB; 16.8 MB reads over rotated buffers, grid-stride and in the M-small "
                      "GEMM's row-slice pattern (256 workgroups, 16 loads per lane in flight); "
                      "the 2048 x 4096 x 4096 GEMM's operand stream alone (256 x 128 tiles in its "
                      "tile order, 3-stage direct-to-LDS ring, its waits and barriers, no arithmetic) "
                      f"over {Ro} rotated operand sets, and over one set (Infinity Cache resident); "
                      "HIP graph replays, median of 5"}


def amd_smi_clocks():
    """gfx (mean over the XCDs) and memory clocks from one `amd-smi metric -c --json`, or
    None where the tool is missing or fails."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-c", "--json"], capture_output=True, text=True,
                           timeout=20)
        data = json.loads(r.stdout)
        clock = data["gpu_data"][0]["clock"] if isinstance(data, dict) else data[0]["clock"]
        gfx = [v["clk"]["value"] for k, v in clock.items() if k.startswith("gfx_")
               and isinstance(v, dict) and isinstance(v.get("clk"), dict)]
        mem = [v["clk"]["value"] for k, v in clock.items() if k.startswith("mem_")
               and isinstance(v, dict) and isinstance(v.get("clk"), dict)]
        return {"gfx_MHz": round(sum(gfx) / len(gfx), 1) if gfx else None,
                "mem_MHz": mem[0] if mem else None}
    except Exception:
        return None


def clocks_under_load(fn, torch, period, seconds=2.0):
    """amd-smi samples while the HIP graph of `fn` (one period of rotated calls) replays back
    to back for about `seconds`; and one sample at idle before."""
    import threading
    idle = amd_smi_clocks()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(period):
            fn(i)
    samples, stop = [], threading.Event()

    def poll():
        while not stop.is_set():
            c = amd_smi_clocks()
            if c is None:
                return
            samples.append(c)
    th = threading.Thread(target=poll)
    torch.cuda.synchronize()
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            g.replay()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    gfx = [c["gfx_MHz"] for c in samples if c.get("gfx_MHz")]
    return {"idle": idle, "under_load_samples": len(samples),
            "under_load_gfx_MHz": sorted(gfx), "under_load_mem_MHz":
            samples[-1]["mem_MHz"] if samples else None}


def mfma_record():
    """The committed rocprofv3 MFMA-counter record of the prefill GEMM, when taken on the
    current kernel source."""
    if not os.path.exists(MFMA_RECORD):
        return None
    rec = json.load(open(MFMA_RECORD))
    if rec.get("source_hash") != source_hash(GEMM_SOURCES):
        return None
    return {k: rec[k] for k in ("mfma_busy_frac", "mfma_busy_cycles", "gui_active_cycles",
                                "mops_i8", "kernel") if k in rec}


def bench_decode(torch, np, b, dev, steps, warmup, eager=False):
    """M=16 weight-streaming GEMM: GB/s with weight copies rotated past the Infinity Cache."""
    d = prepare("decode", torch, np, b, dev)
    M, N, K = d["inp"].M, d["inp"].N, d["inp"].K
    xq, sx = b.w8a8_quantize_rows(d["x"])
    R = rotation(N * K)
    wqs = [d["wq"].clone() for _ in range(R)]
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    xq2, sx2 = torch.empty_like(xq), torch.empty_like(sx)
    gemm = lambda i: b.w8a8_gemm(xq, sx, wqs[i % R], d["sw"], out=out)

    def step(i):
        b.w8a8_quantize_rows(d["x"], xq2, sx2)
        b.w8a8_gemm(xq2, sx2, wqs[i % R], d["sw"], out=out)

    fused = lambda i: b.w8a8_fused_linear(d["x"], wqs[i % R], d["sw"], out=out)

    for i in range(warmup):
        step(i)
        fused(i)
    # the single launch gives the two-launch step's output bit for bit
    step(0)
    two = out.clone()
    fused(0)
    if not torch.equal(two.view(torch.int16), out.view(torch.int16)):
        raise SystemExit("fused linear differs from quantize_rows + gemm")
    ms_gemm = time_median(gemm, steps, torch, R, eager)
    ms_step = time_median(step, steps, torch, R, eager)
    ms_fused = time_median(fused, steps, torch, R, eager)
    gemm_bytes = M * K + 4 * M + N * K + 4 * N + 2 * M * N
    layer_bytes = 2 * M * K + N * K + 4 * N + 2 * M * N
    gbs = gemm_bytes / (ms_gemm * 1e-3) / 1e9
    return {"workload": f"decode M={M} K={K} N={N}", "gemm_us": round(ms_gemm * 1e3, 3),
            "gemm_GBps": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "gemm_bytes": gemm_bytes, "step_us": round(ms_step * 1e3, 3),
            "step_GBps": round(layer_bytes / (ms_step * 1e-3) / 1e9, 1),
            "fused_linear_us": round(ms_fused * 1e3, 3),
            "fused_linear_GBps": round(layer_bytes / (ms_fused * 1e-3) / 1e9, 1),
            "layer_bytes": layer_bytes, "weight_copies_rotated": R}


PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, TFLOP/s


def w4a16_cpu_baseline(inp, np, gpu_rows=None):
    """The CPU oracle (dequantization + float64-summed bf16 GEMM) on a bounded row sample;
    with gpu_rows(r) (the timed kernel's bf16 output bits for rows 0..r-1 of the same inputs)
    the oracle's rows are compared with them (the `parity` entry)."""
    import oracle
    M, K = inp.x_bits.shape
    N = inp.wq4.shape[0]

    def run(rows):
        t0 = time.perf_counter()
        w = oracle.w4a16_dequant(inp.wq4, inp.scales, inp.zeros)
        out = oracle.bf16_gemm(inp.x_bits[:rows], w)
        return time.perf_counter() - t0, out

    probe = min(M, 8)
    t_probe = run(probe)[0]
    rows = int(min(M, max(probe, probe * 15.0 / max(t_probe, 1e-6))))
    t, out = run(rows)
    parity = None
    if gpu_rows is not None:
        ulps = bf16_ulps(gpu_rows(rows), out, np)
        parity = {"rows": rows, "max_ulp": int(ulps.max()),
                  "frac_beyond_1ulp": float((ulps > 1).mean()),
                  "bar": "the fp32 summation bound of the tests (at most 1e-3 of the outputs "
                         "beyond 1 ulp)"}
    return {"value": round(2.0 * rows * N * K / t / 1e12, 6), "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"rows 0..{rows - 1} of the W4A16 layer (M={M}, N={N}, K={K}): "
                      f"dequantization of the whole weight + float64-summed bf16 GEMM, "
                      f"{t:.2f} s wall", "parity": parity}


def bench_w4a16(args, torch, np, b, dev):
    """W4A16 fused dequant GEMM (one launch per step) on the pages' N = K = 4096, group 128
    layer; with the M = 16 .. 1024 sweep of the pages' table, fused against the unfused
    route (w4a16_dequant, then the vendor library's bf16 matmul)."""
    from quantized_gemm_quantize_amd.inputs import W4A16_CONFIGS, W4A16_M, make_w4a16

    cfg = W4A16_CONFIGS[args.config]
    N, K, G = cfg["N"], cfg["K"], cfg["G"]
    w_bytes = N * K // 2 + 2 * 2 * N * (K // G)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def setup(M, signed=False, half=False):
        inp = make_w4a16(M, N, K, G, seed=0, signed=signed, half=half)
        R = rotation(w_bytes + 2 * M * K + 2 * M * N)
        dt = torch.float16 if half else torch.bfloat16
        h = lambda bits: t(bits.view(np.int16)).view(dt)
        x = h(inp.x_bits)
        ws = [(t(inp.wq4), h(inp.scales), h(inp.zeros)) for _ in range(R)]
        outs = [torch.empty((M, N), dtype=dt, device=dev) for _ in range(R)]
        return inp, x, ws, outs, R

    def fused_time(M, steps, signed=False, half=False):
        inp, x, ws, outs, R = setup(M, signed, half)
        fn = lambda i: b.w4a16_gemm(x, *ws[i % R], signed=signed, out=outs[i % R])
        for i in range(max(args.warmup, R)):
            fn(i)
        return inp, time_median(fn, steps, torch, R, args.eager), R, x, ws

    M = cfg["M"]
    inp, ms, R, x, ws = fused_time(M, args.steps)
    ms_step = time_loop(lambda i: b.w4a16_gemm(x, *ws[i % R]), args.steps, torch, period=R,
                        eager=args.eager)
    flops = 2.0 * M * N * K
    value = flops / (ms_step * 1e-3) / 1e12
    if M <= 64:
        nbytes = 2 * M * K + w_bytes + 2 * M * N
        gbs = nbytes / (ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4)}
    else:
        tf = flops / (ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
    roof.update({"traffic": None, "kernel": "w4a16_gemm", "avg_launch_us": round(ms * 1e3, 3)})
    peaks = None
    if not args.no_peaks:
        peaks = measure_peaks(torch, args.eager)
        if roof["bound"] == "mfma":
            roof["frac_measured"] = round(roof["achieved"] / peaks["mfma_bf16_TFLOPs"], 4)
            roof["peak_measured"] = peaks["mfma_bf16_TFLOPs"]
        else:
            t_ideal = ((2 * M * K + w_bytes) / (peaks["hbm_read_GBps"] * 1e9)
                       + 2 * M * N / (peaks["hbm_write_GBps"] * 1e9))
            roof["frac_measured"] = round(t_ideal / (ms * 1e-3), 4)
    # the other code and value formats at the same M (signed codes, binary16 values)
    formats = {}
    for name, sg, hf in (("s4_bf16", True, False), ("u4_f16", False, True), ("s4_f16", True, True)):
        formats[name + "_us"] = round(fused_time(M, max(50, args.steps // 4), sg, hf)[1] * 1e3, 3)

    sweep = []
    for m in W4A16_M:
        _, ms_f, Rm, xm, wsm = fused_time(m, max(50, args.steps // 4))
        wbuf = torch.empty((N, K), dtype=torch.bfloat16, device=dev)

        def unfused(i):
            b.w4a16_dequant(*wsm[i % Rm], out=wbuf)
            torch.matmul(xm, wbuf.t())
        for i in range(5):
            unfused(i)
        ms_u = time_median(unfused, max(50, args.steps // 4), torch, Rm, eager=True)
        sweep.append({"M": m, "fused_us": round(ms_f * 1e3, 3),
                      "fused_TFLOPs": round(2.0 * m * N * K / (ms_f * 1e-3) / 1e12, 1),
                      "unfused_us": round(ms_u * 1e3, 3)})
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic", "timing": "eager launches" if args.eager else "HIP graph replay",
        "config": {"workload": f"{args.config} M={M} K={K} N={N} group={G}",
                   "step": "w4a16_gemm", "seed": 0, "input_sets_rotated": R},
        "roofline": roof,
        "gemm_only": {"us": round(ms * 1e3, 3), "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 1)},
        "formats": formats,
        "sweep_n4096_k4096_g128": sweep,
    }
    if not args.no_cpu_baseline:
        out0 = b.w4a16_gemm(x, *ws[0])
        torch.cuda.synchronize()
        gpu_rows = lambda r: out0[:r].view(torch.int16).cpu().numpy().view(np.uint16)
        line["cpu_baseline"] = w4a16_cpu_baseline(inp, np, gpu_rows)
    if peaks is not None:
        line["peaks"] = peaks
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the layer is "
              "data parallel over rows, so N GPUs would each run this same kernel on M/N rows.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.copy_calibration:
        nbytes = 256 << 20
        src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": nbytes, "copies": 5}), flush=True)
        return

    if args.peaks:
        print(json.dumps({"peaks": measure_peaks(torch, args.eager)}), flush=True)
        return
    from quantized_gemm_quantize_amd import binding as b
    b.load()
    dev = torch.device("cuda:0")
    name = args.config
    if name.startswith("w4a16"):
        bench_w4a16(args, torch, np, b, dev)
        return
    d = prepare(name, torch, np, b, dev)
    inp = d["inp"]
    M, N, K = inp.M, inp.N, inp.K
    bsr = bool(inp.bs)
    sp24 = "values24" in d

    # rotated input sets: X, weights and outputs at distinct addresses
    if bsr:
        w_bytes = d["values"].numel()
    elif sp24:
        w_bytes = N * K // 2 + N * K // 8
    else:
        w_bytes = N * K
    per_set = 2 * M * K + M * K + w_bytes + 2 * M * N
    R = rotation(per_set)
    xs = [d["x"].clone() for _ in range(R)]
    if bsr:
        ws = [d["values"].clone() for _ in range(R)]
    elif sp24:
        ws = [(d["values24"].clone(), d["meta24"].clone()) for _ in range(R)]
    else:
        ws = [d["wq"].clone() for _ in range(R)]
    xqs = [torch.empty((M, K), dtype=torch.int8, device=dev) for _ in range(R)]
    sxs = [torch.empty((M,), dtype=torch.float32, device=dev) for _ in range(R)]
    outs = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(R)]

    def quant(i):
        j = i % R
        b.w8a8_quantize_rows(xs[j], xqs[j], sxs[j])

    def gemm(i):
        j = i % R
        if bsr:
            b.w8a8_bsr_gemm(xqs[j], sxs[j], d["crow"], d["col"], ws[j], d["sw"], out=outs[j])
        elif sp24:
            b.w8a8_sparse24_gemm(xqs[j], sxs[j], ws[j][0], ws[j][1], d["sw"], out=outs[j])
        else:
            b.w8a8_gemm(xqs[j], sxs[j], ws[j], d["sw"], out=outs[j])

    def step(i):
        quant(i)
        gemm(i)

    for i in range(max(args.warmup, R)):
        step(i)
    torch.cuda.synchronize()
    eager_out = outs[0].clone()
    eager_xq, eager_sx = xqs[0].clone(), sxs[0].clone()
    ms_step = time_loop(step, args.steps, torch, period=R, eager=args.eager)
    # graph replays recompute the same outputs: check the first set bit for bit
    if not torch.equal(outs[0].view(torch.int16), eager_out.view(torch.int16)):
        raise RuntimeError("graph replay output differs from the eager output")
    # the kernels alone: median of 5 regions of K calls each
    ms_gemm = time_median(gemm, args.steps, torch, R, args.eager)
    # quantize alone touches only X, its codes and scales: rotate enough of those sets that
    # they, too, exceed twice the Infinity Cache
    Rq = max(R, rotation(3 * M * K + 4 * M))
    xs_q = xs + [d["x"].clone() for _ in range(Rq - R)]
    xqs_q = xqs + [torch.empty((M, K), dtype=torch.int8, device=dev) for _ in range(Rq - R)]
    sxs_q = sxs + [torch.empty((M,), dtype=torch.float32, device=dev) for _ in range(Rq - R)]
    ms_quant = time_median(lambda i: b.w8a8_quantize_rows(xs_q[i % Rq], xqs_q[i % Rq], sxs_q[i % Rq]),
                           args.steps, torch, Rq, args.eager)
    del xs_q, xqs_q, sxs_q
    # the vendor library on the same rotated inputs: torch._int_mm (hipBLASLt), int8 x int8
    # -> int32 with no dequant epilogue (it writes 4 bytes per output, we write 2). Launched
    # eagerly, never captured into a graph (a library call may record memsets); at tens of
    # microseconds per call the launches still run back to back on the GPU.
    library = None
    if not bsr and not sp24 and M > 16:
        ms_lib = time_median(lambda i: torch._int_mm(xqs[i % R], ws[i % R].t()), args.steps,
                             torch, R, eager=True)
        library = {"kernel": "torch._int_mm (hipBLASLt) int8 -> int32, no dequant epilogue",
                   "us": round(ms_lib * 1e3, 3),
                   "TOPs": round(2.0 * M * N * K / (ms_lib * 1e-3) / 1e12, 1),
                   "w8a8_gemm_speedup": round(ms_lib / ms_gemm, 3)}

    # the addmm epilogue (alpha, beta, a per-channel bias) of the dense and BSR kernels
    addmm = None
    if not bsr and not sp24:
        bias = torch.randn(N, device=dev, dtype=torch.float32) * 0.5
        ms_addmm = time_median(
            lambda i: b.w8a8_gemm_addmm(xqs[i % R], sxs[i % R], ws[i % R], d["sw"], bias=bias,
                                        alpha=0.75, beta=1.5, out=outs[i % R]),
            args.steps, torch, R, args.eager)
        addmm = {"kernel": "w8a8_gemm_addmm", "us": round(ms_addmm * 1e3, 3),
                 "vs_plain": round(ms_addmm / ms_gemm, 3)}
    bsr_addmm = None
    if bsr:
        bias = torch.randn(N, device=dev, dtype=torch.float32) * 0.5
        ms_addmm = time_median(
            lambda i: b.w8a8_bsr_gemm_addmm(xqs[i % R], sxs[i % R], d["crow"], d["col"], ws[i % R],
                                            d["sw"], bias=bias, alpha=0.75, beta=1.5,
                                            out=outs[i % R]),
            args.steps, torch, R, args.eager)
        bsr_addmm = {"kernel": "w8a8_bsr_gemm_addmm", "us": round(ms_addmm * 1e3, 3),
                     "vs_plain": round(ms_addmm / ms_gemm, 3)}

    ops = 2.0 * M * N * K
    if bsr:
        # stored blocks only: each 64x64 block is a 64-deep product for all M rows
        ops = 2.0 * M * 64 * 64 * int(d["values"].shape[0])
    elif sp24:
        # the kept products only: two of every four weights
        ops = 1.0 * M * N * K
    value = ops / (ms_step * 1e-3) / 1e12
    gemm_tops = ops / (ms_gemm * 1e-3) / 1e12
    q_bytes = 2 * M * K + M * K + 4 * M

    traffic = None
    if os.path.exists(TRAFFIC_RECORD) and name == "prefill_outliers":
        rec = json.load(open(TRAFFIC_RECORD))
        if rec.get("source_hash") == source_hash(GEMM_SOURCES):
            traffic = rec.get("bytes_per_launch")

    if bsr or M <= 64:
        # HBM bound: the BSR output write, or the M <= 64 weight stream
        gemm_bytes = M * K + 4 * M + w_bytes + 4 * N + 2 * M * N
        roof = {"bound": "hbm", "achieved": round(gemm_bytes / (ms_gemm * 1e-3) / 1e9, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
        roof["frac"] = round(roof["achieved"] / PEAK_HBM_GBS, 4)
    else:
        roof = {"bound": "mfma", "achieved": round(gemm_tops, 1), "peak": PEAK_INT8_TOPS,
                "unit": "TOP/s", "frac": round(gemm_tops / PEAK_INT8_TOPS, 4)}
    roof["traffic"] = traffic
    peaks = clocks = None
    if not args.no_peaks:
        peaks = measure_peaks(torch, args.eager)
        if roof["bound"] == "mfma":
            roof["frac_measured"] = round(gemm_tops / peaks["mfma_int8_TOPs"], 4)
            roof["peak_measured"] = peaks["mfma_int8_TOPs"]
        else:
            rbytes = M * K + 4 * M + w_bytes + 4 * N
            t_ideal = rbytes / (peaks["hbm_read_GBps"] * 1e9) + 2 * M * N / (peaks["hbm_write_GBps"] * 1e9)
            roof["frac_measured"] = round(t_ideal / (ms_gemm * 1e-3), 4)
        clocks = clocks_under_load(step, torch, R)
    if roof["bound"] == "mfma" and name == "prefill_outliers":
        roof["mfma_counters"] = mfma_record()
        if peaks:
            roof["operand_stream_us"] = peaks["prefill_operand_stream_us"]
            roof["frac_of_operand_stream"] = round(peaks["prefill_operand_stream_us"] / (ms_gemm * 1e3), 4)
    kernel = "w8a8_bsr_gemm" if bsr else "w8a8_sparse24_gemm" if sp24 else "w8a8_gemm"
    roof["kernel"] = kernel
    roof["avg_launch_us"] = round(ms_gemm * 1e3, 3)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "timing": "eager launches" if args.eager else "HIP graph replay",
        "config": {"workload": f"{name} M={M} K={K} N={N}"
                   + (f" BSR 64x64 nnzb={d['values'].shape[0]}" if bsr else "")
                   + (" 2:4 weight (ops: kept products, M*N*K)" if sp24 else ""),
                   "step": "w8a8_quantize_rows + " + kernel,
                   "seed": 0, "input_sets_rotated": R},
        "roofline": roof,
        "quantize_rows": {"us": round(ms_quant * 1e3, 3),
                          "GBps": round(q_bytes / (ms_quant * 1e-3) / 1e9, 1),
                          "frac_of_hbm_peak": round(q_bytes / (ms_quant * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                          "input_sets_rotated": Rq},
        "gemm_only": {"us": round(ms_gemm * 1e3, 3), "TOPs": round(gemm_tops, 1),
                      "frac_of_int8_peak": round(gemm_tops / PEAK_INT8_TOPS, 4)},
    }
    if sp24:
        line["gemm_only"]["dense_equivalent_TOPs"] = round(2 * gemm_tops, 1)
    if library is not None:
        line["library_int_mm"] = library
    if addmm is not None:
        line["gemm_addmm"] = addmm
    if bsr_addmm is not None:
        line["bsr_addmm"] = bsr_addmm
    if not args.no_decode and name == "prefill_outliers":
        line["decode_m16"] = bench_decode(torch, np, b, dev, args.steps, args.warmup, args.eager)
        if peaks is not None:
            dm = line["decode_m16"]
            t_floor = min(peaks["read_16_8MB_us"], peaks["read_16_8MB_rows_us"])
            dm["vs_measured_read_floor"] = round(t_floor / dm["gemm_us"], 4)
    if peaks is not None:
        line["peaks"] = peaks
        line["clocks"] = clocks
    if not args.no_cpu_baseline:
        gpu_rows = lambda r: (eager_xq[:r].cpu().numpy(), eager_sx[:r].cpu().numpy(),
                              eager_out[:r].view(torch.int16).cpu().numpy().view(np.uint16))
        line["cpu_baseline"] = cpu_baseline(name, np, gpu_rows)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the W4A16 group-quantized linear on one MI355X.

    python bench.py [--gpus 1] [--steps 3000] [--warmup 20] [--quick]

A step is one call of the online hot path, wq_linear_sparse (kernel chosen by
M, sparse term fused), on the headline workload: the decode GEMV of a Llama-7B
MLP up-projection, x fp16 [1, 4096], W [11008, 4096] INT4 g128.  The weights are quantized and
packed on the GPU by wq_quantize_rtn / wq_pack before timing (offline steps,
reported separately under "offline").

Inputs stay resident in HBM: R copies of the layer (packed codes, scales,
zeros, CSR, x, y) totalling >= 1 GiB are rotated so no launch is served from
the 256 MB Infinity Cache.  After W warm-up launches, the K timed launches go
in chunks of at most 256, each queued behind a busy-wait kernel; HIP events on
the launch stream, recorded after the busy-wait and after the chunk's last
launch, bracket the chunk, which the GPU runs back to back (the busy-wait lasts
long enough for the host to submit the chunk, and the run checks that it did).
The value is the sum over the chunks: the GPU time of exactly K launches.  Five
runs, between synchronizations; the median gives the figures (p10 and p90
beside them).  The other workloads size their runs to at least 200 launches and
20 ms, from one timed run of 20.

Printed: ONE JSON line with the metric (GB/s, algorithmic bytes), the roofline
of the dominant kernel, the CPU oracle baseline, and the other workloads
(batched decode + sparse, prefill, the 70B down-projection M sweep and one GPU's
shard of it, the decode and prefill layers with a rank-32 low-rank branch and as
act-order layers), and,
as context, torch's device copy of the same byte count.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFS = 2516.6     # 256 CU x 2.4 GHz x 4096 flop/clk, dense
ROTATE_BYTES = 1 << 30


def alg_bytes(M, N, K, nnz, y_bytes=2, rank=0, act_order=False, bits=4, group=128):
    """Bytes the method must move: packed codes (bits / 8 per weight), fp16
    scale+zero per group, CSR, the fp16 low-rank factors, the int32 channel
    permutation of an act-order layer, x, y."""
    csr = (6 * nnz + 4 * (N + 1)) if nnz else 0
    perm = 4 * K if act_order else 0
    return (N * K * bits // 8 + N * (K // group) * 4 + csr + 2 * rank * (K + N) + perm + M * K * 2 +
            M * N * y_bytes)


def alg_flops(M, N, K, nnz, rank=0):
    return 2 * M * N * K + 2 * M * nnz + 2 * M * rank * (K + N)


class Layer:
    """A quantized layer on the GPU, produced by the library's own quantizer."""

    def __init__(self, wq, torch, index, M, K=None, rank=0, act_order=False, w4a8=False, bits=4, group=128,
                 sparse_ppm=None):
        W, x, cfg = workloads.make(index, M=M, K=K)
        N, K = W.shape
        self.wq = wq
        self.N, self.K, self.M, self.rank, self.act_order, self.w4a8 = N, K, M, rank, act_order, w4a8
        self.bits, self.group = bits, group
        if w4a8:
            self.outliers = torch.from_numpy(workloads.x_outlier_channels(index, M=M, K=K)).cuda()
            self.ws_bytes = wq.linear_w4a8_workspace_bytes(M, N, K)
        self.sparse_k = workloads.sparse_k_for(cfg, N, K)
        if sparse_ppm is not None:
            self.sparse_k = sparse_ppm * N * K // 1_000_000
        Wd = torch.from_numpy(W).cuda()
        if act_order:
            self.perm = torch.from_numpy(workloads.channel_permutation(index + 7, K)).cuda()
            q = wq.quantize_rtn_act_order(Wd, self.perm, sparse_k=self.sparse_k)
            self.ws_bytes = wq.linear_act_order_workspace_bytes(M, N, K)
        else:
            q = wq.quantize_rtn(Wd, sparse_k=self.sparse_k, group=group, bits=bits)
        self.packed = wq.pack(q["codes"], bits=bits)
        self.scales, self.zeros = q["scales"], q["zeros"]
        self.row_ptr, self.col, self.val = q["row_ptr"], q["col"], q["val"]
        del q, Wd
        self.x = torch.from_numpy(x.view(np.int16).copy()).cuda().view(torch.float16)
        if rank:
            L1, L2 = workloads.lowrank_factors(index + 100 * M, rank, N, K)
            self.L1 = torch.from_numpy(L1.view(np.int16).copy()).cuda().view(torch.float16)
            self.L2 = torch.from_numpy(L2.view(np.int16).copy()).cuda().view(torch.float16)
            self.ws_bytes = wq.linear_lowrank_workspace_bytes(M, N, K, rank)
        torch.cuda.synchronize()

    def sets(self, torch, rotate_bytes):
        """R independent copies of every input/output, R * bytes >= rotate_bytes."""
        nb = alg_bytes(self.M, self.N, self.K, self.sparse_k, rank=self.rank, act_order=self.act_order,
                       bits=self.bits, group=self.group)
        R = max(1, min(64, math.ceil(rotate_bytes / nb)))
        out = []
        for r in range(R):
            s = dict(x=self.x.clone(), packed=self.packed.clone(), scales=self.scales.clone(),
                     zeros=self.zeros.clone(), row_ptr=self.row_ptr.clone(), col=self.col.clone(),
                     val=self.val.clone(),
                     y=torch.empty((self.M, self.N), dtype=torch.float16, device="cuda"))
            if self.rank:
                s.update(L1=self.L1.clone(), L2=self.L2.clone(),
                         ws=torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda"))
            if self.act_order:
                s.update(perm=self.perm.clone(), ws=torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda"))
            if self.w4a8:
                s.update(outliers=self.outliers.clone(),
                         ws=torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda"))
            if not (self.rank or self.act_order or self.w4a8):
                # the plain product's split-K partials, allocated once per set (not per launch)
                nws = self.wq.linear_workspace_bytes(self.M, self.N, self.K)
                s["ws"] = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
            out.append(s)
        return out


def launch(wq, s, kernel="auto"):
    if "outliers" in s:
        wq.linear_w4a8(s["x"], s["outliers"], s["packed"], s["scales"], s["zeros"], out=s["y"], workspace=s["ws"])
    elif "perm" in s:
        wq.linear_act_order(s["x"], s["perm"], s["packed"], s["scales"], s["zeros"], s["row_ptr"], s["col"],
                            s["val"], out=s["y"], kernel=kernel, workspace=s["ws"])
    elif "L1" in s:
        wq.linear_lowrank(s["x"], s["packed"], s["scales"], s["zeros"], s["L1"], s["L2"], s["row_ptr"], s["col"],
                          s["val"], out=s["y"], kernel=kernel, workspace=s["ws"])
    else:
        wq.linear_sparse(s["x"], s["packed"], s["scales"], s["zeros"], s["row_ptr"], s["col"], s["val"],
                         out=s["y"], kernel=kernel, workspace=s["ws"])


def time_launches(wq, torch, sets, steps, warmup, kernel="auto", repeats=5):
    """Warm up, then time `repeats` runs of `steps` launches rotating over the
    buffer sets; returns the milliseconds per launch of every run."""
    stream = torch.cuda.Stream()
    host_us = 0.0
    with torch.cuda.stream(stream):
        for i in range(warmup):
            t0 = time.perf_counter()
            launch(wq, sets[i % len(sets)], kernel)
            if i > 0:  # the first launch of a kernel also loads it
                host_us = max(host_us, (time.perf_counter() - t0) * 1e6)
    torch.cuda.synchronize()
    return [timed_launches(torch, stream, lambda i: launch(wq, sets[i % len(sets)], kernel), steps,
                           host_us or HOST_US_PER_LAUNCH) / steps
            for _ in range(repeats)]


# Host time to submit one launch when none was measured (about 13 us through the
# binding for one kernel), used to size the busy-wait that runs ahead of a timed run.
HOST_US_PER_LAUNCH = 40.0
ENGINE_GHZ = 2.4  # peak engine clock: the busy-wait lasts at least its cycles / 2.4 GHz
CHUNK = 256       # launches per busy-wait (at most three kernels each: well inside the queue)


def timed_launches(torch, stream, fn, steps, host_us=HOST_US_PER_LAUNCH):
    """Milliseconds of GPU time of `steps` launches fn(0) .. fn(steps - 1) on
    `stream`, between synchronizations.

    The launches go in chunks of at most CHUNK. Each chunk is queued behind a
    busy-wait kernel long enough for the host to submit the whole chunk while it
    runs, and HIP events recorded after the busy-wait and after the chunk's last
    launch bracket it, so the GPU runs the chunk back to back and the events see
    GPU work only (a graph replay instead adds about 8 us of its own per replay,
    which a 20-launch run would spread over its launches). Chunks keep the queue
    from filling up, which would stall the host until the busy-wait ends. The
    busy-wait is timed too: if the host took longer than that to submit a chunk,
    the run raises rather than report host time as GPU time. Returns the sum over
    the chunks."""
    total = 0.0
    for c0 in range(0, steps, CHUNK):
        n = min(CHUNK, steps - c0)
        prime_us = 500.0 + 3.0 * max(host_us, 10.0) * n
        for attempt in range(4):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            with torch.cuda.stream(stream):
                torch.cuda.synchronize()
                ev[0].record(stream)
                torch.cuda._sleep(int(prime_us * 1e3 * ENGINE_GHZ))
                t0 = time.perf_counter()
                ev[1].record(stream)
                for i in range(c0, c0 + n):
                    fn(i)
                ev[2].record(stream)
                host_ms = (time.perf_counter() - t0) * 1e3
            torch.cuda.synchronize()
            if host_ms <= ev[0].elapsed_time(ev[1]):
                break
            # the host fell behind (a slow host, or a tracer): the chunk is discarded
            # and run again behind a busy-wait twice as long
            prime_us *= 2
        else:
            raise RuntimeError(f"host submission ({host_ms:.3f} ms) outlasted the busy-wait "
                               f"({ev[0].elapsed_time(ev[1]):.3f} ms): the timed run would include host gaps")
        total += ev[1].elapsed_time(ev[2])
    return total


def run_length(wq, torch, sets, kernel, min_ms=20.0, min_steps=200, max_steps=20000):
    """Launches per timed run so that one run spans at least min_steps and about
    min_ms, from one timed run of 20 launches."""
    t = time_launches(wq, torch, sets, 20, 3, kernel, repeats=1)[0]  # warm: a kernel's first launch loads it
    return int(min(max_steps, max(min_steps, math.ceil(min_ms / t))))


def measure(wq, torch, index, M, steps, warmup, kernel="auto", K=None, replays=5, rank=0, mode=""):
    """steps = None: enough launches per run for >= 20 ms (and >= 200 launches);
    rank > 0: with a low-rank branch of that rank; mode "ao": the layer in a
    permuted channel order, x gathered through the permutation; mode "w8": the
    W4A8 product with the configuration's activation outlier channels in fp16
    (the layer has no CSR then); mode "b3": 3-bit codes in the 3-bit packing;
    "g64": one (s, z) per 64 input channels; "b3g64": both; "sp": the layer's
    outliers at 0.45 % of the weights (the batched-decode layer's density), also
    where the configuration has none (the prefill layer)."""
    act_order, w4a8 = mode == "ao", mode == "w8"
    bits = 3 if mode in ("b3", "b3g64") else 4
    group = 64 if mode in ("g64", "b3g64") else 128
    L = Layer(wq, torch, index, M, K, rank, act_order, w4a8, bits, group,
              sparse_ppm=workloads.SPARSE_PPM_DENSE_AND_SPARSE if mode == "sp" else None)
    if w4a8:
        L.sparse_k = 0
    sets = L.sets(torch, ROTATE_BYTES)
    if steps is None:
        steps = run_length(wq, torch, sets, kernel)
    runs = time_launches(wq, torch, sets, steps, warmup, kernel, repeats=replays)
    ms = float(np.median(runs))
    nb = alg_bytes(M, L.N, L.K, L.sparse_k, rank=rank, act_order=act_order, bits=bits, group=group)
    nf = alg_flops(M, L.N, L.K, L.sparse_k, rank=rank)
    used = kernel if kernel != "auto" else wq.auto_kernel(M, L.N, L.K)
    if w4a8:
        used = "w4a8"
    res = dict(config=index, M=M, N=L.N, K=L.K, nnz=L.sparse_k, rank=rank, mode=mode, kernel=used,
               steps=steps,
               us_per_launch=ms * 1e3,
               us_p10=float(np.percentile(runs, 10)) * 1e3, us_p90=float(np.percentile(runs, 90)) * 1e3,
               replays=len(runs),
               alg_bytes=nb, alg_flops=nf, GBps=nb / (ms * 1e-3) / 1e9, TFLOPs=nf / (ms * 1e-3) / 1e12,
               rotated_sets=len(sets))
    res["hbm_frac"] = res["GBps"] / HBM_PEAK_GBS
    res["mfma_frac"] = res["TFLOPs"] / MFMA_F16_PEAK_TFS
    del sets, L
    torch.cuda.empty_cache()
    return res


def stream_copy(torch, nbytes, steps=100):
    """Context, not the denominator: torch's device-to-device copy of nbytes per
    launch (nbytes read + nbytes written), rotating over >= 1 GiB of sources so
    that reads come from HBM. Of torch's streaming kernels it is the fastest here,
    so it shows what a generic library kernel reaches at this transfer size."""
    n = nbytes // 4
    R = max(1, min(64, math.ceil(ROTATE_BYTES / nbytes)))
    bufs = [torch.ones(n, dtype=torch.int32, device="cuda") for _ in range(R)]
    dst = torch.empty(n, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for i in range(R):
            dst.copy_(bufs[i])
    torch.cuda.synchronize()
    us = timed_launches(torch, stream, lambda i: dst.copy_(bufs[i % R]), steps) / steps * 1e3
    del bufs, dst
    torch.cuda.empty_cache()
    return {"bytes_read": n * 4, "bytes_written": n * 4, "us_per_launch": us,
            "GBps_read_plus_write": 2 * n * 4 / (us * 1e-6) / 1e9}


def device_context(torch):
    """The GPU's own figures, to check the public ones the rooflines use (256 CUs,
    2.4 GHz peak engine clock, 160 KB of LDS per CU): torch's device properties,
    and the peak clock and compute units that rocminfo reports for the agent."""
    import re
    import subprocess
    p = torch.cuda.get_device_properties(0)
    d = {"name": p.name, "gcn_arch": getattr(p, "gcnArchName", ""), "compute_units": p.multi_processor_count,
         "total_memory_GiB": round(p.total_memory / 2**30, 1), "l2_cache_bytes": getattr(p, "L2_cache_size", None),
         "wave_size": getattr(p, "warp_size", None)}
    try:
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
        arch = d["gcn_arch"].split(":")[0]
        for block in out.split("*******"):
            if arch and re.search(r"^\s*Name:\s+" + re.escape(arch) + r"\s*$", block, re.M):
                for line in block.splitlines():
                    if "Max Clock Freq. (MHz):" in line:
                        d["rocminfo_max_clock_mhz"] = int(line.split(":")[1].split()[0])
                    if line.strip().startswith("Compute Unit:"):
                        d["rocminfo_compute_units"] = int(line.split(":")[1].split()[0])
                break
    except (OSError, ValueError, subprocess.SubprocessError):
        pass
    return d


def stream_read(torch, nbytes, steps=200):
    """Context for the decode rows: one launch of a plain streaming-read kernel
    (libwq_probe.so) over nbytes, rotating over >= 1 GiB of sources, timed like the
    layer (median of five runs)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "quantized_gemm_rtn_amd", "libwq_probe.so"))
    lib.wq_probe_stream_read.restype = ctypes.c_int
    lib.wq_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    nbytes = (nbytes + 15) // 16 * 16
    R = max(1, min(64, math.ceil(ROTATE_BYTES / nbytes)))
    bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device="cuda") for _ in range(R)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()

    def go(i):
        rc = lib.wq_probe_stream_read(ctypes.c_void_p(bufs[i % R].data_ptr()), nbytes,
                                      ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"wq_probe_stream_read returned {rc}")

    with torch.cuda.stream(stream):
        for i in range(R):
            go(i)
    torch.cuda.synchronize()
    runs = [timed_launches(torch, stream, go, steps) / steps for _ in range(5)]
    us = float(np.median(runs)) * 1e3
    del bufs
    torch.cuda.empty_cache()
    return {"bytes_read": nbytes, "us_per_launch": us, "GBps": nbytes / (us * 1e-6) / 1e9,
            "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}


def measure_offline(wq, torch, index):
    """Split + quantize + pack of one configuration's weights (offline, once per model)."""
    W, _, cfg = workloads.make(index, M=1)
    N, K = W.shape
    sk = workloads.sparse_k_for(cfg, N, K)
    Wd = torch.from_numpy(W).cuda()
    ws = torch.empty(max(1, wq.quantize_workspace_bytes(N, K, sk)), dtype=torch.uint8, device="cuda")
    for _ in range(2):
        q = wq.quantize_rtn(Wd, sparse_k=sk, workspace=ws)
        wq.pack(q["codes"])
    torch.cuda.synchronize()
    reps = 5
    t0 = time.perf_counter()
    for _ in range(reps):
        q = wq.quantize_rtn(Wd, sparse_k=sk, workspace=ws)
        wq.pack(q["codes"])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / reps * 1e3
    return dict(config=index, N=N, K=K, sparse_k=sk, ms=ms, weights_per_s=N * K / (ms * 1e-3))


DECODE_SOURCES = ("gemv_kernels.h", "gemv.hip", "wq_device.h")


def kernel_source_hash():
    """Short hash of the sources of the headline's decode kernel: a recorded traffic
    figure only describes the kernel it was measured on."""
    import hashlib
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        with open(os.path.join(ROOT, "quantized_gemm_rtn_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per launch of the decode kernel on the headline workload, from the
    committed rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE, calibrated on a
    device copy of known size), or None when that summary describes another
    version of the kernel."""
    path = os.path.join(ROOT, "profiles", "gemv_decode_7b_up_proj_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(budget_s=12.0):
    """The oracle's linear (fp64 dequantize + BLAS matmul) on the headline
    workload, on this host's cores, repeated until the time budget is spent."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    W, x, cfg = workloads.make(2)
    t0 = time.perf_counter()
    L = oracle.quantize_layer(W, 0)
    t_quant = time.perf_counter() - t0
    N, K = W.shape
    t0 = time.perf_counter()
    oracle.dequant(L["q"], L["s"], L["z"])
    t_deq = time.perf_counter() - t0
    times = []
    t_end = time.perf_counter() + budget_s
    while not times or time.perf_counter() < t_end:
        t0 = time.perf_counter()
        oracle.linear_ref(x, L["q"], L["s"], L["z"])
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    nb = alg_bytes(1, N, K, 0)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = ",".join(sorted({i.get("internal_api", "?") for i in threadpool_info() if i.get("user_api") == "blas"}))
    except Exception:  # pragma: no cover
        blas = "?"
    return {"value": nb / t / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"oracle linear_ref (fp64 dequantize + BLAS) on the full decode layer x[1,4096] "
                      f"W[11008,4096], median of {len(times)} runs ({t * 1e3:.1f} ms each)",
            "host": {"cpu_count": os.cpu_count(), "model": model, "blas": blas},
            "phases_ms": {"quantize_fp32": round(t_quant * 1e3, 1), "dequantize_fp64": round(t_deq * 1e3, 1),
                          "linear_ref": round(t * 1e3, 1)}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3000,
                    help="launches per timed run of the headline workload (the default spans about 20 ms)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--quick", action="store_true", help="headline workload only")
    ap.add_argument("--replays", type=int, default=5, help="timed runs per workload (median, p10, p90)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--workloads", default="", help="extra workloads as config:M[:kernel[:K[:rank[:mode]]]],... "
                    "(mode ao: an act-order layer; w8: the W4A8 product) "
                    "(default: the batched-decode, prefill and 70B-sweep set)")
    ap.add_argument("--no-offline", action="store_true", help="skip timing the offline quantizer")
    ap.add_argument("--rows-only", action="store_true",
                    help="time only the --workloads rows, each for --steps launches per run, and print them as one "
                         "JSON line (for per-row kernel traces and counters)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="run one device-to-device copy of BYTES first (reference for counter runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this layer needs no collective and the build targets a single "
              "MI355X; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_gemm_rtn_amd as wq
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    wq.load()
    if args.copy_calibration:
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.rows_only:
        out = []
        for item in args.workloads.split(","):
            f = item.split(":")
            mode = f[5] if len(f) > 5 else ""
            r = measure(wq, torch, int(f[0]), int(f[1]), args.steps, args.warmup,
                        kernel=f[2] if len(f) > 2 and f[2] else "auto", K=int(f[3]) if len(f) > 3 and f[3] else None,
                        replays=args.replays, rank=int(f[4]) if len(f) > 4 and f[4] else 0, mode=mode)
            print(f"# {item} {r['kernel']} {r['us_per_launch']:.2f} us {r['GBps']:.1f} GB/s "
                  f"{r['TFLOPs']:.1f} TF/s", file=sys.stderr, flush=True)
            out.append(r)
        print(json.dumps({"rows": out}), flush=True)
        return

    head = measure(wq, torch, 2, 1, args.steps, args.warmup, replays=args.replays)
    print(f"# headline 2:1 {head['kernel']} {head['us_per_launch']:.2f} us  {head['GBps']:.1f} GB/s "
          f"({100 * head['hbm_frac']:.1f}% of HBM peak)", file=sys.stderr, flush=True)
    rows = []
    offline = []
    if not args.quick:
        if args.workloads:
            plan = []
            for item in args.workloads.split(","):
                f = item.split(":")
                plan.append((int(f[0]), int(f[1]), f[2] if len(f) > 2 and f[2] else "auto",
                             int(f[3]) if len(f) > 3 and f[3] else None, int(f[4]) if len(f) > 4 and f[4] else 0,
                             f[5] if len(f) > 5 else ""))
        else:
            plan = [(3, 16, "auto", None, 0, ""), (4, 2048, "auto", None, 0, ""),
                    (5, 1, "auto", None, 0, ""), (5, 8, "auto", None, 0, ""),
                    (5, 64, "auto", None, 0, ""), (5, 512, "auto", None, 0, "")]
            # the other kernel on either side of the crossover, and the MFMA decode
            # kernel where a single row takes the single-row kernel
            for M in (8, 64):
                other = "gemm" if wq.auto_kernel(M, 8192, 28672) == "gemv" else "gemv"
                plan.append((5, M, other, None, 0, ""))
            plan.append((5, 1, "gemv_mfma", None, 0, ""))
            # one GPU's shard of the 70B down-projection split over 8 GPUs along K
            # (K / 8 = 3584 input channels, 28 groups)
            plan += [(5, 1, "auto", 3584, 0, ""), (5, 512, "auto", 3584, 0, "")]
            # the decode and prefill layers with a rank-32 low-rank branch, and as act-order layers
            plan += [(2, 1, "auto", None, 32, ""), (4, 2048, "auto", None, 32, ""),
                     (2, 1, "auto", None, 0, "ao"), (4, 2048, "auto", None, 0, "ao")]
            # the prefill layer as a W4A8 product with its 8 fp16 outlier channels
            plan += [(4, 2048, "auto", None, 0, "w8")]
            # the prefill layer and the 70B layer at M = 512 with CSR outliers at 0.45 %
            # of the weights (the dense-and-sparse prefill)
            plan += [(4, 2048, "auto", None, 0, "sp"), (5, 512, "auto", None, 0, "sp")]
            # the decode layers with 3-bit codes and with 64-channel groups
            plan += [(2, 1, "auto", None, 0, "b3"), (2, 1, "auto", None, 0, "g64"), (2, 1, "auto", None, 0, "b3g64"),
                     (5, 8, "auto", None, 0, "b3"), (4, 2048, "auto", None, 0, "b3")]
        for index, M, kern, Kov, rank, mode in plan:
            r = measure(wq, torch, index, M, None, args.warmup, kernel=kern, K=Kov, replays=args.replays,
                        rank=rank, mode=mode)
            rows.append(r)
            print(f"# {r['config']}:{r['M']}{'' if Kov is None else ' K=%d' % Kov}{' r=%d' % rank if rank else ''}"
                  f"{' act-order' if mode == 'ao' else ''}{' w4a8' if mode == 'w8' else ''}"
                  f"{' ' + mode if mode in ('b3', 'g64', 'b3g64', 'sp') else ''} "
                  f"{r['kernel']:4s} "
                  f"{r['us_per_launch']:9.2f} us  "
                  f"{r['GBps']:8.1f} GB/s ({100 * r['hbm_frac']:5.1f}%)  {r['TFLOPs']:7.1f} TF/s "
                  f"({100 * r['mfma_frac']:5.1f}%)", file=sys.stderr, flush=True)
    if not args.quick and not args.no_offline:
        for index in (2, 5):
            o = measure_offline(wq, torch, index)
            offline.append(o)
            print(f"# offline {o}", file=sys.stderr, flush=True)

    context = None
    if not args.quick:
        context = {"device": device_context(torch),
                   "stream_read_headline_bytes": stream_read(torch, alg_bytes(1, 11008, 4096, 0)),
                   "stream_read_70b_m1_bytes": stream_read(torch, alg_bytes(1, 8192, 28672, 117440)),
                   "torch_copy_headline_bytes": stream_copy(torch, alg_bytes(1, 11008, 4096, 0)),
                   "torch_copy_256MiB": stream_copy(torch, 256 << 20, steps=20)}
        print(f"# device (context): {context['device']}", file=sys.stderr, flush=True)
        for k in ("stream_read_headline_bytes", "stream_read_70b_m1_bytes"):
            c = context[k]
            print(f"# {k} (context): {c['us_per_launch']:.2f} us  {c['GBps']:.1f} GB/s "
                  f"({100 * c['hbm_frac']:.1f}%)", file=sys.stderr, flush=True)
        print(f"# torch copy (context): {context['torch_copy_headline_bytes']['GBps_read_plus_write']:.1f} GB/s "
              f"(read + write) at the headline size, "
              f"{context['torch_copy_256MiB']['GBps_read_plus_write']:.1f} GB/s at 256 MiB", file=sys.stderr, flush=True)
    cpu = None if args.no_cpu else cpu_baseline()
    us = head["us_per_launch"]
    line = {
        "metric": "W4A16 linear: decode GB/s (% HBM peak), prefill TFLOP/s (% MFMA peak)",
        "value": round(head["GBps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": us / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "decode GEMV, Llama-7B MLP up-proj: x fp16 [1,4096], W [11008,4096] "
                               "INT4 asym g128 packed 8/uint32, y fp16",
                   "M": 1, "N": 11008, "K": 4096, "group": 128, "kernel": head["kernel"],
                   "rotated_sets": head["rotated_sets"], "us_p10": round(head["us_p10"], 3),
                   "us_p90": round(head["us_p90"], 3), "replays": head["replays"]},
        "roofline": {"bound": "hbm", "achieved": round(head["GBps"], 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(head["hbm_frac"], 4), "traffic": recorded_traffic()},
        "cpu_baseline": cpu,
        "context": context,
        "workloads": rows,
        "offline": offline,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

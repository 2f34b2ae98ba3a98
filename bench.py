#!/usr/bin/env python3
"""Benchmark of the dense-GEMM library on one MI355X.

Headline: TFLOPS and fraction of the dense BF16 matrix-core peak for the FFN
projection C[1024,12288] = X[1024,4096] . W[4096,12288] (bf16 in, FP32
accumulation, bf16 out), and HBM GB/s of the M=1 decode shape.  The other
workloads (decode M=4/16, FP32 256^3 and 4096^3, batched attention scores,
the ragged 1000x12280x4100 GEMM) are reported in "workloads".

Timing: inputs are generated on the host from fixed seeds, copied to HBM, and
rotated over R buffer sets (R x working set >= 512 MiB) so that successive
calls cannot be served from the 256 MiB Infinity Cache.  After about a second
of untimed calls (clocks settle) and W warmup calls, each workload runs 7
batches of n back-to-back calls (n such that a batch lasts >= 20 ms and
7 n >= K for the headline), each batch bracketed by HIP events recorded on
the stream the kernels run on.  The time per call of a batch is its event
interval / n; reported are the median over the batches (the headline value)
with the minimum and maximum.  GPU clocks and power are read with rocm-smi
before and after the run; the host's CPU model is recorded with the oracle's
CPU times (all threads on a sample of the FFN projection, and one thread on
the FP32 256^3 product).

One JSON line is printed on stdout.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6    # 256 CUs x 4096 FLOP/clk x 2.4 GHz, dense
PEAK_F32_TFLOPS = 157.3      # FP32 matrix
PEAK_HBM_GBPS = 8000.0
PEAK_FP8_TFLOPS = 5033.2     # dense E4M3 matrix-core peak (2x bf16)
METRIC = "TFLOPS & % MFMA peak, BF16 1024x4096x12288; GB/s at M=1 decode"
KERNEL_SRC = os.path.join(ROOT, "dense_gemm_05_amd", "csrc", "g5_device.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_bf16_ms_256x192_ffn_1024x12288x4096_traffic.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class guarded:
    """Runs one workload so that a Python-level failure (a status error, a
    parity assertion) is logged and recorded under its name in `workloads`
    instead of ending the run: the JSON line, with every other workload, is
    still printed.  A fault that breaks the GPU context ends the process as
    before."""

    def __init__(self, name, workloads):
        self.name, self.workloads = name, workloads

    def __enter__(self):
        return self

    def __exit__(self, et, ev, tb):
        if et is None or not issubclass(et, Exception):
            return False
        import traceback
        traceback.print_exception(et, ev, tb, file=sys.stderr)
        log(f"{self.name}: FAILED ({et.__name__}: {ev})")
        self.workloads.append({"name": self.name, "error": f"{et.__name__}: {ev}"})
        return True


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--only", default="all", choices=["all", "ffn", "decode", "decode_swiglu", "sgemm", "batched", "ragged", "swiglu", "shard", "fp8", "scores_nt", "decode_nt", "fp8_example_5_8", "square", "affine", "linear_nt", "wgrad_tn", "act_chain", "copy"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--batches", type=int, default=7, help="timed batches per workload (median reported)")
    ap.add_argument("--batch-ms", type=float, default=20.0, help="minimum length of a timed batch")
    ap.add_argument("--prewarm-seconds", type=float, default=1.0,
                    help="untimed calls before each workload's warmup, so that GPU clocks settle")
    return ap.parse_args()


def gpu_clocks():
    """Clock levels and power of GPU 0 as rocm-smi reports them (None fields
    when the tool is missing or fails; it runs as a child process)."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "-d", "0", "--showclocks", "--showpower", "--showperflevel", "--json"],
                           capture_output=True, text=True, timeout=30)
        data = json.loads(r.stdout)
        card = next(iter(data.values())) if isinstance(data, dict) and data else {}
        return {"time": time.strftime("%H:%M:%S"), **{k.strip(): v for k, v in card.items()}}
    except Exception as e:  # noqa: BLE001 -- a missing tool must not stop the benchmark
        return {"time": time.strftime("%H:%M:%S"), "error": f"{type(e).__name__}: {e}"}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def kernel_label(plan):
    """Kernel template a BF16 tiled plan launches (as in launch_bf16)."""
    name = plan.name.decode()
    tm, tn = plan.tile_m, plan.tile_n
    if plan.family == 2 and plan.variant in (1, 2, 3):
        av, masked = {1: (16, "false"), 2: (16, "true"), 3: (4, "true")}[plan.variant]
        wg = "2,4" if tm == 256 and tn in (192, 256) else "4,2"
        sk = "true" if plan.ksplit > 1 else "false"
        return (f"k_bf16_ms<{tm},{tn},{wg},4,4,{av},{masked},0,{sk},false,false,false> ({name}, grid {plan.grid}, "
                f"{plan.threads} threads)")
    return f"{name} variant {plan.variant} (grid {plan.grid}, {plan.threads} threads)"


def kernel_hash():
    """Hash of the source the FFN kernel is built from: the device header
    holding the shared helpers and the LDS-ring kernel with its epilogue
    (edits to the other kernels leave stored counter readings valid)."""
    with open(KERNEL_SRC, encoding="utf-8") as fh:
        return hashlib.sha256(fh.read().encode()).hexdigest()[:16]


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        msg = ("bench.py measures one GPU only: this library has no multi-GPU path "
               "(each GPU would run its own shard of the GEMM; see the sharding notes). Use --gpus 1.")
        print(json.dumps({"error": msg, "n_gpus": args.gpus}))
        print(msg, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gemm_inputs as gi
    from __graft_entry__ import _ensure_built
    _ensure_built()
    import dense_gemm_05_amd as g5

    clocks_before = gpu_clocks()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    # caller-owned scratch for the paths that split K over workgroups or
    # realign rows (one stream, so one workspace serves every call)
    ws = g5.Workspace(dev)

    def to_dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    timings = {}

    def timed(fn_list, steps, warmup, prewarm=None, label=None):
        """fn_list: one closure per buffer set.  Returns the median ms per call.

        Before the W warmup calls, the workload runs untimed for about
        `prewarm` seconds: the GPU's clocks take a fraction of a second of
        sustained load to settle, and the first hundreds of microseconds of
        calls otherwise run measurably slower than the steady state.

        Then `batches` batches of n back-to-back calls are each bracketed by
        HIP events on the stream the calls run on, with n chosen so that a
        batch lasts at least `batch_ms` (from a probe after the warmup) and
        n x batches >= steps.  The time per call of a batch is its event
        interval / n; the median over the batches is returned and the
        median, minimum and maximum are kept under `label`, with the host's
        own enqueue time per call (a host time close to the device time would
        mean the GPU waits for the host)."""
        R = len(fn_list)
        t_end = time.time() + (args.prewarm_seconds if prewarm is None else prewarm)
        i = 0
        while time.time() < t_end:
            for _ in range(20):
                fn_list[i % R]()
                i += 1
            torch.cuda.synchronize()
        for i in range(warmup):
            fn_list[i % R]()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        # batch size: grown from a probe until one untimed batch lasts
        # batch_ms (a short probe overestimates the steady-state time)
        n = max(10, min(200, warmup))
        for _ in range(4):
            e0.record(stream)
            for i in range(n):
                fn_list[i % R]()
            e1.record(stream)
            torch.cuda.synchronize()
            took = e0.elapsed_time(e1)
            if took >= args.batch_ms:
                break
            n = int(n * args.batch_ms * 1.1 / max(took, 1e-3)) + 1
        nb = args.batches
        n = max(-(-steps // nb), n)
        per_call, host = [], []
        for b in range(nb):
            e0.record(stream)
            h0 = time.perf_counter()
            for i in range(n):
                fn_list[i % R]()
            h1 = time.perf_counter()
            e1.record(stream)
            torch.cuda.synchronize()
            per_call.append(e0.elapsed_time(e1) / n)
            host.append((h1 - h0) * 1e3 / n)
        srt = sorted(per_call)
        med = srt[nb // 2] if nb % 2 else 0.5 * (srt[nb // 2 - 1] + srt[nb // 2])
        if label is not None:
            timings[label] = {"median_us": round(med * 1e3, 3), "min_us": round(srt[0] * 1e3, 3),
                              "max_us": round(srt[-1] * 1e3, 3), "batches": nb, "calls_per_batch": n,
                              "batch_ms_median": round(med * n, 2),
                              "host_enqueue_us_per_call": round(min(host) * 1e3, 3)}
            if min(host) > 0.9 * med:
                log(f"{label}: host enqueue {min(host) * 1e3:.1f} us/call is close to the device time "
                    f"{med * 1e3:.1f} us: the GPU may be waiting for the host")
        return med

    def rotations(set_bytes):
        return min(64, max(1, -(-512 * 2 ** 20 // set_bytes)))

    out = {"metric": METRIC, "value": None, "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded; N(0,1) X, N(0,1/64) W)",
           "config": {"workload": "bf16 FFN projection X[1024,4096] . W[4096,12288] -> C bf16, FP32 accumulate",
                      "M": 1024, "N": 12288, "K": 4096, "global_batch": 1024, "parallelism": "single GPU"}}
    workloads = []
    ffn_rows_gpu = None

    if args.only == "copy":
        # Calibration for HBM byte counters: a plain device-to-device copy of
        # 1 GiB (torch's copy kernel) reads and writes exactly 1 GiB.
        n = 1 << 28
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy: 3 x 1 GiB device copies done")
        print(json.dumps({"copy_bytes_per_launch": 4 * n, "launches": 3}))
        return

    # ------------------------------------------------------------ FFN (headline)
    if args.only in ("all", "ffn"):
        with guarded("ffn", workloads):
            M, N, K = 1024, 12288, 4096
            log("FFN: generating inputs")
            X, W = gi.ffn_inputs(M, K, N)
            R = rotations(2 * (M * K + K * N + M * N))
            dX = [to_dev_bf16(X) for _ in range(R)]
            dW = [to_dev_bf16(W) for _ in range(R)]
            dC = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
            fns = [(lambda i=i: g5.gemm_bf16(dX[i], dW[i], dC[i], workspace=ws)) for i in range(R)]
            st, plan = g5.plan_query(g5.GEMM_OP_BF16, M, N, K)
            ms = timed(fns, args.steps, args.warmup, label="ffn_bf16_1024x12288x4096")
            flops = 2.0 * M * N * K
            tflops = flops / (ms * 1e-3) / 1e12
            log(f"FFN: {ms * 1e3:.2f} us/call, {tflops:.1f} TFLOPS ({100 * tflops / PEAK_BF16_TFLOPS:.1f}% of peak), "
                f"config {plan.name.decode()}, R={R}")
            tm = timings["ffn_bf16_1024x12288x4096"]
            out["value"] = round(tflops, 2)
            out["value_min"] = round(flops / (tm["max_us"] * 1e-6) / 1e12, 2)
            out["value_max"] = round(flops / (tm["min_us"] * 1e-6) / 1e12, 2)
            out["ms_per_step"] = round(ms, 5)
            out["steps"] = tm["batches"] * tm["calls_per_batch"]
            out["timing"] = {"batches": tm["batches"], "calls_per_batch": tm["calls_per_batch"],
                             "median_us": tm["median_us"], "min_us": tm["min_us"], "max_us": tm["max_us"],
                             "statistic": "median over batches of (event interval / calls)"}
            traffic = None
            if os.path.exists(TRAFFIC_FILE):
                with open(TRAFFIC_FILE) as fh:
                    tr = json.load(fh)
                if tr.get("kernel_sha256_16") == kernel_hash():
                    traffic = tr.get("hbm_bytes_per_launch")
            out["roofline"] = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                               "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                               "kernel": kernel_label(plan),
                               "flops_per_launch": flops}
            workloads.append({"name": "ffn_bf16_1024x12288x4096", "us": round(ms * 1e3, 3),
                              "tflops": round(tflops, 2), "frac_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
                              "config": plan.name.decode(), "rotations": R})
            ffn_rows_gpu = (X, W, dC[(args.steps - 1) % R])

    # ------------------------------------------------------------ decode
    if args.only in ("all", "decode"):
        with guarded("decode", workloads):
            N, K = 12288, 4096
            for M in (1, 4, 16):
                X, W = gi.decode_inputs(M, K, N)
                alg_bytes = 2 * (M * K + K * N + M * N)
                R = rotations(alg_bytes)
                dX = [to_dev_bf16(X) for _ in range(R)]
                dW = [to_dev_bf16(W) for _ in range(R)]
                dC = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
                fns = [(lambda i=i: g5.gemm_bf16(dX[i], dW[i], dC[i], workspace=ws)) for i in range(R)]
                ms = timed(fns, max(200, args.steps), args.warmup, label=f"decode_bf16_m{M}_12288x4096")
                gbps = alg_bytes / (ms * 1e-3) / 1e9
                log(f"decode M={M}: {ms * 1e3:.2f} us/call, {gbps:.0f} GB/s ({100 * gbps / PEAK_HBM_GBPS:.1f}% of HBM)")
                rec = {"name": f"decode_bf16_m{M}_12288x4096", "us": round(ms * 1e3, 3), "GBps": round(gbps, 1),
                       "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4), "alg_bytes": alg_bytes, "rotations": R}
                workloads.append(rec)
                if M == 1:
                    out["decode_m1"] = {"GBps": round(gbps, 1), "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4),
                                        "us": round(ms * 1e3, 3), "alg_bytes": alg_bytes}
                del dX, dW, dC

    # ------------------------------------------------------------ decode through the fused SwiGLU
    if args.only in ("all", "decode_swiglu"):
        with guarded("decode_swiglu", workloads):
            # One token through the FFN's gate and up projections with the merged
            # weight Wgu [4096, 2 x 12288] and the SwiGLU product applied as the
            # small-M kernels store, next to the plain product of the same token
            # with the same merged weight (the same 192 MiB read, 24576 bf16
            # outputs): the fusion's cost over the bytes it has to read.
            N, K = 12288, 4096
            X, Wgu = gi.swiglu_inputs(16, K, N)
            for M in (1, 16):
                Xm = np.ascontiguousarray(X[:M])
                alg_bytes = 2 * (M * K + K * 2 * N + M * N)
                R = rotations(alg_bytes)
                dX = [to_dev_bf16(Xm) for _ in range(R)]
                dW = [to_dev_bf16(Wgu) for _ in range(R)]
                dZ = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
                dQ = [torch.empty((M, N), dtype=torch.uint8, device=dev) for _ in range(R)]
                dP = [torch.empty((M, 2 * N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
                fused = [(lambda i=i: g5.gemm_bf16_swiglu(dX[i], dW[i], dZ[i], workspace=ws)) for i in range(R)]
                fused8 = [(lambda i=i: g5.gemm_bf16_swiglu_e4m3(dX[i], dW[i], 16.0, dQ[i], workspace=ws))
                          for i in range(R)]
                fused_nows = [(lambda i=i: g5.gemm_bf16_swiglu(dX[i], dW[i], dZ[i])) for i in range(R)]
                plain = [(lambda i=i: g5.gemm_bf16(dX[i], dW[i], dP[i], workspace=ws)) for i in range(R)]
                ms = timed(fused, 200, args.warmup, label=f"decode_swiglu_m{M}_2x12288x4096")
                ms_n = timed(fused_nows, 200, args.warmup, label=f"decode_swiglu_m{M}_no_workspace")
                ms_p = timed(plain, 200, args.warmup, label=f"decode_plain_merged_m{M}_24576x4096")
                ms8 = timed(fused8, 200, args.warmup, label=f"decode_swiglu_e4m3_m{M}")
                gbps = alg_bytes / (ms * 1e-3) / 1e9
                log(f"decode SwiGLU M={M}: fused {ms * 1e3:.2f} us ({gbps:.0f} GB/s), without workspace "
                    f"{ms_n * 1e3:.2f} us; plain product with the merged weight {ms_p * 1e3:.2f} us "
                    f"(fused / plain {ms / ms_p:.3f}); E4M3FN output {ms8 * 1e3:.2f} us")
                workloads.append({"name": f"decode_swiglu_bf16_m{M}_2x12288x4096", "us": round(ms * 1e3, 3),
                                  "GBps": round(gbps, 1), "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4),
                                  "no_workspace_us": round(ms_n * 1e3, 3),
                                  "plain_merged_product_us": round(ms_p * 1e3, 3),
                                  "fused_over_plain": round(ms / ms_p, 4), "e4m3_output_us": round(ms8 * 1e3, 3),
                                  "alg_bytes": alg_bytes, "rotations": R})
                del dX, dW, dZ, dP, dQ

    # ------------------------------------------------------------ decode with a linear layer's weight
    if args.only in ("all", "decode_nt"):
        with guarded("decode_nt", workloads):
            # The same decode rows against W stored as a linear layer's weight,
            # Wt [12288, 4096]: a GEMV over the contiguous rows of Wt.
            N, K = 12288, 4096
            for M in (1, 4, 16):
                X, W = gi.decode_inputs(M, K, N)
                Wt = np.ascontiguousarray(W.T)
                alg_bytes = 2 * (M * K + K * N + M * N)
                R = rotations(alg_bytes)
                dX = [to_dev_bf16(X) for _ in range(R)]
                dW = [to_dev_bf16(Wt) for _ in range(R)]
                dC = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
                fns = [(lambda i=i: g5.gemm_bf16_nt(dX[i], dW[i], dC[i], workspace=ws)) for i in range(R)]
                ms = timed(fns, max(200, args.steps), args.warmup, label=f"decode_nt_bf16_m{M}_12288x4096")
                gbps = alg_bytes / (ms * 1e-3) / 1e9
                log(f"decode NT M={M}: {ms * 1e3:.2f} us/call, {gbps:.0f} GB/s ({100 * gbps / PEAK_HBM_GBPS:.1f}% of HBM)")
                workloads.append({"name": f"decode_nt_bf16_m{M}_12288x4096", "us": round(ms * 1e3, 3),
                                  "GBps": round(gbps, 1), "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4),
                                  "alg_bytes": alg_bytes, "rotations": R})
                del dX, dW, dC

    # ------------------------------------------------------------ FP32
    if args.only in ("all", "sgemm"):
        with guarded("sgemm", workloads):
            for n, wl, steps in ((256, gi.W_SGEMM_SMALL, 500), (4096, gi.W_SGEMM_LARGE, 20)):
                A, B = gi.sgemm_inputs(n, workload=wl)
                R = rotations(4 * 3 * n * n)
                dA = [torch.from_numpy(A).to(dev) for _ in range(R)]
                dB = [torch.from_numpy(B).to(dev) for _ in range(R)]
                dC = [torch.empty((n, n), device=dev) for _ in range(R)]
                fns = [(lambda i=i: g5.gemm_sgemm(dA[i], dB[i], dC[i])) for i in range(R)]
                ms = timed(fns, steps, 5, label=f"sgemm_f32_{n}^3")
                tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
                log(f"sgemm {n}^3: {ms * 1e3:.2f} us/call, {tf:.1f} TFLOPS ({100 * tf / PEAK_F32_TFLOPS:.1f}% of fp32 peak)")
                workloads.append({"name": f"sgemm_f32_{n}^3", "us": round(ms * 1e3, 3), "tflops": round(tf, 2),
                                  "frac_peak": round(tf / PEAK_F32_TFLOPS, 4), "rotations": R})
                del dA, dB, dC

    # ------------------------------------------------------------ bf16 square
    if args.only in ("all", "square"):
        with guarded("square", workloads):
            # bf16 4096^3 -> bf16: 256 tiles of 256x256, one per CU.
            n = 4096
            g = np.random.default_rng([gi.SEED_BASE + 900, n])
            A = gi.to_bf16_bits(gi.normal(g, (n, n)))
            B = gi.to_bf16_bits(gi.normal(g, (n, n), 0.125))
            R = rotations(2 * 3 * n * n)
            dA = [to_dev_bf16(A) for _ in range(R)]
            dB = [to_dev_bf16(B) for _ in range(R)]
            dC = [torch.empty((n, n), dtype=torch.bfloat16, device=dev) for _ in range(R)]
            fns = [(lambda i=i: g5.gemm_bf16(dA[i], dB[i], dC[i], workspace=ws)) for i in range(R)]
            st, plan = g5.plan_query(g5.GEMM_OP_BF16, n, n, n)
            ms = timed(fns, 50, 10, label="square_bf16_4096^3")
            tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
            log(f"bf16 4096^3: {ms * 1e3:.2f} us/call, {tf:.1f} TFLOPS ({100 * tf / PEAK_BF16_TFLOPS:.1f}%), "
                f"{plan.name.decode()}")
            workloads.append({"name": "square_bf16_4096^3", "us": round(ms * 1e3, 3), "tflops": round(tf, 2),
                              "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4), "config": plan.name.decode(),
                              "rotations": R})
            del dA, dB, dC

    # ------------------------------------------------------------ batched
    if args.only in ("all", "batched"):
        with guarded("batched", workloads):
            Q, KT = gi.batched_inputs()
            bt, M, K = Q.shape
            N = KT.shape[2]
            alg_bytes = 2 * Q.size + 2 * KT.size + 4 * bt * M * N
            R = rotations(alg_bytes)
            dQ = [to_dev_bf16(Q) for _ in range(R)]
            dK = [to_dev_bf16(KT) for _ in range(R)]
            dC = [torch.empty((bt, M, N), device=dev) for _ in range(R)]
            fns = [(lambda i=i: g5.gemm_bf16_batched(dQ[i], dK[i], dC[i], workspace=ws)) for i in range(R)]
            ms = timed(fns, 100, 10, label="batched_bf16_32x1024x1024x128_f32out")
            flops = 2.0 * bt * M * N * K
            t_roof = max(flops / (PEAK_BF16_TFLOPS * 1e12), alg_bytes / (PEAK_HBM_GBPS * 1e9))
            gbps = alg_bytes / (ms * 1e-3) / 1e9
            log(f"batched 32x1024x1024x128: {ms * 1e3:.2f} us/call, {gbps:.0f} GB/s, roofline frac {t_roof / (ms * 1e-3):.3f}")
            workloads.append({"name": "batched_bf16_32x1024x1024x128_f32out", "us": round(ms * 1e3, 3),
                              "GBps": round(gbps, 1), "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                              "frac_roofline": round(t_roof / (ms * 1e-3), 4), "alg_bytes": alg_bytes, "rotations": R})
            del dQ, dK, dC

    # ------------------------------------------------------------ ragged
    if args.only in ("all", "ragged"):
        with guarded("ragged", workloads):
            A, B = gi.ragged_inputs()
            M, K = A.shape
            N = B.shape[1]
            R = rotations(2 * (M * K + K * N) + 4 * M * N)
            dA = [to_dev_bf16(A) for _ in range(R)]
            dB = [to_dev_bf16(B) for _ in range(R)]
            dC = [torch.empty((M, N), device=dev) for _ in range(R)]
            fns = [(lambda i=i: g5.gemm_bf16(dA[i], dB[i], dC[i], workspace=ws)) for i in range(R)]
            ms = timed(fns, 30, 5, label="ragged_bf16_1000x12280x4100_f32out")
            tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
            log(f"ragged 1000x12280x4100: {ms * 1e3:.2f} us/call, {tf:.1f} TFLOPS ({100 * tf / PEAK_BF16_TFLOPS:.1f}%)")
            workloads.append({"name": "ragged_bf16_1000x12280x4100_f32out", "us": round(ms * 1e3, 3),
                              "tflops": round(tf, 2), "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4), "rotations": R})
            del dA, dB, dC

    # ------------------------------------------------------------ fused SwiGLU FFN
    if args.only in ("all", "swiglu"):
        with guarded("swiglu", workloads):
            # The FFN's gate and up projections of X with one merged weight
            # [4096, 2 x 12288] and the SwiGLU product in the epilogue, next to
            # the same two projections as plain calls (bf16 g and u written out).
            M, N, K = 1024, 12288, 4096
            X, Wgu = gi.swiglu_inputs(M, K, N)
            alg_bytes = 2 * (M * K + K * 2 * N + M * N)
            R = rotations(alg_bytes)
            dX = [to_dev_bf16(X) for _ in range(R)]
            dW = [to_dev_bf16(Wgu) for _ in range(R)]
            dZ = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
            dG = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
            dU = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
            fused = [(lambda i=i: g5.gemm_bf16_swiglu(dX[i], dW[i], dZ[i], workspace=ws)) for i in range(R)]
            plain = [(lambda i=i: (g5.gemm_bf16(dX[i], dW[i][:, :N], dG[i], workspace=ws), g5.gemm_bf16(dX[i], dW[i][:, N:], dU[i], workspace=ws)))
                     for i in range(R)]
            # The unfused program: the two projections, then Z = bf16(bf16(SiLU(g)) * u)
            # as the activation chain's separate passes over the written g and u
            # (SiLU, then the product: the same roundings as the fused epilogue).
            dT = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
            unfused = [(lambda i=i: (plain[i](), g5.act_silu(dG[i], dT[i]), g5.act_mul(dT[i], dU[i], dZ[i])))
                       for i in range(R)]
            # Z stored as E4M3FN codes against a fixed range (the page's
            # continuation of the example): fused into the same epilogue, next
            # to the bf16 SwiGLU followed by the separate quantization pass
            # (the activation chain's quantization step: the same codes).
            amax = 16.0
            dQ = [torch.empty((M, N), dtype=torch.uint8, device=dev) for _ in range(R)]
            fused8 = [(lambda i=i: g5.gemm_bf16_swiglu_e4m3(dX[i], dW[i], amax, dQ[i], workspace=ws)) for i in range(R)]
            quant_after = [(lambda i=i: (fused[i](), g5.act_quantize_e4m3(dZ[i], amax, dQ[i]))) for i in range(R)]
            ms = timed(fused, 30, 5, label="swiglu_ffn_bf16_1024x2x12288x4096")
            ms_plain = timed(plain, 30, 5, label="swiglu_ffn_two_plain_projections")
            ms_unfused = timed(unfused, 30, 5, label="swiglu_ffn_unfused_program")
            ms8 = timed(fused8, 30, 5, label="swiglu_ffn_e4m3_1024x2x12288x4096")
            ms_qa = timed(quant_after, 30, 5, label="swiglu_ffn_bf16_then_quantize")
            flops = 2.0 * 2 * M * N * K
            tf = flops / (ms * 1e-3) / 1e12
            tf8 = flops / (ms8 * 1e-3) / 1e12
            log(f"swiglu FFN 1024x(2x12288)x4096: fused {ms * 1e3:.2f} us ({tf:.1f} TFLOPS); "
                f"two plain projections {ms_plain * 1e3:.2f} us; unfused program (projections + element-wise "
                f"SiLU and product) {ms_unfused * 1e3:.2f} us; E4M3FN output fused {ms8 * 1e3:.2f} us "
                f"({tf8:.1f} TFLOPS), bf16 output then a separate quantization {ms_qa * 1e3:.2f} us")
            workloads.append({"name": "swiglu_ffn_bf16_1024x2x12288x4096", "us": round(ms * 1e3, 3),
                              "tflops": round(tf, 2), "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                              "two_plain_projections_us": round(ms_plain * 1e3, 3),
                              "unfused_program_us": round(ms_unfused * 1e3, 3), "rotations": R})
            workloads.append({"name": "swiglu_ffn_e4m3_1024x2x12288x4096", "us": round(ms8 * 1e3, 3),
                              "tflops": round(tf8, 2), "frac_peak": round(tf8 / PEAK_BF16_TFLOPS, 4),
                              "bf16_output_us": round(ms * 1e3, 3),
                              "bf16_then_quantize_us": round(ms_qa * 1e3, 3), "amax": amax, "rotations": R})
            del dX, dW, dZ, dG, dU, dQ, dT

    # ------------------------------------------------------------ the activation chain (Example 5-4)
    if args.only in ("all", "act_chain"):
        with guarded("act_chain", workloads):
            # The activation chain on stored G and U [1024, 12288] (bf16, 24 MiB
            # each): T = SiLU(G), Z = T (.) U and Z quantized to one byte, as
            # separate passes and fused.  Each program's bytes are the page's
            # accounting of the tensors it reads and writes once.
            M, N = 1024, 12288
            G, U = gi.act_chain_inputs(M, N)
            E = 2 * M * N                                  # one bf16 tensor
            R = rotations(3 * E)
            dG = [to_dev_bf16(G) for _ in range(R)]
            dU = [to_dev_bf16(U) for _ in range(R)]
            dT = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
            dZ = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
            dQ = [torch.empty((M, N), dtype=torch.uint8, device=dev) for _ in range(R)]
            amax = 256.0
            # each program's bytes: the library's per-call model summed over its calls
            mb = lambda *steps: int(sum(g5.lib().gemm_model_act_chain_bytes(st, M, N) for st in steps))
            S, P, F, Q, F3 = (g5.GEMM_ACT_SILU, g5.GEMM_ACT_MUL, g5.GEMM_ACT_SWIGLU, g5.GEMM_ACT_QUANT,
                              g5.GEMM_ACT_SWIGLU_E4M3)
            progs = [
                ("silu_then_product", mb(S, P),
                 lambda i: (g5.act_silu(dG[i], dT[i]), g5.act_mul(dT[i], dU[i], dZ[i]))),
                ("fused_silu_product", mb(F), lambda i: g5.act_swiglu(dG[i], dU[i], dZ[i])),
                ("three_steps", mb(S, P, Q),
                 lambda i: (g5.act_silu(dG[i], dT[i]), g5.act_mul(dT[i], dU[i], dZ[i]),
                            g5.act_quantize_e4m3(dZ[i], amax, dQ[i]))),
                ("fused_two_then_quantize", mb(F, Q),
                 lambda i: (g5.act_swiglu(dG[i], dU[i], dZ[i]), g5.act_quantize_e4m3(dZ[i], amax, dQ[i]))),
                ("fused_three", mb(F3), lambda i: g5.act_swiglu_e4m3(dG[i], dU[i], amax, dQ[i])),
            ]
            res = {}
            for name, nbytes, fn in progs:
                ms = timed([(lambda i=i, fn=fn: fn(i)) for i in range(R)], 200, args.warmup,
                           label=f"act_chain_{name}")
                res[name] = (ms * 1e3, nbytes / (ms * 1e-3) / 1e9, nbytes)
            log("activation chain 1024x12288 (Example 5-4): " + "; ".join(
                f"{k} {v[0]:.2f} us ({v[2] / 2**20:.0f} MiB, {v[1]:.0f} GB/s)" for k, v in res.items()))
            f2, u2 = res["fused_silu_product"], res["silu_then_product"]
            f3, u3 = res["fused_three"], res["three_steps"]
            workloads.append({"name": "act_chain_example_5_4_1024x12288",
                              "us": round(f2[0], 3), "GBps": round(f2[1], 1), "frac_hbm": round(f2[1] / PEAK_HBM_GBPS, 4),
                              "programs": {k: {"us": round(v[0], 3), "GBps": round(v[1], 1),
                                               "MiB": round(v[2] / 2**20, 1)} for k, v in res.items()},
                              "fused_over_separate_two_steps": round(f2[0] / u2[0], 4),
                              "page_traffic_ratio_two_steps": round(mb(F) / mb(S, P), 4),
                              "fused_over_separate_three_steps": round(f3[0] / u3[0], 4),
                              "page_traffic_ratio_three_steps": round(mb(F3) / mb(S, P, Q), 4),
                              "amax": amax, "rotations": R})
            del dG, dU, dT, dZ, dQ

    # ------------------------------------------------------------ column shard (split K)
    if args.only in ("all", "shard"):
        with guarded("shard", workloads):
            # The 1024x1536x4096 shard of an 8-way column split of the FFN
            # projection: 96 tiles of 128x128 for 256 CUs, so K is split over
            # workgroups.
            M, N, K = 1024, 1536, 4096
            X, W = gi.ffn_inputs()
            W = np.ascontiguousarray(W[:, :N])
            R = rotations(2 * (M * K + K * N + M * N))
            dX = [to_dev_bf16(X) for _ in range(R)]
            dW = [to_dev_bf16(W) for _ in range(R)]
            dC = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
            fns = [(lambda i=i: g5.gemm_bf16(dX[i], dW[i], dC[i], workspace=ws)) for i in range(R)]
            st, plan = g5.plan_query(g5.GEMM_OP_BF16, M, N, K)
            ms = timed(fns, 100, 10, label="shard_bf16_1024x1536x4096")
            tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
            log(f"shard 1024x1536x4096: {ms * 1e3:.2f} us/call, {tf:.1f} TFLOPS, {plan.name.decode()} ksplit {plan.ksplit}")
            workloads.append({"name": "shard_bf16_1024x1536x4096", "us": round(ms * 1e3, 3), "tflops": round(tf, 2),
                              "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4), "config": plan.name.decode(),
                              "ksplit": plan.ksplit, "rotations": R})
            del dX, dW, dC

    # ------------------------------------------------------------ FP8 FFN
    if args.only in ("all", "fp8"):
        with guarded("fp8", workloads):
            # The FFN projection in E4M3FN: W^T [12288,4096] quantized per output
            # channel once (weights), X quantized per token on every call, then
            # the scaled FP8 product into bf16.
            M, N, K = 1024, 12288, 4096
            X, W = gi.ffn_inputs()
            Wt = np.ascontiguousarray(W.T)
            R = rotations(M * K * 3 + N * K + 2 * M * N)
            dX = [to_dev_bf16(X) for _ in range(R)]
            qW = [g5.gemm_fp8_quantize_rows(to_dev_bf16(Wt)) for _ in range(R)]
            qX = [g5.gemm_fp8_quantize_rows(dX[i]) for i in range(R)]
            dC = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
            gemm = [(lambda i=i: g5.gemm_fp8_nt(qX[i][0], qX[i][1], qW[i][0], qW[i][1], dC[i], workspace=ws)) for i in range(R)]
            quant = [(lambda i=i: g5.gemm_fp8_quantize_rows(dX[i], qX[i][0], qX[i][1])) for i in range(R)]
            both = [(lambda i=i: (g5.gemm_fp8_quantize_rows(dX[i], qX[i][0], qX[i][1]),
                                  g5.gemm_fp8_nt(qX[i][0], qX[i][1], qW[i][0], qW[i][1], dC[i], workspace=ws))) for i in range(R)]
            ms_g = timed(gemm, 50, 10, label="fp8_ffn_e4m3_1024x12288x4096")
            ms_q = timed(quant, 100, 10, label="fp8_quantize_x_1024x4096")
            ms_b = timed(both, 50, 10, label="fp8_quantize_and_gemm")
            fl = 2.0 * M * N * K
            tf = fl / (ms_g * 1e-3) / 1e12
            log(f"fp8 FFN: GEMM {ms_g * 1e3:.2f} us ({tf:.1f} TFLOPS, {tf / PEAK_FP8_TFLOPS:.3f} of fp8 peak); "
                f"quantize X {ms_q * 1e3:.2f} us; both {ms_b * 1e3:.2f} us")
            workloads.append({"name": "fp8_ffn_e4m3_1024x12288x4096", "us": round(ms_g * 1e3, 3), "tflops": round(tf, 2),
                              "frac_peak": round(tf / PEAK_FP8_TFLOPS, 4), "peak": PEAK_FP8_TFLOPS,
                              "quantize_x_us": round(ms_q * 1e3, 3), "quantize_and_gemm_us": round(ms_b * 1e3, 3),
                              "rotations": R})
            del dX, qX, dC
            # decode with the FP8 weight: M rows of X quantized, the GEMV over Wt's codes
            for Md in (1, 16):
                Xd, _ = gi.decode_inputs(Md, K, N)
                alg = N * K + Md * K + 4 * Md + 4 * N + 2 * Md * N        # codes, factors, bf16 C
                Rd = rotations(alg)
                qW2 = [qW[i % R] for i in range(Rd)]
                qXd = [g5.gemm_fp8_quantize_rows(to_dev_bf16(Xd)) for _ in range(Rd)]
                dCd = [torch.empty((Md, N), dtype=torch.bfloat16, device=dev) for _ in range(Rd)]
                fns = [(lambda i=i: g5.gemm_fp8_nt(qXd[i][0], qXd[i][1], qW2[i][0], qW2[i][1], dCd[i], workspace=ws)) for i in range(Rd)]
                ms_d = timed(fns, 200, 10, label=f"fp8_decode_m{Md}_12288x4096")
                gbps = alg / (ms_d * 1e-3) / 1e9
                log(f"fp8 decode M={Md}: {ms_d * 1e3:.2f} us/call, {gbps:.0f} GB/s ({100 * gbps / PEAK_HBM_GBPS:.1f}% of HBM)")
                workloads.append({"name": f"fp8_decode_m{Md}_12288x4096", "us": round(ms_d * 1e3, 3), "GBps": round(gbps, 1),
                                  "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4), "alg_bytes": alg, "rotations": Rd})
                del qXd, dCd, qW2
            del qW

    # ------------------------------------------------------------ FP8, Example 5-8's shape
    if args.only in ("all", "fp8_example_5_8"):
        with guarded("fp8_example_5_8", workloads):
            # A [4096, 4096] (bf16 here, fp16 on the page) quantized per row on
            # every call, then multiplied by an FP8 weight stored [4096, 1536]
            # (quantized per output column once, into Bt), 16-bit output: the
            # separate quantization the page's traffic count favours (444 MiB
            # with 128x128 tiles, against 620 MiB fused into the GEMM).
            import ctypes
            M, N, K = 4096, 1536, 4096
            g = np.random.default_rng([gi.SEED_BASE + 7400])
            X = gi.to_bf16_bits(gi.normal(g, (M, K)))
            W = gi.to_bf16_bits(gi.normal(g, (K, N), 0.125))
            R = rotations(2 * M * K + M * K + K * N + 2 * M * N)
            dX = [to_dev_bf16(X) for _ in range(R)]
            qW = [g5.gemm_fp8_quantize_cols(to_dev_bf16(W)) for _ in range(R)]
            qX = [g5.gemm_fp8_quantize_rows(dX[i]) for i in range(R)]
            dC = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
            both = [(lambda i=i: (g5.gemm_fp8_quantize_rows(dX[i], qX[i][0], qX[i][1]),
                                  g5.gemm_fp8_nt(qX[i][0], qX[i][1], qW[i][0], qW[i][1], dC[i], workspace=ws)))
                    for i in range(R)]
            gemm = [(lambda i=i: g5.gemm_fp8_nt(qX[i][0], qX[i][1], qW[i][0], qW[i][1], dC[i], workspace=ws))
                    for i in range(R)]
            sxf = [torch.empty((M,), dtype=torch.float32, device=dev) for _ in range(R)]
            fused = [(lambda i=i: g5.gemm_fp8_nt_quant_a(dX[i], qW[i][0], qW[i][1], dC[i], scale_x=sxf[i],
                                                         workspace=ws)) for i in range(R)]
            ms_b = timed(both, 50, 10, label="fp8_example_5_8_quantize_and_gemm")
            ms_g = timed(gemm, 50, 10, label="fp8_example_5_8_gemm")
            ms_f = timed(fused, 50, 10, label="fp8_example_5_8_quantized_inside_gemm")
            sep, fus = ctypes.c_double(), ctypes.c_double()
            g5.lib().gemm_model_quant_traffic(M, N, K, 128, 128, 2, 1, 1, 2, ctypes.byref(sep), ctypes.byref(fus))
            tf = 2.0 * M * N * K / (ms_g * 1e-3) / 1e12
            log(f"fp8 Example 5-8 4096x1536x4096: quantize + GEMM {ms_b * 1e3:.2f} us, GEMM {ms_g * 1e3:.2f} us "
                f"({tf:.1f} TFLOPS); quantized inside the GEMM {ms_f * 1e3:.2f} us; "
                f"model traffic separate {sep.value / 2**20:.0f} MiB, fused {fus.value / 2**20:.0f} MiB")
            workloads.append({"name": "fp8_example_5_8_4096x1536x4096", "us": round(ms_b * 1e3, 3),
                              "gemm_us": round(ms_g * 1e3, 3), "gemm_tflops": round(tf, 2),
                              "quantized_inside_gemm_us": round(ms_f * 1e3, 3),
                              "gemm_frac_peak": round(tf / PEAK_FP8_TFLOPS, 4),
                              "model_traffic_separate_MiB": round(sep.value / 2**20, 1),
                              "model_traffic_fused_MiB": round(fus.value / 2**20, 1), "rotations": R})
            del dX, qW, qX, dC, sxf

    # ------------------------------------------------------------ attention scores from row-major K
    if args.only in ("all", "scores_nt"):
        with guarded("scores_nt", workloads):
            Q, KT = gi.batched_inputs()
            Km = np.ascontiguousarray(np.transpose(KT, (0, 2, 1)))
            bt, M, K = Q.shape
            N = Km.shape[1]
            alg_bytes = 2 * Q.size + 2 * Km.size + 4 * bt * M * N
            R = rotations(alg_bytes)
            dQ = [to_dev_bf16(Q) for _ in range(R)]
            dK = [to_dev_bf16(Km) for _ in range(R)]
            dC = [torch.empty((bt, M, N), device=dev) for _ in range(R)]
            fns = [(lambda i=i: g5.gemm_bf16_nt_batched(dQ[i], dK[i], dC[i], workspace=ws)) for i in range(R)]
            ms = timed(fns, 100, 10, label="scores_nt_bf16_32x1024x1024x128_f32out")
            gbps = alg_bytes / (ms * 1e-3) / 1e9
            log(f"scores Q.K^T from row-major K (NT): {ms * 1e3:.2f} us/call, {gbps:.0f} GB/s")
            workloads.append({"name": "scores_nt_bf16_32x1024x1024x128_f32out", "us": round(ms * 1e3, 3),
                              "GBps": round(gbps, 1), "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4), "alg_bytes": alg_bytes,
                              "rotations": R})
            del dQ, dK, dC

    # ------------------------------------------------------------ FFN projection with bias and residual
    if args.only in ("all", "affine"):
        with guarded("affine", workloads):
            # C := X.W + bias + C (beta = 1: a residual add into the bf16 output),
            # against the plain projection on the same buffers.
            M, N, K = 1024, 12288, 4096
            X, W = gi.ffn_inputs()
            g = np.random.default_rng([gi.SEED_BASE + gi.W_FFN, 6])
            bias = gi.to_bf16_bits(gi.normal(g, (N,)))
            R = rotations(2 * (M * K + K * N + 2 * M * N))
            dX = [to_dev_bf16(X) for _ in range(R)]
            dW = [to_dev_bf16(W) for _ in range(R)]
            db = [to_dev_bf16(bias) for _ in range(R)]
            dC = [torch.zeros((M, N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
            fns = [(lambda i=i: g5.gemm_bf16_affine(dX[i], dW[i], dC[i], bias=db[i], beta=1.0, workspace=ws)) for i in range(R)]
            plain = [(lambda i=i: g5.gemm_bf16(dX[i], dW[i], dC[i], workspace=ws)) for i in range(R)]
            ms = timed(fns, 50, 10, label="ffn_bias_residual_bf16_1024x12288x4096")
            ms_plain = timed(plain, 50, 10, label="ffn_plain_same_buffers")
            tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
            log(f"FFN + bias + residual: {ms * 1e3:.2f} us ({tf:.1f} TFLOPS); plain projection {ms_plain * 1e3:.2f} us")
            workloads.append({"name": "ffn_bias_residual_bf16_1024x12288x4096", "us": round(ms * 1e3, 3),
                              "tflops": round(tf, 2), "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                              "plain_projection_us": round(ms_plain * 1e3, 3), "rotations": R})
            del dX, dW, db, dC

    # ------------------------------------------------------------ linear layer: weight [out, in] and bias (NT)
    if args.only in ("all", "linear_nt"):
        with guarded("linear_nt", workloads):
            # y = X . W^T + b with W stored [12288, 4096] as a linear layer keeps
            # it, bf16 out, next to the same product without the bias.
            M, N, K = 1024, 12288, 4096
            X, W = gi.ffn_inputs()
            Wt = np.ascontiguousarray(W.T)
            g = np.random.default_rng([gi.SEED_BASE + gi.W_FFN, 7])
            bias = gi.to_bf16_bits(gi.normal(g, (N,)))
            R = rotations(2 * (M * K + K * N + M * N))
            dX = [to_dev_bf16(X) for _ in range(R)]
            dW = [to_dev_bf16(Wt) for _ in range(R)]
            db = [to_dev_bf16(bias) for _ in range(R)]
            dC = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
            fns = [(lambda i=i: g5.gemm_bf16_nt_affine(dX[i], dW[i], dC[i], bias=db[i], workspace=ws)) for i in range(R)]
            plain = [(lambda i=i: g5.gemm_bf16_nt(dX[i], dW[i], dC[i], workspace=ws)) for i in range(R)]
            ms = timed(fns, 50, 10, label="linear_nt_bias_bf16_1024x12288x4096")
            ms_plain = timed(plain, 50, 10, label="linear_nt_without_bias")
            tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
            log(f"linear layer X.W^T + b (W [12288,4096]): {ms * 1e3:.2f} us ({tf:.1f} TFLOPS); "
                f"without bias {ms_plain * 1e3:.2f} us")
            workloads.append({"name": "linear_nt_bias_bf16_1024x12288x4096", "us": round(ms * 1e3, 3),
                              "tflops": round(tf, 2), "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                              "without_bias_us": round(ms_plain * 1e3, 3), "rotations": R})
            del dX, dW, db, dC

    # ------------------------------------------------------------ weight gradient from row-major X (TN)
    if args.only in ("all", "wgrad_tn"):
        with guarded("wgrad_tn", workloads):
            # dW [4096, 12288] = X^T . dY with X [1024, 4096] as stored (At) and
            # dY [1024, 12288]: 103 GFLOP over K = 1024 tokens.
            X, dY = gi.wgrad_inputs()
            K, M = X.shape
            N = dY.shape[1]
            R = rotations(2 * (M * K + K * N + M * N))
            dX = [to_dev_bf16(X) for _ in range(R)]
            dD = [to_dev_bf16(dY) for _ in range(R)]
            dC = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
            fns = [(lambda i=i: g5.gemm_bf16_tn(dX[i], dD[i], dC[i], workspace=ws)) for i in range(R)]
            st, plan = g5.plan_query(g5.GEMM_OP_BF16_TN, M, N, K)
            ms = timed(fns, 50, 10, label="wgrad_tn_bf16_4096x12288x1024")
            tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
            log(f"weight gradient X^T.dY 4096x12288x1024 (TN): {ms * 1e3:.2f} us ({tf:.1f} TFLOPS), {plan.name.decode()}")
            workloads.append({"name": "wgrad_tn_bf16_4096x12288x1024", "us": round(ms * 1e3, 3), "tflops": round(tf, 2),
                              "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4), "config": plan.name.decode(),
                              "rotations": R})
            del dX, dD, dC

    out["workloads"] = workloads
    out["workload_timing"] = timings
    out["gpu_clocks"] = {"before": clocks_before, "after": gpu_clocks()}

    # ------------------------------------------------------------ CPU oracle
    if not args.no_cpu and ffn_rows_gpu is not None:
        import resource

        import oracle

        def cpu_seconds():
            ru = resource.getrusage(resource.RUSAGE_SELF)
            return ru.ru_utime + ru.ru_stime

        X, W, dCl = ffn_rows_gpu
        Cg = dCl.view(torch.int16).cpu().numpy().view(np.uint16)
        threads = oracle.num_threads()
        t = time.time()
        oracle.gemm_bf16(np.ascontiguousarray(X[:8]), W)       # calibration, 8 rows
        per_row = (time.time() - t) / 8
        rows = int(max(8, min(1024, args.cpu_seconds / max(per_row, 1e-6))))
        # The whole projection is repeated until about cpu_seconds of CPU
        # work have been timed (one pass when a pass is longer than that).
        Xs = np.ascontiguousarray(X[:rows])
        reps, secs, cpu0 = 0, 0.0, cpu_seconds()
        while reps == 0 or (secs < args.cpu_seconds and reps < 20):
            t = time.time()
            ref = oracle.gemm_bf16(Xs, W)
            secs += time.time() - t
            reps += 1
        busy = (cpu_seconds() - cpu0) / secs
        cpu_tflops = 2.0 * reps * rows * 12288 * 4096 / secs / 1e12
        got = gi.bf16_bits_to_f32(Cg[:rows]).astype(np.float64)
        bound = 2.0 ** -8 * np.abs(ref) + 1e-3 * 64.0
        worst = float((np.abs(got - ref) / bound).max())
        log(f"oracle: {reps} x {rows} rows in {secs:.1f} s on {threads} threads ({busy:.1f} cores busy) -> "
            f"{cpu_tflops * 1e3:.2f} GFLOPS; GPU rows within bar, worst err/bound {worst:.3f}")
        # FP32 256^3 (the small square product) on one thread, best of 5
        A1, B1 = gi.sgemm_inputs(256, workload=gi.W_SGEMM_SMALL)
        oracle.set_num_threads(1)
        one = []
        for _ in range(5):
            t = time.time()
            oracle.gemm_f32(A1, B1)
            one.append(time.time() - t)
        oracle.set_num_threads(threads)
        log(f"oracle FP32 256^3 on 1 thread: {min(one) * 1e3:.1f} ms")
        out["cpu_baseline"] = {"value": round(cpu_tflops, 6), "unit": "TFLOPS", "cores": threads,
                               "kind": "oracle",
                               "sample": f"{reps} pass(es) over the first {rows} of 1024 rows of the FFN projection "
                                         f"(x 12288 cols, K=4096), FP64 triple loop, {secs:.1f} s in total",
                               "cores_busy": round(busy, 2),
                               "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
                               "cpus_allowed": len(os.sched_getaffinity(0)),
                               "sgemm_256_1thread_ms": round(min(one) * 1e3, 3),
                               "gpu_rows_worst_err_over_bound": round(worst, 4)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Throughput of one EDiT attention-layer forward on one MI355X.

One step = one edit_attn_forward call (ConvFusion queries, Spatial-Compressor
keys/values, linear attention, output projection) over one batch of the
workload's synthetic input, which is resident in HBM before timing starts.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload pixart2048]

Prints one JSON line. `value` is image tokens/s over the K timed steps
(timing-only HIP events, recorded without a system-scope fence, on the stream
the library launches on, bracketed by device synchronisation). `roofline` covers the step with the longest average
duration: its algorithmic work per launch over its average duration, timed
live with events the library records between its steps, against MI355X's
published peak. `cpu_baseline` times the float64 CPU oracle on a bounded
sample of the same workload on the host's cores.
"""
import argparse
import ctypes
import dataclasses
import glob
import hashlib
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # dense matrix-core (f32: vector/matrix fp32)

STEP_NAMES = ["cf_conv3x3", "gn_stats", "cf_act", "q_proj", "kv_proj", "sc_dwconv", "kv_state",
              "linattn_apply", "out_proj"]
STEP_KERNELS = {  # kernels launched per step at bf16 (rocprofv3 names start with these)
    # bf16, H*W a multiple of 256 and W of 32..128 or a multiple of 256: the kernel-row conv; otherwise the
    # tap-by-tap implicit GEMM. Both carry the GroupNorm partials and the restore fold.
    "cf_conv3x3": "conv3x3_rows_kernel<W, E_BIAS_GN> (else gemm_dma_kernel<256 or 128, 96, 4, 1, A_CONV3, E_BIAS_GN>)",
    "gn_stats": "gn_finalize_channels_kernel",
    "cf_act": "gn_apply_kernel",
    "q_proj": "gemm_dma_kernel<128, 192, 2, 2, A_CAT2, E_BIAS_RELU>",
    "kv_proj": "gemm_dma_kernel<128, 192, 2, 2, A_PLAIN, E_BIAS>",
    "sc_dwconv": "dwconv_kv_state_kernel (the depthwise convs and the state partials)",
    "kv_state": "kv_state_finalize_kernel", "linattn_apply": "linattn_apply_kernel",
    "out_proj": "gemm_dma_kernel<128, 192, 2, 2, A_PLAIN, E_BIAS>",
}


def gn_tile_rows(s):
    """Rows per statistics tile of the conv's epilogue (the library's rule):
    256 where the conv runs on the kernel-row kernel (bf16, H*W a multiple of
    256, W of 32..128 or a multiple of 256); else 256, or 128 where 256-row
    tiles would fill fewer than half of the 256 CUs."""
    if s.dtype == "bf16" and s.N % 256 == 0 and s.C % 64 == 0 and s.Cr % 96 == 0 and \
            (s.W in (32, 64, 128) or s.W % 256 == 0):
        return 256
    return 128 if (s.B * s.N // 256) * (s.Cr // 96) < 128 and s.N % 128 == 0 else 256


def stats_in_conv(s):
    """Whether the bf16 conv's epilogue computes the GroupNorm partial
    statistics (and its launch the restore fold): the library does so when
    the conv runs on the direct-load kernel and its row tiles never
    straddle two samples."""
    return s.dtype == "bf16" and s.N % gn_tile_rows(s) == 0 and s.C % 64 == 0 and s.Cr % 96 == 0


def algorithmic_work(s):
    """Per-launch algorithmic flops and HBM bytes of each step: every input
    read once, every output written once, weights included."""
    es = 2 if s.dtype == "bf16" else 4
    B, N, C, Cr, h, d = s.B, s.N, s.C, s.Cr, s.heads, s.head_dim
    M, Mc = B * N, B * s.Nc
    st = B * h * (d * d + d) * 4
    conv = (2.0 * M * Cr * 9 * C, es * (M * C + Cr * 9 * C + M * Cr + Cr))
    stats = (3.0 * M * Cr, es * M * Cr)
    act = (3.0 * M * Cr, es * 2 * M * Cr)
    # the fold [W_q | W_q W_cf2], b_q + W_q b_cf2
    fold = (2.0 * C * C * Cr, es * (C * C + C * Cr + 2 * C + C * (C + Cr) + C))
    if stats_in_conv(s):
        # the statistics leave the conv in registers; the gn_stats step merges the per-(tile, channel)
        # partials (M / rows x C/r x 2 floats); the fold runs in the conv's launch
        tiles = M // gn_tile_rows(s)
        conv = (conv[0] + stats[0] + fold[0], conv[1] + fold[1] + 8 * tiles * Cr)
        stats = (3.0 * tiles * Cr, 8 * tiles * Cr)
    else:
        act = (act[0] + fold[0], act[1] + fold[1])
    dw = (2.0 * 9 * Mc * 2 * C, es * (2 * M * C + 2 * Mc * C + 2 * 10 * C))
    state = (2.0 * Mc * C * (d + 1), es * 2 * Mc * C + st)
    if s.dtype == "bf16":
        # one pass makes K', V' and the state partials (K', V' are not read back); the kv_state step
        # merges the per-(head, 256-token chunk) partials
        parts = B * h * ((s.Nc + 255) // 256) * (16 * ((d + 16) // 16)) * (16 * ((d + 15) // 16)) * 4
        dw = (dw[0] + state[0], dw[1] + st)
        state = (float(parts) / 4, parts + st)
    return {
        "cf_conv3x3": conv,
        "gn_stats": stats,
        # GN + LeakyReLU over xc (and the fold, when the conv's launch does not take it)
        "cf_act": act,
        # ReLU([X | act] [W_q | W_q W_cf2]^T + b)
        "q_proj": (2.0 * M * C * (C + Cr), es * (M * C + M * Cr + M * C + C * (C + Cr) + C)),
        "kv_proj": (2.0 * M * 2 * C * C, es * (M * C + 2 * M * C + 2 * C * C + 2 * C)),
        "sc_dwconv": dw,
        "kv_state": state,
        "linattn_apply": (2.0 * M * C * (d + 1), es * 2 * M * C + st),
        "out_proj": (2.0 * M * C * C, es * (2 * M * C + C * C + C)),
    }


def kernel_source_hash():
    """sha256 over the library's kernel and launch sources. HBM counters taken
    for one version of the kernels describe that version only."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "linear_compressed_attention_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, step):
    """HBM bytes per launch of `step` from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary (already scaled by the copy calibration), or None when
    there is none or the kernels have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"edit_layer_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    src = kernel_source_hash()
    with open(path) as fh:
        for line in fh:
            f = line.split()
            if len(f) == 4 and f[0] == "traffic" and f[1] == step and f[3] == src:
                return float(f[2])
    return None


def pct(v, q):
    v = sorted(v)
    i = q * (len(v) - 1)
    lo = int(i)
    hi = min(lo + 1, len(v) - 1)
    return v[lo] + (v[hi] - v[lo]) * (i - lo)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


STEP_BOUND = {"cf_conv3x3": "mfma", "gn_stats": "hbm", "cf_act": "hbm", "q_proj": "mfma", "kv_proj": "mfma",
              "sc_dwconv": "hbm", "kv_state": "hbm", "linattn_apply": "hbm", "out_proj": "mfma"}


def device_info():
    """The device measured: name, architecture, CU count and peak clock from
    the HIP runtime, and the peaks they imply (dense bf16 MFMA 4096 and fp32
    vector 256 flop/clk/CU on CDNA4) beside the published ones the
    rooflines use."""
    import torch

    p = torch.cuda.get_device_properties(0)
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipDeviceGetAttribute.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.c_int, ctypes.c_int]
    khz = ctypes.c_int(0)
    if hip.hipDeviceGetAttribute(ctypes.byref(khz), 5, 0) != 0:   # hipDeviceAttributeClockRate (kHz)
        khz.value = 0
    cus, ghz = p.multi_processor_count, khz.value / 1e6
    return {"name": p.name, "arch": p.gcnArchName, "cus": cus, "max_clock_mhz": round(khz.value / 1e3),
            "derived_peak_bf16_mfma_tflops": round(cus * 4096 * ghz / 1e3, 1),
            "derived_peak_fp32_vector_tflops": round(cus * 256 * ghz / 1e3, 1),
            "published_peak_bf16_mfma_tflops": PEAK_MFMA_TFLOPS["bf16"], "published_peak_hbm_gbs": PEAK_HBM_GBS}


class HipEvents:
    """hipEvent_t handles from the process's HIP runtime (the one torch loaded). They only time: created
    without the system-scope fence on recording (hipEventDisableSystemFence), so that the cache writeback
    and invalidation a fenced event adds between two steps are not counted in either step; they are read
    after a full device synchronisation."""

    DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence (hip_runtime_api.h)

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE)
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
            out.append(e.value)
        return out

    def record(self, e, stream):
        """Record e on a torch stream."""
        rc = self.hip.hipEventRecord(e, ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


def timed_steps(step, K, stream):
    """K calls of step() back to back between two timing-only events, bracketed by device synchronisation:
    (milliseconds on the GPU, wall seconds, per-call milliseconds). The per-call durations come from a second
    pass of K calls with an event between each two; every event recorded on the stream costs the chip a few
    microseconds, so they run slightly longer than the first pass's mean and serve only as its spread."""
    import torch
    tev = HipEvents()
    e = tev.create(2)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    tev.record(e[0], stream)
    for _ in range(K):
        step()
    tev.record(e[1], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = tev.elapsed_ms(e[0], e[1])
    ev = tev.create(K + 1)
    tev.record(ev[0], stream)
    for i in range(K):
        step()
        tev.record(ev[i + 1], stream)
    torch.cuda.synchronize()
    per_iter = [tev.elapsed_ms(ev[i], ev[i + 1]) for i in range(K)]
    tev.destroy(e + ev)
    return ms, wall, per_iter


def cpu_baseline(shape, inp, min_runs, budget_s, eta="ratio", query="convfusion", kv="compressed"):
    """The float64 oracle, as it stands, on the host cores: at least
    `min_runs` full layer forwards of the same workload, more while the total
    stays under `budget_s` seconds."""
    from threadpoolctl import threadpool_info
    from oracle import edit_oracle as O
    times = []
    while len(times) < min_runs or (sum(times) + statistics.median(times) < budget_s and len(times) < 50):
        t0 = time.perf_counter()
        if shape.n_text:
            O.mmedit_hybrid_forward(inp["x"], inp["x_txt"], inp["w"], inp["w_txt"], shape, eta=eta)
        elif (query, kv) != ("convfusion", "compressed"):
            O.edit_attn_variant_forward(inp["x"], inp["w"], shape, query, kv, inp.get("w_kcf"))
        else:
            O.edit_attn_forward(inp["x"], inp["w"], shape)
        times.append(time.perf_counter() - t0)
    med = statistics.median(times)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    what = "MM-EDiT hybrid" if shape.n_text else "EDiT layer"
    return {"value": round(shape.B * shape.N / med, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(times)} full float64 {what} forwards of the same workload "
                      f"({shape.B * shape.N} image tokens each, {sum(times):.1f} s of CPU work), "
                      f"median {med:.2f} s; cores = BLAS threads",
            "seconds_per_layer": round(med, 3), "affinity_cores": len(os.sched_getaffinity(0)),
            "cpu_model": cpu_model()}


def backward_work(s):
    """Algorithmic flops of one edit_attn_backward call: the GEMM-shaped
    products (input and weight gradients of every Linear and of the 3x3 conv,
    the folded query weights' two small products) and the linear-attention
    core (t = S dy twice per query, dS and dz over the tokens, dK' and dV')."""
    B, N, C, Cr, h, d = s.B, s.N, s.C, s.Cr, s.heads, s.head_dim
    M, Mc = B * N, B * s.Nc
    gemm = (2.0 * M * C * C * 2          # dy = dout W_o, dW_o
            + 4.0 * M * C * C * 2        # dx from [dk0 | dv0], dW_k and dW_v
            + 2.0 * M * C * C + 2.0 * M * C * Cr     # dx and dact from dq_pre
            + 2.0 * M * C * C + 2.0 * M * C * Cr     # dW' over [x | act]
            + 2.0 * M * C * 9 * Cr * 2   # conv input gradient, dW_cf1
            + 2.0 * 2 * C * C * Cr)      # dW_q's and dW_cf2's small products
    core = 2.0 * M * C * d * 2 + 2.0 * M * C * (d + 2) + 2.0 * 2 * Mc * C * d
    return gemm + core


def bench_backward(args, s, inp):
    """Times edit_attn_backward (after one forward fills its workspace) and
    prints the JSON line; the oracle backward is timed beside it."""
    import numpy as np
    import torch

    import linear_compressed_attention_amd as lca
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if s.dtype == "bf16" else torch.float32
    x = torch.from_numpy(inp["x"]).to(dev).to(tdt)
    w = {k: torch.from_numpy(v).to(dev).to(tdt) for k, v in inp["w"].items()}
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream()
    fws = torch.empty(lca.edit_attn_workspace_size(s), dtype=torch.uint8, device=dev)
    lca.edit_attn_forward(s, w, x, y, fws, stream)
    rng = np.random.default_rng(1)
    dout_np = rng.standard_normal((s.B, s.N, s.C)).astype(np.float32)
    dy = torch.from_numpy(dout_np).to(dev).to(tdt)
    dx = torch.empty_like(x)
    grads = {k: torch.empty_like(v) for k, v in w.items()}
    bws = torch.empty(lca.edit_attn_backward_workspace_size(s), dtype=torch.uint8, device=dev)

    def step():
        lca.edit_attn_backward(s, w, x, dy, fws, dx, grads, bws, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    ms, wall, per_iter = timed_steps(step, K, stream)
    assert torch.isfinite(dx).all().item(), "non-finite dx"
    flops = backward_work(s)
    ach = flops / (ms / K * 1e-3) / 1e12
    peak = PEAK_MFMA_TFLOPS[s.dtype]
    cpu = None
    if args.cpu_runs > 0:
        from threadpoolctl import threadpool_info
        from oracle import edit_backward as OB
        times = []
        while len(times) < args.cpu_runs or (sum(times) + statistics.median(times) < args.cpu_budget
                                             and len(times) < 20):
            t0 = time.perf_counter()
            OB.edit_attn_backward(inp["x"], inp["w"], s, dout_np)
            times.append(time.perf_counter() - t0)
        med = statistics.median(times)
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        cpu = {"value": round(s.B * s.N / med, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"{len(times)} full float64 layer backwards (forward recomputed inside, as the oracle "
                         f"does) of the same workload, median {med:.2f} s; cores = BLAS threads",
               "cpu_model": cpu_model()}
    wl = (f"{args.workload}: EDiT attention layer backward (dx and the 18 parameter gradients from the "
          f"forward's workspace), B={s.B}, {s.H}x{s.W} token grid ({s.N} tokens), C={s.C}, {s.heads} heads x "
          f"{s.head_dim}, r={s.reduction}, {s.gn_groups} GN groups, {s.dtype}")
    out = {
        "metric": "image tokens/sec per EDiT attention layer backward",
        "value": round(s.B * s.N * K / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms / K, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": s.dtype, "device": device_info(),
        "data": "synthetic (seeded N(0,1) activations and upstream gradient, N(0,0.02^2) weights)",
        "config": {"workload": wl, "B": s.B, "H": s.H, "W": s.W, "C": s.C, "heads": s.heads,
                   "head_dim": s.head_dim, "reduction": s.reduction, "gn_groups": s.gn_groups, "pass": "backward"},
        "roofline": {"bound": "mfma", "achieved": round(ach, 1), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(ach / peak, 4), "traffic": None,
                     "kernel": "edit_attn_backward, all launches (algorithmic flops over the call's time)",
                     "work_per_launch": flops},
        "cpu_baseline": cpu,
        "ms_per_step_p10_p50_p90": [round(pct(per_iter, q), 5) for q in (0.1, 0.5, 0.9)],
        "wall_s_timed_region": round(wall, 4),
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed forwards first; about 100 bring the chip to the steady rate of back-to-back layers")
    ap.add_argument("--workload", default="pixart2048")
    ap.add_argument("--cpu-runs", type=int, default=3, help="minimum oracle runs for cpu_baseline (0 = skip)")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="further oracle runs while their total stays under this many seconds")
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="forwards timed with a 512 MiB buffer written before each (0 = skip)")
    ap.add_argument("--profile-steps", type=int, default=None,
                    help="timed forwards for the per-step breakdown (default: --steps)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy (outside the timed region) whose HBM counter "
                         "readings calibrate FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--exact-eta", action="store_true",
                    help="hybrid workloads: time mmedit_hybrid_exact_forward (eta per row) instead of the ratio")
    ap.add_argument("--query", default="convfusion", choices=["convfusion", "linear"],
                    help="ablation variant: query processing (EDiT workloads)")
    ap.add_argument("--kv", default="compressed", choices=["compressed", "full", "key_convfusion"],
                    help="ablation variant: key/value processing (EDiT workloads)")
    ap.add_argument("--backward", action="store_true",
                    help="time the layer backward (edit_attn_backward) instead of the forward")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); multi-GPU runs are not part of this "
              "build: the layer shards by grid bands with one per-head state all-reduce, which is designed "
              "but not implemented here.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import linear_compressed_attention_amd as lca
    from seeded_inputs import CONFIGS, make_inputs

    s = CONFIGS[args.workload]
    hybrid = s.n_text > 0
    variant = (args.query, args.kv) != ("convfusion", "compressed")
    if hybrid and variant:
        print("the ablation variants apply to the EDiT layer, not the hybrid", file=sys.stderr)
        sys.exit(2)
    if args.exact_eta and not hybrid:
        print("--exact-eta applies to the hybrid workloads", file=sys.stderr)
        sys.exit(2)
    inp = make_inputs(s, seed=0, key_convfusion=args.kv == "key_convfusion")
    if args.backward:
        if hybrid or variant or args.exact_eta:
            print("--backward applies to the EDiT layer itself", file=sys.stderr)
            sys.exit(2)
        bench_backward(args, s, inp)
        return
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if s.dtype == "bf16" else torch.float32
    x = torch.from_numpy(inp["x"]).to(dev).to(tdt)
    w = {k: torch.from_numpy(v).to(dev).to(tdt) for k, v in inp["w"].items()}
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream()
    if hybrid:
        xt = torch.from_numpy(inp["x_txt"]).to(dev).to(tdt)
        wt = {k: torch.from_numpy(v).to(dev).to(tdt) for k, v in inp["w_txt"].items()}
        yt = torch.empty_like(xt)
        ws = torch.empty(lca.mmedit_hybrid_workspace_size(s, s.n_text), dtype=torch.uint8, device=dev)

        hfwd = lca.mmedit_hybrid_exact_forward if args.exact_eta else lca.mmedit_hybrid_forward

        def step():
            hfwd(s, s.n_text, w, wt, x, xt, y, yt, ws, stream)
    elif variant:
        kcf = ({k: torch.from_numpy(v).to(dev).to(tdt) for k, v in inp["w_kcf"].items()}
               if args.kv == "key_convfusion" else None)
        ws = torch.empty(lca.edit_attn_variant_workspace_size(s, args.query, args.kv), dtype=torch.uint8,
                         device=dev)

        def step():
            lca.edit_attn_variant_forward(s, args.query, args.kv, w, kcf, x, y, ws, stream)
    else:
        ws = torch.empty(lca.edit_attn_workspace_size(s), dtype=torch.uint8, device=dev)

        def step():
            lca.edit_attn_forward(s, w, x, y, ws, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K forwards back to back, as the layers of a model run, between two timing-only events
    # (no system-scope fence on recording; read after the device synchronisation).
    K = args.steps
    ms, wall, per_iter = timed_steps(step, K, stream)
    ms_per_step = ms / K
    value = s.B * s.N * K / (ms / 1e3)
    assert torch.isfinite(y).all().item(), "non-finite output"

    # Cold variant: 512 MiB written between forwards so that no intermediate
    # of the previous forward is still in the 256 MB last-level cache.
    cold = None
    if args.cold_steps > 0:
        junk = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cms = []
        for i in range(args.cold_steps):
            junk.fill_(i & 0xFF)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            step()
            b.record(stream)
            b.synchronize()
            cms.append(a.elapsed_time(b))
        del junk
        cold = {"steps": args.cold_steps, "ms_median": round(statistics.median(cms), 5),
                "tokens_per_s": round(s.B * s.N / (statistics.median(cms) / 1e3), 1)}

    # Per-step durations from events the library records between its steps.
    P = args.profile_steps or K
    hev = HipEvents()
    evs = [hev.create(len(STEP_NAMES) + 1) for _ in range(P)]
    torch.cuda.synchronize()
    # The hybrid's image path runs these same kernels on the same image shape.
    s_img = dataclasses.replace(s, n_text=0) if hybrid else s
    ws_img = (torch.empty(lca.edit_attn_workspace_size(s_img), dtype=torch.uint8, device=dev)
              if hybrid or variant else ws)
    # A bounded spin kernel first, so that every timed forward is already
    # queued when the GPU reaches it: the step intervals then hold no host
    # launch latency.
    torch.cuda._sleep(50_000_000)
    for e in evs:
        arr = (ctypes.c_void_p * len(e))(*e)
        lca.edit_attn_forward_timed(s_img, w, x, y, ws_img, arr, stream)
    torch.cuda.synchronize()
    per_step = {n: [] for n in STEP_NAMES}
    for e in evs:
        for i, n in enumerate(STEP_NAMES):
            per_step[n].append(hev.elapsed_ms(e[i], e[i + 1]))
    for e in evs:
        hev.destroy(e)

    work = algorithmic_work(s)
    steps = {}
    for n in STEP_NAMES:
        us = 1e3 * statistics.mean(per_step[n])
        fl, by = work[n]
        if STEP_BOUND[n] == "mfma":
            ach = fl / (us * 1e-6) / 1e12
            peak = PEAK_MFMA_TFLOPS[s.dtype]
            unit = "TFLOP/s"
        else:
            ach = by / (us * 1e-6) / 1e9
            peak = PEAK_HBM_GBS
            unit = "GB/s"
        steps[n] = {"us": round(us, 2), "bound": STEP_BOUND[n], "achieved": round(ach, 1), "unit": unit,
                    "frac": round(ach / peak, 4), "flops": fl, "bytes": by, "kernels": STEP_KERNELS[n]}
    single = [n for n in STEP_NAMES if "+" not in STEP_KERNELS[n]]
    dom = max(single, key=lambda n: steps[n]["us"])
    d = steps[dom]
    roofline = {"bound": d["bound"], "achieved": d["achieved"],
                "peak": PEAK_MFMA_TFLOPS[s.dtype] if d["bound"] == "mfma" else PEAK_HBM_GBS,
                "unit": d["unit"], "frac": d["frac"], "traffic": measured_traffic(args.workload, dom), "kernel": dom,
                "avg_us": d["us"], "work_per_launch": d["flops"] if d["bound"] == "mfma" else d["bytes"]}
    layer_floor_us = sum(max(work[n][0] / (PEAK_MFMA_TFLOPS[s.dtype] * 1e6), work[n][1] / (PEAK_HBM_GBS * 1e3))
                         for n in STEP_NAMES)

    # A plain device-to-device copy: the achievable HBM rate beside the
    # published peak, and (under rocprofv3 --pmc) the HBM counter calibration.
    nb = 512 << 20
    src = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 3 if args.copy_calibration else 10
    a.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    b.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * nb * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    roofline["achievable_hbm_GBs"] = round(copy_gbs, 1)
    if d["bound"] == "hbm":
        roofline["frac_of_achievable"] = round(d["achieved"] / copy_gbs, 4)
    # every HBM-bound step also against the copy rate this box reached
    for n in STEP_NAMES:
        if steps[n]["bound"] == "hbm":
            steps[n]["frac_of_achievable"] = round(steps[n]["achieved"] / copy_gbs, 4)

    cpu = None
    if args.cpu_runs > 0:
        cpu = cpu_baseline(s, inp, args.cpu_runs, args.cpu_budget, eta="exact" if args.exact_eta else "ratio",
                           query=args.query, kv=args.kv)

    if hybrid:
        metric = "image tokens/sec per MM-EDiT hybrid attention layer fwd (text rows included in the time)"
        wl = (f"{args.workload}: MM-EDiT hybrid attention layer forward, B={s.B}, {s.H}x{s.W} image grid "
              f"({s.N} image tokens, {s.Nc} compressed) + {s.n_text} text tokens, C={s.C}, {s.heads} heads x "
              f"{s.head_dim}, r={s.reduction}, {s.gn_groups} GN groups, {s.dtype}")
        if args.exact_eta:
            wl += ", eta computed per image row (exact)"
    else:
        metric = "image tokens/sec per EDiT attention layer fwd at 16384 tokens; % HBM/MFMA peak"
        wl = (f"{args.workload}: EDiT attention layer forward, B={s.B}, {s.H}x{s.W} token grid "
              f"({s.N} tokens, {s.Nc} compressed K/V tokens), C={s.C}, {s.heads} heads x "
              f"{s.head_dim}, r={s.reduction}, {s.gn_groups} GN groups, {s.dtype}")
        if variant:
            wl += f", ablation variant query={args.query} kv={args.kv}"
    out = {
        "metric": metric,
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": s.dtype, "data": "synthetic (seeded N(0,1) activations, N(0,0.02^2) weights)",
        "device": device_info(),
        "config": {"workload": wl, "B": s.B, "H": s.H, "W": s.W, "C": s.C, "heads": s.heads,
                   "head_dim": s.head_dim, "reduction": s.reduction, "gn_groups": s.gn_groups,
                   **({"n_text": s.n_text} if hybrid else {}),
                   **({"eta": "exact"} if args.exact_eta else {}),
                   **({"query": args.query, "kv": args.kv} if variant else {})},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "ms_per_step_p10_p50_p90": [round(pct(per_iter, q), 5) for q in (0.1, 0.5, 0.9)],
        "cold": cold,
        "layer_roofline": {"floor_us": round(layer_floor_us, 1),
                           "frac": round(layer_floor_us / (ms_per_step * 1e3), 4),
                           **({"covers": "image path only"} if hybrid else {}),
                           **({"covers": "the layer's own steps (breakdown taken on the layer, not the variant)"}
                              if variant else {})},
        "steps_breakdown": {n: {k: v for k, v in steps[n].items()
                                if k in ("us", "bound", "achieved", "unit", "frac", "frac_of_achievable")}
                            for n in STEP_NAMES},
        "wall_s_timed_region": round(wall, 4),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

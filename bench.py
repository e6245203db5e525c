"""Benchmark of the FP8 fused attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload outlier] [--no-cpu]

One step = the whole FP8 path on one batch of synthetic input resident in HBM:
quantize_qkv_fp8 (rotate + block-scale + e4m3) then attn_fp8_fwd.  `value` is
algorithmic TFLOP/s of that step (4*D FLOP per visible query/key pair; causal
pairs discounted), quantisation included.  The same run also reports the
attention alone, the attention options (Schraudolph exponentials; power-of-two
block scales applied by the scaled MFMA), the quantiser alone, the BF16 twin, the accuracy against the
FP64 oracle on a bounded sample, the roofline of the attention kernel and the
oracle's CPU throughput, and the packed variable-length document workloads
(quantiser + attention with document-local scales, longest-first against
document order), and decode against an FP8 K/V cache (GB/s against the HBM
peak).  Prints ONE JSON line.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 attn fwd TFLOP/s (hd128, seq 8192) + RMSE vs FP64, ratio to BF16 RMSE"
FP8_PEAK_TFLOPS = 5000.0          # MI355X dense FP8 MFMA
BF16_PEAK_TFLOPS = 2500.0
HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = ["fp8_attention_forward_amd/csrc/attn_fp8.hip", "fp8_attention_forward_amd/csrc/fp8_tiles.h",
                  "fp8_attention_forward_amd/csrc/attn_internal.h", "fp8_attention_forward_amd/csrc/common.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fp8_outlier_traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="outlier")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline and accuracy sample")
    ap.add_argument("--no-packed", action="store_true", help="skip the packed variable-length document workloads")
    ap.add_argument("--no-decode", action="store_true", help="skip the FP8 K/V-cache decode workloads")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the causal, ablation-shape and channel-outlier configurations")
    ap.add_argument("--decode-only", action="store_true",
                    help="run only the decode workloads (for profiling); --copy-mb adds a calibration copy")
    ap.add_argument("--decode-split", type=int, default=0,
                    help="decode key ranges: 0 = the library's choice (balanced shares), >0 = fixed ranges of that "
                         "many keys per wave")
    ap.add_argument("--attn-only", action="store_true", help="time only attn_fp8_fwd launches (for profiling)")
    ap.add_argument("--bf16", action="store_true", help="with --attn-only: time the BF16 twin's launches instead")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="with --attn-only: first run one plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def smi_clocks():
    """Clock limits the device reports (amd-smi, a child process; None if unavailable).
    The clock held under load is not sampled here: the rocprofv3 summaries derive
    it from GRBM_GUI_ACTIVE over the launch time."""
    import subprocess
    try:
        res = subprocess.run(["amd-smi", "metric", "-g", "0", "--clock", "--json"], capture_output=True, text=True,
                             timeout=30)
        clk = json.loads(res.stdout)["gpu_data"][0]["clock"]
        mhz = lambda d, key: d[key]["value"] if isinstance(d.get(key), dict) else None
        return {"gfx_min_mhz": mhz(clk["gfx_0"], "min_clk"), "gfx_max_mhz": mhz(clk["gfx_0"], "max_clk"),
                "mem_mhz": mhz(clk["mem_0"], "clk"), "source": "amd-smi metric --clock (device limits)"}
    except Exception:
        return None


def kernel_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(workload):
    """HBM bytes per attention launch from the committed rocprofv3 counter summary, if still valid."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_hash") != kernel_hash() or t.get("workload") != workload:
        return None
    return t.get("bytes_per_launch")


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(every (batch, head) is independent: heads shard across GPUs with no communication)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import fp8_attention_forward_amd as fa
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    if args.decode_only:
        if args.copy_mb:
            src = torch.empty(args.copy_mb << 20, dtype=torch.uint8, device=dev)
            dst = torch.empty_like(src)
            src.fill_(1)
            torch.cuda.synchronize()
            dst.copy_(src)
            torch.cuda.synchronize()
        print(json.dumps({"mode": "decode_only",
                          "kv_decode": decode_leg(args, fa, workloads, torch, dev, torch.cuda.current_stream(dev))}))
        return 0
    w = workloads.WORKLOADS[args.workload]
    q_np, k_np, v_np = workloads.generate_workload(w)
    q, k, v = (torch.from_numpy(x).to(dev) for x in (q_np, k_np, v_np))
    B, H, N, D, sb = w.B, w.H, w.N, w.D, w.scale_block
    nb = -(-N // sb)
    q8, k8, v8 = (torch.empty((B, H, N, D), dtype=torch.uint8, device=dev) for _ in range(3))
    qd, kd, vd = (torch.empty((B, H, nb), dtype=torch.float32, device=dev) for _ in range(3))
    o = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    qout = (q8, k8, v8, qd, kd, vd)
    stream = torch.cuda.current_stream(dev)

    def quant():
        fa.quantize_qkv_fp8(q, k, v, scale_block=sb, hadamard=w.hadamard, seed=w.sign_seed, out=qout)

    def attn():
        fa.attn_fp8_fwd(q8, k8, v8, qd, kd, vd, scale_block=sb, hadamard=w.hadamard, causal=w.causal, out=(o, lse))

    flops = w.flops()
    ev = lambda: torch.cuda.Event(enable_timing=True)

    if args.attn_only:
        if args.copy_mb:
            src = torch.empty(args.copy_mb << 20, dtype=torch.uint8, device=dev)
            dst = torch.empty_like(src)
            src.fill_(1)
            torch.cuda.synchronize()
            dst.copy_(src)
            torch.cuda.synchronize()
        run = attn
        if args.bf16:
            # (inputs cast to BF16 before the timed launches)
            qb, kb, vb = (x.to(torch.bfloat16) for x in (q, k, v))
            ob, lb = torch.empty_like(o), torch.empty_like(lse)
            run = lambda: fa.attn_bf16_fwd(qb, kb, vb, causal=w.causal, out=(ob, lb))
        else:
            quant()
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            run()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        print(json.dumps({"mode": "attn_only", "kernel": "attn_bf16_fwd" if args.bf16 else "attn_fp8_fwd",
                          "workload": w.name, "ms_per_launch": ms, "tflops": flops / (ms * 1e-3) / 1e12}))
        return 0

    # ---- timed region: K steps of quantise + attention, events around each attention launch
    for _ in range(args.warmup):
        quant()
        attn()
    torch.cuda.synchronize()
    marks = [(ev(), ev()) for _ in range(args.steps)]
    start, stop = ev(), ev()
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        quant()
        marks[i][0].record(stream)
        attn()
        marks[i][1].record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_step = total_ms / args.steps
    attn_ms = [a.elapsed_time(b) for a, b in marks]
    attn_avg = sum(attn_ms) / len(attn_ms)
    srt = sorted(attn_ms)
    attn_med = srt[len(srt) // 2]
    attn_p10, attn_p90 = srt[len(srt) // 10], srt[min(len(srt) - 1, (9 * len(srt)) // 10)]

    # ---- quantiser alone (GB/s of algorithmic bytes: read 4 B, write 1 B per element, + descales)
    qs, qe = ev(), ev()
    nq = max(10, args.steps // 2)
    qs.record(stream)
    for _ in range(nq):
        quant()
    qe.record(stream)
    torch.cuda.synchronize()
    quant_ms = qs.elapsed_time(qe) / nq
    quant_bytes = 3 * B * H * N * D * 5 + 3 * B * H * nb * 4

    # The option legs and the BF16 twin report the median of per-launch HIP
    # events (a transient stall of the box moves a block mean, not the median).
    def median_ms(fn, n):
        for _ in range(3):
            fn()
        marks = [(ev(), ev()) for _ in range(n)]
        torch.cuda.synchronize()
        for a, b in marks:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in marks]))

    n_opt = max(10, args.steps // 4)

    # ---- option: Schraudolph's bit-level exponential for the probabilities
    o_sch = torch.empty_like(o)
    l_sch = torch.empty_like(lse)

    def attn_sch():
        fa.attn_fp8_fwd(q8, k8, v8, qd, kd, vd, scale_block=sb, hadamard=w.hadamard, causal=w.causal,
                        out=(o_sch, l_sch), exp2="schraudolph")

    sch_ms = median_ms(attn_sch, n_opt)

    # ---- option: power-of-two (E8M0) block scales applied by the scaled MFMA
    mx_out = tuple(torch.empty_like(x) for x in qout)
    o_mx = torch.empty_like(o)
    l_mx = torch.empty_like(lse)

    def quant_mx():
        fa.quantize_qkv_fp8(q, k, v, scale_block=sb, hadamard=w.hadamard, seed=w.sign_seed, out=mx_out, mx=True)

    def attn_mx():
        fa.attn_fp8_fwd(*mx_out, scale_block=sb, hadamard=w.hadamard, causal=w.causal, out=(o_mx, l_mx), mx=True)

    quant_mx()
    mx_ms = median_ms(attn_mx, n_opt)

    # ---- both options together (FLAMIA's inference form: microscaling and a
    # bit-level exponential)
    o_fl = torch.empty_like(o)
    l_fl = torch.empty_like(lse)

    def attn_fl():
        fa.attn_fp8_fwd(*mx_out, scale_block=sb, hadamard=w.hadamard, causal=w.causal, out=(o_fl, l_fl), mx=True,
                        exp2="schraudolph")

    fl_ms = median_ms(attn_fl, n_opt)

    # ---- option: power-of-two scales per (scale block x 32 channels), the
    # scaled MFMA's own granularity
    mx32_out = (torch.empty_like(q8), torch.empty_like(k8), torch.empty_like(v8),
                torch.empty((B, H, nb, D // 32), dtype=torch.float32, device=dev),
                torch.empty((B, H, nb, D // 32), dtype=torch.float32, device=dev),
                torch.empty((B, H, nb, D // 32), dtype=torch.float32, device=dev))
    o_m32 = torch.empty_like(o)
    l_m32 = torch.empty_like(lse)

    def quant_mx32():
        fa.quantize_qkv_fp8(q, k, v, scale_block=sb, hadamard=w.hadamard, seed=w.sign_seed, out=mx32_out, mx32=True)

    def attn_mx32():
        fa.attn_fp8_fwd(*mx32_out, scale_block=sb, hadamard=w.hadamard, causal=w.causal, out=(o_m32, l_m32),
                        mx32=True)

    quant_mx32()
    m32_ms = median_ms(attn_mx32, n_opt)

    # ---- BF16 twin (inputs cast outside the timed region).  Timed after every
    # FP8 leg of this workload: at its MFMA load the chip lowers its clock, and
    # launches that follow soon after would inherit the lower clock.
    qb, kb, vb = (x.to(torch.bfloat16) for x in (q, k, v))
    ob = torch.empty_like(o)
    lb = torch.empty_like(lse)
    bf16_ms = median_ms(lambda: fa.attn_bf16_fwd(qb, kb, vb, causal=w.causal, out=(ob, lb)), max(5, args.steps // 4))
    time.sleep(1.0)   # (let the clock recover before the packed-document and decode legs)

    # fresh outputs of the paths for the accuracy sample
    quant()
    attn()
    attn_sch()
    quant_mx()
    attn_mx()
    attn_fl()
    quant_mx32()
    attn_mx32()
    torch.cuda.synchronize()

    attn_tflops = flops / (attn_avg * 1e-3) / 1e12
    attn_bytes = 3 * B * H * N * D + 3 * B * H * nb * 4 + B * H * N * D * 2 + B * H * N * 4
    result = {
        "metric": METRIC,
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B{B} H{H} N{N} D{D} {'causal' if w.causal else 'non-causal'}, "
                               f"scale block {sb}, rotation {'on' if w.hadamard else 'off'}, {w.kind} inputs",
                   "B": B, "H": H, "N": N, "D": D, "causal": w.causal, "scale_block": sb,
                   "hadamard": w.hadamard, "quantisation": "included"},
        "attn_only": {"tflops": round(attn_tflops, 2), "ms_avg": round(attn_avg, 4), "ms_median": round(attn_med, 4),
                      "ms_p10": round(attn_p10, 4), "ms_p90": round(attn_p90, 4),
                      "tflops_median": round(flops / (attn_med * 1e-3) / 1e12, 2),
                      "frac_fp8_peak": round(attn_tflops / FP8_PEAK_TFLOPS, 4)},
        "quantiser": {"ms": round(quant_ms, 4), "gbs": round(quant_bytes / (quant_ms * 1e-3) / 1e9, 1),
                      "frac_hbm_peak": round(quant_bytes / (quant_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "exp2_schraudolph": {"tflops": round(flops / (sch_ms * 1e-3) / 1e12, 2), "ms": round(sch_ms, 4),
                             "frac_fp8_peak": round(flops / (sch_ms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4),
                             "note": "attention alone, probabilities by Schraudolph's bit-level exponential"},
        "mx_scales": {"tflops": round(flops / (mx_ms * 1e-3) / 1e12, 2), "ms": round(mx_ms, 4),
                      "frac_fp8_peak": round(flops / (mx_ms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4),
                      "note": "attention alone, power-of-two block scales applied by the scaled FP8 MFMA"},
        "mx_scales_schraudolph": {"tflops": round(flops / (fl_ms * 1e-3) / 1e12, 2), "ms": round(fl_ms, 4),
                                  "frac_fp8_peak": round(flops / (fl_ms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4),
                                  "note": "attention alone, both options: power-of-two block scales and "
                                          "Schraudolph's exponential"},
        "mx32_scales": {"tflops": round(flops / (m32_ms * 1e-3) / 1e12, 2), "ms": round(m32_ms, 4),
                        "frac_fp8_peak": round(flops / (m32_ms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4),
                        "note": "attention alone, power-of-two scales per (scale block x 32 channels) on the "
                                "scaled FP8 MFMA"},
        "bf16_twin": {"tflops": round(flops / (bf16_ms * 1e-3) / 1e12, 2), "ms": round(bf16_ms, 4),
                      "frac_bf16_peak": round(flops / (bf16_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / FP8_PEAK_TFLOPS, 4), "traffic": traffic_for(w.name),
                     "algorithmic_bytes": attn_bytes, "kernel": "attn_fp8_kernel"},
        "data_sha256": {nm: hashlib.sha256(np.ascontiguousarray(x).tobytes()).hexdigest()[:16]
                        for nm, x in (("q", q_np), ("k", k_np), ("v", v_np))},
        "toolchain": {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None),
                      "numpy": np.__version__, "hipcc": hipcc_version(),
                      "arch": getattr(torch.cuda.get_device_properties(0), "gcnArchName", None),
                      "device": torch.cuda.get_device_name(0), "clocks": smi_clocks()},
    }

    if not args.no_packed:
        result["packed_docs"] = packed_leg(args, fa, workloads, torch, dev, stream)
    if not args.no_decode:
        result["kv_decode"] = decode_leg(args, fa, workloads, torch, dev, stream)
    samples = []
    if not args.no_configs:
        result["configs"], samples = configs_leg(args, fa, workloads, torch, dev, stream, w, (q, k, v), q_np, k_np,
                                                 v_np)
    if not args.no_cpu:
        result.update(cpu_leg(w, q_np, k_np, v_np, o, ob, o_sch, o_mx, o_fl, o_m32))
        if samples:
            config_accuracy(result["configs"], samples)
    print(json.dumps(result))
    return 0


CONFIG_NAMES = ("outlier_causal", "ablation", "channel", "channel_norot")


def configs_leg(args, fa, workloads, torch, dev, stream, w0, dev0, q0_np, k0_np, v0_np):
    """The other configurations of the metric: the outlier workload made causal
    (the same tensors), the ablation shape (FP8 path against the BF16 twin), and
    channel outliers with and without the rotation.  Per configuration: one step
    (quantise + attention) and the attention alone, median of per-launch HIP
    events, inputs resident in HBM; the BF16 twin where the configuration
    compares against it.  Returns the timings and, for the accuracy report, the
    FP8 / BF16 outputs of two heads on a fixed sample of query rows."""
    import numpy as np
    ev = lambda: torch.cuda.Event(enable_timing=True)
    out, samples = {}, []
    cache = {}
    for name in CONFIG_NAMES:
        w = workloads.WORKLOADS[name]
        key = (w.kind, w.B, w.H, w.N, w.D, w.data_seed)
        if key == (w0.kind, w0.B, w0.H, w0.N, w0.D, w0.data_seed):
            arrs, (q, k, v) = (q0_np, k0_np, v0_np), dev0
        else:
            if key not in cache:
                cache.clear()
                a = workloads.generate_workload(w)
                cache[key] = (a, tuple(torch.from_numpy(x).to(dev) for x in a))
            arrs, (q, k, v) = cache[key]
        B, H, N, D, sb = w.B, w.H, w.N, w.D, w.scale_block
        nb = -(-N // sb)
        q8, k8, v8 = (torch.empty((B, H, N, D), dtype=torch.uint8, device=dev) for _ in range(3))
        qd, kd, vd = (torch.empty((B, H, nb), dtype=torch.float32, device=dev) for _ in range(3))
        o = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)

        def quant():
            fa.quantize_qkv_fp8(q, k, v, scale_block=sb, hadamard=w.hadamard, seed=w.sign_seed,
                                out=(q8, k8, v8, qd, kd, vd))

        def attn():
            fa.attn_fp8_fwd(q8, k8, v8, qd, kd, vd, scale_block=sb, hadamard=w.hadamard, causal=w.causal,
                            out=(o, lse))

        def timed(fn, n):
            for _ in range(3):
                fn()
            marks = [(ev(), ev()) for _ in range(n)]
            torch.cuda.synchronize()
            for a, b in marks:
                a.record(stream)
                fn()
                b.record(stream)
            torch.cuda.synchronize()
            return float(np.median([a.elapsed_time(b) for a, b in marks]))

        n = max(10, args.steps // 4)
        step_ms = timed(lambda: (quant(), attn()), n)
        attn_ms = timed(attn, n)
        flops = w.flops()
        r = {"workload": f"{name}: B{B} H{H} N{N} D{D} {'causal' if w.causal else 'non-causal'}, scale block {sb}, "
                         f"rotation {'on' if w.hadamard else 'off'}, {w.kind} inputs",
             "step_ms": round(step_ms, 4), "tflops_step": round(flops / (step_ms * 1e-3) / 1e12, 2),
             "attn_ms": round(attn_ms, 4), "attn_tflops": round(flops / (attn_ms * 1e-3) / 1e12, 2),
             "attn_frac_fp8_peak": round(flops / (attn_ms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4)}
        ob = None
        if name != "channel_norot":
            qb, kb, vb = (x.to(torch.bfloat16) for x in (q, k, v))
            ob, lb = torch.empty_like(o), torch.empty_like(lse)
            bf_ms = timed(lambda: fa.attn_bf16_fwd(qb, kb, vb, causal=w.causal, out=(ob, lb)), n)
            del qb, kb, vb
            time.sleep(1.0)   # (let the clock recover before the next configuration's FP8 timing)
            r.update({"bf16_ms": round(bf_ms, 4), "bf16_tflops": round(flops / (bf_ms * 1e-3) / 1e12, 2),
                      "fp8_speedup_over_bf16": round(bf_ms / attn_ms, 3)})
        quant()
        attn()
        torch.cuda.synchronize()
        rows = np.sort(np.random.default_rng(11).choice(N, size=min(N, 512), replace=False))
        heads = [(0, 0), (B - 1, H - 1)]
        ridx = torch.from_numpy(rows).to(dev)
        grab = lambda t: [t[b, h].index_select(0, ridx).float().cpu().numpy().astype(np.float64) for b, h in heads]
        samples.append((name, w, arrs, rows, heads, grab(o), grab(ob) if ob is not None else None))
        out[name] = r
    cache.clear()
    return out, samples


def config_accuracy(configs, samples):
    """Oracle leg, continued: RMSE and cosine against FP64 exact attention of the
    FP8 path (and the BF16 twin) for each configuration, on the sampled rows."""
    import numpy as np

    from oracle import attention as oatt

    for name, w, (q_np, k_np, v_np), rows, heads, o8, o16 in samples:
        e8, e16, ra = [], [], []
        for i, (b, h) in enumerate(heads):
            sl = (slice(b, b + 1), slice(h, h + 1))
            orf, _ = oatt.reference_attention(q_np[sl], k_np[sl], v_np[sl], w.causal, rows=rows)
            e8.append((o8[i] - orf[0, 0]).ravel())
            if o16 is not None:
                e16.append((o16[i] - orf[0, 0]).ravel())
            ra.append(orf[0, 0].ravel())
        e8, ra = np.concatenate(e8), np.concatenate(ra)
        cos = lambda e: float(np.dot(ra + e, ra) / (np.linalg.norm(ra + e) * np.linalg.norm(ra)))
        acc = {"sample": f"{len(heads)} heads x {len(rows)} query rows vs FP64 exact attention",
               "fp8_rmse": float(np.sqrt(np.mean(e8 ** 2))), "fp8_max_err": float(np.max(np.abs(e8))),
               "fp8_cosine": cos(e8), "rms_o": float(np.sqrt(np.mean(ra ** 2)))}
        if e16:
            e16 = np.concatenate(e16)
            acc.update({"bf16_rmse": float(np.sqrt(np.mean(e16 ** 2))), "bf16_cosine": cos(e16)})
            acc["ratio_fp8_to_bf16_rmse"] = acc["fp8_rmse"] / acc["bf16_rmse"] if acc["bf16_rmse"] > 0 else None
        configs[name]["accuracy"] = acc


DECODE_NAMES = ("decode_gqa", "decode_gqa_spec")


def decode_partials(w, L, split, waves=2048):
    """Partials one decode call writes (and the merge reads back): fixed ranges,
    one per four ranges of each (sequence, K/V head) that holds keys; balanced
    shares, one per piece, i.e. per interval between consecutive share and
    segment boundaries of the flat tile order (64-key tiles, sequence-major,
    then K/V head)."""
    import numpy as np
    if split:
        return int(w.Hkv * (-(-L // (4 * split))).sum())
    nt = -(-L // 64)
    T = int(w.Hkv * nt.sum())
    W = min(waves, -(-min(waves, w.B * w.Hkv * -(-w.Ncap // 64)) // 4) * 4, T)
    cuts = {T * i // W for i in range(1, W)}
    seg = np.cumsum(np.repeat(nt, w.Hkv))
    cuts |= {int(x) for x in seg[:-1] if 0 < x < T}
    return len(cuts) + 1


def decode_leg(args, fa, workloads, torch, dev, stream):
    """Decode against an FP8 K/V cache: attn_fp8_decode (range kernel + merge)
    with the cache and the new queries already quantised and resident in HBM.
    HBM-bound: reported as the K/V cache bytes read per second and as all
    algorithmic bytes (cache codes and descales, queries, partials written and
    read back, outputs) per second against the 8 TB/s peak."""
    import numpy as np
    out = {}
    for name in DECODE_NAMES:
        w = workloads.DECODE_WORKLOADS[name]
        q, k, v = (torch.from_numpy(x).to(dev) for x in workloads.generate_decode_workload(w))
        _, k8, v8, _, kd, vd = fa.quantize_qkv_fp8(k, k, v, scale_block=w.scale_block, hadamard=w.hadamard,
                                                   seed=w.sign_seed)
        q8, _, _, qd, _, _ = fa.quantize_qkv_fp8(q, q, q, scale_block=w.scale_block, hadamard=w.hadamard,
                                                 seed=w.sign_seed)
        del q, k, v
        sl_np = w.seqlens()
        sl = torch.from_numpy(sl_np).to(dev)
        split = fa.attn_fp8_decode_split(w.B, w.Hkv, w.Ncap, args.decode_split)
        ws = torch.empty(fa.attn_fp8_decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.Sq, w.Ncap, w.D, args.decode_split),
                         dtype=torch.uint8, device=dev)
        o = torch.empty((w.B, w.Hq, w.Sq, w.D), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)

        def call():
            fa.attn_fp8_decode(q8, qd, k8, v8, kd, vd, sl, scale_block=w.scale_block, hadamard=w.hadamard,
                               causal=w.causal, split=args.decode_split, out=(o, lse), workspace=ws)

        for _ in range(5):
            call()
        n = max(20, args.steps)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(n):
            call()
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / n
        L = sl_np.astype(np.int64)
        kv = w.kv_bytes()
        mq = (w.Hq // w.Hkv) * w.Sq
        total = (kv + 2 * 4 * w.Hkv * int((-(-L // w.scale_block)).sum()) + w.B * w.Hq * w.Sq * (w.D + 4)
                 + 2 * decode_partials(w, L, split) * mq * (w.D + 2) * 4 + w.B * w.Hq * w.Sq * (2 * w.D + 4))
        out[name] = {
            "workload": f"B{w.B} Hq{w.Hq} Hkv{w.Hkv} Sq{w.Sq} D{w.D} cache {w.Ncap}, lengths "
                        f"{int(L.min())}..{int(L.max())} (mean {int(L.mean())}), scale block {w.scale_block}",
            "us": round(ms * 1e3, 2), "schedule": f"fixed ranges of {split} keys" if split else "balanced shares",
            "kv_cache_gbs": round(kv / (ms * 1e-3) / 1e9, 1),
            "algorithmic_gbs": round(total / (ms * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(total / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "tflops": round(w.flops() / (ms * 1e-3) / 1e12, 2),
        }
        del q8, k8, v8, qd, kd, vd, ws
    return out


PACKED_NAMES = ("packed_skewed_causal", "packed_long_causal", "packed_equal_causal", "packed_skewed")


def packed_leg(args, fa, workloads, torch, dev, stream):
    """Packed variable-length documents (FLAMIA's packed workloads: 16 heads,
    d = 128, T = 131072): one step = quantize_qkv_fp8_varlen +
    attn_fp8_fwd_varlen (schedule kernel + attention), inputs resident in HBM.
    Also the attention alone in longest-first and in natural (document) order.
    Every workload here draws the same tensors; only the document lengths differ."""
    import numpy as np
    out = {}
    w0 = workloads.PACKED_WORKLOADS[PACKED_NAMES[0]]
    q, k, v = (torch.from_numpy(x).to(dev) for x in workloads.generate_packed_workload(w0))
    o = torch.empty((w0.H, w0.T, w0.D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w0.H, w0.T), dtype=torch.float32, device=dev)
    steps = max(5, args.steps // 4)
    for name in PACKED_NAMES:
        w = workloads.PACKED_WORKLOADS[name]
        assert (w.kind, w.H, w.T, w.D, w.data_seed) == (w0.kind, w0.H, w0.T, w0.D, w0.data_seed)
        cu_np = w.cu_seqlens()
        cu = torch.from_numpy(cu_np).to(dev)
        nd = len(cu_np) - 1
        ws = torch.empty(fa.attn_fp8_varlen_workspace_bytes(w.T, nd), dtype=torch.uint8, device=dev)
        qq = fa.quantize_qkv_fp8_varlen(q, k, v, cu, scale_block=w.scale_block, hadamard=w.hadamard,
                                        seed=w.sign_seed)

        def quant():
            fa.quantize_qkv_fp8_varlen(q, k, v, cu, scale_block=w.scale_block, hadamard=w.hadamard,
                                       seed=w.sign_seed, out=qq)

        def attn(order="longest_first"):
            fa.attn_fp8_fwd_varlen(*qq, cu, scale_block=w.scale_block, hadamard=w.hadamard, causal=w.causal,
                                   out=(o, lse), order=order, workspace=ws)

        def timed(fn, n):
            for _ in range(2):
                fn()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(n):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / n

        step_ms = timed(lambda: (quant(), attn()), steps)
        attn_ms = timed(attn, steps)
        nat_ms = timed(lambda: attn("natural"), steps)
        quant_ms = timed(quant, steps)
        flops = w.flops()
        lens = np.diff(cu_np)
        out[name] = {
            "workload": f"H{w.H} T{w.T} D{w.D} {'causal' if w.causal else 'non-causal'}, {nd} documents "
                        f"({w.mix}, lengths {int(lens.min())}..{int(lens.max())}), scale block {w.scale_block}, "
                        f"{w.kind} inputs",
            "tflops_step": round(flops / (step_ms * 1e-3) / 1e12, 2), "ms_step": round(step_ms, 4),
            "attn_tflops": round(flops / (attn_ms * 1e-3) / 1e12, 2), "attn_ms": round(attn_ms, 4),
            "attn_natural_order_ms": round(nat_ms, 4),
            "longest_first_speedup": round(nat_ms / attn_ms, 3),
            "quantiser_ms": round(quant_ms, 4),
        }
    return out


def hipcc_version():
    import subprocess
    try:
        out = subprocess.run(["/opt/rocm/bin/hipcc", "--version"], capture_output=True, text=True, timeout=20).stdout
        return next((l.strip() for l in out.splitlines() if "HIP version" in l), None)
    except (OSError, subprocess.SubprocessError):
        return None


def cpu_leg(w, q_np, k_np, v_np, o_gpu, ob_gpu, osch_gpu, omx_gpu, ofl_gpu, om32_gpu):
    """Oracle leg: time the FP64 reference on a bounded sample of the workload on
    the host cores and use the same reference rows for the accuracy report."""
    import numpy as np

    from oracle import attention as oatt

    cores = len(os.sched_getaffinity(0))
    # whole heads (every query row), in a fixed order, until ~12 s of CPU time or 64 heads
    order = [(b, h) for h in range(w.H) for b in range(w.B)]
    order = order[::max(1, len(order) // 64)][:64]
    rows = np.arange(w.N)
    t0 = time.perf_counter()
    refs, heads = [], []
    for (b, h) in order:
        sl = (slice(b, b + 1), slice(h, h + 1))
        refs.append(oatt.reference_attention(q_np[sl], k_np[sl], v_np[sl], w.causal, rows=rows))
        heads.append((b, h))
        if time.perf_counter() - t0 > 12.0:
            break
    cpu_s = time.perf_counter() - t0
    # BLAS threads actually used, and one core alone on 1024 query rows of one head
    blas_threads = None
    single = None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        blas_threads = max((i["num_threads"] for i in blas), default=None)
        with threadpool_limits(1):
            r1 = np.arange(1024)
            t1 = time.perf_counter()
            oatt.reference_attention(q_np[:1, :1], k_np[:1, :1], v_np[:1, :1], w.causal, rows=r1)
            s1 = time.perf_counter() - t1
        p1 = sum(int(r) + 1 for r in r1) if w.causal else len(r1) * w.N
        single = {"gflops": round(4 * w.D * p1 / s1 / 1e9, 2), "sample": f"1 thread, 1024 query rows x {w.N} keys"}
    except ImportError:
        pass
    used = cores if blas_threads is None else min(cores, blas_threads)
    if w.causal:
        pairs = sum(int(r) + 1 for r in rows)
    else:
        pairs = len(rows) * w.N
    cpu_flops = 4 * w.D * pairs * len(heads)
    e8, e16, es, emx, efl, em32, ref_all = [], [], [], [], [], [], []
    for (b, h), (orf, _) in zip(heads, refs):
        g8 = o_gpu[b, h][rows].float().cpu().numpy().astype(np.float64)
        g16 = ob_gpu[b, h][rows].float().cpu().numpy().astype(np.float64)
        gs = osch_gpu[b, h][rows].float().cpu().numpy().astype(np.float64)
        e8.append((g8 - orf[0, 0]).ravel())
        e16.append((g16 - orf[0, 0]).ravel())
        es.append((gs - orf[0, 0]).ravel())
        gm = omx_gpu[b, h][rows].float().cpu().numpy().astype(np.float64)
        gf = ofl_gpu[b, h][rows].float().cpu().numpy().astype(np.float64)
        efl.append((gf - orf[0, 0]).ravel())
        emx.append((gm - orf[0, 0]).ravel())
        g32 = om32_gpu[b, h][rows].float().cpu().numpy().astype(np.float64)
        em32.append((g32 - orf[0, 0]).ravel())
        ref_all.append(orf[0, 0].ravel())
    e8, e16, es, ra = np.concatenate(e8), np.concatenate(e16), np.concatenate(es), np.concatenate(ref_all)
    emx = np.concatenate(emx)
    efl = np.concatenate(efl)
    em32 = np.concatenate(em32)
    rmse8 = float(np.sqrt(np.mean(e8 ** 2)))
    rmse16 = float(np.sqrt(np.mean(e16 ** 2)))
    rmses = float(np.sqrt(np.mean(es ** 2)))
    cos = lambda e: float(np.dot(ra + e, ra) / (np.linalg.norm(ra + e) * np.linalg.norm(ra)))
    return {
        "accuracy": {"sample": f"{len(heads)} heads x {len(rows)} query rows vs FP64 exact attention",
                     "fp8_rmse": rmse8, "fp8_max_err": float(np.max(np.abs(e8))), "fp8_cosine": cos(e8),
                     "bf16_rmse": rmse16, "bf16_max_err": float(np.max(np.abs(e16))), "bf16_cosine": cos(e16),
                     "ratio_fp8_to_bf16_rmse": rmse8 / rmse16 if rmse16 > 0 else None,
                     "fp8_schraudolph_rmse": rmses, "fp8_schraudolph_cosine": cos(es),
                     "fp8_mx_rmse": float(np.sqrt(np.mean(emx ** 2))), "fp8_mx_cosine": cos(emx),
                     "fp8_mx_schraudolph_rmse": float(np.sqrt(np.mean(efl ** 2))),
                     "fp8_mx_schraudolph_cosine": cos(efl),
                     "fp8_mx32_rmse": float(np.sqrt(np.mean(em32 ** 2))), "fp8_mx32_cosine": cos(em32),
                     "bound_ratio": 2.0, "rms_o": float(np.sqrt(np.mean(ra ** 2)))},
        "cpu_baseline": {"value": round(cpu_flops / cpu_s / 1e12, 6), "unit": "TFLOP/s", "cores": used,
                         "kind": "oracle", "cores_available": cores, "single_thread": single,
                         "sample": f"FP64 exact attention (numpy BLAS) of {len(heads)} whole heads "
                                   f"({len(rows)} queries x {w.N} keys each), {cpu_s:.1f} s wall"},
    }


if __name__ == "__main__":
    sys.exit(main())

#!/usr/bin/env python3
"""Throughput of the LUT-based approximate FP32 GEMM on one MI355X.

Default workload: one approximate GEMM C = A B with m = n = k = 8192, A and B
~ N(0, 1) (seeded, synthetic), and the M = 8 table of the exact mantissa
product with a seeded +/-1 perturbation of every entry. A step is one
``approx_gemm`` call (decode pass + GEMM kernel) with the inputs already in
HBM. Other workloads (--config 1, 2, 3, 5) are available for reference runs.

Prints ONE JSON line: the metric (G approximate MAC/s over K timed steps),
the GEMM kernel's roofline record (timed with HIP events inside the library,
on the stream the kernel runs on, over K more steps that follow the timed
ones) and the oracle's single-thread CPU throughput on a bounded sample of the
same workload.

--multiplier native runs the same workload with the library's native
multiplier (the FP32 fused multiply-add in place of the table: ApproxTrain
Section V / Fig. 6 compare the simulated multiplier against the native one);
--multiplier library times torch.matmul in FP32 on the GEMM workloads, for
context. --table-bits M (9..11: tables in global memory), --exp-bits E
(formats with fewer exponent bits) and --gemv [--rows R] (batch-1 or
few-row inference through the row-vector kernel) time the other parts of
the library. None of these is the headline.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X figures used by the roofline record
CUS, LANES_PER_CU, CLOCK_HZ = 256, 64, 2.4e9
VALU_PEAK_TOPS = CUS * LANES_PER_CU * CLOCK_HZ / 1e12     # 39.32 T 32-bit lane-ops/s
OPS_PER_MAC = 3                                           # address, assemble, accumulate
HBM_PEAK_GBS = 8000.0
# LDS: 128 bytes per clock per CU, i.e. 32 four-byte lanes: one 16-bit table
# lookup per lane
LDS_PEAK_LOOKUPS = CUS * 32 * CLOCK_HZ / 1e12             # 19.66 T lookups/s
# lookups/s that the table rows the kernel reads sustain, measured by the
# LDS probe (python3 bench.py --lds-probe): random rows of one 256-byte column
# at M = 7 (two bank rows: conflicts); at M = 8, rows of normally distributed
# mantissas read from the 640-byte columns with second copies, the copy of
# each row chosen per half-wave as the decode pass does
LDS_LOOKUP_CEILING = {7: 9.39, 8: 8.31}
LDS_CEILING_PATTERN = {7: "random rows of a 256-byte column",
                       8: "normal-mantissa rows, 640-byte columns with second copies chosen per half-wave"}
FP32_MFMA_PEAK_TFLOPS = 157.3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    p = os.path.join(ROOT, "approximate_multiplier_dnn_amd", "csrc", "kernels.hip")
    with open(p, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def build_lds_probe():
    """The LDS lookup-rate probe (lds_probe.hip, beside this script), built
    into _build/ with hipcc when missing or older than its sources."""
    import subprocess
    src = os.path.join(ROOT, "lds_probe.hip")
    dep = os.path.join(ROOT, "approximate_multiplier_dnn_amd", "csrc", "replica.h")
    out = os.path.join(ROOT, "_build", "lds_probe")
    if not os.path.exists(out) or os.path.getmtime(out) < max(os.path.getmtime(src), os.path.getmtime(dep)):
        os.makedirs(os.path.dirname(out), exist_ok=True)
        subprocess.run(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang",
                        "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", ROOT, "-o", out, src], check=True)
    return out


def traffic_record(workload):
    """HBM bytes per GEMM-kernel launch from the committed counter summary,
    if it was taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f).get(workload)
    if not rec or rec.get("kernel_sha") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def build_workload(config, am, torch, mult="table", table_bits=0, gemv=False, gemv_rows=1):
    from datagen import configs as cfg
    from datagen import PERTURB_SEED, pm_one

    model, M, pert = cfg.lut_spec(config)
    if table_bits:                     # the same table recipe at another mantissa width
        M = table_bits
        if pert is not None:
            pert = pm_one(PERTURB_SEED, 1 << (2 * M))
    if mult == "table":
        lut = am.approx_lut_build(am.MODEL_EXACT if model == "exact" else am.MODEL_MITCHELL, M, pert)
        am.approx_lut_load(lut, M)
    else:
        am.approx_native_load()
        lut, M = None, 0
    if mult == "library" and config not in (1, 4):
        raise SystemExit("--multiplier library covers the square GEMM workloads (1 and 4) only")
    d = lambda a: torch.from_numpy(a).cuda()
    info = {}
    if config in (1, 4):
        size = 64 if config == 1 else 8192
        A, B = cfg.gemm_square(config, size)
        rows = gemv_rows if gemv else size     # --gemv: batch-1 (or few-row) inference through the same B
        A = A[:rows].copy()
        Ad, Bd = d(A), d(B)
        Cd = torch.empty((rows, size), dtype=torch.float32, device="cuda")

        def step():
            if mult == "library":
                torch.matmul(Ad, Bd, out=Cd)
            else:
                am.approx_gemm(0, 0, rows, size, size, Ad, size, Bd, size, Cd, size)

        workload = f"gemm_{size}x{size}x{size}_lut_m{M}_{'perturbed' if pert is not None else model}"
        if mult != "table":
            workload = f"gemm_{size}x{size}x{size}_" + ("native_fp32_fma" if mult == "native" else "torch_matmul_fp32")
        if gemv:
            workload = workload.replace(f"gemm_{size}x", f"gemv_{rows}x", 1)
        info = dict(m=size, n=size, k=size, table=f"{model} M={M}" + (" +-1 perturbed" if pert is not None else ""))
        if mult != "table":
            info["table"] = "none (native FP32 multiplier)" if mult == "native" else "none (torch.matmul FP32)"
        host = dict(A=A, B=B, lut=lut, M=M, macs=rows * size * size)
        info["m"] = rows
    elif config == 2:
        layers = cfg.mlp_tensors()
        dev_layers = [tuple(d(t) for t in L) for L in layers]
        calls = []
        for (name, ta, tb, m, n, k, an, bn) in cfg.mlp_gemms():
            X, W, dY = dev_layers[int(name[-1])]
            ops = {"X": X, "W": W, "dY": dY}
            A, B = ops[an], ops[bn]
            C = torch.empty((m, n), dtype=torch.float32, device="cuda")
            calls.append((ta, tb, m, n, k, A, A.shape[1], B, B.shape[1], C, n))

        # A training step's dependencies: the forward chain, then per layer
        # (top down) the input gradient on this stream and the weight
        # gradient, which needs the layer's output gradient, on a second one.
        names = [g[0] for g in cfg.mlp_gemms()]
        byname = dict(zip(names, calls))
        nl = len(names) // 3
        side = torch.cuda.Stream()
        evs = [torch.cuda.Event() for _ in range(nl + 1)]

        def step():
            cur = torch.cuda.current_stream()
            for l in range(nl):
                am.approx_gemm(*byname[f"fwd{l}"], stream=cur)
            evs[0].record(cur)
            for i, l in enumerate(reversed(range(nl))):
                side.wait_event(evs[i])
                am.approx_gemm(*byname[f"wgrad{l}"], stream=side)
                am.approx_gemm(*byname[f"dgrad{l}"], stream=cur)
                evs[i + 1].record(cur)
            cur.wait_stream(side)

        workload = "mlp_784-1024-1024-10_b256_fwd_dgrad_wgrad_" + ("lut_m7_mitchell" if lut is not None else "native_fp32_fma")
        info = dict(batch=256, widths=[784, 1024, 1024, 10])
        host = dict(layers=layers, lut=lut, M=M)
    elif config == 3:
        s = cfg.CONV_SHAPE
        x, w, dy = cfg.conv_tensors()
        xd, wd, dyd = d(x), d(w), d(dy)
        N, H, W, C, K, R, S = s["N"], s["H"], s["W"], s["C"], s["K"], s["R"], s["S"]
        st, pd = s["stride"], s["pad"]
        y = torch.empty((N, H, W, K), dtype=torch.float32, device="cuda")
        dx = torch.empty((N, H, W, C), dtype=torch.float32, device="cuda")
        dw = torch.empty((R, S, C, K), dtype=torch.float32, device="cuda")

        def step():
            am.approx_conv2d_fwd(N, H, W, C, K, R, S, st, pd, xd, wd, y)
            am.approx_conv2d_dgrad(N, H, W, C, K, R, S, st, pd, dyd, wd, dx)
            am.approx_conv2d_wgrad(N, H, W, C, K, R, S, st, pd, xd, dyd, dw)

        workload = "conv2d_3x3_s1_p1_nhwc_128x32x32x64_to_64_fwd_dgrad_wgrad_" + (
            "lut_m7_mitchell" if lut is not None else "native_fp32_fma")
        info = dict(N=N, H=H, W=W, C=C, K=K, R=R, S=S)
        host = dict(x=x, w=w, dy=dy, lut=lut, M=M)
    elif config == 5:
        s = cfg.MHA_SHAPE
        Bz, T, D, Hh = s["batch"], s["seq"], s["d_model"], s["heads"]
        dh = D // Hh
        X, Wqkv, Wo = cfg.mha_tensors()
        Xd, Wqkvd, Wod = d(X), d(Wqkv), d(Wo)
        qkv = torch.empty((Bz * T, 3 * D), dtype=torch.float32, device="cuda")
        S_ = torch.empty((Bz, Hh, T, T), dtype=torch.float32, device="cuda")
        O = torch.empty((Bz * T, D), dtype=torch.float32, device="cuda")
        Y = torch.empty((Bz * T, D), dtype=torch.float32, device="cuda")

        # per (sequence, head) pointers into the fused QKV buffer, the score
        # and output tensors: one batched call per product stage
        pairs = [(b, h) for b in range(Bz) for h in range(Hh)]
        base, f = qkv.data_ptr(), 4
        q_ptr = am.pointer_array([base + f * (b * T * 3 * D + h * dh) for b, h in pairs])
        k_ptr = am.pointer_array([base + f * (b * T * 3 * D + D + h * dh) for b, h in pairs])
        v_ptr = am.pointer_array([base + f * (b * T * 3 * D + 2 * D + h * dh) for b, h in pairs])
        s_ptr = am.pointer_array([S_.data_ptr() + f * (b * Hh + h) * T * T for b, h in pairs])
        P = torch.empty_like(S_)
        p_ptr = am.pointer_array([P.data_ptr() + f * (b * Hh + h) * T * T for b, h in pairs])
        o_ptr = am.pointer_array([O.data_ptr() + f * (b * T * D + h * dh) for b, h in pairs])
        nb = len(pairs)

        def step():
            am.approx_gemm(0, 0, Bz * T, 3 * D, D, Xd, D, Wqkvd, 3 * D, qkv, 3 * D)
            am.approx_gemm_batched(0, 1, T, T, dh, q_ptr, 3 * D, k_ptr, 3 * D, s_ptr, T, nb)
            torch.softmax(S_ * (1.0 / dh ** 0.5), dim=-1, out=P)
            am.approx_gemm_batched(0, 0, T, dh, T, p_ptr, T, v_ptr, 3 * D, o_ptr, D, nb)
            am.approx_gemm(0, 0, Bz * T, D, D, O, D, Wod, D, Y, D)

        workload = "mha_b16_s512_d768_h12_qkv_qk_pv_out_" + ("lut_m7_mitchell" if lut is not None else "native_fp32_fma")
        info = dict(batch=Bz, seq=T, d_model=D, heads=Hh, note="softmax between the products is in the step time")
        host = dict(X=X, Wqkv=Wqkv, lut=lut, M=M)
    else:
        raise SystemExit(f"unknown config {config}")
    return step, workload, info, host


def cpu_baseline(config, host):
    """The oracle, single-threaded, on a bounded sample of the workload."""
    import numpy as np

    import oracle
    from datagen import configs as cfg

    t0 = time.perf_counter()
    if config in (1, 4):
        A, B = host["A"], host["B"]
        rows = min(64 if config == 1 else 32, A.shape[0])
        oracle.gemm(np.ascontiguousarray(A[:rows]), B, host["lut"], host["M"], E=host.get("E", 8))
        macs = rows * B.shape[0] * B.shape[1]
        sample = f"rows 0-{rows - 1} of the {A.shape[0]}x{B.shape[1]}x{B.shape[0]} GEMM ({macs:.3g} MACs)"
    elif config == 2:
        macs = 0
        for (name, ta, tb, m, n, k, an, bn) in cfg.mlp_gemms():
            X, W, dY = host["layers"][int(name[-1])]
            ops = {"X": X, "W": W, "dY": dY}
            if name.startswith("wgrad"):
                continue   # the three weight gradients are skipped to bound the sample
            oracle.gemm(ops[an], ops[bn], host["lut"], host["M"], transA=bool(ta), transB=bool(tb), E=host.get("E", 8))
            macs += m * n * k
        sample = f"the 6 forward and input-gradient GEMMs of one pass ({macs:.3g} MACs)"
    elif config == 3:
        x, w, dy = host["x"][:1], host["w"], host["dy"][:1]
        oracle.conv2d_fwd(x, w, host["lut"], host["M"], (1, 1), (1, 1), E=host.get("E", 8))
        oracle.conv2d_dgrad(dy, w, x.shape, host["lut"], host["M"], (1, 1), (1, 1), E=host.get("E", 8))
        oracle.conv2d_wgrad(x, dy, w.shape, host["lut"], host["M"], (1, 1), (1, 1), E=host.get("E", 8))
        macs = 3 * 32 * 32 * 64 * 9 * 64
        sample = f"image 0 of 128, fwd + dgrad + wgrad ({macs:.3g} MACs)"
    else:
        rows = 64
        X, Wqkv = host["X"], host["Wqkv"]
        oracle.gemm(np.ascontiguousarray(X[:rows]), Wqkv, host["lut"], host["M"], E=host.get("E", 8))
        macs = rows * Wqkv.shape[0] * Wqkv.shape[1]
        sample = f"rows 0-{rows - 1} of the QKV projection ({macs:.3g} MACs)"
    dt = time.perf_counter() - t0
    unit = "G approximate MAC/s" if host["lut"] is not None else "G MAC/s"
    return {"value": macs / dt / 1e9, "unit": unit, "cores": 1, "kind": "oracle",
            "sample": sample, "seconds": round(dt, 2)}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=4, help="workload 1-5 (4: 8192^3 GEMM, the headline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--table-bits", type=int, default=0,
                    help="build the workload's table at this mantissa width instead (1-11; 9-11 are read "
                         "from global memory)")
    ap.add_argument("--exp-bits", type=int, default=8,
                    help="exponent width E (1-8) of the approximate multiplier's format (1, E, M); operands are "
                         "cast to it before each product (8: FP32, the default)")
    ap.add_argument("--gemv", action="store_true",
                    help="with --config 1 or 4: one row of A (batch-1 inference), the row-vector kernel")
    ap.add_argument("--rows", type=int, default=1,
                    help="with --gemv: rows of A (small-batch inference, 1 to 64: 4-row blocks of the row-vector "
                         "kernel)")
    ap.add_argument("--multiplier", choices=("table", "native", "library"), default="table",
                    help="table: the approximate multiplier (default); native: the library's FP32 FMA in "
                         "the same kernels; library: torch.matmul FP32 (GEMM workloads only)")
    ap.add_argument("--lds-probe", action="store_true",
                    help="instead of the workload, run the LDS table-lookup rate probe")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of the workload, run one plain device copy of this many bytes "
                         "(calibrates the HBM byte counters used for roofline.traffic)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the library runs each call on one GPU and has no sharding across GPUs", file=sys.stderr)
        sys.exit(2)

    if args.lds_probe:
        import subprocess
        sys.exit(subprocess.run([build_lds_probe()]).returncode)

    import torch

    assert torch.cuda.is_available(), "no GPU"
    torch.cuda.set_device(0)
    if args.copy_bytes:
        n = args.copy_bytes // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n * 4, "read_bytes": n * 4, "written_bytes": n * 4}), flush=True)
        return

    import approximate_multiplier_dnn_amd as am
    from datagen import configs as cfg
    log(f"building workload {args.config} ...")
    torch.backends.cuda.matmul.allow_tf32 = False
    if args.gemv and args.config not in (1, 4):
        raise SystemExit("--gemv goes with the square GEMM workloads (--config 1 or 4)")
    if args.rows != 1 and not args.gemv:
        raise SystemExit("--rows goes with --gemv")
    if args.gemv and not 1 <= args.rows <= 64:
        raise SystemExit("--rows: 1 to 64")
    step, workload, info, host = build_workload(args.config, am, torch, args.multiplier, args.table_bits, args.gemv,
                                                args.rows)
    if args.exp_bits != 8:
        if args.multiplier != "table":
            raise SystemExit("--exp-bits applies to the table multiplier only")
        am.approx_exponent_bits_set(args.exp_bits)
        workload += f"_e{args.exp_bits}"
        info["exponent_bits"] = args.exp_bits
        host["E"] = args.exp_bits
    macs = host.get("macs") or cfg.macs(args.config)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed steps (the metric): nothing inside them but the steps themselves
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    # the same number of steps again with the library's HIP events around
    # every GEMM-kernel launch, on the stream it runs on (the roofline's
    # kernel time; the event records add a few microseconds per launch, so
    # they stay out of the metric's steps)
    am.approx_profile_read()           # drop anything recorded so far
    am.approx_profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    am.approx_profile_enable(False)
    launches, kern_ms = am.approx_profile_read()
    if args.multiplier == "library":   # torch.matmul runs on torch's stream: time it there
        launches, kern_ms = args.steps, ev0.elapsed_time(ev1)
    ms_per_step = dt * 1e3 / args.steps
    value = macs * args.steps / dt / 1e9
    log(f"{workload}: {ms_per_step:.3f} ms/step, {value:.1f} G MAC/s; "
        f"kernel {launches} launches, {kern_ms / max(launches, 1):.3f} ms avg")

    kern_s = kern_ms / 1e3
    mac_rate = macs * args.steps / kern_s if kern_s > 0 else 0.0     # MAC/s over kernel time
    if args.gemv and args.multiplier != "library":
        # the row-vector kernel streams B from HBM once per launch (one launch
        # takes all rows of A, in blocks of 4): algorithmic bytes per launch =
        # its rows of A + B read + its rows of C written
        per_step = max(launches // max(args.steps, 1), 1)
        rb = host["A"].shape[0] / per_step
        kk, nn = host["B"].shape
        nbytes = 4 * (rb * kk + kk * nn + rb * nn)
        achieved = nbytes / (kern_s / max(launches, 1)) / 1e9 if kern_s > 0 else 0.0
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "amx::gemv_kernel",
                    "kernel_ms_avg": round(kern_ms / max(launches, 1), 4),
                    "launches_per_step": launches // max(args.steps, 1),
                    "kernel_G_mac_per_s": round(mac_rate / 1e9, 1)}
    elif args.multiplier == "library":
        achieved = 2 * mac_rate / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 3), "peak": FP32_MFMA_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / FP32_MFMA_PEAK_TFLOPS, 4), "traffic": None,
                    "kernel": "torch.matmul (FP32)", "kernel_ms_avg": round(kern_ms / max(launches, 1), 4)}
    else:
        # roofline of the GEMM kernel: algorithmic lane-ops over kernel time
        ops = OPS_PER_MAC if args.multiplier == "table" else 1        # native: one FMA per MAC
        achieved = ops * mac_rate / 1e12
        roofline = {
            "bound": "alu",
            "achieved": round(achieved, 3),
            "peak": round(VALU_PEAK_TOPS, 2),
            "unit": "TOP/s",
            "frac": round(achieved / VALU_PEAK_TOPS, 4),
            "traffic": traffic_record(workload),
            "kernel": "amx::gemv_kernel" if args.config == 1 else "amx::main_kernel",
            "kernel_ms_avg": round(kern_ms / max(launches, 1), 4),
            "launches_per_step": launches // max(args.steps, 1),
            "ops_per_mac": ops,
            "kernel_G_mac_per_s": round(mac_rate / 1e9, 1),
        }
        if args.multiplier == "table" and host["M"] > 8:
            roofline["table"] = "global memory (M > 8 does not fit LDS)"
        elif args.multiplier == "table":
            # the second roof: one 16-bit LDS lookup per MAC
            lookups = mac_rate / 1e12
            M = host["M"]
            roofline["lds"] = {
                "achieved_T_lookups_per_s": round(lookups, 3),
                "peak_T_lookups_per_s": round(LDS_PEAK_LOOKUPS, 2),
                "frac": round(lookups / LDS_PEAK_LOOKUPS, 4),
                "measured_ceiling_T_per_s": LDS_LOOKUP_CEILING.get(M),
                "ceiling_pattern": LDS_CEILING_PATTERN.get(M),
                "frac_of_ceiling": round(lookups / LDS_LOOKUP_CEILING[M], 4)
                if M in LDS_LOOKUP_CEILING else None,
            }
    metric = {"table": "G approximate MAC/s (LUT-simulated FP32 GEMM)",
              "native": "G MAC/s (native FP32 multiplier, same kernels)",
              "library": "G MAC/s (torch.matmul FP32)"}[args.multiplier]
    rec = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "G approximate MAC/s" if args.multiplier == "table" else "G MAC/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": dict(workload=workload, **info),
        "roofline": roofline,
    }
    if not args.no_cpu_baseline and args.multiplier != "library":
        log("timing the oracle on a CPU sample ...")
        rec["cpu_baseline"] = cpu_baseline(args.config, host)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

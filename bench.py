"""Benchmark: one DeepSeekMoE layer step at DeepSeek-V3 shape on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload v3_bf16|v3_fp8|skew_balance|mid_bf16|tiny_fp32]
                    [--no-cpu-baseline] [--no-configs] [--no-probes] [--backward]
                    [--vendor-calibration]

A step is the whole hot path on one batch already resident in HBM:
route -> permute -> expert FFN (routed + shared) -> combine -> bias update.
Prints ONE JSON line.  `value` is tokens per second of the whole step;
`roofline` describes the dominant stage, the grouped expert GEMMs (gate/up
with fused SwiGLU, then down), timed live with HIP events on the stream they
run on, against the roofline (HBM or MFMA) that bounds its algorithmic work,
with the HBM traffic the rocprofv3 counter summaries under profiles/ record
for the same GEMM sources; `cpu_baseline` is the CPU oracle timed on a
bounded sample of the same workload on this host.  Unless --no-configs, the
line also carries `configs`: the FP8 workload (with its own roofline and
oracle time), the decode-sized skewed batch (bias-balancing trajectory and
the layer at T = 128) and the small workloads, measured after the headline;
for the launch-bound ones (T = 128 and the small layers) also as one HIP
graph replay per step (`graph_ms_per_step`).

--backward measures the layer's backward instead: a step is the four backward
calls -- combine backward, expert FFN backward (two dgrad and two wgrad GEMMs,
reading the a, b, h the training forward kept; FP8 workloads quantise every
GEMM operand), gate/centroid backward, input gradient --
on the state of one training forward step, reported as its own metric.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"bf16": 2516.6e12, "fp8": 5033.2e12, "hbm": 8.0e12}

METRIC = "MoE-layer fwd tokens/s at V3 shape; grouped-GEMM % of MFMA peak"
METRIC_BWD = "MoE-layer bwd tokens/s at V3 shape; expert-backward GEMM % of MFMA peak"


def ffn_flops(c):
    T, k, d, I, Is = c["T"], c["k"], c["d"], c["I"], c["Is"]
    return 6.0 * T * k * d * I + 6.0 * T * d * Is


def ffn_weight_bytes(c):
    eb = 1 if c.get("fp8") else 2
    return eb * (3.0 * c["N"] * c["d"] * c["I"] + 3.0 * c["d"] * c["Is"])


def ffn_bytes(c):
    """Algorithmic HBM bytes of one moe_expert_ffn call, each tensor read or
    written once: the expert weights (+ FP8 block scales), the permuted token
    rows and x (shared expert) read, h written and read back, y (routed and
    shared) written.  Activations are E4M3 codes + 1x128 fp32 scales in the
    FP8 path, bf16 otherwise; y is bf16 in both."""
    T, k, d, I, Is, N = c["T"], c["k"], c["d"], c["I"], c["Is"], c["N"]
    TK = T * k
    fp8 = bool(c.get("fp8"))
    ab = 1 + 4.0 / 128 if fp8 else 2  # bytes per activation element (code + scale share)
    w = ffn_weight_bytes(c)
    if fp8:
        w += 4.0 * (N * (2 * I // 128) * (d // 128) + N * (d // 128) * (I // 128)
                    + (2 * Is // 128) * (d // 128) + (d // 128) * (Is // 128))
    acts = ab * (TK * d + T * d)          # x_perm, x read by gate/up
    acts += 2 * ab * (TK * I + T * Is)    # h written, then read by down
    acts += 2.0 * (TK * d + T * d)        # y_perm, y_shared written
    return w + acts


def ffn_bwd_flops(c, recompute=False):
    """dgrad down (2 M d I), dgrad up (4 M d I), wgrad down (2 M d I), wgrad up
    (4 M d I) for M = T*k routed rows, the same for the shared expert over T
    rows, and with recompute (always on FP8) also a, b (4 M d I)"""
    T, k, d, I, Is = c["T"], c["k"], c["d"], c["I"], c["Is"]
    f = 16.0 if recompute else 12.0
    return f * T * k * d * I + f * T * d * Is


def ffn_bwd_bytes(c, recompute=False):
    """Algorithmic HBM bytes of one moe_expert_ffn_backward call (bf16), each
    GEMM reading its operands and writing its result once: weights W2^T and
    W13^T (the dgrads), and W13 with recompute; x_perm, dY, a/b, h, da/db, dX
    and the weight gradients as each GEMM reads or writes them."""
    T, k, d, I, Is, N = c["T"], c["k"], c["d"], c["I"], c["Is"], c["N"]
    if c.get("fp8"):
        return ffn_bwd_bytes_fp8(c, recompute)
    def one(M, I, n):
        w = 2.0 * n * (d * I + 2 * I * d)                        # W2^T, W13^T read
        rec = 0.0
        if recompute:
            w += 2.0 * n * 2 * I * d                             # W13 read
            rec = 2.0 * (M * d + M * 2 * I + M * I)              # x in; a, b and h out
        dgd = 2.0 * (M * d + M * 2 * I + M * 2 * I)              # dY, a/b in; da/db out
        dgu = 2.0 * (M * 2 * I + M * d)                          # da/db in; dX out
        wgd = 2.0 * (M * d + M * I) + 2.0 * n * d * I            # dY, h in; dW2 out
        wgu = 2.0 * (M * 2 * I + M * d) + 2.0 * n * 2 * I * d    # da/db, x in; dW13 out
        return w + rec + dgd + dgu + wgd + wgu
    return one(T * k, I, N) + (one(T, Is, 1) if Is > 0 else 0.0)


def ffn_bwd_bytes_fp8(c, recompute=False):
    """Algorithmic HBM bytes of one moe_expert_ffn_backward_fp8 call: each GEMM
    reads its E4M3 operands (codes, plus 4 bytes of scale per 128 codes) and
    writes its result once, and each quantised operand is produced once from its
    bf16 tensor:  with recompute (W13, x codes -> a, b, h bf16), dY row tiles, dgrad
    down (W2^T, dY codes -> dh), SwiGLU' (dh, a, b -> [da db] bf16 and codes),
    dgrad up (W13^T, [da db] codes -> dX), the row-direction tiles of dY, h,
    [da db] and x (bf16 in, codes out), and the weight-gradient GEMMs (codes
    in, dW2 and dW13 bf16 out)."""
    T, k, d, I, Is, N = c["T"], c["k"], c["d"], c["I"], c["Is"], c["N"]
    q = 1 + 4.0 / 128  # code + scale share
    def one(M, I, n):
        w = n * (d * I + 2 * I * d) * q                             # W2^T, W13^T codes
        b = 0.0
        if recompute:
            w += n * 2 * I * d * q                                  # W13 codes
            b += q * M * d + 2.0 * M * 3 * I                        # x in, a/b/h out
        b += 2.0 * M * d + q * M * d                                # dY row tiles
        b += q * M * d + 2.0 * M * I                                # dgrad down
        b += 2.0 * M * 3 * I + 2.0 * M * 2 * I + q * M * 2 * I      # SwiGLU'
        b += q * M * 2 * I + 2.0 * M * d                            # dgrad up
        b += 2.0 * M * (2 * d + 3 * I) + q * M * (2 * d + 3 * I)    # row-direction tiles
        b += q * M * (2 * d + 3 * I) + 2.0 * n * 3 * I * d          # weight gradients
        return w + b
    return one(T * k, I, N) + (one(T, Is, 1) if Is > 0 else 0.0)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="v3_bf16")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward", action="store_true",
                    help="time the layer's backward (four calls) instead of the forward step")
    ap.add_argument("--no-configs", action="store_true",
                    help="measure the headline workload only (no v3_fp8, skew_balance, "
                         "tiny_fp32, mid_bf16 block)")
    ap.add_argument("--vendor-calibration", action="store_true",
                    help="time the vendor GEMM library (torch.bmm / torch._scaled_mm, i.e. "
                         "hipBLASLt) on the expert FFN's per-expert shapes and on large dense "
                         "GEMMs, print one JSON line, then exit")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the measured-peak probes (HBM read, MFMA loop)")
    ap.add_argument("--traffic-run", action="store_true",
                    help="run the expert FFN 3 times and a 1 GiB copy 3 times (for rocprofv3 "
                         "--pmc FETCH_SIZE / WRITE_SIZE passes), then exit")
    ap.add_argument("--counter-run", action="store_true",
                    help="run 1 + 2 layer steps, the bf16 and FP8 MFMA probes and a 1 GiB copy "
                         "3 times (for rocprofv3 --pmc passes over the whole step), then exit")
    ap.add_argument("--counter-summary", nargs=3, metavar=("MFMA_CSV", "FETCH_CSV", "WRITE_CSV"),
                    help="per-kernel MFMA busy share and HBM bytes of a --counter-run, then exit")
    ap.add_argument("--sq-summary", nargs=2, metavar=("PASS_A_CSV", "PASS_B_CSV"),
                    help="the expert GEMMs' SQ issue and stall counters from two --counter-run "
                         "passes (the SQ_PASSES counter sets), then exit")
    ap.add_argument("--stats-summary", metavar="KERNEL_STATS_CSV",
                    help="print the per-kernel table of a rocprofv3 --stats run, then exit")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise the two counter CSVs of a --traffic-run into the text "
                         "that profiles/ keeps, then exit")
    return ap.parse_args()


GEMM_SOURCES = ("gemm.hip", "gemm_common.h", "gemm_fp8.hip")
COPY_BYTES = 1 << 30
PROFILE_DIR = os.path.join(ROOT, "profiles")


def gemm_source_hash(backward=False):
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES + (("gemm_bwd.hip", "backward_fp8.hip") if backward else ()):
        with open(os.path.join(ROOT, "sparse_moe_layer_bias_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_file(workload, backward=False):
    return os.path.join(PROFILE_DIR, "expert_ffn%s_%s_traffic.txt" %
                        ("_backward" if backward else "", workload))


def recorded_traffic(workload, backward=False):
    """HBM bytes per expert-FFN (or expert-FFN backward) call recorded under
    profiles/, or None when absent or taken on GEMM sources other than the
    current ones."""
    path = traffic_file(workload, backward)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line:
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("gemm_source_hash") != gemm_source_hash(backward):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def traffic_summary(fetch_csv, write_csv, workload, backward=False):
    import csv
    import collections

    def per_kernel(path, counter):
        acc = collections.defaultdict(list)
        with open(path) as f:
            rows = [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        for r in rows:
            acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return acc

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")
    # the calibration copies are the last 3 dispatches of the copy kernel
    copy_k = [k for k in fetch if "copybuffer" in k.lower()]
    if not copy_k or len(fetch[copy_k[0]]) < 3:
        raise SystemExit("no calibration copy found")
    cf = sum(fetch[copy_k[0]][-3:]) / 3 * 1024.0
    cw = sum(write[copy_k[0]][-3:]) / 3 * 1024.0
    f_scale = COPY_BYTES / cf
    w_scale = COPY_BYTES / cw
    lines = []
    if backward and "fp8" in workload:
        # moe_expert_ffn_backward_fp8 launches several kernels more than once:
        # sum every dispatch of the last measured call (from its tile map to
        # the calibration copies)
        def ordered(path, counter):
            with open(path) as f:
                rows = [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]
            return sorted((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"]))
                          for r in rows)
        fo, wo = ordered(fetch_csv, "FETCH_SIZE"), ordered(write_csv, "WRITE_SIZE")
        wmap = {i: v for i, _, v in wo}
        starts = [j for j, (_, k, _) in enumerate(fo) if "ffn_tile_map" in k]
        j0 = starts[-1]
        j1 = next(j for j in range(j0, len(fo)) if "copybuffer" in fo[j][1].lower())
        per = collections.OrderedDict()
        for i, k, v in fo[j0:j1]:
            if "moe::" not in k:  # the calibration's own buffer fill
                continue
            e = per.setdefault(k, [0.0, 0.0, 0])
            e[0] += v * 1024.0 * f_scale
            e[1] += wmap.get(i, 0.0) * 1024.0 * w_scale
            e[2] += 1
        total = 0.0
        for k, (fb, wb, n) in per.items():
            total += fb + wb
            lines.append("kernel: %s | fetch %.4g B | write %.4g B | dispatches in the call %d" %
                         (k[:90], fb, wb, n))
        out = ["workload: %s" % workload,
               "calibration_copy_kernel: %s" % copy_k[0][:90],
               "calibration_fetch_scale: %.5f" % f_scale,
               "calibration_write_scale: %.5f" % w_scale]
        out += lines
        out += ["hbm_bytes_per_launch: %.6g" % total,
                "gemm_source_hash: %s" % gemm_source_hash(backward)]
        return "\n".join(out)
    # the kernels of one call; each averaged over its last 3 dispatches, the
    # 3 measured calls (the backward's setup also runs forward kernels)
    if backward:  # with the training forward's saved activations: no recompute (mode 2)
        ffn = [k for k in fetch if "wgrad" in k or "ffn_tile_map" in k or
               any("ffn_gemm_bf16_kernel<%d," % m in k for m in (1, 3))]
    else:
        ffn = [k for k in fetch if "ffn_" in k]
    total = 0.0
    for k in ffn:
        fl, wl = fetch[k][-3:], write.get(k, [0.0])[-3:]
        fb = sum(fl) / len(fl) * 1024.0 * f_scale
        wb = sum(wl) / len(wl) * 1024.0 * w_scale
        total += fb + wb
        lines.append("kernel: %s | fetch %.4g B | write %.4g B | dispatches averaged %d" %
                     (k[:90], fb, wb, len(fl)))
    out = ["workload: %s" % workload,
           "calibration_copy_kernel: %s" % copy_k[0][:90],
           "calibration_fetch_scale: %.5f" % f_scale,
           "calibration_write_scale: %.5f" % w_scale]
    out += lines
    out += ["hbm_bytes_per_launch: %.6g" % total,
            "gemm_source_hash: %s" % gemm_source_hash(backward)]
    return "\n".join(out)


def stats_summary(path):
    import csv
    rows = list(csv.DictReader(open(path)))
    out = ["%-72s %6s %12s %12s %7s" % ("kernel", "calls", "avg_us", "total_us", "pct")]
    for r in rows:
        out.append("%-72s %6s %12.1f %12.1f %7.2f" % (
            r["Name"][:72], r["Calls"], float(r["AverageNs"]) / 1e3,
            float(r["TotalDurationNs"]) / 1e3, float(r["Percentage"])))
    return "\n".join(out)


def counter_run(cfg, layer, dev):
    """One warm step, two counted steps, then the calibration kernels: the MFMA
    probes (a register-resident MFMA loop keeps the MFMA pipe busy all the
    time) and a 1 GiB device copy (known bytes)."""
    import torch
    from sparse_moe_layer_bias_amd import probe
    x, E = dev["x"], dev["centroids"]
    bias = dev["bias"].clone()
    layer.forward(x, E, bias)
    torch.cuda.synchronize()
    for _ in range(2):
        layer.forward(x, E, bias)
    torch.cuda.synchronize()
    probe.mfma_rate("bf16", iters=2000, blocks=256, reps=1)
    probe.mfma_rate("fp8", iters=1000, blocks=256, reps=1)
    a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()


def counter_summary(mfma_csv, fetch_csv, write_csv, workload):
    """Per libmoe kernel of a --counter-run: average duration, MFMA busy share
    and HBM bytes.  SQ_VALU_MFMA_BUSY_CYCLES / GRBM_GUI_ACTIVE is expressed
    relative to the MFMA probe of the same dtype (busy every cycle: 100%);
    FETCH_SIZE / WRITE_SIZE are scaled so that the 1 GiB copy reads / writes
    1 GiB."""
    import csv
    import collections

    def load(path, counters):
        per = collections.defaultdict(lambda: collections.defaultdict(list))
        dur = collections.defaultdict(list)
        seen = set()
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] not in counters:
                    continue
                per[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
                key = (r["Kernel_Name"], r["Dispatch_Id"])
                if key not in seen:
                    seen.add(key)
                    dur[r["Kernel_Name"]].append(
                        (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
        return per, dur

    m, mdur = load(mfma_csv, ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"))
    fe, _ = load(fetch_csv, ("FETCH_SIZE",))
    wr, _ = load(write_csv, ("WRITE_SIZE",))

    def busy(k):
        b = sum(m[k]["SQ_VALU_MFMA_BUSY_CYCLES"])
        g = sum(m[k]["GRBM_GUI_ACTIVE"])
        return b / g if g else 0.0

    probes = {dt: [k for k in m if "probe_mfma_kernel<%d>" % code in k]
              for dt, code in (("bf16", 1), ("fp8", 2))}
    ref = {dt: busy(ks[0]) for dt, ks in probes.items() if ks}
    copy_k = [k for k in fe if "copybuffer" in k.lower()]
    if not copy_k or not ref:
        raise SystemExit("calibration kernels missing")
    f_scale = COPY_BYTES / (sum(fe[copy_k[0]]["FETCH_SIZE"][-3:]) / 3 * 1024.0)
    w_scale = COPY_BYTES / (sum(wr[copy_k[0]]["WRITE_SIZE"][-3:]) / 3 * 1024.0)
    fp8 = "fp8" in workload
    out = ["workload: %s" % workload,
           "calibration: MFMA busy/active of the probes = bf16 %.4g, fp8 %.4g (= 100%%); "
           "byte scales fetch %.5f, write %.5f (1 GiB copy)" % (ref.get("bf16", 0), ref.get("fp8", 0),
                                                              f_scale, w_scale),
           "%-58s %5s %10s %9s %10s %10s %9s %7s" % ("kernel", "disp", "avg_us", "mfma_busy",
                                                    "read_MB", "write_MB", "GB/s", "%8TB/s")]
    for k in m:
        if "moe::" not in k or "probe" in k:
            continue
        n = len(mdur[k])
        d = sum(mdur[k]) / n
        bz = busy(k) / ref["fp8" if ("fp8" in k or fp8 and "gemm" in k) else "bf16"]
        rb = sum(fe[k]["FETCH_SIZE"]) / max(len(fe[k]["FETCH_SIZE"]), 1) * 1024.0 * f_scale
        wb = sum(wr[k]["WRITE_SIZE"]) / max(len(wr[k]["WRITE_SIZE"]), 1) * 1024.0 * w_scale
        gbs = (rb + wb) / d / 1e9 if d > 0 else 0.0
        out.append("%-58s %5d %10.1f %8.1f%% %10.1f %10.1f %9.0f %6.1f%%" % (
            k.replace("moe::", "")[:58], n, d * 1e6, 100 * bz, rb / 1e6, wb / 1e6, gbs,
            100 * gbs / (PEAK["hbm"] / 1e9)))
    return "\n".join(out)


SQ_PASSES = (
    ("SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS",
     "SQ_ACTIVE_INST_VMEM", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VALU", "GRBM_GUI_ACTIVE"),
    ("SQ_VMEM_TA_ADDR_FIFO_FULL", "SQ_VMEM_TA_CMD_FIFO_FULL", "SQ_LDS_BANK_CONFLICT",
     "SQ_LDS_DATA_FIFO_FULL", "SQ_LDS_CMD_FIFO_FULL", "SQ_INST_LEVEL_VMEM",
     "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES", "GRBM_GUI_ACTIVE"))


def sq_summary(csv_a, csv_b, workload):
    """The expert GEMMs' issue and stall counters of two --counter-run passes
    (SQ_PASSES): each counter's mean per dispatch, and the shares of wave time
    spent waiting on a counter (SQ_WAIT_ANY), waiting to issue
    (SQ_WAIT_INST_ANY), issuing VALU (MFMA included) and LDS instructions, the
    share of MFMA-busy cycles in which the VALU also ran, and LDS bank
    conflicts per LDS-active cycle."""
    import csv
    import collections
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    for tag, path in (("A", csv_a), ("B", csv_b)):
        with open(path) as f:
            for r in csv.DictReader(f):
                k = r["Kernel_Name"]
                if "ffn_gemm" not in k:
                    continue
                c = r["Counter_Name"] + ("_" + tag if r["Counter_Name"] == "GRBM_GUI_ACTIVE" else "")
                per[k.split("(")[0].replace("void ", "").replace("moe::", "")][c].append(
                    float(r["Counter_Value"]))
    out = ["workload: %s" % workload]
    for k, cs in per.items():
        m = {c: sum(v) / len(v) for c, v in cs.items()}
        out.append("kernel: %s  (dispatches averaged: %d)" % (k, len(cs["SQ_WAVE_CYCLES"])))
        out += ["  %-30s %16.0f" % (c, m[c]) for c in sorted(m)]
        w = m["SQ_WAVE_CYCLES"]
        for name, num, den in (("wait_any / wave_cycles", "SQ_WAIT_ANY", w),
                               ("wait_inst_any / wave_cycles", "SQ_WAIT_INST_ANY", w),
                               ("active_valu / wave_cycles", "SQ_ACTIVE_INST_VALU", w),
                               ("active_lds / wave_cycles", "SQ_ACTIVE_INST_LDS", w),
                               ("mfma_coexec / mfma_busy", "SQ_VALU_MFMA_COEXEC_CYCLES",
                                m["SQ_VALU_MFMA_BUSY_CYCLES"]),
                               ("lds_bank_conflict / active_lds", "SQ_LDS_BANK_CONFLICT",
                                m["SQ_ACTIVE_INST_LDS"])):
            out.append("  %-32s %.3f" % (name, m[num] / den if den else 0.0))
    return "\n".join(out)


def traffic_run(cfg, layer, dev, backward=False):
    import torch
    x = dev["x"]
    layer.route(x, dev["centroids"], dev["bias"])
    layer.permute(x)
    torch.cuda.synchronize()
    if backward:
        import moe_inputs
        dout = moe_inputs.make_upstream_grad(cfg, 0, "cuda")
        layer.expert_ffn(x)
        layer.combine(x)
        layer.backward(dout, x, dev["centroids"])  # buffers, and the dy_perm the FFN reads
        torch.cuda.synchronize()
        for _ in range(3):
            layer.expert_ffn_backward(dout, x)
    else:
        for _ in range(3):
            layer.expert_ffn(x)
    a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()


def cpu_baseline(cfg, dev, log, rows=4096):
    """Time the oracle (untuned) on a bounded sample of the workload and scale
    to tokens/s: route, permute and combine on S tokens; the SwiGLU expert on R
    rows of expert 0, counted k+1 times per token (k routed rows + the shared
    expert row)."""
    import numpy as np

    import moe_inputs
    from oracle import oracle as orc

    S = cfg["T"]          # every token of the batch for route / permute / combine
    R = min(rows, S)      # rows through the oracle's SwiGLU expert
    xs = moe_inputs.to_host(dev["x"][:S])
    E = moe_inputs.to_host(dev["centroids"])
    b = moe_inputs.to_host(dev["bias"])
    w13 = moe_inputs.to_host(dev["w13"][0])
    w2 = moe_inputs.to_host(dev["w2"][0])
    orc.lib()
    t0 = time.perf_counter()
    r = orc.route(xs, E, b, cfg["k"], cfg["G"], cfg["TG"])
    t1 = time.perf_counter()
    off, src, dst = orc.permute(r["idx"], cfg["N"])
    xp = orc.gather_rows(xs, src)
    t2 = time.perf_counter()
    if cfg.get("fp8"):
        xq, xsc = orc.quant_act_fp8(xs)
        q13, s13 = orc.quant_weight_fp8(w13)
        q2, s2 = orc.quant_weight_fp8(w2)
        t3a = time.perf_counter()
        y = orc.swiglu_ffn_fp8(xq[:R], xsc[:R], q13, s13, q2, s2)
        t3 = time.perf_counter()
        ffn_s = t3 - t3a
    else:
        t3a = time.perf_counter()
        y = orc.swiglu_ffn(xs[:R], w13, w2)
        t3 = time.perf_counter()
        ffn_s = t3 - t3a
    ys = np.resize(y, (S, y.shape[1]))
    yp = np.resize(y, (S * cfg["k"], y.shape[1]))
    t4 = time.perf_counter()
    orc.combine(xs, ys, yp, r["gate"], dst, cfg["dtype"])
    orc.bias_update(r["counts"], S * cfg["k"], b)
    t5 = time.perf_counter()
    per_token = ((t1 - t0) + (t2 - t1) + (t5 - t4)) / S + ffn_s / R * (cfg["k"] + 1)
    cores = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    log("cpu oracle: route %.2fs permute %.3fs ffn(%d rows) %.2fs combine %.3fs -> %.4f s/token"
        % (t1 - t0, t2 - t1, R, ffn_s, t5 - t4, per_token))
    return {"value": 1.0 / per_token, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "route, permute, combine and bias update on all %d tokens of the batch; "
                      "the SwiGLU expert on %d rows of expert 0, its per-row time counted "
                      "k+1=%d times per token (k routed rows + the shared row)"
                      % (S, R, cfg["k"] + 1)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_layer(cfg, dev, log, single_thread=False):
    """The oracle's whole layer step (route, permute, every expert, combine)
    on the whole batch, no sample and no extrapolation -- for the small
    workloads, where it takes seconds.  With single_thread, also timed on one
    host thread."""
    import moe_inputs
    from oracle import oracle as orc

    h = {n: moe_inputs.to_host(v) for n, v in dev.items()}
    orc.lib()

    def run():
        t0 = time.perf_counter()
        orc.layer_forward(h, cfg)
        return time.perf_counter() - t0

    cores = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    dt = run()
    out = {"value": cfg["T"] / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "sample": "the whole layer step on all %d tokens" % cfg["T"], "cpu": cpu_model()}
    if single_thread:
        prev = orc.set_threads(1)
        try:
            dt1 = run()
        finally:
            orc.set_threads(prev)
        out["single_thread"] = {"value": cfg["T"] / dt1, "unit": "tokens/s", "cores": 1}
    log("cpu oracle, whole layer: %d tokens in %.3f s" % (cfg["T"], dt))
    return out


def cpu_baseline_backward(cfg, dev, log):
    """Time the oracle's backward (untuned) on a bounded sample and scale to
    tokens/s: the combine, gate/logit, centroid and input gradients on all T
    tokens; the SwiGLU expert backward on R rows of expert 0, its per-row time
    counted k+1 times per token (k routed rows + the shared row)."""
    import numpy as np

    import moe_inputs
    from oracle import oracle as orc

    S = cfg["T"]
    R = min(128, S)
    k, N = cfg["k"], cfg["N"]
    xs = moe_inputs.to_host(dev["x"][:S])
    E = moe_inputs.to_host(dev["centroids"])
    b = moe_inputs.to_host(dev["bias"])
    w13 = moe_inputs.to_host(dev["w13"][0])
    w2 = moe_inputs.to_host(dev["w2"][0])
    dout = moe_inputs.to_host(moe_inputs.make_upstream_grad(cfg, 0, "cpu", T=S))
    orc.lib()
    r = orc.route(xs, E, b, k, cfg["G"], cfg["TG"], want_scores=True)
    off, src, dst = orc.permute(r["idx"], N)
    yp = np.resize(dout, (S * k, dout.shape[1]))  # stand-in expert outputs (timing only)
    t0 = time.perf_counter()
    dyp, dg = orc.combine_backward(dout, yp, r["gate"], dst)
    t1 = time.perf_counter()
    if cfg.get("fp8"):
        xq, xsc = orc.quant_act_fp8(xs[:R])
        q13, s13 = orc.quant_weight_fp8(w13)
        q2, s2 = orc.quant_weight_fp8(w2)
        t1 = time.perf_counter()
        dA, _, _ = orc.swiglu_ffn_backward_fp8(xq, xsc, xs[:R], q13, s13, q2, s2, dout[:R])
    else:
        dA, _, _ = orc.swiglu_ffn_backward(xs[:R], w13, w2, dout[:R])
    t2 = time.perf_counter()
    dz = orc.route_backward(r["scores"], r["idx"], dg)
    orc.centroid_grad(xs, r["idx"], dz, N)
    dxp = np.resize(dA, (S * k, dA.shape[1]))
    dxs = np.resize(dA, (S, dA.shape[1]))
    orc.input_grad(dout, dxs, dxp, dst, dz, r["idx"], E)
    t3 = time.perf_counter()
    per_token = ((t1 - t0) + (t3 - t2)) / S + (t2 - t1) / R * (k + 1)
    cores = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    log("cpu oracle backward: combine %.2fs expert(%d rows) %.2fs route+input %.2fs -> %.4f "
        "s/token" % (t1 - t0, R, t2 - t1, t3 - t2, per_token))
    return {"value": 1.0 / per_token, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "combine, gate/logit, centroid and input gradients on all %d tokens; "
                      "the SwiGLU expert backward (recompute, dgrads, weight gradients) on %d "
                      "rows of expert 0, its per-row time counted k+1=%d times per token"
                      % (S, R, k + 1)}


def run_backward(args, cfg, dev, log):
    """Time K backward steps on the state of one forward step; one JSON line."""
    import torch

    import moe_inputs
    from sparse_moe_layer_bias_amd.layer import MoeLayer

    T = cfg["T"]
    layer = MoeLayer(cfg, dev["w13"], dev["w2"], dev["ws13"], dev["ws2"], train=True)
    x, E = dev["x"], dev["centroids"]
    dout = moe_inputs.make_upstream_grad(cfg, args.seed, "cuda")
    stream = torch.cuda.current_stream()
    layer.forward(x, E, dev["bias"].clone(), update_bias=False)
    for _ in range(args.warmup):
        layer.backward(dout, x, E)
    torch.cuda.synchronize()
    log("warmup done")
    stages = ["combine_backward", "expert_ffn_backward", "route_backward", "input_grad"]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
          for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(args.steps):
        layer.backward(dout, x, E, events=ev[s])
    t_stop.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_stop) / args.steps
    stage_ms = {st: sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps))
                / args.steps for i, st in enumerate(stages)}
    log("stages ms:", json.dumps({k: round(v, 4) for k, v in stage_ms.items()}))
    flops = ffn_bwd_flops(cfg)
    nbytes = ffn_bwd_bytes(cfg)
    ffn_s = stage_ms["expert_ffn_backward"] / 1e3
    achieved = flops / ffn_s
    peak = PEAK["fp8" if cfg.get("fp8") else "bf16"]
    hbm_bound = nbytes / PEAK["hbm"] > flops / peak
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": nbytes / ffn_s / 1e9, "peak": PEAK["hbm"] / 1e9,
                "unit": "GB/s", "frac": nbytes / ffn_s / PEAK["hbm"]}
    else:
        roof = {"bound": "mfma", "achieved": achieved / 1e12, "peak": peak / 1e12,
                "unit": "TFLOP/s", "frac": achieved / peak}
    roof.update({"kernel": ("expert FFN backward, FP8: dgrad down, "
                            "SwiGLU' + 1x128 tiles, dgrad up, 128x1 row-direction tiles, "
                            "wgrad down and up; a, b, h saved by the training forward"
                            if cfg.get("fp8") else
                            "expert FFN backward GEMMs (dgrad down+SwiGLU', dgrad up, wgrad "
                            "down, wgrad up; a, b, h saved by the training forward)"),
                 "traffic": recorded_traffic(args.workload, backward=True),
                 "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
                 "mfma_tflops": achieved / 1e12, "mfma_frac": achieved / peak})
    result = {
        "metric": METRIC_BWD,
        "value": T / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if cfg.get("fp8") else cfg["dtype"],
        "data": "synthetic",
        "config": {"workload": "%s backward: T=%d d=%d, %d routed experts top-%d%s + 1 "
                               "shared, SwiGLU I=%d, %s" %
                               (args.workload, T, cfg["d"], cfg["N"], cfg["k"],
                                (" (%d groups, top-%d)" % (cfg["G"], cfg["TG"]))
                                if cfg["G"] > 1 else "", cfg["I"], cfg["dtype"]),
                   "global_batch": T, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "stages_ms": stage_ms,
    }
    if not args.no_cpu_baseline:
        try:
            result["cpu_baseline"] = cpu_baseline_backward(cfg, dev, log)
        except Exception as ex:  # report, never hide
            log("cpu baseline failed:", repr(ex))
            result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


STAGES = ["route", "permute", "expert_ffn", "combine", "bias_update"]


def vendor_calibration(log):
    """What the vendor GEMM library reaches on this GPU, as context for the
    grouped expert GEMMs' fractions of the published peaks: bf16 batched GEMMs
    with the V3 layer's per-expert shapes (256 experts x 256 rows; right
    operands contiguous), large dense bf16 and FP8 GEMMs (per-tensor scales),
    each timed with events over several calls."""
    import torch

    out = {}

    def timeit(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps / 1e3

    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    for name, B, M, K, N in (("bf16 gate/up 256 x (256x7168 . 7168x4096)", 256, 256, 7168, 4096),
                             ("bf16 down 256 x (256x2048 . 2048x7168)", 256, 256, 2048, 7168),
                             ("bf16 dense 16384x7168 . 7168x16384", 1, 16384, 7168, 16384)):
        X = torch.randn(B, M, K, device="cuda", dtype=torch.bfloat16, generator=g)
        W = torch.randn(B, K, N, device="cuda", dtype=torch.bfloat16, generator=g).contiguous()
        t = timeit(lambda: torch.bmm(X, W), 5)
        fl = 2.0 * B * M * K * N
        out[name] = {"ms": t * 1e3, "tflops": fl / t / 1e12, "frac_of_peak": fl / t / PEAK["bf16"],
                     "weight_GBps": 2.0 * B * K * N / t / 1e9}
        log("vendor %s: %.3f ms, %.0f TFLOP/s" % (name, t * 1e3, fl / t / 1e12))
        del X, W
        torch.cuda.empty_cache()
    f8 = torch.float8_e4m3fn
    for name, M, K, N in (("fp8 dense 16384x7168 . 7168x16384", 16384, 7168, 16384),):
        A = torch.randn(M, K, device="cuda", generator=g).to(f8)
        Bm = torch.randn(N, K, device="cuda", generator=g).to(f8)
        one = torch.tensor(1.0, device="cuda")
        t = timeit(lambda: torch._scaled_mm(A, Bm.t(), scale_a=one, scale_b=one,
                                            out_dtype=torch.bfloat16), 5)
        fl = 2.0 * M * K * N
        out[name] = {"ms": t * 1e3, "tflops": fl / t / 1e12, "frac_of_peak": fl / t / PEAK["fp8"]}
        log("vendor %s: %.3f ms, %.0f TFLOP/s" % (name, t * 1e3, fl / t / 1e12))
        del A, Bm
    return out


def load_stats(counts, T, k):
    """max/mean load and idle experts of one step's per-expert counts"""
    mean = T * k / len(counts)
    return {"max_over_mean": float(max(counts)) / mean, "idle_experts": int(sum(c == 0 for c in counts))}


def skew_balance(args, dev, log):
    """The skewed decode-step workload: 100 steps of route + end-of-step bias
    update over fresh T = 128 batches with Zipf(1.2)-skewed expert popularity
    (moe_route + moe_bias_update only, timed), the load trajectory (replayed
    untimed: the same steps give the same bits), the fitted popularity slope at
    b = 0, and the whole layer at T = 128 with the V3-shaped experts."""
    import numpy as np
    import torch

    import moe_inputs
    import sparse_moe_layer_bias_amd as moe
    from sparse_moe_layer_bias_amd.layer import MoeLayer

    c5 = dict(moe_inputs.CONFIGS["skew_balance"])
    T, N, k, steps = c5["T"], c5["N"], c5["k"], c5["steps"]
    E = moe_inputs.make_skew_centroids(c5, args.seed, "cpu").cuda()
    xs = [moe_inputs.make_skew_tokens(c5, s, args.seed, "cuda") for s in range(steps + 1)]
    cfg = moe.cfg_from_dict(c5)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, k), dtype=torch.float32, device="cuda")
    counts = torch.empty((N,), dtype=torch.int32, device="cuda")
    ws = torch.empty((max(moe.moe_route_workspace_size(cfg), 256),), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()

    def run(record=None):
        bias = torch.zeros(N, device="cuda")
        for s in range(steps):
            moe.moe_route(cfg, xs[s], E, bias, None, idx, gate, counts, ws)
            if record is not None:
                record[s].copy_(counts)
            moe.moe_bias_update(N, T * k, counts, 0.001, bias)
        if record is not None:  # the routing after the last update
            moe.moe_route(cfg, xs[steps], E, bias, None, idx, gate, counts, ws)
            record[steps].copy_(counts)
        return bias

    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    run()
    e1.record(stream)
    torch.cuda.synchronize()
    us_step = e0.elapsed_time(e1) * 1e3 / steps
    rec = torch.empty((steps + 1, N), dtype=torch.int32, device="cuda")
    bias_end = run(rec)
    torch.cuda.synchronize()
    cnt = rec.cpu().numpy()
    traj = {str(s): load_stats(cnt[s], T, k) for s in (0, steps // 2, steps)}
    # popularity at b = 0: top-1 choice of every token of every batch
    top1 = np.zeros(N, np.int64)
    zero = torch.zeros(N, device="cuda")
    for s in range(steps + 1):
        moe.moe_route(cfg, xs[s], E, zero, None, idx, gate, counts, ws)
        top1 += np.bincount(idx[:, 0].cpu().numpy(), minlength=N)
    f = np.sort(top1)[::-1]
    f = f[f > 0]
    rank = np.arange(1, len(f) + 1)
    slope = float(np.polyfit(np.log(rank), np.log(f / f.sum()), 1)[0])
    log("skew balance: %.1f us/step; load %s; top-1 popularity slope %.2f" %
        (us_step, json.dumps(traj), slope))
    # the whole layer at T = 128 over the V3-shaped experts, bias from the trajectory
    lay = MoeLayer(c5, dev["w13"], dev["w2"], dev["ws13"], dev["ws2"])
    x = xs[steps]
    b = bias_end.clone()
    ms, st = time_forward(lay, x, E, b, 20, 3)
    touched = int((lay.counts > 0).sum().item())
    gms = time_graph(lay, x, E, bias_end.clone(), 20, 3)
    d, I, Is = c5["d"], c5["I"], c5["Is"]
    wbytes = 2.0 * 3 * d * (touched * I + Is)
    log("decode layer T=128: %.3f ms/step (%.3f as one graph), %d experts touched, stages %s" %
        (ms, gms, touched, json.dumps({a: round(v, 4) for a, v in st.items()})))
    del lay
    torch.cuda.empty_cache()
    return {"route_plus_bias_update_us_per_step": us_step,
            "load": traj, "load_steps": "routing at steps 0, %d and %d (after that many updates)"
                                        % (steps // 2, steps),
            "zipf_slope_top1_b0": slope,
            "layer_T128_v3_experts": {
                "ms_per_step": ms, "tokens_per_s": T / (ms / 1e3), "stages_ms": st,
                "graph_ms_per_step": gms, "experts_touched": touched,
                "expert_weight_GBps": wbytes / (st["expert_ffn"] / 1e3) / 1e9}}


def extra_configs(args, dev, log):
    """The other four workloads, measured in the same run after the headline
    one: V3 with FP8 expert GEMMs (its own roofline and oracle time), the
    skewed decode-step balance workload, and the two small layers."""
    import torch

    import moe_inputs
    from sparse_moe_layer_bias_amd.layer import MoeLayer

    out = {}
    c4 = dict(moe_inputs.CONFIGS["v3_fp8"])
    lay = MoeLayer(c4, dev["w13"], dev["w2"], dev["ws13"], dev["ws2"])
    ms, st = time_forward(lay, dev["x"], dev["centroids"], dev["bias"].clone(), 10, 3)
    del lay
    torch.cuda.empty_cache()
    out["v3_fp8"] = {"ms_per_step": ms, "tokens_per_s": c4["T"] / (ms / 1e3), "stages_ms": st,
                     "roofline": ffn_roofline(c4, st["expert_ffn"] / 1e3, "v3_fp8")}
    log("v3_fp8: %.3f ms/step, stages %s" % (ms, json.dumps({a: round(v, 4)
                                                              for a, v in st.items()})))
    if not args.no_cpu_baseline:
        try:
            out["v3_fp8"]["cpu_baseline"] = cpu_baseline(c4, dev, log, rows=512)
        except Exception as ex:  # report, never hide
            log("cpu baseline (fp8) failed:", repr(ex))
            out["v3_fp8"]["cpu_baseline"] = None
    out["skew_balance"] = skew_balance(args, dev, log)
    for name in ("tiny_fp32", "mid_bf16"):
        c = dict(moe_inputs.CONFIGS[name])
        d2 = moe_inputs.make_layer_inputs(c, args.seed, "cuda")
        lay = MoeLayer(c, d2["w13"], d2["w2"], d2["ws13"], d2["ws2"])
        ms, st = time_forward(lay, d2["x"], d2["centroids"], d2["bias"].clone(), 20, 5)
        gms = time_graph(lay, d2["x"], d2["centroids"], d2["bias"].clone(), 20, 5)
        out[name] = {"ms_per_step": ms, "tokens_per_s": c["T"] / (ms / 1e3), "stages_ms": st,
                     "graph_ms_per_step": gms, "graph_tokens_per_s": c["T"] / (gms / 1e3)}
        log("%s: %.4f ms/step, %.4f ms/step as one graph" % (name, ms, gms))
        if not args.no_cpu_baseline:
            try:
                out[name]["cpu_baseline"] = cpu_baseline_layer(c, d2, log,
                                                               single_thread=name == "tiny_fp32")
            except Exception as ex:  # report, never hide
                log("cpu baseline (%s) failed: %r" % (name, ex))
                out[name]["cpu_baseline"] = None
        del lay, d2
    return out


def time_graph(layer, x, E, bias, steps, warmup):
    """The same step captured once as a HIP graph (MoeLayer.capture_forward:
    the five calls, no host work in between), W untimed replays, then K
    replays timed with HIP events on the current stream.  Returns ms per
    step."""
    import torch
    layer.capture_forward(x, E, bias)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        layer.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        layer.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def time_forward(layer, x, E, bias, steps, warmup):
    """W untimed steps, then K whole steps timed with HIP events on the stream
    the calls are enqueued on (one event pair around the K steps, and one
    event between consecutive stages of each step).  Returns ms per step and
    the mean ms of each stage."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        layer.forward(x, E, bias)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)]
          for _ in range(steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(steps):
        e = ev[s]
        e[0].record(stream)
        layer.route(x, E, bias)
        e[1].record(stream)
        layer.permute(x)
        e[2].record(stream)
        layer.expert_ffn(x)
        e[3].record(stream)
        layer.combine(x)
        e[4].record(stream)
        layer.bias_update(bias)
        e[5].record(stream)
    t_stop.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_stop) / steps
    stage_ms = {st: sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)) / steps
                for i, st in enumerate(STAGES)}
    return ms_per_step, stage_ms


def time_seq_balance_loss(layer, seq_len, reps=20):
    """The sequence-wise balance loss of the last routed step (moe_seq_balance_loss),
    timed with HIP events over `reps` calls on the stream it runs on."""
    import torch
    from sparse_moe_layer_bias_amd import (moe_seq_balance_loss,
                                           moe_seq_balance_loss_workspace_size)
    T, N, k = layer.c["T"], layer.c["N"], layer.c["k"]
    if T % seq_len:
        return None
    dev = layer.scores.device
    loss = torch.empty(T // seq_len, dtype=torch.float32, device=dev)
    ws = torch.empty(max(moe_seq_balance_loss_workspace_size(layer.cfg, seq_len), 16),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    moe_seq_balance_loss(layer.cfg, seq_len, 1e-4, layer.scores, layer.idx, loss, ws)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        moe_seq_balance_loss(layer.cfg, seq_len, 1e-4, layer.scores, layer.idx, loss, ws)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    nbytes = T * N * 4 + T * k * 4
    return {"seq_len": seq_len, "alpha": 1e-4, "us_per_call": us,
            "read_GBps": nbytes / (us * 1e-6) / 1e9, "loss": [float(v) for v in loss.cpu()]}


def ffn_roofline(cfg, ffn_s, workload):
    """The expert FFN call (both grouped GEMM launches and the tile map) against
    the roofline that bounds its algorithmic work: the larger of the time at
    the MFMA peak of its dtype and the time at the HBM peak."""
    fp8 = bool(cfg.get("fp8"))
    flops = ffn_flops(cfg)
    achieved = flops / ffn_s
    peak = PEAK["fp8" if fp8 else "bf16"]
    nbytes = ffn_bytes(cfg)
    if nbytes / PEAK["hbm"] > flops / peak:
        roof = {"bound": "hbm", "achieved": nbytes / ffn_s / 1e9, "peak": PEAK["hbm"] / 1e9,
                "unit": "GB/s", "frac": nbytes / ffn_s / PEAK["hbm"]}
    else:
        roof = {"bound": "mfma", "achieved": achieved / 1e12, "peak": peak / 1e12,
                "unit": "TFLOP/s", "frac": achieved / peak}
    roof.update({"kernel": "grouped expert GEMMs (gate/up+SwiGLU, down)%s" %
                           (", FP8 E4M3" if fp8 else ""),
                 "traffic": recorded_traffic(workload),
                 "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
                 "mfma_tflops": achieved / 1e12, "mfma_frac": achieved / peak})
    return roof


def main():
    args = parse()
    if args.stats_summary:
        print(stats_summary(args.stats_summary))
        return
    if args.traffic_summary:
        print(traffic_summary(args.traffic_summary[0], args.traffic_summary[1], args.workload,
                              args.backward))
        return
    if args.counter_summary:
        print(counter_summary(*args.counter_summary, args.workload))
        return
    if args.sq_summary:
        print(sq_summary(*args.sq_summary, args.workload))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import moe_inputs
    import sparse_moe_layer_bias_amd as moe
    from sparse_moe_layer_bias_amd.layer import MoeLayer

    def log(*a):
        print(*a, file=sys.stderr, flush=True)

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    if args.vendor_calibration:
        print(json.dumps({"vendor_calibration": vendor_calibration(log)}), flush=True)
        return
    moe.lib()
    cfg = dict(moe_inputs.CONFIGS[args.workload])
    T = cfg["T"]
    log("generating inputs for", args.workload, cfg)
    dev = moe_inputs.make_layer_inputs(cfg, args.seed, "cuda")
    if args.backward and not args.traffic_run:
        run_backward(args, cfg, dev, log)
        return
    layer = MoeLayer(cfg, dev["w13"], dev["w2"], dev["ws13"], dev["ws2"], train=args.backward)
    x, E = dev["x"], dev["centroids"]
    bias = dev["bias"].clone()
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    if args.traffic_run:
        traffic_run(cfg, layer, dev, args.backward)
        log("traffic run done")
        return
    if args.counter_run:
        counter_run(cfg, layer, dev)
        log("counter run done")
        return

    ms_per_step, stage_ms = time_forward(layer, x, E, bias, args.steps, args.warmup)
    log("warmup done; stages ms:", json.dumps({k: round(v, 4) for k, v in stage_ms.items()}))
    fp8 = bool(cfg.get("fp8"))
    roof = ffn_roofline(cfg, stage_ms["expert_ffn"] / 1e3, args.workload)
    flops = ffn_flops(cfg)
    peak = PEAK["fp8" if fp8 else "bf16"]
    nbytes = ffn_bytes(cfg)
    ffn_s = stage_ms["expert_ffn"] / 1e3
    achieved = flops / ffn_s
    hbm_bound = roof["bound"] == "hbm"
    if not args.no_probes:
        # the same ceilings measured on this GPU, after the timed region: the
        # HBM read rate of the GEMMs' global -> LDS copies alone, and the rate
        # of a register-resident loop of their MFMA instruction (its clock is
        # the rate over the published flop per cycle)
        from sparse_moe_layer_bias_amd import probe
        rd = probe.hbm_read_rate()
        mf = probe.mfma_rate("fp8" if fp8 else "bf16")
        roof["measured_peak"] = {"hbm_read_GBps": rd / 1e9, "mfma_tflops": mf / 1e12,
                                 "mfma_clock_GHz": mf / (peak / 2.4e9) / 1e9}
        roof["frac_of_measured"] = (nbytes / ffn_s / rd) if hbm_bound else (achieved / mf)
        roof["mfma_frac_of_measured"] = achieved / mf
        log("measured peaks:", json.dumps(roof["measured_peak"]))
    result = {
        "metric": METRIC,
        "value": T / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if fp8 else cfg["dtype"],
        "data": "synthetic",
        "config": {"workload": "%s: T=%d d=%d, %d routed experts top-%d%s + %d shared, "
                               "SwiGLU I=%d, %s expert GEMMs" %
                               (args.workload, T, cfg["d"], cfg["N"], cfg["k"],
                                (" (%d groups, top-%d)" % (cfg["G"], cfg["TG"]))
                                if cfg["G"] > 1 else "", 1, cfg["I"],
                                "FP8 E4M3" if fp8 else cfg["dtype"]),
                   "global_batch": T, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "stages_ms": stage_ms,
        "layer_tflops": (flops + 2.0 * T * cfg["d"] * cfg["N"]) / (ms_per_step / 1e3) / 1e12,
    }
    # the sequence-wise balance loss of the step's routing (sequences of 4096
    # tokens), a statistic beside the step, not part of its time
    result["seq_balance_loss"] = time_seq_balance_loss(layer, min(4096, T))
    if not args.no_cpu_baseline:
        try:
            result["cpu_baseline"] = cpu_baseline(cfg, dev, log)
        except Exception as ex:  # report, never hide
            log("cpu baseline failed:", repr(ex))
            result["cpu_baseline"] = None
    if args.workload == "v3_bf16" and not args.no_configs:
        del layer
        torch.cuda.empty_cache()
        result["configs"] = extra_configs(args, dev, log)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

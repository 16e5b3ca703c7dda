"""Benchmark of the dual-branch W4A4 FFN layer on one MI355X.

One step = the whole hot path over one batch of synthetic input:
calibrate (per-channel activation maxima) -> weight column ranges -> plan
(Eq. (2) scales, Eq. (4) top-k, fold + MXFP4 pack) -> fused activation
quantize -> dual-branch GEMM (bf16 output), every stage a kernel of
libmixed_gemm on torch's current HIP stream.

Default workload: the Wan2.2-A14B FFN up-projection at 480p,
M = 32760 tokens x K = 5120 -> N = 13824, alpha = 0.6, k = 64, 1x32 blocks.

Prints ONE JSON line.  `value` = 2*M*K*N / (time of one whole step), in
TFLOP/s; the dual-GEMM kernel's own rate is in `roofline`.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
    python bench.py --power-probe S   board power (hwmon) while the GEMM and the quantize
                                 each run back to back for S seconds after the timed
                                 steps (default 2; 0 leaves the `power` object out)
    python bench.py --suite      one JSON line per configuration point: the
                                 480p up/down-projections (three weight-scale
                                 layouts, raw, smoothed and percentile outlier
                                 scores), the 720p (k, alpha) sweep and the
                                 720p FFN block
                                 (three layouts), each with kernel rates (warm,
                                 and the GEMM also cold) and the fidelity of the
                                 three modes against the unquantized float64 layer
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
# the host cores this process may run on, and the threads the oracle baseline
# uses: all of them, unless the environment already caps the thread pools
# (a shared host's share); BLAS is told that count before numpy is imported
HOST_CORES = len(os.sched_getaffinity(0))
_cap = min([int(os.environ[v]) for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS")
            if os.environ.get(v, "").isdigit() and int(os.environ[v]) > 0] + [HOST_CORES])
BASELINE_THREADS = _cap
for _v in ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_v, str(BASELINE_THREADS))

PEAK_FP4_TFLOPS = 10100.0          # MI355X dense MXFP4 MFMA (published)
PEAK_HBM_GBS = 8000.0              # MI355X HBM3E (published)
METRIC = "dual-branch W4A4 FFN GEMM effective TFLOPS, % MXFP4 MFMA peak (480p/720p)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "dual_gemm_ffn0_480p_traffic.json")
# the dual GEMM's sources: its kernel file and the headers it includes
GEMM_SRCS = [os.path.join(ROOT, "mixed_gemm_amd", "csrc", f) for f in ("k_gemm.hip", "mg_device.h", "mg_internal.h")]


def _code_only(src: str) -> str:
    """C/C++ source with comments removed and whitespace runs collapsed (string
    and character literals kept), so that only changes to the code itself
    change the hash below."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def gemm_source_hash() -> str:
    """Hash of the dual GEMM's code (comments and layout excluded)."""
    h = hashlib.sha256()
    for f in GEMM_SRCS:
        h.update(_code_only(open(f, encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def measured_traffic() -> float | None:
    """HBM bytes per dual-GEMM launch from the committed rocprofv3 counter
    summary, or None when there is none or the kernel source changed since."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != gemm_source_hash():
        return None
    return float(t["bytes_per_launch"])


def cpu_baseline(w, X, W, rows: int) -> dict:
    """The oracle as it stands, on a bounded sample: the weight ranges and plan
    on the full W, and the per-row work (calibration, quantize, float64 dual
    GEMM) on `rows` rows, whose cost is scaled to the workload's M."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import layer
    with threadpool_limits(limits=BASELINE_THREADS):
        return _cpu_baseline(layer, threadpool_info, w, X, W, rows)


def _cpu_baseline(layer, threadpool_info, w, X, W, rows: int) -> dict:
    t0 = time.perf_counter()
    a = layer.act_max(X[:rows])                                   # per-row work
    t1 = time.perf_counter()
    wr = layer.weight_range(W)                                    # per-weight work
    p = layer.plan(a, wr, W, w.alpha, w.k)
    t2 = time.perf_counter()
    qa = layer.quantize_act(X[:rows], p["s"], p["O"])             # per-row work
    Y = layer.dual_gemm_f64(qa["Aq"], qa["As"], p["Wq"], p["Ws"], qa["XO"], p["WO"])
    t3 = time.perf_counter()
    assert Y.shape == (rows, w.N)
    t_plan, t_rows = t2 - t1, (t1 - t0) + (t3 - t2)
    t_full = t_plan + t_rows * w.M / rows
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(w.flops() / t_full / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "host_cores": HOST_CORES,
            "kind": "oracle",
            "sample": (f"the whole oracle step, all {w.M} rows: weight ranges and plan {t_plan:.1f} s, "
                       f"per-row work {t_rows:.1f} s" if rows == w.M else
                       f"oracle step on {rows} of {w.M} rows (weight ranges and plan {t_plan:.1f} s; "
                       f"per-row work {t_rows:.1f} s scaled x{w.M / rows:.1f}); est. full step {t_full:.0f} s")}


COPY_BYTES = 256 << 20            # plain copy used to calibrate the HBM byte counters


def _hwmon_power_files() -> tuple[str | None, str | None]:
    """The GPU's board power reading and cap (microwatts) from the amdgpu hwmon
    sysfs files, when this host exposes them."""
    import glob
    for d in sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*")):
        inp = next((os.path.join(d, f) for f in ("power1_input", "power1_average")
                    if os.path.exists(os.path.join(d, f))), None)
        if inp:
            cap = os.path.join(d, "power1_cap")
            return inp, cap if os.path.exists(cap) else None
    return None, None


def power_probe(seconds: float, runs: dict) -> dict:
    """Board power while each of `runs` (name -> launch function) runs back to
    back for `seconds`, sampled every 20 ms from a host thread (the first
    0.3 s of each run, while the clock settles, is left out), and at idle."""
    import threading

    import numpy as np
    import torch

    inp, cap = _hwmon_power_files()
    if inp is None:
        return {"available": False}
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                samples.append((time.perf_counter(), int(open(inp).read()) / 1e6))
            except (OSError, ValueError):
                pass
            stop.wait(0.02)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    out = {"available": True, "source": inp}
    if cap:
        out["cap_w"] = int(open(cap).read()) / 1e6
    torch.cuda.synchronize()
    time.sleep(1.0)
    windows = {"idle": (time.perf_counter() - 0.7, time.perf_counter())}
    for name, fn in runs.items():
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        n = 0
        while time.perf_counter() - t0 < seconds:
            for _ in range(20):
                fn()
            n += 20
            torch.cuda.synchronize()
        e1.record()
        e1.synchronize()
        windows[name] = (t0 + 0.3, time.perf_counter())
        out[name + "_us"] = round(e0.elapsed_time(e1) * 1e3 / n, 1)
        out[name + "_launches"] = n
        time.sleep(1.0)
    stop.set()
    th.join()
    for name, (a, b) in windows.items():
        v = [w for t, w in samples if a <= t <= b]
        out[name + "_w"] = round(float(np.mean(v)), 1) if v else None
        out[name + "_samples"] = len(v)
    return out


def summarize_pmc(fetch_csv: str, write_csv: str, out_json: str) -> dict:
    """HBM bytes per dual-GEMM launch from two rocprofv3 --pmc runs of this
    script with --copy-calibration (FETCH_SIZE, then WRITE_SIZE, in KiB per
    dispatch).  Each counter is scaled by what it reads for the plain copy of
    COPY_BYTES (read COPY_BYTES, write COPY_BYTES) in the same run."""
    import csv

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            vals.setdefault(name, {}).setdefault(r["Dispatch_Id"], 0.0)
            vals[name][r["Dispatch_Id"]] += float(r["Counter_Value"])
        return {k: sorted(v.values()) for k, v in vals.items()}

    def pick(d, pred):
        ks = [k for k in d if pred(k)]
        assert ks, "kernel not found in counter file"
        vals = [v for k in ks for v in d[k]]
        return sorted(vals)[len(vals) // 2]          # median dispatch

    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")
    is_gemm = lambda k: "dual_gemm_tiled" in k
    is_copy = lambda k: "copyBuffer" in k      # the runtime's device-to-device copy kernel
    fetch_kib, write_kib = pick(f, is_gemm), pick(w, is_gemm)
    copy_fetch_kib, copy_write_kib = pick(f, is_copy), pick(w, is_copy)
    fetch_scale = COPY_BYTES / (copy_fetch_kib * 1024)
    write_scale = COPY_BYTES / (copy_write_kib * 1024)
    res = {"kernel": "dual_gemm_tiled (bf16 output)", "workload": "ffn0_480p_32760x5120x13824",
           "fetch_kib": fetch_kib, "write_kib": write_kib,
           "copy_fetch_kib": copy_fetch_kib, "copy_write_kib": copy_write_kib,
           "fetch_scale": fetch_scale, "write_scale": write_scale,
           "bytes_per_launch": fetch_kib * 1024 * fetch_scale + write_kib * 1024 * write_scale,
           "kernel_source_sha256_16": gemm_source_hash()}
    json.dump(res, open(out_json, "w"), indent=1)
    return res


# ----------------------------------------------------------------------------- suite

FID_ROWS = 64
COLD_BYTES = 1 << 30      # written between cold timings: evicts the L2s and the 256 MB MALL


def _suite_tools():
    import numpy as np
    import torch

    import mixed_gemm_amd as mg
    import synth

    stream = torch.cuda.current_stream()
    scratch = torch.empty(COLD_BYTES // 4, dtype=torch.float32, device="cuda")

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    def to_f64(a):
        a = np.asarray(a)
        return (synth.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)

    def y_host(t):
        return t.view(torch.int16).cpu().numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.cpu().numpy()

    def timed(fn, reps=10, warmup=20, cold=False):
        """mean ms of fn() over reps launches after `warmup` untimed ones (the
        clock settles over the first launches after a pause), HIP events on the
        current stream around the reps launches back to back; cold: a 1 GiB
        write before each launch, outside its own pair of events."""
        for _ in range(warmup):
            fn()
        if not cold:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                fn()
            b.record(stream)
            b.synchronize()
            return a.elapsed_time(b) / reps
        ts = []
        for _ in range(reps):
            scratch.fill_(1.0)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.mean(ts))

    def rel_fro(Y, Yref):
        return float(np.linalg.norm(to_f64(Y) - Yref) / np.linalg.norm(Yref))

    return np, torch, mg, synth, dev, to_f64, y_host, timed, rel_fro


def _emit(d):
    print(json.dumps(d), flush=True)


def suite(args) -> int:
    np, torch, mg, synth, dev, to_f64, y_host, timed, rel_fro = _suite_tools()
    torch.cuda.set_device(0)
    g = np.random.default_rng(12345)

    def layer_point(w, X_h, W_h, Xd, Wd, points, layout="1x32", score="max"):
        """Timings + fidelity of one layer for each (k, alpha) in points."""
        M, K, N = X_h.shape[0], w.K, w.N
        bf = w.dtype == "bf16"
        act_max = torch.empty(K, dtype=torch.float32, device="cuda")
        w_max = torch.empty(K, dtype=torch.float32, device="cuda")

        def calib():
            mg.mg_calib_reset(act_max)
            mg.mg_calib_act(Xd, act_max)
        t_calib = timed(calib)
        t_wr = timed(lambda: mg.mg_weight_range(Wd, w_max))
        # score "pNN.N": Eq. (4) ranks the nearest-rank NN.N% quantile of |x| per channel
        pct_q = float(score[1:]) / 100.0 if score.startswith("p") else None
        desc_score = "max" if pct_q is not None else score
        rank_stat, t_pct = None, None
        if pct_q is not None:
            rank_stat = torch.empty(K, dtype=torch.float32, device="cuda")
            st = mg.PctState(K)

            def pct():
                mg.mg_pct_reset(st)
                mg.mg_pct_count(st, 0, Xd)
                mg.mg_pct_select(st, 0, pct_q)
                mg.mg_pct_count(st, 1, Xd)
                mg.mg_pct_select(st, 1, pct_q, rank_stat)
            t_pct = timed(pct)

        def build(p):
            if rank_stat is None:
                mg.mg_plan_build(p, act_max, w_max, Wd)
            else:
                mg.mg_smooth_scales(p, act_max, w_max)
                mg.mg_outlier_set(p, rank_stat)
                mg.mg_fold_pack(p, Wd)
        rows = np.arange(M) if M <= FID_ROWS else np.sort(g.choice(M, FID_ROWS, replace=False))
        Xs = Xd[torch.from_numpy(rows).cuda()].contiguous()
        Yref = to_f64(X_h[rows]) @ to_f64(W_h).T
        Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

        def fidelity(k, alpha, smooth):
            p = mg.Plan.empty(mg.make_desc(K, N, k, alpha, layout, smooth, desc_score))
            build(p)
            return rel_fro(y_host(mg.forward(p, Xs)), Yref)

        uniform = fidelity(0, 0.5, False)
        smooth_only = {}
        for k, alpha in points:
            desc = mg.make_desc(K, N, k, alpha, layout, True, desc_score)
            p = mg.Plan.empty(desc)
            t_plan = timed(lambda: build(p))
            a = mg.Act.empty(desc, M)
            t_quant = timed(lambda: mg.mg_quantize_act(p, Xd, a))
            t_gemm = timed(lambda: mg.mg_dual_gemm(p, a, Y))
            t_gemm_cold = timed(lambda: mg.mg_dual_gemm(p, a, Y), reps=5, warmup=1, cold=True)
            if alpha not in smooth_only:
                smooth_only[alpha] = fidelity(0, alpha, True)
            fl = 2.0 * M * K * N
            xb = 2 if bf else 4
            quant_bytes = M * K * xb + M * K // 2 + M * K // 32 + 2 * M * k
            pack_bytes = N * K * xb + N * K // 2 + N * K // 32 + 2 * N * k
            _emit({"suite": "dual-branch W4A4 layer",
                   "config": {"workload": w.name, "M": M, "K": K, "N": N, "k": k, "alpha": alpha,
                              "weight_blocks": layout, "outlier_score": score, "output": "bf16"},
                   "gemm_ms": round(t_gemm, 4), "gemm_tflops": round(fl / t_gemm / 1e9, 1),
                   "gemm_pct_mxfp4_peak": round(100 * fl / t_gemm / 1e9 / PEAK_FP4_TFLOPS, 2),
                   "gemm_ms_cold": round(t_gemm_cold, 4),
                   "gemm_tflops_cold": round(fl / t_gemm_cold / 1e9, 1),
                   "quant_ms": round(t_quant, 4), "quant_gbs": round(quant_bytes / t_quant / 1e6, 1),
                   "quant_pct_hbm": round(100 * quant_bytes / t_quant / 1e6 / PEAK_HBM_GBS, 2),
                   "calib_ms": round(t_calib, 4), "calib_gbs": round(M * K * xb / t_calib / 1e6, 1),
                   "weight_range_ms": round(t_wr, 4),
                   "plan_ms": round(t_plan, 4), "plan_gbs": round(pack_bytes / t_plan / 1e6, 1),
                   "fidelity_rel_fro": {"uniform": round(uniform, 5),
                                        "smooth_only": round(smooth_only[alpha], 5),
                                        "smooth_split": round(fidelity(k, alpha, True), 5)},
                   "fidelity_rows": int(rows.size),
                   **({"pct_ms": round(t_pct, 4), "pct_gbs": round(2 * M * K * xb / t_pct / 1e6, 1)}
                      if t_pct is not None else {})})
            del a
        del Y

    def layer_config(w, points, layouts=("1x32",), scores=("max",)):
        X_h, W_h = w.make_x(), w.make_w()
        Xd, Wd = dev(X_h), dev(W_h)
        for lay in layouts:
            for sc in scores:
                layer_point(w, X_h, W_h, Xd, Wd, points, lay, sc)
        del Xd, Wd
        torch.cuda.empty_cache()

    layer_config(synth.TINY, [(synth.TINY.k, synth.TINY.alpha)])
    layer_config(synth.FFN0_480P, [(synth.FFN0_480P.k, synth.FFN0_480P.alpha)], ("1x32", "32x32", "128x1"),
                 ("max", "smoothed", "p99.9"))
    layer_config(synth.FFN2_480P, [(synth.FFN2_480P.k, synth.FFN2_480P.alpha)], ("1x32", "32x32", "128x1"),
                 ("max", "smoothed", "p99.9"))
    layer_config(synth.FFN0_720P, [(k, a) for a in synth.SWEEP_ALPHA for k in synth.SWEEP_K])

    # ---- the 720p FFN block
    w0, w2, M = synth.BLOCK_FFN0, synth.BLOCK_FFN2, synth.BLOCK_M
    W0_h, W2_h = w0.make_w(), w2.make_w()
    W0d, W2d = dev(W0_h), dev(W2_h)
    Xcal = [dev(w0.make_x(M=M, x_seed=sd)) for sd in synth.BLOCK_CALIB_SEEDS]
    act0, act2 = mg.ffn_block_stats(Xcal, W0d)
    del Xcal
    torch.cuda.empty_cache()
    X5_h = w0.make_x(M=M, x_seed=synth.BLOCK_EVAL_SEED)
    X5 = dev(X5_h)
    rows = np.sort(g.choice(M, FID_ROWS, replace=False))
    Xs = X5[torch.from_numpy(rows).cuda()].contiguous()
    z = to_f64(X5_h[rows]) @ to_f64(W0_h).T
    c = float(np.sqrt(2.0 / np.pi))
    href = 0.5 * z * (1.0 + np.tanh(c * (z + 0.044715 * z ** 3)))     # float64 GELU-tanh
    Yref = href @ to_f64(W2_h).T
    for lay in ("1x32", "32x32", "128x1"):
        def block_fid(k0, a0, k2, a2, smooth):
            p0 = mg.Plan.empty(mg.make_desc(w0.K, w0.N, k0, a0, lay, smooth))
            p2 = mg.Plan.empty(mg.make_desc(w2.K, w2.N, k2, a2, lay, smooth))
            for p, am, Wd_ in ((p0, act0, W0d), (p2, act2, W2d)):
                wm = torch.empty(p.desc.K, dtype=torch.float32, device="cuda")
                mg.mg_weight_range(Wd_, wm)
                mg.mg_plan_build(p, am, wm, Wd_)
            y = mg.ffn_block_forward(mg.FFNBlock(p0, p2), Xs)
            return rel_fro(y_host(y), Yref)
        blk = mg.ffn_block_plans(act0, act2, W0d, W2d, w0.alpha, w0.k, w2.alpha, w2.k, lay)
        a0 = mg.Act.empty(blk.plan0.desc, M)
        a2 = mg.Act.empty(blk.plan2.desc, M)
        Y0 = torch.empty((M, w0.N), dtype=torch.bfloat16, device="cuda")
        h = torch.empty_like(Y0)
        Y2 = torch.empty((M, w2.N), dtype=torch.bfloat16, device="cuda")

        def run_block():              # GELU and ffn.2's quantize fused in one pass
            mg.mg_forward(blk.plan0, X5, a0, Y0)
            mg.mg_gelu_quantize_act(blk.plan2, Y0, a2)
            mg.mg_dual_gemm(blk.plan2, a2, Y2)

        def run_block_epilogue():     # GELU and ffn.2's quantize in ffn.0's GEMM epilogue
            mg.mg_quantize_act(blk.plan0, X5, a0)
            mg.mg_dual_gemm_gelu_quant(blk.plan0, a0, blk.plan2, a2)
            mg.mg_dual_gemm(blk.plan2, a2, Y2)

        def run_block_unfused():
            mg.mg_forward(blk.plan0, X5, a0, Y0)
            mg.mg_gelu_tanh_bf16(Y0, h)
            mg.mg_forward(blk.plan2, h, a2, Y2)
        t_block = timed(run_block, reps=5)
        t_block_unfused = timed(run_block_unfused, reps=5)
        t_block_epi = timed(run_block_epilogue, reps=5)
        t_g0q = timed(lambda: mg.mg_dual_gemm_gelu_quant(blk.plan0, a0, blk.plan2, a2))
        t_gq = timed(lambda: mg.mg_gelu_quantize_act(blk.plan2, Y0, a2))
        t_g0 = timed(lambda: mg.mg_dual_gemm(blk.plan0, a0, Y0))
        t_gelu = timed(lambda: mg.mg_gelu_tanh_bf16(Y0, h))
        t_q2 = timed(lambda: mg.mg_quantize_act(blk.plan2, h, a2))
        t_g2 = timed(lambda: mg.mg_dual_gemm(blk.plan2, a2, Y2))
        fl0, fl2 = 2.0 * M * w0.K * w0.N, 2.0 * M * w2.K * w2.N
        _emit({"suite": "dual-branch W4A4 layer",
               "config": {"workload": "ffn_block_720p_75600x5120x13824x5120", "M": M, "k": [w0.k, w2.k],
                          "alpha": [w0.alpha, w2.alpha], "weight_blocks": lay, "output": "bf16"},
               "block_ms": round(t_block, 4), "block_tflops": round((fl0 + fl2) / t_block / 1e9, 1),
               "block_ms_unfused_gelu": round(t_block_unfused, 4),
               "block_ms_gemm_epilogue": round(t_block_epi, 4),
               "ffn0_gemm_ms": round(t_g0, 4),
               "ffn0_gemm_gelu_quant_ms": round(t_g0q, 4),
               "gelu_quant_ms": round(t_gq, 4),
               "gelu_quant_gbs": round((M * w2.K * 2.53125 + 2 * M * w2.k) / t_gq / 1e6, 1),
               "ffn0_gemm_tflops": round(fl0 / t_g0 / 1e9, 1), "ffn2_gemm_tflops": round(fl2 / t_g2 / 1e9, 1),
               "gelu_ms": round(t_gelu, 4), "gelu_gbs": round(4 * M * w0.N / t_gelu / 1e6, 1),
               "ffn2_quant_ms": round(t_q2, 4),
               "ffn2_quant_gbs": round((M * w2.K * 2.53125 + 2 * M * w2.k) / t_q2 / 1e6, 1),
               "fidelity_rel_fro": {"uniform": round(block_fid(0, 0.5, 0, 0.5, False), 5),
                                    "smooth_only": round(block_fid(0, w0.alpha, 0, w2.alpha, True), 5),
                                    "smooth_split": round(block_fid(w0.k, w0.alpha, w2.k, w2.alpha, True), 5)},
               "fidelity_rows": int(rows.size)})
        del a0, a2, Y0, h, Y2, blk
        torch.cuda.empty_cache()
    del X5, Xs, W0d, W2d
    torch.cuda.empty_cache()

    # ---- per-step routing by prediction on a drifting sequence (480p up-projection shape)
    w = synth.FFN0_480P
    steps, drift = 6, 0.1
    seq = synth.drifting_act(w.M, w.K, steps + 1, sigma=0.25, frac=0.02, mult=25.0, drift=drift,
                             ch_seed=601, x_seed=610)
    W_h = w.make_w()
    Wd = dev(W_h)
    a_cal = mg.calibrate([dev(seq[0])], w.K)                  # offline calibration batch
    static = mg.plan(a_cal, Wd, w.alpha, w.k)
    router = mg.DynamicRouter(Wd, a_cal, w.alpha, w.k)
    a_s = mg.Act.empty(static.desc, w.M)
    a_d = mg.Act.empty(router.desc, w.M)
    Y = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
    fl = 2.0 * w.M * w.K * w.N
    t_static, t_dyn = [], []
    for t in range(1, steps + 1):
        Xd = dev(seq[t])
        rows = np.sort(g.choice(w.M, FID_ROWS, replace=False))
        Xs = Xd[torch.from_numpy(rows).cuda()].contiguous()
        Yref = to_f64(seq[t][rows]) @ to_f64(W_h).T
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        torch.cuda.synchronize()
        e[0].record()
        mg.mg_forward(static, Xd, a_s, Y)
        e[1].record()
        fid_s = rel_fro(y_host(mg.forward(static, Xs)), Yref)
        used = router.plans[router.cur]
        torch.cuda.synchronize()
        e[2].record()
        router.step(Xd, a_d, Y)                               # detect + GEMM; the next plan overlaps
        e[3].record()
        torch.cuda.synchronize()
        fid_d = rel_fro(y_host(mg.forward(used, Xs)), Yref)
        t_static.append(e[0].elapsed_time(e[1]))
        t_dyn.append(e[2].elapsed_time(e[3]))
        _emit({"suite": "per-step outlier routing",
               "config": {"workload": w.name, "M": w.M, "K": w.K, "N": w.N, "k": w.k, "alpha": w.alpha,
                          "step": t, "drift_per_step": drift, "heavy_channels": int(round(0.02 * w.K))},
               "static_ms": round(t_static[-1], 4), "routed_ms": round(t_dyn[-1], 4),
               "static_tflops": round(fl / t_static[-1] / 1e9, 1), "routed_tflops": round(fl / t_dyn[-1] / 1e9, 1),
               "fidelity_rel_fro": {"static": round(fid_s, 5), "routed": round(fid_d, 5)},
               "fidelity_rows": FID_ROWS})
        del Xd, Xs
    torch.cuda.synchronize()
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=30,
                    help="untimed steps first: the GEMM needs ~20 launches to reach its steady rate")
    ap.add_argument("--workload", default="ffn0_480p_32760x5120x13824")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="rows of the workload the oracle runs for cpu_baseline (0: all of them; at 480p about "
                         "10-20 s of CPU work)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run a plain device copy of 256 MiB (HBM counter calibration)")
    ap.add_argument("--power-probe", type=float, default=2.0, metavar="SECONDS",
                    help="after the timed steps, run the dual GEMM and then the quantize back to back for "
                         "SECONDS each while sampling board power (hwmon); adds a `power` object")
    ap.add_argument("--suite", action="store_true",
                    help="one JSON line per configuration point (see the module docstring)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the dual-GEMM traffic summary from two rocprofv3 --pmc runs and exit")
    args = ap.parse_args()
    if args.summarize_pmc:
        print(json.dumps(summarize_pmc(*args.summarize_pmc, TRAFFIC_FILE)))
        return 0
    if args.gpus == 1 and args.suite:
        return suite(args)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer shards along tokens with no exchange in the forward pass)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import mixed_gemm_amd as mg
    import synth

    w = synth.ALL[args.workload]
    torch.cuda.set_device(0)
    X_h, W_h = w.make_x(), w.make_w()
    bf = w.dtype == "bf16"

    def dev(a):
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16) if bf else a).cuda()
        return t.view(torch.bfloat16) if bf else t

    X, W = dev(X_h), dev(W_h)
    M, K, N = w.M, w.K, w.N
    desc = mg.make_desc(K, N, w.k, w.alpha, "1x32", True)
    plan = mg.Plan.empty(desc)
    act = mg.Act.empty(desc, M)
    act_max = torch.empty(K, dtype=torch.float32, device="cuda")
    w_max = torch.empty(K, dtype=torch.float32, device="cuda")
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    stages = ("calib", "wrange", "plan", "quant", "gemm")
    ev = {s: [] for s in stages}

    def step(record: str):
        """One pass of the path.  record = "gemm": HIP events around the dual
        GEMM only (the timed steps); "stages": events between all stages (each
        event pair costs a few microseconds of the step, so these steps run
        after the timed ones); "": none (warm-up)."""
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] if record else None
        if record == "stages":
            marks[0].record(stream)
        mg.mg_calib_reset(act_max)
        mg.mg_calib_act(X, act_max)
        if record == "stages":
            marks[1].record(stream)
        mg.mg_weight_range(W, w_max)
        if record == "stages":
            marks[2].record(stream)
        mg.mg_plan_build(plan, act_max, w_max, W)
        if record == "stages":
            marks[3].record(stream)
        mg.mg_quantize_act(plan, X, act)
        if record:
            marks[4].record(stream)
        mg.mg_dual_gemm(plan, act, Y)
        if record:
            marks[5].record(stream)
            for i, s in enumerate(stages):
                if record == "stages" or s == "gemm":
                    ev[s if record == "stages" else "gemm_timed"].append((marks[i], marks[i + 1]))

    ev["gemm_timed"] = []
    for _ in range(args.warmup):
        step("")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step("gemm")
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    # per-stage intervals: the same number of further steps, events between stages
    for _ in range(args.steps):
        step("stages")
    torch.cuda.synchronize()
    ms = {s: float(np.mean([a.elapsed_time(b) for a, b in ev[s]])) for s in stages}
    ms["gemm"] = float(np.mean([a.elapsed_time(b) for a, b in ev["gemm_timed"]]))

    flops = w.flops()
    value = flops / (ms_step * 1e-3) / 1e12
    gemm_tflops = flops / (ms["gemm"] * 1e-3) / 1e12
    quant_bytes = M * K * (2 if bf else 4) + M * K // 2 + M * K // 32 + 2 * M * w.k
    calib_bytes = M * K * (2 if bf else 4)
    traffic = measured_traffic()
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4+bf16",
        "data": "synthetic (seeded heavy-tailed activations, Gaussian weights)",
        "config": {"workload": w.name, "M": M, "K": K, "N": N, "k": w.k, "alpha": w.alpha,
                   "weight_blocks": "1x32", "output": "bf16"},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": PEAK_FP4_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_FP4_TFLOPS, 4),
                     "traffic": traffic},
        "kernel_ms": {s: round(v, 4) for s, v in ms.items()},
        "gemm_tflops": round(gemm_tflops, 2),
        "gemm_pct_mxfp4_peak": round(100 * gemm_tflops / PEAK_FP4_TFLOPS, 2),
        "quant_gbs": round(quant_bytes / (ms["quant"] * 1e-3) / 1e9, 1),
        "quant_pct_hbm": round(100 * quant_bytes / (ms["quant"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
        "calib_gbs": round(calib_bytes / (ms["calib"] * 1e-3) / 1e9, 1),
    }
    if args.copy_calibration:
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    if args.power_probe > 0:
        out["power"] = power_probe(args.power_probe, {"gemm": lambda: mg.mg_dual_gemm(plan, act, Y),
                                                      "quant": lambda: mg.mg_quantize_act(plan, X, act)})
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, X_h, W_h, args.cpu_rows if 0 < args.cpu_rows < M else M)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

"""Throughput of the cached flow-matching DiT step on one MI355X.

Workload: 32-layer, 4096-wide DiT (32 heads x 128, SwiGLU 16384), text-to-
image layout of 256 text prefix tokens + a 64x64 target latent grid (4096
target tokens), seeded synthetic bf16 weights N(0, 1/fan_in) and N(0,1)
inputs. One extract step builds the prefix KV cache; the timed steps are
cached Euler steps (dit_step_cached + euler_update) walking the 8-step Turbo
schedule. Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
GEMM_SRC = os.path.join(ROOT, "diffusion_transformer_amd", "csrc", "gemm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_gateup_c2_cached.json")
# the dominant kernel of the cached step: the fused gate/up GEMM + SwiGLU
GATEUP_KERNEL = "gemm_w4p_swiglu_kernel"
# its grid: one 256-thread workgroup per CU (256 CUs), each walking 8 tiles
GATEUP_GRID = 256 * 256
GATEUP_LABEL = ("gemm_w4p_swiglu_kernel (gate/up + SwiGLU, persistent: one workgroup per CU, "
                "256x256 tiles, 4 waves of 128x128)")


def source_sha(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(config, batch):
    """HBM bytes per gate/up GEMM launch from the committed rocprofv3 PMC
    runs (FETCH_SIZE and WRITE_SIZE scaled by a copy-kernel calibration), or
    None when the kernel source changed since those counters were taken or
    the workload is not the one they were taken on (c2, one latent)."""
    if config != "c2" or batch != 1:
        return None
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        if t.get("source_sha256") != source_sha(GEMM_SRC):
            return None
        return t["bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        return None


def summarize_profiles(trace_dir, fetch_dir, write_dir, command, out_md, out_json):
    """Turn rocprofv3 CSV output (kernel stats + FETCH_SIZE/WRITE_SIZE
    counter runs that include the --calib-copy kernel) into the committed
    summaries."""
    import csv
    stats = list(csv.DictReader(open(os.path.join(trace_dir, "run_kernel_stats.csv"))))
    lines = [f"# rocprofv3 kernel stats: cached DiT step, c2 workload", "",
             f"Command (from the repository root on the MI355X machine):", "", "```", command, "```", "",
             "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for r in stats[:16]:
        nm = r["Name"].replace("dit::(anonymous namespace)::", "").replace("|", "/")[:80]
        lines.append(f"| {nm} | {r['Calls']} | {float(r['AverageNs'])/1e3:.1f} | "
                     f"{float(r['MinNs'])/1e3:.1f} | {float(r['MaxNs'])/1e3:.1f} | {float(r['Percentage']):.2f} |")
    res = {}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = list(csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))))
        cp = [r for r in rows if "bfloat16_copy" in r["Kernel_Name"]]
        calib = max(cp, key=lambda r: int(r["Dispatch_Id"]))
        known_kib = (1 << 28) * (4 if name == "FETCH_SIZE" else 2) / 1024.0
        factor = known_kib / float(calib["Counter_Value"])
        gu = [float(r["Counter_Value"]) for r in rows
              if GATEUP_KERNEL in r["Kernel_Name"] and int(r["Grid_Size"]) == GATEUP_GRID]
        res[name] = {"calib_kib": float(calib["Counter_Value"]), "known_kib": known_kib,
                     "factor": factor, "gateup_kib_avg": sum(gu) / len(gu), "n": len(gu)}
    fb = res["FETCH_SIZE"]["gateup_kib_avg"] * res["FETCH_SIZE"]["factor"] * 1024
    wb = res["WRITE_SIZE"]["gateup_kib_avg"] * res["WRITE_SIZE"]["factor"] * 1024
    lines += ["", "## HBM traffic of the gate/up GEMM (cached step, 4096 x 32768 x 4096)", "",
              "Two counter runs of the same command with `--steps 2 --calib-copy`, one counter each:",
              "`rocprofv3 --pmc FETCH_SIZE ...` and `rocprofv3 --pmc WRITE_SIZE ...`.",
              "Calibration: the fp32->bf16 copy of 2^28 elements reads 1 GiB and writes 512 MiB.", "",
              "| counter | copy kernel reads (KiB) | known (KiB) | factor | gate/up per launch (KiB) | scaled bytes |",
              "|---|---|---|---|---|---|"]
    for name in ("FETCH_SIZE", "WRITE_SIZE"):
        r = res[name]
        lines.append(f"| {name} | {r['calib_kib']:.0f} | {r['known_kib']:.0f} | {r['factor']:.4f} | "
                     f"{r['gateup_kib_avg']:.0f} (n={r['n']}) | "
                     f"{r['gateup_kib_avg'] * r['factor'] * 1024:.4g} |")
    alg = (4096 * 4096 + 2 * 16384 * 4096 + 4096 * 16384) * 2
    lines += ["", f"Total {fb + wb:.4g} bytes per launch vs {alg:.4g} algorithmic "
                  f"(A 32 MiB + B 256 MiB read, 128 MiB written): x{(fb + wb) / alg:.2f}."]
    open(out_md, "w").write("\n".join(lines) + "\n")
    hbm_kernels_summary(trace_dir, fetch_dir, write_dir, command, res,
                        os.path.join(ROOT, "profiles", "hbm_kernels_c2_cached.md"))
    json.dump({"kernel": GATEUP_LABEL + ", cached c2 (M=4096)",
               "source_sha256": source_sha(GEMM_SRC), "fetch": res["FETCH_SIZE"],
               "write": res["WRITE_SIZE"], "bytes_per_launch": fb + wb,
               "algorithmic_bytes": alg}, open(out_json, "w"), indent=1)


# Bandwidth-bound kernels of the c2 cached step (T = 4096 target rows,
# H = 4096): kernel-name match, grid size (work-items), which of the matching
# launches in dispatch order to take (index -> bool), algorithmic bytes per
# launch. A step launches four GEMVs with the same grid (two workgroups per
# CU), in the order timestep MLP 1, timestep MLP 2, modulation, final scale.
HBM_KERNELS = [
    ("LayerNorm + modulation (ln_mod_kernel)", "ln_mod_kernel", 2048 * 256, None,
     4096 * 4096 * (4 + 2) + 2 * 4096 * 4),
    ("final AdaLN + proj_out (final_out_kernel)", "final_out_kernel", 256 * 256, None,
     4096 * 4096 * 4 + 4096 * 64 * 4 + 4096 * 4 + 64 * 4096 * 2),
    ("img_in (img_in_kernel)", "img_in_kernel", 8 * 64 * 256, None,
     4096 * 4096 * 4 + 4096 * 64 * 4 + 4096 * 64 * 2),
    ("modulation GEMV [16384 x 4096] (gemv_kernel)", "gemv_kernel", 512 * 256, lambda i: i % 4 == 2,
     16384 * 4096 * 2 + 4096 * 4 + 16384 * 4),
    ("Euler update x += dsigma * v, 4096 x 64 (euler_kernel)", "euler_kernel", 1024 * 256, None,
     4096 * 64 * 12),
]


def hbm_kernels_summary(trace_dir, fetch_dir, write_dir, command, calib, out_md):
    """Calibrated FETCH_SIZE / WRITE_SIZE bytes per launch of the
    bandwidth-bound kernels, against their algorithmic bytes and the kernel
    trace's average duration (same command as the gate/up summary)."""
    import csv
    trace = list(csv.DictReader(open(os.path.join(trace_dir, "run_kernel_trace.csv"))))

    def grid(r):   # total work-items (the trace lists the grid per axis)
        if r.get("Grid_Size"):
            return int(r["Grid_Size"])
        return int(r["Grid_Size_X"]) * int(r.get("Grid_Size_Y") or 1) * int(r.get("Grid_Size_Z") or 1)
    lines = ["# rocprofv3 HBM bytes of the bandwidth-bound kernels: cached DiT step, c2 workload", "",
             "Commands (from the repository root on the MI355X machine; R = repository root):", "", "```",
             command, "```", "",
             f"FETCH_SIZE x{calib['FETCH_SIZE']['factor']:.4f}, WRITE_SIZE x{calib['WRITE_SIZE']['factor']:.4f} "
             "(the fp32->bf16 copy of 2^28 elements reads 1 GiB and writes 512 MiB). Durations: kernel "
             "trace of the timed run. HBM peak 8 TB/s.", "",
             "| kernel | launches | avg us | fetched MB | written MB | algorithmic MB | measured / alg "
             "| GB/s (alg bytes) | % of 8 TB/s |", "|---|---|---|---|---|---|---|---|---|"]
    def pick(rows, match, g, sel):
        rows = sorted((r for r in rows if match in r["Kernel_Name"] and grid(r) == g),
                      key=lambda r: int(r["Dispatch_Id"]))
        return [r for i, r in enumerate(rows) if sel is None or sel(i)]
    for label, match, g, sel, alg in HBM_KERNELS:
        ns = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in pick(trace, match, g, sel)]
        by = {}
        for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
            rows = pick(csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))), match, g, sel)
            by[name] = (sum(float(r["Counter_Value"]) for r in rows) / len(rows) * calib[name]["factor"] * 1024
                        if rows else float("nan"))
        if not ns:
            continue
        avg = sum(ns) / len(ns)
        gbs = alg / avg
        lines.append(f"| {label} | {len(ns)} | {avg / 1e3:.1f} | {by['FETCH_SIZE'] / 1e6:.1f} | "
                     f"{by['WRITE_SIZE'] / 1e6:.1f} | {alg / 1e6:.1f} | "
                     f"{(by['FETCH_SIZE'] + by['WRITE_SIZE']) / alg:.2f} | {gbs:.0f} | "
                     f"{gbs / PEAK_HBM_GBS * 100:.1f} |")
    open(out_md, "w").write("\n".join(lines) + "\n")


def summarize_counters(counter_dir, fetch_dir, write_dir, command, out_md,
                       title="cached DiT step, c2 workload", ln_section=True):
    """Per-kernel rocprofv3 counter evidence for the cached step: MFMA
    instructions (all v_mfma_f32_32x32x16_bf16, 32768 flop each) over the
    dispatch's own duration against the dense bf16 peak, the matrix-core
    busy counter, LDS traffic, and for the LayerNorm the calibrated HBM bytes
    (FETCH_SIZE / WRITE_SIZE runs) against the HBM peak."""
    import csv
    from collections import defaultdict

    def per_dispatch(d):
        rows = list(csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))))
        out = defaultdict(lambda: {"counters": defaultdict(float)})
        for r in rows:
            e = out[r["Dispatch_Id"]]
            e["name"] = r["Kernel_Name"]
            e["grid"] = int(r["Grid_Size"])
            e["counters"][r["Counter_Name"]] += float(r["Counter_Value"])
            if r.get("End_Timestamp"):
                e["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        kt = os.path.join(d, "run_kernel_trace.csv")
        if os.path.exists(kt):
            for r in csv.DictReader(open(kt)):
                if r["Dispatch_Id"] in out:
                    out[r["Dispatch_Id"]]["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        return out

    disp = per_dispatch(counter_dir)
    # O (K = hidden) and down (K = ffn) share the residual epilogue; per
    # workgroup the down projection issues ffn/hidden times the MFMAs
    def per_wg(e):
        return e["counters"]["SQ_INSTS_MFMA"] / max(e["grid"] // 256, 1)

    mf = [per_wg(e) for e in disp.values() if "gemm_w4_kernel<2" in e["name"]]
    split = (min(mf) + max(mf)) / 2 if mf else 0

    def cls(e):
        n = e["name"]
        if "gemm_w4_kernel<5" in n:
            return "QKV GEMM + norm/RoPE/cache epilogue"
        if GATEUP_KERNEL in n:
            return "gate/up GEMM (SwiGLU epilogue)"
        if "gemm_w4_kernel<2" in n:
            return "O GEMM (residual epilogue)" if per_wg(e) < split else "down GEMM (residual epilogue)"
        if "attn3_kernel" in n:
            return "attention, cached steps (pipelined kernel)"
        if "attn2_kernel" in n:
            return "attention, extract step (cache build)"
        return None

    groups = defaultdict(list)
    for e in disp.values():
        c = cls(e)
        if c and "ns" in e:
            groups[c].append(e)
    lines = [f"# rocprofv3 counters per kernel: {title}", "",
             "Commands (from the repository root on the MI355X machine; R = repository root):", "", "```",
             command, "```", "",
             "MFMA: `SQ_INSTS_MFMA` x 32768 flop (every MFMA here is v_mfma_f32_32x32x16_bf16) over "
             "each dispatch's own duration, against the dense bf16 peak of 2.5 PFLOP/s. "
             "`SQ_VALU_MFMA_BUSY_CYCLES` is shown as a fraction of 1024 SIMDs x "
             "`GRBM_GUI_ACTIVE`/8 (eight XCDs), i.e. per cycle at the clock the kernel actually ran.", "",
             "| kernel | dispatches | avg us | MFMA instr | TFLOP/s | % bf16 peak | MFMA busy / SIMD-cycle "
             "| clock GHz | LDS instr | LDS bank conflicts |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    for c in ("QKV GEMM + norm/RoPE/cache epilogue", "O GEMM (residual epilogue)",
              "gate/up GEMM (SwiGLU epilogue)", "down GEMM (residual epilogue)",
              "attention, cached steps (pipelined kernel)", "attention, extract step (cache build)"):
        es = groups.get(c)
        if not es:
            continue
        n = len(es)
        ns = sum(e["ns"] for e in es) / n
        cs = {k: sum(e["counters"][k] for e in es) / n for k in es[0]["counters"]}
        tf = cs["SQ_INSTS_MFMA"] * 32768 / (ns * 1e-9) / 1e12
        cyc = cs["GRBM_GUI_ACTIVE"] / 8
        busy = cs["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * cyc) if cyc else float("nan")
        lines.append(f"| {c} | {n} | {ns / 1e3:.1f} | {cs['SQ_INSTS_MFMA']:.4g} | {tf:.0f} | "
                     f"{tf / PEAK_BF16_TFLOPS * 100:.1f} | {busy * 100:.1f}% | {cyc / ns:.2f} | "
                     f"{cs['SQ_INSTS_LDS']:.4g} | {cs['SQ_LDS_BANK_CONFLICT']:.3g} |")
    # LayerNorm: calibrated HBM bytes per dispatch
    res = {}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        dd = per_dispatch(d)
        cp = [e for e in dd.values() if "bfloat16_copy" in e["name"]]
        calib = cp[-1]["counters"][name]
        known_kib = (1 << 28) * (4 if name == "FETCH_SIZE" else 2) / 1024.0
        ln = [e for e in dd.values() if "ln_mod_kernel" in e["name"] and "ns" in e and e["grid"] == 2048 * 256]
        res[name] = (known_kib / calib, ln)
    ff, lnf = res["FETCH_SIZE"]
    wf, lnw = res["WRITE_SIZE"]
    if ln_section and lnf and lnw:
        fb = sum(e["counters"]["FETCH_SIZE"] for e in lnf) / len(lnf) * ff * 1024
        wb = sum(e["counters"]["WRITE_SIZE"] for e in lnw) / len(lnw) * wf * 1024
        ns = (sum(e["ns"] for e in lnf) + sum(e["ns"] for e in lnw)) / (len(lnf) + len(lnw))
        alg = 4096 * 4096 * 6
        lines += ["", "## LayerNorm + modulation (4096 rows x 4096): HBM bytes", "",
                  "| dispatches | avg us | fetched bytes | written bytes | algorithmic | GB/s (measured bytes) "
                  "| % of 8 TB/s |", "|---|---|---|---|---|---|---|",
                  f"| {len(lnf)}+{len(lnw)} | {ns / 1e3:.1f} | {fb:.4g} | {wb:.4g} | {alg:.4g} | "
                  f"{(fb + wb) / (ns * 1e-9) / 1e9:.0f} | {(fb + wb) / (ns * 1e-9) / 1e9 / PEAK_HBM_GBS * 100:.1f} |",
                  "", f"(FETCH_SIZE x{ff:.3f}, WRITE_SIZE x{wf:.3f} from the fp32->bf16 copy calibration; "
                  "durations are those of the counter runs.)"]
    open(out_md, "w").write("\n".join(lines) + "\n")


def describe(cfg):
    """Token layout of a workload in words, e.g. '256 text + 64x64 target'."""
    parts = []
    segs = list(cfg["segments"])
    i = 0
    while i < len(segs):
        seg, n = segs[i], 1
        while i + n < len(segs) and segs[i + n] == seg:
            n += 1
        if seg[0] == "text":
            w = f"{seg[1] * n} text"
        else:
            w = f"{seg[1]}x{seg[2]} {'reference' if seg[0] == 'ref' else 'target'}"
            w = f"{n} x {w}s" if n > 1 else w
        parts.append(w)
        i += n
    kind = {0: "text-to-image", 1: "image editing"}.get(sum(s[0] == "ref" for s in cfg["segments"]),
                                                       "multi-reference")
    return f"{kind}, " + " + ".join(parts) + " tokens"


def layer_flops(T, S, H, F, nh, d):
    """Algorithmic FLOPs of one cached layer: QKV, O, gate/up, down GEMMs
    (2 flop per MAC) and attention over all S keys (QKᵀ and PV)."""
    return {"gemm_qkv": 2 * T * H * 3 * H, "gemm_o": 2 * T * H * H,
            "gemm_gateup": 2 * T * H * 2 * F, "gemm_down": 2 * T * F * H,
            "attention": 4 * T * S * d * nh}


def cpu_baseline(cfg, seconds_hint=True):
    """The fp64 oracle timed on this host on a bounded sample: one of the
    32 layers of the cached step (all 4096 target rows against a 256-row
    prefix cache), scaled x32 to a full cached step."""
    import oracle as O
    from diffusion_transformer_amd import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [os.cpu_count()])
    except Exception:
        cores = os.cpu_count()
    c1 = dict(cfg)
    c1["n_layers"] = 1
    W = synth.make_weights(c1, seed=21)
    I = synth.make_inputs(c1, seed=21)
    dims = O.DitDims(hidden=cfg["hidden"], n_heads=cfg["n_heads"], head_dim=cfg["head_dim"],
                     ffn=cfg["ffn"], n_layers=1, latent=cfg["latent"], time_dim=cfg["time_dim"],
                     rope_dims=tuple(cfg["rope_dims"]))
    lay = O.build_layout(cfg["segments"])
    rng = np.random.default_rng(3)
    cache = [(rng.standard_normal((lay.P, dims.n_heads, dims.head_dim)),
              rng.standard_normal((lay.P, dims.n_heads, dims.head_dim)))]
    t0 = time.perf_counter()
    O.forward_cached(W, dims, lay, cache, I["x0"], 0.978453)
    dt = time.perf_counter() - t0
    step_s = dt * cfg["n_layers"]
    return {"value": lay.T / step_s, "unit": "target tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": (f"1 of {cfg['n_layers']} layers of one cached step (T={lay.T} target rows, "
                       f"P={lay.P} cached prefix rows, fp64 NumPy), {dt:.1f} s measured, "
                       f"scaled x{cfg['n_layers']}")}


def run_conditions(dev, batch, peaks):
    """What every number above was measured under: batch, prefix cache,
    guidance scale, software versions, device and, from the register-only
    MFMA loop, the clock the matrix cores effectively ran at (each of the
    1024 SIMDs retires 1024 bf16 flop per clock at full rate)."""
    import torch
    props = torch.cuda.get_device_properties(dev)
    cond = {"batch": batch,
            "prefix_cache": "on: value and latency are cached steps; extract_ms is the cache build",
            "cfg_scale": 1.0,
            "hip": torch.version.hip, "torch": torch.__version__,
            "device": f"{props.name} ({getattr(props, 'gcnArchName', '?')}), "
                      f"{props.multi_processor_count} CUs, {props.total_memory / 2**30:.0f} GiB"}
    if peaks:
        cond["mfma_loop_clock_ghz"] = round(peaks["mfma_bf16_tflops"] * 1e12 / (1024 * 1024) / 1e9, 3)
    return cond


def measured_peaks(L, dev):
    """The ceilings this GPU actually reaches, next to the spec peaks: a
    register-only bf16 MFMA loop on N(0,1) operands (the library's own
    32x32x16 instruction, one workgroup of 4 waves per CU, ~0.5 s per
    launch, best of 3) and a 1 GiB fp32 device-to-device copy (bytes read +
    written, median of 10)."""
    import torch
    g = torch.Generator(device=dev).manual_seed(7)
    ops = torch.randn(1 << 19, generator=g, device=dev).to(torch.bfloat16)   # 1 MiB
    blocks, iters = 256, 400
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    flop = blocks * 4 * iters * 64 * 32768
    best = 0.0
    for _ in range(3):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        L.dit_debug_mfma_loop(ops, out, blocks, iters)
        b.record()
        torch.cuda.synchronize()
        best = max(best, flop / (a.elapsed_time(b) / 1e3) / 1e12)
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    L.dit_debug_stream_copy(src, dst)
    ts = []
    for _ in range(10):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        L.dit_debug_stream_copy(src, dst)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    gbs = 2 * src.numel() * 4 / (float(np.median(ts)) / 1e3) / 1e9
    del src, dst
    return {"mfma_bf16_tflops": round(best, 1), "hbm_copy_gbs": round(gbs, 1),
            "method": "register-only v_mfma_f32_32x32x16_bf16 loop on N(0,1) bf16 operands "
                      "(256 workgroups x 4 waves, 8 chains per wave, best of 3); "
                      "1 GiB device copy with 16-byte accesses (the library's copy kernel), "
                      "read + written bytes (median of 10)"}


def visible_pairs(row_limit, rows):
    """Visible (query, key) pairs of the given query rows under the
    row-limit form of the block-causal mask."""
    return int(np.sum(row_limit[rows].astype(np.int64) + 1))


def time_workload(rt, L, name, steps=5):
    """Cached and extract step times of another workload with the same
    model (same layer shapes): the editing and multi-reference layouts."""
    import torch
    from diffusion_transformer_amd import synth
    cfg = synth.config(name)
    H, F, nh, d, Lc = cfg["hidden"], cfg["ffn"], cfg["n_heads"], cfg["head_dim"], cfg["n_layers"]
    I = synth.make_inputs(cfg, seed=21)
    seq = rt.sequence(cfg["segments"])
    P, T, S = seq.P, seq.T, seq.S
    pre = rt.prefix_hidden(I)
    x = torch.from_numpy(I["x0"]).to(rt.device)
    sig = cfg["sigmas"]
    cache = rt.alloc_cache(seq)
    ws = rt.alloc_workspace(S)
    v = torch.empty_like(x)
    stream = torch.cuda.current_stream()

    def ev():
        return torch.cuda.Event(enable_timing=True)
    rt.step_extract(seq, pre, x.clone(), sig[0], cache, v, ws)
    ex = []
    for _ in range(2):
        a, b = ev(), ev()
        a.record(stream)
        rt.step_extract(seq, pre, x.clone(), sig[0], cache, v, ws)
        b.record(stream)
        torch.cuda.synchronize()
        ex.append(a.elapsed_time(b))
    xc = x.clone()
    rt.step_cached(seq, xc, sig[1], cache, v, ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        j = 1 + (k % (len(sig) - 2))
        rt.step_cached(seq, xc, sig[j], cache, v, ws)
        L.euler_update(xc, v, sig[j], sig[j + 1])
    torch.cuda.synchronize()
    cached_ms = (time.perf_counter() - t0) * 1000.0 / steps
    L.dit_profile_enable(rt.model, "attention")
    for k in range(2):
        rt.step_cached(seq, xc, sig[1 + k], cache, v, ws)
    torch.cuda.synchronize()
    att_ms, att_n = L.dit_profile_read(rt.model)
    L.dit_profile_enable(rt.model, "off")
    att_avg = att_ms / max(att_n, 1)
    lim = seq.host["row_limit"]
    gemm = lambda n: 2 * n * H * (3 * H + H + 2 * F) + 2 * n * F * H
    fl_cached = Lc * (gemm(T) + 4 * d * nh * visible_pairs(lim, np.arange(P, S)))
    fl_extract = Lc * (gemm(S) + 4 * d * nh * visible_pairs(lim, np.arange(S)))
    att_tf = 4 * d * nh * T * S / (att_avg / 1e3) / 1e12
    extract_ms = float(np.median(ex))
    out = {"workload": f"{name}: {describe(cfg)}", "prefix_tokens": P, "target_tokens": T,
           "ms_per_cached_step": round(cached_ms, 3), "target_tok_s": round(T / (cached_ms / 1e3), 1),
           "step_frac_bf16_peak": round(fl_cached / (cached_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "extract_ms": round(extract_ms, 3), "extract_over_cached": round(extract_ms / cached_ms, 3),
           "flop_ratio_extract_over_cached": round(fl_extract / fl_cached, 3),
           "token_ratio_S_over_T": round(S / T, 3),
           "attention_ms_per_layer": round(att_avg, 4),
           "attention_frac_bf16_peak": round(att_tf / PEAK_BF16_TFLOPS, 4)}
    del cache, ws
    torch.cuda.empty_cache()
    return out


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-trace":
        # bench.py --summarize-trace TRACE_DIR TITLE "COMMAND" OUT_MD
        import csv
        stats = list(csv.DictReader(open(os.path.join(sys.argv[2], "run_kernel_stats.csv"))))
        lines = [f"# rocprofv3 kernel stats: {sys.argv[3]}", "",
                 "Command (from the repository root on the MI355X machine; R = repository root):", "",
                 "```", sys.argv[4], "```", "",
                 "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
        for r in stats[:14]:
            nm = r["Name"].replace("dit::(anonymous namespace)::", "").replace("|", "/")[:80]
            lines.append(f"| {nm} | {r['Calls']} | {float(r['AverageNs'])/1e3:.1f} | "
                         f"{float(r['MinNs'])/1e3:.1f} | {float(r['MaxNs'])/1e3:.1f} | "
                         f"{float(r['Percentage']):.2f} |")
        open(sys.argv[5], "w").write("\n".join(lines) + "\n")
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-counters":
        # bench.py --summarize-counters COUNTER_DIR FETCH_DIR WRITE_DIR "COMMAND" [OUT_MD "TITLE"]
        if len(sys.argv) > 7:
            summarize_counters(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], sys.argv[6], sys.argv[7],
                               ln_section=False)
        else:
            summarize_counters(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5],
                               os.path.join(ROOT, "profiles", "counters_c2_cached.md"))
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-prof":
        # bench.py --summarize-prof TRACE_DIR FETCH_DIR WRITE_DIR "COMMAND"
        summarize_profiles(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5],
                           os.path.join(ROOT, "profiles", "gemm_gateup_c2_cached.md"), TRAFFIC_FILE)
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c2")
    ap.add_argument("--batch", type=int, default=1,
                    help="target latents denoised together against one shared prefix")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--only-timed", action="store_true",
                    help="run only cache build + warmup + timed cached steps (for profilers)")
    ap.add_argument("--workloads", default="c3,c4",
                    help="other workloads with the same layer shapes timed in the same run "
                         "(reusing the loaded weights), reported under 'workloads'")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured MFMA / copy ceilings")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after timing, run one fp32->bf16 conversion of 2^28 elements "
                         "(1 GiB read, 512 MiB written) to calibrate byte counters")
    args = ap.parse_args()
    if args.only_timed:
        args.no_breakdown = True
        args.no_peaks = True
        args.workloads = ""
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from diffusion_transformer_amd import _lib as L
    from diffusion_transformer_amd import synth
    from diffusion_transformer_amd.runtime import DitRuntime, random_weights_device

    dev = torch.device("cuda:0")
    cfg = synth.config(args.config)
    H, F, nh, d, Lc = cfg["hidden"], cfg["ffn"], cfg["n_heads"], cfg["head_dim"], cfg["n_layers"]
    print(f"[bench] workload {args.config}: generating weights on GPU", file=sys.stderr, flush=True)
    Wd = random_weights_device(cfg, 21, dev)
    rt = DitRuntime(cfg, Wd, device=dev, on_device=True)
    I = synth.make_inputs(cfg, seed=21)
    B = args.batch
    seq = rt.sequence(cfg["segments"], batch=B)
    P, T1, S = seq.P, seq.T, seq.S
    T = B * T1          # target rows of all elements
    pre = rt.prefix_hidden(I)
    x = torch.cat([torch.from_numpy(I["x0"])] +
                  [torch.from_numpy(synth._rng(100 + b, "x_batch").standard_normal(
                      (T1, cfg["latent"]), dtype=np.float32)) for b in range(1, B)]).to(dev)
    sig = cfg["sigmas"]
    cache = rt.alloc_cache(seq)
    ws = rt.alloc_workspace(seq.S_all)
    v = torch.empty_like(x)
    stream = torch.cuda.current_stream()

    def extract(xx):
        rt.step_extract(seq, pre, xx, sig[0], cache, v, ws)

    def cached(k, xx):
        # cached steps walk the Turbo schedule's steps 2..8
        j = 1 + (k % (len(sig) - 2))
        rt.step_cached(seq, xx, sig[j], cache, v, ws)
        L.euler_update(xx, v, sig[j], sig[j + 1])

    print(f"[bench] P={P} T={T} S={S} L={Lc}: warmup", file=sys.stderr, flush=True)
    extract(x)
    xw = x.clone()
    for k in range(args.warmup):
        cached(k, xw)
    torch.cuda.synchronize()

    # ---- timed region: K cached Euler steps; dominant kernel timed by
    # events the library records around each of its launches ----
    L.dit_profile_enable(rt.model, "gemm_gateup")
    xt = x.clone()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record(stream)
    for k in range(args.steps):
        cached(k, xt)
        evs[k + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gu_ms, gu_n = L.dit_profile_read(rt.model)
    L.dit_profile_enable(rt.model, "off")
    step_ms = np.array([evs[k].elapsed_time(evs[k + 1]) for k in range(args.steps)])
    ms_per_step = wall * 1000.0 / args.steps
    value = T / (ms_per_step / 1000.0)
    print(f"[bench] cached step {ms_per_step:.3f} ms, {value:.0f} target tok/s", file=sys.stderr,
          flush=True)

    fl = layer_flops(T, S, H, F, nh, d)   # T = all elements' target rows, each over S keys
    gu_avg = gu_ms / max(gu_n, 1)
    gu_tflops = fl["gemm_gateup"] / (gu_avg / 1e3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(gu_tflops, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(gu_tflops / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(args.config, B), "kernel": GATEUP_LABEL,
                "avg_launch_ms": round(gu_avg, 4), "launches": gu_n}

    if args.calib_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty(1 << 28, dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- extract step and full 8-step loop ----
    extract_ms = loop_ms = float("nan")
    ex = []
    for _ in range(0 if args.only_timed else 3):
        a = torch.cuda.Event(enable_timing=True); b = torch.cuda.Event(enable_timing=True)
        a.record(stream); extract(x.clone()); b.record(stream); torch.cuda.synchronize()
        ex.append(a.elapsed_time(b))
    if not args.only_timed:
        extract_ms = float(np.median(ex))
        xl = x.clone()
        a = torch.cuda.Event(enable_timing=True); b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        rt.step_extract(seq, pre, xl, sig[0], cache, v, ws)
        L.euler_update(xl, v, sig[0], sig[1])
        for j in range(1, len(sig) - 1):
            rt.step_cached(seq, xl, sig[j], cache, v, ws)
            L.euler_update(xl, v, sig[j], sig[j + 1])
        b.record(stream)
        torch.cuda.synchronize()
        loop_ms = a.elapsed_time(b)

    # ---- per-kernel breakdown of the cached step (separate passes) ----
    breakdown = {}
    if not args.no_breakdown:
        hbm_bytes = {   # algorithmic bytes per launch of the bandwidth-bound kernels
            "ln": T * H * (4 + 2) + 2 * H * 4,
            "final": T * H * 4 + T * cfg["latent"] * 4 + H * 4 + cfg["latent"] * H * 2,
            "img_in": T * H * 4 + T * cfg["latent"] * 4 + H * cfg["latent"] * 2,
            "gemv_mod": 4 * H * H * 2 + H * 4 + 4 * H * 4,
        }
        for name in ("gemm_qkv", "gemm_o", "gemm_gateup", "gemm_down", "attention", "ln", "final",
                     "img_in", "gemv_mod"):
            L.dit_profile_enable(rt.model, name)
            xb = x.clone()
            for k in range(3):
                cached(k, xb)
            torch.cuda.synchronize()
            ms, n = L.dit_profile_read(rt.model)
            avg = ms / max(n, 1)
            entry = {"avg_ms": round(avg, 4), "per_step_ms": round(ms / 3, 3)}
            if name in fl:
                tf = fl[name] / (avg / 1e3) / 1e12
                entry.update({"tflops": round(tf, 1), "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)})
            elif name in hbm_bytes:
                by = hbm_bytes[name]
                gbs = by / (avg / 1e3) / 1e9
                entry.update({"gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)})
            breakdown[name] = entry
        L.dit_profile_enable(rt.model, "off")

    # ---- the same model on the other workloads (same layer shapes) ----
    others = {}
    for name in [w for w in args.workloads.split(",") if w and w != args.config and B == 1]:
        print(f"[bench] workload {name} with the same weights", file=sys.stderr, flush=True)
        others[name] = time_workload(rt, L, name)

    peaks = None
    if not args.no_peaks:
        print("[bench] measured MFMA / copy ceilings", file=sys.stderr, flush=True)
        peaks = measured_peaks(L, dev)
        roofline["frac_measured_peak"] = round(gu_tflops / peaks["mfma_bf16_tflops"], 4)
        for name, e in breakdown.items():
            if "tflops" in e:
                e["frac_measured_mfma_peak"] = round(e["tflops"] / peaks["mfma_bf16_tflops"], 4)
            if "gbs" in e:
                e["frac_measured_copy_peak"] = round(e["gbs"] / peaks["hbm_copy_gbs"], 4)

    step_flops = Lc * sum(fl.values())
    out = {
        "metric": "target tokens/s per cached Euler step (32-layer DiT); MFMA % of bf16 peak",
        "value": round(value, 1),
        "unit": "target tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1/fan_in) bf16 weights, N(0,1) inputs)",
        "config": {"workload": f"{args.config}: {describe(cfg)}"
                               + (f", {B} target latents sharing the prefix" if B > 1 else "")
                               + f", {Lc} layers, hidden {H}, "
                               f"{nh}x{d} heads, SwiGLU {F}, cached Euler step (Turbo schedule)",
                   "prefix_tokens": P, "target_tokens": T1, "layers": Lc, "batch": B,
                   "parallelism": "single GPU"},
        "latency_ms": {"p50": round(float(np.percentile(step_ms, 50)), 3),
                       "p95": round(float(np.percentile(step_ms, 95)), 3),
                       "p99": round(float(np.percentile(step_ms, 99)), 3)},
        "step_tflops": round(step_flops / (ms_per_step / 1e3) / 1e12, 1),
        "step_frac_bf16_peak": round(step_flops / (ms_per_step / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "extract_ms": None if extract_ms != extract_ms else round(extract_ms, 3),
        "extract_over_cached": None if extract_ms != extract_ms else round(extract_ms / ms_per_step, 3),
        "loop_8step_ms": None if loop_ms != loop_ms else round(loop_ms, 3),
        "roofline": roofline,
        "kernels": breakdown,
        "measured_peaks": peaks,
        "workloads": others,
        "run_conditions": run_conditions(dev, B, peaks),
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the fp64 oracle on the host (cpu_baseline)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg)
    else:
        out["cpu_baseline"] = None
    rt.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

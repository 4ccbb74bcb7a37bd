#!/usr/bin/env python3
"""Throughput of the action-expert denoise loop on one MI355X.

One bench "step" is one ``vla_denoise`` call: the whole hot path (prologue,
N Euler steps of the 36-layer expert, every Euler update) over one batch of
synthetic inputs resident in HBM. The headline workload is the LingBot-shaped
expert (36 layers, hidden 1024, 16/2 heads of 128, SwiGLU 4096, prefix KV 256,
chunk 50x75, 10 Euler steps, batch 1, bf16 weights and activations, fp32
accumulation). ``value`` is denoise steps per second (Euler steps of the whole
batch per second); chunks per second are reported beside it.

Also reported:
  * ``call_roofline``: the whole call's algorithmic bytes (batch 1) or flops
    (batch 64) over its time, against the HBM or bf16 MFMA peak, with the
    target fraction beside it;
  * ``roofline``: the kernel family that takes the largest share of a layer's
    time, its algorithmic bytes (or flops) per launch over its mean launch
    time, measured with HIP events around each launch; ``roofline_worst`` is
    the family furthest below its roofline;
  * ``cpu_baseline``: the CPU oracle (its fp32 twin: the same code on float32
    inputs) on a bounded sample of every workload, on all cores of the
    process's affinity mask and, for the two batch-1 bf16 workloads of the
    smallest sizes, on one thread; the fp64 oracle once for reference;
  * ``v2_b1``, ``fp8_b1``, ``batch64``: the V2-shaped 50-step loop, the E4M3
    weight tier (25 steps) and the batched-replica workload (64 requests,
    GEMM M = 3200), each with its call roofline;
  * ``prefill``: the prefix K/V construction that precedes the loop (the
    36-layer LingBot-shaped backbone over a 256-token prefix) at 1 and 16
    requests per call, as tokens per second with its weight-streaming and
    MFMA fractions.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "denoise steps/s & chunks/s (36L bf16, chunk 50×75, b=1/64); % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0

CALL_TARGET = {"hbm": 0.70, "mfma": 0.50}   # batch-1 HBM and batch-64 bf16 MFMA fractions aimed at

# HBM traffic of each kernel family of the batch-1 layer from rocprofv3
# FETCH_SIZE / WRITE_SIZE counter runs, scaled by what the counters read for a
# plain copy of known size. The summary records a hash of the kernel sources;
# once they change, the figures no longer describe the kernels and `traffic`
# is reported as null.
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "layer_kernels_lingbot_b1_counters.txt")
# kernel family -> (kernel name in the trace, which of that name's launches per layer)
TRAFFIC_KERNELS = {
    "qkv_rope_gemm": ("skinny_gemm_kernel<0, 2, true>", 0, 1),
    "gqa_attention": ("attn_kernel<", 0, 1),
    "o_proj_gemm": ("skinny_gemm_kernel<0, 4, true>", 0, 2),
    "gate_up_swiglu_gemm": ("skinny_gemm_kernel<0, 3, true>", 0, 1),
    "down_gemm": ("skinny_gemm_kernel<0, 4, true>", 1, 2),
}
KERNEL_SOURCES = ("vla_flow_matching_denoise_amd/csrc/common.h", "vla_flow_matching_denoise_amd/csrc/kernels_layer.h")
COPY_BYTES = 256 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def call_work(cfg):
    """Algorithmic bytes and flops of one call (weights streamed once per Euler step)."""
    H, L, A, T, B, P = cfg.hidden, cfg.n_layers, cfg.action_dim, cfg.horizon, cfg.batch, cfg.prefix_len
    nq, nkv, dh, I, E, N = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.intermediate, cfg.time_emb_dim, cfg.n_steps
    wb = 1 if cfg.weight_dtype == "fp8_e4m3" else 2
    block_params = L * ((nq + 2 * nkv) * dh * H + H * nq * dh + 2 * I * H + H * I)
    scales = L * ((nq + 2 * nkv) * dh + H + 2 * I + H) * 4 if wb == 1 else 0
    inout_params = 2 * H * A
    mod_params = (6 * L + 2) * H * H + H * E + H * H
    prefix = B * L * P * nkv * dh * 2 * 2
    per_step = block_params * wb + scales + prefix + inout_params * 2 + (H + A) * 4
    once = mod_params * 2 + ((6 * L + 2) * H + 2 * H) * 4 + 2 * B * T * A * 4 + B * (N + 1) * 4
    bytes_call = N * per_step + once
    M = B * T
    flops_call = (N * (2 * M * (block_params + inout_params) + 4 * B * nq * T * (P + T) * dh * L)
                  + 2 * B * N * mod_params)
    return bytes_call, flops_call


def time_calls(ex, inputs, n_steps, warmup, steps):
    import torch
    pk, pv, x0, ts = inputs
    out = torch.empty_like(x0)
    ex.denoise(pk, pv, x0, ts, n_steps, out=out)         # first call captures the graph (untimed)
    torch.cuda.synchronize()
    for _ in range(warmup):
        ex.denoise(pk, pv, x0, ts, n_steps, out=out)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        ex.denoise(pk, pv, x0, ts, n_steps, out=out)
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])  # ms
    return wall, per_call, out


def kernel_rooflines(ex, cfg, iters):
    """Mean launch time of every kernel family of the layer (HIP events per launch)."""
    from vla_flow_matching_denoise_amd import binding as B
    names = {B.VLA_KERNEL_QKV: "qkv_rope_gemm", B.VLA_KERNEL_ATTN: "gqa_attention",
             B.VLA_KERNEL_O: "o_proj_gemm", B.VLA_KERNEL_GATE_UP: "gate_up_swiglu_gemm",
             B.VLA_KERNEL_DOWN: "down_gemm"}
    res = {}
    for k, name in names.items():
        us, by, fl = B.vla_profile_kernel(ex.ctx, k, iters)
        res[name] = {"us": us, "bytes": by, "flops": fl,
                     "GBps": by / us / 1e3, "TFLOPs": fl / us / 1e6}
    return res


def _roof(name, r, bound, mfma_peak):
    if bound == "hbm":
        ach, peak, unit = r["GBps"], HBM_PEAK_GBS, "GB/s"
    else:
        ach, peak, unit = r["TFLOPs"], mfma_peak, "TFLOP/s"
    return {"bound": bound, "kernel": name, "achieved": round(ach, 2), "peak": peak, "unit": unit,
            "frac": round(ach / peak, 4), "traffic": None, "us_per_launch": round(r["us"], 3),
            "algorithmic_bytes_per_launch": int(r["bytes"]), "algorithmic_flops_per_launch": int(r["flops"])}


def dominant(res, bound, mfma_peak=BF16_PEAK_TFLOPS):
    """The kernel family with the largest share of a layer's time (every family
    runs once per layer), and the family furthest below its roofline."""
    name = max(res, key=lambda n: res[n]["us"])
    worst = min(res, key=lambda n: _roof(n, res[n], bound, mfma_peak)["frac"])
    return name, _roof(name, res[name], bound, mfma_peak), _roof(worst, res[worst], bound, mfma_peak)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(family):
    """Bytes per launch of a kernel family from the committed counter summary,
    or None when absent or taken on kernel sources other than the current ones."""
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None
    fields = {}
    with open(TRAFFIC_SUMMARY) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_sha256_16") != kernel_source_hash():
        return None
    try:
        return int(float(fields[f"traffic_bytes_per_launch.{family}"]))
    except (KeyError, ValueError):
        return None


def counter_run(iters):
    """Workload of the counter runs: a plain copy of COPY_BYTES (calibration),
    then `iters` whole layers of the batch-1 workload (every kernel family of
    the layer launches once per layer)."""
    import torch
    import synth
    from vla_flow_matching_denoise_amd import binding as B
    from vla_flow_matching_denoise_amd.expert import Expert, dims_from_config
    torch.cuda.set_device(0)
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    cfg = synth.config(2)
    ex = Expert(synth.make_weights(cfg, seed=0), dims_from_config(cfg))
    dev_in, _ = build_inputs(cfg)
    ex.denoise(*dev_in, cfg.n_steps)             # fills the modulation table
    torch.cuda.synchronize()
    B.vla_profile_kernel(ex.ctx, B.VLA_KERNEL_GATE_UP, iters)
    torch.cuda.synchronize()
    ex.close()
    log(f"[bench] counter run done: copy of {COPY_BYTES} B x3, {iters} layers")


def _counter_rows(d):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    with open(files[0]) as fh:
        return list(csv.DictReader(fh))


def _per_dispatch(rows, counter, match):
    """Counter value per dispatch (summed over its instances), in dispatch order."""
    vals = {}
    for r in rows:
        if r.get("Counter_Name") == counter and match(r.get("Kernel_Name", "")):
            d = int(r["Dispatch_Id"])
            vals[d] = vals.get(d, 0.0) + float(r["Counter_Value"])
    return [vals[d] for d in sorted(vals)]


def traffic_from(fetch_dir, write_dir, cmd_fetch, cmd_write):
    """Writes the counter summary from two rocprofv3 --pmc output folders."""
    out = {}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(d)
        copy = _per_dispatch(rows, name, lambda k: "copy" in k.lower())
        if not copy:
            raise SystemExit(f"{name}: no copy dispatches")
        scale = (COPY_BYTES / 1024.0) / max(copy)      # bytes of KiB reported, per counted KiB
        out[name] = {"copy_kib": max(copy), "scale": scale, "fam": {}}
        for fam, (kname, which, per_layer) in TRAFFIC_KERNELS.items():
            vals = _per_dispatch(rows, name, lambda k, kname=kname: kname in k)[which::per_layer]
            if not vals:
                raise SystemExit(f"{name}: no dispatches of {kname}")
            out[name]["fam"][fam] = (float(np.mean(vals)), len(vals))
    lines = [
        "# HBM traffic per launch of each kernel family of one expert layer,",
        "# LingBot-shaped batch-1 workload (M = 50 rows, hidden 1024, 16/2 heads of 128, SwiGLU 4096, prefix 256).",
        "# Two rocprofv3 counter runs of `python bench.py --counter-run`, each scaled by the",
        "# counter's reading for a plain device copy of 256 MiB (read 256 MiB, write 256 MiB).",
        "# O and down share one kernel instance: launches alternate O, down within a layer.",
        "# Defaults of the run: weights read non-temporally; the only L2 read-ahead is the norm before a",
        "# layer loading that layer's QKV weights (~5.2 MB), whose fetches count against the norm launch",
        "# (resnorm, not listed), not the QKV GEMM that uses them.",
        f"# fetch command: {cmd_fetch}",
        f"# write command: {cmd_write}",
        f"# summary: python bench.py --traffic-from <fetch dir> <write dir>",
        f"copy_fetch_kib: {out['FETCH_SIZE']['copy_kib']:.1f}",
        f"copy_write_kib: {out['WRITE_SIZE']['copy_kib']:.1f}",
        f"fetch_scale: {out['FETCH_SIZE']['scale']:.4f}",
        f"write_scale: {out['WRITE_SIZE']['scale']:.4f}",
    ]
    for fam in TRAFFIC_KERNELS:
        fk, n = out["FETCH_SIZE"]["fam"][fam]
        wk, _ = out["WRITE_SIZE"]["fam"][fam]
        fb, wb = fk * out["FETCH_SIZE"]["scale"] * 1024.0, wk * out["WRITE_SIZE"]["scale"] * 1024.0
        lines += [f"dispatches.{fam}: {n}", f"fetch_kib_mean.{fam}: {fk:.1f}", f"write_kib_mean.{fam}: {wk:.1f}",
                  f"traffic_bytes_per_launch.{fam}: {fb + wb:.0f}"]
    lines.append(f"source_sha256_16: {kernel_source_hash()}")
    with open(TRAFFIC_SUMMARY, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


WAVES_SUMMARY = os.path.join(ROOT, "profiles", "layer_kernels_lingbot_b1_wave_states.txt")
WAVE_COUNTERS = ("SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_SCA",
                 "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_WAVES", "GRBM_GUI_ACTIVE")


def waits_from(pmc_dir, cmd):
    """Summary of where the waves of each batch-1 layer kernel family spend
    their time (bench.py --counter-run under rocprofv3 --pmc <WAVE_COUNTERS>):
    the share of wave-resident cycles spent waiting (on memory, barriers or
    dependencies: SQ_WAIT_ANY), waiting to issue (SQ_WAIT_INST_ANY), and
    executing instructions, with the VALU (MFMA included), LDS and scalar
    parts of the latter;
    the wave counters are quad-cycles summed over the shader engines, so
    their ratios need no scaling. Also the mean resident waves per CU while
    the kernel ran (wave cycles over GRBM_GUI_ACTIVE / 8, per 256 CUs)."""
    rows = _counter_rows(pmc_dir)
    res = {}
    for fam, (kname, which, per_layer) in TRAFFIC_KERNELS.items():
        v = {}
        for c in WAVE_COUNTERS:
            vals = _per_dispatch(rows, c, lambda k, kname=kname: kname in k)[which::per_layer]
            if not vals:
                raise SystemExit(f"{c}: no dispatches of {kname}")
            v[c] = (float(np.mean(vals)), len(vals))
        res[fam] = v
    lines = [
        "# Wave states per launch of each kernel family of one expert layer, LingBot-shaped batch-1",
        "# workload (M = 50 rows): shares of the waves' resident cycles (all SQ wave counters are",
        "# quad-cycles summed over the shader engines). wait = SQ_WAIT_ANY (waiting on memory, barriers",
        "# or dependencies), issue_wait = SQ_WAIT_INST_ANY, active = SQ_ACTIVE_INST_ANY with its VALU",
        "# (MFMA included), LDS and scalar (SQ_ACTIVE_INST_SCA) parts; waves_per_cu = SQ_WAVE_CYCLES x 4",
        "# / (GRBM_GUI_ACTIVE / 8) / 256.",
        "# Launches that read weights ahead into L2 (the norms' QKV read-ahead by default) include",
        "# those read-ahead workgroups (their waves wait on loads).",
        "# O and down share one kernel instance: launches alternate O, down within a layer.",
        f"# command: {cmd}",
        "# summary: python bench.py --waits-from <pmc dir>",
        "# family | dispatches | waves | wait | issue_wait | active | active_valu | active_lds | active_scalar | waves_per_cu",
    ]
    for fam, v in res.items():
        wc = max(v["SQ_WAVE_CYCLES"][0], 1.0)
        fr = lambda c: v[c][0] / wc
        kcyc = max(v["GRBM_GUI_ACTIVE"][0] / XCDS, 1.0)
        lines.append(f"{fam} | {v['SQ_WAVE_CYCLES'][1]} | {v['SQ_WAVES'][0]:.0f} | {fr('SQ_WAIT_ANY'):.3f} | "
                     f"{fr('SQ_WAIT_INST_ANY'):.3f} | {fr('SQ_ACTIVE_INST_ANY'):.3f} | {fr('SQ_ACTIVE_INST_VALU'):.3f} | "
                     f"{fr('SQ_ACTIVE_INST_LDS'):.3f} | {fr('SQ_ACTIVE_INST_SCA'):.3f} | "
                     f"{v['SQ_WAVE_CYCLES'][0] * 4 / kcyc / 256:.2f}")
    with open(WAVES_SUMMARY, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


MFMA_SUMMARY = os.path.join(ROOT, "profiles", "gemm_attention_lingbot_b64_mfma_counters.txt")
MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F8", "SQ_VALU_MFMA_BUSY_CYCLES",
                 "SQ_BUSY_CU_CYCLES", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "GRBM_GUI_ACTIVE")
SIMDS = 256 * 4   # MI355X: 256 CUs of 4 SIMDs
XCDS = 8          # GRBM_GUI_ACTIVE comes summed over the XCDs' instances


def _kernel_durations(d):
    """Dispatch id -> duration in ns from a rocprofv3 kernel trace under `d`."""
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        return {}
    out = {}
    with open(files[0]) as fh:
        for r in csv.DictReader(fh):
            try:
                out[int(r["Dispatch_Id"])] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            except (KeyError, ValueError):
                pass
    return out


def mfma_from(pmc_dir, cmd):
    """Summary of the batch-64 MFMA counter run (bench.py --counter-run-b64
    under rocprofv3 --pmc <MFMA_COUNTERS> --kernel-trace): per kernel of the
    layer, the hardware's MFMA operations (x 512 flops each) against the
    algorithmic flops, the MFMA-busy share of all SIMD cycles while the
    kernel ran (busy cycles / (GRBM_GUI_ACTIVE x SIMDs), as rocprofv3's
    MfmaUtil), the CU-busy share, achieved TFLOP/s over the traced duration,
    and LDS bank conflicts per active LDS cycle."""
    rows = _counter_rows(pmc_dir)
    dur = _kernel_durations(pmc_dir)
    per = {}   # dispatch -> {"kernel", counter -> value}
    for r in rows:
        d = int(r["Dispatch_Id"])
        e = per.setdefault(d, {"kernel": r.get("Kernel_Name", "")})
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    fams = {}
    for d, e in sorted(per.items()):
        k = e["kernel"]
        if not any(t in k for t in ("gemm_kernel<", "gemm8_kernel<", "attn_rows_kernel<")):
            continue
        fams.setdefault(k, []).append((d, e))
    lines = [
        "# MFMA counters per kernel of one expert layer, LingBot-shaped batch-64 workload: one-step denoise",
        "# calls in the default mode, two halves of 32 requests (M = 1600 rows each), with bf16 weights",
        "# (gemm_kernel), then E4M3 weights with per-token E4M3 activations (gemm8_kernel).",
        f"# command: {cmd}",
        f"# summary: python bench.py --mfma-from <pmc dir>",
        "# flops_hw = (MOPS_BF16 + MOPS_F8) x 512 per dispatch; cycles = GRBM_GUI_ACTIVE / 8 (the counter",
        f"# comes summed over the 8 XCDs); mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x {SIMDS} SIMDs), as",
        "# rocprofv3's MfmaUtil; cu_busy = SQ_BUSY_CU_CYCLES / (cycles x 256 CUs);",
        "# lds_conflict = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; us from the kernel trace of the same run.",
        "# kernel | dispatches | us | flops_hw (GFLOP) | TFLOP/s | mfma_busy | cu_busy | lds_conflict",
    ]
    for k, lst in fams.items():
        mops = np.mean([e.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + e.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0)
                        for _, e in lst])
        cyc = [max(e.get("GRBM_GUI_ACTIVE", 0.0) / XCDS, 1.0) for _, e in lst]   # GPU cycles of the dispatch
        busy = np.mean([e.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (c * SIMDS) for (_, e), c in zip(lst, cyc)])
        cu = np.mean([e.get("SQ_BUSY_CU_CYCLES", 0.0) / (c * SIMDS / 4) for (_, e), c in zip(lst, cyc)])
        conf = np.mean([e.get("SQ_LDS_BANK_CONFLICT", 0.0) / max(e.get("SQ_LDS_IDX_ACTIVE", 1.0), 1.0)
                        for _, e in lst])
        ds = [dur[d] for d, _ in lst if d in dur]
        us = float(np.mean(ds)) / 1e3 if ds else float("nan")
        fl = mops * 512
        name = k.split("(")[0].replace("void ", "")
        lines.append(f"{name} | {len(lst)} | {us:.2f} | {fl / 1e9:.2f} | {fl / us / 1e6:.1f} | {busy:.3f} | "
                     f"{cu:.3f} | {conf:.3f}")
    with open(MFMA_SUMMARY, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def prefill_work(bcfg):
    """Weight bytes read and GEMM + attention flops of one prefill call (the
    last layer stops after its QKV projection)."""
    H, I, L, P, B = bcfg.hidden, bcfg.intermediate, bcfg.n_layers, bcfg.prefix_len, bcfg.batch
    qd, kvd = bcfg.n_q_heads * bcfg.head_dim, bcfg.n_kv_heads * bcfg.head_dim
    per_layer = H * (qd + 2 * kvd) + H * qd + 2 * H * I + H * I
    params = per_layer * (L - 1) + H * (qd + 2 * kvd)
    rows = (qd + 2 * kvd + H + 2 * I + H) * (L - 1) + qd + 2 * kvd   # output rows (E4M3 scales)
    M = B * P
    attn = (L - 1) * B * bcfg.n_q_heads * 2 * P * (P + 1) * bcfg.head_dim  # causal: P(P+1)/2 pairs, 2 products
    wbytes = params * (1 if bcfg.weight_dtype == "fp8_e4m3" else 2) + (rows * 4 if bcfg.weight_dtype == "fp8_e4m3" else 0)
    return wbytes + 2 * L * H * 4, 2 * M * params + attn


def gpu_backbone_weights(bcfg, seed=0):
    """Random-init backbone weights drawn on the GPU (the values do not change
    the timing): N(0, std^2) linears in bf16 (or per-row E4M3 codes with
    max|row| / 448 scales), 1 + N(0, 0.1^2) norm weights."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(seed)
    H, I = bcfg.hidden, bcfg.intermediate
    qd, kvd = bcfg.n_q_heads * bcfg.head_dim, bcfg.n_kv_heads * bcfg.head_dim
    shapes = {"wq": (qd, H), "wk": (kvd, H), "wv": (kvd, H), "wo": (H, qd), "wg": (I, H), "wu": (I, H),
              "wd": (H, I)}
    W = {k: [] for k in ("n1", "n2", *shapes)}
    for _ in range(bcfg.n_layers):
        for n in ("n1", "n2"):
            W[n].append(1.0 + 0.1 * torch.randn(H, device="cuda", generator=g))
        for n, shp in shapes.items():
            w = bcfg.weight_std * torch.randn(shp, device="cuda", generator=g)
            if bcfg.weight_dtype == "fp8_e4m3":
                sc = (w.abs().amax(dim=1) / 448.0).clamp_min(1e-30)
                W[n].append((w / sc[:, None]).to(torch.float8_e4m3fn).view(torch.uint8))
                W.setdefault("s" + n[1], []).append(sc.float().contiguous())
            else:
                W[n].append(w.to(torch.bfloat16).view(torch.int16))
    return W


def bench_prefill(batches, warmup, steps, weight_dtype="bf16", prefix_len=None):
    import torch
    import synth
    from vla_flow_matching_denoise_amd.prefill import Prefill, backbone_dims_from_config
    base = synth.backbone(2).replace(weight_dtype=weight_dtype)
    if prefix_len:
        base = base.replace(prefix_len=prefix_len)
    W = gpu_backbone_weights(base)
    out = {}
    for b in batches:
        bcfg = base.replace(batch=b)
        pf = Prefill(W, backbone_dims_from_config(bcfg))
        emb = torch.randn((b, bcfg.prefix_len, bcfg.hidden), device="cuda").to(torch.bfloat16).view(torch.int16)
        k, v = pf(emb)                                    # first call captures the graph (untimed)
        for _ in range(warmup):
            pf(emb, k, v)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            pf(emb, k, v)
        torch.cuda.synchronize()
        t = (time.perf_counter() - t0) / steps
        pf.close()
        wbytes, flops = prefill_work(bcfg)
        peak = FP8_PEAK_TFLOPS if weight_dtype == "fp8_e4m3" else BF16_PEAK_TFLOPS
        out[f"b{b}"] = {"ms_per_call": round(t * 1e3, 4), "tokens_per_s": round(b * bcfg.prefix_len / t, 1),
                        "weights_GBps": round(wbytes / t / 1e9, 1),
                        "weights_hbm_frac": round(wbytes / t / 1e9 / HBM_PEAK_GBS, 4),
                        "TFLOPs": round(flops / t / 1e12, 1),
                        "mfma_frac": round(flops / t / 1e12 / peak, 4)}
    del W
    return out


def build_inputs(cfg, seed=0):
    import synth
    from vla_flow_matching_denoise_amd.expert import to_device
    pk, pv = synth.make_prefix(cfg, seed=seed)
    x0 = synth.make_noise(cfg, seed=seed)
    ts = synth.make_schedule(cfg.n_steps, cfg.batch)
    return tuple(to_device(a) for a in (pk, pv, x0, ts)), (pk, pv, x0, ts)


def gpu_inputs(cfg, seed=0):
    """Inputs of the workload's shapes drawn on the GPU (prefix K/V and noise
    N(0, 1), the uniform schedule): for legs whose values do not change the
    timing."""
    import torch
    import synth
    from vla_flow_matching_denoise_amd.expert import to_device
    g = torch.Generator(device="cuda").manual_seed(seed)
    shp = (cfg.batch, cfg.n_layers, cfg.prefix_len, cfg.n_kv_heads, cfg.head_dim)
    pk = torch.randn(shp, device="cuda", generator=g).to(torch.bfloat16).view(torch.int16)
    pv = torch.randn(shp, device="cuda", generator=g).to(torch.bfloat16).view(torch.int16)
    x0 = torch.randn((cfg.batch, cfg.horizon, cfg.action_dim), device="cuda", generator=g)
    return pk, pv, x0, to_device(synth.make_schedule(cfg.n_steps, cfg.batch))


def gpu_expert_weights(cfg, seed=0):
    """Random-init bf16 expert weights of the workload's shapes drawn on the GPU
    (N(0, std^2) linears and biases; the values do not change the timing)."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(seed)
    H, A, E, L, I = cfg.hidden, cfg.action_dim, cfg.time_emb_dim, cfg.n_layers, cfg.intermediate
    qd, kvd = cfg.n_q_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim

    def w(*shape):
        return (cfg.weight_std * torch.randn(shape, device="cuda", generator=g)).to(torch.bfloat16).view(torch.int16)

    def b(n):
        return cfg.weight_std * torch.randn(n, device="cuda", generator=g)

    W = {"in_w": w(H, A), "in_b": b(H), "out_w": w(A, H), "out_b": b(A), "t1_w": w(H, E), "t1_b": b(H),
         "t2_w": w(H, H), "t2_b": b(H), "modf_w": w(2 * H, H), "modf_b": b(2 * H),
         "mod_w": [w(6 * H, H) for _ in range(L)], "mod_b": [b(6 * H) for _ in range(L)]}
    shapes = {"wq": (qd, H), "wk": (kvd, H), "wv": (kvd, H), "wo": (H, qd), "wg": (I, H), "wu": (I, H),
              "wd": (H, I)}
    for n, shp in shapes.items():
        W[n] = [w(*shp) for _ in range(L)]
    return W


def leg(ex, cfg, dev_in, warmup, steps, bound="hbm", peak=None):
    """Times `steps` calls of one workload; rates and the call roofline."""
    wall, per_call, _ = time_calls(ex, dev_in, cfg.n_steps, warmup, steps)
    t = wall / steps
    by, fl = call_work(cfg)
    if bound == "hbm":
        ach, pk, unit, work = by / t / 1e9, HBM_PEAK_GBS, "GB/s", {"algorithmic_bytes": int(by)}
    else:
        ach, pk, unit, work = fl / t / 1e12, peak or BF16_PEAK_TFLOPS, "TFLOP/s", {"algorithmic_tflop": round(fl / 1e12, 3)}
    return {"ms_per_call": round(t * 1e3, 4), "steps_per_s": round(cfg.n_steps / t, 3),
            "chunks_per_s": round(cfg.batch / t, 3),
            "p50_ms": round(float(np.percentile(per_call, 50)), 4),
            "p95_ms": round(float(np.percentile(per_call, 95)), 4),
            "call_roofline": {"bound": bound, **work, "achieved": round(ach, 1), "peak": pk, "unit": unit,
                              "frac": round(ach / pk, 4)}}


# ------------------------------- CPU baseline --------------------------------

def cpu_model() -> str:
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    return "unknown"


def random_decoded_weights(cfg, dtype=np.float32, seed=0):
    """Float weights of the workload's shapes, N(0, std^2), in the layout the
    oracle takes after decoding (for timing a workload whose encoded weights
    are not on the host; the values do not change the CPU time)."""
    r = np.random.default_rng([seed, 7, cfg.model_tag])
    H, A, E, L, I = cfg.hidden, cfg.action_dim, cfg.time_emb_dim, cfg.n_layers, cfg.intermediate
    qd, kvd = cfg.n_q_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim

    def g(*shape):
        return (r.standard_normal(shape, dtype=np.float32) * np.float32(cfg.weight_std)).astype(dtype)

    W = {"in_w": g(H, A), "in_b": g(H), "out_w": g(A, H), "out_b": g(A), "t1_w": g(H, E), "t1_b": g(H),
         "t2_w": g(H, H), "t2_b": g(H), "modf_w": g(2 * H, H), "modf_b": g(2 * H),
         "mod_w": [g(6 * H, H) for _ in range(L)], "mod_b": [g(6 * H) for _ in range(L)]}
    shapes = {"wq": (qd, H), "wk": (kvd, H), "wv": (kvd, H), "wo": (H, qd), "wg": (I, H), "wu": (I, H),
              "wd": (H, I)}
    for n, shp in shapes.items():
        W[n] = [g(*shp) for _ in range(L)]
    return W


def _oracle_steps_per_s(W, cfg, n_steps, dtype, min_s=2.0):
    """One request of `cfg` through the oracle: one untimed call, then calls
    of `n_steps` Euler steps until at least `min_s`; returns (Euler steps per
    second of one request, seconds, calls)."""
    import oracle
    import synth
    d = oracle.ExpertDims.from_config(cfg)
    r = np.random.default_rng(3)
    pk = r.standard_normal((1, cfg.n_layers, cfg.prefix_len, cfg.n_kv_heads, cfg.head_dim)).astype(dtype)
    pv = r.standard_normal(pk.shape).astype(dtype)
    x0 = r.standard_normal((1, cfg.horizon, cfg.action_dim)).astype(np.float32)
    ts = synth.make_schedule(n_steps, 1)
    oracle.denoise(W, d, pk, pv, x0, ts)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.denoise(W, d, pk, pv, x0, ts)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_s:
            return reps * n_steps / dt, dt, reps


def cpu_baselines(raw2, raw4):
    """The oracle as it stands on the host CPU: its fp32 twin (the same code on
    float32 weights and inputs) on a bounded sample of every workload (one
    request; whole 10-step calls of the tiny workload, single Euler steps of
    the 36-layer ones, converted to the workload's steps/s and chunks/s), with
    the BLAS threads set to every core of the process's affinity mask, and on
    one thread for the tiny and LingBot batch-1 workloads; the fp64 oracle once
    on the LingBot workload."""
    import oracle
    import synth
    from threadpoolctl import threadpool_limits
    cores = len(os.sched_getaffinity(0))
    model = cpu_model()
    t_start = time.perf_counter()
    per, one = {}, {}

    def rates(cfg, sps_one_request):
        # requests are independent: a batch step of B requests costs B single-request
        # steps, and a request finishes after the workload's N steps
        return {"steps_per_s": round(sps_one_request / cfg.batch, 4),
                "chunks_per_s": round(sps_one_request / cfg.n_steps, 5)}

    c1 = synth.config(1)
    W1 = oracle.decode_weights(synth.make_weights(c1), np.float32)
    c2 = synth.config(2)
    W2 = oracle.decode_weights(raw2, np.float32)
    with threadpool_limits(cores):
        sps, dt, n = _oracle_steps_per_s(W1, c1, c1.n_steps, np.float32)
        per["tiny_b1"] = {**rates(c1, sps), "sample": f"{n} call(s) of 10 steps, {dt:.2f} s"}
        sps2, dt, n = _oracle_steps_per_s(W2, c2, 1, np.float32)
        per["lingbot_b1"] = {**rates(c2, sps2), "sample": f"{n} Euler step(s) of 36 layers, {dt:.2f} s"}
        c5 = synth.config(5)
        per["lingbot_b64"] = {**rates(c5, sps2), "sample": "one request's Euler step (as lingbot_b1) x 64 requests"}
        c4 = synth.config(4)
        W4 = oracle.decode_weights(raw4, np.float32)
        sps4, dt, n = _oracle_steps_per_s(W4, c4, 1, np.float32)
        per["lingbot_fp8_b1"] = {**rates(c4, sps4),
                                 "sample": f"{n} Euler step(s), E4M3 weights decoded to fp32, {dt:.2f} s"}
        del W4
        c3 = synth.config(3)
        W3 = random_decoded_weights(c3, np.float32)
        sps3, dt, n = _oracle_steps_per_s(W3, c3, 1, np.float32)
        per["v2_b1"] = {**rates(c3, sps3), "sample": f"{n} Euler step(s) of 36 layers (hidden 1536, prefix 512), "
                                                     f"{dt:.2f} s"}
        del W3
    with threadpool_limits(1):
        sps, dt, n = _oracle_steps_per_s(W1, c1, c1.n_steps, np.float32)
        one["tiny_b1"] = {**rates(c1, sps), "sample": f"{n} call(s) of 10 steps, {dt:.2f} s"}
        sps, dt, n = _oracle_steps_per_s(W2, c2, 1, np.float32)
        one["lingbot_b1"] = {**rates(c2, sps), "sample": f"{n} Euler step(s), {dt:.2f} s"}
    del W2
    W64 = oracle.decode_weights(raw2, np.float64)
    with threadpool_limits(cores):
        sps64, dt, n = _oracle_steps_per_s(W64, c2, 1, np.float64)
    del W64
    return {"value": per["lingbot_b1"]["steps_per_s"], "unit": "denoise_steps/s", "cores": cores,
            "kind": "oracle",
            "sample": "fp32 twin of the oracle, one request of the LingBot batch-1 workload, "
                      + per["lingbot_b1"]["sample"],
            "cpu_model": model, "blas_threads": cores,
            "per_workload": per, "one_thread": one,
            "fp64_lingbot_b1": {"steps_per_s": round(sps64, 4), "sample": f"{n} Euler step(s), {dt:.2f} s"},
            "total_s": round(time.perf_counter() - t_start, 1)}


# ------------------------------- batch-64 counters ---------------------------

def counter_run_b64(iters):
    """Workload of the batch-64 MFMA counter runs: two one-step denoise calls
    of the batch-64 workload in the default mode, where the batch runs as two
    halves of 32 requests (M = 1600 rows each), so each layer GEMM and the row
    attention launch 2 x 2 x 36 times; first with bf16 weights, then with
    E4M3 weights and per-token E4M3 activations.  (``iters`` is unused: the
    calls fix the launch counts.)"""
    import torch
    import synth
    from vla_flow_matching_denoise_amd.expert import Expert, dims_from_config
    torch.cuda.set_device(0)
    for wd in ("bf16", "fp8_e4m3"):
        cfg = synth.config(5).replace(weight_dtype=wd, n_steps=1)
        ex = Expert(synth.make_weights(cfg, seed=0), dims_from_config(cfg))
        dev_in = gpu_inputs(cfg)
        for _ in range(2):
            ex.denoise(*dev_in, cfg.n_steps)
        torch.cuda.synchronize()
        ex.close()
        log(f"[bench] batch-64 counter run ({wd}) done")


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30, help="timed denoise calls")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--profile-iters", type=int, default=144)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-batch64", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the V2, E4M3, MXFP4 and persistent legs")
    ap.add_argument("--prefill-only", action="store_true", help="time only the prefill leg (for kernel profiles)")
    ap.add_argument("--counter-run", action="store_true",
                    help="run only the workload of the batch-1 rocprofv3 counter runs (copy calibration + layers)")
    ap.add_argument("--counter-run-b64", action="store_true",
                    help="run only the workload of the batch-64 MFMA counter runs")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the traffic summary from two rocprofv3 --pmc output folders")
    ap.add_argument("--traffic-cmds", nargs=2, metavar=("FETCH_CMD", "WRITE_CMD"), default=("?", "?"))
    ap.add_argument("--mfma-from", metavar="PMC_DIR", help="write the batch-64 MFMA counter summary")
    ap.add_argument("--mfma-cmd", default="?")
    ap.add_argument("--waits-from", metavar="PMC_DIR", help="write the batch-1 wave-state counter summary")
    ap.add_argument("--waits-cmd", default="?")
    args = ap.parse_args()
    if args.traffic_from:
        traffic_from(*args.traffic_from, *args.traffic_cmds)
        return
    if args.mfma_from:
        mfma_from(args.mfma_from, args.mfma_cmd)
        return
    if args.waits_from:
        waits_from(args.waits_from, args.waits_cmd)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}). Each GPU would run an independent "
              f"replica of the loop on its own requests.", file=sys.stderr)
        sys.exit(2)

    if args.counter_run:
        counter_run(72)
        return
    if args.counter_run_b64:
        counter_run_b64(36)
        return

    import torch
    import synth
    from vla_flow_matching_denoise_amd import binding as B
    from vla_flow_matching_denoise_amd.expert import Expert, dims_from_config
    torch.cuda.set_device(0)
    if args.prefill_only:
        print(json.dumps({"prefill": bench_prefill((1, 16), args.warmup, args.steps),
                          "prefill_e4m3": bench_prefill((1, 16), args.warmup, args.steps, "fp8_e4m3")}), flush=True)
        return

    cfg = synth.config(2)
    log(f"[bench] generating weights for {cfg.name}")
    raw = synth.make_weights(cfg, seed=0)
    ex = Expert(raw, dims_from_config(cfg))
    dev_in, host_in = build_inputs(cfg)
    log(f"[bench] timing {args.steps} calls of {cfg.n_steps} Euler steps (warmup {args.warmup})")
    head = leg(ex, cfg, dev_in, args.warmup, args.steps)
    t_call = head["ms_per_call"] / 1e3
    kr = kernel_rooflines(ex, cfg, args.profile_iters)
    dom, roof, worst = dominant(kr, "hbm")
    roof["traffic"] = recorded_traffic(dom)
    worst["traffic"] = recorded_traffic(worst["kernel"])
    if ex.get_option(B.VLA_OPT_L2_PREFETCH) & 3:  # the attention launch reads O / gate_up weights ahead
        for r in (roof, worst):
            if r["kernel"] == "gqa_attention":
                r["traffic_note"] = ("includes the O and gate_up weights that the launch's idle workgroups "
                                     "load into L2 for the next GEMMs")
    persistent = None
    if not args.no_extra:
        # the opt-in persistent single-launch path on the same workload
        ex.set_option(B.VLA_OPT_PERSISTENT, 1)
        if ex.persistent_active:
            persistent = leg(ex, cfg, dev_in, args.warmup, args.steps)
            persistent["status"] = ex.get_option(B.VLA_OPT_PERSISTENT_STATUS)
        ex.set_option(B.VLA_OPT_PERSISTENT, 0)
    ex.close()
    cr = head.pop("call_roofline")
    result = {
        "metric": METRIC,
        "value": round(cfg.n_steps * cfg.batch / t_call, 3),
        "unit": "denoise_steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_call * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02^2) weights, N(0,1) prefix KV and noise)",
        "config": {"workload": "lingbot_36L_h1024_gqa16x2x128_swiglu4096_prefix256_chunk50x75_euler10_b1",
                   "batch": cfg.batch, "euler_steps": cfg.n_steps, "chunk": [cfg.horizon, cfg.action_dim],
                   "prefix_len": cfg.prefix_len},
        "chunks_per_s": head["chunks_per_s"],
        "p50_ms": head["p50_ms"],
        "p95_ms": head["p95_ms"],
        "call_roofline": {**cr, "target_frac": CALL_TARGET["hbm"],
                          "target_steps_per_s": round(CALL_TARGET["hbm"] * cfg.n_steps / (cr["algorithmic_bytes"]
                                                      / (HBM_PEAK_GBS * 1e9)), 1)},
        "roofline": roof,
        "roofline_worst": worst,
        "kernels": {k: {"us": round(v["us"], 3), "GBps": round(v["GBps"], 1), "TFLOPs": round(v["TFLOPs"], 2),
                        "hbm_frac": round(v["GBps"] / HBM_PEAK_GBS, 4)} for k, v in kr.items()},
        "persistent_b1": persistent,
    }

    if not args.no_extra:
        # V2-shaped loop: hidden 1536, SwiGLU 6144, prefix 512, chunk 50x55, 50 Euler steps
        cfg3 = synth.config(3)
        log("[bench] V2-shaped workload (weights drawn on the GPU)")
        ex3 = Expert(gpu_expert_weights(cfg3), dims_from_config(cfg3))
        torch.cuda.synchronize()
        result["v2_b1"] = {"workload": "v2_36L_h1536_gqa16x2x128_swiglu6144_prefix512_chunk50x55_euler50_b1",
                           **leg(ex3, cfg3, gpu_inputs(cfg3), 2, max(5, args.steps // 3))}
        ex3.close()
        torch.cuda.empty_cache()
        # E4M3 weight tier: per-row E4M3 block linears, bf16 activations, 25 steps
        cfg4 = synth.config(4)
        log("[bench] E4M3-weight batch-1 workload")
        raw4 = synth.make_weights(cfg4, seed=0)
        ex4 = Expert(raw4, dims_from_config(cfg4))
        dev4, _ = build_inputs(cfg4)
        result["fp8_b1"] = {"workload": "lingbot_36L_h1024_e4m3_weights_bf16_activations_chunk50x75_euler25_b1",
                            "dtype": "e4m3 weights, bf16 activations, f32 accumulation",
                            **leg(ex4, cfg4, dev4, args.warmup, args.steps)}
        kr4 = kernel_rooflines(ex4, cfg4, args.profile_iters)
        result["fp8_b1"]["kernels"] = {k: {"us": round(v["us"], 3), "GBps": round(v["GBps"], 1)} for k, v in kr4.items()}
        ex4.close()
        # the same batch-1 workload with E4M3 block linears and MXFP4 gate/up
        cfgm = synth.config(4).replace(weight_dtype="fp8_mxfp4gu", n_steps=cfg.n_steps)
        log("[bench] batch-1 E4M3 + MXFP4 gate_up workload")
        exm = Expert(synth.make_weights(cfgm, seed=0), dims_from_config(cfgm))
        devm, _ = build_inputs(cfgm)
        lm = leg(exm, cfgm, devm, args.warmup, args.steps)
        krm = kernel_rooflines(exm, cfgm, args.profile_iters)
        exm.close()
        lm.pop("call_roofline")
        result["b1_e4m3_mxfp4_gate_up"] = {
            "workload": "lingbot_36L_h1024_chunk50x75_euler10_b1_e4m3_mxfp4_gate_up", **lm,
            "gate_up": {"us": round(krm["gate_up_swiglu_gemm"]["us"], 3),
                        "algorithmic_bytes": int(krm["gate_up_swiglu_gemm"]["bytes"]),
                        "GBps": round(krm["gate_up_swiglu_gemm"]["GBps"], 1),
                        "frac": round(krm["gate_up_swiglu_gemm"]["GBps"] / HBM_PEAK_GBS, 4)},
            "e4m3_gate_up_us": round(kr4["gate_up_swiglu_gemm"]["us"], 3)}
    else:
        raw4 = None

    if not args.no_batch64:
        cfg5 = synth.config(5)
        log("[bench] batch-64 workload")
        ex5 = Expert(raw, dims_from_config(cfg5))
        dev5, _ = build_inputs(cfg5)
        n5 = max(3, args.steps // 5)
        l5 = leg(ex5, cfg5, dev5, 2, n5, bound="mfma")
        parts5 = ex5.get_option(B.VLA_OPT_SPLIT_BATCH)
        kr5 = kernel_rooflines(ex5, cfg5, 36)
        _, roof5, worst5 = dominant(kr5, "mfma")
        ex5.close()
        kernels_note = ("each kernel family timed alone (HIP events, 36 launches) on all 3200 rows in one launch; "
                        "the call runs the batch as %d concurrent parts (0: one batch)")
        result["batch64"] = {
            "workload": "lingbot_36L_h1024_chunk50x75_euler10_b64", **l5, "parts": parts5,
            "target_frac": CALL_TARGET["mfma"], "roofline": roof5, "roofline_worst": worst5,
            "kernels_note": kernels_note % parts5,
            "kernels": {k: {"us": round(v["us"], 2), "TFLOPs": round(v["TFLOPs"], 1),
                            "mfma_frac": round(v["TFLOPs"] / BF16_PEAK_TFLOPS, 4)} for k, v in kr5.items()},
        }
        # the same batch with E4M3 block weights: per-token E4M3 activations and
        # the FP8 MFMA (its own tier; the bf16 figures above are the metric's)
        cfg8 = synth.config(4).replace(batch=cfg5.batch, n_steps=cfg5.n_steps)
        log("[bench] batch-64 E4M3 workload")
        ex8 = Expert(raw4 if raw4 is not None else synth.make_weights(cfg8, seed=0), dims_from_config(cfg8))
        dev8, _ = build_inputs(cfg8)
        l8 = leg(ex8, cfg8, dev8, 2, n5, bound="mfma", peak=FP8_PEAK_TFLOPS)
        parts8 = ex8.get_option(B.VLA_OPT_SPLIT_BATCH)
        kr8 = kernel_rooflines(ex8, cfg8, 36)
        _, roof8, _ = dominant(kr8, "mfma", FP8_PEAK_TFLOPS)
        ex8.close()
        result["batch64_e4m3"] = {
            "workload": "lingbot_36L_h1024_chunk50x75_euler10_b64_e4m3_weights_per_token_e4m3_activations",
            "dtype": "e4m3 x e4m3 -> f32", **l8, "parts": parts8, "roofline": roof8,
            "kernels_note": kernels_note % parts8,
            "kernels": {k: {"us": round(v["us"], 2), "TFLOPs": round(v["TFLOPs"], 1)} for k, v in kr8.items()},
        }

    if not args.no_prefill:
        log("[bench] prefix K/V construction (36-layer backbone prefill)")
        result["prefill"] = {
            "workload": "lingbot_backbone_36L_h2048_gqa16x2x128_swiglu11008_prefix256",
            "unit": "prefix tokens/s", "dtype": "bf16",
            "data": "synthetic (N(0,0.02^2) bf16 weights drawn on the GPU, N(0,1) embeddings)",
            **bench_prefill((1, 16), 3, max(5, args.steps // 3)),
            # the pages' prefix runs FP8: E4M3 weights and per-token E4M3 inputs
            # (mfma_frac against the 5 PFLOP/s FP8 peak)
            "e4m3": bench_prefill((1, 16), 3, max(5, args.steps // 3), "fp8_e4m3"),
            # the V2-shaped loop's prefix length
            "p512": bench_prefill((1,), 3, max(5, args.steps // 3), prefix_len=512),
        }

    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline")
        if raw4 is None:
            raw4 = synth.make_weights(synth.config(4), seed=0)
        result["cpu_baseline"] = cpu_baselines(raw, raw4)

    print(json.dumps(result), flush=True)
    try:  # the line is out; a problem found here is reported, never raised
        for problem in check_line(result):
            log(f"[bench] report line: {problem}")
    except Exception as e:  # noqa: BLE001
        log(f"[bench] report line check failed: {e!r}")


def check_line(d) -> list:
    """Problems with a bench report line (an empty list when it is well formed):
    the keys and types the report contract asks for, a fraction that is not
    achieved / peak, a value that does not follow from the time per step."""
    problems = []
    want = {"metric": str, "value": (int, float), "unit": str, "n_gpus": int, "steps": int, "warmup": int,
            "ms_per_step": (int, float), "higher_is_better": bool, "scaling": str, "dtype": str, "data": str,
            "config": dict, "roofline": dict, "cpu_baseline": dict}
    for k, t in want.items():
        if k not in d:
            problems.append(f"missing {k}")
        elif not isinstance(d[k], t) or (t == int and isinstance(d[k], bool)):
            problems.append(f"{k} has type {type(d[k]).__name__}")
    if "vs_baseline" not in d:
        problems.append("missing vs_baseline")
    if problems:
        return problems
    if d["scaling"] not in ("weak", "strong"):
        problems.append(f"scaling {d['scaling']!r}")
    if not isinstance(d["config"].get("workload"), str):
        problems.append("config has no workload name")
    roof = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac"):
        if k not in roof:
            problems.append(f"roofline misses {k}")
    if "traffic" not in roof:
        problems.append("roofline misses traffic (null when unmeasured)")
    if all(k in roof for k in ("achieved", "peak", "frac")) and roof["peak"]:
        if abs(roof["achieved"] / roof["peak"] - roof["frac"]) > 1e-3:
            problems.append("roofline frac is not achieved / peak")
    if roof.get("bound") not in ("hbm", "mfma", "alu"):
        problems.append(f"roofline bound {roof.get('bound')!r}")
    cpu = d["cpu_baseline"]
    for k in ("value", "unit", "cores", "kind", "sample"):
        if k not in cpu:
            problems.append(f"cpu_baseline misses {k}")
    if d["ms_per_step"] > 0 and d["n_gpus"] == 1:
        steps_per_call = d["config"].get("euler_steps", 1) * d["config"].get("batch", 1)
        if abs(steps_per_call / (d["ms_per_step"] / 1e3) - d["value"]) > 1e-2 * d["value"]:
            problems.append("value does not follow from ms_per_step")
    return problems


if __name__ == "__main__":
    main()

"""Benchmark of the MSA forward path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--mode literal|structured]

A prefill step is one pass of the whole prefill path over the 128K workload
(N = 131072, H_q = 64, H_kv = 8, d_h = 128, d_idx = 64, B_k = 128, k = 16):
msa_index_topk (index scoring, causal max-pool, Top-k) then msa_sparse_attn_fwd
(inverse index, KV-outer attention, LSE combine).  A decode step is msa_decode for
64 sequences with 128K-token caches.  Inputs are synthetic (seeded, resident in
HBM before timing starts); the headline figures use one input mode and the other
mode is reported beside them.  One JSON line is printed, with the roofline of the
dominant kernel (KV-outer phase 1, timed by events the library records around it)
and the CPU oracle timed on a sample of query rows.

FLOP accounting (exact, from the work the method must do): index
d_idx * H_kv * N (N + 1) (every causal (query, key) pair per group, 2 FLOP per
multiply-add) plus main 4 * d_h * H_q * (attended (query, key) pairs); the
nominal count of Eq. 12 (MSA paper review, section 3) is reported beside it.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time


def flops_gqa_eq12(N: int, H_q: int, d_h: int) -> int:
    """Dense causal GQA attention FLOPs as counted by Eq. 12 (MSA paper review, section 3)."""
    return 2 * H_q * d_h * N * N


def flops_msa_eq12(N: int, H_q: int, H_kv: int, d_h: int, d_idx: int, B_k: int, k: int) -> int:
    """MSA FLOPs as counted by Eq. 12: index branch H_kv d_idx N^2 + main branch 4 H_q d_h N k B_k."""
    return H_kv * d_idx * N * N + 4 * H_q * d_h * N * k * B_k


def flops_index_exact(N: int, H_kv: int, d_idx: int) -> int:
    """2 FLOP x d_idx per causal (query, key) pair and group: d_idx * H_kv * N (N + 1)."""
    return d_idx * H_kv * N * (N + 1)


def attended_pairs(block_idx, B_k: int, G: int) -> int:
    """Sum over (query, head) of the tokens attended: sum over chosen blocks of |block ∩ [0, i]|."""
    import torch
    N = block_idx.shape[0]
    i = torch.arange(N, device=block_idx.device, dtype=torch.int64).view(N, 1, 1)
    b = block_idx.to(torch.int64)
    valid = (b >= 0) & (b <= i // B_k)
    n = torch.clamp(torch.minimum(i - b * B_k + 1, torch.full_like(b, B_k)), min=0)
    return int((n * valid).sum().item()) * G


PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

ROOT = os.path.dirname(os.path.abspath(__file__))


def kernel_rooflines(pre, peaks):
    """Roofline of each timed kernel of the prefill step against the vendor peak and,
    when measured, against this GPU's own ceiling: the index kernel on MFMA (its exact
    FLOP count), KV-outer phase 1 and the combine on HBM (their algorithmic bytes)."""
    out = {}
    ms_idx = pre["ms_index_topk"]
    tf = pre["flop_index"] / (ms_idx / 1e3) / 1e12
    out["index_topk_kernel"] = {"bound": "mfma", "achieved": round(tf, 1), "unit": "TFLOP/s",
                                "peak": PEAK_BF16_TFLOPS, "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
    gb1 = pre["phase1_algorithmic_bytes"] / (pre["ms_kvouter_phase1"] / 1e3) / 1e9
    out["attn_kvouter_kernel"] = {"bound": "hbm", "achieved": round(gb1, 1), "unit": "GB/s", "peak": PEAK_HBM_GBS,
                                  "frac": round(gb1 / PEAK_HBM_GBS, 4)}
    gbc = pre["combine_GB_s"]
    out["combine_kernel"] = {"bound": "hbm", "achieved": gbc, "unit": "GB/s", "peak": PEAK_HBM_GBS,
                             "frac": round(gbc / PEAK_HBM_GBS, 4)}
    if peaks:
        out["index_topk_kernel"]["frac_of_measured"] = round(tf / peaks["mfma_bf16_tflops"], 4)
        out["attn_kvouter_kernel"]["frac_of_measured_copy"] = round(gb1 / peaks["hbm_copy_GB_s"], 4)
        out["combine_kernel"]["frac_of_measured_read"] = round(gbc / peaks["hbm_read_GB_s"], 4)
    return out
# Sources the KV-outer kernel is compiled from: a recorded traffic figure holds only
# while their hash is unchanged.
# What decides the KV-outer kernel's memory traffic: its own code (the phase-1 part
# of sparse_attn.hip), the workspace layout and the launches up to it, and the shared
# device helpers.  The counter summary is reused only while these are unchanged.
ATTN_FILE = "block_sparse_gqa_index_amd/csrc/sparse_attn.hip"
ATTN_HELPERS = ("block_sparse_gqa_index_amd/csrc/msa_device.h",)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_kvouter_kernel_128k_traffic.txt")


def _attn_kernel_text() -> str:
    src = open(os.path.join(ROOT, ATTN_FILE)).read()
    p1 = src.index("// " + "-" * 69 + " phase 1")
    p2 = src.index("// " + "-" * 69 + " phase 2")
    lay = src.index("AttnWorkspace attn_workspace_layout(")
    launch = src.index("hipError_t launch_sparse_attn_window(")
    p1_end = src.index("hipEventRecord(events[2]", launch)  # the launcher up to phase 1's launch
    parts = [src[p1:p2], src[lay:src.index("\n}\n", lay)], src[launch:p1_end]]
    for f in ATTN_HELPERS:
        parts.append(open(os.path.join(ROOT, f)).read())
    return "\0".join(parts)


def attn_source_hash() -> str:
    import hashlib
    return hashlib.sha256(_attn_kernel_text().encode()).hexdigest()


def recorded_traffic(mode: str):
    """HBM bytes per launch of the KV-outer kernel from the committed counter summary,
    or None when the kernel's sources changed since the counters were taken."""
    try:
        rec = {}
        with open(TRAFFIC_FILE) as fh:
            for line in fh:
                if ":" in line and not line.startswith("#"):
                    key, val = line.split(":", 1)
                    rec[key.strip()] = val.strip()
        if rec.get("source_sha256") != attn_source_hash() or rec.get("mode") != mode:
            return None
        return int(float(rec["hbm_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


def write_traffic_summary(fetch_csv: str, write_csv: str, mode: str, command: str) -> str:
    """Turn two rocprofv3 counter passes (FETCH_SIZE, WRITE_SIZE; KiB per dispatch) into
    HBM bytes per launch of the KV-outer kernel, each counter scaled by what it reads
    for the calibration copies of COPY_BYTES made at the start of the profiled run."""
    import csv
    per = {}
    for path, counter in ((fetch_csv, "FETCH_SIZE"), (write_csv, "WRITE_SIZE")):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]][:COPY_REPS]
        attn = [float(r["Counter_Value"]) for r in rows if "attn_kvouter_kernel" in r["Kernel_Name"]]
        if len(copies) < COPY_REPS or not attn:
            raise SystemExit(f"{path}: calibration copies or KV-outer dispatches missing")
        kib_copy = sum(copies) / len(copies)
        factor = COPY_BYTES / (kib_copy * 1024.0)
        kib = sum(attn) / len(attn)
        per[counter] = (kib, kib_copy, factor, kib * 1024.0 * factor, len(attn))
    total = per["FETCH_SIZE"][3] + per["WRITE_SIZE"][3]
    lines = [
        "# HBM traffic of attn_kvouter_kernel<8> (KV-outer phase 1), 128K prefill",
        "# (N=131072 H_q=64 H_kv=8 d_h=128 B_k=128 k=16), one launch per step.",
        "# Counters in KiB per dispatch; each scaled by the ratio of the true size of a",
        f"# plain device copy ({COPY_BYTES} bytes read and written) to what the counter reads for it.",
        f"# command: {command}",
        f"kernel: attn_kvouter_kernel",
        f"mode: {mode}",
        f"source_sha256: {attn_source_hash()}",
    ]
    for c, (kib, kib_copy, factor, b, n) in per.items():
        lines += [f"{c.lower()}_kib_per_dispatch: {kib:.1f}", f"{c.lower()}_dispatches: {n}",
                  f"{c.lower()}_copy_kib: {kib_copy:.1f}", f"{c.lower()}_copy_factor: {factor:.4f}",
                  f"{c.lower()}_bytes_per_launch: {b:.0f}"]
    lines.append(f"hbm_bytes_per_launch: {total:.0f}")
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return TRAFFIC_FILE


STATS_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                          "prefill_128k_decode_128k_kernel_stats.txt")


def write_stats_summary(stats_csv: str, log_path: str, command: str) -> str:
    """Short text form of a rocprofv3 ``--kernel-trace --stats`` run of this script: the
    library's kernels from ``*_kernel_stats.csv`` and the HIP-event phase times the same
    run printed in its JSON line (``log_path``)."""
    import csv
    import re
    rows = []
    for r in csv.DictReader(open(stats_csv)):
        name = r["Name"].replace("(anonymous namespace)::", "")
        m = re.search(r"msa::([A-Za-z0-9_]+(?:<[^()]*?>)?)\(", name)
        if m:
            rows.append((m.group(1), int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                         float(r["MaxNs"]) / 1e3, float(r["TotalDurationNs"])))
    rows.sort(key=lambda x: -x[5])
    res = None
    for line in open(log_path):
        if line.startswith("{") and '"metric"' in line:
            res = json.loads(line)
    if res is None:
        raise SystemExit(f"{log_path}: no result line")
    pre, dec = res["prefill"], res.get("decode")
    lines = [
        "# rocprofv3 kernel statistics: " + res["config"]["workload"] + f" ({res['config']['mode']} inputs)",
        "# and " + (dec["workload"] if dec else "no decode") + "; MI355X, one GPU.",
        f"# command: {command}",
        f"# {res['warmup']} warmup + {res['steps']} timed prefill steps; rows of the stats CSV for the",
        "# library's kernels (times in microseconds).  HIP events in the same run (timed steps):",
        f"# index {pre['ms_index_topk'] * 1e3:.1f} us, inverse index {pre['ms_inverse_index'] * 1e3:.1f} us, "
        f"phase 1 {pre['ms_kvouter_phase1'] * 1e3:.1f} us, combine {pre['ms_combine'] * 1e3:.1f} us"
        + (f"; decode step {dec['ms_per_step'] * 1e3:.1f} us" if dec else "") + ".",
        "",
        f"{'kernel':<44} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10}",
    ]
    for name, calls, avg, mn, mx, _ in rows:
        lines.append(f"{name:<44} {calls:>6} {avg:>10.1f} {mn:>10.1f} {mx:>10.1f}")
    os.makedirs(os.path.dirname(STATS_FILE), exist_ok=True)
    with open(STATS_FILE, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return STATS_FILE


COUNTERS_FILE = os.path.join(ROOT, "profiles", "kernel_counters_128k.txt")
UTIL_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT",
                 "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_BUSY_CU_CYCLES", "SQ_ACTIVE_INST_LDS", "GRBM_GUI_ACTIVE")


def write_counter_summary(util_csv: str, fetch_csv: str, write_csv: str, command: str) -> str:
    """Per-kernel counter summary of the library's kernels from three rocprofv3 --pmc
    passes over the same short run (utilisation counters; FETCH_SIZE; WRITE_SIZE), each
    value averaged over the kernel's dispatches.  Utilisation is per cycle of the
    kernel: GRBM_GUI_ACTIVE is summed over the 8 XCDs, so a dispatch lasts GUI / 8
    shader cycles; MFMA busy is per SIMD (1024 of them), VALU / LDS activity per CU
    (256).  HBM bytes are scaled by what each counter reads for the 1 GiB calibration
    copies at the start of the run (FETCH_SIZE and WRITE_SIZE are in KiB)."""
    import csv
    import re

    def short(name):
        name = name.replace("(anonymous namespace)::", "")
        m = re.search(r"msa::([A-Za-z0-9_]+(?:<[^()]*?>)?)\(", name)
        return m.group(1) if m else None

    def load(path):
        per = {}
        for r in csv.DictReader(open(path)):
            n = short(r["Kernel_Name"]) if "msa::" in r["Kernel_Name"] else (
                "copy" if "copyBuffer" in r["Kernel_Name"] else None)
            if n is None:
                continue
            d = per.setdefault(n, {}).setdefault(int(r["Dispatch_Id"]), {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            d["_ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        return per

    util, fetch, write = load(util_csv), load(fetch_csv), load(write_csv)

    def avg(per, n, c):
        v = [d[c] for d in per.get(n, {}).values() if c in d]
        return sum(v) / len(v) if v else float("nan")

    def copy_factor(per, c):
        v = sorted(per.get("copy", {}).items())[:COPY_REPS]
        kib = sum(d[c] for _, d in v) / max(1, len(v))
        return COPY_BYTES / (kib * 1024.0)

    ff, fw = copy_factor(fetch, "FETCH_SIZE"), copy_factor(write, "WRITE_SIZE")
    lines = [
        "# rocprofv3 counters of the library's kernels: 128K prefill (N=131072 H_q=64 H_kv=8 d_h=128",
        "# B_k=128 k=16, literal inputs) with its KL pass, LSE_idx emission and backward, the paged",
        "# and packed 128K decode (64 sequences) and the split-form Top-k at the pages' table",
        "# shapes; MI355X, one GPU.  Per kernel: dispatches,",
        "# mean duration, shader clock (GUI cycles / duration), MFMA busy per SIMD, VALU busy,",
        "# LDS-indexed activity and LDS bank-conflict cycles per CU (fractions of the kernel's",
        "# cycles), and HBM bytes fetched / written per dispatch (calibrated by 1 GiB copies:",
        f"# FETCH x {ff:.4f}, WRITE x {fw:.4f}).",
        f"# command: {command}",
        "",
        f"{'kernel':<46} {'n':>3} {'ms':>8} {'MHz':>6} {'mfma':>6} {'valu':>6} {'lds':>6} {'ldsbc':>6} "
        f"{'fetch_GB':>9} {'write_GB':>9} {'GB/s':>7}",
    ]
    names = sorted((n for n in util if n != "copy"), key=lambda n: -avg(util, n, "_ns"))
    for n in names:
        ns = avg(util, n, "_ns")
        gui = avg(util, n, "GRBM_GUI_ACTIVE") / 8
        if not (ns > 20000):  # below 20 us the counter windows are not meaningful
            continue
        mfma = avg(util, n, "SQ_VALU_MFMA_BUSY_CYCLES") / (gui * 1024)
        valu = avg(util, n, "SQ_ACTIVE_INST_VALU") / (gui * 256)
        lds = avg(util, n, "SQ_LDS_IDX_ACTIVE") / (gui * 256)
        bc = avg(util, n, "SQ_LDS_BANK_CONFLICT") / (gui * 256)
        fb = avg(fetch, n, "FETCH_SIZE") * 1024 * ff / 1e9
        wb = avg(write, n, "WRITE_SIZE") * 1024 * fw / 1e9
        fns = avg(fetch, n, "_ns")
        lines.append(f"{n:<46} {len(util[n]):>3} {ns / 1e6:>8.3f} {gui / (ns / 1e3):>6.0f} {mfma:>6.3f} {valu:>6.3f} "
                     f"{lds:>6.3f} {bc:>6.3f} {fb:>9.3f} {wb:>9.3f} {(fb + wb) / (fns / 1e9):>7.0f}")
    os.makedirs(os.path.dirname(COUNTERS_FILE), exist_ok=True)
    with open(COUNTERS_FILE, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return COUNTERS_FILE


COPY_BYTES = 1 << 30
COPY_REPS = 3


def calibration_copies():
    """Plain device-to-device copies of COPY_BYTES, made before any other GPU work so
    that a counter run can scale its readings by them."""
    import torch
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(COPY_REPS):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


CLOCK_HZ = 100e6  # the GPU's constant-rate clock (s_memrealtime)


def load_balance(msa, call, max_wg=1024):
    """Per-workgroup start / end clocks of one persistent-grid launch (the library's
    clock hook) reduced to: span, mean busy fraction of the grid over the span, the
    time every workgroup is running (last start to first end), and the tail from the
    first workgroup to finish to the last."""
    import torch
    clk = torch.zeros(2 * max_wg, dtype=torch.int64, device="cuda")
    torch.cuda.synchronize()
    msa.msa_set_profile_clock(clk)
    try:
        call()
        torch.cuda.synchronize()
    finally:
        msa.msa_set_profile_clock(None)
    c = clk.view(-1, 2).cpu()
    c = c[(c[:, 0] != 0) & (c[:, 1] != 0)].double()
    if c.shape[0] == 0:
        return None
    us = lambda ticks: round(float(ticks) / CLOCK_HZ * 1e6, 2)
    t0, t1 = c[:, 0].min(), c[:, 1].max()
    span = float(t1 - t0)
    ends = c[:, 1].sort().values
    return {"workgroups": int(c.shape[0]), "span_us": us(span),
            "busy_frac": round(float((c[:, 1] - c[:, 0]).sum()) / (c.shape[0] * span), 4),
            "all_running_us": us(max(0.0, float(c[:, 1].min() - c[:, 0].max()))),
            "tail_first_end_to_last_us": us(t1 - ends[0]),
            "tail_p90_end_to_last_us": us(t1 - ends[int(0.9 * (len(ends) - 1))]),
            "last_start_us": us(c[:, 0].max() - t0)}


def run_prefill(msa, synth, cfg, mode, steps, warmup, with_kl=False, with_bwd=False):
    import torch
    dev = "cuda"
    N, H_q, H_kv, k, B_k = cfg.N, cfg.H_q, cfg.H_kv, cfg.k, cfg.B_k
    G = H_q // H_kv
    log(f"generating {cfg.name} ({mode}) inputs")
    inp = synth.make_prefill(cfg, mode, device=dev)
    block_idx = torch.empty((N, H_kv, k), dtype=torch.int32, device=dev)
    o = torch.empty((N, H_q, cfg.d_h), dtype=torch.float32, device=dev)
    lse = torch.empty((N, H_q), dtype=torch.float32, device=dev)
    ws = torch.empty(msa.msa_sparse_attn_fwd_workspace(N, H_q, H_kv, k, B_k=B_k), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    n_win = msa.msa_sparse_attn_fwd_windows(N, H_q, H_kv, k, ws.numel(), B_k=B_k)
    # Per step: index start, attention start, attention end, then 4 per query window.
    n_ev = 3 + 4 * n_win

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
            msa.msa_set_profile_events(ev[3:])
        msa.msa_index_topk(inp.q_idx, inp.k_idx, k, B_k=B_k, block_idx=block_idx)
        if ev is not None:
            ev[1].record(stream)
        msa.msa_sparse_attn_fwd(inp.q, inp.k, inp.v, block_idx, B_k=B_k, o=o, lse=lse, workspace=ws)
        if ev is not None:
            ev[2].record(stream)
            msa.msa_set_profile_events(None)

    log(f"prefill {mode}: warmup {warmup}")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(steps)]
    for e in evs:  # create the event handles before the timed region
        for x in e:
            x.record(stream)
    torch.cuda.synchronize()
    log(f"prefill {mode}: timed {steps} steps ({n_win} query window(s) per attention call)")
    t0 = time.perf_counter()
    for s in range(steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg = lambda a, b: sum(e[a].elapsed_time(e[b]) for e in evs) / steps
    # Phase times summed over the query windows of a call.
    wsum = lambda p: sum(avg(3 + 4 * w + p, 4 + 4 * w + p) for w in range(n_win))
    t_index, t_attn = avg(0, 1), avg(1, 2)
    t_inv, t_phase1, t_combine = wsum(0), wsum(1), wsum(2)
    ms_step = wall * 1e3 / steps

    pairs = attended_pairs(block_idx, B_k, G)
    f_index = flops_index_exact(N, H_kv, cfg.d_idx)
    f_main = 4 * cfg.d_h * pairs
    f_total = f_index + f_main
    f_eq12 = flops_msa_eq12(N, H_q, H_kv, cfg.d_h, cfg.d_idx, B_k, k)
    r_off = torch.arange(H_kv, device=dev).view(1, H_kv, 1) * cfg.B
    ids = (block_idx.to(torch.int64) + r_off)[block_idx >= 0]
    fan = torch.bincount(ids, minlength=H_kv * cfg.B).view(H_kv, cfg.B)
    slot_pairs = int((block_idx >= 0).sum().item())     # (query, group, slot) pairs
    lists = int((fan > 0).sum().item())                  # (group, block) lists with work
    # KV-outer phase 1, per (query, group, slot) pair: G q rows gathered (bf16), G
    # unnormalised partial rows written (bf16) and G (max, sum) fp32 pairs; per
    # (group, block) list: its K and V block (bf16) once.
    p1_bytes = slot_pairs * G * (cfg.d_h * 2 + cfg.d_h * 2 + 8) + lists * 2 * B_k * cfg.d_h * 2
    # Combine, per pair: the partial row and (max, sum) read; per (query, head): o and lse written.
    cb_bytes = slot_pairs * G * (cfg.d_h * 2 + 8) + N * H_q * (cfg.d_h * 4 + 4) + N * H_kv * k * 4
    res = {
        "ms_per_step": round(ms_step, 4),
        "tokens_per_s": round(N / (ms_step / 1e3), 1),
        "tflops": round(f_total / (ms_step / 1e3) / 1e12, 2),
        "tflops_eq12_nominal": round(f_eq12 / (ms_step / 1e3) / 1e12, 2),
        "mfma_peak_frac": round(f_total / (ms_step / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "flop_index": f_index, "flop_main": f_main, "flop_eq12": f_eq12,
        "ms_index_topk": round(t_index, 4), "ms_sparse_attn_fwd": round(t_attn, 4),
        "ms_inverse_index": round(t_inv, 4), "ms_kvouter_phase1": round(t_phase1, 4),
        "ms_combine": round(t_combine, 4), "query_windows": n_win,
        "index_tflops": round(f_index / (t_index / 1e3) / 1e12, 2),
        "phase1_tflops": round(f_main / (t_phase1 / 1e3) / 1e12, 2),
        "phase1_algorithmic_bytes": p1_bytes,
        "combine_GB_s": round(cb_bytes / (t_combine / 1e3) / 1e9, 1),
        "slot_pairs": slot_pairs, "lists": lists,
        "block0_fanin_per_group": int(fan[:, 0].float().mean().item()), "max_fanin": int(fan.max().item()),
        "median_fanin": float(fan.float().median().item()),
    }
    res["phase1_load_balance"] = load_balance(
        msa, lambda: msa.msa_sparse_attn_fwd(inp.q, inp.k, inp.v, block_idx, B_k=B_k, o=o, lse=lse, workspace=ws))
    del ws
    if with_kl:
        res["kl"] = run_kl(msa, inp, cfg, block_idx, lse, slot_pairs, lists, pairs, steps)
    if with_bwd:
        res["backward"] = run_bwd(msa, inp, cfg, block_idx, o, lse, slot_pairs, pairs, max(2, steps // 4))
    del o, lse, block_idx
    return res, inp


def run_varlen(msa, synth, vcfg, mode, steps, warmup):
    """Packed variable-length prefill: index Top-k and attention over a batch of
    sequences of different lengths packed on the token axis (cu_seqlens)."""
    import torch
    dev = "cuda"
    B_k, H_q, H_kv, k = vcfg.B_k, vcfg.H_q, vcfg.H_kv, vcfg.k
    G = H_q // H_kv
    lengths = synth.varlen_lengths(vcfg)
    log(f"generating {vcfg.name} ({mode}) packed inputs: {len(lengths)} sequences")
    p = synth.packed_prefill(lengths, H_q, H_kv, k, vcfg.seed, mode, device=dev)
    T, batch, max_len = sum(lengths), len(lengths), max(lengths)
    bi = torch.empty((T, H_kv, k), dtype=torch.int32, device=dev)
    o = torch.empty((T, H_q, 128), dtype=torch.float32, device=dev)
    lse = torch.empty((T, H_q), dtype=torch.float32, device=dev)
    ws = torch.empty(msa.msa_sparse_attn_fwd_varlen_workspace(T, batch, H_q, H_kv, k, B_k=B_k), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        msa.msa_index_topk_varlen(p.q_idx, p.k_idx, p.cu_seqlens, max_len, k, B_k=B_k, block_idx=bi)
        if ev is not None:
            ev[1].record(stream)
        msa.msa_sparse_attn_fwd_varlen(p.q, p.k, p.v, bi, p.cu_seqlens, B_k=B_k, o=o, lse=lse, workspace=ws)
        if ev is not None:
            ev[2].record(stream)

    log(f"varlen {mode}: warmup {warmup}, timed {steps} steps")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t0 = time.perf_counter()
    for s in range(steps):
        step(evs[s])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    avg = lambda a, b: sum(e[a].elapsed_time(e[b]) for e in evs) / steps
    cu = p.cu_seqlens.cpu().tolist()
    # Exact work per sequence: its own causal index scores and attended tokens.
    f_index = sum(flops_index_exact(L, H_kv, 64) for L in lengths)
    f_main = 4 * 128 * sum(attended_pairs(bi[cu[s]:cu[s + 1]], B_k, G) for s in range(batch) if lengths[s] > 0)
    f = f_index + f_main
    del p, bi, o, lse, ws
    torch.cuda.empty_cache()
    return {"workload": f"packed prefill T={T} batch={batch} lengths {min(lengths)}..{max_len} H_q={H_q} "
                        f"H_kv={H_kv} B_k={B_k} k={k}",
            "ms_per_step": round(ms, 4), "tokens_per_s": round(T / (ms / 1e3), 1),
            "ms_index_topk": round(avg(0, 1), 4), "ms_sparse_attn_fwd": round(avg(1, 2), 4),
            "tflops": round(f / (ms / 1e3) / 1e12, 2),
            "mfma_peak_frac": round(f / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4), "steps": steps}


def run_bwd(msa, inp, cfg, block_idx, o, lse, slot_pairs, pairs, steps):
    """The Main Branch backward on the step's selection and outputs, for a seeded
    upstream gradient, timed on its own (a training step's second half)."""
    import torch
    N, H_q, H_kv, k = cfg.N, cfg.H_q, cfg.H_kv, cfg.k
    G = H_q // H_kv
    dev = "cuda"
    torch.cuda.empty_cache()
    g = torch.Generator(device=dev).manual_seed(cfg.seed)
    dO = torch.randn((N, H_q, cfg.d_h), generator=g, device=dev).to(torch.bfloat16)
    dq = torch.empty((N, H_q, cfg.d_h), dtype=torch.float32, device=dev)
    dk = torch.empty((N, H_kv, cfg.d_h), dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)
    ws = torch.empty(msa.msa_sparse_attn_bwd_workspace(N, H_q, H_kv, k), dtype=torch.uint8, device=dev)

    def step():
        msa.msa_sparse_attn_bwd(inp.q, inp.k, inp.v, o, lse, dO, block_idx, dq=dq, dk=dk, dv=dv, workspace=ws)

    step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # S, dP, dV, dK and dQ: five products of 2 d_h FLOP per attended (query, head, key).
    flops = 10 * cfg.d_h * pairs
    out = {"ms": round(ms, 4), "tflops": round(flops / (ms / 1e3) / 1e12, 2),
           "mfma_peak_frac": round(flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4), "steps": steps,
           "workspace_bytes": int(ws.numel()), "main_kernel_load_balance": load_balance(msa, step)}
    del ws, dO, dq, dk, dv
    torch.cuda.empty_cache()
    return out


def run_kl(msa, inp, cfg, block_idx, lse, slot_pairs, lists, pairs, steps):
    """The KL alignment pass (Eq. 9-10) on the step's selection and lse, timed on its
    own: it follows the forward in training and is not part of the timed step."""
    import torch
    N, H_q, H_kv, k, B_k = cfg.N, cfg.H_q, cfg.H_kv, cfg.k, cfg.B_k
    G = H_q // H_kv
    dev = "cuda"
    kws = torch.empty(msa.msa_sparse_kl_fwd_workspace(N, H_q, H_kv, k), dtype=torch.uint8, device=dev)
    kl = torch.empty((N, H_kv), dtype=torch.float32, device=dev)
    lse_idx = torch.empty((N, H_kv), dtype=torch.float32, device=dev)
    loss = torch.empty((1,), dtype=torch.float32, device=dev)

    def kl_step():
        msa.msa_sparse_kl_fwd(inp.q, inp.k, inp.q_idx, inp.k_idx, block_idx, lse, kl=kl, lse_idx=lse_idx, loss=loss,
                              workspace=kws)

    kl_step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        kl_step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # Per (query, group, slot) pair: G q rows, the index query row, G lse values and
    # the 32-byte partial; per (group, block) list: its K block and index-key block.
    nbytes = slot_pairs * (G * cfg.d_h * 2 + cfg.d_idx * 2 + G * 4 + 32) + lists * B_k * (cfg.d_h + cfg.d_idx) * 2
    # QK for every attended (query, head, key) and one index dot product per (query, group, key).
    flops = 2 * cfg.d_h * pairs + 2 * cfg.d_idx * (pairs // G)
    out = {"ms": round(ms, 4), "algorithmic_bytes": nbytes, "GB_s": round(nbytes / (ms / 1e3) / 1e9, 1),
           "tflops": round(flops / (ms / 1e3) / 1e12, 2), "loss": round(float(loss.item()), 6), "steps": steps}
    del kws, kl, loss
    # LSE_idx emitted by the forward (msa_sparse_attn_fwd_lse_idx): its cost over the
    # plain forward, both timed here on the same inputs and workspace.
    torch.cuda.empty_cache()
    ws = torch.empty(msa.msa_sparse_attn_fwd_workspace(N, H_q, H_kv, k, B_k=B_k), dtype=torch.uint8, device=dev)
    o = torch.empty((N, H_q, cfg.d_h), dtype=torch.float32, device=dev)
    lse2 = torch.empty((N, H_q), dtype=torch.float32, device=dev)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    t_plain = timed(lambda: msa.msa_sparse_attn_fwd(inp.q, inp.k, inp.v, block_idx, B_k=B_k, o=o, lse=lse2,
                                                    workspace=ws))
    t_li = timed(lambda: msa.msa_sparse_attn_fwd_lse_idx(inp.q, inp.k, inp.v, inp.q_idx, inp.k_idx, block_idx,
                                                         B_k=B_k, o=o, lse=lse2, lse_idx=lse_idx, workspace=ws))
    out["forward_ms"] = round(t_plain, 4)
    out["forward_with_lse_idx_ms"] = round(t_li, 4)
    out["lse_idx_emission_ms"] = round(t_li - t_plain, 4)
    del ws, o, lse2
    # The KL value with that LSE_idx given (no index log partition in the pass).
    kws = torch.empty(msa.msa_sparse_kl_fwd_workspace(N, H_q, H_kv, k), dtype=torch.uint8, device=dev)
    kl = torch.empty((N, H_kv), dtype=torch.float32, device=dev)
    loss = torch.empty((1,), dtype=torch.float32, device=dev)
    t_given = timed(lambda: msa.msa_sparse_kl_fwd_from_lse_idx(inp.q, inp.k, inp.q_idx, inp.k_idx, block_idx, lse,
                                                               lse_idx, B_k=B_k, kl=kl, loss=loss, workspace=kws))
    out["from_lse_idx_ms"] = round(t_given, 4)
    out["from_lse_idx_loss"] = round(float(loss.item()), 6)
    del kws, kl, loss, lse_idx
    return out


def run_decode(msa, synth, dcfg, mode, steps, warmup, paged=False):
    import torch
    dev = "cuda"
    B_k = dcfg.B_k
    log(f"generating {dcfg.name} ({mode}) decode inputs")
    d = synth.make_decode(dcfg, mode, device=dev)
    max_len = max(d.lengths)
    dbi = torch.empty((dcfg.batch, dcfg.H_kv, dcfg.k), dtype=torch.int32, device=dev)
    do = torch.empty((dcfg.batch, dcfg.H_q, dcfg.d_h), dtype=torch.float32, device=dev)
    dl = torch.empty((dcfg.batch, dcfg.H_q), dtype=torch.float32, device=dev)
    dws = torch.empty(msa.msa_decode_workspace(dcfg.batch, dcfg.H_q, dcfg.H_kv, dcfg.k, max_len),
                      dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def decode_step():
        msa.msa_decode(d.q, d.q_idx, d.k_cache, d.v_cache, d.k_idx_cache, d.cu_seqlens, max_len, dcfg.k,
                       block_idx=dbi, o=do, lse=dl, workspace=dws)

    for _ in range(warmup):
        decode_step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        decode_step()
    e1.record(stream)
    torch.cuda.synchronize()
    dms = e0.elapsed_time(e1) / steps
    T = int(d.cu_seqlens[-1].item())
    # every cached index key (d_idx bf16) + K and V of the chosen blocks of every group
    chosen = int((dbi >= 0).sum().item())
    dbytes = T * dcfg.d_idx * 2 + chosen * B_k * dcfg.d_h * 2 * 2
    del d
    out = {
        "workload": f"decode batch={dcfg.batch} L={min(synth.decode_lengths(dcfg))}..{max_len} H_q={dcfg.H_q} "
                    f"H_kv={dcfg.H_kv} k={dcfg.k}",
        "ms_per_step": round(dms, 4), "tokens_per_s": round(dcfg.batch / (dms / 1e3), 1),
        "algorithmic_bytes": dbytes, "GB_s": round(dbytes / (dms / 1e3) / 1e9, 1),
        "hbm_peak_frac": round(dbytes / (dms / 1e3) / 1e9 / PEAK_HBM_GBS, 4), "steps": steps,
    }
    if paged:
        torch.cuda.empty_cache()
        out["paged_fp8"] = run_decode_paged(msa, synth, dcfg, mode, steps, warmup)
    return out


def run_decode_paged(msa, synth, dcfg, mode, steps, warmup):
    """The same decode over a paged cache with FP8 E4M3 K/V (bf16 index keys)."""
    import torch
    dev = "cuda"
    B_k = dcfg.B_k
    log(f"generating {dcfg.name} ({mode}) paged FP8 decode inputs")
    p = synth.make_decode_paged(dcfg, mode, device=dev)
    del p.contiguous.k_cache, p.contiguous.v_cache
    torch.cuda.empty_cache()
    max_len = max(p.lengths)
    dbi = torch.empty((dcfg.batch, dcfg.H_kv, dcfg.k), dtype=torch.int32, device=dev)
    do = torch.empty((dcfg.batch, dcfg.H_q, dcfg.d_h), dtype=torch.float32, device=dev)
    dl = torch.empty((dcfg.batch, dcfg.H_q), dtype=torch.float32, device=dev)
    dws = torch.empty(msa.msa_decode_workspace(dcfg.batch, dcfg.H_q, dcfg.H_kv, dcfg.k, max_len),
                      dtype=torch.uint8, device=dev)

    def step():
        msa.msa_decode_paged(p.q, p.q_idx, p.k_pages, p.v_pages, p.k_scale, p.v_scale, p.kidx_pages, p.block_table,
                             p.seqlens, max_len, dcfg.k, block_idx=dbi, o=do, lse=dl, workspace=dws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    dms = e0.elapsed_time(e1) / steps
    T = sum(p.lengths)
    chosen = int((dbi >= 0).sum().item())
    # every cached index key (bf16) + the FP8 K and V rows of the chosen blocks
    dbytes = T * dcfg.d_idx * 2 + chosen * B_k * dcfg.d_h * 1 * 2
    del p
    return {"ms_per_step": round(dms, 4), "tokens_per_s": round(dcfg.batch / (dms / 1e3), 1),
            "algorithmic_bytes": dbytes, "GB_s": round(dbytes / (dms / 1e3) / 1e9, 1),
            "hbm_peak_frac": round(dbytes / (dms / 1e3) / 1e9 / PEAK_HBM_GBS, 4), "steps": steps}


def run_table1(msa, steps=5):
    """Top-k alone from given block scores at the shapes of the pages' Top-k table
    ([N, B, k] rows; one score row per query, causal prefix b <= i / B_k), timed with
    events.  The table's own row count and dtype are not stated: context only."""
    import torch
    out = []
    for N, B, k in ((131072, 1024, 16), (131072, 1024, 32), (524288, 4096, 16), (524288, 8192, 32)):
        B_k = N // B
        g = torch.Generator(device="cuda").manual_seed(N + B + k)
        M = torch.randn((N, 1, B), generator=g, device="cuda")
        bi = torch.empty((N, 1, k), dtype=torch.int32, device="cuda")
        msa.msa_topk_from_scores(M, k, B_k=B_k, block_idx=bi)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            msa.msa_topk_from_scores(M, k, B_k=B_k, block_idx=bi)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / steps * 1e3
        causal_bytes = 4 * (B * (B + 1) // 2) * B_k  # the scores each row reads
        gbs = causal_bytes / (us / 1e6) / 1e9
        chunks = (B + 63) // 64  # 64-block chunks of the longest row: which kernel runs
        kernel = ("topk_from_scores_kernel<16>" if chunks <= 16 else
                  "topk_from_scores_kernel<32>" if chunks <= 32 else "topk_from_scores_long_kernel")
        out.append({"N": N, "blocks": B, "k": k, "B_k": B_k, "kernel": kernel, "us": round(us, 1),
                    "GB_s": round(gbs, 1), "hbm_peak_frac": round(gbs / PEAK_HBM_GBS, 4)})
        del M, bi
        torch.cuda.empty_cache()
    return out


def measured_peaks():
    """Measured ceilings of this GPU, beside the vendor figures: a register-only bf16
    MFMA loop (32x32x16, four independent chains per wave, two waves per SIMD), a
    streaming read of 4 GiB and a 2 GiB device copy, each timed with HIP events."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "block_sparse_gqa_index_amd", "libmsa_peaks.so"))
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.msa_peak_mfma.argtypes = [I32, I32, I32, P, P]
    lib.msa_peak_read.argtypes = [P, I64, I32, P, P]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps / 1e3

    waves, iters = 8, 20000
    sink = torch.empty(cus * waves * 64, dtype=torch.float32, device="cuda")
    t = timed(lambda: lib.msa_peak_mfma(cus, waves, iters, sink.data_ptr(), stream.cuda_stream), 3)
    mfma = cus * waves * iters * 4 * 32768 / t / 1e12
    buf = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    out = torch.empty(1, dtype=torch.int32, device="cuda")
    t = timed(lambda: lib.msa_peak_read(buf.data_ptr(), buf.numel(), cus, out.data_ptr(), stream.cuda_stream), 5)
    read = buf.numel() / t / 1e9
    src, dst = buf[: 2 << 30], buf[2 << 30:]
    t = timed(lambda: dst.copy_(src), 5)
    copy = 2 * src.numel() / t / 1e9
    del buf, sink
    torch.cuda.empty_cache()
    return {"mfma_bf16_tflops": round(mfma, 1), "hbm_read_GB_s": round(read, 1), "hbm_copy_GB_s": round(copy, 1),
            "vendor_mfma_bf16_tflops": PEAK_BF16_TFLOPS, "vendor_hbm_GB_s": PEAK_HBM_GBS}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, cfg, n_rows):
    """The oracle on a uniform sample of query rows of the same prefill (all groups and
    heads), timed in two halves by query position, which fit a per-row cost
    t(i) = a + b i (index scoring grows with i; the attention budget is fixed): the
    full 128K and 1M runs are extrapolated from it, and the 4K workload is run whole."""
    import numpy as np
    import oracle
    import synth
    N, k, B_k = cfg.N, cfg.k, cfg.B_k
    log(f"cpu baseline: oracle on {n_rows} sampled query rows")
    g = np.random.default_rng(cfg.seed)
    rows = np.sort(g.choice(N, size=min(n_rows, N), replace=False))
    qi_h, ki_h = inp.q_idx.cpu(), inp.k_idx.cpu()
    q_h, k_h, v_h = inp.q.cpu(), inp.k.cpu(), inp.v.cpu()

    def run(rs):
        t0 = time.perf_counter()
        M = oracle.block_scores(qi_h, ki_h, B_k, rows=rs)
        bi = oracle.topk(M, k, B_k, rows=rs)
        oracle.sparse_attn(q_h, k_h, v_h, bi, B_k, rows=rs)
        return time.perf_counter() - t0

    lo, hi = rows[: len(rows) // 2], rows[len(rows) // 2:]
    t_lo, t_hi = run(lo), run(hi)
    tc = t_lo + t_hi
    # Mean row cost of each half is a + b * (its mean position).
    c_lo, c_hi = t_lo / len(lo), t_hi / len(hi)
    b = (c_hi - c_lo) / (hi.mean() - lo.mean())
    a = c_lo - b * lo.mean()
    full = lambda n: n * a + b * n * (n - 1) / 2
    del qi_h, ki_h, q_h, k_h, v_h
    # The 4K workload (H_q = 4, H_kv = 1, k = 8) whole.
    c0 = synth.CONFIGS["c0"]
    i0 = synth.make_prefill(c0, "literal", device="cpu")
    t0 = time.perf_counter()
    M0 = oracle.block_scores(i0.q_idx, i0.k_idx, c0.B_k)
    oracle.sparse_attn(i0.q, i0.k, i0.v, oracle.topk(M0, c0.k, c0.B_k), c0.B_k)
    t_c0 = time.perf_counter() - t0
    return {"value": round(len(rows) / tc, 3), "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "sample": f"{len(rows)} uniformly drawn query rows of the same {N}-token prefill (all groups and "
                      f"heads; index scoring, Top-k and attention), {tc:.1f} s",
            "full_4k_prefill_s": round(t_c0, 2),
            "extrapolated": {"model": "per-row cost t(i) = a + b i fitted on the two halves of the sample",
                             "a_s": a, "b_s": b,
                             "prefill_128k_s": round(full(N), 1),
                             "prefill_1m_s": round(full(1 << 20), 1),
                             "prefill_1m_tokens_per_s": round((1 << 20) / full(1 << 20), 3)}}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--mode", default="literal", choices=["literal", "structured"],
                    help="input mode of the headline figures; the other mode is reported beside them")
    ap.add_argument("--workload", default="c2")
    ap.add_argument("--decode-workload", default="c3_128k")
    ap.add_argument("--cpu-rows", type=int, default=4096, help="query rows in the oracle's timed sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-kl", action="store_true", help="skip the separately timed KL alignment pass")
    ap.add_argument("--no-paged", action="store_true", help="skip the paged FP8 decode measurement")
    ap.add_argument("--no-bwd", action="store_true", help="skip the separately timed backward")
    ap.add_argument("--table1", action="store_true",
                    help="time Top-k alone at the pages' Top-k table shapes (the default; kept for recorded commands)")
    ap.add_argument("--no-table1", action="store_true", help="skip Top-k alone at the pages' Top-k table shapes")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the 128K prefill with B_k = 64 and the packed variable-length batch")
    ap.add_argument("--single-mode", action="store_true", help="skip the second input mode")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured MFMA / HBM peak kernels")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the 32K and 1M prefill and the mixed-length decode lines")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="start with plain copies of known size (for counter runs)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic summary from two rocprofv3 counter CSVs and exit")
    ap.add_argument("--traffic-command", default="", help="the command the counter CSVs came from")
    ap.add_argument("--counters-from", nargs=3, metavar=("UTIL_CSV", "FETCH_CSV", "WRITE_CSV"),
                    help="write the per-kernel counter summary from three rocprofv3 --pmc runs and exit")
    ap.add_argument("--stats-from", nargs=2, metavar=("STATS_CSV", "RUN_LOG"),
                    help="write the kernel statistics summary from a rocprofv3 --stats run and exit")
    args = ap.parse_args(argv)

    if args.stats_from:
        print(write_stats_summary(args.stats_from[0], args.stats_from[1], args.traffic_command))
        return 0
    if args.counters_from:
        print(write_counter_summary(*args.counters_from, args.traffic_command))
        return 0
    if args.traffic_from:
        print(write_traffic_summary(args.traffic_from[0], args.traffic_from[1], args.mode, args.traffic_command))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the MSA path here has no multi-GPU mode "
              "(each GPU would own a share of the KV groups and run the same kernels).", file=sys.stderr)
        return 2

    import torch
    import block_sparse_gqa_index_amd as msa
    import synth

    torch.cuda.set_device(0)
    if args.calibrate_copy:
        calibration_copies()
    cfg = synth.CONFIGS[args.workload]
    N, H_q, H_kv, k, B_k = cfg.N, cfg.H_q, cfg.H_kv, cfg.k, cfg.B_k
    other = "structured" if args.mode == "literal" else "literal"

    pre, inp = run_prefill(msa, synth, cfg, args.mode, args.steps, args.warmup, with_kl=not args.no_kl,
                           with_bwd=not args.no_bwd)
    result = {
        "metric": "MSA prefill tokens/s + TFLOP/s at 128K; decode tokens/s at 128K KV (1 GPU)",
        "value": pre["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": f"synthetic ({args.mode} mode, seeded)",
        "config": {"workload": f"prefill N={N} H_q={H_q} H_kv={H_kv} d_h={cfg.d_h} d_idx={cfg.d_idx} "
                               f"B_k={B_k} k={k}", "mode": args.mode, "seq_len": N, "batch": 1},
        "prefill": pre,
    }
    # The dominant kernel is the KV-outer phase 1; it is bound by its HBM bytes
    # (about 126 FLOP per byte, below the bf16 ridge of about 312).  It runs once per
    # query window: bytes per launch / average launch time = total bytes / total time.
    gbs = pre["phase1_algorithmic_bytes"] / (pre["ms_kvouter_phase1"] / 1e3) / 1e9
    traffic = recorded_traffic(args.mode)
    result["roofline"] = {"kernel": "attn_kvouter_kernel", "bound": "hbm", "achieved": round(gbs, 1),
                          "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                          "traffic": traffic,
                          "algorithmic_bytes": pre["phase1_algorithmic_bytes"],
                          "launches_per_step": pre["query_windows"],
                          "mfma_frac": round(pre["phase1_tflops"] / PEAK_BF16_TFLOPS, 4)}

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, cfg, args.cpu_rows)
    if not args.no_table1:
        log("Top-k alone at the table shapes")
        result["topk_table1"] = run_table1(msa)
    del inp
    torch.cuda.empty_cache()
    peaks = None
    if not args.no_peaks:
        log("measured peaks: MFMA loop, streaming read, device copy")
        peaks = measured_peaks()
        result["measured_peaks"] = peaks
    result["rooflines"] = kernel_rooflines(pre, peaks)
    if peaks and "topk_table1" in result:
        for row in result["topk_table1"]:
            row["frac_of_measured_read"] = round(row["GB_s"] / peaks["hbm_read_GB_s"], 4)

    if not args.no_decode:
        dcfg = synth.CONFIGS[args.decode_workload]
        result["decode"] = run_decode(msa, synth, dcfg, args.mode, max(args.steps, 50), args.warmup,
                                      paged=not args.no_paged)
        if peaks:
            dec = result["decode"]
            dec["frac_of_measured_read"] = round(dec["GB_s"] / peaks["hbm_read_GB_s"], 4)
            if "paged_fp8" in dec:
                dec["paged_fp8"]["frac_of_measured_read"] = round(dec["paged_fp8"]["GB_s"] / peaks["hbm_read_GB_s"], 4)
        torch.cuda.empty_cache()
    if not args.no_extra:
        c64 = synth.CONFIGS["c2_bk64"]
        pre64, inp64 = run_prefill(msa, synth, c64, args.mode, args.steps, args.warmup)
        del inp64
        torch.cuda.empty_cache()
        pre64["workload"] = (f"prefill N={c64.N} H_q={c64.H_q} H_kv={c64.H_kv} d_h={c64.d_h} d_idx={c64.d_idx} "
                             f"B_k={c64.B_k} k={c64.k}")
        result["prefill_bk64"] = pre64
        result["varlen"] = run_varlen(msa, synth, synth.VARLEN_CONFIGS["c2_varlen"], args.mode, args.steps,
                                      args.warmup)
    if not args.no_configs:
        # The pages' other contexts (32K and 1M prefill) and the decode batch with its
        # specified mixed lengths, in the headline input mode.
        other_cfgs = {}
        pre1, inp1 = run_prefill(msa, synth, synth.CONFIGS["c1"], args.mode, args.steps, args.warmup)
        del inp1
        torch.cuda.empty_cache()
        pre1["workload"] = "prefill N=32768 H_q=32 H_kv=4 d_h=128 d_idx=64 B_k=128 k=16"
        other_cfgs["prefill_32k"] = pre1
        if not args.no_decode:
            other_cfgs["decode_mixed"] = run_decode(msa, synth, synth.CONFIGS["c3"], args.mode, max(args.steps, 50),
                                                    args.warmup)
            torch.cuda.empty_cache()
        c4 = synth.CONFIGS["c4"]
        pre4, inp4 = run_prefill(msa, synth, c4, args.mode, max(1, min(args.steps, 3)), 1)
        del inp4
        torch.cuda.empty_cache()
        pre4["workload"] = "prefill N=1048576 H_q=64 H_kv=8 d_h=128 d_idx=64 B_k=128 k=16"
        other_cfgs["prefill_1m"] = pre4
        result["configs"] = other_cfgs
    if not args.single_mode:
        pre2, inp2 = run_prefill(msa, synth, cfg, other, args.steps, args.warmup)
        del inp2
        torch.cuda.empty_cache()
        result[other] = {"prefill": pre2}
        if not args.no_decode:
            result[other]["decode"] = run_decode(msa, synth, synth.CONFIGS[args.decode_workload], other,
                                                 max(args.steps, 50), args.warmup)
            torch.cuda.empty_cache()
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

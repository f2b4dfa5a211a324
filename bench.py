#!/usr/bin/env python3
"""Benchmark of the token-sparse attention hot path on one MI355X.

One step = the whole path over one batch: for every layer, block scoring -> block selection
-> permutation-free sparse attention forward (residual updated in place), then the segmented
backward of every layer in reverse order.  Inputs are seeded synthetic tensors already
resident in HBM.  Prints ONE JSON line.

The metric counts kept-token FLOPs of the attention forward and backward only:
fwd = 4*D*Hq*P and bwd = 10*D*Hq*P per batch row, P = Nk(Nk+1)/2 causal pairs among the
Nk kept tokens; recomputation and scoring FLOPs are not counted.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2516.6     # 256 CU x 4096 bf16 flop/clk/CU x 2.4 GHz, dense
HBM_PEAK_GBS = 8000.0
KERNELS = ("k_slse64", "k_sblock_mass", "k_eq2_tiles", "k_eq2_reduce", "k_select", "k_pack_tp",
           "k_fwd64", "k_fwd_combine", "k_prep64", "k_bwd64", "k_kv_reduce", "k_proj_gather", "k_proj_scatter",
           "k_proj_logits", "k_ce_rows", "k_proj_dh", "k_mlp_act_gated", "k_mlp_block",
           "k_proj_gather_scatter")
METRIC = "fwd+bwd token-sparse attn TFLOP/s (kept FLOPs) & tokens/s at S=32K; % MFMA peak"
# MFMA work the backward kernel executes per (query head, causal kept pair), in units of D flop:
# its dK/dV tiles form S, dP, dV and dK (8 D), its dQ tiles S, dP and dQ (6 D)
BWD_EXECUTED_D = 14.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="c5", help="workload name (c1..c5); c5 is the S=32K one")
    ap.add_argument("--kept", choices=["selected", "scattered"], default="selected",
                    help="attention over the selected blocks, or over a seeded scattered set")
    ap.add_argument("--segments", type=int, default=0, help="override backward segment count")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--summarize", nargs=4, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR", "BENCH_LOG"),
                    help="no GPU work: turn rocprofv3 csv output of this bench (kernel trace, then "
                         "FETCH_SIZE and WRITE_SIZE passes run with --copy-calibration) into the "
                         "summaries kept under profiles/")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB elementwise copy (HBM counter calibration)")
    return ap.parse_args()


# The sources the dominant kernel (k_bwd64) is compiled from: its traffic counters stay valid
# while their code is unchanged (comments and layout do not count).
ROOFLINE_SOURCES = ("attn64.hip", "tiles64.h", "common.h", "kernels.h")


def kernel_source_hash() -> str:
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "token_sparse_attention_jenga_amd", "csrc")
    for name in ROOFLINE_SOURCES:
        with open(os.path.join(csrc, name)) as f:
            code = f.read()
        code = re.sub(r"/\*.*?\*/", " ", code, flags=re.S)     # block comments
        code = re.sub(r"//[^\n]*", " ", code)                    # line comments
        code = " ".join(code.split())                            # layout
        h.update(name.encode())
        h.update(code.encode())
    return h.hexdigest()[:16]


# k_proj<MODE> instances (one template, several launch names: the logits and dL/dh products of
# the loss are both the plain mode)
PROJ_MODES = {0: "k_proj<gather>", 1: "k_proj<scatter>", 2: "k_proj<plain>",
              3: "k_proj<gather_scatter>", 4: "k_proj<mlp_gated>", 5: "k_proj<mlp_relu>"}


def _short(name: str) -> str:
    for mode, label in PROJ_MODES.items():
        if f"::k_proj<{mode}>" in name:
            return label
    for k in KERNELS + ("k_score_reduce", "k_loss_mean"):
        if f"::{k}<" in name or f"::{k}(" in name:
            return k
    if "neg_kernel" in name:
        return "calibration copy (elementwise neg, 1 GiB)"
    return name.split("(")[0][:70]


def summarize(trace_dir, fetch_dir, write_dir, bench_log, cfg_name="c5"):
    """Write profiles/kernels_<cfg>.md (per-kernel times from the rocprofv3 kernel trace next to
    the bench's own HIP-event averages, and HBM bytes per dispatch from FETCH_SIZE / WRITE_SIZE)
    and profiles/traffic_k_bwd64_<cfg>.json.  Only the dispatches of the bench's steps count:
    the first (warmup + 2 * steps) * (launches per step) dispatches of each kernel in issue
    order (warm-up, timed and instrumented passes); later sections of the bench (memory sweep,
    scattered kept sets, NEXT rows) launch the same kernels at other sizes.  Counter bytes are
    scaled by the ratio known bytes / counter of the calibration copy, which moves exactly 1 GiB
    each way."""
    import csv
    with open(bench_log) as f:
        line = [x for x in f if x.startswith("{")][-1]
    bench = json.loads(line)
    K, W = bench["steps"], bench["warmup"]
    ev = bench.get("kernel_avg_us", {})
    per_step = {k: v["launches"] // K for k, v in ev.items()}       # instrumented pass: K steps
    budget = {k: (W + 2 * K) * n for k, n in per_step.items()}

    def first_n(rows, key, name_of):
        seen, out = {}, []
        for r in sorted(rows, key=key):
            k = name_of(r)
            if k in budget:
                seen[k] = seen.get(k, 0) + 1
                if seen[k] > budget[k]:
                    continue
            out.append((k, r))
        return out

    trace = list(csv.DictReader(open(os.path.join(trace_dir, "run_kernel_trace.csv"))))
    dur = {}
    for k, r in first_n(trace, lambda r: int(r["Start_Timestamp"]), lambda r: _short(r["Kernel_Name"])):
        n, t = dur.get(k, (0, 0.0))
        dur[k] = (n + 1, t + (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)

    def counters(d):
        rows = list(csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))))
        agg = {}
        for k, r in first_n(rows, lambda r: int(r["Dispatch_Id"]), lambda r: _short(r["Kernel_Name"])):
            n, t = agg.get(k, (0, 0.0))
            agg[k] = (n + 1, t + float(r["Counter_Value"]) * 1024.0)
        return agg
    fetch, write = counters(fetch_dir), counters(write_dir)
    cal = "calibration copy (elementwise neg, 1 GiB)"
    f_fac = 2**30 / (fetch[cal][1] / fetch[cal][0])
    w_fac = 2**30 / (write[cal][1] / write[cal][0])
    lines = [f"# Kernel times and HBM bytes, {cfg_name} bench step (rocprofv3)", "",
             "Commands (`<repo>` the repository root, `<out>` any output directory; "
             "`cd /tmp && export TMPDIR=/tmp` first):", "",
             "    rocprofv3 --kernel-trace --stats --output-format csv -d <out>/prof_trace -o run "
             "-- python3 <repo>/bench.py --steps 2 --warmup 1 --no-cpu-baseline > <out>/prof_trace.log",
             "    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/prof_fetch -o run -- "
             "python3 <repo>/bench.py --steps 2 --warmup 1 --no-cpu-baseline --copy-calibration",
             "    rocprofv3 --pmc WRITE_SIZE ... (same, -d <out>/prof_write)",
             "    python3 bench.py --summarize <out>/prof_trace <out>/prof_fetch <out>/prof_write "
             "<out>/prof_trace.log", "",
             f"Kernel source hash {kernel_source_hash()} (code of the attention kernel sources, comments and "
             "layout excluded).  Only the dispatches of the bench's steps are counted: per kernel, the first "
             "(warmup + 2 x steps) x (launches per step) dispatches in issue order (warm-up, timed and "
             "instrumented passes of the same step); the bench's later sections (memory sweep, scattered "
             "kept sets, NEXT rows) are left out.", "",
             f"Calibration: the 1 GiB copy reads FETCH_SIZE {fetch[cal][1] / fetch[cal][0] / 2**20:.1f} MiB and "
             f"WRITE_SIZE {write[cal][1] / write[cal][0] / 2**20:.1f} MiB, so counter bytes are scaled by "
             f"{f_fac:.3f} (fetch) and {w_fac:.3f} (write).", "",
             "| kernel | dispatches | rocprof avg us | bench event avg us | fetch MiB/dispatch | write MiB/dispatch |",
             "|---|---|---|---|---|---|"]
    for k in sorted(dur, key=lambda k: -dur[k][1]):
        if k not in budget:
            continue
        n, t = dur[k]
        e = ev.get(k, {}).get("avg_us", "")
        fm = f"{fetch[k][1] / fetch[k][0] * f_fac / 2**20:.1f}" if k in fetch else ""
        wm = f"{write[k][1] / write[k][0] * w_fac / 2**20:.1f}" if k in write else ""
        lines.append(f"| {k} | {n} | {t / n:.1f} | {e} | {fm} | {wm} |")
    # Eq. 2 scoring (a NEXT row) runs in a section of its own, once per layer at the workload's
    # size, so every dispatch of its kernels counts
    eq = bench.get("eq2_scoring") or {}
    import re
    shape = dict(re.findall(r"(\w+)=(\d+)", bench.get("config", {}).get("workload", "")))
    one_size = [k for k in ("k_eq2_tiles", "k_eq2_reduce") if k in dur]
    if one_size:
        qk = int(shape.get("B", 0)) * int(shape.get("S", 0)) * (int(shape.get("Hq", 0)) + int(shape.get("Hkv", 0))) \
            * int(shape.get("D", 0)) * 2
        lines += ["", "Eq. 2 scoring, every dispatch of the bench's Eq. 2 section (one call per layer at the "
                  f"workload's size; Q and K hold {qk / 2**20:.0f} MiB per layer):", "",
                  "| kernel | dispatches | rocprof avg us | bench event avg us | fetch MiB/dispatch | write MiB/dispatch |",
                  "|---|---|---|---|---|---|"]
        for k in one_size:
            n, t = dur[k]
            e = eq.get("k_eq2_tiles_avg_us", "") if k == "k_eq2_tiles" else ""
            fm = f"{fetch[k][1] / fetch[k][0] * f_fac / 2**20:.1f}" if k in fetch else ""
            wm = f"{write[k][1] / write[k][0] * w_fac / 2**20:.1f}" if k in write else ""
            lines.append(f"| {k} | {n} | {t / n:.1f} | {e} | {fm} | {wm} |")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"kernels_{cfg_name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    k = "k_bwd64"
    t = {"kernel": k, "config": cfg_name, "kernel_source_hash": kernel_source_hash(),
         "dispatches": fetch[k][0], "fetch_scale": round(f_fac, 4), "write_scale": round(w_fac, 4),
         "fetch_bytes_per_launch": round(fetch[k][1] / fetch[k][0] * f_fac),
         "write_bytes_per_launch": round(write[k][1] / write[k][0] * w_fac)}
    t["hbm_bytes_per_launch"] = t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"]
    with open(os.path.join(ROOT, "profiles", f"traffic_{k}_{cfg_name}.json"), "w") as f:
        json.dump(t, f, indent=1)
        f.write("\n")
    print("\n".join(lines))
    print(json.dumps(t))


def main():
    args = parse()
    if args.summarize:
        summarize(*args.summarize, cfg_name=args.config)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the token-sparse attention path here is single-GPU "
              "(no collectives); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import token_sparse_attention_jenga_amd as J
    from synth import config_by_name
    from synth.generate import make_layer, make_resid_dout, random_kept_blocks

    cfg = config_by_name(args.config)
    dev = torch.device("cuda:0")
    B, S, Hq, Hkv, D, blk = cfg.batch, cfg.seq_len, cfg.n_heads_q, cfg.n_heads_kv, cfg.head_dim, cfg.block
    nkb = S // blk
    L = cfg.n_layers
    nseg = args.segments or cfg.n_segments
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32

    # ---------------- inputs (seeded, generated on the host in parallel, then resident) ----
    t0 = time.time()
    with cf.ThreadPoolExecutor(max_workers=min(L, 8)) as ex:
        futs = [ex.submit(make_layer, cfg, l, None, False) for l in range(L)]
        x0_np, dout_np = make_resid_dout(cfg)
        layers_np = [f.result() for f in futs]
    layers = []
    for l, li in enumerate(layers_np):
        q = torch.from_numpy(li.q).to(dev).to(tdt)       # RNE cast on the device: same bits as
        k = torch.from_numpy(li.k).to(dev).to(tdt)       # the host-side rounding of the oracle
        v = torch.from_numpy(li.v).to(dev).to(tdt)
        layers.append({"q": q, "k": k, "v": v})
    gen_s = time.time() - t0
    x0 = torch.from_numpy(x0_np).to(dev)
    dout = torch.from_numpy(dout_np).to(dev)
    resid = x0.clone()
    sample_np = (layers_np[0].q[:, :, :8], layers_np[0].k[:, :, :8], layers_np[0].v[:, :, :8],
                 dout_np[:, :, :8])
    del layers_np, x0_np

    if cfg.select_mode == "topk":
        mode, maxk = J.JENGA_SELECT_TOPK, J.topk_count(cfg.select_param, nkb)
    else:
        mode, maxk = J.JENGA_SELECT_THRESH_REL, nkb
    flags = J.JENGA_FORCE_FIRST_BLOCK if cfg.force_first else 0
    ncap = maxk * blk
    for l, st in enumerate(layers):
        p = J.make_problem(st["q"], st["k"], st["v"], blk)
        st["p"] = p
        st["scores"] = torch.empty((B, nkb), dtype=torch.float32, device=dev)
        st["kept"] = torch.empty((B, nkb), dtype=torch.int32, device=dev)
        st["nk"] = torch.empty((B,), dtype=torch.int32, device=dev)
        st["o"] = torch.empty((B, ncap, Hq, D), dtype=tdt, device=dev)
        st["lse"] = torch.empty((B, Hq, ncap), dtype=torch.float32, device=dev)
        st["dq"] = torch.zeros((B, S, Hq, D), dtype=torch.float32, device=dev)
        st["dk"] = torch.zeros((B, S, Hkv, D), dtype=torch.float32, device=dev)
        st["dv"] = torch.zeros((B, S, Hkv, D), dtype=torch.float32, device=dev)
        if l == 0:   # one set of workspaces: the layers run one after another on one stream
            ws_s = J.alloc_workspace(J.workspace_bytes(p, J.JENGA_OP_SCORE), dev)
            ws_f = J.alloc_workspace(J.workspace_bytes(p, J.JENGA_OP_FWD, maxk), dev)
            ws_b = J.alloc_workspace(J.workspace_bytes(p, J.JENGA_OP_BWD, maxk, nseg), dev)
        st["ws_s"], st["ws_f"], st["ws_b"] = ws_s, ws_f, ws_b
        if args.kept == "scattered":
            kb = random_kept_blocks(nkb, maxk, 5999 + l)
            arr = np.full((B, nkb), -1, np.int32)
            arr[:, :maxk] = kb
            st["kept_att"] = torch.from_numpy(arr).to(dev)
            st["nk_att"] = torch.full((B,), maxk, dtype=torch.int32, device=dev)

    stream = torch.cuda.current_stream()

    def run_step(ev=None):
        for l, st in enumerate(layers):
            if ev is not None:
                ev[l][0].record(stream)
            J.jenga_score_blocks(st["p"], st["q"], st["k"], st["scores"], st["ws_s"])
            if ev is not None:
                ev[l][1].record(stream)
            J.jenga_select_blocks(st["p"], st["scores"], mode, cfg.select_param, flags, st["kept"], st["nk"])
            if ev is not None:
                ev[l][2].record(stream)
            ka, na = (st["kept_att"], st["nk_att"]) if args.kept == "scattered" else (st["kept"], st["nk"])
            J.jenga_sparse_attn_fwd(st["p"], st["q"], st["k"], st["v"], ka, na, maxk, resid, st["o"],
                                    st["lse"], st["ws_f"])
            if ev is not None:
                ev[l][3].record(stream)
        for l in reversed(range(L)):
            st = layers[l]
            ka, na = (st["kept_att"], st["nk_att"]) if args.kept == "scattered" else (st["kept"], st["nk"])
            if ev is not None:
                ev[l][4].record(stream)
            J.jenga_sparse_attn_bwd_segmented(st["p"], st["q"], st["k"], st["v"], ka, na, maxk, st["o"],
                                              st["lse"], dout, st["dq"], st["dk"], st["dv"], nseg,
                                              st["ws_b"])
            if ev is not None:
                ev[l][5].record(stream)

    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()
    nks = []
    for st in layers:
        na = st["nk_att"] if args.kept == "scattered" else st["nk"]
        nks.append([int(x) * blk for x in na.cpu().numpy()])

    K = args.steps
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(L)] for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # the timed steps carry only the per-layer phase events (6 per layer and step); the
    # library's per-kernel events are off here and run in a separate pass below
    J.timing_enable(False)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(K):
        run_step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / K
    phase = {"score": 0.0, "select": 0.0, "fwd": 0.0, "bwd": 0.0}
    for i in range(K):
        for l in range(L):
            e = evs[i][l]
            phase["score"] += e[0].elapsed_time(e[1])
            phase["select"] += e[1].elapsed_time(e[2])
            phase["fwd"] += e[2].elapsed_time(e[3])
            phase["bwd"] += e[4].elapsed_time(e[5])
    phase = {kk: vv / K for kk, vv in phase.items()}

    pairs = sum(nk * (nk + 1) / 2 for per in nks for nk in per)        # over layers and batch rows
    fwd_flop = 4.0 * D * Hq * pairs
    bwd_flop = 10.0 * D * Hq * pairs
    attn_ms = phase["fwd"] + phase["bwd"]
    tflops = (fwd_flop + bwd_flop) / (attn_ms * 1e-3) / 1e12
    score_flop = 2.0 * D * Hq * B * L * S * (S + 1) / 2       # one q.k per causal pair and head

    # Per-kernel times: the same K steps again, with the library's own HIP events around every
    # launch (recorded on the stream each kernel runs on).  Kept out of the headline steps above
    # so that the headline carries no per-launch instrumentation.
    torch.cuda.synchronize()
    J.timing_enable(True)
    inst0, inst1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    inst0.record(stream)
    for i in range(K):
        run_step()
    inst1.record(stream)
    J.timing_enable(False)
    torch.cuda.synchronize()
    inst_ms_per_step = inst0.elapsed_time(inst1) / K
    peak_steps = torch.cuda.max_memory_allocated()       # before any later section resets it

    # dominant attention kernel: k_bwd64 (one launch per backward segment, running the dK/dV
    # and dQ tiles of the segment).  Its algorithmic work, as the metric counts it, is the
    # backward's five 2*D contractions per (query head, causal kept pair): 10*D.  What it
    # executes is seven: the dK/dV tiles recompute the scores and form dP, dV and dK; the dQ
    # tiles recompute the scores and dP and form dQ (14*D), reported beside it.
    kern_ms = {}
    for name in KERNELS:
        n, t = J.timing_query(name)
        if n:
            kern_ms[name] = (n, t)
    n_bwd, t_bwd = kern_ms.get("k_bwd64", (0, 0.0))
    roofline = None
    if n_bwd:
        bwd_flop_launch = 10.0 * D * Hq * pairs * K / n_bwd
        exec_flop_launch = BWD_EXECUTED_D * D * Hq * pairs * K / n_bwd
        avg_ms = t_bwd / n_bwd
        achieved = bwd_flop_launch / (avg_ms * 1e-3) / 1e12
        executed = exec_flop_launch / (avg_ms * 1e-3) / 1e12
        traffic = None
        tfile = os.path.join(ROOT, "profiles", f"traffic_k_bwd64_{args.config}.json")
        if os.path.exists(tfile) and args.kept == "selected" and nseg == cfg.n_segments:
            with open(tfile) as f:
                tj = json.load(f)
            if tj.get("kernel_source_hash") == kernel_source_hash():
                traffic = tj.get("hbm_bytes_per_launch")
        roofline = {"kernel": "k_bwd64", "bound": "mfma", "achieved": round(achieved, 2),
                    "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                    "algorithmic_flop_per_launch": bwd_flop_launch, "launches": n_bwd,
                    "avg_launch_us": round(avg_ms * 1e3, 2),
                    "executed_flop_per_launch": exec_flop_launch,
                    "executed_tflops": round(executed, 2),
                    "executed_frac": round(executed / BF16_PEAK_TFLOPS, 4),
                    "timed_in": "a separate instrumented pass of the same steps "
                                f"({round(inst_ms_per_step, 3)} ms per step)"}
    kernel_avg_us = {kk: {"launches": n, "avg_us": round(1e3 * t / n, 2)} for kk, (n, t) in kern_ms.items()}

    # Eq. 2 literal scoring (the NEXT-row scoring mode), timed on its own after the steps: one
    # call per layer, MFMA work 2*D*Hq per element of every causal score block
    eq2 = None
    if cfg.dtype == "bf16" and blk in (64, 128):
        p0 = layers[0]["p"]
        ws_e = J.alloc_workspace(J.workspace_bytes(p0, J.JENGA_OP_SCORE_EQ2), dev)
        sc_e = torch.empty((B, nkb), dtype=torch.float32, device=dev)
        for st in layers:                                              # warm-up
            J.jenga_score_blocks_eq2(st["p"], st["q"], st["k"], sc_e, ws_e)
        torch.cuda.synchronize()
        J.timing_enable(True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(K):
            for st in layers:
                J.jenga_score_blocks_eq2(st["p"], st["q"], st["k"], sc_e, ws_e)
        e1.record(stream)
        J.timing_enable(False)
        torch.cuda.synchronize()
        eq2_ms = e0.elapsed_time(e1) / (K * L)
        eq2_flop = 2.0 * D * Hq * B * blk * blk * nkb * (nkb + 1) / 2
        n_t, t_t = J.timing_query("k_eq2_tiles")
        eq2 = {"ms_per_layer": round(eq2_ms, 4), "tflops": round(eq2_flop / (eq2_ms * 1e-3) / 1e12, 2),
               "pct_bf16_mfma_peak": round(100 * eq2_flop / (eq2_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 2),
               "k_eq2_tiles_avg_us": round(1e3 * t_t / max(n_t, 1), 2),
               "work": "2*D*Hq flop per element of every causal b x b score block"}
        del ws_e, sc_e

    # Permutation-free projections (the NEXT-row fusion of token movement into the linear
    # layers), at this workload's d_model = Hq*D with seeded synthetic bf16 weights: QKV
    # (d -> 3d) reads the kept rows of the hidden states, O (d -> d) adds into the residual in
    # place.  Timed per layer over each layer's own kept set.
    proj = None
    if cfg.dtype == "bf16" and (Hq * D) % 128 == 0:
        dm = Hq * D
        gen = torch.Generator(device=dev).manual_seed(4242)
        xh = torch.randn((B, S, dm), generator=gen, device=dev).to(torch.bfloat16)
        wqkv = (torch.randn((3 * dm, dm), generator=gen, device=dev) / dm ** 0.5).to(torch.bfloat16)
        wo = (torch.randn((dm, dm), generator=gen, device=dev) / dm ** 0.5).to(torch.bfloat16)
        yo = torch.randn((B, ncap, dm), generator=gen, device=dev).to(torch.bfloat16)
        res2 = resid.view(B, S, dm)
        for st in layers:                                              # warm-up
            J.proj_gather(xh, wqkv, st["kept"], st["nk"], maxk, blk)
            J.proj_scatter_add(yo, wo, st["kept"], st["nk"], maxk, blk, res2)
        torch.cuda.synchronize()
        J.timing_enable(True)
        for _ in range(K):
            for st in layers:
                J.proj_gather(xh, wqkv, st["kept"], st["nk"], maxk, blk)
                J.proj_scatter_add(yo, wo, st["kept"], st["nk"], maxk, blk, res2)
        J.timing_enable(False)
        torch.cuda.synchronize()
        rows = sum(nk for per in nks for nk in per) / L                  # kept rows per layer
        ng, tg = J.timing_query("k_proj_gather")
        ns, ts = J.timing_query("k_proj_scatter")
        g_ms, s_ms = tg / max(ng, 1), ts / max(ns, 1)
        g_tf = 2.0 * rows * dm * 3 * dm / (g_ms * 1e-3) / 1e12
        s_tf = 2.0 * rows * dm * dm / (s_ms * 1e-3) / 1e12
        proj = {"d_model": dm, "kept_rows_per_layer": rows,
                "qkv_gather_ms": round(g_ms, 4), "qkv_gather_tflops": round(g_tf, 2),
                "o_scatter_add_ms": round(s_ms, 4), "o_scatter_add_tflops": round(s_tf, 2),
                "pct_bf16_mfma_peak": round(100 * (2.0 * rows * dm * 4 * dm) /
                                            ((g_ms + s_ms) * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 2)}
        del xh, wqkv, wo, yo

    # Token elimination in the MLP block (NEXT row): a Llama-2-7B-shaped gated SiLU MLP
    # (d_model of this workload, 11008 units) over the B*S tokens with seeded synthetic bf16
    # weights: activation + token/block informativeness, selection at this workload's keep
    # rule, and the down projection of the kept tokens into the residual.
    mlp = None
    if cfg.dtype == "bf16" and (Hq * D) % 128 == 0:
        dm, F = Hq * D, 11008
        gen = torch.Generator(device=dev).manual_seed(99)
        xm = torch.randn((B, S, dm), generator=gen, device=dev).to(torch.bfloat16)
        wg = (torch.randn((F, dm), generator=gen, device=dev) / dm ** 0.5).to(torch.bfloat16)
        wu = (torch.randn((F, dm), generator=gen, device=dev) / dm ** 0.5).to(torch.bfloat16)
        wdn = (torch.randn((dm, F), generator=gen, device=dev) / F ** 0.5).to(torch.bfloat16)
        res2 = resid.view(B, S, dm)
        pm = J.make_proj_problem(xm, wg, xm.new_empty((B, S, F)), blk, S)
        ws_m = J.alloc_workspace(J.mlp_workspace_bytes(pm, J.JENGA_MLP_SILU_GATED), dev)
        J.sparse_mlp_forward(xm, wg, wu, wdn, res2, blk, mode, cfg.select_param, workspace=ws_m)
        torch.cuda.synchronize()
        J.timing_enable(True)
        nk_m = []
        for _ in range(K):
            _, _, nkm, _ = J.sparse_mlp_forward(xm, wg, wu, wdn, res2, blk, mode, cfg.select_param,
                                                workspace=ws_m)
            nk_m.append(nkm)
        J.timing_enable(False)
        torch.cuda.synchronize()
        kept_rows = float(torch.stack(nk_m).double().mean().item()) * blk * B
        na, ta = J.timing_query("k_mlp_act_gated")
        nb_, tb = J.timing_query("k_mlp_block")
        nd_, td = J.timing_query("k_proj_gather_scatter")
        a_ms, b_ms, d_ms = ta / max(na, 1), tb / max(nb_, 1), td / max(nd_, 1)
        a_tf = 2.0 * B * S * dm * 2 * F / (a_ms * 1e-3) / 1e12
        d_tf = 2.0 * kept_rows * F * dm / (d_ms * 1e-3) / 1e12
        mlp = {"d_model": dm, "units": F, "tokens": B * S, "kept_rows": kept_rows,
               "act_scores_ms": round(a_ms + b_ms, 4), "act_gemm_tflops": round(a_tf, 2),
               "block_scores_ms": round(b_ms, 4),
               "down_kept_ms": round(d_ms, 4), "down_kept_tflops": round(d_tf, 2),
               "pct_bf16_mfma_peak_act": round(100 * a_tf / BF16_PEAK_TFLOPS, 2)}
        del xm, wg, wu, wdn, ws_m

    # Segment-based peak cutting of the language-model-head loss (NEXT row): the head of this
    # workload's d_model over its B*S tokens and a 32000-entry vocabulary, seeded synthetic
    # bf16 weights and targets, in 1 and in 8 segments: time and the transient (workspace) bytes.
    loss_seg = None
    if cfg.dtype == "bf16" and (Hq * D) % 128 == 0 and (B * S) % 256 == 0:
        dm, V, T = Hq * D, 32000, B * S
        gen = torch.Generator(device=dev).manual_seed(777)
        hh = torch.randn((T, dm), generator=gen, device=dev).to(torch.bfloat16)
        wv = (torch.randn((V, dm), generator=gen, device=dev) / dm ** 0.5).to(torch.bfloat16)
        wvt = wv.t().contiguous()
        tg = torch.randint(0, V, (T,), generator=gen, device=dev, dtype=torch.int32)
        loss_seg = {"tokens": T, "d_model": dm, "vocab": V}
        for nseg_l in (1, 8):
            pl = J.loss_problem(T, dm, V, nseg_l)
            # transient: the allocator's peak during one call (the call allocates its workspace
            # and outputs from torch) minus what stays allocated after it (the outputs)
            torch.cuda.synchronize()
            base_l = torch.cuda.memory_allocated()
            torch.cuda.reset_peak_memory_stats()
            outs_l = J.lm_head_ce(hh, wv, wvt, tg, nseg_l)
            torch.cuda.synchronize()
            transient_l = torch.cuda.max_memory_allocated() - torch.cuda.memory_allocated()
            outputs_l = torch.cuda.memory_allocated() - base_l
            del outs_l
            ws_l = J.alloc_workspace(J.loss_workspace_bytes(pl), dev)
            J.lm_head_ce(hh, wv, wvt, tg, nseg_l, ws_l)                  # warm-up
            torch.cuda.synchronize()
            l0, l1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            l0.record(stream)
            for _ in range(K):
                J.lm_head_ce(hh, wv, wvt, tg, nseg_l, ws_l)
            l1.record(stream)
            torch.cuda.synchronize()
            ms = l0.elapsed_time(l1) / K
            loss_seg[f"segments_{nseg_l}"] = {
                "ms": round(ms, 3), "tflops": round(4.0 * T * dm * V / (ms * 1e-3) / 1e12, 2),
                "transient_mib": round(transient_l / 2**20, 1),
                "outputs_mib": round(outputs_l / 2**20, 1)}
            del ws_l
        del hh, wv, wvt, tg

    copy_ms = None
    if args.copy_calibration:
        # plain elementwise copy (16-byte vector loads/stores), 1 GiB read + 1 GiB written
        a = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        bcopy = torch.empty_like(a)
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        torch.neg(a, out=bcopy)
        c1.record(stream)
        torch.cuda.synchronize()
        copy_ms = c0.elapsed_time(c1)
        del a, bcopy

    mem = {"max_allocated_gib": round(peak_steps / 2**30, 2),
           "saved_activations_mib_per_layer": round(
               (B * ncap * Hq * D * (2 if cfg.dtype == "bf16" else 4) + B * Hq * ncap * 4 + B * nkb * 4) / 2**20, 2),
           "fwd_workspace_mib": round(layers[0]["ws_f"].numel() / 2**20, 2),
           "bwd_workspace_mib": round(layers[0]["ws_b"].numel() / 2**20, 2)}

    # Per-step evidence beside the metric: the exponentials per second of scoring (one exp per
    # causal pair per query head, in the row pass; the block-mass pass adds one per query and
    # key block, not counted), and the backward prologue's
    # bytes per second (per kept query row and head: dOut row fp32 and o_saved row in, lse in;
    # D, lse2, the dOut row in operand dtype and its transposed copy out).
    es = 2 if cfg.dtype == "bf16" else 4
    score_exps = 1.0 * Hq * B * L * S * (S + 1) / 2
    step_evidence = {"score_exp_per_s": round(score_exps / (phase["score"] * 1e-3), 1)}
    n_prep, t_prep = kern_ms.get("k_prep64", (0, 0.0))
    if n_prep:
        prep_bytes = float(sum(sum(per) for per in nks)) * Hq * (4 * D + 2 * es * D + es * D + 12) / n_prep * K
        step_evidence["prep_gbs"] = round(prep_bytes / (t_prep / n_prep * 1e-3) / 1e9, 1)

    # The same fwd+bwd over the layers with a seeded scattered kept set per layer (the selected
    # sets of this workload come out nearly contiguous): same kept count, so the same FLOPs.
    scattered = None
    if args.kept == "selected" and cfg.select_mode == "topk":
        for l, st in enumerate(layers):
            kb = random_kept_blocks(nkb, maxk, 5999 + l)
            arr = np.full((B, nkb), -1, np.int32)
            arr[:, :maxk] = kb
            st["kept_sc"] = torch.from_numpy(arr).to(dev)
            st["nk_sc"] = torch.full((B,), maxk, dtype=torch.int32, device=dev)

        def attn_pass():
            for st in layers:
                J.jenga_sparse_attn_fwd(st["p"], st["q"], st["k"], st["v"], st["kept_sc"], st["nk_sc"], maxk,
                                        resid, st["o"], st["lse"], st["ws_f"])
            for l in reversed(range(L)):
                st = layers[l]
                J.jenga_sparse_attn_bwd_segmented(st["p"], st["q"], st["k"], st["v"], st["kept_sc"],
                                                  st["nk_sc"], maxk, st["o"], st["lse"], dout, st["dq"],
                                                  st["dk"], st["dv"], nseg, st["ws_b"])
        attn_pass()
        torch.cuda.synchronize()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(1, min(K, 3))
        s0.record(stream)
        for _ in range(reps):
            attn_pass()
        s1.record(stream)
        torch.cuda.synchronize()
        sc_ms = s0.elapsed_time(s1) / reps
        sc_pairs = L * B * (maxk * blk) * (maxk * blk + 1) / 2
        scattered = {"kept": f"default_rng(5999 + layer) choice of {maxk} of {nkb} blocks, sorted",
                     "attn_ms_per_step": round(sc_ms, 3),
                     "tflops": round(14.0 * D * Hq * sc_pairs / (sc_ms * 1e-3) / 1e12, 2)}

    # Memory at this workload's shapes, one layer, over keep ratios and segment counts, measured
    # with torch's allocator counters around the calls (every buffer comes from torch; the
    # library allocates nothing): the forward's peak (saved activations + its workspace), the
    # activations it leaves for the backward (o_saved, lse, the kept list), and the backward's
    # transient peak.  Q/K/V, the residual and the gradients are caller-owned and excluded.
    memory_sweep = []
    if cfg.dtype == "bf16":
        st0 = layers[0]
        dq_m = torch.zeros_like(st0["dq"])
        dk_m = torch.zeros_like(st0["dk"])
        dv_m = torch.zeros_like(st0["dv"])
        res_m = x0.clone()
        mib = lambda x: round(x / 2**20, 2)
        for r in (0.125, 0.25, 0.5, 0.75, 1.0):
            kk = J.topk_count(r, nkb)
            kb_np = np.full((B, nkb), -1, np.int32)
            kb_np[:, :kk] = random_kept_blocks(nkb, kk, 7000 + kk)
            for nn in (1, 8):
                torch.cuda.synchronize()
                base = torch.cuda.memory_allocated()
                torch.cuda.reset_peak_memory_stats()
                kept_m = torch.from_numpy(kb_np).to(dev)
                nk_m = torch.full((B,), kk, dtype=torch.int32, device=dev)
                o_m, lse_m = J.sparse_attn_fwd(st0["q"], st0["k"], st0["v"], kept_m, nk_m, kk, blk, res_m)
                torch.cuda.synchronize()
                fwd_peak = torch.cuda.max_memory_allocated() - base
                saved = torch.cuda.memory_allocated() - base
                torch.cuda.reset_peak_memory_stats()
                base2 = torch.cuda.memory_allocated()
                J.sparse_attn_bwd(st0["q"], st0["k"], st0["v"], kept_m, nk_m, kk, blk, o_m, lse_m, dout,
                                  n_segments=nn, grads=(dq_m, dk_m, dv_m))
                torch.cuda.synchronize()
                bwd_peak = torch.cuda.max_memory_allocated() - base2
                # the same backward with one set of segment buffers (each prologue a launch of
                # its own): the least transient the backward runs with
                torch.cuda.reset_peak_memory_stats()
                base3 = torch.cuda.memory_allocated()
                J.sparse_attn_bwd(st0["q"], st0["k"], st0["v"], kept_m, nk_m, kk, blk, o_m, lse_m, dout,
                                  n_segments=nn, grads=(dq_m, dk_m, dv_m), min_workspace=True)
                torch.cuda.synchronize()
                bwd_peak_min = torch.cuda.max_memory_allocated() - base3
                memory_sweep.append({
                    "keep": r, "n_segments": nn, "kept_tokens": B * kk * blk,
                    "fwd_peak_mib": mib(fwd_peak), "saved_activation_mib": mib(saved),
                    "bwd_transient_mib": mib(bwd_peak), "bwd_transient_min_mib": mib(bwd_peak_min)})
                del kept_m, nk_m, o_m, lse_m
        del dq_m, dk_m, dv_m, res_m

    # ---------------- CPU baseline: the oracle on a bounded sample of the same workload ----
    cpu = None
    if not args.no_cpu_baseline:
        sel_mode = {"topk": 0, "thresh_rel": 1}[cfg.select_mode]
        cpu = cpu_baseline(cfg, sample_np, layers[0]["scores"].cpu().numpy(),
                           (sel_mode, cfg.select_param, cfg.force_first))

    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: S={S} B={B} Hq={Hq} Hkv={Hkv} D={D} block={blk} "
                               f"{cfg.select_mode} {cfg.select_param} layers={L} segments={nseg} "
                               f"kept={args.kept}",
                   "global_batch": B, "seq_len": S, "parallelism": "single-gpu"},
        "pct_bf16_mfma_peak": round(100 * tflops / BF16_PEAK_TFLOPS, 2),
        "attn_ms_per_step": round(attn_ms, 3),
        "tokens_per_s_attn": round(B * S / (attn_ms * 1e-3), 1),
        "tokens_per_s_pipeline": round(B * S / (ms_per_step * 1e-3), 1),
        "phase_ms_per_step": {kk: round(vv, 3) for kk, vv in phase.items()},
        "fwd_tflops": round(fwd_flop / (phase["fwd"] * 1e-3) / 1e12, 2),
        "bwd_tflops": round(bwd_flop / (phase["bwd"] * 1e-3) / 1e12, 2),
        "score_tflops_algorithmic": round(score_flop / (phase["score"] * 1e-3) / 1e12, 2),
        "kept_tokens_per_layer": nks,
        "eq2_scoring": eq2,
        "proj_fused": proj,
        "loss_segmented": loss_seg,
        "mlp_elimination": mlp,
        "roofline": roofline,
        "kernel_avg_us": kernel_avg_us,
        "cpu_baseline": cpu,
        "memory": mem,
        "memory_sweep": memory_sweep,
        "step_evidence": step_evidence,
        "scattered_kept": scattered,
        "input_gen_s": round(gen_s, 1),
    }
    if copy_ms is not None:
        out["copy_calibration"] = {"kernel": "elementwise neg, float32, 1 GiB in + 1 GiB out",
                                   "ms": round(copy_ms, 4),
                                   "gbs": round(2 * 2**30 / (copy_ms * 1e-3) / 1e9, 1)}
    print(json.dumps(out), flush=True)


def host_facts():
    """The host the oracle baseline ran on: logical CPUs, the CPUs this process may use,
    physical cores and model (lscpu), and the BLAS thread count NumPy's BLAS runs with."""
    import subprocess
    facts = {"os_cpu_count": os.cpu_count()}
    try:
        facts["usable_cpus"] = len(os.sched_getaffinity(0))
    except Exception:
        pass
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        kv = {}
        for line in out.splitlines():
            if ":" in line:
                a, b = line.split(":", 1)
                kv[a.strip()] = b.strip()
        facts["cpu_model"] = kv.get("Model name")
        if kv.get("Core(s) per socket") and kv.get("Socket(s)"):
            facts["physical_cores"] = int(kv["Core(s) per socket"]) * int(kv["Socket(s)"])
        if kv.get("Thread(s) per core"):
            facts["threads_per_core"] = int(kv["Thread(s) per core"])
    except Exception:
        pass
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"] + [0])
    except Exception:
        pass
    facts["blas_threads"] = threads or None
    facts["omp_num_threads"] = os.environ.get("OMP_NUM_THREADS")
    return facts


def cpu_baseline(cfg, sample, scores0, select_args, budget_s: float = 12.0, score_budget_s: float = 5.0):
    """The oracle as written (float64 NumPy, BLAS threaded over the host cores) timed per op on
    bounded samples of this workload's layer 0:
      score:  block scores of a causal prefix of min(S, 4096) tokens, one query head after
              another for about score_budget_s seconds;
      select: the selection rule on the GPU's scores of layer 0 (all blocks);
      fwd, bwd: attention forward and backward over kept blocks 0..k-1 (a self-contained causal
              prefix of the literal top-k set's size), one query head after another until
              about budget_s seconds have been spent.
    `value` is fwd+bwd TFLOP/s on the metric's kept-FLOP count."""
    import oracle
    from synth.generate import to_bf16_bits_f32
    q_all, k_all, v_all, dout_all = sample
    host = host_facts()
    bf = (lambda a: to_bf16_bits_f32(a)) if cfg.dtype == "bf16" else (lambda a: a)
    G = cfg.n_heads_q // cfg.n_heads_kv
    kv_of = lambda h: min(h // G, k_all.shape[2] - 1)
    prep = lambda a, S_s, i: np.ascontiguousarray(a[:, :S_s, i:i + 1])
    D, B = cfg.head_dim, cfg.batch

    # score
    S_sc = min(cfg.seq_len, 4096)
    hs, t_sc = 0, 0.0
    while hs < q_all.shape[2] and t_sc < score_budget_s:
        q, k = bf(prep(q_all, S_sc, hs)), bf(prep(k_all, S_sc, kv_of(hs)))
        t0 = time.time()
        oracle.block_scores(q, k, cfg.block)
        t_sc += time.time() - t0
        hs += 1
    score_flop = 2.0 * D * hs * B * S_sc * (S_sc + 1) / 2

    # select
    mode, param, ff = select_args
    reps, t0 = 0, time.time()
    while reps < 20 or time.time() - t0 < 0.2:
        for b in range(scores0.shape[0]):
            oracle.select_blocks(scores0[b], mode, param, ff)
        reps += 1
    t_sel = (time.time() - t0) / reps

    # fwd, bwd
    nb = min(cfg.n_blocks, 128)
    S_s = nb * cfg.block
    kept = np.arange(nb)
    heads, t_f, t_b = 0, 0.0, 0.0
    while heads < q_all.shape[2] and t_f + t_b < budget_s:
        h = heads
        q, k, v = bf(prep(q_all, S_s, h)), bf(prep(k_all, S_s, kv_of(h))), bf(prep(v_all, S_s, kv_of(h)))
        dout = prep(dout_all, S_s, h)
        t0 = time.time()
        oracle.attn_fwd_compact(q, k, v, kept, cfg.block)
        t1 = time.time()
        oracle.attn_bwd_compact(q, k, v, kept, cfg.block, dout)
        t2 = time.time()
        t_f += t1 - t0
        t_b += t2 - t1
        heads += 1
    pairs = B * S_s * (S_s + 1) / 2
    fwd_flop, bwd_flop = 4.0 * D * heads * pairs, 10.0 * D * heads * pairs
    return {"value": round((fwd_flop + bwd_flop) / (t_f + t_b) / 1e12, 5), "unit": "TFLOP/s",
            "cores": int(host.get("blas_threads") or host.get("usable_cpus") or os.cpu_count()),
            "kind": "oracle", "seconds": round(t_sc + t_f + t_b + t_sel * reps, 2),
            "sample": f"layer 0; fwd+bwd: query heads 0..{heads - 1}, kept blocks 0..{nb - 1} ({S_s} kept "
                      f"tokens, a self-contained causal prefix), float64 NumPy",
            "per_op": {
                "score": {"seconds": round(t_sc, 3), "gflops": round(score_flop / t_sc / 1e9, 3),
                          "sample": f"query heads 0..{hs - 1}, causal prefix of {S_sc} tokens",
                          "work": "2*D flop per causal (query, key) pair and head"},
                "select": {"us_per_call": round(1e6 * t_sel, 1), "n_blocks": int(scores0.shape[1]),
                           "batch_rows": int(scores0.shape[0])},
                "fwd": {"seconds": round(t_f, 3), "gflops": round(fwd_flop / t_f / 1e9, 3)},
                "bwd": {"seconds": round(t_b, 3), "gflops": round(bwd_flop / t_b / 1e9, 3)}},
            "host": host}


if __name__ == "__main__":
    main()

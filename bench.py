"""Benchmark of the Prism dynamic block-sparse attention hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 2k] [--no-cpu-baseline]
    python bench.py --profile profiles     # rocprofv3 passes -> text summaries

One step is one pass of the whole hot path over one batch of synthetic input
resident in HBM: zone statistics and shapes, block-major permutation of Q, K,
V and dO, pooled scoring and hybrid top-k/top-p selection, sparse attention
forward and backward, and the inverse permutation of O, dQ, dK and dV.

The headline value is the effective sparse-attention throughput of the whole
step: F_eff = sum over heads, query blocks i and selected key blocks j of
14 * B_i * B_j * d (4 for the forward, 10 for the backward; executed blocks
only), divided by the step time.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import re
import subprocess
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective sparse-attn TFLOP/s fwd+bwd at 2K tokens; % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
CSRC = os.path.join(ROOT, "dynamic_block_sparse_amd", "csrc")
# kernels launched by one tile-order build, one prism_sparse_attn_fwd and one
# prism_sparse_attn_bwd call, with their launch counts (csr_scan and fill_i32
# also run elsewhere, always over the same heads x blocks shape)
# (one head group: the workload's heads fit the library's default group)
SPLIT_KERNELS = {"fill_i32_kernel": 3, "csr_scan_kernel": 2, "split_cost_kernel": 1, "split_pick_kernel": 1,
                 "split_rows_kernel": 1, "split_count_kernel": 1, "split_fill_kernel": 1}
ORDER_KERNELS = {"fill_i32_kernel": 2, "order_count_kernel": 1, "csr_scan_kernel": 1, "order_fill_kernel": 1}


def _merge(*ds, **kw):
    out = {}
    for d in ds + (kw,):
        for k, v in d.items():
            out[k] = out.get(k, 0) + v
    return out


FWD_KERNELS = _merge(SPLIT_KERNELS, ORDER_KERNELS, attn_fwd_mfma_kernel=1, attn_fwd_chunk_kernel=1,
                     attn_fwd_combine_kernel=1)
BWD_KERNELS = _merge(SPLIT_KERNELS, ORDER_KERNELS, {"attn_bwd_dot_kernel": 1, "fill_i32_kernel": 2,
                                                    "tr_count_kernel": 1, "csr_scan_kernel": 1, "tr_fill_kernel": 1,
                                                    "tr_sort_kernel": 1},
                     attn_dq_mfma_kernel=1, attn_dq_chunk_kernel=1, attn_dq_combine_kernel=1, attn_dkdv_mfma_kernel=1)
PMC_REGEX = ("attn_|split_|permute_heads|tr_count|tr_fill|tr_sort|csr_scan|order_|fill_i32|zone_profile|pool_kernel|"
             "logits_kernel|select_reg|select_write")
ATTN_REGEX = "attn_(fwd|dq|dkdv)_(mfma|chunk)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="2k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip the measurements of the next rows (the profile passes use this)")
    ap.add_argument("--flat-ratio", type=float, default=0.5,
                    help="flat ratio of the routed-forward measurement (next row f3)")
    ap.add_argument("--profile", metavar="DIR", help="run the rocprofv3 passes and write summaries into DIR")
    ap.add_argument("--calibrate", action="store_true",
                    help="only run the two counter calibration kernels once (the profile passes use this)")
    return ap.parse_args()


def calibrate(cfg):
    """The two kernels the HBM counters are calibrated on, one launch each, on
    one tensor of the workload's size ([N, heads, d]): the permutation of a
    raster tensor into block-major order (streaming reads and writes) and a
    torch gather of its 64-row tiles in random order (16 KB runs, as the
    attention kernels load them).  Each reads and writes the tensor once."""
    from dynamic_block_sparse_amd.path import PrismPath
    from workloads.synth import make_inputs
    x = make_inputs(cfg, device="cuda", tensors=("v",))
    path = PrismPath(cfg.T, cfg.H, cfg.W, cfg.heads, cfg.d, cfg.top_k, cfg.top_p, 1.0)
    path.shapes(x["v"], x["a"])
    t = path.block_major_like(x["v"])
    torch.cuda.synchronize()
    path.permute(x["v"], out=t)
    tiles = x["v"].reshape(-1, 64 * cfg.d)              # [N * heads / 64, 64 rows of one head]
    idx = torch.randperm(tiles.shape[0], device="cuda")
    torch.cuda.synchronize()
    g = torch.index_select(tiles, 0, idx)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_bytes_each_way": int(x["v"].numel() * x["v"].element_size()),
                      "gather_rows": int(g.shape[0]), "gather_row_bytes": int(g.shape[1] * g.element_size())}),
          flush=True)


def source_hash():
    """sha256 over the HIP/C++ sources: a counter summary is only used while it matches."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(CSRC, "*"))):
        if f.endswith((".hip", ".cpp", ".hpp", ".h")):
            h.update(os.path.basename(f).encode())
            with open(f, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def traffic_file(cfg_name):
    return os.path.join(ROOT, "profiles", f"attn_bwd_{cfg_name}_traffic.txt")


def read_traffic(cfg_name):
    """HBM-side bytes per backward call from the committed counter summary, or
    None when there is none or the kernels changed since it was taken."""
    f = traffic_file(cfg_name)
    if not os.path.exists(f):
        return None
    kv = {}
    for line in open(f):
        m = re.match(r"^([a-z0-9_]+):\s*(\S+)", line)
        if m:
            kv[m.group(1)] = m.group(2)
    if kv.get("source_sha256") != source_hash() or "bytes_per_call" not in kv:
        return None
    return float(kv["bytes_per_call"])


def effective_flops(path, sels, d):
    """F_eff from the selected sets (bookkeeping on the CSR, not part of the path)."""
    offs = path.block_offsets[:path.nb + 1].to(torch.int64)
    B = (offs[1:] - offs[:-1]).to(torch.float64)
    pairs = 0.0
    sizes = []
    for sel in sels:
        for h in range(sel.offsets.shape[0]):
            tot = int(sel.total[h])
            idx = sel.idx[h, :tot].to(torch.int64)
            o = sel.offsets[h].to(torch.int64)
            cs = torch.cat([torch.zeros(1, dtype=torch.float64, device=B.device), torch.cumsum(B[idx], 0)])
            keys_per_row = cs[o[1:]] - cs[o[:-1]]
            pairs += float((B * keys_per_row).sum())
            sizes.append((o[1:] - o[:-1]).double().mean().item())
    return 4.0 * pairs * d, 10.0 * pairs * d, float(np.mean(sizes))


def cpu_baseline(cfg, x, zone_shape_host, budget_s):
    """The float64 oracle, as it stands, on a bounded sample of the same
    workload: attention forward and backward of head 0 for query blocks taken
    in a seeded random order until the time budget is spent."""
    from oracle import prism_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = 1
    sc = float(np.float32(1.0 / math.sqrt(cfg.d)))
    pi = orc.permutation(cfg.T, cfg.H, cfg.W, zone_shape_host)
    offs, NB = orc.block_layout(zone_shape_host)
    names = ("q", "k", "v", "do") if cfg.backward else ("q", "k", "v")
    Qp, Kp, Vp, *rest = (orc.to_block_major(x[n][:, 0:1, :].float().cpu().numpy(), pi) for n in names)
    dOp = rest[0] if rest else None
    per_pair = 14.0 if cfg.backward else 4.0
    t0 = time.perf_counter()
    Kb = orc.pool_blocks(Kp, offs, 0)
    Qb = orc.pool_blocks(Qp, offs, 0)
    order = np.random.default_rng(0).permutation(NB)
    flops = 0.0
    nblocks = 0
    for i in order:
        L = orc.block_logits(Qb[i:i + 1], Kb, sc)[0]
        sel, _ = orc.select_row(L, cfg.top_k, cfg.top_p)
        orc.attn_fwd_block(Qp, Kp, Vp, offs, sel, i, 0, sc)
        if cfg.backward:
            orc.attn_bwd_block(Qp, Kp, Vp, dOp, offs, sel, i, 0, sc)
        Bi = offs[i + 1] - offs[i]
        flops += per_pair * Bi * float(sum(offs[j + 1] - offs[j] for j in sel)) * cfg.d
        nblocks += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"float64 oracle pooling of head 0 (all {NB} blocks) then per query block: scores, "
                      f"selection, attention forward{' and backward' if cfg.backward else ''}, for {nblocks} "
                      f"query blocks of head 0 in seeded random order ({dt:.1f} s)"}


def _run(cmd, log, limit):
    print("[profile] " + " ".join(cmd), file=sys.stderr, flush=True)
    with open(log, "w") as fh:
        r = subprocess.run(cmd, stdout=fh, stderr=subprocess.STDOUT, timeout=limit)
    if r.returncode != 0:
        sys.exit(f"[profile] failed with status {r.returncode}; see {log}")
    return [l for l in open(log) if l.startswith("{")]


def _counter_rows(root):
    rows = []
    for f in glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    per = {}
    for r in rows:
        key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"] or 0)
    return sorted(per.items())


def _short(name):
    name = name.replace("(anonymous namespace)::", "")
    return re.sub(r"\(.*", "", name).replace("void ", "").replace("prism::", "")


def _ours(name):
    """A kernel of libprism (namespace prism), as opposed to torch's."""
    return re.match(r"(void )?prism::", name) is not None


def profile(args):
    """rocprofv3 passes over this bench (kernel trace, FETCH_SIZE, WRITE_SIZE),
    summarised as text into the --profile folder; the raw rocprofv3 output goes
    to profile_raw beside it.  The GPU is only used by the child processes."""
    out = args.profile
    os.makedirs(out, exist_ok=True)
    raw = os.path.join(os.path.dirname(os.path.abspath(out)), "profile_raw")
    os.makedirs(raw, exist_ok=True)
    me = [sys.executable, "-u", os.path.abspath(__file__), "--config", args.config, "--no-cpu-baseline",
          "--no-next-rows"]
    rel = lambda p: os.path.relpath(p, ROOT)
    # library switches in effect (the child processes inherit them)
    env = " ".join(f"{k}={v}" for k, v in sorted(os.environ.items()) if k.startswith("PRISM_"))
    made_by = (env + " " if env else "") + f"python bench.py --profile {out} --config {args.config}"

    def cmd_for(prof, steps, warmup):
        run = ["--steps", str(steps), "--warmup", str(warmup)]
        return prof + ["--"] + me + run, " ".join(prof + ["--", "python", "bench.py", "--config", args.config,
                                                         "--no-cpu-baseline", "--no-next-rows"] + run)

    tdir = os.path.join(raw, "trace")
    tcmd, tshow = cmd_for(["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d", tdir, "-o",
                           "trace"], 3, 1)
    tshow = tshow.replace(tdir, rel(tdir))
    lines = _run(tcmd, os.path.join(raw, "trace.log"), 600)
    bench_line = json.loads(lines[-1]) if lines else {}
    stats = glob.glob(os.path.join(raw, "trace", "**", "*kernel_stats.csv"), recursive=True)
    rows = list(csv.DictReader(open(stats[0])))
    avg = {_short(r["Name"]): float(r["AverageNs"]) for r in rows}
    fwd_ns = sum(v * FWD_KERNELS.get(k.split("<")[0], 0) for k, v in avg.items())
    bwd_ns = sum(v * BWD_KERNELS.get(k.split("<")[0], 0) for k, v in avg.items())
    with open(os.path.join(out, f"attn_{args.config}_kernel_stats.txt"), "w") as fh:
        fh.write(f"# rocprofv3 kernel statistics, {args.config} workload, 4 steps (1 warm-up)\n")
        fh.write("# command: " + tshow + "\n")
        fh.write(f"# made by: {made_by}\n\n")
        fh.write(f"{'kernel':62s} {'calls':>6s} {'avg_ms':>10s} {'total_ms':>10s} {'pct':>6s}\n")
        other = [0, 0.0, 0.0]
        for r in rows:
            name = _short(r["Name"])
            if not _ours(r["Name"]):
                other[0] += int(r["Calls"])
                other[1] += float(r["TotalDurationNs"])
                other[2] += float(r["Percentage"])
                continue
            fh.write(f"{name[:62]:62s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e6:10.3f} "
                     f"{float(r['TotalDurationNs']) / 1e6:10.3f} {float(r['Percentage']):6.2f}\n")
        fh.write(f"{'other (torch: synthetic inputs and bookkeeping, outside the timed path)':62s} {other[0]:6d} "
                 f"{'':>10s} {other[1] / 1e6:10.3f} {other[2]:6.2f}\n")
        fh.write(f"\nprism_sparse_attn_fwd call (its kernels' average durations x launches): {fwd_ns / 1e6:.3f} ms\n")
        fh.write(f"prism_sparse_attn_bwd call (its kernels' average durations x launches): {bwd_ns / 1e6:.3f} ms\n")
        if bench_line:
            fh.write(f"bench stage_ms of the same run (HIP events): {json.dumps(bench_line.get('stage_ms'))}\n")
    # calibration: both counters over the two calibration kernels (one launch
    # each, a process of their own)
    import workloads.synth as synth
    cfg = synth.CONFIGS[args.config]
    es = 2 if cfg.dtype == "bf16" else 4
    copy_bytes = cfg.N * cfg.heads * cfg.d * es   # each calibration kernel reads and writes one whole tensor
    cal_regex = "permute_heads|gather|index_select"
    cal = {}
    cal_cmds = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        d = os.path.join(raw, "cal_" + ctr.lower())
        cmd = ["rocprofv3", "--pmc", ctr, "--kernel-include-regex", cal_regex, "--output-format", "csv", "-d", d,
               "-o", "cal", "--", sys.executable, "-u", os.path.abspath(__file__), "--config", args.config,
               "--calibrate"]
        cal_cmds[ctr] = (f"rocprofv3 --pmc {ctr} --kernel-include-regex '{cal_regex}' --output-format csv -d {rel(d)} "
                         f"-o cal -- python bench.py --config {args.config} --calibrate")
        _run(cmd, d + ".log", 300)
        rows_ = _counter_rows(d)
        ip = [i for i, ((_, k), _) in enumerate(rows_) if "permute_heads" in k]
        # the calibration gather: every gather launch after the permutation
        # (torch may split it; the input generation's own gathers come before)
        gath = [v for (_, k), v in rows_[ip[-1] + 1:] if "gather" in k or "index_select" in k] if ip else []
        if not ip or not gath:
            sys.exit("[profile] the calibration run did not record both calibration kernels")
        cal[ctr] = {"permute": copy_bytes / (1024.0 * rows_[ip[-1]][1]), "gather": copy_bytes / (1024.0 * sum(gath))}
    # counters: one pass each
    res = {}
    pcmds = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        d = os.path.join(raw, ctr.lower())
        cmd, show = cmd_for(["rocprofv3", "--pmc", ctr, "--kernel-include-regex", PMC_REGEX, "--output-format", "csv",
                             "-d", d, "-o", ctr.lower()], 1, 0)
        pcmds[ctr] = show.replace(d, rel(d)).replace(PMC_REGEX, "'" + PMC_REGEX + "'")
        _run(cmd, d + ".log", 300)
        rows_ = _counter_rows(d)
        # the timed step's dispatches: from its zone statistics on (the set-up
        # before it also computes the shapes and a sizing selection)
        first = max(i for i, ((_, k), _) in enumerate(rows_) if "zone_profile" in k)
        res[ctr] = rows_[first:]
    # the scale of each counter: algorithmic / counted bytes on the permutation
    # kernel; the gather's factor is recorded beside it as a check
    scale = {ctr: cal[ctr]["permute"] for ctr in cal}

    def call_range(seq, first, last, after=None):
        """dispatches of one call: from the last `first` kernel (or, with
        `after`, the one following the last `after` kernel before it) through
        the last `last` kernel"""
        end = max(i for i, (k, _) in enumerate(seq) if last in k)
        if after is None:
            start = max(i for i, (k, _) in enumerate(seq[:end + 1]) if first in k)
        else:
            start = max(i for i, (k, _) in enumerate(seq[:end + 1]) if after in k) + 1
        return seq[start:end + 1]

    calls = {"bwd": {}, "fwd": {}}
    for ctr, rows_ in res.items():
        seq = [(k, v) for (_, k), v in rows_]
        calls["bwd"][ctr] = [(_short(k), v) for k, v in call_range(seq, "attn_bwd_dot", "attn_dkdv")]
        # the forward call: everything after the selection's last CSR write up
        # to the forward's last attention kernel
        fwd_last = "attn_fwd_combine" if any("attn_fwd_combine" in k for k, _ in seq) else "attn_fwd_mfma"
        calls["fwd"][ctr] = [(_short(k), v) for k, v in call_range(seq, None, fwd_last, after="select_write")]
    fetch = write = 0.0
    for which, per_call in calls.items():
        f_b = sum(v for _, v in per_call["FETCH_SIZE"]) * 1024 * scale["FETCH_SIZE"]
        w_b = sum(v for _, v in per_call["WRITE_SIZE"]) * 1024 * scale["WRITE_SIZE"]
        if which == "bwd":
            fetch, write = f_b, w_b
        api = "prism_sparse_attn_bwd" if which == "bwd" else "prism_sparse_attn_fwd"
        with open(os.path.join(out, f"attn_{which}_{args.config}_traffic.txt"), "w") as fh:
            fh.write(f"# HBM-side traffic of one {api} call, {args.config} workload, from rocprofv3 counters\n")
            for ctr, show in pcmds.items():
                fh.write(f"# {ctr} pass: {show}\n")
            for ctr, show in cal_cmds.items():
                fh.write(f"# {ctr} calibration pass: {show}\n")
            fh.write(f"# made by: {made_by}\n")
            fh.write(f"# calibration: each calibration kernel reads and writes {copy_bytes} bytes (one tensor); the\n"
                     f"# counters (KiB per dispatch) are scaled by algorithmic/counted on the permutation kernel\n"
                     f"# (streaming); a gather of the tensor's 16 KB tiles in random order, the attention kernels'\n"
                     f"# access pattern, gives the check factor beside it\n\n")
            for ctr in cal:
                fh.write(f"scale_{ctr.lower()}: {scale[ctr]:.4f}\n")
                fh.write(f"check_scale_{ctr.lower()}_gather: {cal[ctr]['gather']:.4f}\n")
            for ctr, items in per_call.items():
                for k, v in items:
                    fh.write(f"  {ctr} {k}: {v:.0f} KiB\n")
            fh.write(f"fetch_bytes_per_call: {f_b:.6g}\n")
            fh.write(f"write_bytes_per_call: {w_b:.6g}\n")
            fh.write(f"bytes_per_call: {f_b + w_b:.6g}\n")
            fh.write(f"source_sha256: {source_hash()}\n")
    # the bandwidth-bound stages from the same two passes: bytes per dispatch,
    # counted (scaled as above) against algorithmic
    nb_run = int(bench_line.get("config", {}).get("blocks", 0)) if bench_line else 0
    C = cfg.heads * cfg.d
    stage_alg = {"zone_profile": ("zone statistics: read V, the a map", cfg.N * C * es + 4 * cfg.N),
                 "permute_heads": ("permutation of one tensor: read + write", 2 * cfg.N * C * es),
                 "pool_kernel": ("block means: read Q and K", 2 * cfg.N * C * es),
                 "logits_kernel": ("scores: write fp32 [NB, NB] per head", cfg.heads * nb_run * nb_run * 4),
                 "select_reg": ("selection: read the scores", cfg.heads * nb_run * nb_run * 4),
                 "select_write": ("CSR write: read the scores", cfg.heads * nb_run * nb_run * 4)}
    with open(os.path.join(out, f"stages_{args.config}_traffic.txt"), "w") as fh:
        fh.write(f"# HBM-side traffic of the bandwidth-bound stages, {args.config} workload, from the same rocprofv3 "
                 f"passes\n")
        for ctr, show in pcmds.items():
            fh.write(f"# {ctr} pass: {show}\n")
        fh.write(f"# made by: {made_by}\n")
        fh.write("# bytes per dispatch: the counters (KiB) scaled as in the attention traffic summary\n\n")
        fh.write("# per call of the stage: the kernel's dispatches of one step summed (the permutation: per tensor;\n"
                 "# the scores and the selection run one launch per head group)\n\n")
        fh.write(f"{'kernel':28s} {'dispatches':>10s} {'fetch_GB':>10s} {'write_GB':>10s} {'algorithmic_GB':>15s} "
                 f"{'counted/alg':>12s}  work\n")
        for key, (what, alg_b) in stage_alg.items():
            f_v = [v for (_, k), v in res["FETCH_SIZE"] if key in k]
            w_v = [v for (_, k), v in res["WRITE_SIZE"] if key in k]
            if not f_v or not w_v:
                continue
            per = len(f_v) if key == "permute_heads" else 1   # the permutation: the average launch (one tensor)
            fb = sum(f_v) / per * 1024 * scale["FETCH_SIZE"]
            wb = sum(w_v) / per * 1024 * scale["WRITE_SIZE"]
            ratio = (fb + wb) / alg_b if alg_b else float("nan")
            fh.write(f"{key:28s} {len(f_v):10d} {fb / 1e9:10.3f} {wb / 1e9:10.3f} {alg_b / 1e9:15.3f} {ratio:12.3f}  "
                     f"{what}\n")
    # utilisation counters of the attention kernels, one pass per counter group
    groups = {"mfma_lds": ["MfmaUtil", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS", "SQ_WAIT_INST_LDS"],
              "waits": ["SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_ACTIVE_INST_ANY", "SQ_BUSY_CYCLES"],
              "l2": ["TCC_HIT_sum", "TCC_MISS_sum"]}
    vals, shows = {}, {}
    for g, ctrs in groups.items():
        d = os.path.join(raw, g)
        cmd, show = cmd_for(["rocprofv3", "--pmc"] + ctrs + ["--kernel-include-regex", ATTN_REGEX, "--output-format",
                                                              "csv", "-d", d, "-o", g], 1, 0)
        shows[g] = show.replace(d, rel(d)).replace(ATTN_REGEX, "'" + ATTN_REGEX + "'")
        _run(cmd, d + ".log", 300)
        rows = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                rows += list(csv.DictReader(fh))
        for r in rows:
            key = (_short(r["Kernel_Name"]), r["Counter_Name"])
            vals.setdefault(key, {}).setdefault(r["Dispatch_Id"], 0.0)
            vals[key][r["Dispatch_Id"]] += float(r["Counter_Value"] or 0)
    with open(os.path.join(out, f"attn_{args.config}_counters.txt"), "w") as fh:
        fh.write(f"# rocprofv3 counters of the attention kernels, {args.config} workload, one step\n")
        for g, show in shows.items():
            fh.write(f"# {g} pass: {show}\n")
        fh.write(f"# made by: {made_by}\n\n")
        kernels = sorted({k for k, _ in vals})
        for k in kernels:
            m = {c: sum(v.values()) / len(v) for (kk, c), v in vals.items() if kk == k}
            fh.write(f"{k}\n")
            for c in sorted(m):
                fh.write(f"  {c}: {m[c]:.6g}\n")
            if m.get("SQ_WAVE_CYCLES"):
                fh.write(f"  wait share (SQ_WAIT_ANY / SQ_WAVE_CYCLES): {m['SQ_WAIT_ANY'] / m['SQ_WAVE_CYCLES']:.3f}\n")
            if m.get("TCC_HIT_sum") is not None and m.get("TCC_MISS_sum") is not None:
                hr = m["TCC_HIT_sum"] / max(1.0, m["TCC_HIT_sum"] + m["TCC_MISS_sum"])
                fh.write(f"  L2 hit rate: {hr:.3f}\n")
    print(f"[profile] wrote summaries into {out}", file=sys.stderr, flush=True)


def measure_norm_map(cfg, reps=10):
    """prism_audio_norm_map on a synthetic cross-attention output of the
    workload's shape (N tokens x heads*d channels, the workload's dtype), timed
    with HIP events on the launch stream outside the step.  Algorithmic bytes:
    the rows read once and the fp32 map written once."""
    import workloads.synth as synth
    from dynamic_block_sparse_amd import prism as P
    print("[bench] audio norm map", file=sys.stderr, flush=True)
    h = synth.cross_attn_output(cfg, device="cuda")
    N, C = h.shape
    a = torch.empty(N, dtype=torch.float32, device="cuda")
    ws = torch.empty(P.prism_workspace_size(P.OP_NORM_MAP, N, 0, 0, 0, 0), dtype=torch.uint8, device="cuda")
    for _ in range(3):
        P.prism_audio_norm_map(h, N, C, C, a, ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        P.prism_audio_norm_map(h, N, C, C, a, ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    alg = N * C * h.element_size() + 4 * N
    del h
    gbs = alg / (ms * 1e-3) / 1e9
    return {"input": f"{N} x {C} {cfg.dtype}", "ms": round(ms, 4), "algorithmic_bytes": alg,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4)}}


def measure_routed(path, qp, kp, vp, ratio, dop=None, reps=3):
    """Sharpness routing and the routed forward (flat blocks on the block-mean
    path) against the exact forward, on the first head group of the step's
    permuted tensors, timed with HIP events outside the step."""
    print("[bench] routed forward", file=sys.stderr, flush=True)
    sel = path.select(qp, kp, 0, want_logits=True)
    flat, _ = path.route(sel, ratio, want_sharpness=True)
    path.forward(qp, kp, vp, sel)
    path.routed_forward(qp, kp, vp, sel, flat)
    torch.cuda.synchronize()

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    route_ms = timed(lambda: path.route(sel, ratio))
    op, rop = path.block_major_like(qp), path.block_major_like(qp)
    res_e, res_r = (path.residual_like(op), path.residual_like(rop)) if dop is not None else (None, None)
    exact_ms = timed(lambda: path.forward(qp, kp, vp, sel, op=op, ores=res_e))
    routed_ms = timed(lambda: path.routed_forward(qp, kp, vp, sel, flat, op=rop, ores=res_r))
    bwd = {}
    if dop is not None:
        _, lse = path.forward(qp, kp, vp, sel, op=op, ores=res_e)
        _, rlse = path.routed_forward(qp, kp, vp, sel, flat, op=rop, ores=res_r)
        grads = tuple(path.block_major_like(qp) for _ in range(3))
        path.backward(qp, kp, vp, op, dop, lse, sel, grads=grads, ores=res_e)
        path.routed_backward(qp, kp, vp, rop, dop, rlse, sel, flat, grads=grads, ores=res_r)
        torch.cuda.synchronize()
        eb = timed(lambda: path.backward(qp, kp, vp, op, dop, lse, sel, grads=grads, ores=res_e))
        rb = timed(lambda: path.routed_backward(qp, kp, vp, rop, dop, rlse, sel, flat, grads=grads, ores=res_r))
        bwd = {"exact_backward_ms": round(eb, 3), "routed_backward_ms": round(rb, 3),
               "fwd_bwd_speedup": round((exact_ms + eb) / (route_ms + routed_ms + rb), 3)}
        del lse, rlse, grads
    del op, rop, res_e, res_r
    sizes = (path.block_offsets[1:path.nb + 1] - path.block_offsets[:path.nb]).to(torch.float64)
    flat_tokens = float((flat.to(torch.float64) * sizes).sum()) / (path.hc * path.N)
    del sel
    return {"flat_ratio": ratio, "heads": path.hc, "flat_token_fraction": round(flat_tokens, 4),
            "route_ms": round(route_ms, 3), "exact_forward_ms": round(exact_ms, 3),
            "routed_forward_ms": round(routed_ms, 3),
            "forward_speedup": round(exact_ms / (routed_ms + route_ms), 3), **bwd}


def measure_zone_order(cfg, x, path, qp, kp, vp, dop=None, reps=3):
    """The Hilbert zone order against raster order on the same inputs: block
    layout, permutation of Q, K, V (and dO), selection, forward and backward of
    the first head group, timed with HIP events outside the step.  Both orders
    select the same work (same blocks, renumbered), so the effective FLOPs are
    reported for each as a check."""
    from dynamic_block_sparse_amd.path import PrismPath
    print("[bench] hilbert zone order", file=sys.stderr, flush=True)
    hp = PrismPath(cfg.T, cfg.H, cfg.W, cfg.heads, cfg.d, cfg.top_k, cfg.top_p, path.scale, head_chunk=path.hc,
                   zone_order="hilbert")
    hp.shapes(x["v"], x["a"])
    names = ("q", "k", "v") + (("do",) if dop is not None else ())
    hb = {n: hp.permute(x[n]) for n in names}

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    res = {}
    for tag, p, t in (("raster", path, {"q": qp, "k": kp, "v": vp, "do": dop}), ("hilbert", hp, hb)):
        sel = p.select(t["q"], t["k"], 0)
        op = p.block_major_like(t["q"])
        ores = p.residual_like(op) if dop is not None else None
        _, lse = p.forward(t["q"], t["k"], t["v"], sel, op=op, ores=ores)
        r = {"permute_ms": round(timed(lambda: p.permute(x["q"], out=t["q"])), 3),
             "select_ms": round(timed(lambda: p.select(t["q"], t["k"], 0)), 3),
             "forward_ms": round(timed(lambda: p.forward(t["q"], t["k"], t["v"], sel, op=op, lse=lse, ores=ores)), 3)}
        f_fwd, f_bwd, mean_sel = effective_flops(p, [sel], cfg.d)
        if dop is not None:
            grads = tuple(p.block_major_like(t["q"]) for _ in range(3))
            r["backward_ms"] = round(timed(lambda: p.backward(t["q"], t["k"], t["v"], op, t["do"], lse, sel,
                                                              grads=grads, ores=ores)), 3)
            del grads
        r["effective_tflop"] = round((f_fwd + (f_bwd if dop is not None else 0.0)) / 1e12, 6)
        r["mean_selected_blocks"] = round(mean_sel, 3)
        res[tag] = r
        del sel, op, lse
    del hb
    att = lambda r: r["forward_ms"] + r.get("backward_ms", 0.0)
    res["heads"] = path.hc
    res["attention_speedup"] = round(att(res["raster"]) / att(res["hilbert"]), 3)
    return res



def measure_subblock(cfg, path, qp, kp, vp, dop=None, reps=3):
    """Sub-block scoring (prism_select_subblock) against the plain pooled
    scores (prism_select) on the first head group of the step's permuted
    tensors: selection time, the selected work, and the attention time over
    each selection, timed with HIP events outside the step."""
    print("[bench] sub-block scoring", file=sys.stderr, flush=True)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    res = {}
    for scoring in ("block", "subblock"):
        sel = path.select(qp, kp, 0, scoring=scoring)
        r = {"select_ms": round(timed(lambda: path.select(qp, kp, 0, scoring=scoring)), 3)}
        op = path.block_major_like(qp)
        ores = path.residual_like(op) if dop is not None else None
        _, lse = path.forward(qp, kp, vp, sel, op=op, ores=ores)
        r["forward_ms"] = round(timed(lambda: path.forward(qp, kp, vp, sel, op=op, lse=lse, ores=ores)), 3)
        if dop is not None:
            grads = tuple(path.block_major_like(qp) for _ in range(3))
            r["backward_ms"] = round(timed(lambda: path.backward(qp, kp, vp, op, dop, lse, sel, grads=grads,
                                                                 ores=ores)), 3)
            del grads
        f_fwd, f_bwd, mean_sel = effective_flops(path, [sel], cfg.d)
        r["effective_tflop"] = round((f_fwd + (f_bwd if dop is not None else 0.0)) / 1e12, 4)
        r["mean_selected_blocks"] = round(mean_sel, 3)
        res[scoring] = r
        del sel, op, lse
    res["heads"] = path.hc
    return res



def measure_reuse(cfg, x, path, reps=2):
    """Selection reuse across diffusion steps: PrismPath.step with a fresh
    selection against a step that reuses the cached zone shapes, layout and
    selected sets (zone statistics, shapes and selection skipped), on the
    workload's inputs, timed with HIP events outside the measured step."""
    print("[bench] selection reuse", file=sys.stderr, flush=True)
    args = (x["q"], x["k"], x["v"], x["a"], x.get("do"))

    def timed(reuse):
        path.step(*args, reuse=reuse)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            path.step(*args, reuse=reuse)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    fresh = timed(False)
    reused = timed(True)
    return {"fresh_step_ms": round(fresh, 3), "reused_step_ms": round(reused, 3),
            "saved_per_reused_step_ms": round(fresh - reused, 3)}


def main():
    args = parse()
    if args.profile:
        profile(args)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus above 1 is not supported (the path shards by head, one process per GPU, with no kernel change)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    from workloads.synth import CONFIGS, make_inputs
    from dynamic_block_sparse_amd import prism as P
    from dynamic_block_sparse_amd.path import PrismPath

    cfg = CONFIGS[args.config]
    if args.calibrate:
        calibrate(cfg)
        return
    print(f"[bench] generating {cfg.name} inputs", file=sys.stderr, flush=True)
    x = make_inputs(cfg, device="cuda")
    torch.cuda.synchronize()
    sc = float(np.float32(1.0 / math.sqrt(cfg.d)))
    path = PrismPath(cfg.T, cfg.H, cfg.W, cfg.heads, cfg.d, cfg.top_k, cfg.top_p, sc,
                     head_chunk=1 if cfg.heads_sequential else None)
    nb = path.shapes(x["v"], x["a"])
    # buffers allocated once, outside the timed region
    # block-major tensors live head-major ([heads, N, d] storage, [N, heads, d] views)
    bm = lambda: path.block_major_like(x["q"])
    qp, kp, vp = bm(), bm(), bm()
    dop = bm() if cfg.backward else None
    outs = {n: torch.empty_like(x["q"]) for n in (("o", "dq", "dk", "dv") if cfg.backward else ("o",))}
    # the bf16 residual of O, which the backward's row dot reads (training steps only)
    ores = path.residual_like(outs["o"]) if cfg.backward else None
    ld, hs = qp.stride(0), qp.stride(1)
    hc = path.hc
    lse = torch.empty((hc, cfg.N), dtype=torch.float32, device="cuda")
    # CSR capacity from the counts: one sizing selection per head group
    # before the timed region (the timed steps select the same sets again)
    for src, dst in ((x["q"], qp), (x["k"], kp)):
        path.permute(src, out=dst)
    for h0 in range(0, cfg.heads, hc):
        path.select(qp, kp, h0)
    cap = path._cap_guess()
    torch.cuda.synchronize()
    sel_bufs = []
    for _ in range(0, cfg.heads, hc):
        from dynamic_block_sparse_amd.path import Selection
        sel_bufs.append(Selection(torch.empty((hc, nb + 1), dtype=torch.int32, device="cuda"),
                                  torch.empty((hc, cap), dtype=torch.int32, device="cuda"),
                                  torch.empty(hc, dtype=torch.int64, device="cuda"), cap, None))
    # the calls run one after another on one stream, so one workspace serves them all
    ws_sizes = {"zone": P.prism_workspace_size(P.OP_ZONE_SHAPES, cfg.N, 1, cfg.heads * cfg.d, 0, 0),
                "sel": P.prism_workspace_size(P.OP_SELECT, cfg.N, hc, cfg.d, nb, 0),
                "fwd": P.prism_workspace_size(P.OP_ATTN_FWD, cfg.N, hc, cfg.d, nb, cap),
                "bwd": P.prism_workspace_size(P.OP_ATTN_BWD, cfg.N, hc, cfg.d, nb, cap)}
    ws_all = torch.empty(max(ws_sizes.values()), dtype=torch.uint8, device="cuda")
    ws_zone, ws_sel, ws_fwd, ws_bwd = (ws_all[:ws_sizes[k]] for k in ("zone", "sel", "fwd", "bwd"))
    C = cfg.heads * cfg.d
    stages = ["shapes", "permute_in", "select", "attn_fwd", "attn_bwd"]
    # the attention kernels write O, dQ, dK and dV straight to raster order
    # (the inverse permutation applied in their epilogues)
    lay = path.raster_layout(outs["o"])

    def step(ev):
        ev[0].record()
        n = P.prism_zone_shapes(cfg.T, cfg.H, cfg.W, x["v"], C, x["v"].stride(0), x["a"], path.zone_shape,
                                path.block_offsets, path.nb_dev, ws_zone, want_nb=False)
        ev[1].record()
        for src, dst in ((x["q"], qp), (x["k"], kp), (x["v"], vp)) + (((x["do"], dop),) if cfg.backward else ()):
            path.permute(src, out=dst)
        ev[2].record()
        for g, h0 in enumerate(range(0, cfg.heads, hc)):
            s = sel_bufs[g]
            q, k, v = (t[:, h0:h0 + hc] for t in (qp, kp, vp))
            o = outs["o"][:, h0:h0 + hc]
            P.prism_select(q, k, cfg.N, hc, cfg.d, ld, hs, path.block_offsets, nb, cfg.top_k, cfg.top_p, sc,
                           s.offsets, s.idx, cap, s.total, ws_sel)
            ev[3 + 3 * g].record()
            r = ores[:, h0:h0 + hc] if ores is not None else None
            P.prism_sparse_attn_fwd(q, k, v, o, lse, cfg.N, hc, cfg.d, ld, hs, path.block_offsets, nb, s.offsets,
                                    s.idx, cap, sc, ws=ws_fwd, layout=lay, o_res=r)
            ev[4 + 3 * g].record()
            if cfg.backward:
                do_ = dop[:, h0:h0 + hc]
                gq, gk, gv = (outs[n][:, h0:h0 + hc] for n in ("dq", "dk", "dv"))
                P.prism_sparse_attn_bwd(q, k, v, o, do_, lse, gq, gk, gv, cfg.N, hc, cfg.d, ld, hs,
                                        path.block_offsets, nb, s.offsets, s.idx, cap, sc, ws_bwd, layout=lay,
                                        o_res=r)
            ev[5 + 3 * g].record()
        ev[-1].record()

    ngroups = cfg.heads // hc
    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(3 + 3 * ngroups + 1)]
    for _ in range(args.warmup):
        step(mk())
    torch.cuda.synchronize()
    evs = [mk() for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps (NB {nb})", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall / args.steps * 1e3
    short = [int(s.total.max().item()) for s in sel_bufs if int(s.total.max().item()) > cap]
    if short:
        raise RuntimeError(f"a head's selection needed {max(short)} CSR entries, above the sized capacity {cap}")
    # device memory the step holds: inputs, block-major copies, outputs, the
    # selections and the shared workspace (what torch has allocated)
    memory = {"allocated_gb": round(torch.cuda.memory_allocated() / 1e9, 2),
              "workspace_gb": round(ws_all.numel() / 1e9, 3),
              "csr_entries_per_head": cap}
    acc = {s: 0.0 for s in stages}
    for ev in evs:
        acc["shapes"] += ev[0].elapsed_time(ev[1])
        acc["permute_in"] += ev[1].elapsed_time(ev[2])
        prev = ev[2]
        for g in range(ngroups):
            acc["select"] += prev.elapsed_time(ev[3 + 3 * g])
            acc["attn_fwd"] += ev[3 + 3 * g].elapsed_time(ev[4 + 3 * g])
            acc["attn_bwd"] += ev[4 + 3 * g].elapsed_time(ev[5 + 3 * g])
            prev = ev[5 + 3 * g]
    stage_ms = {s: acc[s] / args.steps for s in stages}
    f_fwd, f_bwd, mean_sel = effective_flops(path, sel_bufs, cfg.d)
    f_eff = f_fwd + (f_bwd if cfg.backward else 0.0)
    attn_ms = stage_ms["attn_fwd"] + stage_ms["attn_bwd"]
    value = f_eff / (ms_step * 1e-3) / 1e12
    attn_tflops = f_eff / (attn_ms * 1e-3) / 1e12
    dom = "attn_bwd" if cfg.backward and stage_ms["attn_bwd"] >= stage_ms["attn_fwd"] else "attn_fwd"
    dom_flops = f_bwd if dom == "attn_bwd" else f_fwd
    achieved = dom_flops / (stage_ms[dom] * 1e-3) / 1e12
    roofline = {"kernel": "sparse attention backward (prism_sparse_attn_bwd)" if dom == "attn_bwd"
                else "sparse attention forward (prism_sparse_attn_fwd)",
                "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": read_traffic(cfg.name) if dom == "attn_bwd" else None}
    # algorithmic bytes of the HBM-bound stages: V once plus the audio map (zone
    # statistics), read + write of every permuted tensor, Q and K once (selection)
    es = 2 if cfg.dtype == "bf16" else 4
    ntens = 4 if cfg.backward else 3
    alg = {"shapes": cfg.N * C * es + 4 * cfg.N, "permute_in": ntens * 2 * cfg.N * C * es,
           "select": 2 * cfg.N * C * es}
    stage_gbs = {k: round(b / (stage_ms[k] * 1e-3) / 1e9, 1) for k, b in alg.items()}
    result = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if cfg.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.T}x{cfg.H}x{cfg.W} grid ({cfg.N} tokens), {cfg.heads} heads x "
                               f"d={cfg.d}, top-k {cfg.top_k}, top-p {cfg.top_p}, "
                               f"{'fwd+bwd' if cfg.backward else 'fwd'}",
                   "tokens": cfg.N, "heads": cfg.heads, "head_dim": cfg.d, "blocks": nb,
                   "mean_selected_blocks": round(mean_sel, 2), "selected_fraction": round(mean_sel / nb, 5)},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 3),
        "attention_only_tflops": round(attn_tflops, 3),
        "attention_only_pct_of_bf16_peak": round(100 * attn_tflops / PEAK_BF16_TFLOPS, 3),
        "effective_tflop_per_step": round(f_eff / 1e12, 4),
        "stage_ms": {s: round(v, 3) for s, v in stage_ms.items()},
        "stage_gbs_algorithmic": stage_gbs,
        "roofline": roofline,
        "device_memory": memory,
    }
    if not args.no_next_rows:
        result["next_rows"] = {"f1_audio_norm_map": measure_norm_map(cfg),
                               "f3_routed_forward": measure_routed(path, qp, kp, vp, args.flat_ratio, dop),
                               "f4_hilbert_zone_order": measure_zone_order(cfg, x, path, qp, kp, vp, dop),
                               "f4_subblock_scoring": measure_subblock(cfg, path, qp, kp, vp, dop)}
        if ms_step < 5000:   # whole extra steps: skipped for the long clip (about 20 s a step)
            result["next_rows"]["f2_selection_reuse"] = measure_reuse(cfg, x, path)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(cfg, x, path.zone_shape.cpu().numpy(), args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

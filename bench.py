"""Benchmark of the Prism dynamic block-sparse attention hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 2k] [--no-cpu-baseline]

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
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective sparse-attn TFLOP/s fwd+bwd at 2K tokens; % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="2k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    return ap.parse_args()


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
    Qp, Kp, Vp, dOp = (orc.to_block_major(x[n][:, 0:1, :].float().cpu().numpy(), pi) for n in ("q", "k", "v", "do"))
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
        orc.attn_bwd_block(Qp, Kp, Vp, dOp, offs, sel, i, 0, sc)
        Bi = offs[i + 1] - offs[i]
        flops += 14.0 * Bi * float(sum(offs[j + 1] - offs[j] for j in sel)) * cfg.d
        nblocks += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"float64 oracle pooling of head 0 (all {NB} blocks) then per query block: scores, "
                      f"selection, attention forward and backward, for {nblocks} query blocks of head 0 "
                      f"in seeded random order ({dt:.1f} s)"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus above 1 is not supported",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    from workloads.synth import CONFIGS, make_inputs
    from dynamic_block_sparse_amd import prism as P
    from dynamic_block_sparse_amd.path import PrismPath

    cfg = CONFIGS[args.config]
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
    op = bm()
    grads = (bm(), bm(), bm()) if cfg.backward else None
    outs = {n: torch.empty_like(x["q"]) for n in (("o", "dq", "dk", "dv") if cfg.backward else ("o",))}
    ld, hs = qp.stride(0), qp.stride(1)
    hc = path.hc
    lse = torch.empty((hc, cfg.N), dtype=torch.float32, device="cuda")
    cap = nb * nb
    sel_bufs = []
    for _ in range(0, cfg.heads, hc):
        from dynamic_block_sparse_amd.path import Selection
        sel_bufs.append(Selection(torch.empty((hc, nb + 1), dtype=torch.int32, device="cuda"),
                                  torch.empty((hc, cap), dtype=torch.int32, device="cuda"),
                                  torch.empty(hc, dtype=torch.int64, device="cuda"), cap, None))
    ws_zone = torch.empty(P.prism_workspace_size(P.OP_ZONE_SHAPES, cfg.N, 1, cfg.heads * cfg.d, 0, 0),
                          dtype=torch.uint8, device="cuda")
    ws_sel = torch.empty(P.prism_workspace_size(P.OP_SELECT, cfg.N, hc, cfg.d, nb, cap), dtype=torch.uint8,
                         device="cuda")
    ws_bwd = torch.empty(P.prism_workspace_size(P.OP_ATTN_BWD, cfg.N, hc, cfg.d, nb, cap), dtype=torch.uint8,
                         device="cuda")
    C = cfg.heads * cfg.d
    stages = ["shapes", "permute_in", "select", "attn_fwd", "attn_bwd", "permute_out"]

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
            q, k, v, o = (t[:, h0:h0 + hc] for t in (qp, kp, vp, op))
            P.prism_select(q, k, cfg.N, hc, cfg.d, ld, hs, path.block_offsets, nb, cfg.top_k, cfg.top_p, sc,
                           s.offsets, s.idx, cap, s.total, ws_sel)
            ev[3 + 3 * g].record()
            P.prism_sparse_attn_fwd(q, k, v, o, lse, cfg.N, hc, cfg.d, ld, hs, path.block_offsets, nb, s.offsets,
                                    s.idx, cap, sc)
            ev[4 + 3 * g].record()
            if cfg.backward:
                do_, gq, gk, gv = (t[:, h0:h0 + hc] for t in (dop,) + grads)
                P.prism_sparse_attn_bwd(q, k, v, o, do_, lse, gq, gk, gv, cfg.N, hc, cfg.d, ld, hs,
                                        path.block_offsets, nb, s.offsets, s.idx, cap, sc, ws_bwd)
            ev[5 + 3 * g].record()
        srcs = (op,) + (grads if cfg.backward else ())
        for src, name in zip(srcs, outs):
            path.permute(src, inverse=True, out=outs[name])
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
        acc["permute_out"] += prev.elapsed_time(ev[-1])
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
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None}
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
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(cfg, x, path.zone_shape.cpu().numpy(), args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

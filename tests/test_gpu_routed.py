"""GPU parity of the sharpness routing and the routed forward (exact path for
sharp query blocks, block-mean path for flat ones) against the float64 oracle.

The oracle runs the whole chain on host copies of the same seeded inputs:
zone shapes, permutation, pooled scores, selection, sharpness, routing, and
per block either exact attention or the block-mean expansion.  Sharpness is
compared where the two sides' pooled scores agree; flat flags are compared
unless the routing cut falls within 1e-10 of a tie (flagged, never seen).
"""
import math

import numpy as np
import pytest
import torch

from oracle import prism_oracle as orc
from parity_bars import TOL, assert_close
from workloads.synth import CONFIGS, custom, make_inputs

pytestmark = pytest.mark.gpu


CASES = [
    custom("r_bf16_d128", T=16, H=16, W=24, heads=2, d=128, dtype="bf16", top_k=3, top_p=0.8,
           kinds=(("smooth", 0.5), ("static", 0.25), ("fast1", 0.25)),
           sigma={"smooth": 0.3, "static": 1e-3, "fast1": 0.1}, n_blobs=2, blob_std=(3.0, 4.0, 4.0), seed=12),
    custom("r_f32_d64", T=8, H=16, W=16, heads=1, d=64, dtype="f32", top_k=4, top_p=0.9, seed=11),
    custom("r_diffuse", T=16, H=16, W=16, heads=2, d=128, dtype="bf16", top_k=2, top_p=0.95,
           kinds=(("static", 1 / 3), ("aniso", 1 / 3), ("noisy", 1 / 3)),
           sigma={"static": 1e-3, "aniso": 0.1, "noisy": 1.0}, beta=0.3, seed=18),
]


def _np(t):
    return t.detach().float().cpu().numpy() if t.dtype != torch.float64 else t.detach().cpu().numpy()


def _path(cfg, heads=None, hc=None):
    from dynamic_block_sparse_amd.path import PrismPath
    return PrismPath(cfg.T, cfg.H, cfg.W, heads or cfg.heads, cfg.d, cfg.top_k, cfg.top_p,
                     float(np.float32(1.0 / math.sqrt(cfg.d))), head_chunk=hc)


def _close_grad(got, want, dtype, what):
    assert_close(np.asarray(got), np.asarray(want), dtype, what, grad=True)


def _check_head(h, hh, path, sel, flat_g, M_g, op, lse, xs, zs, pi, cfg, ratio, blocks, v_att=None, dq=None):
    """Oracle chain for head h (global index into the input tensors), compared
    on `blocks` (None: every block).  hh indexes the GPU head chunk."""
    offs, nb = zs["block_offsets"], zs["NB"]
    sc = float(np.float32(1.0 / math.sqrt(cfg.d)))
    V = v_att if v_att is not None else xs["v"]
    Qp, Kp, Vp = (orc.to_block_major(_np(t[:, h:h + 1, :]), pi) for t in (xs["q"], xs["k"], V))
    L = orc.block_logits(orc.pool_blocks(Qp, offs, 0), orc.pool_blocks(Kp, offs, 0), sc)
    Lg = sel.logits[hh].cpu().numpy()
    clean = not (Lg != L).any()
    co, ci, flags = orc.select(L, cfg.top_k, cfg.top_p)
    M = orc.block_sharpness(L)
    flat = orc.flat_route(M, ratio)
    Mg = M_g[hh].cpu().numpy()
    if clean:
        np.testing.assert_allclose(Mg, M, rtol=1e-10, atol=1e-300)
        n_flat = int(math.floor(ratio * nb))
        ms = np.sort(M)
        tie = 0 < n_flat < nb and abs(ms[n_flat] - ms[n_flat - 1]) <= 1e-10 * max(ms[n_flat], 1e-300)
        fg = flat_g[hh].cpu().numpy().astype(bool)
        if not tie:
            np.testing.assert_array_equal(fg, flat)
    else:
        fg = flat_g[hh].cpu().numpy().astype(bool)
    print(f"head {h}: {int(flat.sum())} of {nb} blocks flat, pooled scores identical: {clean}", flush=True)
    Og = _np(op[:, hh, :])
    lg = lse[hh].cpu().numpy()
    errs = {"flat": [], "sharp": []}
    derrs = {"flat dQ": [], "sharp dQ": []}
    dOp = orc.to_block_major(_np(xs["do"][:, h:h + 1, :]), pi) if dq is not None else None
    for i in (range(nb) if blocks is None else blocks):
        if flags[i] or fg[i] != flat[i]:
            continue
        s = ci[co[i]:co[i + 1]]
        fn = orc.taylor_attn_fwd_block if flat[i] else orc.attn_fwd_block
        o_ref, l_ref = fn(Qp, Kp, Vp, offs, s, i, 0, sc)
        errs["flat" if flat[i] else "sharp"].append((Og[offs[i]:offs[i + 1]], o_ref))
        np.testing.assert_allclose(lg[offs[i]:offs[i + 1]], l_ref, atol=1e-4 if cfg.dtype == "f32" else 2e-3)
        if dq is not None:
            dq_ref = (orc.taylor_attn_bwd_block if flat[i] else orc.attn_bwd_block)(Qp, Kp, Vp, dOp, offs, s, i, 0,
                                                                                    sc)[0]
            derrs["flat dQ" if flat[i] else "sharp dQ"].append((_np(dq[offs[i]:offs[i + 1], hh, :]), dq_ref))
    for kind, pairs in derrs.items():
        if pairs:
            got = np.concatenate([p_[0] for p_ in pairs])
            want = np.concatenate([p_[1] for p_ in pairs])
            _close_grad(got, want, cfg.dtype, f"head {h} {kind} ({len(pairs)} blocks)")
    mx, mean = TOL[cfg.dtype]
    for kind, pairs in errs.items():
        if not pairs:
            continue
        got = np.concatenate([p[0] for p in pairs])
        want = np.concatenate([p[1] for p in pairs])
        err = np.abs(got - want)
        print(f"head {h} {kind}: {len(pairs)} blocks, max-abs {err.max():.3e} mean-abs {err.mean():.3e}", flush=True)
        assert err.max() <= mx and err.mean() <= mean, kind
    return int(flat.sum())


def _run_small(cfg, ratio):
    x = make_inputs(cfg, device="cuda")
    path = _path(cfg)
    path.shapes(x["v"], x["a"])
    qp, kp, vp = path.permute(x["q"]), path.permute(x["k"]), path.permute(x["v"])
    sel = path.select(qp, kp, want_logits=True)
    flat, M = path.route(sel, ratio, want_sharpness=True)
    op = path.block_major_like(qp).fill_(float("nan"))
    _, lse = path.routed_forward(qp, kp, vp, sel, flat, op=op)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(op).all())
    zs = orc.zone_shapes(_np(x["v"]).reshape(cfg.N, -1), _np(x["a"]), cfg.T, cfg.H, cfg.W)
    assert zs["NB"] == path.nb and not zs["near_tie"].any()
    pi = orc.permutation(cfg.T, cfg.H, cfg.W, zs["shape"])
    return x, path, sel, flat, M, op, lse, zs, pi


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
@pytest.mark.parametrize("ratio", [0.5, 1.0])
def test_routed_forward_small(cfg, ratio):
    x, path, sel, flat, M, op, lse, zs, pi = _run_small(cfg, ratio)
    for h in range(cfg.heads):
        _check_head(h, h, path, sel, flat, M, op, lse, x, zs, pi, cfg, ratio, None)


def test_routed_forward_with_no_flat_block_is_the_exact_forward():
    cfg = CASES[0]
    x = make_inputs(cfg, device="cuda")
    path = _path(cfg)
    path.shapes(x["v"], x["a"])
    qp, kp, vp = path.permute(x["q"]), path.permute(x["k"]), path.permute(x["v"])
    sel = path.select(qp, kp, want_logits=True)
    flat = path.route(sel, 0.0)
    assert int(flat.sum()) == 0
    o1, l1 = path.routed_forward(qp, kp, vp, sel, flat)
    o2, l2 = path.forward(qp, kp, vp, sel)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_routed_forward_2k_size(progress):
    cfg = CONFIGS["2k"]
    rng = np.random.default_rng(77)
    heads = sorted(rng.choice(cfg.heads, size=2, replace=False).tolist())
    progress(f"routed 2k: heads {heads}, generating")
    x = make_inputs(cfg, device="cuda", tensors=("v",))
    xs = make_inputs(cfg, device="cuda", heads=heads, tensors=("q", "k", "do"))
    path = _path(cfg, heads=2)
    path.shapes(x["v"], x["a"])
    v_att = x["v"][:, heads]
    qp, kp, vp = path.permute(xs["q"]), path.permute(xs["k"]), path.permute(v_att)
    sel = path.select(qp, kp, want_logits=True)
    flat, M = path.route(sel, 0.5, want_sharpness=True)
    op = path.block_major_like(qp).fill_(float("nan"))
    ores = path.residual_like(op)
    _, lse = path.routed_forward(qp, kp, vp, sel, flat, op=op, ores=ores)
    dop = path.permute(xs["do"])
    grads = tuple(path.block_major_like(qp).fill_(float("nan")) for _ in range(3))
    path.routed_backward(qp, kp, vp, op, dop, lse, sel, flat, grads=grads, ores=ores)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(op).all())
    for g in grads:
        assert bool(torch.isfinite(g).all())
    progress("routed 2k: oracle zone statistics")
    zs = orc.zone_shapes(_np(x["v"]).reshape(cfg.N, -1), _np(x["a"]), cfg.T, cfg.H, cfg.W)
    assert zs["NB"] == path.nb
    pi = orc.permutation(cfg.T, cfg.H, cfg.W, zs["shape"])
    blocks = sorted(rng.choice(zs["NB"], size=48, replace=False).tolist())
    xs_full = {"q": xs["q"], "k": xs["k"], "v": v_att, "do": xs["do"]}
    for hh, h in enumerate(heads):
        progress(f"routed 2k: head {h}")
        _check_head(hh, hh, path, sel, flat, M, op, lse, xs_full, zs, pi, cfg, 0.5, blocks, dq=grads[0])


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
@pytest.mark.parametrize("ratio", [0.5, 1.0])
def test_routed_backward_small(cfg, ratio):
    x = make_inputs(cfg, device="cuda")
    path = _path(cfg)
    path.shapes(x["v"], x["a"])
    qp, kp, vp, dop = (path.permute(x[n]) for n in ("q", "k", "v", "do"))
    sel = path.select(qp, kp, want_logits=True)
    flat = path.route(sel, ratio)
    op = path.block_major_like(qp)
    ores = path.residual_like(op)
    _, lse = path.routed_forward(qp, kp, vp, sel, flat, op=op, ores=ores)
    grads = tuple(path.block_major_like(qp).fill_(float("nan")) for _ in range(3))
    path.routed_backward(qp, kp, vp, op, dop, lse, sel, flat, grads=grads, ores=ores)
    torch.cuda.synchronize()
    for g in grads:
        assert bool(torch.isfinite(g).all())
    zs = orc.zone_shapes(_np(x["v"]).reshape(cfg.N, -1), _np(x["a"]), cfg.T, cfg.H, cfg.W)
    pi = orc.permutation(cfg.T, cfg.H, cfg.W, zs["shape"])
    offs = zs["block_offsets"]
    sc = float(np.float32(1.0 / math.sqrt(cfg.d)))
    for h in range(cfg.heads):
        Qp, Kp, Vp, dOp = (orc.to_block_major(_np(x[n][:, h:h + 1, :]), pi) for n in ("q", "k", "v", "do"))
        L = orc.block_logits(orc.pool_blocks(Qp, offs, 0), orc.pool_blocks(Kp, offs, 0), sc)
        assert not (sel.logits[h].cpu().numpy() != L).any()
        co, ci, flags = orc.select(L, cfg.top_k, cfg.top_p)
        assert not flags.any()
        fl = orc.flat_route(orc.block_sharpness(L), ratio)
        np.testing.assert_array_equal(flat[h].cpu().numpy().astype(bool), fl)
        ref = orc.routed_attention(Qp, Kp, Vp, offs, co, ci, fl, 0, sc, dOp=dOp)
        for name, g in (("dQ", grads[0]), ("dK", grads[1]), ("dV", grads[2])):
            _close_grad(_np(g[:, h, :]), ref[name], cfg.dtype, f"{cfg.name} r={ratio} head {h} {name}")


def test_routed_backward_with_no_flat_block_is_the_exact_backward():
    cfg = CASES[0]
    x = make_inputs(cfg, device="cuda")
    path = _path(cfg)
    path.shapes(x["v"], x["a"])
    qp, kp, vp, dop = (path.permute(x[n]) for n in ("q", "k", "v", "do"))
    sel = path.select(qp, kp, want_logits=True)
    flat = path.route(sel, 0.0)
    op = path.block_major_like(qp)
    ores = path.residual_like(op)
    _, lse = path.forward(qp, kp, vp, sel, op=op, ores=ores)
    g1 = path.routed_backward(qp, kp, vp, op, dop, lse, sel, flat, ores=ores)
    g2 = path.backward(qp, kp, vp, op, dop, lse, sel, ores=ores)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)

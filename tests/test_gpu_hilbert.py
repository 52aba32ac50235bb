"""GPU parity of the Hilbert zone order (next row after the exact path): block
offsets, the permutation and the whole path against the oracle run with the
same zone order."""
import math

import numpy as np
import pytest
import torch

from oracle import prism_oracle as orc
from parity_bars import TOL, assert_close
from workloads.synth import CONFIGS, custom, make_inputs

pytestmark = pytest.mark.gpu


CASES = [
    custom("h_bf16_d128", T=16, H=24, W=16, heads=2, d=128, dtype="bf16", top_k=3, top_p=0.8,
           kinds=(("smooth", 0.5), ("static", 0.25), ("fast1", 0.25)),
           sigma={"smooth": 0.3, "static": 1e-3, "fast1": 0.1}, n_blobs=2, blob_std=(3.0, 4.0, 4.0), seed=31),
    custom("h_f32_d64", T=16, H=16, W=16, heads=1, d=64, dtype="f32", top_k=4, top_p=0.9, seed=32),
]


def _np(t):
    return t.detach().float().cpu().numpy()


def _close(got, want, dtype, what, grad=False, terms=None):
    assert_close(np.asarray(got), np.asarray(want), dtype, what, grad=grad, terms=terms)


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_hilbert_order_end_to_end(cfg):
    from dynamic_block_sparse_amd.path import PrismPath
    x = make_inputs(cfg, device="cuda")
    sc = float(np.float32(1.0 / math.sqrt(cfg.d)))
    path = PrismPath(cfg.T, cfg.H, cfg.W, cfg.heads, cfg.d, cfg.top_k, cfg.top_p, sc, zone_order="hilbert")
    out = path.step(x["q"], x["k"], x["v"], x["a"], x["do"])
    torch.cuda.synchronize()
    order = orc.hilbert_zone_order(cfg.T, cfg.H, cfg.W)
    zs = orc.zone_shapes(_np(x["v"]).reshape(cfg.N, -1), _np(x["a"]), cfg.T, cfg.H, cfg.W)
    assert not zs["near_tie"].any()
    np.testing.assert_array_equal(path.zone_shape.cpu().numpy(), zs["shape"])
    offs, nb = orc.block_layout(zs["shape"], order)
    assert path.nb == nb
    np.testing.assert_array_equal(path.block_offsets[:nb + 1].cpu().numpy(), offs)
    pi = orc.permutation(cfg.T, cfg.H, cfg.W, zs["shape"], order)
    qp = path.permute(x["q"])
    np.testing.assert_array_equal(_np(qp), _np(x["q"])[pi])
    np.testing.assert_array_equal(_np(path.permute(qp, inverse=True)), _np(x["q"]))
    sel = out["selections"][0]
    for h in range(cfg.heads):
        Qp, Kp, Vp, dOp = (orc.to_block_major(_np(x[n][:, h:h + 1, :]), pi) for n in ("q", "k", "v", "do"))
        L = orc.block_logits(orc.pool_blocks(Qp, offs, 0), orc.pool_blocks(Kp, offs, 0), sc)
        co, ci, flags = orc.select(L, cfg.top_k, cfg.top_p)
        assert not flags.any()
        og = sel.offsets[h].cpu().numpy()
        ig = sel.idx[h, :og[-1]].cpu().numpy()
        np.testing.assert_array_equal(og, co)
        np.testing.assert_array_equal(ig, ci)
        att = orc.attention(Qp, Kp, Vp, offs, co, ci, 0, sc, dOp=dOp)
        _close(_np(out["o"][:, h, :]), orc.to_raster(att["O"], pi), cfg.dtype, f"{cfg.name} O h{h}")
        for g, name in (("dq", "dQ"), ("dk", "dK"), ("dv", "dV")):
            _close(_np(out[g][:, h, :]), orc.to_raster(att[name], pi), cfg.dtype, f"{cfg.name} {name} h{h}", grad=True,
                   terms=orc.to_raster(att["t" + name[1]], pi))


def test_hilbert_order_2k_size(progress):
    """Full 2K grid, two heads: Hilbert block offsets and permutation bit-exact
    against the oracle; each Hilbert-order selected set, renumbered to raster
    block indices, equal to the raster path's set for the same query block (the
    pooled scores do not depend on where a zone sits in the sequence); the
    Hilbert-order forward output of sampled query blocks within the bf16 bar of
    the oracle's attention over the oracle's selection."""
    from dynamic_block_sparse_amd.path import PrismPath
    cfg = CONFIGS["2k"]
    heads = [3, 20]
    progress("hilbert 2k: generating")
    x = make_inputs(cfg, device="cuda", tensors=("v",))
    xs = make_inputs(cfg, device="cuda", heads=heads, tensors=("q", "k"))
    sc = float(np.float32(1.0 / math.sqrt(cfg.d)))
    paths = {o: PrismPath(cfg.T, cfg.H, cfg.W, 2, cfg.d, cfg.top_k, cfg.top_p, sc, zone_order=o)
             for o in ("raster", "hilbert")}
    res = {}
    for o, p in paths.items():
        p.shapes(x["v"], x["a"])
        qp, kp, vp = p.permute(xs["q"]), p.permute(xs["k"]), p.permute(x["v"][:, heads])
        sel = p.select(qp, kp)
        op, _ = p.forward(qp, kp, vp, sel)
        res[o] = dict(qp=qp, sel=sel, o=p.permute(op, inverse=True))
    torch.cuda.synchronize()
    progress("hilbert 2k: oracle zone statistics")
    zs = orc.zone_shapes(_np(x["v"]).reshape(cfg.N, -1), _np(x["a"]), cfg.T, cfg.H, cfg.W)
    assert not zs["near_tie"].any()
    order = orc.hilbert_zone_order(cfg.T, cfg.H, cfg.W)
    hp = paths["hilbert"]
    np.testing.assert_array_equal(hp.zone_shape.cpu().numpy(), zs["shape"])
    offs, nb = orc.block_layout(zs["shape"], order)
    assert hp.nb == nb == paths["raster"].nb
    np.testing.assert_array_equal(hp.block_offsets[:nb + 1].cpu().numpy(), offs)
    pi = torch.from_numpy(orc.permutation(cfg.T, cfg.H, cfg.W, zs["shape"], order)).cuda()
    assert torch.equal(res["hilbert"]["qp"], xs["q"][pi])
    # Hilbert block b (zone order[pos], local block j) -> raster block first[order[pos]] + j
    nblk = 512 // np.asarray(orc.candidate_shapes())[zs["shape"]].prod(axis=1)
    first = np.concatenate([[0], np.cumsum(nblk)[:-1]])
    to_raster = np.concatenate([first[m] + np.arange(nblk[m]) for m in order])
    progress("hilbert 2k: selections")
    for h in range(2):
        rows = {}
        for o in ("raster", "hilbert"):
            s = res[o]["sel"]
            co = s.offsets[h].cpu().numpy()
            rows[o] = (co, s.idx[h, :co[-1]].cpu().numpy())
        (rco, rci), (hco, hci) = rows["raster"], rows["hilbert"]
        for b in range(nb):
            got = np.sort(to_raster[hci[hco[b]:hco[b + 1]]])
            r = to_raster[b]
            np.testing.assert_array_equal(got, np.sort(rci[rco[r]:rco[r + 1]]), err_msg=f"head {h} block {b}")
    # attention: sampled Hilbert-order query blocks against the oracle
    progress("hilbert 2k: oracle attention on sampled blocks")
    pi_np = pi.cpu().numpy()
    rng = np.random.default_rng(71)
    blocks = sorted(rng.choice(nb, size=24, replace=False).tolist())
    sc2 = hp.scale
    for h in range(2):
        Qp, Kp, Vp = (orc.to_block_major(_np(t[:, h:h + 1, :]), pi_np) for t in (xs["q"], xs["k"], x["v"][:, heads]))
        Kbar = orc.pool_blocks(Kp, offs, 0)
        got = _np(res["hilbert"]["o"][:, h])
        for b in blocks:
            qbar = orc.pool_blocks(Qp[offs[b]:offs[b + 1]], np.array([0, offs[b + 1] - offs[b]]), 0)
            L = orc.block_logits(qbar, Kbar, sc2)[0]
            s_b, flag = orc.select_row(L, cfg.top_k, cfg.top_p)
            if flag:
                continue
            o_ref, _ = orc.attn_fwd_block(Qp, Kp, Vp, offs, s_b, b, 0, sc2)
            _close(got[pi_np[offs[b]:offs[b + 1]]], o_ref, "bf16", f"2k O h{heads[h]} block {b}")

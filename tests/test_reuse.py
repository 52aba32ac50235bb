"""Selection reuse across diffusion steps and the adaptive sparsity schedule
(DFSAttn article, adaptive mask caching).  The schedule's values are this
library's reading (the article gives none); the reuse semantics are checked
on the GPU against the oracle: attention of new inputs over the sets selected
from earlier ones."""
import math

import numpy as np
import pytest
import torch

from parity_bars import assert_close

from oracle import prism_oracle as orc
from workloads.synth import custom, make_inputs


def _path_module():
    import importlib
    return importlib.import_module("dynamic_block_sparse_amd.path")


def test_sparsity_schedule_moves_from_permissive_to_the_workload_values():
    path = pytest.importorskip("dynamic_block_sparse_amd.path")
    steps = 11
    ks, ps = zip(*(path.sparsity_schedule(t, steps, (64, 1.0), (16, 0.95)) for t in range(steps)))
    assert (ks[0], ps[0]) == (64, 1.0) and (ks[-1], ps[-1]) == (16, 0.95)
    assert all(a >= b for a, b in zip(ks, ks[1:])) and all(a >= b for a, b in zip(ps, ps[1:]))
    assert all(isinstance(k, int) for k in ks)
    assert ks[5] == 40 and math.isclose(ps[5], 0.975)          # the midpoint
    assert path.sparsity_schedule(0, 1, (64, 1.0), (16, 0.95)) == (16, 0.95)
    with pytest.raises(ValueError):
        path.sparsity_schedule(11, 11, (64, 1.0), (16, 0.95))


def test_reuse_pattern():
    path = pytest.importorskip("dynamic_block_sparse_amd.path")
    assert [path.reuses_selection(t, 3) for t in range(7)] == [False, True, True, False, True, True, False]
    assert not any(path.reuses_selection(t, 1) for t in range(5))
    with pytest.raises(ValueError):
        path.reuses_selection(0, 0)


CFG = custom("reuse_bf16", T=16, H=16, W=24, heads=2, d=128, dtype="bf16", top_k=3, top_p=0.8,
             kinds=(("smooth", 0.5), ("static", 0.25), ("fast1", 0.25)),
             sigma={"smooth": 0.3, "static": 1e-3, "fast1": 0.1}, n_blobs=2, blob_std=(3.0, 4.0, 4.0), seed=91)
CFG_NEXT = custom("reuse_bf16_next", T=16, H=16, W=24, heads=2, d=128, dtype="bf16", top_k=3, top_p=0.8,
                  kinds=(("smooth", 0.5), ("static", 0.25), ("fast1", 0.25)),
                  sigma={"smooth": 0.3, "static": 1e-3, "fast1": 0.1}, n_blobs=2, blob_std=(3.0, 4.0, 4.0), seed=92)


def _np(t):
    return t.detach().float().cpu().numpy()


def _close(got, want, what, grad=False, terms=None):
    assert_close(np.asarray(got), np.asarray(want), "bf16", what, grad=grad, terms=terms)


@pytest.mark.gpu
def test_reused_selection_matches_the_oracle_over_the_earlier_sets():
    path_mod = _path_module()
    x1 = make_inputs(CFG, device="cuda")
    x2 = make_inputs(CFG_NEXT, device="cuda")
    sc = float(np.float32(1.0 / math.sqrt(CFG.d)))
    path = path_mod.PrismPath(CFG.T, CFG.H, CFG.W, CFG.heads, CFG.d, CFG.top_k, CFG.top_p, sc)
    with pytest.raises(ValueError):
        path.step(x2["q"], x2["k"], x2["v"], x2["a"], x2["do"], reuse=True)
    out1 = path.step(x1["q"], x1["k"], x1["v"], x1["a"], x1["do"])
    offs_gpu = path.block_offsets[:path.nb + 1].clone()
    out2 = path.step(x2["q"], x2["k"], x2["v"], x2["a"], x2["do"], reuse=True)
    torch.cuda.synchronize()
    assert out2["selections"][0] is out1["selections"][0]
    assert torch.equal(path.block_offsets[:path.nb + 1], offs_gpu)
    path.release_selection()
    with pytest.raises(ValueError):
        path.step(x2["q"], x2["k"], x2["v"], x2["a"], x2["do"], reuse=True)
    # oracle: layout and sets from the first inputs, attention of the second ones over them
    zs = orc.zone_shapes(_np(x1["v"]).reshape(CFG.N, -1), _np(x1["a"]), CFG.T, CFG.H, CFG.W)
    assert not zs["near_tie"].any()
    offs = zs["block_offsets"]
    pi = orc.permutation(CFG.T, CFG.H, CFG.W, zs["shape"])
    for h in range(CFG.heads):
        Q1, K1 = (orc.to_block_major(_np(x1[n][:, h:h + 1, :]), pi) for n in ("q", "k"))
        L = orc.block_logits(orc.pool_blocks(Q1, offs, 0), orc.pool_blocks(K1, offs, 0), sc)
        co, ci, flags = orc.select(L, CFG.top_k, CFG.top_p)
        assert not flags.any()
        Q2, K2, V2, dO2 = (orc.to_block_major(_np(x2[n][:, h:h + 1, :]), pi) for n in ("q", "k", "v", "do"))
        att = orc.attention(Q2, K2, V2, offs, co, ci, 0, sc, dOp=dO2)
        _close(_np(out2["o"][:, h, :]), orc.to_raster(att["O"], pi), f"O h{h}")
        for g, name in (("dq", "dQ"), ("dk", "dK"), ("dv", "dV")):
            _close(_np(out2[g][:, h, :]), orc.to_raster(att[name], pi), f"{name} h{h}", grad=True,
                   terms=orc.to_raster(att["t" + name[1]], pi))

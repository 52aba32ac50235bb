"""GPU parity of sub-block scoring (prism_select_subblock) with the oracle's
subblock_logits followed by the oracle's selection: the fp32 scores equal the
float64 definition rounded once (rare one-ulp differences from the summation
order allowed), the selected sets bit-exact; at full 2K size on sampled rows."""
import math

import numpy as np
import pytest
import torch

from oracle import prism_oracle as orc
from workloads.synth import CONFIGS, custom, make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    custom("sb_bf16_d128", T=16, H=16, W=24, heads=2, d=128, dtype="bf16", top_k=3, top_p=0.8,
           kinds=(("smooth", 0.5), ("static", 0.25), ("fast1", 0.25)),
           sigma={"smooth": 0.3, "static": 1e-3, "fast1": 0.1}, n_blobs=2, blob_std=(3.0, 4.0, 4.0), seed=51),
    custom("sb_f32_d64", T=16, H=16, W=16, heads=1, d=64, dtype="f32", top_k=2, top_p=0.9,
           kinds=(("static", 0.5), ("smooth", 0.5)), sigma={"static": 1e-3, "smooth": 0.3}, seed=52),
    custom("sb_diffuse", T=16, H=16, W=16, heads=2, d=128, dtype="bf16", top_k=2, top_p=0.95,
           kinds=(("static", 1 / 3), ("aniso", 1 / 3), ("noisy", 1 / 3)),
           sigma={"static": 1e-3, "aniso": 0.1, "noisy": 1.0}, beta=0.3, seed=53),
]


def _np(t):
    return t.detach().float().cpu().numpy()


def _path(cfg, heads=None, scoring="subblock"):
    from dynamic_block_sparse_amd.path import PrismPath
    return PrismPath(cfg.T, cfg.H, cfg.W, heads or cfg.heads, cfg.d, cfg.top_k, cfg.top_p,
                     float(np.float32(1.0 / math.sqrt(cfg.d))), scoring=scoring)


def _check_scores(got, want, what):
    diff = got != want
    print(f"{what}: {int(diff.sum())} of {diff.size} scores one ulp off", flush=True)
    assert diff.mean() < 1e-4, what
    if diff.any():
        ulp = np.spacing(np.abs(want[diff]).astype(np.float32))
        assert np.all(np.abs(got[diff] - want[diff]) <= ulp), what


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_subblock_selection_small(cfg):
    print(f"case {cfg.name}", flush=True)
    x = make_inputs(cfg, device="cuda")
    path = _path(cfg)
    path.shapes(x["v"], x["a"])
    qp, kp = path.permute(x["q"]), path.permute(x["k"])
    sel = path.select(qp, kp, want_logits=True)
    torch.cuda.synchronize()
    zs = orc.zone_shapes(_np(x["v"]).reshape(cfg.N, -1), _np(x["a"]), cfg.T, cfg.H, cfg.W)
    assert not zs["near_tie"].any()
    offs = zs["block_offsets"]
    np.testing.assert_array_equal(path.block_offsets[:path.nb + 1].cpu().numpy(), offs)
    sizes = np.diff(offs)
    assert (sizes > 64).any(), "the case must hold blocks of more than one run"
    pi = orc.permutation(cfg.T, cfg.H, cfg.W, zs["shape"])
    for h in range(cfg.heads):
        Qp, Kp = (orc.to_block_major(_np(x[n][:, h:h + 1, :]), pi) for n in ("q", "k"))
        L = orc.subblock_logits(Qp, Kp, offs, 0, path.scale)
        _check_scores(sel.logits[h].cpu().numpy(), L, f"{cfg.name} h{h}")
        co, ci, flags = orc.select(L, cfg.top_k, cfg.top_p)
        og = sel.offsets[h].cpu().numpy()
        ig = sel.idx[h, :og[-1]].cpu().numpy()
        for i in range(path.nb):
            if flags[i]:
                continue
            np.testing.assert_array_equal(ig[og[i]:og[i + 1]], ci[co[i]:co[i + 1]], err_msg=f"head {h} row {i}")


def test_subblock_scores_of_64_token_pairs_are_the_plain_scores():
    cfg = CASES[0]
    x = make_inputs(cfg, device="cuda")
    path = _path(cfg)
    path.shapes(x["v"], x["a"])
    qp, kp = path.permute(x["q"]), path.permute(x["k"])
    sub = path.select(qp, kp, want_logits=True)
    plain = path.select(qp, kp, want_logits=True, scoring="block")
    torch.cuda.synchronize()
    B = np.diff(path.block_offsets[:path.nb + 1].cpu().numpy())
    small = B == 64
    assert small.any() and (~small).any()
    Ls, Lp = sub.logits.cpu().numpy(), plain.logits.cpu().numpy()
    pair = small[:, None] & small[None, :]
    for h in range(cfg.heads):
        assert (Ls[h][pair] == Lp[h][pair]).all()
        assert (Ls[h][~pair] >= Lp[h][~pair] - np.spacing(np.abs(Lp[h][~pair]))).all()   # Jensen


def test_subblock_selection_2k_sampled(progress):
    cfg = CONFIGS["2k"]
    heads = [4, 15]
    progress("sub-block 2k: generating")
    x = make_inputs(cfg, device="cuda", tensors=("v",))
    xs = make_inputs(cfg, device="cuda", heads=heads, tensors=("q", "k"))
    path = _path(cfg, heads=2)
    path.shapes(x["v"], x["a"])
    qp, kp = path.permute(xs["q"]), path.permute(xs["k"])
    sel = path.select(qp, kp, want_logits=True)
    torch.cuda.synchronize()
    progress("sub-block 2k: oracle zone statistics")
    zs = orc.zone_shapes(_np(x["v"]).reshape(cfg.N, -1), _np(x["a"]), cfg.T, cfg.H, cfg.W)
    assert not zs["near_tie"].any() and zs["NB"] == path.nb
    offs = zs["block_offsets"]
    pi = orc.permutation(cfg.T, cfg.H, cfg.W, zs["shape"])
    rng = np.random.default_rng(61)
    B = np.diff(offs)
    rows = sorted(set(rng.choice(np.nonzero(B == 256)[0], 8, replace=False).tolist()
                      + rng.choice(np.nonzero(B == 64)[0], 8, replace=False).tolist()))
    for hh, h in enumerate(heads):
        progress(f"sub-block 2k: head {h}")
        Qp, Kp = (orc.to_block_major(_np(xs[n][:, hh:hh + 1, :]), pi) for n in ("q", "k"))
        L = orc.subblock_logits(Qp, Kp, offs, 0, path.scale, rows=rows)
        got = sel.logits[hh].cpu().numpy()[rows]
        _check_scores(got, L, f"2k head {h}")
        og = sel.offsets[hh].cpu().numpy()
        ig = sel.idx[hh, :og[-1]].cpu().numpy()
        for r, i in enumerate(rows):
            s, flag = orc.select_row(L[r], cfg.top_k, cfg.top_p)
            if flag:
                continue
            np.testing.assert_array_equal(ig[og[i]:og[i + 1]], s, err_msg=f"head {h} row {i}")

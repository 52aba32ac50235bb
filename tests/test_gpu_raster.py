"""Attention outputs written straight to raster order (prism_raster_layout)
equal the block-major outputs scattered by prism_block_permute_heads, bit for
bit: the same kernels compute every row, only the row addresses differ.  The
raster path itself is compared with the oracle by the end-to-end parity tests
(PrismPath.step writes raster outputs)."""
import math

import numpy as np
import pytest
import torch

from workloads.synth import CONFIGS, custom, make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    (custom("ra_bf16_d128", T=16, H=16, W=24, heads=2, d=128, dtype="bf16", top_k=3, top_p=0.8,
            kinds=(("smooth", 0.5), ("static", 0.25), ("fast1", 0.25)),
            sigma={"smooth": 0.3, "static": 1e-3, "fast1": 0.1}, n_blobs=2, blob_std=(3.0, 4.0, 4.0), seed=81),
     "raster"),
    (custom("ra_f32_d64", T=8, H=16, W=16, heads=2, d=64, dtype="f32", top_k=4, top_p=0.9, seed=82), "raster"),
    (custom("ra_bf16_hilbert", T=16, H=24, W=16, heads=3, d=64, dtype="bf16", top_k=2, top_p=0.9,
            kinds=(("static", 0.5), ("smooth", 0.5)), sigma={"static": 1e-3, "smooth": 0.3}, seed=83), "hilbert"),
]


def _check(path, x, heads_slice=None):
    qp, kp, vp, dop = (path.permute(x[n]) for n in ("q", "k", "v", "do"))
    sel = path.select(qp, kp)
    ob = path.block_major_like(qp)
    orr = torch.empty_like(x["q"])
    rb, rr = path.residual_like(ob), path.residual_like(orr)
    _, lse = path.forward(qp, kp, vp, sel, op=ob, ores=rb)
    _, lse2 = path.forward(qp, kp, vp, sel, op=orr, raster=True, ores=rr)
    gb = path.backward(qp, kp, vp, ob, dop, lse, sel, ores=rb)
    gr = path.backward(qp, kp, vp, orr, dop, lse2, sel, raster=True, ores=rr)
    torch.cuda.synchronize()
    assert torch.equal(lse, lse2)
    assert torch.equal(path.permute(ob, inverse=True), orr)
    if rb is not None:
        assert torch.equal(path.permute(rb, inverse=True), rr)
    for name, a, b in zip(("dQ", "dK", "dV"), gb, gr):
        assert torch.equal(path.permute(a, inverse=True), b), name


@pytest.mark.parametrize("cfg,order", CASES, ids=lambda c: c.name if hasattr(c, "name") else c)
def test_raster_outputs_are_the_block_major_outputs_scattered(cfg, order):
    from dynamic_block_sparse_amd.path import PrismPath
    print(f"case {cfg.name} ({order})", flush=True)
    x = make_inputs(cfg, device="cuda")
    path = PrismPath(cfg.T, cfg.H, cfg.W, cfg.heads, cfg.d, cfg.top_k, cfg.top_p,
                     float(np.float32(1.0 / math.sqrt(cfg.d))), zone_order=order)
    path.shapes(x["v"], x["a"])
    _check(path, x)


def test_raster_outputs_2k_two_heads(progress):
    from dynamic_block_sparse_amd.path import PrismPath
    cfg = CONFIGS["2k"]
    progress("raster 2k: generating")
    xv = make_inputs(cfg, device="cuda", tensors=("v",))
    x = make_inputs(cfg, device="cuda", heads=[2, 9], tensors=("q", "k", "v", "do"))
    path = PrismPath(cfg.T, cfg.H, cfg.W, 2, cfg.d, cfg.top_k, cfg.top_p, float(np.float32(1.0 / math.sqrt(cfg.d))))
    path.shapes(xv["v"], xv["a"])
    del xv
    progress("raster 2k: attention")
    _check(path, x)

"""The no-allocation zone shapes call against the workspace call, on the GPU.

prism_zone_shapes_noalloc runs the kernels of prism_zone_shapes with their
scratch in the library's fixed device array.  Two calls in a row, the second
on a smaller grid, must each give the workspace call's outputs bit for bit:
zone shapes, block offsets, NB and the float64 zone records (the same kernels
on the same inputs sum in the same order).  The second call also shows that
what the first left in the array does not reach the outputs."""
import numpy as np
import pytest
import torch

from workloads.synth import CONFIGS, custom, make_inputs

pytestmark = pytest.mark.gpu


def _run(P, cfg, x, noalloc):
    nZ = cfg.N // 512
    C = cfg.heads * cfg.d
    v = x["v"].reshape(cfg.N, C)
    zs = torch.full((nZ,), 255, dtype=torch.uint8, device="cuda")
    offs = torch.full((8 * nZ + 1,), -1, dtype=torch.int32, device="cuda")
    nb_dev = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    rec = torch.full((nZ * P.ZS_STRIDE,), float("nan"), dtype=torch.float64, device="cuda")
    if noalloc:
        nb = P.prism_zone_shapes_noalloc(cfg.T, cfg.H, cfg.W, v, C, v.stride(0), x["a"], zs, offs, nb_dev,
                                         zone_stats=rec)
    else:
        ws = torch.empty(P.prism_workspace_size(P.OP_ZONE_SHAPES, cfg.N, 1, C, 0, 0), dtype=torch.uint8,
                         device="cuda")
        nb = P.prism_zone_shapes(cfg.T, cfg.H, cfg.W, v, C, v.stride(0), x["a"], zs, offs, nb_dev, ws,
                                 zone_stats=rec)
    torch.cuda.synchronize()
    return nb, zs.cpu(), offs.cpu(), nb_dev.cpu(), rec.cpu()


def test_noalloc_zone_shapes_match_the_workspace_call_twice():
    from dynamic_block_sparse_amd import prism as P
    small = custom("noalloc_small", T=16, H=24, W=16, heads=2, d=64, dtype="bf16", top_k=2, top_p=0.9,
                   kinds=(("static", 0.5), ("noisy", 0.5)), sigma={"static": 1e-3, "noisy": 1.0}, seed=71)
    for cfg in (CONFIGS["2k"], small):
        print(f"case {cfg.name}", flush=True)
        x = make_inputs(cfg, device="cuda", tensors=("v",))
        want = _run(P, cfg, x, noalloc=False)
        got = _run(P, cfg, x, noalloc=True)
        nb = want[0]
        assert got[0] == nb and int(got[3][0]) == nb
        assert torch.equal(got[1], want[1])
        assert torch.equal(got[2][:nb + 1], want[2][:nb + 1])
        assert torch.equal(got[4].view(torch.int64), want[4].view(torch.int64))   # float64 records, bit for bit
        print(f"case {cfg.name}: NB {nb}, outputs identical", flush=True)
        del x

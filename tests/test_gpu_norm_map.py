"""GPU parity of prism_audio_norm_map against the float64 oracle.

The norms are sums of exactly representable squares in float64, so the kernel
and the oracle agree to the last bits; the map is the float64 quotient rounded
once to float32.  Where the two float64 norms are equal bit for bit (and so are
the maxima) the maps must be equal bit for bit; anywhere else the norms must
agree to 1e-14 relative and the maps to one float32 step.
"""
import numpy as np
import pytest
import torch

from oracle import prism_oracle as orc
from workloads.synth import CONFIGS, cross_attn_output

pytestmark = pytest.mark.gpu


def _run(h, C, ld):
    from dynamic_block_sparse_amd import prism as P
    N = h.shape[0]
    a = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
    norms = torch.full((N,), float("nan"), dtype=torch.float64, device="cuda")
    ws = torch.empty(P.prism_workspace_size(P.OP_NORM_MAP, N, 0, 0, 0, 0), dtype=torch.uint8, device="cuda")
    P.prism_audio_norm_map(h, N, C, ld, a, ws, norms=norms)
    torch.cuda.synchronize()
    return norms.cpu().numpy(), a.cpu().numpy()


def _compare(got_n, got_a, want_n, want_a, what):
    np.testing.assert_allclose(got_n, want_n, rtol=1e-14, atol=0, err_msg=what)
    same = (got_n == want_n) & (got_n.max() == want_n.max())
    assert np.array_equal(got_a[same], want_a[same]), what
    ulps = np.abs(got_a.view(np.int32).astype(np.int64) - want_a.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1, what
    print(f"{what}: {int((~same).sum())} rows with different float64 rounding, max ulp {int(ulps.max())}", flush=True)


# (N, C, ld, dtype): 16-byte path with and without a tail, the element-load
# path (ld not a 16-byte multiple), one row, more rows than workgroup slots
CASES = [
    (1, 1, 1, torch.float32),
    (37, 100, 104, torch.bfloat16),
    (300, 3072, 3072, torch.bfloat16),
    (129, 513, 520, torch.float32),
    (50, 64, 67, torch.bfloat16),
    (61, 30, 33, torch.float32),
    (20000, 64, 72, torch.float32),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"N{c[0]}_C{c[1]}_ld{c[2]}_{str(c[3])[6:]}")
def test_norm_map_small(case):
    N, C, ld, dt = case
    g = torch.Generator().manual_seed(N * 131 + C)
    full = torch.randn((N, ld), generator=g) * torch.rand((N, 1), generator=g) * 3
    full[::7] *= 1e-3                       # rows of very different magnitude
    h = full.to(dt)
    want_n, want_a = orc.audio_norm_map(h[:, :C].float().numpy())
    got_n, got_a = _run(h.cuda(), C, ld)
    _compare(got_n, got_a, want_n, want_a, f"N={N} C={C} ld={ld} {dt}")


def test_norm_map_all_zero_clip():
    h = torch.zeros((100, 48), dtype=torch.bfloat16, device="cuda")
    got_n, got_a = _run(h, 48, 48)
    assert (got_n == 0).all() and (got_a == 0).all()


def test_norm_map_2k_size(progress):
    cfg = CONFIGS["2k"]
    progress("norm map 2k: generating")
    h = cross_attn_output(cfg, device="cuda")
    N, C = h.shape
    got_n, got_a = _run(h, C, C)
    progress("norm map 2k: oracle")
    want_n, want_a = orc.audio_norm_map(h.cpu().float().numpy(), chunk=32768)
    _compare(got_n, got_a, want_n, want_a, "2k")
    assert got_a.max() == 1.0 and got_a.min() >= 0.0

"""Parity of the HIP path (through the C ABI) with the float64 oracle.

Small grids (the named tiny workload among them) are compared element by
element in full; the named workloads 720p, 1080p, 2K and long are compared at
full size, in the launch configuration the benchmark uses, on seeded samples
of heads, rows and blocks, plus whole-tensor identities of the gradients.
Every expected value comes from the oracle run on the generator's inputs;
nothing from the HIP path is fed to the oracle.

Bars: zone volumes, shapes, block offsets, permutations and selected sets
bit-exact (decisions the oracle marks as lying on a boundary are reported
and excluded; none are expected); pooled scores equal to the float32 rounding
of the float64 definition; attention outputs O within max-abs 2e-2 and
mean-abs 2e-3 for bf16 inputs and 1e-4 for fp32 inputs; gradients element by
element within the same absolute bar plus the storage rounding of the
element itself (2^-8 |ref| for bf16, 2^-23 |ref| for fp32), and mean-abs
within the absolute bar scaled by max(1, mean |ref|).
"""
import math

import numpy as np
import pytest
import torch

from oracle import prism_oracle as orc
from parity_bars import TOL, assert_close, check_gradient_sums
from workloads.synth import CONFIGS, custom, make_inputs

pytestmark = pytest.mark.gpu

def _np(t):
    """Exact host copy as float32 (bf16 -> f32 is exact) or float64 for fp64."""
    if t.dtype == torch.float64:
        return t.detach().cpu().numpy()
    return t.detach().float().cpu().numpy()


def _path(cfg, heads=None, hc=None):
    from dynamic_block_sparse_amd.path import PrismPath
    return PrismPath(cfg.T, cfg.H, cfg.W, heads or cfg.heads, cfg.d, cfg.top_k, cfg.top_p,
                     float(np.float32(1.0 / math.sqrt(cfg.d))), head_chunk=hc)


SMALL = [
    custom("s_f32_d64", T=8, H=16, W=16, heads=1, d=64, dtype="f32", top_k=4, top_p=0.9, seed=11),
    custom("s_bf16_d128", T=16, H=16, W=24, heads=2, d=128, dtype="bf16", top_k=3, top_p=0.8,
           kinds=(("smooth", 0.5), ("static", 0.25), ("fast1", 0.25)),
           sigma={"smooth": 0.3, "static": 1e-3, "fast1": 0.1}, n_blobs=2, blob_std=(3.0, 4.0, 4.0), seed=12),
    custom("s_bf16_d64", T=8, H=24, W=16, heads=3, d=64, dtype="bf16", top_k=2, top_p=0.95,
           kinds=(("aniso", 0.5), ("noisy", 0.5)), sigma={"aniso": 0.1, "noisy": 1.0}, beta=3.0, seed=13),
    custom("s_f32_d128", T=16, H=8, W=16, heads=2, d=128, dtype="f32", top_k=1, top_p=0.5, beta=1.0, seed=14),
    custom("s_one_zone_k0_p0", T=8, H=8, W=8, heads=1, d=64, dtype="bf16", top_k=0, top_p=0.0, seed=15),
    custom("s_dense", T=8, H=16, W=8, heads=2, d=64, dtype="bf16", top_k=10 ** 6, top_p=0.5, seed=16),
    custom("s_p1", T=8, H=8, W=16, heads=1, d=128, dtype="bf16", top_k=1, top_p=1.0, seed=17),
    # small-norm queries: diffuse scores, Top-p keeps most blocks (the long clip's regime)
    custom("s_diffuse", T=16, H=16, W=16, heads=2, d=128, dtype="bf16", top_k=2, top_p=0.95,
           kinds=(("static", 1 / 3), ("aniso", 1 / 3), ("noisy", 1 / 3)),
           sigma={"static": 1e-3, "aniso": 0.1, "noisy": 1.0}, beta=0.3, seed=18),
    # the named tiny workload itself (8x16x16, one head of 64 channels, fp32, seed 0, forward only)
    CONFIGS["tiny"],
]


def _oracle_full(cfg, x):
    """Oracle end to end on host copies of the generator's tensors."""
    T, H, W = cfg.T, cfg.H, cfg.W
    N = cfg.N
    V = _np(x["v"]).reshape(N, -1)
    zs = orc.zone_shapes(V, _np(x["a"]), T, H, W)
    pi = orc.permutation(T, H, W, zs["shape"])
    offs = zs["block_offsets"]
    sc = float(np.float32(1.0 / math.sqrt(cfg.d)))
    res = {"zs": zs, "pi": pi, "heads": []}
    for h in range(cfg.heads):
        Qp, Kp, Vp = (orc.to_block_major(_np(x[n][:, h:h + 1, :]), pi) for n in ("q", "k", "v"))
        dOp = orc.to_block_major(_np(x["do"][:, h:h + 1, :]), pi) if "do" in x else None
        L = orc.block_logits(orc.pool_blocks(Qp, offs, 0), orc.pool_blocks(Kp, offs, 0), sc)
        co, ci, flags = orc.select(L, cfg.top_k, cfg.top_p)
        att = orc.attention(Qp, Kp, Vp, offs, co, ci, 0, sc, dOp=dOp)
        res["heads"].append(dict(L=L, co=co, ci=ci, flags=flags, att=att))
    return res


def _csr_rows(offsets, idx, nb):
    return [idx[offsets[i]:offsets[i + 1]] for i in range(nb)]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_small_end_to_end(cfg):
    print(f"case {cfg.name}", flush=True)
    x = make_inputs(cfg, device="cuda")
    path = _path(cfg)
    out = path.step(x["q"], x["k"], x["v"], x["a"], x.get("do"))
    torch.cuda.synchronize()
    ref = _oracle_full(cfg, x)
    zs = ref["zs"]
    # zone decisions and layout
    assert not zs["near_tie"].any()
    assert path.nb == zs["NB"]
    np.testing.assert_array_equal(path.zone_shape.cpu().numpy(), zs["shape"])
    np.testing.assert_array_equal(path.block_offsets[:path.nb + 1].cpu().numpy(), zs["block_offsets"])
    rec = path.zone_stats.cpu().numpy().reshape(-1, 16)
    np.testing.assert_allclose(rec[:, 0:3], zs["sigma2_v"], rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(rec[:, 3:6], zs["r"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(rec[:, 6], zs["abar"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(rec[:, 7:10], zs["sigma2_a"], rtol=1e-11, atol=1e-17)
    np.testing.assert_allclose(rec[:, 10:13], zs["vhat"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(rec[:, 13], zs["rho"], rtol=1e-12, atol=1e-15)
    np.testing.assert_array_equal(rec[:, 15], zs["B"])
    # selection (one head chunk = all heads)
    sel = out["selections"][0]
    offs_g = sel.offsets.cpu().numpy()
    idx_g = sel.idx.cpu().numpy()
    assert (sel.total.cpu().numpy() <= sel.cap).all()
    for h, hr in enumerate(ref["heads"]):
        rows_g = _csr_rows(offs_g[h], idx_g[h], path.nb)
        for i in range(path.nb):
            if hr["flags"][i]:
                continue
            np.testing.assert_array_equal(rows_g[i], hr["ci"][hr["co"][i]:hr["co"][i + 1]], err_msg=f"head {h} row {i}")
    # attention, raster order
    for h, hr in enumerate(ref["heads"]):
        att = hr["att"]
        assert_close(_np(out["o"][:, h, :]), orc.to_raster(att["O"], ref["pi"]), cfg.dtype, f"O h{h}")
        lse_g = out["lse_block_major"][h].cpu().numpy()
        np.testing.assert_allclose(lse_g, att["lse"], atol=1e-4 if cfg.dtype == "f32" else 2e-3)
        if "do" in x:
            for g, name in (("dq", "dQ"), ("dk", "dK"), ("dv", "dV")):
                assert_close(_np(out[g][:, h, :]), orc.to_raster(att[name], ref["pi"]), cfg.dtype, f"{name} h{h}",
                             grad=True, terms=orc.to_raster(att["t" + name[1]], ref["pi"]))


def test_small_selection_logits_are_the_rounded_float64_scores():
    cfg = SMALL[1]
    x = make_inputs(cfg, device="cuda")
    path = _path(cfg)
    path.shapes(x["v"], x["a"])
    qp, kp = path.permute(x["q"]), path.permute(x["k"])
    sel = path.select(qp, kp, want_logits=True)
    torch.cuda.synchronize()
    ref = _oracle_full(cfg, x)
    L = sel.logits.cpu().numpy()
    for h, hr in enumerate(ref["heads"]):
        diff = L[h] != hr["L"]
        assert diff.mean() < 1e-4
        if diff.any():
            ulp = np.spacing(np.abs(hr["L"][diff]).astype(np.float32))
            assert np.all(np.abs(L[h][diff] - hr["L"][diff]) <= ulp)


def test_small_determinism():
    cfg = SMALL[2]
    x = make_inputs(cfg, device="cuda")
    x["do"] = torch.randn_like(x["q"], dtype=torch.float32).to(x["q"].dtype)
    outs = []
    for _ in range(2):
        path = _path(cfg)
        o = path.step(x["q"], x["k"], x["v"], x["a"], x["do"])
        torch.cuda.synchronize()
        sel = o["selections"][0]
        valid = torch.cat([sel.idx[h, :int(sel.total[h])] for h in range(cfg.heads)])
        outs.append((path.zone_stats.clone(), sel.offsets.clone(), valid, o["o"], o["dq"], o["dk"], o["dv"]))
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.uint8) if a.dtype != torch.int32 else a,
                           b.view(torch.uint8) if b.dtype != torch.int32 else b)


def test_backward_head_order_is_invisible():
    """With 16 heads the dK/dV launch visits heads in a work-balanced order
    (runs of 2 heads per XCD).  Heads whose queries are scaled differently
    select different numbers of blocks, so that order is not the identity.
    One call over all heads must give, bit for bit, what one call per head
    gives (where the order is trivially the identity), and every head must
    match the oracle."""
    cfg = custom("s_16_heads", T=8, H=16, W=16, heads=16, d=64, dtype="bf16", top_k=2, top_p=0.9,
                 kinds=(("smooth", 0.5), ("noisy", 0.5)), sigma={"smooth": 0.1, "noisy": 1.0}, beta=2.0, seed=19)
    x = make_inputs(cfg, device="cuda")
    # query gains from diffuse (0.2) to sharp (3): per-head selections differ in size
    gain = torch.linspace(0.2, 3.0, cfg.heads, device="cuda").to(x["q"].dtype)
    x["q"] = (x["q"] * gain[None, :, None]).contiguous()
    runs = []
    for hc in (cfg.heads, 1):
        path = _path(cfg, hc=hc)
        out = path.step(x["q"], x["k"], x["v"], x["a"], x["do"])
        torch.cuda.synchronize()
        runs.append(out)
    tot = torch.cat([s.total for s in runs[0]["selections"]]).double()
    assert float(tot.max() / tot.min()) > 2.0, tot.tolist()
    for n in ("o", "dq", "dk", "dv"):
        assert torch.equal(runs[0][n].view(torch.uint16), runs[1][n].view(torch.uint16)), n
    ref = _oracle_full(cfg, x)
    pi = ref["pi"]
    for h, hr in enumerate(ref["heads"]):
        att = hr["att"]
        assert_close(_np(runs[0]["o"][:, h]), orc.to_raster(att["O"], pi), cfg.dtype, f"O h{h}")
        for g, name in (("dq", "dQ"), ("dk", "dK"), ("dv", "dV")):
            assert_close(_np(runs[0][g][:, h]), orc.to_raster(att[name], pi), cfg.dtype, f"{name} h{h}",
                         grad=True, terms=orc.to_raster(att["t" + name[1]], pi))


@pytest.mark.parametrize("idx", [0, 1], ids=["f32", "bf16"])
def test_zone_statistics_both_load_paths(idx):
    """The zone statistics kernel loads V rows with 16-byte direct LDS loads when
    C and the token stride allow it, and with 4-byte loads otherwise (here a
    token stride of C + 2 elements).  Both must give the oracle's decisions."""
    cfg = SMALL[idx]
    print(f"case {cfg.name}", flush=True)
    x = make_inputs(cfg, device="cuda", tensors=("v",))
    C = cfg.heads * cfg.d
    v2 = x["v"].reshape(cfg.N, C)
    wide = torch.zeros((cfg.N, C + 2), dtype=v2.dtype, device="cuda")
    wide[:, :C] = v2
    zs = orc.zone_shapes(_np(v2), _np(x["a"]), cfg.T, cfg.H, cfg.W)
    recs = []
    for v in (v2, wide[:, :C]):
        path = _path(cfg)
        path.shapes(v, x["a"])
        torch.cuda.synchronize()
        assert path.nb == zs["NB"]
        np.testing.assert_array_equal(path.zone_shape.cpu().numpy(), zs["shape"])
        np.testing.assert_array_equal(path.block_offsets[:path.nb + 1].cpu().numpy(), zs["block_offsets"])
        rec = path.zone_stats.cpu().numpy().reshape(-1, 16)
        np.testing.assert_allclose(rec[:, 0:3], zs["sigma2_v"], rtol=1e-12, atol=1e-300)
        np.testing.assert_allclose(rec[:, 3:6], zs["r"], rtol=1e-12, atol=1e-15)
        recs.append(rec)
    if cfg.dtype == "bf16":
        # same slab split and the same exact sums: bitwise equal
        np.testing.assert_array_equal(recs[0], recs[1])


@pytest.mark.parametrize("idx", [1, 2, 5, 7], ids=lambda i: SMALL[i].name)
def test_selection_kernels_agree(idx, monkeypatch):
    """prism_select keeps a row's keys in registers up to 16384 blocks and uses
    an LDS radix select beyond; PRISM_SELECT_RADIX=1 forces the latter, which
    must give the identical CSR."""
    cfg = SMALL[idx]
    print(f"case {cfg.name}", flush=True)
    x = make_inputs(cfg, device="cuda")
    path = _path(cfg)
    path.shapes(x["v"], x["a"])
    qp, kp = path.permute(x["q"]), path.permute(x["k"])
    a = path.select(qp, kp)
    monkeypatch.setenv("PRISM_SELECT_RADIX", "1")
    b = path.select(qp, kp)
    torch.cuda.synchronize()
    assert torch.equal(a.offsets, b.offsets)
    assert torch.equal(a.total, b.total)
    for h in range(cfg.heads):
        t = int(a.total[h])
        assert torch.equal(a.idx[h, :t], b.idx[h, :t])


PAIRS_D64 = custom("s_pairs_d64", T=16, H=16, W=16, heads=2, d=64, dtype="bf16", top_k=3, top_p=0.9,
                   kinds=(("static", 0.5), ("smooth", 0.5)), sigma={"static": 1e-3, "smooth": 0.3}, seed=21)


@pytest.mark.parametrize("cfg", [SMALL[1], SMALL[7], PAIRS_D64], ids=lambda c: c.name)
def test_forward_sibling_tiles_bit_identical(cfg, monkeypatch):
    """The forward runs the two 64-row tiles of a 128- or 256-token block in
    one workgroup over their shared selected list (PRISM_FWD_PAIRS=1) or one
    tile per workgroup (0, the default); each row's arithmetic is the same,
    so O, its residual and lse must be identical bit for bit."""
    print(f"case {cfg.name}", flush=True)
    x = make_inputs(cfg, device="cuda")
    path = _path(cfg)
    path.shapes(x["v"], x["a"])
    sizes = np.diff(path.block_offsets.cpu().numpy())
    assert (sizes >= 128).any(), "the grid needs blocks of more than one tile"
    qp, kp, vp = path.permute(x["q"]), path.permute(x["k"]), path.permute(x["v"])
    sel = path.select(qp, kp)
    outs = {}
    for flag in ("1", "0"):
        monkeypatch.setenv("PRISM_FWD_PAIRS", flag)
        ores = path.residual_like(path.block_major_like(qp)) if cfg.dtype == "bf16" else None
        o, lse = path.forward(qp, kp, vp, sel, ores=ores)
        torch.cuda.synchronize()
        outs[flag] = (o.clone(), lse.clone(), None if ores is None else ores.clone())
    assert torch.equal(outs["1"][0], outs["0"][0])
    assert torch.equal(outs["1"][1], outs["0"][1])
    if outs["1"][2] is not None:
        assert torch.equal(outs["1"][2], outs["0"][2])


@pytest.mark.parametrize("idx", [1, 2, 7], ids=lambda i: SMALL[i].name)
def test_selection_by_head_groups(idx, monkeypatch):
    """prism_select scores the heads in groups that fit the score budget; a
    budget of one byte forces groups of one head.  The CSR must be identical,
    with and without the caller's full score buffer, and so must the
    sub-block variant's."""
    cfg = SMALL[idx]
    print(f"case {cfg.name}", flush=True)
    x = make_inputs(cfg, device="cuda")
    path = _path(cfg)
    path.shapes(x["v"], x["a"])
    qp, kp = path.permute(x["q"]), path.permute(x["k"])
    cap = path.nb * path.nb
    ref = {s: path.select(qp, kp, cap=cap, want_logits=True, scoring=s) for s in ("block", "subblock")}
    monkeypatch.setenv("PRISM_SCORE_GROUP_BYTES", "1")
    for scoring in ("block", "subblock"):
        for want in (False, True):
            got = path.select(qp, kp, cap=cap, want_logits=want, scoring=scoring)
            torch.cuda.synchronize()
            a = ref[scoring]
            assert torch.equal(a.offsets, got.offsets), (scoring, want)
            assert torch.equal(a.total, got.total), (scoring, want)
            for h in range(cfg.heads):
                t = int(a.total[h])
                assert torch.equal(a.idx[h, :t], got.idx[h, :t]), (scoring, want, h)
            if want:
                assert torch.equal(a.logits, got.logits), scoring


@pytest.mark.parametrize("idx", [2, 7], ids=lambda i: SMALL[i].name)
def test_csr_capacity_from_counts(idx):
    """Without an explicit cap, path.select sizes the CSR from the counts: a
    short first guess is followed by one call at the largest count, and the
    CSR equals the one made with the never-truncating nb * nb."""
    cfg = SMALL[idx]
    print(f"case {cfg.name}", flush=True)
    x = make_inputs(cfg, device="cuda")
    path = _path(cfg)
    path.shapes(x["v"], x["a"])
    qp, kp = path.permute(x["q"]), path.permute(x["k"])
    full = path.select(qp, kp, cap=path.nb * path.nb)
    path._cap_seen = 1                       # a guess of one entry per head: always short here
    sized = path.select(qp, kp)
    torch.cuda.synchronize()
    need = int(full.total.max())
    assert need > 1
    assert sized.cap == need
    assert torch.equal(full.offsets, sized.offsets)
    assert torch.equal(full.total, sized.total)
    for h in range(cfg.heads):
        t = int(full.total[h])
        assert torch.equal(full.idx[h, :t], sized.idx[h, :t])


@pytest.mark.parametrize("idx", [1, 2], ids=lambda i: SMALL[i].name)
def test_vector_alu_attention_in_bf16(idx, monkeypatch):
    """PRISM_ATTN_SIMT=1 runs the bf16 attention on the vector-ALU kernels; they
    must meet the same bar against the oracle."""
    cfg = SMALL[idx]
    print(f"case {cfg.name}", flush=True)
    monkeypatch.setenv("PRISM_ATTN_SIMT", "1")
    x = make_inputs(cfg, device="cuda")
    path = _path(cfg)
    out = path.step(x["q"], x["k"], x["v"], x["a"], x.get("do"))
    torch.cuda.synchronize()
    ref = _oracle_full(cfg, x)
    for h, hr in enumerate(ref["heads"]):
        att = hr["att"]
        assert_close(_np(out["o"][:, h, :]), orc.to_raster(att["O"], ref["pi"]), cfg.dtype, f"O h{h}")
        for g, name in (("dq", "dQ"), ("dk", "dK"), ("dv", "dV")):
            assert_close(_np(out[g][:, h, :]), orc.to_raster(att[name], ref["pi"]), cfg.dtype, f"{name} h{h}",
                          grad=True)


def test_permutation_round_trip_with_strided_rows():
    cfg = SMALL[1]
    x = make_inputs(cfg, device="cuda")
    path = _path(cfg)
    path.shapes(x["v"], x["a"])
    wide = torch.zeros((cfg.N, cfg.heads + 1, cfg.d), dtype=x["q"].dtype, device="cuda")
    wide[:, :cfg.heads] = x["q"]
    view = wide[:, :cfg.heads]                       # token stride (heads+1)*d
    yp = path.permute(view)                          # all heads in one call
    back = path.permute(yp, inverse=True)
    assert torch.equal(back, x["q"])
    pi = orc.permutation(cfg.T, cfg.H, cfg.W, path.zone_shape.cpu().numpy())
    np.testing.assert_array_equal(_np(yp), _np(x["q"])[pi])
    # one call per head gives the same bytes both ways
    assert torch.equal(path.permute_per_head(view), yp)
    assert torch.equal(path.permute_per_head(yp, inverse=True), x["q"])


# ---------------------------------------------------------------- named workloads at full size

FULL = ["720p", "1080p", "2k", "long"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name, progress):
    cfg = CONFIGS[name]
    progress(f"case {name}: generating")
    rng = np.random.default_rng(1234)
    if cfg.heads_sequential:
        heads = sorted(rng.choice(cfg.heads, size=2, replace=False).tolist())
        hc = 1
    else:
        heads = None
        hc = None
    x = make_inputs(cfg, device="cuda", tensors=("v",))
    xs = make_inputs(cfg, device="cuda", heads=heads, tensors=("q", "k", "do")) if heads else \
        make_inputs(cfg, device="cuda", tensors=("q", "k", "do"))
    nh = len(heads) if heads else cfg.heads
    v_att = x["v"][:, heads] if heads else x["v"]
    path = _path(cfg, heads=nh, hc=hc)
    path.shapes(x["v"], x["a"])
    torch.cuda.synchronize()
    progress(f"case {name}: NB {path.nb}")
    # zone decisions against the oracle on all zones
    progress(f"case {name}: oracle zone statistics")
    zs = orc.zone_shapes(_np(x["v"]).reshape(cfg.N, -1), _np(x["a"]), cfg.T, cfg.H, cfg.W)
    ok = ~zs["near_tie"]
    progress(f"case {name}: near-tie zones {int((~ok).sum())}")
    assert path.nb == zs["NB"] or (~ok).any()
    np.testing.assert_array_equal(path.zone_shape.cpu().numpy()[ok], zs["shape"][ok])
    if ok.all():
        np.testing.assert_array_equal(path.block_offsets[:path.nb + 1].cpu().numpy(), zs["block_offsets"])
    pi = orc.permutation(cfg.T, cfg.H, cfg.W, zs["shape"])
    offs = zs["block_offsets"]
    nb = zs["NB"]
    # permutation: sampled rows of the permuted q
    qp, kp, vp = path.permute(xs["q"]), path.permute(xs["k"]), path.permute(v_att)
    dop = path.permute(xs["do"]) if cfg.backward else None
    rows = rng.choice(cfg.N, size=4096, replace=False)
    np.testing.assert_array_equal(_np(qp[torch.from_numpy(rows).cuda()]), _np(xs["q"][torch.from_numpy(pi[rows]).cuda()]))
    sc = float(np.float32(1.0 / math.sqrt(cfg.d)))
    check_heads = list(range(nh)) if heads else sorted(rng.choice(cfg.heads, size=min(2, cfg.heads),
                                                                    replace=False).tolist())
    # the launch configuration the benchmark times: outputs written straight to
    # raster order, head chunks as in the benchmark; NaN-filled, so every row
    # must be written whatever order the tiles are visited in
    op = torch.empty_like(xs["q"]).fill_(float("nan"))
    ores = path.residual_like(op) if cfg.backward else None
    grads = tuple(torch.empty_like(xs["q"]).fill_(float("nan")) for _ in range(3)) if cfg.backward else None
    sels, lses = {}, {}
    for h0 in range(0, nh, path.hc):
        sel = path.select(qp, kp, h0, want_logits=True)
        _, lse = path.forward(qp, kp, vp, sel, op=op, h0=h0, raster=True, ores=ores)
        if cfg.backward:
            path.backward(qp, kp, vp, op, dop, lse, sel, grads=grads, h0=h0, raster=True, ores=ores)
        for hh in range(path.hc):
            sels[h0 + hh] = (sel, hh)
            lses[h0 + hh] = lse[hh]
    torch.cuda.synchronize()
    progress(f"case {name}: GPU path done")
    for t in (op,) + (grads or ()):
        assert bool(torch.isfinite(t[:, :nh]).all())
    if cfg.backward:
        check_gradient_sums(grads[1][:, :nh], grads[2][:, :nh], xs["do"], cfg.dtype, name, log=progress)
        progress(f"case {name}: gradient sums of all {nh} heads within their bars")
    pi_t = torch.from_numpy(pi).cuda()
    bm = lambda t, a, b, h: _np(t[pi_t[a:b], h, :])   # block-major rows a..b-1 of a raster output
    for h in check_heads:
        sel, hh = sels[h]
        Qp, Kp, Vp = (orc.to_block_major(_np(t[:, h:h + 1, :]), pi) for t in (xs["q"], xs["k"], v_att))
        L = orc.block_logits(orc.pool_blocks(Qp, offs, 0), orc.pool_blocks(Kp, offs, 0), sc)
        Lg = sel.logits[hh].cpu().numpy()
        mism = Lg != L
        progress(f"case {name} head {h}: logit mismatches {int(mism.sum())} of {L.size}")
        assert mism.mean() < 1e-6
        progress(f"case {name} head {h}: oracle selection")
        co, ci, flags = orc.select(L, cfg.top_k, cfg.top_p)
        bad_rows = set(np.nonzero(mism.any(axis=1))[0].tolist()) | set(np.nonzero(flags)[0].tolist())
        og = sel.offsets[hh].cpu().numpy()
        ig = sel.idx[hh, :og[-1]].cpu().numpy()
        sizes = np.diff(co)
        progress(f"case {name} head {h}: mean |S_i| {sizes.mean():.1f} blocks ({sizes.mean() / nb:.4f} of NB), "
              f"flagged rows {int(flags.sum())}")
        for i in range(nb):
            if i in bad_rows:
                continue
            if not np.array_equal(ig[og[i]:og[i + 1]], ci[co[i]:co[i + 1]]):
                raise AssertionError(f"{name} head {h} row {i}: selection differs")
        # forward and dQ on sampled query blocks, dK/dV on sampled key blocks
        dOp = orc.to_block_major(_np(xs["do"][:, h:h + 1, :]), pi) if cfg.backward else None
        lg = lses[h].cpu().numpy()
        errs = {"O": [], "dQ": [], "dK": [], "dV": []}
        # query blocks in seeded random order, up to 64, within an oracle budget
        # of (query rows x selected keys); at least one block is checked
        qcost = lambda i: float(offs[i + 1] - offs[i]) * float(sum(offs[j + 1] - offs[j] for j in ci[co[i]:co[i + 1]]))
        qb, spent = [], 0.0
        for i in rng.permutation(nb):
            c = qcost(i)
            if qb and spent + c > 4e8:
                continue
            qb.append(i)
            spent += c
            if len(qb) >= 64:
                break
        progress(f"case {name} head {h}: checking {len(qb)} query blocks")
        for n_done, i in enumerate(qb):
            s = ci[co[i]:co[i + 1]]
            o_ref, lse_ref = orc.attn_fwd_block(Qp, Kp, Vp, offs, s, i, 0, sc)
            errs["O"].append((bm(op, offs[i], offs[i + 1], h), o_ref))
            np.testing.assert_allclose(lg[offs[i]:offs[i + 1]], lse_ref, atol=2e-3)
            if cfg.backward:
                r = orc.attn_bwd_block(Qp, Kp, Vp, dOp, offs, s, i, 0, sc, with_terms=True)
                errs["dQ"].append((bm(grads[0], offs[i], offs[i + 1], h), r[0], r[4]))
            if n_done % 8 == 7:
                progress(f"case {name} head {h}: {n_done + 1} query blocks checked")
        if cfg.backward:
            # key blocks: the cheapest first (oracle cost = query rows x selected
            # keys of every user row), at least 16 with a user, then more in
            # seeded random order while the cost stays within a budget; blocks
            # that no query block selects must have exactly zero gradients.
            users_of = _users_of_keys(co, ci, nb)
            bsz = np.diff(offs).astype(np.float64)
            keys_of_row = np.add.reduceat(bsz[ci], co[:-1]) * (np.diff(co) > 0)
            cost_of_row = bsz * keys_of_row
            kcost = np.array([float(cost_of_row[u].sum()) for u in users_of])
            used = np.array([len(u) > 0 for u in users_of])
            # oracle budgets in query rows x keys (about 1e8 per second of float64 work)
            budget, spent, picked = 2e9, 0.0, []
            for j in np.lexsort((np.arange(nb), kcost)):
                j = int(j)
                if len(picked) >= 16 or spent + kcost[j] > budget:
                    break
                if used[j]:
                    picked.append(j)
                    spent += kcost[j]
            budget = spent + 2e9
            for j in rng.permutation(nb):
                if len(picked) >= 32:
                    break
                j = int(j)
                if not used[j] or j in picked or spent + kcost[j] > budget:
                    continue
                picked.append(j)
                spent += kcost[j]
            fan = []
            for j in picked:
                u = users_of[j]
                dk_ref, dv_ref, tk, tv = orc.key_block_grads(Qp, Kp, Vp, dOp, offs, co, ci, j, 0, sc, rows=u,
                                                             with_terms=True)
                errs["dK"].append((bm(grads[1], offs[j], offs[j + 1], h), dk_ref, tk))
                errs["dV"].append((bm(grads[2], offs[j], offs[j + 1], h), dv_ref, tv))
                fan.append(len(u))
                progress(f"case {name} head {h}: key block {j} ({len(u)} users) checked")
            if fan:
                progress(f"case {name} head {h}: {len(picked)} key blocks checked for dK/dV "
                         f"(users per block: min {min(fan)}, median {int(np.median(fan))}, max {max(fan)})")
            if name != "long":   # on the long clip every key block has thousands of users
                assert len(picked) >= min(16, int(used.sum()))
            unused = np.nonzero(~used)[0]
            if unused.size:
                rows = np.concatenate([np.arange(offs[j], offs[j + 1]) for j in unused])
                for g in (1, 2):
                    assert bool((grads[g][pi_t[torch.from_numpy(rows).cuda()], h, :] == 0).all())
                progress(f"case {name} head {h}: {unused.size} unselected key blocks have zero dK, dV")
        for k, pairs in errs.items():
            if pairs:
                got = np.concatenate([p[0] for p in pairs])
                want = np.concatenate([p[1] for p in pairs])
                terms = np.concatenate([p[2] for p in pairs]) if k != "O" else None
                assert_close(got, want, cfg.dtype, f"{name} head {h} {k}", grad=(k != "O"), terms=terms,
                             log=progress)


def _users_of_keys(co, ci, nb):
    """For each key block, the query blocks whose selected set holds it
    (ascending)."""
    rows_of = np.repeat(np.arange(nb), np.diff(co))
    order = np.argsort(ci, kind="stable")
    cuts = np.searchsorted(ci[order], np.arange(nb + 1))
    return [rows_of[order[cuts[j]:cuts[j + 1]]] for j in range(nb)]


def test_degenerate_zero_values_and_map():
    """V and the audio map all zero: every zone is constant (each directional
    ratio 1/3, the reading for a zero variance sum), O is exactly 0, and so are
    dQ and dK (dP = dO V^T = 0 and D = rowsum(dO * O) = 0); dV = P^T dO is not."""
    cfg = SMALL[1]
    x = make_inputs(cfg, device="cuda")
    x["v"] = torch.zeros_like(x["v"])
    x["a"] = torch.zeros_like(x["a"])
    path = _path(cfg)
    out = path.step(x["q"], x["k"], x["v"], x["a"], x["do"])
    torch.cuda.synchronize()
    ref = _oracle_full(cfg, x)
    zs = ref["zs"]
    assert not zs["near_tie"].any()
    np.testing.assert_array_equal(path.zone_shape.cpu().numpy(), zs["shape"])
    np.testing.assert_array_equal(path.block_offsets[:path.nb + 1].cpu().numpy(), zs["block_offsets"])
    assert bool((out["o"] == 0).all()) and bool((out["dq"] == 0).all()) and bool((out["dk"] == 0).all())
    for h, hr in enumerate(ref["heads"]):
        assert_close(_np(out["dv"][:, h, :]), orc.to_raster(hr["att"]["dV"], ref["pi"]), cfg.dtype, f"dV h{h}",
                     grad=True, terms=orc.to_raster(hr["att"]["tV"], ref["pi"]))


def test_more_than_16384_blocks_uses_the_radix_selection(progress):
    """A grid of noisy zones (every block 64 tokens) with NB above 16384: the
    selection runs on the LDS radix kernel by default.  Layout bit-exact,
    sampled selection rows bit-exact, sampled forward blocks within the bar."""
    cfg = custom("nb_large", T=128, H=72, W=128, heads=1, d=128, dtype="bf16", top_k=16, top_p=0.95,
                 kinds=(("noisy", 1.0),), sigma={"noisy": 1.0}, beta=2.0, seed=19)
    progress("nb>16384: generating")
    x = make_inputs(cfg, device="cuda", tensors=("q", "k", "v"))
    path = _path(cfg)
    path.shapes(x["v"], x["a"])
    assert path.nb > 16384, path.nb
    qp, kp, vp = path.permute(x["q"]), path.permute(x["k"]), path.permute(x["v"])
    sel = path.select(qp, kp)
    op, lse = path.forward(qp, kp, vp, sel)
    torch.cuda.synchronize()
    progress(f"nb>16384: NB {path.nb}, oracle")
    zs = orc.zone_shapes(_np(x["v"]).reshape(cfg.N, -1), _np(x["a"]), cfg.T, cfg.H, cfg.W)
    assert not zs["near_tie"].any()
    offs = zs["block_offsets"]
    np.testing.assert_array_equal(path.block_offsets[:path.nb + 1].cpu().numpy(), offs)
    pi = orc.permutation(cfg.T, cfg.H, cfg.W, zs["shape"])
    sc = float(np.float32(1.0 / math.sqrt(cfg.d)))
    Qp, Kp, Vp = (orc.to_block_major(_np(x[n]), pi) for n in ("q", "k", "v"))
    Kbar = orc.pool_blocks(Kp, offs, 0)
    og = sel.offsets[0].cpu().numpy()
    ig = sel.idx[0, :og[-1]].cpu().numpy()
    Og = _np(op[:, 0, :])
    rng = np.random.default_rng(23)
    checked, pairs = 0, []
    for i in sorted(rng.choice(path.nb, size=24, replace=False).tolist()):
        qbar = orc.pool_blocks(Qp[offs[i]:offs[i + 1]], np.array([0, offs[i + 1] - offs[i]]), 0)
        L = orc.block_logits(qbar, Kbar, sc)[0]
        s, flag = orc.select_row(L, cfg.top_k, cfg.top_p)
        if flag:
            continue
        np.testing.assert_array_equal(ig[og[i]:og[i + 1]], s, err_msg=f"row {i}")
        o_ref, _ = orc.attn_fwd_block(Qp, Kp, Vp, offs, s, i, 0, sc)
        pairs.append((Og[offs[i]:offs[i + 1]], o_ref))
        checked += 1
    assert checked >= 12
    assert_close(np.concatenate([p[0] for p in pairs]), np.concatenate([p[1] for p in pairs]), cfg.dtype,
                  "nb>16384 O")


def test_maximum_block_count(progress):
    """NB at the library's 32768-block limit (a 128^3 grid of noisy zones, every
    block 64 tokens): the radix selection's LDS holds the whole row (128 KB).
    Layout bit-exact; on sampled query blocks the selection rows are bit-exact
    and O, lse and dQ are within the bars; every O, dQ, dK and dV row is written
    and finite (NaN-filled beforehand).  The noise level that puts every zone
    at 64-token blocks leaves Q at a spread of about 8 and K, V at about 4; they
    are scaled by powers of two (exact in bf16): K and V to unit spread, Q to a
    spread of 4, which keeps scores of spread 4 and O at unit scale, where the
    bars (absolute for O) are stated.  The zone decisions are ratios of V
    statistics and do not change."""
    cfg = custom("nb_max", T=128, H=128, W=128, heads=1, d=128, dtype="bf16", top_k=16, top_p=0.95,
                 kinds=(("noisy", 1.0),), sigma={"noisy": 4.0}, beta=2.0, seed=19)
    progress("nb max: generating")
    x = make_inputs(cfg, device="cuda", tensors=("q", "k", "v", "do"))
    for n, f in (("q", 0.5), ("k", 0.25), ("v", 0.25)):
        x[n] = x[n] * f
    path = _path(cfg)
    path.shapes(x["v"], x["a"])
    assert path.nb == 32768, path.nb
    qp, kp, vp, dop = (path.permute(x[n]) for n in ("q", "k", "v", "do"))
    sel = path.select(qp, kp)
    op = path.block_major_like(qp).fill_(float("nan"))
    ores = path.residual_like(op)
    _, lse = path.forward(qp, kp, vp, sel, op=op, ores=ores)
    grads = tuple(path.block_major_like(qp).fill_(float("nan")) for _ in range(3))
    path.backward(qp, kp, vp, op, dop, lse, sel, grads=grads, ores=ores)
    torch.cuda.synchronize()
    for t in (op,) + grads:
        assert bool(torch.isfinite(t).all())
    progress("nb max: oracle")
    zs = orc.zone_shapes(_np(x["v"]).reshape(cfg.N, -1), _np(x["a"]), cfg.T, cfg.H, cfg.W)
    assert not zs["near_tie"].any()
    offs = zs["block_offsets"]
    np.testing.assert_array_equal(path.block_offsets[:path.nb + 1].cpu().numpy(), offs)
    pi = orc.permutation(cfg.T, cfg.H, cfg.W, zs["shape"])
    sc = float(np.float32(1.0 / math.sqrt(cfg.d)))
    Qp, Kp, Vp, dOp = (orc.to_block_major(_np(x[n]), pi) for n in ("q", "k", "v", "do"))
    Kbar = orc.pool_blocks(Kp, offs, 0)
    og = sel.offsets[0].cpu().numpy()
    ig = sel.idx[0, :og[-1]].cpu().numpy()
    Og, dQg, lg = _np(op[:, 0, :]), _np(grads[0][:, 0, :]), lse[0].cpu().numpy()
    rng = np.random.default_rng(29)
    o_pairs, dq_pairs = [], []
    for i in sorted(rng.choice(path.nb, size=24, replace=False).tolist()):
        qbar = orc.pool_blocks(Qp[offs[i]:offs[i + 1]], np.array([0, offs[i + 1] - offs[i]]), 0)
        s, flag = orc.select_row(orc.block_logits(qbar, Kbar, sc)[0], cfg.top_k, cfg.top_p)
        if flag:
            continue
        np.testing.assert_array_equal(ig[og[i]:og[i + 1]], s, err_msg=f"row {i}")
        o_ref, lse_ref = orc.attn_fwd_block(Qp, Kp, Vp, offs, s, i, 0, sc)
        np.testing.assert_allclose(lg[offs[i]:offs[i + 1]], lse_ref, atol=2e-3)
        o_pairs.append((Og[offs[i]:offs[i + 1]], o_ref))
        r = orc.attn_bwd_block(Qp, Kp, Vp, dOp, offs, s, i, 0, sc, with_terms=True)
        dq_pairs.append((dQg[offs[i]:offs[i + 1]], r[0], r[4]))
    assert len(o_pairs) >= 12
    assert max(float(np.abs(p[1]).max()) for p in o_pairs) > 0.5   # O at unit scale
    progress(f"nb max: {len(o_pairs)} query blocks checked")
    for what, pairs, grad in (("O", o_pairs, False), ("dQ", dq_pairs, True)):
        assert_close(np.concatenate([p[0] for p in pairs]), np.concatenate([p[1] for p in pairs]), cfg.dtype,
                     f"nb max {what}", grad=grad, terms=np.concatenate([p[2] for p in pairs]) if grad else None)


def test_high_fan_in_key_block(progress):
    """dK and dV of a key block that more than a thousand query blocks select:
    the long accumulation over its users' rows (the regime of the long clip,
    where a key block has thousands of users), small enough for the float64
    oracle.  A grid of noisy zones (blocks of 64 tokens); every query gets a
    shared offset w along a unit vector u, and the key rows of one block get
    c u on top of their own values, so that this block ranks near the top of
    every row.  Selection bit-exact on all rows; the block's dK and dV in full
    against the oracle, summed over all of its users; O and dQ on sampled user
    blocks."""
    cfg = custom("hub", T=32, H=64, W=64, heads=1, d=128, dtype="bf16", top_k=8, top_p=0.5,
                 kinds=(("noisy", 1.0),), sigma={"noisy": 1.0}, beta=1.0, seed=31)
    progress("hub: generating")
    x = make_inputs(cfg, device="cuda")
    path = _path(cfg)
    path.shapes(x["v"], x["a"])
    torch.cuda.synchronize()
    zs = orc.zone_shapes(_np(x["v"]).reshape(cfg.N, -1), _np(x["a"]), cfg.T, cfg.H, cfg.W)
    assert not zs["near_tie"].any()
    offs, nb = zs["block_offsets"], zs["NB"]
    np.testing.assert_array_equal(path.block_offsets[:path.nb + 1].cpu().numpy(), offs)
    pi = orc.permutation(cfg.T, cfg.H, cfg.W, zs["shape"])
    g = torch.Generator().manual_seed(5)
    u = torch.randn(cfg.d, generator=g, dtype=torch.float64)
    u = (u / u.norm()).float().cuda()
    hub = nb // 2 + 3
    q = (x["q"].float() + 4.0 * u).to(torch.bfloat16)
    k = x["k"].float()
    k[torch.from_numpy(pi[offs[hub]:offs[hub + 1]]).cuda(), 0, :] += 25.0 * u
    k = k.to(torch.bfloat16)
    qp, kp, vp, dop = (path.permute(t) for t in (q, k, x["v"], x["do"]))
    sel = path.select(qp, kp)
    op = torch.empty_like(q).fill_(float("nan"))
    ores = path.residual_like(op)
    grads = tuple(torch.empty_like(q).fill_(float("nan")) for _ in range(3))
    _, lse = path.forward(qp, kp, vp, sel, op=op, raster=True, ores=ores)
    path.backward(qp, kp, vp, op, dop, lse, sel, grads=grads, raster=True, ores=ores)
    torch.cuda.synchronize()
    for t in (op,) + grads:
        assert bool(torch.isfinite(t).all())
    progress(f"hub: GPU path done (NB {nb}), oracle")
    sc = float(np.float32(1.0 / math.sqrt(cfg.d)))
    Qp, Kp, Vp, dOp = (orc.to_block_major(_np(t), pi) for t in (q, k, x["v"], x["do"]))
    L = orc.block_logits(orc.pool_blocks(Qp, offs, 0), orc.pool_blocks(Kp, offs, 0), sc)
    co, ci, flags = orc.select(L, cfg.top_k, cfg.top_p)
    og = sel.offsets[0].cpu().numpy()
    ig = sel.idx[0, :og[-1]].cpu().numpy()
    for i in range(nb):
        if not flags[i]:
            np.testing.assert_array_equal(ig[og[i]:og[i + 1]], ci[co[i]:co[i + 1]], err_msg=f"row {i}")
    users = _users_of_keys(co, ci, nb)[hub]
    progress(f"hub: key block {hub} has {len(users)} users; mean |S_i| {np.diff(co).mean():.1f}")
    assert len(users) >= 1000
    dk_ref, dv_ref, tk, tv = orc.key_block_grads(Qp, Kp, Vp, dOp, offs, co, ci, hub, 0, sc, rows=users,
                                                 with_terms=True)
    pi_t = torch.from_numpy(pi).cuda()
    rows = pi_t[offs[hub]:offs[hub + 1]]
    assert_close(_np(grads[1][rows, 0, :]), dk_ref, cfg.dtype, "hub dK", grad=True, terms=tk)
    assert_close(_np(grads[2][rows, 0, :]), dv_ref, cfg.dtype, "hub dV", grad=True, terms=tv)
    rng = np.random.default_rng(37)
    o_pairs, dq_pairs = [], []
    for i in sorted(rng.choice(users, size=16, replace=False).tolist()):
        s = ci[co[i]:co[i + 1]]
        r = pi_t[offs[i]:offs[i + 1]]
        o_ref, _ = orc.attn_fwd_block(Qp, Kp, Vp, offs, s, i, 0, sc)
        o_pairs.append((_np(op[r, 0, :]), o_ref))
        rb = orc.attn_bwd_block(Qp, Kp, Vp, dOp, offs, s, i, 0, sc, with_terms=True)
        dq_pairs.append((_np(grads[0][r, 0, :]), rb[0], rb[4]))
    assert_close(np.concatenate([p[0] for p in o_pairs]), np.concatenate([p[1] for p in o_pairs]), cfg.dtype,
                  "hub O")
    assert_close(np.concatenate([p[0] for p in dq_pairs]), np.concatenate([p[1] for p in dq_pairs]), cfg.dtype,
                 "hub dQ", grad=True, terms=np.concatenate([p[2] for p in dq_pairs]))
    check_gradient_sums(grads[1], grads[2], x["do"], cfg.dtype, "hub")


def test_truncated_selection_attends_over_the_stored_entries():
    """A CSR cut short by a small capacity is not a valid selection, but the
    attention calls are documented for it: each row attends over the entries
    stored for it below cap (a prefix of its ascending list), and a row with
    none gets O = 0 and lse = -inf and contributes no gradient.  sel_total
    still reports the entries each head needed."""
    cfg = SMALL[1]
    x = make_inputs(cfg, device="cuda")
    path = _path(cfg)
    path.shapes(x["v"], x["a"])
    qp, kp, vp, dop = (path.permute(x[n]) for n in ("q", "k", "v", "do"))
    full = path.select(qp, kp)
    need = full.total.cpu().numpy()
    cap = int(need.min()) // 2
    sel = path.select(qp, kp, cap=cap)
    op = path.block_major_like(qp)
    ores = path.residual_like(op)
    _, lse = path.forward(qp, kp, vp, sel, op=op, ores=ores)
    grads = path.backward(qp, kp, vp, op, dop, lse, sel, ores=ores)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sel.total.cpu().numpy(), need)
    ref = _oracle_full(cfg, x)
    offs, pi = ref["zs"]["block_offsets"], ref["pi"]
    nb = len(offs) - 1
    sc = float(np.float32(1.0 / math.sqrt(cfg.d)))
    N, d = cfg.N, cfg.d
    empty_rows = 0
    for h, hr in enumerate(ref["heads"]):
        co, ci = hr["co"], hr["ci"]
        np.testing.assert_array_equal(sel.offsets[h].cpu().numpy(), co)
        np.testing.assert_array_equal(sel.idx[h, :cap].cpu().numpy(), ci[:cap])
        Qp, Kp, Vp, dOp = (orc.to_block_major(_np(x[n][:, h:h + 1, :]), pi) for n in ("q", "k", "v", "do"))
        O, L = np.zeros((N, d)), np.full(N, -np.inf)
        dQ, dK, dV = np.zeros((N, d)), np.zeros((N, d)), np.zeros((N, d))
        tQ, tK, tV = np.zeros((N, d)), np.zeros((N, d)), np.zeros((N, d))
        for i in range(nb):
            stored = ci[co[i]:max(co[i], min(co[i + 1], cap))]
            if stored.size == 0:
                empty_rows += 1
                continue
            O[offs[i]:offs[i + 1]], L[offs[i]:offs[i + 1]] = orc.attn_fwd_block(Qp, Kp, Vp, offs, stored, i, 0, sc)
            dq, keys, dk, dv, tq, tk, tv = orc.attn_bwd_block(Qp, Kp, Vp, dOp, offs, stored, i, 0, sc,
                                                              with_terms=True)
            dQ[offs[i]:offs[i + 1]] = dq
            dK[keys] += dk
            dV[keys] += dv
            tQ[offs[i]:offs[i + 1]] = tq
            tK[keys] += tk
            tV[keys] += tv
        assert_close(_np(op[:, h, :]), O, cfg.dtype, f"truncated O h{h}")
        lg = lse[h].cpu().numpy()
        fin = np.isfinite(L)
        assert (lg[~fin] == -np.inf).all()
        np.testing.assert_allclose(lg[fin], L[fin], atol=2e-3)
        for g, want, t, name in zip(grads, (dQ, dK, dV), (tQ, tK, tV), ("dQ", "dK", "dV")):
            assert_close(_np(g[:, h, :]), want, cfg.dtype, f"truncated {name} h{h}", grad=True, terms=t)
    assert empty_rows > 0


@pytest.mark.parametrize("w,group", [(3, 8), (1, 1), (5, 2)], ids=["w3", "w1_group1", "w5_group2"])
def test_split_rows_match_the_oracle(w, group, monkeypatch):
    """The forward and dQ split rows with long selected lists into key-range
    chunks and merge the chunks' partials.  Forced on every row of a small
    diffuse grid (a threshold of one key tile, ranges of w blocks, heads in
    groups of `group`): O, lse and the gradients against the oracle in full,
    and run to run bitwise."""
    cfg = SMALL[7]     # s_diffuse: Top-p keeps most blocks
    print(f"case {cfg.name} W={w} group={group}", flush=True)
    monkeypatch.setenv("PRISM_SPLIT_T", "1")
    monkeypatch.setenv("PRISM_SPLIT_W", str(w))
    monkeypatch.setenv("PRISM_SPLIT_GROUP", str(group))
    monkeypatch.setenv("PRISM_SPLIT_SLOTS", "256")    # room for every row's chunks
    x = make_inputs(cfg, device="cuda")
    outs = []
    for _ in range(2):
        path = _path(cfg)
        outs.append(path.step(x["q"], x["k"], x["v"], x["a"], x["do"]))
    monkeypatch.setenv("PRISM_SPLIT_T", "0")
    whole = _path(cfg).step(x["q"], x["k"], x["v"], x["a"], x["do"])
    torch.cuda.synchronize()
    for n in ("o", "dq", "dk", "dv"):
        assert torch.equal(outs[0][n], outs[1][n]), n
    # merged chunks sum in another order than one pass over the whole list
    assert not torch.equal(outs[0]["o"], whole["o"]) and not torch.equal(outs[0]["dq"], whole["dq"])
    out = outs[0]
    ref = _oracle_full(cfg, x)
    for h, hr in enumerate(ref["heads"]):
        att = hr["att"]
        assert_close(_np(out["o"][:, h, :]), orc.to_raster(att["O"], ref["pi"]), cfg.dtype, f"split O h{h}")
        np.testing.assert_allclose(out["lse_block_major"][h].cpu().numpy(), att["lse"], atol=2e-3)
        for g, name in (("dq", "dQ"), ("dk", "dK"), ("dv", "dV")):
            assert_close(_np(out[g][:, h, :]), orc.to_raster(att[name], ref["pi"]), cfg.dtype, f"split {name} h{h}",
                         grad=True, terms=orc.to_raster(att["t" + name[1]], ref["pi"]))

"""Seeded synthetic inputs shaped like the video-token workloads of the Prism pages.

The Prism pages train and measure on native 720p / 1080p / 2K joint video-audio
clips whose latent grids hold from hundreds of thousands to over a million
tokens (reading guide at xyznot.com, "Vấn đề và động lực"); no such clips,
weights or cached cross-attention norms exist here, so these generators stand in
for them with the same grid sizes, head layout and value structure.

This module only draws random numbers and lays them out.  It holds none of the
method's arithmetic (no zone statistics, no shapes, no pooling, no selection,
no attention): the HIP path and the float64 oracle both receive the tensors it
returns, bit for bit.

Recipe (all parameters are builder choices unless marked as taken from the
workload description):
  * Zones are 8x8x8 token cubes in raster order.  Each zone gets a kind:
      smooth  - frequency vector f (cycles/token per axis) log-uniform in
                [1/64, 1/16] on every axis
      static  - f = 0 (near-constant values)
      fast1   - f = 1/4 on one random axis, 0 on the others
      aniso   - 1/4, 1/16 and 0 on a random permutation of the axes
      noisy   - a smooth field under heavy noise (sigma = 1)
  * Channel c of a tensor in zone m at token (t, h, w):
        X = alpha_c * sin(2*pi*f_m.(t,h,w) + phi_{m,c}) + sigma_m * xi
    with alpha_c ~ U[0.5, 1.5], phi_{m,c} = phi0_c + 2*pi*kappa_c.(zone coords),
    kappa_c ~ U[-kappa, kappa]^3 cycles per zone (so neighbouring zones look
    alike and far zones decorrelate), xi ~ N(0, 1).
  * Q and K share alpha and phi (the query/key coupling that makes pooled
    scores informative); V draws its own.  Q is scaled by a gain beta that sets
    how concentrated the block scores are.
  * The audio-to-video norm map a is a sum of Gaussian blobs (plus an optional
    background level), clipped to [0, 1].
  * dO ~ N(0, 1) for configurations with a backward pass.
Noise streams are seeded per (config, tensor, head), so a single head can be
regenerated on its own with the same bits as when all heads are generated.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, asdict

import torch


@dataclass(frozen=True)
class Config:
    name: str
    T: int
    H: int
    W: int
    heads: int
    d: int
    dtype: str               # "f32" or "bf16"
    top_k: int
    top_p: float
    backward: bool
    kinds: tuple             # zone kinds and their shares
    sigma: dict              # noise level per zone kind
    n_blobs: int
    blob_cover: float        # fraction of tokens with a >= 0.5 (None: explicit std)
    blob_std: tuple | None   # explicit per-axis std of a blob (tokens)
    a_background: float
    beta: float              # query gain
    kappa: float = 0.15      # phase drift between zones (cycles per zone)
    heads_sequential: bool = False
    seed: int = 0

    @property
    def N(self):
        return self.T * self.H * self.W

    @property
    def n_zones(self):
        return (self.T // 8) * (self.H // 8) * (self.W // 8)

    def describe(self):
        d = asdict(self)
        d["N"] = self.N
        return d


CONFIGS = {
    # 8x16x16 grid, one head of 64 channels in fp32, forward only; every zone a
    # smooth anisotropic field with light noise and one blob of audio coupling.
    "tiny": Config("tiny", 8, 16, 16, 1, 64, "f32", 4, 0.9, False,
                   kinds=(("smooth", 1.0),), sigma={"smooth": 0.1},
                   n_blobs=1, blob_cover=None, blob_std=(2.0, 4.0, 4.0),
                   a_background=0.0, beta=2.0, seed=0),
    # 720p-like 32x48x80 grid, 24 heads x 128, bf16, forward only.
    "720p": Config("720p", 32, 48, 80, 24, 128, "bf16", 8, 0.9, False,
                   kinds=(("smooth", 1.0),), sigma={"smooth": 1.0},
                   n_blobs=3, blob_cover=0.05, blob_std=None,
                   a_background=0.0, beta=2.5, seed=1),
    # 1080p-like 32x72x120 grid: half static zones, half fast along one axis.
    "1080p": Config("1080p", 32, 72, 120, 24, 128, "bf16", 8, 0.95, True,
                    kinds=(("static", 0.5), ("fast1", 0.5)),
                    sigma={"static": 1e-3, "fast1": 0.1},
                    n_blobs=3, blob_cover=0.03, blob_std=None,
                    a_background=0.0, beta=5.0, seed=2),
    # 2K-like 64x72x128 grid: thirds of static, anisotropic and noisy zones.
    "2k": Config("2k", 64, 72, 128, 24, 128, "bf16", 16, 0.95, True,
                 kinds=(("static", 1 / 3), ("aniso", 1 / 3), ("noisy", 1 / 3)),
                 sigma={"static": 1e-3, "aniso": 0.1, "noisy": 1.0},
                 n_blobs=5, blob_cover=0.04, blob_std=None,
                 a_background=0.0, beta=6.0, seed=3),
    # long 2K clip 120x72x128: the 2K zone mix, small-norm (diffuse) queries,
    # uniform 0.05 audio background plus one strong blob; heads one at a time.
    "long": Config("long", 120, 72, 128, 24, 128, "bf16", 16, 0.95, True,
                   kinds=(("static", 1 / 3), ("aniso", 1 / 3), ("noisy", 1 / 3)),
                   sigma={"static": 1e-3, "aniso": 0.1, "noisy": 1.0},
                   n_blobs=1, blob_cover=0.02, blob_std=None,
                   a_background=0.05, beta=3.0, heads_sequential=True, seed=4),
}


def custom(name="custom", T=8, H=16, W=16, heads=1, d=64, dtype="f32", top_k=4,
           top_p=0.9, backward=True, kinds=(("smooth", 1.0),), sigma=None,
           n_blobs=1, blob_cover=None, blob_std=(2.0, 4.0, 4.0), a_background=0.0,
           beta=2.0, kappa=0.15, seed=100):
    """A small configuration for parity cases at sizes other than the named ones."""
    if sigma is None:
        sigma = {k: 0.1 for k, _ in kinds}
    return Config(name, T, H, W, heads, d, dtype, top_k, top_p, backward, tuple(kinds),
                  dict(sigma), n_blobs, blob_cover, blob_std, a_background, beta, kappa,
                  False, seed)


# ----------------------------------------------------------------------------
# parameter draws (small, on the CPU, from one seeded generator per config)

def _zone_params(cfg: Config):
    g = torch.Generator().manual_seed(1_000_003 * (cfg.seed + 1))
    nT, nH, nW = cfg.T // 8, cfg.H // 8, cfg.W // 8
    nZ = nT * nH * nW
    # kind per zone: exact shares, then shuffled
    counts = []
    acc = 0
    for i, (_, share) in enumerate(cfg.kinds):
        c = round(share * nZ) if i < len(cfg.kinds) - 1 else nZ - acc
        counts.append(c)
        acc += c
    labels = []
    for (kind, _), c in zip(cfg.kinds, counts):
        labels += [kind] * c
    perm = torch.randperm(nZ, generator=g).tolist()
    kinds = [labels[p] for p in perm]
    freq = torch.zeros(nZ, 3, dtype=torch.float64)
    sig = torch.zeros(nZ, dtype=torch.float64)
    for m, kind in enumerate(kinds):
        if kind in ("smooth", "noisy"):
            u = torch.rand(3, generator=g, dtype=torch.float64)
            freq[m] = torch.exp(math.log(1 / 64) + u * (math.log(1 / 16) - math.log(1 / 64)))
        elif kind == "static":
            pass
        elif kind == "fast1":
            ax = int(torch.randint(0, 3, (1,), generator=g))
            freq[m, ax] = 0.25
        elif kind == "aniso":
            order = torch.randperm(3, generator=g)
            freq[m, order[0]] = 0.25
            freq[m, order[1]] = 1 / 16
        else:
            raise ValueError(kind)
        sig[m] = cfg.sigma[kind]
    zt = torch.arange(nT).repeat_interleave(nH * nW)
    zh = torch.arange(nH).repeat_interleave(nW).repeat(nT)
    zw = torch.arange(nW).repeat(nT * nH)
    zc = torch.stack([zt, zh, zw], 1).to(torch.float64)
    return kinds, freq, sig, zc


def _channel_params(cfg: Config, which: str):
    tag = {"qk": 11, "v": 23}[which]
    g = torch.Generator().manual_seed(7_919 * (cfg.seed + 1) + tag)
    C = cfg.heads * cfg.d
    alpha = 0.5 + torch.rand(C, generator=g, dtype=torch.float64)
    phi0 = 2 * math.pi * torch.rand(C, generator=g, dtype=torch.float64)
    kap = (2 * torch.rand(C, 3, generator=g, dtype=torch.float64) - 1) * cfg.kappa
    return alpha, phi0, kap


def _noise_gen(cfg: Config, tensor_id: int, head: int, device):
    g = torch.Generator(device=device)
    g.manual_seed(((cfg.seed + 1) * 1_000_000 + tensor_id * 10_000 + head) & 0x7FFFFFFFFFFF)
    return g


def _token_zone_and_phase_base(cfg: Config, freq, device):
    """per-token zone index and the scalar 2*pi*f_m.(t,h,w)"""
    T, H, W = cfg.T, cfg.H, cfg.W
    t = torch.arange(T, device=device).view(T, 1, 1).expand(T, H, W).reshape(-1)
    h = torch.arange(H, device=device).view(1, H, 1).expand(T, H, W).reshape(-1)
    w = torch.arange(W, device=device).view(1, 1, W).expand(T, H, W).reshape(-1)
    nH, nW = H // 8, W // 8
    zone = ((t // 8) * nH + (h // 8)) * nW + (w // 8)
    f = freq.to(device=device, dtype=torch.float32)[zone]
    pos = torch.stack([t, h, w], 1).to(torch.float32)
    theta = 2 * math.pi * (f * pos).sum(1)
    return zone, theta


def _field_head(cfg, head, tensor_id, params, zone, theta, sig_tok, gain, device):
    alpha, phi0, kap, zc = params
    d = cfg.d
    sl = slice(head * d, (head + 1) * d)
    # phase table per (zone, channel of this head)
    phi = (phi0[sl].view(1, d) + 2 * math.pi * (zc @ kap[sl].T)).to(device=device, dtype=torch.float32)
    a = alpha[sl].to(device=device, dtype=torch.float32)
    x = torch.sin(theta.view(-1, 1) + phi[zone]) * a.view(1, d)
    g = _noise_gen(cfg, tensor_id, head, device)
    x += sig_tok.view(-1, 1) * torch.randn(x.shape, generator=g, device=device, dtype=torch.float32)
    if gain != 1.0:
        x *= gain
    return x


def _out_dtype(cfg):
    return torch.float32 if cfg.dtype == "f32" else torch.bfloat16


def audio_map(cfg: Config, device="cpu"):
    """Gaussian blobs (peak 1) plus a background level, clipped to [0, 1]; fp32 [N]."""
    g = torch.Generator().manual_seed(104_729 * (cfg.seed + 1) + 5)
    T, H, W = cfg.T, cfg.H, cfg.W
    dims = torch.tensor([T, H, W], dtype=torch.float64)
    if cfg.blob_std is not None:
        std = torch.tensor(cfg.blob_std, dtype=torch.float64).repeat(cfg.n_blobs, 1)
    else:
        # an ellipsoid with a >= 0.5 has volume (4/3)pi(2 ln 2)^(3/2) * prod(std)
        vol_unit = 4.0 / 3.0 * math.pi * (2 * math.log(2)) ** 1.5
        kfrac = (cfg.blob_cover / (cfg.n_blobs * vol_unit)) ** (1 / 3)
        std = (kfrac * dims).repeat(cfg.n_blobs, 1)
    centers = torch.rand(cfg.n_blobs, 3, generator=g, dtype=torch.float64) * dims
    t = torch.arange(T, dtype=torch.float32, device=device).view(T, 1, 1)
    h = torch.arange(H, dtype=torch.float32, device=device).view(1, H, 1)
    w = torch.arange(W, dtype=torch.float32, device=device).view(1, 1, W)
    a = torch.full((T, H, W), float(cfg.a_background), dtype=torch.float32, device=device)
    for b in range(cfg.n_blobs):
        c = centers[b].tolist()
        s = std[b].tolist()
        r2 = ((t - c[0]) / s[0]) ** 2 + ((h - c[1]) / s[1]) ** 2 + ((w - c[2]) / s[2]) ** 2
        a += torch.exp(-0.5 * r2)
    return a.clamp_(0.0, 1.0).reshape(-1).contiguous()


def cross_attn_output(cfg: Config | str, device="cpu", channels=None, chunk=65536):
    """Synthetic audio-to-video cross-attention output h [N, C] in the config's
    dtype (C = heads * d unless `channels` is given): row n is seeded Gaussian
    noise times (audio_map(n) + 0.01) / sqrt(C), so the per-token magnitude
    follows the audio map's blobs.  Generated `chunk` rows at a time."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    device = torch.device(device)
    C = int(channels or cfg.heads * cfg.d)
    scale = (audio_map(cfg, device) + 0.01) * (1.0 / math.sqrt(C))
    g = torch.Generator(device=device)
    g.manual_seed((cfg.seed + 1) * 7_919_000 + 17)
    out = torch.empty((cfg.N, C), dtype=_out_dtype(cfg), device=device)
    for r0 in range(0, cfg.N, chunk):
        r1 = min(cfg.N, r0 + chunk)
        x = torch.randn((r1 - r0, C), generator=g, device=device, dtype=torch.float32)
        x *= scale[r0:r1].view(-1, 1)
        out[r0:r1] = x.to(out.dtype)
    return out


def make_inputs(cfg: Config | str, device="cpu", heads=None, tensors=("q", "k", "v", "do")):
    """Generate the inputs of one configuration.

    Returns a dict with raster-order tensors q, k, v (and do when the config has
    a backward pass) of shape [N, nh, d] in the config's dtype, the fp32 audio
    map a [N], and the scalar parameters.  `heads` restricts generation to a
    list of head indices (nh = len(heads)); their values equal the
    corresponding heads of a full generation on the same device type.
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    device = torch.device(device)
    heads = list(range(cfg.heads)) if heads is None else list(heads)
    kinds, freq, sig, zc = _zone_params(cfg)
    zone, theta = _token_zone_and_phase_base(cfg, freq, device)
    sig_tok = sig.to(device=device, dtype=torch.float32)[zone]
    out = {"cfg": cfg, "zone_kinds": kinds, "heads": heads}
    odt = _out_dtype(cfg)
    want = [t for t in tensors if t != "do" or cfg.backward]
    pqk = _channel_params(cfg, "qk") + (zc,)
    pv = _channel_params(cfg, "v") + (zc,)
    for name in want:
        buf = torch.empty((cfg.N, len(heads), cfg.d), dtype=odt, device=device)
        for i, hd in enumerate(heads):
            if name == "q":
                x = _field_head(cfg, hd, 1, pqk, zone, theta, sig_tok, cfg.beta, device)
            elif name == "k":
                x = _field_head(cfg, hd, 2, pqk, zone, theta, sig_tok, 1.0, device)
            elif name == "v":
                x = _field_head(cfg, hd, 3, pv, zone, theta, sig_tok, 1.0, device)
            else:
                g = _noise_gen(cfg, 4, hd, device)
                x = torch.randn((cfg.N, cfg.d), generator=g, device=device, dtype=torch.float32)
            buf[:, i, :] = x.to(odt)
            del x
        out[name] = buf
    out["a"] = audio_map(cfg, device)
    out["scale"] = float(torch.tensor(1.0 / math.sqrt(cfg.d), dtype=torch.float32))
    return out

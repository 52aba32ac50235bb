"""Plain float64 CPU oracle for Prism-style dynamic sparse video self-attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The product (the HIP
library and its Python binding) never imports, calls or links it, and it shares
no code, table or constant with the product: every step below is written out
again from the pages, in NumPy float64, slowly and in the pages' order.

Sources ("the pages"):
  [P4] DFSAttn article at gist.science (next row f4 only): 3D Hilbert-curve
       token reordering and sub-block scoring of large blocks.
  [P5] "In-Context Sparse Attention" article at aitrends.kr (next row f3 only):
       query-block sharpness M_i routes blocks to an exact "sharp" group or a
       "flat" group computed with block-mean keys (zeroth-order Taylor).
  [P3] "Prism: Dynamic Sparse Attention cho Huấn luyện Mô hình Tạo Video-Âm thanh
       Đồng thời Độ phân giải Gốc 2K", reading guide at xyznot.com (paper
       2610.05416).  Sections used: "Các ý tưởng cốt lõi" (core ideas) and
       "Phương pháp" (method) with its sub-steps §1 (variation indicator),
       §2 (block volume and shape) and §3 (hybrid Top-k/Top-p).  Its displays
       are unnumbered; here E1 = the directional-variance display of §1,
       E2 = the indicator display of §1, E3 = the log2-optimum display of §2,
       E4 = the selected-set display of §3.
  [P2] "Tencent, 2K 해상도 영상-음성 동시 생성 모델 학습을 2.5배 빠르게 만든
       Prism 공개", news article at ailog.hnlab.kr, section "핵심 내용"
       (three steps: zones, per-zone block shapes, hybrid selection).

Where the pages leave a step open, the reading taken is stated at the function.

Parity status per function:
  pinned by closed forms, brute force or library routines in the CPU tests:
    audio_norm_map (the norm; its normalisation is a reading), candidate_shapes, axis_profiles, video_variance, audio_terms (as read),
    indicator, volume, optimum_log2, nearest_shape, block layout, permutation,
    pool_blocks, block_logits, select_row, attention forward and backward.
    next row f4: hilbert_zone_order (adjacency of consecutive zones on 2^k
    cubes, a permutation, restriction of the enclosing cube's order);
    subblock_logits (reduces to block_logits for 64-token blocks, equals
    them when a block's runs share one mean, closed forms for two and four
    runs, Jensen bounds against brute-force pair scores).
    next row f3: block_sharpness, flat_route, taylor_attn_fwd_block,
    taylor_attn_bwd_block and routed_attention (each pinned
    to closed forms of its reading: uniform and one-hot rows, brute-force
    ranking, constant-key blocks where the expansion is exact, a zero query;
    the backward against torch autograd of the block-mean attention and
    against finite differences).
  parity unpinned (readings with no number on the pages to check against):
    the formula of the audio coupling a_bar and of the normalised directional
    audio variance v_hat (audio_terms), and the density rho (density).  Their
    code is pinned to closed forms of the reading; whether the reading is the
    paper's is unpinned.
"""
from __future__ import annotations

import math

import numpy as np

ZONE = 8                 # macro-zone edge on each axis: [P3] core ideas
VOLUMES = (64, 128, 256)  # block volumes: [P3] core ideas and method §2
TAU128 = 0.5             # [P3] method §2
TAU256 = 0.25            # [P3] method §2
EPS = 1e-6               # [P3] method §1 prints "+ eps" with no value (reading)
SHAPE_TIE = 1e-9         # window for equidistant shapes (reading: the pages give no tie rule)
NEAR = 1e-12             # width of the "near a decision boundary" flags (zones)
# Width of the selection flag, relative to the row's softmax total Z.  A
# selection decided within this distance of p*Z depends on rounding: the HIP
# path sums masses as 2^-48 fixed-point integers, which moves a cumulative
# mass by at most NB * 2^-49 < 6e-11 of Z for NB <= 32768.
CDF_NEAR = 1e-10


# ----------------------------------------------------------------------------
# step 0: the audio-to-video norm map ([P3] method §1: a at each token is the
# 2-norm of the audio-to-video cross-attention output cached from the layer
# before)

def audio_norm_map(Hhat, chunk=None):
    """a_n = ||h_n||_2 over the channels of token n's cross-attention output
    Hhat [N, C], divided by its largest value over the clip.

    Reading: the pages define the norm and state a_bar in [0, 1] but give no
    normalisation; division by the clip-wide maximum is the plainest one that
    lands in [0, 1] (a clip whose outputs are all zero maps to zeros).
    float64 throughout, rounded once to float32 (the map's type).  `chunk`
    processes that many rows at a time (same arithmetic, less memory).
    Returns (norms float64 [N], a float32 [N])."""
    X = np.asarray(Hhat)
    n = X.shape[0]
    step = n if not chunk else int(chunk)
    norms = np.empty(n, dtype=np.float64)
    for r0 in range(0, n, max(step, 1)):
        Y = np.asarray(X[r0:r0 + step], dtype=np.float64)
        norms[r0:r0 + step] = np.sqrt((Y * Y).sum(axis=1))
    top = norms.max() if n else 0.0
    a = norms / top if top > 0 else np.zeros(n, dtype=np.float64)
    return norms, a.astype(np.float32)


# ----------------------------------------------------------------------------
# step 1: macro-zones  ([P3] core ideas: zones of 8x8x8 tokens; [P2] step 1)

def zone_grid(T, H, W):
    """Zone counts per axis.  Grids whose sides are not multiples of 8 are
    rejected (reading: the pages only describe divisible grids)."""
    if T <= 0 or H <= 0 or W <= 0 or T % ZONE or H % ZONE or W % ZONE:
        raise ValueError("grid sides must be positive multiples of 8")
    return T // ZONE, H // ZONE, W // ZONE


def zone_cubes(X, T, H, W):
    """Reshape raster-order rows X [T*H*W, ...] (token n = (t*H + h)*W + w) into
    [n_zones, 8, 8, 8, ...], zones in raster order m = (zt*nH + zh)*nW + zw."""
    nT, nH, nW = zone_grid(T, H, W)
    rest = X.shape[1:]
    Y = X.reshape((nT, ZONE, nH, ZONE, nW, ZONE) + rest)
    order = (0, 2, 4, 1, 3, 5) + tuple(range(6, 6 + len(rest)))
    return Y.transpose(order).reshape((nT * nH * nW, ZONE, ZONE, ZONE) + rest)


# ----------------------------------------------------------------------------
# step 2 and 3: video variation ([P3] method §1, E1)

def axis_profiles(V, T, H, W, zt_chunk=1):
    """Mean-pooled value features along each axis.

    P[m, d, i, c] = mean of channel c over the 64 tokens of zone m whose
    coordinate along axis d (0 = T, 1 = H, 2 = W) is i.  V is [N, C] in any
    float dtype; it is upcast to float64 one slab of zone rows at a time.
    """
    nT, nH, nW = zone_grid(T, H, W)
    C = V.shape[1]
    out = np.empty((nT * nH * nW, 3, ZONE, C), dtype=np.float64)
    slab = ZONE * H * W
    per = nH * nW
    for zt0 in range(0, nT, zt_chunk):
        zt1 = min(nT, zt0 + zt_chunk)
        X = np.asarray(V[zt0 * slab:zt1 * slab], dtype=np.float64)
        cubes = zone_cubes(X, (zt1 - zt0) * ZONE, H, W)     # [z, 8, 8, 8, C]
        out[zt0 * per:zt1 * per, 0] = cubes.mean(axis=(2, 3))
        out[zt0 * per:zt1 * per, 1] = cubes.mean(axis=(1, 3))
        out[zt0 * per:zt1 * per, 2] = cubes.mean(axis=(1, 2))
    return out


def video_variance(P):
    """E1: sigma2[m, d] = (1/D) sum_c (1/Z_d) sum_i (P[m,d,i,c] - mu[m,d,c])^2 with
    mu[m,d,c] the mean of P[m,d,:,c] over i; r[m, d] = sigma2 / sum_d' sigma2.

    Reading: D is the channel count of V as given (all heads' channels: one
    shape per zone, shared by every head).  When the three variances sum to 0
    (a constant zone) each ratio is 1/3.
    """
    mu = P.mean(axis=2, keepdims=True)                      # [nZ, 3, 1, C]
    sigma2 = ((P - mu) ** 2).mean(axis=2).mean(axis=2)      # over i, then over c
    tot = sigma2.sum(axis=1, keepdims=True)
    r = np.where(tot > 0, sigma2 / np.where(tot > 0, tot, 1.0), 1.0 / 3.0)
    return sigma2, r


# ----------------------------------------------------------------------------
# audio terms ([P3] method §1: a = ||h_hat||_2 cached from the previous layer;
# a_bar in [0, 1] and v_hat are named but their formulas are not printed)

def audio_terms(a, T, H, W):
    """Reading: a_bar(m) is the mean of a over the zone's 512 tokens (a is given
    already in [0, 1]); v_hat is built like r in E1: the variance of a's
    axis slice means, normalised by its sum over the three axes (1/3 each when
    that sum is 0).  Parity with the paper unpinned (readings).
    Returns (a_bar [nZ], sigma2_a [nZ, 3], v_hat [nZ, 3])."""
    A = zone_cubes(np.asarray(a, dtype=np.float64).reshape(-1), T, H, W)  # [nZ,8,8,8]
    abar = A.mean(axis=(1, 2, 3))
    prof = np.stack([A.mean(axis=(2, 3)), A.mean(axis=(1, 3)), A.mean(axis=(1, 2))], axis=1)
    s2 = ((prof - prof.mean(axis=2, keepdims=True)) ** 2).mean(axis=2)
    tot = s2.sum(axis=1, keepdims=True)
    vhat = np.where(tot > 0, s2 / np.where(tot > 0, tot, 1.0), 1.0 / 3.0)
    return abar, s2, vhat


def indicator(r, abar, vhat, eps=EPS):
    """E2: g_d(m) = r_{v,d}(m) + a_bar(m) * v_hat_{a,d}(m) + eps."""
    return r + abar[:, None] * vhat + eps


# ----------------------------------------------------------------------------
# step 2 of [P2] / [P3] method §2: volume, optimum, shape

def density(sigma2_v, abar):
    """Reading of the "normalised spatiotemporal information density" rho(m),
    which [P3] §2 names without a formula: the zone's total video variance
    S_v = sum_d sigma2_v, normalised by its maximum over all zones (0 if that
    maximum is 0), combined with the audio coupling by max(., a_bar), so that a
    zone gets large blocks only when it changes little and its audio coupling
    is weak ([P2] step 2).  Parity with the paper unpinned (reading)."""
    S = sigma2_v.sum(axis=1)
    smax = S.max() if S.size else 0.0
    shat = S / smax if smax > 0 else np.zeros_like(S)
    return np.maximum(shat, abar), S


def volume(rho, tau128=TAU128, tau256=TAU256):
    """[P3] §2 thresholds; reading: rho < tau256 -> 256, else rho < tau128 -> 128,
    else 64 (a value equal to a threshold takes the smaller block)."""
    return np.where(rho < tau256, 256, np.where(rho < tau128, 128, 64)).astype(np.int64)


def optimum_log2(g, B):
    """E3: l*_d = -1/2 log2 g_d + 1/3 (S + 1/2 log2 g_T + 1/2 log2 g_H + 1/2 log2 g_W),
    S = log2 B.  g [..., 3], B broadcastable to g[..., 0]."""
    lg = np.log2(g)
    S = np.log2(np.asarray(B, dtype=np.float64))
    return -0.5 * lg + (S[..., None] + 0.5 * lg.sum(axis=-1, keepdims=True)) / 3.0


def candidate_shapes():
    """The 16 candidate shapes of [P3] core ideas (16 shapes, volumes
    64/128/256).  Reading: every (b_T, b_H, b_W) whose edges are powers of two
    that divide the zone edge, excluding edge 1, whose product is a volume;
    that gives 7 + 6 + 3 = 16.  Listed by volume, then lexicographically; this
    order is also the tie-break order."""
    out = []
    for B in VOLUMES:
        for bt in (2, 4, 8):
            for bh in (2, 4, 8):
                for bw in (2, 4, 8):
                    if bt * bh * bw == B:
                        out.append((bt, bh, bw))
    return out


def nearest_shape(lstar, B, delta=SHAPE_TIE):
    """[P3] §2: the candidate of C_B nearest to l* in Euclidean distance in log2
    space.  Reading: distances within delta of the minimum are ties, broken
    toward the lowest candidate index.  Returns (index into candidate_shapes(),
    flag) where flag is True when some candidate's distance lies within NEAR of
    the edge of the tie window."""
    cands = candidate_shapes()
    best = None
    dists = []
    for idx, s in enumerate(cands):
        if s[0] * s[1] * s[2] != B:
            continue
        D = sum((math.log2(s[d]) - float(lstar[d])) ** 2 for d in range(3))
        dists.append((idx, D))
    Dmin = min(D for _, D in dists)
    for idx, D in dists:
        if D <= Dmin + delta:
            best = idx
            break
    flag = any(abs(D - (Dmin + delta)) < NEAR for _, D in dists)
    return best, flag


def decide(sigma2_v, r, abar, vhat, tau128=TAU128, tau256=TAU256, eps=EPS, delta=SHAPE_TIE):
    """Indicator -> density -> volume -> optimum -> shape, per zone."""
    g = indicator(r, abar, vhat, eps)
    rho, S = density(sigma2_v, abar)
    B = volume(rho, tau128, tau256)
    lstar = optimum_log2(g, B)
    shapes = np.empty(len(B), dtype=np.int64)
    flags = np.zeros(len(B), dtype=bool)
    for m in range(len(B)):
        shapes[m], flags[m] = nearest_shape(lstar[m], int(B[m]), delta)
        if abs(rho[m] - tau128) < NEAR or abs(rho[m] - tau256) < NEAR:
            flags[m] = True
    return dict(g=g, rho=rho, S_v=S, B=B, lstar=lstar, shape=shapes, near_tie=flags)


def zone_shapes(V, a, T, H, W, tau128=TAU128, tau256=TAU256, eps=EPS):
    """Stages a1-a3 end to end: V [N, C] and a [N] in raster order."""
    P = axis_profiles(V, T, H, W)
    sigma2_v, r = video_variance(P)
    abar, sigma2_a, vhat = audio_terms(a, T, H, W)
    dec = decide(sigma2_v, r, abar, vhat, tau128, tau256, eps)
    dec.update(sigma2_v=sigma2_v, r=r, abar=abar, sigma2_a=sigma2_a, vhat=vhat)
    dec["block_offsets"], dec["NB"] = block_layout(dec["shape"])
    return dec


# ----------------------------------------------------------------------------
# block-major order.  The pages reorganise tokens into zone-shaped blocks
# ([P3] core ideas, [P2] steps 1-2) and pool and attend blocks as units
# ([P3] §3) but give no order.  Reading: zones in raster order, 512 positions
# each; inside a zone its blocks in raster order over the block grid; inside a
# block its tokens in raster (t, h, w) order.

def block_layout(shape_idx, zone_order=None):
    """block_offsets[NB+1] (token offsets of each block in block-major order) and NB.
    zone_order[pos] = the raster zone at position pos (None: raster order)."""
    cands = candidate_shapes()
    order = range(len(shape_idx)) if zone_order is None else zone_order
    offs = [0]
    for pos, m in enumerate(order):
        bt, bh, bw = cands[int(shape_idx[int(m)])]
        vol = bt * bh * bw
        for j in range(ZONE ** 3 // vol):
            offs.append(ZONE ** 3 * pos + (j + 1) * vol)
    return np.asarray(offs, dtype=np.int64), len(offs) - 1


def hilbert_zone_order(T, H, W):
    """Next row f4 (DFSAttn article, Hilbert-curve reordering, applied to zones):
    the zones sorted by their index along a 3D Hilbert curve.  Reading: the
    curve of J. Skilling's transform ("Programming the Hilbert curve", 2004)
    over the smallest 2^k cube holding the zone grid, axes (t, h, w) with t the
    most significant, zones outside the grid skipped.  Returns order[pos] =
    raster zone index."""
    nT, nH, nW = zone_grid(T, H, W)
    bits = max(1, int(math.ceil(math.log2(max(nT, nH, nW)))))

    def index(x):
        x = list(x)
        top = 1 << (bits - 1)
        q = top
        while q > 1:                       # undo the excess work (inverse rotations)
            low = q - 1
            for i in range(3):
                if x[i] & q:
                    x[0] ^= low
                else:
                    swap = (x[0] ^ x[i]) & low
                    x[0] ^= swap
                    x[i] ^= swap
            q >>= 1
        for i in (1, 2):                   # Gray encode
            x[i] ^= x[i - 1]
        flip, q = 0, top
        while q > 1:
            if x[2] & q:
                flip ^= q - 1
            q >>= 1
        x = [v ^ flip for v in x]
        h = 0
        for bit in range(bits - 1, -1, -1):   # interleave: t, h, w per level
            for i in range(3):
                h = (h << 1) | ((x[i] >> bit) & 1)
        return h

    zones = [(zt, zh, zw) for zt in range(nT) for zh in range(nH) for zw in range(nW)]
    keys = [index(z) for z in zones]
    return np.asarray(sorted(range(len(zones)), key=lambda m: keys[m]), dtype=np.int64)


def _zone_local_order(shape):
    """(it, ih, iw) of the 512 zone positions in block-major order for one shape."""
    bt, bh, bw = shape
    it, ih, iw = [], [], []
    for jt in range(ZONE // bt):
        for jh in range(ZONE // bh):
            for jw in range(ZONE // bw):
                for rt in range(bt):
                    for rh in range(bh):
                        for rw in range(bw):
                            it.append(jt * bt + rt)
                            ih.append(jh * bh + rh)
                            iw.append(jw * bw + rw)
    return np.array(it), np.array(ih), np.array(iw)


def permutation(T, H, W, shape_idx, zone_order=None):
    """pi[p] = raster index of the token at block-major position p; zone_order
    as in block_layout (None: raster order)."""
    nT, nH, nW = zone_grid(T, H, W)
    cands = candidate_shapes()
    local = [_zone_local_order(s) for s in cands]
    pi = np.empty(T * H * W, dtype=np.int64)
    order = range(len(shape_idx)) if zone_order is None else zone_order
    for pos, m in enumerate(order):
        m = int(m)
        c = shape_idx[m]
        zt, rem = divmod(m, nH * nW)
        zh, zw = divmod(rem, nW)
        it, ih, iw = local[int(c)]
        t = ZONE * zt + it
        h = ZONE * zh + ih
        w = ZONE * zw + iw
        pi[ZONE ** 3 * pos:ZONE ** 3 * (pos + 1)] = (t * H + h) * W + w
    return pi


def to_block_major(X, pi):
    """Gather: Y[p] = X[pi[p]]."""
    return X[pi]


def to_raster(Y, pi):
    """Scatter (inverse): X[pi[p]] = Y[p]."""
    X = np.empty_like(Y)
    X[pi] = Y
    return X


# ----------------------------------------------------------------------------
# [P3] §3: pooled block scores and hybrid Top-k / Top-p selection

def pool_blocks(Xp, offs, head):
    """Mean over each block's tokens of one head: Xp [N, heads, d] block-major,
    returns [NB, d] float64.  Reading: the page pools keys into K_bar_j and
    scores them with query blocks; queries are mean-pooled the same way."""
    X = np.asarray(Xp[:, head, :], dtype=np.float64)
    NB = len(offs) - 1
    out = np.empty((NB, X.shape[1]), dtype=np.float64)
    for i in range(NB):
        out[i] = X[offs[i]:offs[i + 1]].mean(axis=0)
    return out


def block_logits(Qbar, Kbar, scale):
    """Pooled scores L[i, j] = scale * Q_bar_i . K_bar_j, evaluated in float64 and
    rounded once to float32 (the precision in which the selection is decided).
    Reading: scale = 1/sqrt(d) as passed (a float32 value); plain scores, no
    block-size weighting."""
    L = float(np.float32(scale)) * (Qbar @ Kbar.T)
    return L.astype(np.float32)



SUB = 64   # sub-block length for the sub-block scoring variant (the smallest block volume)


def subblock_logits(Qp, Kp, offs, head, scale, rows=None):
    """Next row f4, scoring variant (DFSAttn article, sub-block scoring: a
    large block is scored through the finer scores of its parts, and those are
    added up).  Reading: each block is cut into its consecutive SUB-token runs
    in block-major order; every run is mean-pooled; the score of block pair
    (i, j) is the log of the mean, over all run pairs (a in i, b in j), of
    exp(scale * Q_bar_a . K_bar_b).  The addition is taken in probability
    space and divided by the number of pairs, so a pair of 64-token blocks
    keeps its plain pooled score and blocks of every size stay on one scale.
    Float64, with each pair group's maximum factored out, rounded once to
    float32.  rows: the query blocks to score (default all).  Returns
    [len(rows), NB] float32."""
    offs = np.asarray(offs, dtype=np.int64)
    NB = len(offs) - 1
    runs = np.arange(0, offs[-1] + 1, SUB)
    Qs = pool_blocks(Qp, runs, head)
    Ks = pool_blocks(Kp, runs, head)
    sc = float(np.float32(scale))
    first = offs[:-1] // SUB                      # first run of each block
    rows = range(NB) if rows is None else rows
    out = np.empty((len(rows), NB), dtype=np.float32)
    for r, i in enumerate(rows):
        S = sc * (Qs[offs[i] // SUB:offs[i + 1] // SUB] @ Ks.T)        # [runs of i, all key runs]
        m = np.maximum.reduceat(S.max(axis=0), first)                   # per key block
        mean_e = np.add.reduceat(np.exp(S - np.repeat(m, np.diff(offs) // SUB)[None, :]).sum(axis=0), first)
        mean_e /= S.shape[0] * (np.diff(offs) // SUB)
        out[r] = (m + np.log(mean_e)).astype(np.float32)
    return out


def select_row(L, k, p):
    """E4: S_i = Top-k(P_i, k) U Top-p(P_i, p) with P_i = softmax of the row.

    Readings: blocks are ranked by score, ties toward the lower index; Top-p
    is the shortest prefix of that ranking whose probability mass reaches p
    (the crossing block included), taken on a float64 CDF; since both sets are
    prefixes of one ranking, the union is the first max(k, n_p) blocks (at most
    NB).  Returns (sorted selected indices, flag) where flag marks a row whose
    cumulative mass passes within CDF_NEAR*Z of p*Z at some prefix.
    """
    L = np.asarray(L, dtype=np.float64)
    NB = L.shape[0]
    order = np.lexsort((np.arange(NB), -L))
    e = np.exp(L - L.max())
    Z = e.sum()
    cum = np.cumsum(e[order])
    target = p * Z
    hit = np.nonzero(cum >= target)[0]
    n_p = int(hit[0]) + 1 if hit.size else NB
    n = min(NB, max(int(k), n_p))
    flag = bool(np.any(np.abs(cum - target) < CDF_NEAR * Z))
    return np.sort(order[:n]), flag


def select(logits, k, p):
    """All rows of one head -> (offsets [NB+1], indices, flags [NB])."""
    NB = logits.shape[0]
    offs = [0]
    idx = []
    flags = np.zeros(NB, dtype=bool)
    for i in range(NB):
        s, flags[i] = select_row(logits[i], k, p)
        idx.append(s)
        offs.append(offs[-1] + len(s))
    return np.asarray(offs, dtype=np.int64), (np.concatenate(idx) if idx else np.zeros(0, np.int64)), flags


# ----------------------------------------------------------------------------
# [P3] §3: exact attention over the selected key blocks only.  Reading:
# non-causal, no dropout, no bias; the result is dense softmax attention with
# every key outside the selected blocks masked out.

def _keys_of(sel, offs):
    return np.concatenate([np.arange(offs[j], offs[j + 1]) for j in sel])


def attn_fwd_block(Qp, Kp, Vp, offs, sel, i, head, scale):
    """Output rows and log-sum-exp (natural log) of query block i."""
    q = np.asarray(Qp[offs[i]:offs[i + 1], head, :], dtype=np.float64)
    keys = _keys_of(sel, offs)
    k = np.asarray(Kp[keys, head, :], dtype=np.float64)
    v = np.asarray(Vp[keys, head, :], dtype=np.float64)
    s = float(np.float32(scale)) * (q @ k.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    return (e @ v) / l, (m + np.log(l))[:, 0]


def attn_bwd_block(Qp, Kp, Vp, dOp, offs, sel, i, head, scale, with_terms=False):
    """Gradient contributions of query block i, by the chain rule of the
    masked softmax: P = softmax(s), dP = dO V^T, dS = P * (dP - rowsum(P*dP)),
    dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO.  The selection itself is a
    constant (no gradient flows through the discrete choice).  Returns
    (dQ rows of block i, key indices, dK rows, dV rows for those keys).

    with_terms: also return, for every element of dQ, dK and dV, the sum of
    the squares of the products it sums (sum_t (scale dS_qt k_tc)^2 for dQ,
    sum_q (scale dS_qt q_qc)^2 for dK, sum_q (P_qt dO_qc)^2 for dV): the scale
    of the error that rounding one factor of every product (dS or P) to a
    short format leaves in the sum.  Test infrastructure for the parity bars;
    the gradient itself does not use it."""
    sc = float(np.float32(scale))
    q = np.asarray(Qp[offs[i]:offs[i + 1], head, :], dtype=np.float64)
    do = np.asarray(dOp[offs[i]:offs[i + 1], head, :], dtype=np.float64)
    keys = _keys_of(sel, offs)
    k = np.asarray(Kp[keys, head, :], dtype=np.float64)
    v = np.asarray(Vp[keys, head, :], dtype=np.float64)
    s = sc * (q @ k.T)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    P = e / e.sum(axis=1, keepdims=True)
    dP = do @ v.T
    dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
    out = (sc * (dS @ k), keys, sc * (dS.T @ q), P.T @ do)
    if not with_terms:
        return out
    dS2, P2 = dS * dS, P * P
    return out + (sc * sc * (dS2 @ (k * k)), sc * sc * (dS2.T @ (q * q)), P2.T @ (do * do))


def attention(Qp, Kp, Vp, offs, csr_offs, csr_idx, head, scale, dOp=None):
    """Forward (and backward if dOp is given) of one head over every block.
    With dOp, also the summed squared products of every gradient element
    (attn_bwd_block's with_terms) as tQ, tK, tV."""
    N, _, d = Qp.shape
    NB = len(offs) - 1
    O = np.zeros((N, d))
    lse = np.zeros(N)
    dQ = dK = dV = tQ = tK = tV = None
    if dOp is not None:
        dQ, dK, dV = np.zeros((N, d)), np.zeros((N, d)), np.zeros((N, d))
        tQ, tK, tV = np.zeros((N, d)), np.zeros((N, d)), np.zeros((N, d))
    for i in range(NB):
        sel = csr_idx[csr_offs[i]:csr_offs[i + 1]]
        o, l = attn_fwd_block(Qp, Kp, Vp, offs, sel, i, head, scale)
        O[offs[i]:offs[i + 1]] = o
        lse[offs[i]:offs[i + 1]] = l
        if dOp is not None:
            dq, keys, dk, dv, tq, tk, tv = attn_bwd_block(Qp, Kp, Vp, dOp, offs, sel, i, head, scale, with_terms=True)
            dQ[offs[i]:offs[i + 1]] = dq
            dK[keys] += dk
            dV[keys] += dv
            tQ[offs[i]:offs[i + 1]] = tq
            tK[keys] += tk
            tV[keys] += tv
    return dict(O=O, lse=lse, dQ=dQ, dK=dK, dV=dV, tQ=tQ, tK=tK, tV=tV)


def key_block_grads(Qp, Kp, Vp, dOp, offs, csr_offs, csr_idx, j, head, scale, rows=None, with_terms=False):
    """dK and dV rows of key block j alone: the sum over every query block
    whose selected set holds j (used to check sampled key blocks).  `rows`
    optionally limits the scan to candidate query blocks (each is still
    checked for membership).  with_terms: also the summed squared products of
    every element (as attn_bwd_block)."""
    d = Qp.shape[2]
    B = offs[j + 1] - offs[j]
    dK, dV, tK, tV = np.zeros((B, d)), np.zeros((B, d)), np.zeros((B, d)), np.zeros((B, d))
    NB = len(offs) - 1
    for i in (range(NB) if rows is None else sorted(int(r) for r in rows)):
        sel = csr_idx[csr_offs[i]:csr_offs[i + 1]]
        if j not in set(int(x) for x in sel):
            continue
        _, keys, dk, dv, _, tk, tv = attn_bwd_block(Qp, Kp, Vp, dOp, offs, sel, i, head, scale, with_terms=True)
        pos = np.nonzero((keys >= offs[j]) & (keys < offs[j + 1]))[0]
        dK += dk[pos]
        dV += dv[pos]
        tK += tk[pos]
        tV += tv[pos]
    return (dK, dV, tK, tV) if with_terms else (dK, dV)


# ----------------------------------------------------------------------------
# next row f3: sharpness routing and the zeroth-order Taylor path for flat
# query blocks ("In-Context Sparse Attention" article, sections on grouped
# computation and the zeroth-order Taylor kernel)

def block_sharpness(L):
    """M_i, the variance of query block i's softmax distribution.  Reading: the
    distribution is the softmax of the row's pooled scores L[i, :] over all
    key blocks (the scores that the selection ranks); the variance is the
    population variance of its NB probabilities.  float64."""
    X = np.asarray(L, dtype=np.float64)
    NB = X.shape[1]
    P = np.exp(X - X.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    return ((P - 1.0 / NB) ** 2).mean(axis=1)


def flat_route(M, flat_ratio):
    """Flat flags: the floor(flat_ratio * NB) query blocks of lowest sharpness,
    ties toward the lower index; the rest are sharp.  Reading: the article
    names a flat-ratio parameter and a threshold on M_i without values; a
    ratio fixes the threshold per head."""
    M = np.asarray(M, dtype=np.float64)
    NB = M.shape[0]
    n_flat = int(math.floor(float(flat_ratio) * NB))
    order = sorted(range(NB), key=lambda i: (M[i], i))
    flat = np.zeros(NB, dtype=bool)
    flat[order[:n_flat]] = True
    return flat


def taylor_attn_fwd_block(Qp, Kp, Vp, offs, sel, i, head, scale):
    """Flat path for query block i: every selected key block j enters as its
    mean key K_bar_j and mean value V_bar_j, counted B_j times, which is the
    zeroth-order expansion of exp(q.k) around k = K_bar_j:
        O_q = sum_j B_j exp(s q.K_bar_j) V_bar_j / sum_j B_j exp(s q.K_bar_j).
    Reading: the article applies the block-mean kernel to the flat group's
    key blocks; here those are the block's selected set S_i.  Returns the
    output rows and the natural-log log-sum-exp of the weights."""
    q = np.asarray(Qp[offs[i]:offs[i + 1], head, :], dtype=np.float64)
    sel = [int(j) for j in sel]
    kb = np.stack([np.asarray(Kp[offs[j]:offs[j + 1], head, :], dtype=np.float64).mean(axis=0) for j in sel])
    vb = np.stack([np.asarray(Vp[offs[j]:offs[j + 1], head, :], dtype=np.float64).mean(axis=0) for j in sel])
    cnt = np.array([float(offs[j + 1] - offs[j]) for j in sel])
    s = float(np.float32(scale)) * (q @ kb.T) + np.log(cnt)[None, :]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    return (e @ vb) / l, (m + np.log(l))[:, 0]


def taylor_attn_bwd_block(Qp, Kp, Vp, dOp, offs, sel, i, head, scale):
    """Gradient of taylor_attn_fwd_block for query block i, the selection and
    the routing held constant (reading: the article gives no backward; this is
    the chain rule through the block means).  With w_j the weights of the
    forward, D = rowsum(dO * O), dS_j = w_j (dO . V_bar_j - D):
        dq = s sum_j dS_j K_bar_j,
        dK_bar_j = s sum_q dS_qj q,   dV_bar_j = sum_q w_qj dO_q,
    and every token of key block j receives dK_bar_j / B_j and dV_bar_j / B_j.
    Returns (dq [B_i, d], {j: (dK_bar_j, dV_bar_j)})."""
    s_ = float(np.float32(scale))
    q = np.asarray(Qp[offs[i]:offs[i + 1], head, :], dtype=np.float64)
    do = np.asarray(dOp[offs[i]:offs[i + 1], head, :], dtype=np.float64)
    sel = [int(j) for j in sel]
    kb = np.stack([np.asarray(Kp[offs[j]:offs[j + 1], head, :], dtype=np.float64).mean(axis=0) for j in sel])
    vb = np.stack([np.asarray(Vp[offs[j]:offs[j + 1], head, :], dtype=np.float64).mean(axis=0) for j in sel])
    cnt = np.array([float(offs[j + 1] - offs[j]) for j in sel])
    sc = s_ * (q @ kb.T) + np.log(cnt)[None, :]
    w = np.exp(sc - sc.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    o = w @ vb
    D = (do * o).sum(axis=1, keepdims=True)
    dS = w * (do @ vb.T - D)
    dq = s_ * (dS @ kb)
    dkb = s_ * (dS.T @ q)
    dvb = w.T @ do
    return dq, {j: (dkb[n], dvb[n]) for n, j in enumerate(sel)}


def routed_attention(Qp, Kp, Vp, offs, csr_offs, csr_idx, flat, head, scale, dOp=None):
    """Routed forward (and backward): exact attention for sharp query blocks,
    the block-mean path for flat ones; dK and dV sum the exact contributions
    of sharp blocks and the block-mean contributions (dK_bar_j / B_j per token)
    of flat ones."""
    N, _, d = Qp.shape
    NB = len(offs) - 1
    O = np.zeros((N, d))
    lse = np.zeros(N)
    dQ, dK, dV = (np.zeros((N, d)) for _ in range(3)) if dOp is not None else (None, None, None)
    for i in range(NB):
        sel = csr_idx[csr_offs[i]:csr_offs[i + 1]]
        fwd = taylor_attn_fwd_block if flat[i] else attn_fwd_block
        o, l = fwd(Qp, Kp, Vp, offs, sel, i, head, scale)
        O[offs[i]:offs[i + 1]] = o
        lse[offs[i]:offs[i + 1]] = l
        if dOp is None:
            continue
        if flat[i]:
            dq, g = taylor_attn_bwd_block(Qp, Kp, Vp, dOp, offs, sel, i, head, scale)
            dQ[offs[i]:offs[i + 1]] = dq
            for j, (dkb, dvb) in g.items():
                B = offs[j + 1] - offs[j]
                dK[offs[j]:offs[j + 1]] += dkb / B
                dV[offs[j]:offs[j + 1]] += dvb / B
        else:
            dq, keys, dk, dv = attn_bwd_block(Qp, Kp, Vp, dOp, offs, sel, i, head, scale)
            dQ[offs[i]:offs[i + 1]] = dq
            dK[keys] += dk
            dV[keys] += dv
    return dict(O=O, lse=lse, dQ=dQ, dK=dK, dV=dV)

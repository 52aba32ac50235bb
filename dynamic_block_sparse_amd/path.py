"""The Prism hot path end to end on device tensors.

This module only allocates device memory with torch and calls the C ABI in
order (zone shapes -> block-major permutation -> selection -> attention
forward/backward -> inverse permutation); every step runs in libprism's HIP
kernels.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

from . import prism as P


@dataclass
class Selection:
    offsets: torch.Tensor     # int32 [hc, nb+1] per head chunk
    idx: torch.Tensor         # int32 [hc, cap]
    total: torch.Tensor       # int64 [hc]
    cap: int
    logits: torch.Tensor | None


def sparsity_schedule(step, steps, first, last):
    """(top_k, top_p) for diffusion step `step` of `steps` (0-based).

    Next row after the exact path (DFSAttn article, adaptive sparsity: early,
    noisy steps look at almost every block; sparsity grows as the sample
    sharpens).  The article gives no schedule; this reading moves linearly in
    the step index from `first` = (k0, p0), the permissive end, to `last` =
    (k1, p1), the workload's own values, with k rounded to the nearest integer.
    """
    if steps <= 0 or not 0 <= step < steps:
        raise ValueError("need 0 <= step < steps")
    f = step / (steps - 1) if steps > 1 else 1.0
    (k0, p0), (k1, p1) = first, last
    return int(math.floor(k0 + (k1 - k0) * f + 0.5)), p0 + (p1 - p0) * f


def reuses_selection(step, refresh_every):
    """True when step `step` reuses the previous step's selection (a fresh
    selection every `refresh_every` steps, the first step always fresh)."""
    if refresh_every < 1:
        raise ValueError("refresh_every must be at least 1")
    return step % refresh_every != 0


class PrismPath:
    """One attention layer's hot path for a fixed grid and head layout.

    q, k, v, do are raster-order [N, heads, d] tensors (bf16 or fp32) with
    d contiguous.  Heads are processed in chunks of `head_chunk` (all at once
    by default; 1 processes heads one at a time).
    """

    def __init__(self, T, H, W, heads, d, top_k, top_p, scale, head_chunk=None, prm=None, device="cuda",
                 zone_order="raster", scoring="block"):
        """zone_order: "raster" (zones in raster order) or "hilbert" (zones along
        the 3D Hilbert curve, prism_hilbert_zone_order).  scoring: "block"
        (pooled block scores) or "subblock" (64-token runs scored in pairs,
        prism_select_subblock)."""
        if scoring not in ("block", "subblock"):
            raise ValueError("scoring must be 'block' or 'subblock'")
        self.scoring = scoring
        self.T, self.H, self.W = T, H, W
        self.N = T * H * W
        self.nZ = self.N // 512
        self.heads, self.d = heads, d
        self.top_k, self.top_p, self.scale = top_k, top_p, scale
        self.hc = head_chunk or heads
        if heads % self.hc:
            raise ValueError("head_chunk must divide heads")
        self.prm = prm
        self.device = torch.device(device)
        self.zone_shape = torch.empty(self.nZ, dtype=torch.uint8, device=self.device)
        self.block_offsets = torch.empty(8 * self.nZ + 1, dtype=torch.int32, device=self.device)
        self.nb_dev = torch.empty(1, dtype=torch.int32, device=self.device)
        self.zone_stats = torch.empty(self.nZ * P.ZS_STRIDE, dtype=torch.float64, device=self.device)
        self.nb = None
        self._cap_seen = 0   # largest per-head selection count seen (CSR sizing)
        self._reuse = None   # selections of the last fresh step, for step(..., reuse=True)
        if zone_order not in ("raster", "hilbert"):
            raise ValueError("zone_order must be 'raster' or 'hilbert'")
        self.zone_order = None
        if zone_order == "hilbert":
            self.zone_order = torch.tensor(P.prism_hilbert_zone_order(T, H, W), dtype=torch.int32,
                                           device=self.device)

    # -------------------------------------------------------------- stages
    def shapes(self, v, a):
        """v: raster [N, heads', d] or [N, C]; all of its channels enter the
        zone statistics (one shape per zone, shared by every head)."""
        C = v.shape[1] * v.shape[2] if v.dim() == 3 else v.shape[1]
        ws = torch.empty(P.prism_workspace_size(P.OP_ZONE_SHAPES, self.N, 1, C, 0, 0), dtype=torch.uint8,
                         device=self.device)
        self.nb = P.prism_zone_shapes(self.T, self.H, self.W, v, C, v.stride(0), a, self.zone_shape,
                                      self.block_offsets, self.nb_dev, ws, prm=self.prm, zone_stats=self.zone_stats,
                                      zone_order=self.zone_order)
        self._cap_seen = 0
        return self.nb

    def block_major_like(self, x):
        """An [N, heads, d] view over head-major storage ([heads, N, d]): each
        head's block-major rows are contiguous, so a 64-row tile of one head is
        one 16 KB (bf16, d=128) run."""
        N, nh, d = x.shape
        return torch.empty((nh, N, d), dtype=x.dtype, device=x.device).permute(1, 0, 2)

    def permute(self, x, inverse=False, out=None):
        """Gather raster rows into block-major order (head-major storage), or
        scatter block-major rows back into a raster [N, heads, d] tensor; one
        library call for all heads."""
        N, nh, d = x.shape
        if out is None:
            out = torch.empty((N, nh, d), dtype=x.dtype, device=x.device) if inverse else self.block_major_like(x)
        P.prism_block_permute_heads(self.T, self.H, self.W, self.zone_shape, x, out, nh, d, x.stride(0), x.stride(1),
                                    out.stride(0), out.stride(1), 1 if inverse else 0, zone_order=self.zone_order)
        return out

    def permute_per_head(self, x, inverse=False, out=None):
        """The same with one prism_block_permute call per head."""
        N, nh, d = x.shape
        if out is None:
            out = torch.empty((N, nh, d), dtype=x.dtype, device=x.device) if inverse else self.block_major_like(x)
        for h in range(nh):
            P.prism_block_permute(self.T, self.H, self.W, self.zone_shape, x[:, h], out[:, h], d, x.stride(0),
                                  out.stride(0), 1 if inverse else 0, zone_order=self.zone_order)
        return out

    def _cap_guess(self):
        """First CSR capacity per head to try: the largest count seen so far on
        this path, else 4 k entries per row (at most nb * nb)."""
        if self._cap_seen:
            return self._cap_seen
        return min(self.nb * self.nb, 4 * max(self.top_k, 1) * self.nb)

    def select(self, qp, kp, h0=0, want_logits=False, scoring=None, cap=None):
        """scoring: "block" (pooled block scores, prism_select) or "subblock"
        (prism_select_subblock); default the path's own.  cap: CSR capacity per
        head.  Default: sized from the counts, i.e. a first guess, and one more
        call with the largest per-head count when the guess was short (nb * nb
        never truncates)."""
        scoring = scoring or self.scoring
        nb, hc = self.nb, self.hc
        fixed = cap is not None
        cap = int(cap) if fixed else self._cap_guess()
        offsets = torch.empty((hc, nb + 1), dtype=torch.int32, device=self.device)
        total = torch.empty(hc, dtype=torch.int64, device=self.device)
        logits = torch.empty((hc, nb, nb), dtype=torch.float32, device=self.device) if want_logits else None
        op, fn = (P.OP_SELECT, P.prism_select) if scoring == "block" else (P.OP_SELECT_SUB, P.prism_select_subblock)
        ws = torch.empty(P.prism_workspace_size(op, self.N, hc, self.d, nb, 0), dtype=torch.uint8,
                         device=self.device)
        q, k = qp[:, h0:h0 + hc], kp[:, h0:h0 + hc]
        while True:
            idx = torch.empty((hc, cap), dtype=torch.int32, device=self.device)
            fn(q, k, self.N, hc, self.d, q.stride(0), q.stride(1), self.block_offsets, nb, self.top_k, self.top_p,
               self.scale, offsets, idx, cap, total, ws, logits=logits)
            if fixed:
                break
            need = int(total.max().item())
            self._cap_seen = max(self._cap_seen, need)
            if need <= cap:
                break
            cap = need
        return Selection(offsets, idx, total, cap, logits)

    def raster_layout(self, x):
        """prism_raster_layout for a raster [N, heads', d] tensor x: attention
        rows are written straight to raster order (the inverse permutation
        applied in the kernels' epilogues)."""
        zo = self.zone_order.data_ptr() if self.zone_order is not None else None
        return P.PrismRasterLayout(self.T, self.H, self.W, self.zone_shape.data_ptr(), zo, x.stride(0), x.stride(1))

    def residual_like(self, op):
        """A buffer for the bf16 residual of O, laid out like op (None for fp32)."""
        if op.dtype != torch.bfloat16:
            return None
        return torch.empty_strided(op.shape, op.stride(), dtype=op.dtype, device=op.device)

    def forward(self, qp, kp, vp, sel, op=None, lse=None, h0=0, raster=False, ores=None):
        """raster: op is (or is allocated as) a raster [N, heads, d] tensor and
        the kernels write O there directly.  ores: None, or a tensor laid out
        like op that receives the bf16 residual of O (pass it to backward)."""
        hc = self.hc
        if op is None:
            op = torch.empty_like(qp, memory_format=torch.contiguous_format) if raster else self.block_major_like(qp)
        if lse is None:
            lse = torch.empty((hc, self.N), dtype=torch.float32, device=self.device)
        ws = torch.empty(P.prism_workspace_size(P.OP_ATTN_FWD, self.N, hc, self.d, self.nb, sel.cap),
                         dtype=torch.uint8, device=self.device)
        q, k, v, o = (x[:, h0:h0 + hc] for x in (qp, kp, vp, op))
        P.prism_sparse_attn_fwd(q, k, v, o, lse, self.N, hc, self.d, q.stride(0), q.stride(1), self.block_offsets,
                                self.nb, sel.offsets, sel.idx, sel.cap, self.scale, ws=ws,
                                layout=self.raster_layout(op) if raster else None,
                                o_res=ores[:, h0:h0 + hc] if ores is not None else None)
        return op, lse

    def route(self, sel, flat_ratio, want_sharpness=False):
        """Flat flags [hc, nb] (uint8) of a selection made with want_logits=True,
        and the float64 sharpness when asked for."""
        hc, nb = self.hc, self.nb
        flat = torch.empty((hc, nb), dtype=torch.uint8, device=self.device)
        M = torch.empty((hc, nb), dtype=torch.float64, device=self.device)
        P.prism_flat_route(sel.logits, hc, nb, flat_ratio, flat, sharpness=M)
        return (flat, M) if want_sharpness else flat

    def routed_forward(self, qp, kp, vp, sel, flat, op=None, lse=None, h0=0, ores=None):
        hc = self.hc
        if op is None:
            op = self.block_major_like(qp)
        if lse is None:
            lse = torch.empty((hc, self.N), dtype=torch.float32, device=self.device)
        ws = torch.empty(P.prism_workspace_size(P.OP_ROUTED_FWD, self.N, hc, self.d, self.nb, sel.cap),
                         dtype=torch.uint8, device=self.device)
        q, k, v, o = (x[:, h0:h0 + hc] for x in (qp, kp, vp, op))
        P.prism_routed_attn_fwd(q, k, v, o, lse, self.N, hc, self.d, q.stride(0), q.stride(1), self.block_offsets,
                                self.nb, sel.offsets, sel.idx, sel.cap, flat, self.scale, ws,
                                o_res=ores[:, h0:h0 + hc] if ores is not None else None)
        return op, lse

    def routed_backward(self, qp, kp, vp, op, dop, lse, sel, flat, grads=None, h0=0, ores=None):
        hc = self.hc
        if grads is None:
            grads = tuple(self.block_major_like(qp) for _ in range(3))
        dq, dk, dv = grads
        ws = torch.empty(P.prism_workspace_size(P.OP_ROUTED_BWD, self.N, hc, self.d, self.nb, sel.cap),
                         dtype=torch.uint8, device=self.device)
        q, k, v, o, do, gq, gk, gv = (x[:, h0:h0 + hc] for x in (qp, kp, vp, op, dop, dq, dk, dv))
        P.prism_routed_attn_bwd(q, k, v, o, do, lse, gq, gk, gv, self.N, hc, self.d, q.stride(0), q.stride(1),
                                self.block_offsets, self.nb, sel.offsets, sel.idx, sel.cap, flat, self.scale, ws,
                                o_res=ores[:, h0:h0 + hc] if ores is not None else None)
        return dq, dk, dv

    def backward(self, qp, kp, vp, op, dop, lse, sel, grads=None, h0=0, raster=False, ores=None):
        """raster: op and the gradients are raster [N, heads, d] tensors with
        one set of strides (the kernels read O and write dQ, dK, dV there).
        ores: the residual of O written by forward (None: rowsum(dO * O) from
        the rounded O alone)."""
        hc = self.hc
        if grads is None:
            grads = tuple((torch.empty_like(qp, memory_format=torch.contiguous_format) if raster
                           else self.block_major_like(qp)) for _ in range(3))
        dq, dk, dv = grads
        if raster and any(t.stride() != op.stride() for t in grads):
            raise ValueError("raster O and gradients must share their strides")
        ws = torch.empty(P.prism_workspace_size(P.OP_ATTN_BWD, self.N, hc, self.d, self.nb, sel.cap),
                         dtype=torch.uint8, device=self.device)
        q, k, v, o, do, gq, gk, gv = (x[:, h0:h0 + hc] for x in (qp, kp, vp, op, dop, dq, dk, dv))
        P.prism_sparse_attn_bwd(q, k, v, o, do, lse, gq, gk, gv, self.N, hc, self.d, q.stride(0), q.stride(1),
                                self.block_offsets, self.nb, sel.offsets, sel.idx, sel.cap, self.scale, ws,
                                layout=self.raster_layout(op) if raster else None,
                                o_res=ores[:, h0:h0 + hc] if ores is not None else None)
        return dq, dk, dv

    def release_selection(self):
        """Drop the selections kept for step(..., reuse=True)."""
        self._reuse = None

    # -------------------------------------------------------------- whole step
    def step(self, q, k, v, a, do=None, reuse=False):
        """Shapes, permutation, selection, forward (and backward when `do` is
        given), with the outputs written straight to raster order.  Returns
        raster-order results.

        reuse: keep the zone shapes, block layout and selected sets of the
        last step run without reuse (selection reuse across diffusion steps,
        DFSAttn article, cached masks): zone statistics, shapes and selection
        are skipped, and the new tensors are permuted with the cached layout
        and attend over the cached sets.  The sets refer to blocks of that
        layout, so the layout is reused with them.  A step run without reuse
        keeps a reference to its selections for that purpose (their CSR
        buffers stay allocated); release_selection() drops it."""
        if reuse and self._reuse is None:
            raise ValueError("no selection to reuse: run a step without reuse first")
        if not reuse:
            self.shapes(v, a)
        qp, kp, vp = self.permute(q), self.permute(k), self.permute(v)
        dop = self.permute(do) if do is not None else None
        op = torch.empty_like(q)
        ores = self.residual_like(op) if do is not None else None
        grads = tuple(torch.empty_like(q) for _ in range(3)) if do is not None else None
        lses, sels = [], []
        for g, h0 in enumerate(range(0, self.heads, self.hc)):
            sel = self._reuse[g] if reuse else self.select(qp, kp, h0)
            _, lse = self.forward(qp, kp, vp, sel, op=op, h0=h0, raster=True, ores=ores)
            if do is not None:
                self.backward(qp, kp, vp, op, dop, lse, sel, grads=grads, h0=h0, raster=True, ores=ores)
            lses.append(lse)
            sels.append(sel)
        if not reuse:
            self._reuse = sels
        out = {"o": op, "lse_block_major": torch.cat(lses, 0), "selections": sels}
        if do is not None:
            out["dq"], out["dk"], out["dv"] = grads
        return out

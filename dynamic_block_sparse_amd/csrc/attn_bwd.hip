// attn_bwd.hip - gradient of the block-sparse flash attention on gfx950 bf16 MFMA.
//
// Built with the default accumulator-register form of MFMA (see build.py).
#include "attn_common.hpp"

namespace prism {

// ---------------------------------------------------------------- backward
//
// dQ kernel (query-major): 2 waves per 64-row query tile, wave w owns rows
// 32*w .. +31 and streams every selected 64-key tile:
//   S^T = K Q^T, P^T = exp2(S^T - lse), dP^T = V dO^T, dS^T = P^T (dP^T - D),
//   dQ^T += K^T dS^T
// dK/dV kernel (key-major): 4 waves per 64-key tile (two roles per 32-key
// half, below) stream the 64-row tiles of every query block that selected the
// tile's block (transposed CSR, ascending):
//   S = Q K^T, P = exp2(S - lse), dP = dO V^T, dS = P (dP - D),
//   dV^T += dO^T P, dK^T += Q^T dS
// Each output element is accumulated by one lane in a fixed order: the
// backward is deterministic.  dQ, dK and dV rows go to their block-major
// position or, through the RowMap, to their raster token (where the row-dot
// pass also reads O).

// dQ keeps one K and one V tile in LDS and fits 256 registers, so two waves
// share each SIMD (measured at 2K: 82 ms against 100 ms double-buffered at one
// wave per SIMD).  Its loads are split by phase: dP^T, which needs only V,
// runs first while K is still landing; V(t+1) is loaded once every wave has
// finished dP^T, K(t+1) once every wave has finished dQ^T.  dK/dV
// double-buffers its Q and dO tiles.
//
// dQ takes its query tiles in the visiting order built by launch_tile_order
// (grouped by first selected key block).  dK/dV keeps raster order: grouping
// its key tiles by the first query block that selects them was measured 1.6%
// slower at 2K, where neighbouring key tiles already share most of their
// query tiles in L2.

template <int D>
__global__ void __launch_bounds__(128, 2)
attn_dq_mfma_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ Dq,
                    uint16_t* __restrict__ dq, int64_t N, int64_t ld, int64_t hs, const int32_t* __restrict__ offs,
                    int nb, const int32_t* __restrict__ sel_off, const int32_t* __restrict__ sel_idx, int64_t cap,
                    const int32_t* __restrict__ order, const uint8_t* __restrict__ skip, const RowMap om,
                    float scale_log2, float scale) {
    __shared__ uint16_t kbuf[1][64 * D], vbuf[1][64 * D];
    const int ntiles = static_cast<int>(N / 64);
    const int wg = xcd_remap(blockIdx.x);
    const int h = wg / ntiles;
    const int64_t p0 = static_cast<int64_t>(tile_of(order, wg, ntiles)) * 64;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hl = lane >> 5, col = lane & 31;
    const int i = find_block(offs, nb, p0);
    if (skip && skip[static_cast<int64_t>(h) * nb + i]) return;   // routed to another path
    const int32_t* __restrict__ so = sel_off + static_cast<int64_t>(h) * (nb + 1);
    const int32_t* __restrict__ si = sel_idx + static_cast<int64_t>(h) * cap;
    const int e0 = so[i];
    const int e1 = static_cast<int>(min(static_cast<int64_t>(so[i + 1]), cap));
    constexpr int KS = D / 16, DM = D / 32;
    const int64_t row = p0 + 32 * wave + col;
    u32x4_t qb[KS], db[KS];
    {
        const uint16_t* qr = q + row * ld + h * hs;
        const uint16_t* dr = dout + row * ld + h * hs;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            qb[s] = *reinterpret_cast<const u32x4_t*>(qr + 16 * s + 8 * hl);
            db[s] = *reinterpret_cast<const u32x4_t*>(dr + 16 * s + 8 * hl);
        }
    }
    const float lrow = lse[static_cast<int64_t>(h) * N + row] * kLog2e;
    const float drow = Dq[static_cast<int64_t>(h) * N + row];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        settle(qb[s]);
        settle(db[s]);
    }
    settle(lrow);
    settle(drow);
    f32x16_t acc[DM];
#pragma unroll
    for (int m = 0; m < DM; ++m)
#pragma unroll
        for (int x = 0; x < 16; ++x) acc[m][x] = 0.0f;
    const uint16_t* __restrict__ kh_ = k + h * hs;
    const uint16_t* __restrict__ vh_ = v + h * hs;

    TileDma<D, 2> dma;
    dma.init(ld, wave, lane);
    constexpr int PER = TileDma<D, 2>::PER;
    const uint16_t* kt = kbuf[0];
    const uint16_t* vt = vbuf[0];
    TileCursor cur;
    cur.init(si, offs, e0, e1);
    int t = cur.next();
    if (t >= 0) {
        dma.load(vbuf[0], vh_ + static_cast<int64_t>(t) * ld, wave);
        dma.load(kbuf[0], kh_ + static_cast<int64_t>(t) * ld, wave);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER) : "memory");   // this wave's V loads
        __syncthreads();
        while (true) {
            f32x16_t sa[2], pa[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int x = 0; x < 16; ++x) sa[mt][x] = pa[mt][x] = 0.0f;
            // dP^T first: it needs only V, while K may still be landing
#pragma unroll
            for (int s = 0; s < KS; ++s)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
                    pa[mt] = mfma32(sw_read16<D>(vt, 32 * mt + col, 16 * s + 8 * hl), db[s], pa[mt]);
            sched_reads_ahead<2, 2, KS, 2>();
            dma_join();                        // K(t) landed; every wave is done with V(t)
            const int tn = cur.next();
            if (tn >= 0) dma.load(vbuf[0], vh_ + static_cast<int64_t>(tn) * ld, wave);
#pragma unroll
            for (int s = 0; s < KS; ++s)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
                    sa[mt] = mfma32(sw_read16<D>(kt, 32 * mt + col, 16 * s + 8 * hl), qb[s], sa[mt]);
            sched_reads_ahead<2, 2, KS, 2>();
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int x = 0; x < 16; ++x) {
                    const float p = fast_exp2(fmaf(sa[mt][x], scale_log2, -lrow));
                    sa[mt][x] = p * (pa[mt][x] - drow);     // dS^T
                }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const u32x4_t bs = pack_kstep(sa[ks >> 1], ks & 1);
#pragma unroll
                for (int m = 0; m < DM; ++m) acc[m] = mfma32(tr_operand<D>(kt, 16 * ks, 32 * m, lane), bs, acc[m]);
            }
            dma_join();                        // V(tn) landed; every wave is done with K(t)
            if (tn < 0) break;
            dma.load(kbuf[0], kh_ + static_cast<int64_t>(tn) * ld, wave);
        }
    }
    uint16_t* out = dq + row_offset(om, row, h);
#pragma unroll
    for (int m = 0; m < DM; ++m)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x16_t& a = acc[m];
            *reinterpret_cast<u32x2_t*>(out + 32 * m + 8 * g + 4 * hl) =
                u32x2_t{pack2(a[4 * g] * scale, a[4 * g + 1] * scale), pack2(a[4 * g + 2] * scale, a[4 * g + 3] * scale)};
        }
}

// dK/dV: 4 waves per 64-key tile, in two roles per 32-key half.  Role 0 holds
// the half's K fragments and computes S = Q K^T, P and dV^T += dO^T P; role 1
// holds its V fragments and computes dP = dO V^T, dS = P (dP - D) and
// dK^T += Q^T dS, taking P from role 0 through LDS.  A wave then keeps one
// accumulator (dV^T or dK^T of 32 keys) instead of two, two waves fit per SIMD,
// and the MFMA work is the same 16 d-step products per row half as with one
// wave doing both.  The query tile is processed in two 32-row halves so that
// the P exchange needs 4 KB per key half:
//   A  role 0: S(0), P(0), P(0) -> LDS         role 1: dP(0)
//   -- barrier
//   B  role 0: S(1), P(1), dV += P(0)          role 1: dP(1), dS(0), dK += dS(0)
//   -- barrier (role 1 has read P(0))
//      role 0: P(1) -> LDS
//   -- barrier
//   C  role 0: dV += P(1)                      role 1: dS(1), dK += dS(1)
// P and dS are computed exactly as with a single wave, and every accumulator
// takes its 16-row k-steps in ascending order, so results do not depend on the
// split.  (Measured at 2K: 103.5 ms against 107.3 ms for 2 waves that each
// computed all four products for 32 keys in 381 registers, one wave per SIMD.)
// The MFMA runs raise the wave's issue priority and the softmax lowers it, so
// that of the two waves sharing a SIMD the one with matrix work goes first.

template <int D>
__global__ void __launch_bounds__(256, 2)
attn_dkdv_mfma_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                      const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ Dq,
                      uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int64_t N, int64_t ld, int64_t hs,
                      const int32_t* __restrict__ offs, int nb, const int32_t* __restrict__ tr_off,
                      const int32_t* __restrict__ tr_idx, int64_t cap, const float* __restrict__ dkbar,
                      const float* __restrict__ dvbar, const RowMap om, float scale_log2, float scale) {
    // Q and dO tiles, lse (natural log) and D = rowsum(dO * O) of their rows
    __shared__ uint16_t qbuf[2][64 * D], obuf[2][64 * D];
    __shared__ float lbuf[2][64], dbuf[2][64];
    // P of one 32-row half per key half: [key half][register group][lane][4]
    __shared__ float pbuf[2][4][64][4];
    const int ntiles = static_cast<int>(N / 64);
    const int wg = xcd_remap(blockIdx.x);
    const int h = wg / ntiles;
    const int64_t k0 = static_cast<int64_t>(wg % ntiles) * 64;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int role = wave & 1, kh = wave >> 1;
    const int hl = lane >> 5, col = lane & 31;
    const int j = find_block(offs, nb, k0);
    const int32_t* __restrict__ to = tr_off + static_cast<int64_t>(h) * (nb + 1);
    const int32_t* __restrict__ ti = tr_idx + static_cast<int64_t>(h) * cap;
    const int e0 = to[j];
    const int e1 = static_cast<int>(min(static_cast<int64_t>(to[j + 1]), cap));
    constexpr int KS = D / 16, DM = D / 32;
    const int64_t key = k0 + 32 * kh + col;
    // K fragments (role 0) or V fragments (role 1) of this wave's 32 keys
    u32x4_t kv[KS];
    {
        const uint16_t* src = (role ? v : k) + key * ld + h * hs;
#pragma unroll
        for (int s = 0; s < KS; ++s) kv[s] = *reinterpret_cast<const u32x4_t*>(src + 16 * s + 8 * hl);
#pragma unroll
        for (int s = 0; s < KS; ++s) settle(kv[s]);
    }
    f32x16_t acc[DM];   // dV^T (role 0) or dK^T (role 1)
#pragma unroll
    for (int m = 0; m < DM; ++m)
#pragma unroll
        for (int x = 0; x < 16; ++x) acc[m][x] = 0.0f;
    const uint16_t* __restrict__ qh_ = q + h * hs;
    const uint16_t* __restrict__ oh_ = dout + h * hs;
    const float* __restrict__ lh = lse + static_cast<int64_t>(h) * N;
    const float* __restrict__ dh = Dq + static_cast<int64_t>(h) * N;
    float4* __restrict__ pex = reinterpret_cast<float4*>(&pbuf[kh][0][0][0]) + lane;

    TileDma<D, 4> dma;
    dma.init(ld, wave, lane);
    const uint32_t loff = 4 * lane;
    auto issue = [&](int t, int b) {
        dma.load(qbuf[b], qh_ + static_cast<int64_t>(t) * ld, wave);
        dma.load(obuf[b], oh_ + static_cast<int64_t>(t) * ld, wave);
        if (wave == 0) dma4(lh + t, loff, lds_addr(lbuf[b]));
        else if (wave == 1) dma4(dh + t, loff, lds_addr(dbuf[b]));
    };
    auto compute = [&](int b) {
        const uint16_t* rb = role ? obuf[b] : qbuf[b];   // row operand: Q for S, dO for dP
        const uint16_t* tb = role ? qbuf[b] : obuf[b];   // transposed operand: dO^T for dV, Q^T for dK
        const float* lt = lbuf[b];
        const float* dt = dbuf[b];
        // S (role 0) or dP (role 1) of row half mr: register x holds query row
        // 32*mr + 8*(x/4) + 4*hl + x%4 against key col of the wave's half
        auto rows = [&](int mr) {
            __builtin_amdgcn_s_setprio(1);
            f32x16_t x;
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = 0.0f;
#pragma unroll
            for (int s = 0; s < KS; ++s) x = mfma32(sw_read16<D>(rb, 32 * mr + col, 16 * s + 8 * hl), kv[s], x);
            __builtin_amdgcn_s_setprio(0);
            return x;
        };
        auto softmax = [&](f32x16_t& x, int mr) {   // S -> P (role 0)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 l4 = *reinterpret_cast<const float4*>(&lt[32 * mr + 8 * g + 4 * hl]);
                const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) x[4 * g + r] = fast_exp2(fmaf(x[4 * g + r], scale_log2, -lv[r] * kLog2e));
            }
        };
        auto dsoft = [&](f32x16_t& x, int mr) {     // dP -> dS = P (dP - D) (role 1)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 p4 = pex[64 * g];
                const float4 d4 = *reinterpret_cast<const float4*>(&dt[32 * mr + 8 * g + 4 * hl]);
                x[4 * g + 0] = p4.x * (x[4 * g + 0] - d4.x);
                x[4 * g + 1] = p4.y * (x[4 * g + 1] - d4.y);
                x[4 * g + 2] = p4.z * (x[4 * g + 2] - d4.z);
                x[4 * g + 3] = p4.w * (x[4 * g + 3] - d4.w);
            }
        };
        auto publish = [&](const f32x16_t& x) {     // P -> LDS (role 0)
#pragma unroll
            for (int g = 0; g < 4; ++g) pex[64 * g] = float4{x[4 * g], x[4 * g + 1], x[4 * g + 2], x[4 * g + 3]};
        };
        auto accumulate = [&](const f32x16_t& x, int mr) {   // acc += tb^T x over the half's 32 rows
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const u32x4_t bx = pack_kstep(x, k2);
#pragma unroll
                for (int m = 0; m < DM; ++m)
                    acc[m] = mfma32(tr_operand<D>(tb, 32 * mr + 16 * k2, 32 * m, lane), bx, acc[m]);
            }
            __builtin_amdgcn_s_setprio(0);
        };
        f32x16_t x0 = rows(0);
        if (role == 0) {
            softmax(x0, 0);
            publish(x0);
        }
        __syncthreads();
        f32x16_t x1 = rows(1);
        if (role == 0) softmax(x1, 1);
        else dsoft(x0, 0);
        accumulate(x0, 0);
        __syncthreads();   // role 1 has read P of half 0
        if (role == 0) publish(x1);
        __syncthreads();
        if (role) dsoft(x1, 1);
        accumulate(x1, 1);
    };

    TileCursor cur;
    cur.init(ti, offs, e0, e1);
    tile_pipeline(cur, issue, compute);
    uint16_t* out = (role ? dk : dv) + row_offset(om, key, h);
    const float f = role ? scale : 1.0f;
    // routed backward: the block-mean gradient of this key block, shared by its B tokens
    const float* __restrict__ add = role ? dkbar : dvbar;
    const float* __restrict__ addj = add ? add + (static_cast<int64_t>(h) * nb + j) * D : nullptr;
    const float invB = 1.0f / static_cast<float>(offs[j + 1] - offs[j]);
#pragma unroll
    for (int m = 0; m < DM; ++m)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x16_t& a = acc[m];
            const int dc = 32 * m + 8 * g + 4 * hl;
            float r[4] = {a[4 * g] * f, a[4 * g + 1] * f, a[4 * g + 2] * f, a[4 * g + 3] * f};
            if (addj)
#pragma unroll
                for (int x = 0; x < 4; ++x) r[x] += addj[dc + x] * invB;
            *reinterpret_cast<u32x2_t*>(out + dc) = u32x2_t{pack2(r[0], r[1]), pack2(r[2], r[3])};
        }
}

// ---------------------------------------------------------------- launcher

hipError_t launch_attn_bwd_mfma(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                                const float* Dq, void* dq, void* dk, void* dv, int64_t N, int heads, int d, int64_t ld,
                                int64_t hs, const int32_t* offs, int nb, const int32_t* so, const int32_t* si,
                                const int32_t* to, const int32_t* ti, int64_t cap, const int32_t* qorder,
                                const RouteGrad* rg, const RowMap& om, float scale, hipStream_t s) {
    const uint8_t* skip = rg ? rg->skip_q : nullptr;
    const float* dkb = rg ? rg->dkbar : nullptr;
    const float* dvb = rg ? rg->dvbar : nullptr;
    const dim3 grid(static_cast<unsigned>(N / 64 * heads));
    const float sl2 = scale * kLog2e;
    const uint16_t* Q = static_cast<const uint16_t*>(q);
    const uint16_t* K = static_cast<const uint16_t*>(k);
    const uint16_t* V = static_cast<const uint16_t*>(v);
    const uint16_t* O = static_cast<const uint16_t*>(dout);
    uint16_t* dQ = static_cast<uint16_t*>(dq);
    uint16_t* dK = static_cast<uint16_t*>(dk);
    uint16_t* dV = static_cast<uint16_t*>(dv);
    if (d == 128) {
        hipLaunchKernelGGL(attn_dq_mfma_kernel<128>, grid, dim3(128), 0, s, Q, K, V, O, lse, Dq, dQ, N, ld, hs, offs,
                           nb, so, si, cap, qorder, skip, om, sl2, scale);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(attn_dkdv_mfma_kernel<128>, grid, dim3(256), 0, s, Q, K, V, O, lse, Dq, dK, dV, N, ld, hs,
                           offs, nb, to, ti, cap, dkb, dvb, om, sl2, scale);
    } else {
        hipLaunchKernelGGL(attn_dq_mfma_kernel<64>, grid, dim3(128), 0, s, Q, K, V, O, lse, Dq, dQ, N, ld, hs, offs,
                           nb, so, si, cap, qorder, skip, om, sl2, scale);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(attn_dkdv_mfma_kernel<64>, grid, dim3(256), 0, s, Q, K, V, O, lse, Dq, dK, dV, N, ld, hs,
                           offs, nb, to, ti, cap, dkb, dvb, om, sl2, scale);
    }
    return hipGetLastError();
}

}  // namespace prism

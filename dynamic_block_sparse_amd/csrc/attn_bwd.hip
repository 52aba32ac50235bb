// attn_bwd.hip - gradient of the block-sparse flash attention on gfx950 bf16 MFMA.
//
// Built with the default accumulator-register form of MFMA (see build.py).
#include "attn_common.hpp"
#include "attn_split.hpp"

namespace prism {

// ---------------------------------------------------------------- backward
//
// dQ kernel (query-major): 2 waves per 64-row query tile, wave w owns rows
// 32*w .. +31 and streams every selected 64-key tile:
//   S^T = K Q^T, P^T = exp2(S^T - lse), dP^T = V dO^T, dS^T = P^T (dP^T - D),
//   dQ^T += K^T dS^T
// with D = rowsum(dO * O) from the row-dot pass (O plus its residual when the
// forward wrote one); it also sums P dP over the row's keys and leaves that,
// the exact D, in place of the row-dot value for the dK/dV kernel.  (D from
// the forward's O alone carries the rounding of P in the forward's P V; in dK
// that error is summed over every query row that uses the key.)
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
// (grouped by first selected key block).  dK/dV keeps raster order inside a
// head: grouping its key tiles by the first query block that selects them was
// measured 1.6% slower at 2K, where neighbouring key tiles already share most
// of their query tiles in L2.  Its heads are visited in a work-balanced order
// (head_order_kernel, below).

template <int D>
struct DqState {
    f32x16_t acc[D / 32];   // dQ^T of the wave's 32 rows (before the scale)
    float dex;              // this lane's part of sum_t P dP over the keys
};

// One pass of the workgroup's query tile (rows p0 .. p0+63 of head h) over the
// key tiles of selected entries e0 .. e1-1 of `si`.
template <int D>
__device__ __forceinline__ void dq_pass(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kh_,
                                        const uint16_t* __restrict__ vh_, const uint16_t* __restrict__ dout,
                                        const float* __restrict__ lse, const float* __restrict__ Dq, int64_t N,
                                        int64_t ld, int64_t hs, int h, int64_t p0, const int32_t* __restrict__ offs,
                                        const int32_t* __restrict__ si, int e0, int e1, uint16_t* kb, uint16_t* vb,
                                        float scale_log2, DqState<D>& st) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hl = lane >> 5, col = lane & 31;
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
#pragma unroll
    for (int m = 0; m < DM; ++m)
#pragma unroll
        for (int x = 0; x < 16; ++x) st.acc[m][x] = 0.0f;
    float dex = 0.0f;

    TileDma<D, 2> dma;
    dma.init(ld, wave, lane);
    constexpr int PER = TileDma<D, 2>::PER;
    const uint16_t* kt = kb;
    const uint16_t* vt = vb;
    TileCursor cur;
    cur.init(si, offs, e0, e1);
    int t = cur.next();
    if (t >= 0) {
        dma.load(vb, vh_ + static_cast<int64_t>(t) * ld, wave);
        dma.load(kb, kh_ + static_cast<int64_t>(t) * ld, wave);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER) : "memory");   // this wave's V loads
        __syncthreads();
        while (true) {
            f32x16_t sa[2], pa[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int x = 0; x < 16; ++x) sa[mt][x] = pa[mt][x] = 0.0f;
            // dP^T first: it needs only V, while K may still be landing
            rows_x_ksteps<D>(vt, col, hl, db, pa[0], pa[1]);
            dma_join();                        // K(t) landed; every wave is done with V(t)
            const int tn = cur.next();
            if (tn >= 0) dma.load(vb, vh_ + static_cast<int64_t>(tn) * ld, wave);
            rows_x_ksteps<D>(kt, col, hl, qb, sa[0], sa[1]);
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int x = 0; x < 16; ++x) {
                    const float p = fast_exp2(fmaf(sa[mt][x], scale_log2, -lrow));
                    dex = fmaf(p, pa[mt][x], dex);
                    sa[mt][x] = p * (pa[mt][x] - drow);     // dS^T
                }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const u32x4_t bs = pack_kstep(sa[ks >> 1], ks & 1);
#pragma unroll
                for (int m = 0; m < DM; ++m)
                    st.acc[m] = mfma32(tr_operand<D>(kt, 16 * ks, 32 * m, lane), bs, st.acc[m]);
            }
            dma_join();                        // V(tn) landed; every wave is done with K(t)
            if (tn < 0) break;
            dma.load(kb, kh_ + static_cast<int64_t>(tn) * ld, wave);
        }
    }
    st.dex = dex;
}

// Write dQ (scaled, bf16) of the tile's rows and, in place of the row-dot
// value, D = sum_t P dP over the row's keys: the definition of rowsum(dO * O)
// for the exact softmax, from the same fp32 P and dP as dS, which the
// forward's O (P rounded to bf16 in P V) only approximates.  The dK/dV kernel,
// launched after, reads it; each row belongs to one workgroup.
template <int D>
__device__ __forceinline__ void dq_store(const DqState<D>& st, uint16_t* __restrict__ dq, float* __restrict__ Dq,
                                         const RowMap& om, int64_t N, int h, int64_t p0, float scale) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int hl = lane >> 5, col = lane & 31;
    constexpr int DM = D / 32;
    const int64_t row = p0 + 32 * wave + col;
    uint16_t* out = dq + row_offset(om, row, h);
#pragma unroll
    for (int m = 0; m < DM; ++m)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x16_t& a = st.acc[m];
            *reinterpret_cast<u32x2_t*>(out + 32 * m + 8 * g + 4 * hl) =
                u32x2_t{pack2(a[4 * g] * scale, a[4 * g + 1] * scale), pack2(a[4 * g + 2] * scale, a[4 * g + 3] * scale)};
        }
    const float dsum = st.dex + __shfl_xor(st.dex, 32, 64);
    if (hl == 0) Dq[static_cast<int64_t>(h) * N + row] = dsum;
}

template <int D>
__global__ void __launch_bounds__(128, 2)
attn_dq_mfma_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                    const uint16_t* __restrict__ dout, const float* __restrict__ lse, float* __restrict__ Dq,
                    uint16_t* __restrict__ dq, int64_t N, int64_t ld, int64_t hs, const int32_t* __restrict__ offs,
                    int nb, const int32_t* __restrict__ sel_off, const int32_t* __restrict__ sel_idx, int64_t cap,
                    const int32_t* __restrict__ order, const uint8_t* __restrict__ skip, const RowMap om,
                    float scale_log2, float scale) {
    __shared__ uint16_t kbuf[64 * D], vbuf[64 * D];
    const int ntiles = static_cast<int>(N / 64);
    const int wg = xcd_remap(blockIdx.x);
    const int h = wg / ntiles;
    const int64_t p0 = static_cast<int64_t>(tile_of(order, wg, ntiles)) * 64;
    const int i = find_block(offs, nb, p0);
    if (skip && skip[static_cast<int64_t>(h) * nb + i]) return;   // split into chunks, or routed to another path
    const int32_t* __restrict__ so = sel_off + static_cast<int64_t>(h) * (nb + 1);
    const int e0 = so[i];
    const int e1 = static_cast<int>(min(static_cast<int64_t>(so[i + 1]), cap));
    DqState<D> st;
    dq_pass<D>(q, k + h * hs, v + h * hs, dout, lse, Dq, N, ld, hs, h, p0, offs,
               sel_idx + static_cast<int64_t>(h) * cap, e0, e1, kbuf, vbuf, scale_log2, st);
    dq_store<D>(st, dq, Dq, om, N, h, p0, scale);
}

// one key-range chunk of a split row's tile (attn_split.hpp): fp32 partial
// dQ^T in register layout and the lanes' parts of sum P dP
template <int D>
__global__ void __launch_bounds__(128, 2)
attn_dq_chunk_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                     const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ Dq,
                     int64_t N, int64_t ld, int64_t hs, const int32_t* __restrict__ offs,
                     const int32_t* __restrict__ sel_idx, int64_t cap, SplitView sv, float scale_log2) {
    __shared__ uint16_t kbuf[64 * D], vbuf[64 * D];
    int idx;
    if (!split_item_of(sv, idx)) return;   // beyond the plan's item count
    const int4 it = sv.items[idx];
    const int ntiles = static_cast<int>(N / 64);
    const int h = it.x / ntiles;
    const int64_t p0 = static_cast<int64_t>(it.x - h * ntiles) * 64;
    DqState<D> st;
    dq_pass<D>(q, k + h * hs, v + h * hs, dout, lse, Dq, N, ld, hs, h, p0, offs,
               sel_idx + static_cast<int64_t>(h) * cap, it.y, it.z, kbuf, vbuf, scale_log2, st);
    constexpr int DM = D / 32;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    float* __restrict__ P = sv.partials + static_cast<int64_t>(it.w) * fwd_partial_floats(D);
    float4* po = reinterpret_cast<float4*>(P) + wave * DM * 4 * 64 + lane;
#pragma unroll
    for (int m = 0; m < DM; ++m)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            po[(m * 4 + g) * 64] = float4{st.acc[m][4 * g], st.acc[m][4 * g + 1], st.acc[m][4 * g + 2],
                                          st.acc[m][4 * g + 3]};
    P[2 * DM * 16 * 64 + wave * 64 + lane] = st.dex;
}

// per split tile: the chunks' partials summed in chunk order, then written as
// the tile kernel would
template <int D>
__global__ void __launch_bounds__(128)
attn_dq_combine_kernel(uint16_t* __restrict__ dq, float* __restrict__ Dq, int64_t N, const int32_t* __restrict__ offs,
                       int nb, SplitView sv, const RowMap om, float scale) {
    const int ntiles = static_cast<int>(N / 64);
    const int wg = blockIdx.x;
    const int h = wg / ntiles;
    const int64_t p0 = static_cast<int64_t>(wg - h * ntiles) * 64;
    const int i = find_block(offs, nb, p0);
    const int64_t ri = static_cast<int64_t>(h) * nb + i;
    if (!sv.heavy[ri]) return;
    const int nt = (offs[i + 1] - offs[i]) >> 6;
    const int t = static_cast<int>((p0 - offs[i]) >> 6);
    const int nch = sv.nchunk[ri];
    const int64_t slot0 = split_part_base(sv, h) + sv.pbase[static_cast<int64_t>(h) * (nb + 1) + i] + t;
    constexpr int DM = D / 32;
    constexpr int PF = fwd_partial_floats(D);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    DqState<D> st;
#pragma unroll
    for (int m = 0; m < DM; ++m)
#pragma unroll
        for (int x = 0; x < 16; ++x) st.acc[m][x] = 0.0f;
    st.dex = 0.0f;
    for (int c = 0; c < nch; ++c) {
        const float* __restrict__ P = sv.partials + (slot0 + static_cast<int64_t>(c) * nt) * PF;
        const float4* po = reinterpret_cast<const float4*>(P) + wave * DM * 4 * 64 + lane;
#pragma unroll
        for (int m = 0; m < DM; ++m)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 x = po[(m * 4 + g) * 64];
                st.acc[m][4 * g] += x.x;
                st.acc[m][4 * g + 1] += x.y;
                st.acc[m][4 * g + 2] += x.z;
                st.acc[m][4 * g + 3] += x.w;
            }
        st.dex += P[2 * DM * 16 * 64 + wave * 64 + lane];
    }
    dq_store<D>(st, dq, Dq, om, N, h, p0, scale);
}

// dK/dV: 4 waves per 64-key tile, in two roles per 32-key half.  Role 0 holds
// the half's K fragments and computes S = Q K^T, P and dV^T += dO^T P; role 1
// holds its V fragments and computes dP = dO V^T, dS = P (dP - D) and
// dK^T += Q^T dS, taking P from role 0 through LDS.  A wave then keeps one
// accumulator (dV^T or dK^T of 32 keys) instead of two, two waves fit per SIMD,
// and the MFMA work is the same 16 d-step products per row half as with one
// wave doing both.  The query tile is processed in two 32-row halves so that
// the P exchange needs 4 KB per key half:
//   A  role 0: S, P(0) -> LDS                  role 1: dP
//   -- barrier
//   B  role 0: dV += P(0), P(1)                role 1: dS(0), dK += dS(0)
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
                      const uint16_t* __restrict__ dout, const float* __restrict__ lse2, const float* __restrict__ Dq,
                      uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int64_t N, int64_t ld, int64_t hs,
                      const int32_t* __restrict__ offs, int nb, const int32_t* __restrict__ tr_off,
                      const int32_t* __restrict__ tr_idx, int64_t cap, const int32_t* __restrict__ horder,
                      const float* __restrict__ dkbar, const float* __restrict__ dvbar, const RowMap om,
                      float scale_log2, float scale) {
    // Q and dO tiles, lse log2(e) and D = rowsum(dO * O) of their rows
    __shared__ uint16_t qbuf[2][64 * D], obuf[2][64 * D];
    __shared__ float lbuf[2][64], dbuf[2][64];
    // P of one 32-row half per key half: [key half][register group][lane][4]
    __shared__ float pbuf[2][4][64][4];
    const int ntiles = static_cast<int>(N / 64);
    const int wg = xcd_remap(blockIdx.x);
    const int h = horder[wg / ntiles];   // head order of the launch (balanced across XCDs)
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
        // role 1 holds -V (a sign flip, exact in bf16): its products then
        // start from D and give D - dP with no separate subtraction
        const uint32_t flip = role ? 0x80008000u : 0u;
#pragma unroll
        for (int s = 0; s < KS; ++s) kv[s] ^= flip;
    }
    f32x16_t acc[DM];   // dV^T (role 0) or dK^T (role 1)
#pragma unroll
    for (int m = 0; m < DM; ++m)
#pragma unroll
        for (int x = 0; x < 16; ++x) acc[m][x] = 0.0f;
    const uint16_t* __restrict__ qh_ = q + h * hs;
    const uint16_t* __restrict__ oh_ = dout + h * hs;
    const float* __restrict__ lh = lse2 + static_cast<int64_t>(h) * N;
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
    // b, the buffer of the current tile, alternates at run time (an unrolled
    // pair of iterations with constant buffers does not fit the registers).
    auto compute = [&](int b) {
        const uint16_t* tb = role ? qbuf[b] : obuf[b];   // transposed operand: dO^T for dV, Q^T for dK
        const float* dt = dbuf[b];
        const float* l2 = lbuf[b];
        // S (role 0) or D - dP (role 1) of both row halves: register x of half
        // mr holds query row 32*mr + 8*(x/4) + 4*hl + x%4 against key col of
        // the wave's half (two independent MFMA chains, LDS reads two steps
        // ahead).  Each role has its own chain, so role 0's first products
        // take the MFMA's zero operand instead of 32 register moves.
        f32x16_t x0, x1;
        float4 lreg[2][4];   // role 0: the rows' lse log2(e), read before the products
        if (role == 0) {
#pragma unroll
            for (int mr = 0; mr < 2; ++mr)
#pragma unroll
                for (int g = 0; g < 4; ++g) lreg[mr][g] = *reinterpret_cast<const float4*>(&l2[32 * mr + 8 * g + 4 * hl]);
#pragma unroll
            for (int i = 0; i < 16; ++i) x0[i] = x1[i] = 0.0f;
            __builtin_amdgcn_s_setprio(1);
            rows_x_ksteps<D>(qbuf[b], col, hl, kv, x0, x1);
            __builtin_amdgcn_s_setprio(0);
        } else {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 d0 = *reinterpret_cast<const float4*>(&dt[8 * g + 4 * hl]);
                const float4 d1 = *reinterpret_cast<const float4*>(&dt[32 + 8 * g + 4 * hl]);
                x0[4 * g] = d0.x, x0[4 * g + 1] = d0.y, x0[4 * g + 2] = d0.z, x0[4 * g + 3] = d0.w;
                x1[4 * g] = d1.x, x1[4 * g + 1] = d1.y, x1[4 * g + 2] = d1.z, x1[4 * g + 3] = d1.w;
            }
            __builtin_amdgcn_s_setprio(1);
            rows_x_ksteps<D>(obuf[b], col, hl, kv, x0, x1);
            __builtin_amdgcn_s_setprio(0);
        }
        auto softmax = [&](f32x16_t& x, int mr) {   // S -> P (role 0)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 l4 = lreg[mr][g];
                const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) x[4 * g + r] = fast_exp2(fmaf(x[4 * g + r], scale_log2, -lv[r]));
            }
        };
        auto dsoft = [&](f32x16_t& x) {             // D - dP -> -dS = P (D - dP) (role 1)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 p4 = pex[64 * g];
                x[4 * g + 0] *= p4.x;
                x[4 * g + 1] *= p4.y;
                x[4 * g + 2] *= p4.z;
                x[4 * g + 3] *= p4.w;
            }
        };
        auto publish = [&](const f32x16_t& x) {     // P -> LDS (role 0)
#pragma unroll
            for (int g = 0; g < 4; ++g) pex[64 * g] = float4{x[4 * g], x[4 * g + 1], x[4 * g + 2], x[4 * g + 3]};
        };
        auto accumulate = [&](const f32x16_t& x, int mr) {   // acc += tb^T x over the half's 32 rows
            const u32x4_t bx[2] = {pack_kstep(x, 0), pack_kstep(x, 1)};
            __builtin_amdgcn_s_setprio(1);
            tr_accumulate<D, 2>(tb, 32 * mr, bx, acc, lane);
            __builtin_amdgcn_s_setprio(0);
        };
        if (role == 0) {
            softmax(x0, 0);
            publish(x0);
        }
        __syncthreads();
        if (role) dsoft(x0);
        accumulate(x0, 0);
        if (role == 0) softmax(x1, 1);   // under the dV products just issued
        __syncthreads();   // role 1 has read P of half 0
        if (role == 0) publish(x1);
        __syncthreads();
        if (role) dsoft(x1);
        accumulate(x1, 1);
    };

    TileCursor cur;
    cur.init(ti, offs, e0, e1);
    tile_pipeline(cur, issue, compute);
    uint16_t* out = (role ? dk : dv) + row_offset(om, key, h);
    const float f = role ? -scale : 1.0f;   // role 1 summed Q^T (-dS)
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

// ---------------------------------------------------------------- head order of the dK/dV launch
//
// Workgroups are dealt to the 8 XCDs in contiguous ranges of (head, key tile),
// so with H heads an XCD runs H/8 whole heads.  A head's dK/dV work is its
// count of (query tile, key tile) pairs, which Top-p makes uneven across heads
// (diffuse heads select thousands of blocks per row; reading guide, xyznot.com
// paper 2610.05416, "Các ý tưởng cốt lõi"): at 2K the 24 heads range from
// 0.56x to 1.47x of the mean, and the XCD holding the heaviest three finishes
// last.  The launch therefore visits heads in an order whose consecutive runs
// of H/8 heads carry about equal work: heaviest head first into the lightest
// run that still has room.  Each head's tiles and sums are unchanged, so the
// outputs do not depend on the order.

// cost[h] += tiles(j) * sum of tiles(i) over the query blocks i of key block
// j's transposed list: one wave per (key block, head)
__global__ void __launch_bounds__(64)
head_cost_kernel(const int32_t* __restrict__ tr_off, const int32_t* __restrict__ tr_idx, const int32_t* __restrict__ offs,
                 int nb, int64_t cap, unsigned long long* __restrict__ cost) {
    const int j = blockIdx.x, h = blockIdx.y;
    const int32_t* __restrict__ to = tr_off + static_cast<int64_t>(h) * (nb + 1);
    const int32_t* __restrict__ ti = tr_idx + static_cast<int64_t>(h) * cap;
    const int64_t e1 = min(static_cast<int64_t>(to[j + 1]), cap);
    unsigned long long s = 0;
    for (int64_t e = to[j] + threadIdx.x; e < e1; e += 64) {
        const int i = ti[e];
        s += static_cast<unsigned long long>((offs[i + 1] - offs[i]) >> 6);
    }
    s = wave_sum(s);
    if (threadIdx.x == 0 && s) atomicAdd(&cost[h], s * static_cast<unsigned long long>((offs[j + 1] - offs[j]) >> 6));
}

// order[slot] = head; runs of H/8 slots are the XCDs' shares.  Identity when H
// is not a multiple of 8 (ranges would straddle heads) or outside [16, 256].
__global__ void __launch_bounds__(64)
head_order_kernel(const unsigned long long* __restrict__ cost, int heads, int32_t* __restrict__ order) {
    const bool balance = heads % 8 == 0 && heads >= 16 && heads <= 256;
    if (!balance) {
        for (int x = threadIdx.x; x < heads; x += 64) order[x] = x;
        return;
    }
    if (threadIdx.x != 0) return;
    const int per = heads / 8;
    unsigned long long load[8] = {};
    int fill[8] = {};
    uint64_t taken[4] = {};   // heads picked so far (heads <= 256)
    for (int n = 0; n < heads; ++n) {
        int best = -1;   // heaviest head not yet placed, the lower index on ties
        for (int x = 0; x < heads; ++x)
            if (!((taken[x >> 6] >> (x & 63)) & 1) && (best < 0 || cost[x] > cost[best])) best = x;
        taken[best >> 6] |= uint64_t{1} << (best & 63);
        int bin = -1;    // lightest run with room, the lower index on ties
        for (int b = 0; b < 8; ++b)
            if (fill[b] < per && (bin < 0 || load[b] < load[bin])) bin = b;
        order[bin * per + fill[bin]] = best;
        ++fill[bin];
        load[bin] += cost[best];
    }
}

// ---------------------------------------------------------------- launcher

hipError_t launch_head_order(const int32_t* tr_off, const int32_t* tr_idx, const int32_t* offs, int nb, int heads,
                             int64_t cap, unsigned long long* cost, int32_t* order, hipStream_t s) {
    hipError_t e = fill_zero(reinterpret_cast<int32_t*>(cost), 2 * static_cast<int64_t>(heads), s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(head_cost_kernel, dim3(nb, heads), dim3(64), 0, s, tr_off, tr_idx, offs, nb, cap, cost);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(head_order_kernel, dim3(1), dim3(64), 0, s, cost, heads, order);
    return hipGetLastError();
}

hipError_t launch_attn_dq_mfma(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                              float* Dq, void* dq, int64_t N, int heads, int d, int64_t ld, int64_t hs,
                              const int32_t* offs, int nb, const int32_t* so, const int32_t* si, int64_t cap,
                              const int32_t* qorder, const uint8_t* skip, const RowMap& om, float scale,
                              hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(N / 64 * heads));
    const float sl2 = scale * kLog2e;
    const uint16_t* Q = static_cast<const uint16_t*>(q);
    const uint16_t* K = static_cast<const uint16_t*>(k);
    const uint16_t* V = static_cast<const uint16_t*>(v);
    const uint16_t* O = static_cast<const uint16_t*>(dout);
    uint16_t* dQ = static_cast<uint16_t*>(dq);
    if (d == 128)
        hipLaunchKernelGGL(attn_dq_mfma_kernel<128>, grid, dim3(128), 0, s, Q, K, V, O, lse, Dq, dQ, N, ld, hs, offs,
                           nb, so, si, cap, qorder, skip, om, sl2, scale);
    else
        hipLaunchKernelGGL(attn_dq_mfma_kernel<64>, grid, dim3(128), 0, s, Q, K, V, O, lse, Dq, dQ, N, ld, hs, offs,
                           nb, so, si, cap, qorder, skip, om, sl2, scale);
    return hipGetLastError();
}

hipError_t launch_attn_dq_split(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                                float* Dq, void* dq, int64_t N, int heads, int d, int64_t ld, int64_t hs,
                                const int32_t* offs, int nb, const int32_t* si, int64_t cap, const SplitView& sv,
                                const RowMap& om, float scale, hipStream_t s) {
    const float sl2 = scale * kLog2e;
    const uint16_t* Q = static_cast<const uint16_t*>(q);
    const uint16_t* K = static_cast<const uint16_t*>(k);
    const uint16_t* V = static_cast<const uint16_t*>(v);
    const uint16_t* O = static_cast<const uint16_t*>(dout);
    uint16_t* dQ = static_cast<uint16_t*>(dq);
    const dim3 cgrid(static_cast<unsigned>(split_grid(sv)));
    const dim3 tgrid(static_cast<unsigned>(N / 64 * heads));
    if (d == 128) {
        hipLaunchKernelGGL(attn_dq_chunk_kernel<128>, cgrid, dim3(128), 0, s, Q, K, V, O, lse, Dq, N, ld, hs, offs, si,
                           cap, sv, sl2);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(attn_dq_combine_kernel<128>, tgrid, dim3(128), 0, s, dQ, Dq, N, offs, nb, sv, om, scale);
    } else {
        hipLaunchKernelGGL(attn_dq_chunk_kernel<64>, cgrid, dim3(128), 0, s, Q, K, V, O, lse, Dq, N, ld, hs, offs, si,
                           cap, sv, sl2);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(attn_dq_combine_kernel<64>, tgrid, dim3(128), 0, s, dQ, Dq, N, offs, nb, sv, om, scale);
    }
    return hipGetLastError();
}

hipError_t launch_attn_dkdv_mfma(const void* q, const void* k, const void* v, const void* dout, const float* lse2,
                                 const float* Dq, void* dk, void* dv, int64_t N, int heads, int d, int64_t ld,
                                 int64_t hs, const int32_t* offs, int nb, const int32_t* to, const int32_t* ti,
                                 int64_t cap, const int32_t* horder, const RouteGrad* rg, const RowMap& om, float scale,
                                 hipStream_t s) {
    const float* dkb = rg ? rg->dkbar : nullptr;
    const float* dvb = rg ? rg->dvbar : nullptr;
    const dim3 grid(static_cast<unsigned>(N / 64 * heads));
    const float sl2 = scale * kLog2e;
    const uint16_t* Q = static_cast<const uint16_t*>(q);
    const uint16_t* K = static_cast<const uint16_t*>(k);
    const uint16_t* V = static_cast<const uint16_t*>(v);
    const uint16_t* O = static_cast<const uint16_t*>(dout);
    uint16_t* dK = static_cast<uint16_t*>(dk);
    uint16_t* dV = static_cast<uint16_t*>(dv);
    if (d == 128)
        hipLaunchKernelGGL(attn_dkdv_mfma_kernel<128>, grid, dim3(256), 0, s, Q, K, V, O, lse2, Dq, dK, dV, N, ld, hs,
                           offs, nb, to, ti, cap, horder, dkb, dvb, om, sl2, scale);
    else
        hipLaunchKernelGGL(attn_dkdv_mfma_kernel<64>, grid, dim3(256), 0, s, Q, K, V, O, lse2, Dq, dK, dV, N, ld, hs,
                           offs, nb, to, ti, cap, horder, dkb, dvb, om, sl2, scale);
    return hipGetLastError();
}

}  // namespace prism

// attn_fwd.hip - block-sparse flash attention forward on gfx950 bf16 MFMA.
//
// Built with MFMA accumulators in ordinary VGPRs (see build.py): the kernel
// fits in 256 VGPRs that way and was measured faster than with accumulator
// registers.
#include "attn_common.hpp"

namespace prism {

// ---------------------------------------------------------------- forward
//
// 2 waves per 64-row query tile; wave w owns rows 32*w .. +31 and streams
// every selected 64-key tile.  Scores are computed transposed, S^T = K Q^T,
// so a lane owns one query row: its max and sum need one cross-lane swap and
// the O^T rescale is a per-lane scalar.  The running maximum is raised only
// when a tile's maximum exceeds it by more than 8 (log2 units), so O is
// rescaled rarely; exponents stay below 2^8 in between.
//
// LDS holds one K and one V tile (32 KB at d = 128), so four workgroups, two
// waves per SIMD, share a CU and one wave's softmax overlaps another's MFMAs.
// Within the workgroup the loads are split by phase: K(t+1) is loaded as soon
// as every wave has finished the scores of tile t (it lands during softmax and
// P V), V(t+1) once every wave has finished P V (it lands during the next
// scores).  Each phase boundary is one wait-and-barrier.  (Measured at 2K: 71
// ms, against 79 ms with double-buffered K and V at one wave per SIMD.)
//
// The scores run at raised wave priority, the softmax at the default one.
// P enters P V rounded to bf16 and O is divided by the sum of those rounded
// values; the log-sum-exp keeps the exact fp32 sum.  Output rows go to their
// block-major position or, through the RowMap, to their raster token.
//
// Query tiles are taken in the visiting order built by launch_tile_order
// (tiles grouped by their first selected key block): order[h * ntiles + j] is
// the j-th tile of head h.

template <int D>
__global__ void __launch_bounds__(128, 2)
attn_fwd_mfma_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                     uint16_t* __restrict__ o, float* __restrict__ lse, int64_t N, int64_t ld, int64_t hs,
                     const int32_t* __restrict__ offs, int nb, const int32_t* __restrict__ sel_off,
                     const int32_t* __restrict__ sel_idx, int64_t cap, const int32_t* __restrict__ order,
                     const uint8_t* __restrict__ skip, const RowMap om, float scale_log2) {
    __shared__ uint16_t kbuf[64 * D], vbuf[64 * D];
    const int ntiles = static_cast<int>(N / 64);
    const int wg = xcd_remap(blockIdx.x);
    const int h = wg / ntiles;
    const int64_t p0 = static_cast<int64_t>(tile_of(order, wg, ntiles)) * 64;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hl = lane >> 5, col = lane & 31;
    const int i = find_block(offs, nb, p0);
    if (skip && skip[static_cast<int64_t>(h) * nb + i]) return;   // routed to another path
    const uint16_t* __restrict__ kh_ = k + h * hs;
    const uint16_t* __restrict__ vh_ = v + h * hs;
    const int32_t* __restrict__ so = sel_off + static_cast<int64_t>(h) * (nb + 1);
    const int32_t* __restrict__ si = sel_idx + static_cast<int64_t>(h) * cap;
    const int e0 = so[i];
    const int e1 = static_cast<int>(min(static_cast<int64_t>(so[i + 1]), cap));
    constexpr int KS = D / 16, DM = D / 32;
    const int64_t row = p0 + 32 * wave + col;
    u32x4_t qb[KS];
    {
        const uint16_t* qrow = q + row * ld + h * hs;
#pragma unroll
        for (int s = 0; s < KS; ++s) qb[s] = *reinterpret_cast<const u32x4_t*>(qrow + 16 * s + 8 * hl);
#pragma unroll
        for (int s = 0; s < KS; ++s) settle(qb[s]);
    }
    f32x16_t oacc[DM];
#pragma unroll
    for (int m = 0; m < DM; ++m)
#pragma unroll
        for (int x = 0; x < 16; ++x) oacc[m][x] = 0.0f;
    float mrow = -INFINITY, lrow = 0.0f, lrnd = 0.0f;   // row sums of P exact and of P rounded to bf16

    TileDma<D, 2> dma;
    dma.init(ld, wave, lane);
    constexpr int PER = TileDma<D, 2>::PER;
    TileCursor cur;
    cur.init(si, offs, e0, e1);
    int t = cur.next();
    if (t >= 0) {
        dma.load(kbuf, kh_ + static_cast<int64_t>(t) * ld, wave);
        dma.load(vbuf, vh_ + static_cast<int64_t>(t) * ld, wave);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER) : "memory");   // this wave's K loads
        __syncthreads();
        const uint16_t* kt = kbuf;
        const uint16_t* vt = vbuf;
        while (true) {
            __builtin_amdgcn_s_setprio(1);
            f32x16_t s0, s1;
#pragma unroll
            for (int x = 0; x < 16; ++x) s0[x] = s1[x] = 0.0f;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                s0 = mfma32(sw_read16<D>(kt, col, 16 * s + 8 * hl), qb[s], s0);
                s1 = mfma32(sw_read16<D>(kt, 32 + col, 16 * s + 8 * hl), qb[s], s1);
            }
            sched_reads_ahead<2, 2, KS, 2>();
            __builtin_amdgcn_s_setprio(0);
            dma_join();                    // V(t) landed; every wave is done with K(t)
            const int tn = cur.next();
            if (tn >= 0) dma.load(kbuf, kh_ + static_cast<int64_t>(tn) * ld, wave);
            float mx = -INFINITY;
#pragma unroll
            for (int x = 0; x < 16; ++x) mx = fmaxf(mx, fmaxf(s0[x], s1[x]));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * scale_log2;
            if (__any(mx > mrow + 8.0f)) {
                const float mnew = fmaxf(mrow, mx);
                const float alpha = fast_exp2(mrow - mnew);
                mrow = mnew;
                lrow *= alpha;
                lrnd *= alpha;
#pragma unroll
                for (int m = 0; m < DM; ++m)
#pragma unroll
                    for (int x = 0; x < 16; ++x) oacc[m][x] *= alpha;
            }
            float ls = 0.0f;
#pragma unroll
            for (int x = 0; x < 16; ++x) {
                s0[x] = fast_exp2(fmaf(s0[x], scale_log2, -mrow));
                s1[x] = fast_exp2(fmaf(s1[x], scale_log2, -mrow));
                ls += s0[x] + s1[x];
            }
            lrow += ls;
            // P is rounded once to bf16 for P V, and O is normalised by the sum
            // of the same rounded values: O is then an exact convex combination
            // of V rows with the rounded weights, so a rounding error shared by
            // the weights (similar values of P rounding the same way) cancels
            // instead of scaling O.  The log-sum-exp keeps the exact sum.
            const u32x4_t pb[4] = {pack_kstep(s0, 0), pack_kstep(s0, 1), pack_kstep(s1, 0), pack_kstep(s1, 1)};
            float lr = 0.0f;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    lr += __uint_as_float(pb[ks][w] << 16) + __uint_as_float(pb[ks][w] & 0xffff0000u);
            lrnd += lr;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int m = 0; m < DM; ++m) oacc[m] = mfma32(tr_operand<D>(vt, 16 * ks, 32 * m, lane), pb[ks], oacc[m]);
            dma_join();                    // K(tn) landed; every wave is done with V(t)
            if (tn < 0) break;
            dma.load(vbuf, vh_ + static_cast<int64_t>(tn) * ld, wave);
        }
    }
    // lanes l and l^32 hold the two halves of a row's sum
    const float lt = lrow + __shfl_xor(lrow, 32, 64);
    const float inv = 1.0f / (lrnd + __shfl_xor(lrnd, 32, 64));
    uint16_t* orow = o + row_offset(om, row, h);
#pragma unroll
    for (int m = 0; m < DM; ++m)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x16_t& a = oacc[m];
            *reinterpret_cast<u32x2_t*>(orow + 32 * m + 8 * g + 4 * hl) =
                u32x2_t{pack2(a[4 * g] * inv, a[4 * g + 1] * inv), pack2(a[4 * g + 2] * inv, a[4 * g + 3] * inv)};
        }
    if (hl == 0) lse[static_cast<int64_t>(h) * N + row] = (mrow + __log2f(lt)) * kLn2;
}

// ---------------------------------------------------------------- launcher

hipError_t launch_attn_fwd_mfma(const void* q, const void* k, const void* v, void* o, float* lse, int64_t N, int heads,
                                int d, int64_t ld, int64_t hs, const int32_t* offs, int nb, const int32_t* so,
                                const int32_t* si, int64_t cap, const int32_t* order, const uint8_t* skip,
                                const RowMap& om, float scale, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(N / 64 * heads));
    const float sl2 = scale * kLog2e;
    const uint16_t* Q = static_cast<const uint16_t*>(q);
    const uint16_t* K = static_cast<const uint16_t*>(k);
    const uint16_t* V = static_cast<const uint16_t*>(v);
    uint16_t* O = static_cast<uint16_t*>(o);
    if (d == 128)
        hipLaunchKernelGGL(attn_fwd_mfma_kernel<128>, grid, dim3(128), 0, s, Q, K, V, O, lse, N, ld, hs, offs, nb, so,
                           si, cap, order, skip, om, sl2);
    else
        hipLaunchKernelGGL(attn_fwd_mfma_kernel<64>, grid, dim3(128), 0, s, Q, K, V, O, lse, N, ld, hs, offs, nb, so,
                           si, cap, order, skip, om, sl2);
    return hipGetLastError();
}

}  // namespace prism

// attn_fwd.hip - block-sparse flash attention forward on gfx950 bf16 MFMA.
//
// Built with MFMA accumulators in ordinary VGPRs (see build.py): the kernel
// fits in 256 VGPRs that way and was measured faster than with accumulator
// registers.
#include <cstdlib>

#include "attn_common.hpp"
#include "attn_split.hpp"

namespace prism {

// ---------------------------------------------------------------- forward
//
// 2 waves per 64-row query tile; wave w owns rows 32*w .. +31 and streams
// the 64-key tiles of a list of selected blocks.  Scores are computed
// transposed, S^T = K Q^T, so a lane owns one query row: its max and sum need
// one cross-lane swap and the O^T rescale is a per-lane scalar.  The running
// maximum is raised only when a tile's maximum exceeds it by more than 8
// (log2 units), so O is rescaled rarely; exponents stay below 2^8 in between.
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
// values; the log-sum-exp keeps the exact fp32 sum.
//
// Three kernels share that loop:
//   attn_fwd_mfma_kernel   one workgroup per query tile over its block's whole
//                          selected list, taken in the visiting order built by
//                          launch_tile_order (tiles grouped by their first
//                          selected key block); output rows go to their
//                          block-major position or, through the RowMap, to
//                          their raster token.  Tiles whose block is marked in
//                          `skip` exit at once (rows split into key ranges, or
//                          routed to another path).
//   attn_fwd_chunk_kernel  one workgroup per work item of a split plan: one
//                          tile over one key-range chunk of its block's list,
//                          written as an fp32 partial (unnormalised O and the
//                          row statistics).  The items of a head are ordered by
//                          key range, so the workgroups that run together on
//                          one XCD read the same key tiles through its L2.
//   attn_fwd_combine_kernel  merges each split tile's partials in chunk order
//                          and writes O and lse as the tile kernel would.

template <int D>
struct FwdState {
    f32x16_t oacc[D / 32];
    float mrow, lrow, lrnd;   // running max (log2 units) and row sums of P exact and of P rounded to bf16
};

// One pass of the workgroup's query tile (rows p0 .. p0+63 of head h) over the
// key tiles of selected entries e0 .. e1-1 of `si`.
template <int D, int NW = 2>
__device__ __forceinline__ void fwd_pass(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kh_,
                                         const uint16_t* __restrict__ vh_, int64_t ld, int64_t hs, int h, int64_t p0,
                                         const int32_t* __restrict__ offs, const int32_t* __restrict__ si, int e0,
                                         int e1, uint16_t* kbuf, uint16_t* vbuf, float scale_log2, FwdState<D>& st) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hl = lane >> 5, col = lane & 31;
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
#pragma unroll
    for (int m = 0; m < DM; ++m)
#pragma unroll
        for (int x = 0; x < 16; ++x) st.oacc[m][x] = 0.0f;
    float mrow = -INFINITY, lrow = 0.0f, lrnd = 0.0f;

    TileDma<D, NW> dma;
    dma.init(ld, wave, lane);
    constexpr int PER = TileDma<D, NW>::PER;
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
            rows_x_ksteps<D>(kt, col, hl, qb, s0, s1);
            __builtin_amdgcn_s_setprio(0);
            dma_join();                    // V(t) landed; every wave is done with K(t)
            const int tn = cur.next();
            if (tn >= 0) dma.load(kbuf, kh_ + static_cast<int64_t>(tn) * ld, wave);
            // four independent chains of v_max3 over the 32 raw scores
            float mq[4] = {s0[0], s0[1], s0[2], s0[3]};
#pragma unroll
            for (int x = 0; x < 16; ++x) {
                const int c = x & 3;
                mq[c] = x < 4 ? max3_raw(mq[c], s1[x], s1[x]) : max3_raw(mq[c], s0[x], s1[x]);
            }
            float mx = max3_raw(max3_raw(mq[0], mq[1], mq[2]), mq[3], mq[3]);
            mx = max_across_halves(mx) * scale_log2;
            if (__any(mx > mrow + 8.0f)) {
                const float mnew = fmaxf(mrow, mx);
                const float alpha = fast_exp2(mrow - mnew);
                mrow = mnew;
                lrow *= alpha;
                lrnd *= alpha;
#pragma unroll
                for (int m = 0; m < DM; ++m)
#pragma unroll
                    for (int x = 0; x < 16; ++x) st.oacc[m][x] *= alpha;
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
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int w = 0; w < 4; ++w) lrnd = sum_bf16_pair(pb[ks][w], lrnd);
            tr_accumulate<D, 4>(vt, 0, pb, st.oacc, lane);
            dma_join();                    // K(tn) landed; every wave is done with V(t)
            if (tn < 0) break;
            dma.load(vbuf, vh_ + static_cast<int64_t>(tn) * ld, wave);
        }
    }
    st.mrow = mrow;
    st.lrow = lrow;
    st.lrnd = lrnd;
}

// Normalise and write O (and its bf16 residual) and lse of the tile's rows.
template <int D>
__device__ __forceinline__ void fwd_store(const FwdState<D>& st, uint16_t* __restrict__ o, uint16_t* __restrict__ ores,
                                          float* __restrict__ lse, const RowMap& om, int64_t N, int h, int64_t p0) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int hl = lane >> 5, col = lane & 31;
    constexpr int DM = D / 32;
    const int64_t row = p0 + 32 * wave + col;
    // lanes l and l^32 hold the two halves of a row's sum
    const float lt = st.lrow + __shfl_xor(st.lrow, 32, 64);
    const float lsum = st.lrnd + __shfl_xor(st.lrnd, 32, 64);
    const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;   // a row with no stored entry: O = 0, lse = -inf
    const int64_t ro = row_offset(om, row, h);
#pragma unroll
    for (int m = 0; m < DM; ++m)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x16_t& a = st.oacc[m];
            const float r[4] = {a[4 * g] * inv, a[4 * g + 1] * inv, a[4 * g + 2] * inv, a[4 * g + 3] * inv};
            const u32x2_t hi{pack2(r[0], r[1]), pack2(r[2], r[3])};
            const int64_t at = ro + 32 * m + 8 * g + 4 * hl;
            *reinterpret_cast<u32x2_t*>(o + at) = hi;
            if (ores) *reinterpret_cast<u32x2_t*>(ores + at) = residual4(r, hi);
        }
    if (hl == 0) lse[static_cast<int64_t>(h) * N + row] = (st.mrow + __log2f(lt)) * kLn2;
}

// NW = 2: one 64-row tile per workgroup.  NW = 4: two sibling tiles (tiles
// 2u and 2u + 1 of one block, which share the block's selected list) per
// workgroup, waves 2 and 3 taking the second: every K and V tile is loaded
// once for 128 rows, and each wave runs the same loop as with NW = 2.  With
// `pairs` set the NW = 2 launch leaves the paired tiles to the NW = 4 one.
template <int D, int NW>
__global__ void __launch_bounds__(64 * NW, 2)
attn_fwd_mfma_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                     uint16_t* __restrict__ o, float* __restrict__ lse, int64_t N, int64_t ld, int64_t hs,
                     const int32_t* __restrict__ offs, int nb, const int32_t* __restrict__ sel_off,
                     const int32_t* __restrict__ sel_idx, int64_t cap, const int32_t* __restrict__ order,
                     const uint8_t* __restrict__ skip, const RowMap om, float scale_log2, uint16_t* __restrict__ ores,
                     int pairs) {
    __shared__ uint16_t kbuf[64 * D], vbuf[64 * D];
    const int ntiles = static_cast<int>(N / 64);
    const int wg = xcd_remap(blockIdx.x);
    const int h = wg / ntiles;
    const int64_t p0 = static_cast<int64_t>(tile_of(order, wg, ntiles)) * 64;
    const int i = find_block(offs, nb, p0);
    if (skip && skip[static_cast<int64_t>(h) * nb + i]) return;   // split into chunks, or routed to another path
    const int nt = (offs[i + 1] - offs[i]) >> 6;
    const int t = static_cast<int>((p0 - offs[i]) >> 6);
    const bool paired = (t | 1) < nt;   // tile t has a sibling tile t ^ 1
    if (NW == 4 ? (!paired || (t & 1)) : (pairs && paired)) return;
    const int32_t* __restrict__ so = sel_off + static_cast<int64_t>(h) * (nb + 1);
    const int e0 = so[i];
    const int e1 = static_cast<int>(min(static_cast<int64_t>(so[i + 1]), cap));
    FwdState<D> st;
    fwd_pass<D, NW>(q, k + h * hs, v + h * hs, ld, hs, h, p0, offs, sel_idx + static_cast<int64_t>(h) * cap, e0, e1,
                    kbuf, vbuf, scale_log2, st);
    fwd_store<D>(st, o, ores, lse, om, N, h, p0);
}

template <int D>
__global__ void __launch_bounds__(128, 2)
attn_fwd_chunk_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                      int64_t N, int64_t ld, int64_t hs, const int32_t* __restrict__ offs,
                      const int32_t* __restrict__ sel_idx, int64_t cap, SplitView sv, float scale_log2) {
    __shared__ uint16_t kbuf[64 * D], vbuf[64 * D];
    int idx;
    if (!split_item_of(sv, idx)) return;   // beyond the plan's item count
    const int4 it = sv.items[idx];
    const int ntiles = static_cast<int>(N / 64);
    const int h = it.x / ntiles;
    const int64_t p0 = static_cast<int64_t>(it.x - h * ntiles) * 64;
    FwdState<D> st;
    fwd_pass<D>(q, k + h * hs, v + h * hs, ld, hs, h, p0, offs, sel_idx + static_cast<int64_t>(h) * cap, it.y, it.z,
                kbuf, vbuf, scale_log2, st);
    // partial slot: O^T accumulators in register layout, lane-contiguous float4s
    constexpr int DM = D / 32;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    float* __restrict__ P = sv.partials + static_cast<int64_t>(it.w) * fwd_partial_floats(D);
    float4* po = reinterpret_cast<float4*>(P) + wave * DM * 4 * 64 + lane;
#pragma unroll
    for (int m = 0; m < DM; ++m)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            po[(m * 4 + g) * 64] = float4{st.oacc[m][4 * g], st.oacc[m][4 * g + 1], st.oacc[m][4 * g + 2],
                                          st.oacc[m][4 * g + 3]};
    float* tail = P + 2 * DM * 16 * 64 + wave * 64 + lane;
    tail[0] = st.mrow;
    tail[128] = st.lrow;
    tail[256] = st.lrnd;
}

// One workgroup per query tile of the launch; tiles of rows that were not
// split exit at once.  Chunk c of tile t of split row i sits in partial slot
// base(h) + pbase[h][i] + c * ntiles_i + t; the chunks are merged in order
// (each rescaled to the largest maximum), so the result does not depend on
// the order in which the chunk workgroups ran.
template <int D>
__global__ void __launch_bounds__(128)
attn_fwd_combine_kernel(uint16_t* __restrict__ o, float* __restrict__ lse, uint16_t* __restrict__ ores, int64_t N,
                        const int32_t* __restrict__ offs, int nb, SplitView sv, const RowMap om) {
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
    const int tl = 2 * DM * 16 * 64 + wave * 64 + lane;
    float m = -INFINITY;
    for (int c = 0; c < nch; ++c) m = fmaxf(m, sv.partials[(slot0 + static_cast<int64_t>(c) * nt) * PF + tl]);
    FwdState<D> st;
#pragma unroll
    for (int mm = 0; mm < DM; ++mm)
#pragma unroll
        for (int x = 0; x < 16; ++x) st.oacc[mm][x] = 0.0f;
    st.lrow = st.lrnd = 0.0f;
    st.mrow = m;
    for (int c = 0; c < nch; ++c) {
        const float* __restrict__ P = sv.partials + (slot0 + static_cast<int64_t>(c) * nt) * PF;
        const float mc = P[tl];
        const float a = mc == -INFINITY ? 0.0f : fast_exp2(mc - m);
        st.lrow = fmaf(a, P[tl + 128], st.lrow);
        st.lrnd = fmaf(a, P[tl + 256], st.lrnd);
        const float4* po = reinterpret_cast<const float4*>(P) + wave * DM * 4 * 64 + lane;
#pragma unroll
        for (int mm = 0; mm < DM; ++mm)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 x = po[(mm * 4 + g) * 64];
                st.oacc[mm][4 * g] = fmaf(a, x.x, st.oacc[mm][4 * g]);
                st.oacc[mm][4 * g + 1] = fmaf(a, x.y, st.oacc[mm][4 * g + 1]);
                st.oacc[mm][4 * g + 2] = fmaf(a, x.z, st.oacc[mm][4 * g + 2]);
                st.oacc[mm][4 * g + 3] = fmaf(a, x.w, st.oacc[mm][4 * g + 3]);
            }
    }
    fwd_store<D>(st, o, ores, lse, om, N, h, p0);
}

// ---------------------------------------------------------------- launchers

// Sibling tiles in one workgroup: off by default (PRISM_FWD_PAIRS=1 turns it
// on).  Measured at 2K: forward 58.3-58.9 ms with pairs against 57.3 ms
// without, outputs bit-identical; the shared loads do not pay for the
// four-wave barriers.
constexpr int kFwdPairs = 0;

hipError_t launch_attn_fwd_mfma(const void* q, const void* k, const void* v, void* o, float* lse, int64_t N, int heads,
                                int d, int64_t ld, int64_t hs, const int32_t* offs, int nb, const int32_t* so,
                                const int32_t* si, int64_t cap, const int32_t* order, const uint8_t* skip,
                                const RowMap& om, float scale, void* ores, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(N / 64 * heads));
    const float sl2 = scale * kLog2e;
    const uint16_t* Q = static_cast<const uint16_t*>(q);
    const uint16_t* K = static_cast<const uint16_t*>(k);
    const uint16_t* V = static_cast<const uint16_t*>(v);
    uint16_t* O = static_cast<uint16_t*>(o);
    uint16_t* R = static_cast<uint16_t*>(ores);
    const char* ev = std::getenv("PRISM_FWD_PAIRS");
    const int pairs = ev ? (ev[0] == '1') : kFwdPairs;
    if (d == 128)
        hipLaunchKernelGGL((attn_fwd_mfma_kernel<128, 2>), grid, dim3(128), 0, s, Q, K, V, O, lse, N, ld, hs, offs, nb,
                           so, si, cap, order, skip, om, sl2, R, pairs);
    else
        hipLaunchKernelGGL((attn_fwd_mfma_kernel<64, 2>), grid, dim3(128), 0, s, Q, K, V, O, lse, N, ld, hs, offs, nb,
                           so, si, cap, order, skip, om, sl2, R, pairs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !pairs) return e;
    if (d == 128)
        hipLaunchKernelGGL((attn_fwd_mfma_kernel<128, 4>), grid, dim3(256), 0, s, Q, K, V, O, lse, N, ld, hs, offs, nb,
                           so, si, cap, order, skip, om, sl2, R, pairs);
    else
        hipLaunchKernelGGL((attn_fwd_mfma_kernel<64, 4>), grid, dim3(256), 0, s, Q, K, V, O, lse, N, ld, hs, offs, nb,
                           so, si, cap, order, skip, om, sl2, R, pairs);
    return hipGetLastError();
}

hipError_t launch_attn_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, int64_t N,
                                 int heads, int d, int64_t ld, int64_t hs, const int32_t* offs, int nb,
                                 const int32_t* si, int64_t cap, const SplitView& sv, const RowMap& om, float scale,
                                 void* ores, hipStream_t s) {
    const float sl2 = scale * kLog2e;
    const uint16_t* Q = static_cast<const uint16_t*>(q);
    const uint16_t* K = static_cast<const uint16_t*>(k);
    const uint16_t* V = static_cast<const uint16_t*>(v);
    uint16_t* O = static_cast<uint16_t*>(o);
    uint16_t* R = static_cast<uint16_t*>(ores);
    const dim3 cgrid(static_cast<unsigned>(split_grid(sv)));
    const dim3 tgrid(static_cast<unsigned>(N / 64 * heads));
    if (d == 128) {
        hipLaunchKernelGGL(attn_fwd_chunk_kernel<128>, cgrid, dim3(128), 0, s, Q, K, V, N, ld, hs, offs, si, cap, sv,
                           sl2);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(attn_fwd_combine_kernel<128>, tgrid, dim3(128), 0, s, O, lse, R, N, offs, nb, sv, om);
    } else {
        hipLaunchKernelGGL(attn_fwd_chunk_kernel<64>, cgrid, dim3(128), 0, s, Q, K, V, N, ld, hs, offs, si, cap, sv,
                           sl2);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(attn_fwd_combine_kernel<64>, tgrid, dim3(128), 0, s, O, lse, R, N, offs, nb, sv, om);
    }
    return hipGetLastError();
}

}  // namespace prism

// zone_kernels.hip - macro-zone statistics, variation indicator, block volume,
// block shape and block layout (Prism reading guide, xyznot.com paper
// 2610.05416: "Các ý tưởng cốt lõi" for the 8x8x8 zones and the 16 shapes,
// "Phương pháp" §1 for the directional variance and the indicator, §2 for the
// volume thresholds and the log2 optimum).
//
// Three kernels:
//   zone_profile_dma_kernel  one workgroup per (zone, 1 KB channel slab: 512
//                        bf16 or 256 fp32 channels).  The slab of each token row
//                        is loaded straight into LDS (16 bytes per lane, fully
//                        coalesced, double-buffered chunks of 16 tokens); each
//                        thread then owns two (bf16) or one (fp32) channels,
//                        accumulates the 24 axis-slice sums of its channels
//                        over the zone's 512 tokens in float64 (exact for bf16
//                        input), turns them into the per-axis variance of the
//                        slice means, and the workgroup sums those over its
//                        channels in a fixed order.  zone_profile_kernel does
//                        the same with direct 4-byte loads, for layouts the
//                        16-byte loads cannot serve.
//   zone_reduce_kernel   one workgroup per zone: sums the slab partials in slab
//                        order, and builds the audio terms from the 512 values
//                        of the norm map.
//   zone_decide_kernel   one workgroup for the grid: global maximum of S_v,
//                        density, volume, indicator, optimum, nearest shape,
//                        then a scan over zones, in their block-major order,
//                        for the block offsets.
#include "prism_device.hpp"
#include "prism_internal.hpp"

// Float contraction is off in this file: the decisions are taken in float64
// with every product and sum rounded separately, as written.
#pragma clang fp contract(off)

namespace prism {

constexpr int kProfThreads = 256;
constexpr int kProfChannels = 2;                   // per thread
constexpr int kSlab = kProfThreads * kProfChannels;  // channels per workgroup

template <typename TIn, int CPT>
__device__ __forceinline__ void load_channels(const TIn* __restrict__ p, double (&x)[CPT], bool ok0, bool ok1);

template <>
__device__ __forceinline__ void load_channels<uint16_t, 2>(const uint16_t* __restrict__ p, double (&x)[2], bool ok0,
                                                           bool ok1) {
    if (ok1) {
        const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
        x[0] = static_cast<double>(bf16_to_f32(static_cast<uint16_t>(u & 0xFFFFu)));
        x[1] = static_cast<double>(bf16_to_f32(static_cast<uint16_t>(u >> 16)));
    } else {
        x[0] = ok0 ? static_cast<double>(bf16_to_f32(p[0])) : 0.0;
        x[1] = 0.0;
    }
}
template <>
__device__ __forceinline__ void load_channels<float, 2>(const float* __restrict__ p, double (&x)[2], bool ok0,
                                                        bool ok1) {
    if (ok1) {
        const float2 u = *reinterpret_cast<const float2*>(p);
        x[0] = static_cast<double>(u.x);
        x[1] = static_cast<double>(u.y);
    } else {
        x[0] = ok0 ? static_cast<double>(p[0]) : 0.0;
        x[1] = 0.0;
    }
}

// partial[(zone * nslab + slab) * 3 + d] = sum over this slab's channels of
// (1/8) sum_i (slice_mean_{d,i} - mean_i slice_mean_{d,i})^2
template <typename TIn>
__global__ void __launch_bounds__(kProfThreads)
zone_profile_kernel(const TIn* __restrict__ v, int64_t C, int64_t ld, ZoneGrid g, int nslab,
                    double* __restrict__ partial, int vec_ok) {
    __shared__ double red[kProfThreads / kWave];
    const int zone = blockIdx.x;
    const int slab = blockIdx.y;
    const int zt = zone / (g.nH * g.nW);
    const int zh = (zone / g.nW) % g.nH;
    const int zw = zone % g.nW;
    const int64_t c0 = static_cast<int64_t>(slab) * kSlab + 2 * threadIdx.x;
    const bool ok0 = c0 < C;
    const bool ok1 = vec_ok && (c0 + 1 < C);
    const bool ok1s = (c0 + 1 < C);

    double sT[8][2], sH[8][2], sW[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int c = 0; c < 2; ++c) sT[i][c] = sH[i][c] = sW[i][c] = 0.0;

    if (ok0) {
        const int64_t base = ((static_cast<int64_t>(zt) * 8 * g.H + zh * 8) * g.W + zw * 8);
        // rolled loops; the slice sums are picked by comparison, not by a
        // runtime index (which would put them in scratch memory)
#pragma unroll 1
        for (int it = 0; it < 8; ++it) {
#pragma unroll 1
            for (int ih = 0; ih < 8; ++ih) {
                const TIn* row = v + (base + (static_cast<int64_t>(it) * g.H + ih) * g.W) * ld + c0;
                double x[8][2];
#pragma unroll
                for (int iw = 0; iw < 8; ++iw) {
                    if (ok1) {
                        load_channels<TIn, 2>(row + iw * ld, x[iw], true, true);
                    } else {
                        // odd channel count or unaligned rows: two scalar loads
                        double y[2];
                        load_channels<TIn, 2>(row + iw * ld, y, true, false);
                        x[iw][0] = y[0];
                        if (ok1s) {
                            load_channels<TIn, 2>(row + iw * ld + 1, y, true, false);
                            x[iw][1] = y[0];
                        } else {
                            x[iw][1] = 0.0;
                        }
                    }
                }
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    double rs = 0.0;
#pragma unroll
                    for (int iw = 0; iw < 8; ++iw) {
                        sW[iw][c] += x[iw][c];
                        rs += x[iw][c];
                    }
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        if (i == it) sT[i][c] += rs;
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        if (i == ih) sH[i][c] += rs;
                }
            }
        }
    }
    // per channel and axis: variance of the 8 slice means (each slice = 64 tokens)
    double var[3] = {0.0, 0.0, 0.0};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const bool live = (c == 0) ? ok0 : ok1s;
        if (!live) continue;
#pragma unroll
        for (int d = 0; d < 3; ++d) {
            double m[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) m[i] = (d == 0 ? sT[i][c] : d == 1 ? sH[i][c] : sW[i][c]) / 64.0;
            double mu = 0.0;
#pragma unroll
            for (int i = 0; i < 8; ++i) mu += m[i];
            mu /= 8.0;
            double s = 0.0;
#pragma unroll
            for (int i = 0; i < 8; ++i) s += (m[i] - mu) * (m[i] - mu);
            var[d] += s / 8.0;
        }
    }
#pragma unroll
    for (int d = 0; d < 3; ++d) {
        const double t = block_sum(var[d], red);
        if (threadIdx.x == 0) partial[(static_cast<int64_t>(zone) * nslab + slab) * 3 + d] = t;
    }
}

// Same result as zone_profile_kernel, with the slab staged through LDS.
// Requires: C and ld multiples of 16 bytes' worth of elements, v 16-byte aligned.
template <typename TIn>
__global__ void __launch_bounds__(kProfThreads)
zone_profile_dma_kernel(const TIn* __restrict__ v, int64_t C, int64_t ld, ZoneGrid g, int nslab,
                        double* __restrict__ partial) {
    constexpr int CH = 1024 / static_cast<int>(sizeof(TIn));   // channels per slab
    constexpr int CPT = CH / kProfThreads;                      // channels per thread
    constexpr int CHUNK = 16;                                   // tokens per staged chunk
    constexpr int NCHUNK = kZoneTokens / CHUNK;
    __shared__ __attribute__((aligned(16))) uint8_t buf[2][CHUNK * 1024];
    __shared__ double red[kProfThreads / kWave];
    const int zone = blockIdx.x;
    const int slab = blockIdx.y;
    const int zt = zone / (g.nH * g.nW);
    const int zh = (zone / g.nW) % g.nH;
    const int zw = zone % g.nW;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t zbase = (static_cast<int64_t>(zt) * 8 * g.H + zh * 8) * g.W + zw * 8;
    const TIn* __restrict__ vs = v + static_cast<int64_t>(slab) * CH;
    // lane l loads bytes 16 l .. 16 l + 15 of the slab; lanes past C load the
    // slab's first 16 bytes again (always inside the row) and are ignored
    const bool lane_ok = static_cast<int64_t>(slab) * CH + (16 / static_cast<int>(sizeof(TIn))) * lane < C;
    const uint32_t loff = lane_ok ? 16u * lane : 0u;
    // chunk k covers T-slice it = k / 4 and H-rows ih0, ih0 + 1 with ih0 = 2 (k % 4);
    // wave w loads its tokens 4 w .. 4 w + 3 (token j: ih = ih0 + j / 8, iw = j % 8)
    auto issue = [&](int k, int b) {
        const int it = k >> 2, ih0 = (k & 3) * 2;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = 4 * wave + u;
            const int64_t tok = zbase + (static_cast<int64_t>(it) * g.H + ih0 + (j >> 3)) * g.W + (j & 7);
            dma16(vs + tok * ld, loff, lds_addr(buf[b] + j * 1024));
        }
    };
    const int64_t c0 = static_cast<int64_t>(slab) * CH + CPT * threadIdx.x;

    double sT[8][CPT], sH[8][CPT], sW[8][CPT];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int c = 0; c < CPT; ++c) sT[i][c] = sH[i][c] = sW[i][c] = 0.0;

    issue(0, 0);
    dma_join();
    for (int k = 0; k < NCHUNK; ++k) {
        const int b = k & 1;
        if (k + 1 < NCHUNK) issue(k + 1, b ^ 1);
        const int it = k >> 2, ih0 = (k & 3) * 2;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int ih = ih0 + r;
            double x[8][CPT];
#pragma unroll
            for (int iw = 0; iw < 8; ++iw) {
                const uint8_t* p = buf[b] + (8 * r + iw) * 1024 + CPT * sizeof(TIn) * threadIdx.x;
                if constexpr (CPT == 2) {
                    const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
                    x[iw][0] = static_cast<double>(bf16_to_f32(static_cast<uint16_t>(u & 0xFFFFu)));
                    x[iw][1] = static_cast<double>(bf16_to_f32(static_cast<uint16_t>(u >> 16)));
                } else {
                    x[iw][0] = static_cast<double>(*reinterpret_cast<const float*>(p));
                }
            }
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                double rs = 0.0;
#pragma unroll
                for (int iw = 0; iw < 8; ++iw) {
                    sW[iw][c] += x[iw][c];
                    rs += x[iw][c];
                }
                for (int i = 0; i < 8; ++i)
                    if (i == it) sT[i][c] += rs;
                for (int i = 0; i < 8; ++i)
                    if (i == ih) sH[i][c] += rs;
            }
        }
        dma_join();
    }
    double var[3] = {0.0, 0.0, 0.0};
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        if (c0 + c >= C) continue;
#pragma unroll
        for (int d = 0; d < 3; ++d) {
            double m[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) m[i] = (d == 0 ? sT[i][c] : d == 1 ? sH[i][c] : sW[i][c]) / 64.0;
            double mu = 0.0;
#pragma unroll
            for (int i = 0; i < 8; ++i) mu += m[i];
            mu /= 8.0;
            double s2 = 0.0;
#pragma unroll
            for (int i = 0; i < 8; ++i) s2 += (m[i] - mu) * (m[i] - mu);
            var[d] += s2 / 8.0;
        }
    }
#pragma unroll
    for (int d = 0; d < 3; ++d) {
        const double t = block_sum(var[d], red);
        if (threadIdx.x == 0) partial[(static_cast<int64_t>(zone) * nslab + slab) * 3 + d] = t;
    }
}

// rec[zone*16 + ...] per the PRISM_ZS_* layout, except rho and B (decide kernel)
__global__ void __launch_bounds__(64)
zone_reduce_kernel(const double* __restrict__ partial, int nslab, int64_t C, const float* __restrict__ a,
                   ZoneGrid g, double* __restrict__ rec) {
    __shared__ double av[512];
    __shared__ double slice[3][8];
    const int zone = blockIdx.x;
    const int zt = zone / (g.nH * g.nW);
    const int zh = (zone / g.nW) % g.nH;
    const int zw = zone % g.nW;
    // thread t loads the 8 w-values of row (it, ih) = (t / 8, t % 8)
    {
        const int it = threadIdx.x >> 3, ih = threadIdx.x & 7;
        const int64_t n0 = ((static_cast<int64_t>(zt) * 8 + it) * g.H + zh * 8 + ih) * g.W + zw * 8;
#pragma unroll
        for (int iw = 0; iw < 8; ++iw) av[(it * 8 + ih) * 8 + iw] = static_cast<double>(a[n0 + iw]);
    }
    __syncthreads();
    if (threadIdx.x < 24) {
        const int d = threadIdx.x / 8, i = threadIdx.x % 8;
        double s = 0.0;
        for (int x = 0; x < 8; ++x)
            for (int y = 0; y < 8; ++y) {
                const int it = d == 0 ? i : x;
                const int ih = d == 1 ? i : (d == 0 ? x : y);
                const int iw = d == 2 ? i : y;
                s += av[(it * 8 + ih) * 8 + iw];
            }
        slice[d][i] = s / 64.0;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double* r = rec + static_cast<int64_t>(zone) * 16;
        // video: sum the slab partials in slab order, then the channel mean
        double s2v[3];
        for (int d = 0; d < 3; ++d) {
            double t = 0.0;
            for (int s = 0; s < nslab; ++s) t += partial[(static_cast<int64_t>(zone) * nslab + s) * 3 + d];
            s2v[d] = t / static_cast<double>(C);
        }
        const double sv = (s2v[0] + s2v[1]) + s2v[2];
        for (int d = 0; d < 3; ++d) {
            r[0 + d] = s2v[d];
            r[3 + d] = sv > 0.0 ? s2v[d] / sv : 1.0 / 3.0;
        }
        // audio: zone mean, and the variance of each axis' slice means
        double s2a[3];
        double abar = 0.0;
        for (int d = 0; d < 3; ++d) {
            double mu = 0.0;
            for (int i = 0; i < 8; ++i) mu += slice[d][i];
            mu /= 8.0;
            if (d == 0) abar = mu;
            double s = 0.0;
            for (int i = 0; i < 8; ++i) s += (slice[d][i] - mu) * (slice[d][i] - mu);
            s2a[d] = s / 8.0;
        }
        const double sa = (s2a[0] + s2a[1]) + s2a[2];
        r[6] = abar;
        for (int d = 0; d < 3; ++d) {
            r[7 + d] = s2a[d];
            r[10 + d] = sa > 0.0 ? s2a[d] / sa : 1.0 / 3.0;
        }
        r[14] = sv;
    }
}

__global__ void __launch_bounds__(1024)
zone_decide_kernel(double* __restrict__ rec, int nZ, double tau128, double tau256, double eps,
                   const int32_t* __restrict__ order, uint8_t* __restrict__ zone_shape,
                   int32_t* __restrict__ block_offsets, int32_t* __restrict__ nb_dev) {
    __shared__ double redd[16];
    __shared__ int32_t scan[1024];
    __shared__ int32_t carry;
    // global maximum of S_v
    double mx = 0.0;
    for (int m = threadIdx.x; m < nZ; m += blockDim.x) {
        const double s = rec[static_cast<int64_t>(m) * 16 + 14];
        mx = s > mx ? s : mx;
    }
    mx = block_max(mx, redd);
    if (threadIdx.x == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < nZ; base += blockDim.x) {
        const int m = base + threadIdx.x;
        if (m < nZ) {
            double* r = rec + static_cast<int64_t>(m) * 16;
            const double abar = r[6];
            const double shat = mx > 0.0 ? r[14] / mx : 0.0;
            const double rho = shat > abar ? shat : abar;
            const int B = rho < tau256 ? 256 : (rho < tau128 ? 128 : 64);
            double lg[3];
            for (int d = 0; d < 3; ++d) lg[d] = log2(r[3 + d] + abar * r[10 + d] + eps);
            const double S = log2(static_cast<double>(B));
            const double common = (S + 0.5 * ((lg[0] + lg[1]) + lg[2])) / 3.0;
            double ls[3];
            for (int d = 0; d < 3; ++d) ls[d] = -0.5 * lg[d] + common;
            // nearest candidate of volume B; ties within 1e-9 -> lowest index
            double D[16];
            double dmin = 1e300;
            for (int c = 0; c < 16; ++c) {
                int bt, bh, bw;
                shape_of(c, bt, bh, bw);
                if (bt * bh * bw != B) { D[c] = 1e300; continue; }
                const double e0 = log2(static_cast<double>(bt)) - ls[0];
                const double e1 = log2(static_cast<double>(bh)) - ls[1];
                const double e2 = log2(static_cast<double>(bw)) - ls[2];
                D[c] = ((0.0 + e0 * e0) + e1 * e1) + e2 * e2;
                dmin = D[c] < dmin ? D[c] : dmin;
            }
            int pick = 0;
            for (int c = 15; c >= 0; --c)
                if (D[c] <= dmin + 1e-9) pick = c;
            zone_shape[m] = static_cast<uint8_t>(pick);
            r[13] = rho;
            r[15] = static_cast<double>(B);
        }
    }
    __syncthreads();   // every zone's volume is in rec[15]
    // block offsets: an inclusive scan of block counts over the zones in their
    // block-major order (order[pos], or raster when order is NULL)
    for (int base = 0; base < nZ; base += blockDim.x) {
        const int pos = base + threadIdx.x;
        const int m = pos < nZ ? (order ? order[pos] : pos) : 0;
        const int nblk = pos < nZ ? kZoneTokens / static_cast<int>(rec[static_cast<int64_t>(m) * 16 + 15]) : 0;
        scan[threadIdx.x] = nblk;
        __syncthreads();
        for (int off = 1; off < static_cast<int>(blockDim.x); off <<= 1) {
            const int t = threadIdx.x >= off ? scan[threadIdx.x - off] : 0;
            __syncthreads();
            scan[threadIdx.x] += t;
            __syncthreads();
        }
        const int first = carry + scan[threadIdx.x] - nblk;
        if (pos < nZ) {
            const int B = kZoneTokens / nblk;
            for (int j = 0; j < nblk; ++j) block_offsets[first + j] = pos * kZoneTokens + j * B;
        }
        __syncthreads();
        if (threadIdx.x == blockDim.x - 1) carry += scan[threadIdx.x];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        block_offsets[carry] = nZ * kZoneTokens;
        *nb_dev = carry;
    }
}

hipError_t launch_zone_shapes(const void* v, bool bf16, int64_t C, int64_t ld, const float* a, ZoneGrid g, int nZ,
                              double tau128, double tau256, double eps, uint8_t* zone_shape, int32_t* block_offsets,
                              int32_t* nb_dev, double* partial, double* rec, hipStream_t s) {
    const uintptr_t va = reinterpret_cast<uintptr_t>(v);
    const int64_t vec = bf16 ? 8 : 4;   // elements per 16 bytes
    const bool dma_ok = (C % vec) == 0 && (ld % vec) == 0 && (va & 15) == 0;
    int nslab;
    if (dma_ok) {
        const int64_t ch = bf16 ? 512 : 256;
        nslab = static_cast<int>((C + ch - 1) / ch);
        const dim3 grid(nZ, nslab);
        if (bf16)
            hipLaunchKernelGGL(zone_profile_dma_kernel<uint16_t>, grid, dim3(kProfThreads), 0, s,
                               static_cast<const uint16_t*>(v), C, ld, g, nslab, partial);
        else
            hipLaunchKernelGGL(zone_profile_dma_kernel<float>, grid, dim3(kProfThreads), 0, s,
                               static_cast<const float*>(v), C, ld, g, nslab, partial);
    } else {
        nslab = static_cast<int>((C + kSlab - 1) / kSlab);
        const dim3 grid(nZ, nslab);
        if (bf16) {
            const int vec_ok = ((C % 2) == 0) && ((ld % 2) == 0) && ((va & 3) == 0);
            hipLaunchKernelGGL(zone_profile_kernel<uint16_t>, grid, dim3(kProfThreads), 0, s,
                               static_cast<const uint16_t*>(v), C, ld, g, nslab, partial, vec_ok);
        } else {
            const int vec_ok = ((C % 2) == 0) && ((ld % 2) == 0) && ((va & 7) == 0);
            hipLaunchKernelGGL(zone_profile_kernel<float>, grid, dim3(kProfThreads), 0, s,
                               static_cast<const float*>(v), C, ld, g, nslab, partial, vec_ok);
        }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(zone_reduce_kernel, dim3(nZ), dim3(64), 0, s, partial, nslab, C, a, g, rec);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(zone_decide_kernel, dim3(1), dim3(1024), 0, s, rec, nZ, tau128, tau256, eps, g.order,
                       zone_shape, block_offsets, nb_dev);
    return hipGetLastError();
}

// enough for either slab size (256 fp32 channels is the smallest)
size_t zone_partial_doubles(int nZ, int64_t C) {
    return static_cast<size_t>(nZ) * static_cast<size_t>((C + 255) / 256) * 3;
}

}  // namespace prism

// attn_simt.hip - block-sparse attention on the vector ALUs (fp32 arithmetic).
//
// Exact attention over the selected key blocks only, with an online softmax
// (Prism reading guide, xyznot.com paper 2610.05416, "Phương pháp" §3), and
// its gradient (the chain rule of the masked softmax; the pages do not
// describe the backward).  This is the path for fp32 tensors; it also accepts
// bf16 tensors (computing in fp32), which the library uses when the MFMA
// kernels are disabled.
//
// One wave per 64-row tile: thread r owns one query row (forward, dQ) or one
// key row (dK/dV); the other side streams through LDS in chunks of 32 rows.
#include "prism_device.hpp"
#include "prism_internal.hpp"

namespace prism {

constexpr int kChunk = 32;

template <typename T>
__device__ __forceinline__ float ld_elem(const T* p);
template <>
__device__ __forceinline__ float ld_elem<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ld_elem<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }
template <typename T>
__device__ __forceinline__ void st_elem(T* p, float x);
template <>
__device__ __forceinline__ void st_elem<float>(float* p, float x) { *p = x; }
template <>
__device__ __forceinline__ void st_elem<uint16_t>(uint16_t* p, float x) { *p = f32_to_bf16(x); }

// index of the block holding token position p (offs ascending, offs[0] = 0)
__device__ __forceinline__ int block_of(const int32_t* __restrict__ offs, int nb, int64_t p) {
    int a = 0, b = nb;  // offs[a] <= p < offs[b]
    while (b - a > 1) {
        const int m = (a + b) >> 1;
        if (offs[m] <= p) a = m;
        else b = m;
    }
    return a;
}

template <typename T, int D>
__global__ void __launch_bounds__(64)
attn_fwd_simt_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, T* __restrict__ o,
                     float* __restrict__ lse, int64_t N, int64_t ld, int64_t hs, const int32_t* __restrict__ offs,
                     int nb, const int32_t* __restrict__ sel_off, const int32_t* __restrict__ sel_idx, int64_t cap,
                     const uint8_t* __restrict__ skip, const RowMap om, float scale, T* __restrict__ ores) {
    __shared__ float Ks[kChunk][D + 1];
    __shared__ float Vs[kChunk][D + 1];
    const int h = blockIdx.y;
    const int64_t p0 = static_cast<int64_t>(blockIdx.x) * 64;
    const int64_t p = p0 + threadIdx.x;
    const int i = block_of(offs, nb, p0);
    if (skip && skip[static_cast<int64_t>(h) * nb + i]) return;   // routed to another path
    const T* __restrict__ qh = q + h * hs;
    const T* __restrict__ kh = k + h * hs;
    const T* __restrict__ vh = v + h * hs;
    float qr[D], acc[D];
#pragma unroll
    for (int c = 0; c < D; ++c) {
        qr[c] = ld_elem(qh + p * ld + c) * scale;
        acc[c] = 0.0f;
    }
    float m = -INFINITY, l = 0.0f;
    const int32_t* __restrict__ so = sel_off + static_cast<int64_t>(h) * (nb + 1);
    const int32_t* __restrict__ si = sel_idx + static_cast<int64_t>(h) * cap;
    const int e1 = static_cast<int>(min(static_cast<int64_t>(so[i + 1]), cap));
    for (int e = so[i]; e < e1; ++e) {
        const int j = si[e];
        for (int t0 = offs[j]; t0 < offs[j + 1]; t0 += kChunk) {
            __syncthreads();
            for (int x = threadIdx.x; x < kChunk * D; x += 64) {
                const int r = x / D, c = x % D;
                Ks[r][c] = ld_elem(kh + static_cast<int64_t>(t0 + r) * ld + c);
                Vs[r][c] = ld_elem(vh + static_cast<int64_t>(t0 + r) * ld + c);
            }
            __syncthreads();
            float s[kChunk];
            float cm = -INFINITY;
#pragma unroll
            for (int r = 0; r < kChunk; ++r) {
                float a = 0.0f;
#pragma unroll
                for (int c = 0; c < D; ++c) a = fmaf(qr[c], Ks[r][c], a);
                s[r] = a;
                cm = fmaxf(cm, a);
            }
            const float mn = fmaxf(m, cm);
            const float corr = __expf(m - mn);
            l *= corr;
#pragma unroll
            for (int c = 0; c < D; ++c) acc[c] *= corr;
#pragma unroll
            for (int r = 0; r < kChunk; ++r) {
                const float pr = __expf(s[r] - mn);
                l += pr;
#pragma unroll
                for (int c = 0; c < D; ++c) acc[c] = fmaf(pr, Vs[r][c], acc[c]);
            }
            m = mn;
        }
    }
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;   // a row with no stored entry: O = 0, lse = -inf
    const int64_t ro = row_offset(om, p, h);
#pragma unroll
    for (int c = 0; c < D; ++c) {
        const float x = acc[c] * inv;
        st_elem(o + ro + c, x);
        if (ores) st_elem(ores + ro + c, x - ld_elem(o + ro + c));   // bf16 residual (NULL for fp32)
    }
    lse[static_cast<int64_t>(h) * N + p] = m + __logf(l);
}

// Dq[h][p] = sum_c dO[p,h,c] * O[p,h,c], and lse2[h][p] = lse[h][p] log2(e) (the
// base-2 form that the dK/dV kernel loads per tile).  LPR lanes share a row,
// each with 16 bytes of O and of dO (EPV elements); a workgroup covers 64 rows
// of one head.
template <typename T, int D>
__global__ void __launch_bounds__(256)
attn_bwd_dot_kernel(const T* __restrict__ o, const T* __restrict__ dout, int64_t N, int heads, int64_t ld, int64_t hs,
                    const RowMap om, float* __restrict__ Dq, const T* __restrict__ ores, const float* __restrict__ lse,
                    float* __restrict__ lse2) {
    constexpr int EPV = 16 / static_cast<int>(sizeof(T));
    constexpr int LPR = D / EPV;            // lanes per row (power of two, <= 64)
    constexpr int RPI = 256 / LPR;          // rows per workgroup step
    const int h = blockIdx.y;
    const int sub = threadIdx.x % LPR;
#pragma unroll
    for (int it = 0; it < 64 / RPI; ++it) {
        const int64_t p = static_cast<int64_t>(blockIdx.x) * 64 + it * RPI + threadIdx.x / LPR;
        float s = 0.0f;
        if (p < N) {
            const int64_t ro = row_offset(om, p, h) + sub * EPV;
            const uint4 a = *reinterpret_cast<const uint4*>(o + ro);
            const uint4 b = *reinterpret_cast<const uint4*>(dout + p * ld + h * hs + sub * EPV);
            uint4 c = make_uint4(0, 0, 0, 0);
            if (ores) c = *reinterpret_cast<const uint4*>(ores + ro);
            const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w}, wc[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (EPV == 8) {
                    // O = hi + residual: both halves enter the row dot
                    const float lo_o = bf16_to_f32(static_cast<uint16_t>(wa[e] & 0xFFFFu)) +
                                       bf16_to_f32(static_cast<uint16_t>(wc[e] & 0xFFFFu));
                    const float hi_o = bf16_to_f32(static_cast<uint16_t>(wa[e] >> 16)) +
                                       bf16_to_f32(static_cast<uint16_t>(wc[e] >> 16));
                    s = fmaf(bf16_to_f32(static_cast<uint16_t>(wb[e] & 0xFFFFu)), lo_o, s);
                    s = fmaf(bf16_to_f32(static_cast<uint16_t>(wb[e] >> 16)), hi_o, s);
                } else {
                    s = fmaf(__uint_as_float(wb[e]), __uint_as_float(wa[e]), s);
                }
            }
        }
#pragma unroll
        for (int off = LPR / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off, kWave);
        if (p < N && sub == 0) {
            Dq[static_cast<int64_t>(h) * N + p] = s;
            if (lse2) lse2[static_cast<int64_t>(h) * N + p] = lse[static_cast<int64_t>(h) * N + p] * kLog2e;
        }
    }
}

template <typename T, int D>
__global__ void __launch_bounds__(64)
attn_dq_simt_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                    const T* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ Dq,
                    T* __restrict__ dq, int64_t N, int64_t ld, int64_t hs, const int32_t* __restrict__ offs, int nb,
                    const int32_t* __restrict__ sel_off, const int32_t* __restrict__ sel_idx, int64_t cap,
                    const uint8_t* __restrict__ skip, const RowMap om, float scale) {
    __shared__ float Ks[kChunk][D + 1];
    __shared__ float Vs[kChunk][D + 1];
    const int h = blockIdx.y;
    const int64_t p0 = static_cast<int64_t>(blockIdx.x) * 64;
    const int64_t p = p0 + threadIdx.x;
    const int i = block_of(offs, nb, p0);
    if (skip && skip[static_cast<int64_t>(h) * nb + i]) return;   // routed to another path
    const T* __restrict__ kh = k + h * hs;
    const T* __restrict__ vh = v + h * hs;
    float qr[D], dor[D], acc[D];
#pragma unroll
    for (int c = 0; c < D; ++c) {
        qr[c] = ld_elem(q + p * ld + h * hs + c) * scale;
        dor[c] = ld_elem(dout + p * ld + h * hs + c);
        acc[c] = 0.0f;
    }
    const float L = lse[static_cast<int64_t>(h) * N + p];
    const float Dd = Dq[static_cast<int64_t>(h) * N + p];
    const int32_t* __restrict__ so = sel_off + static_cast<int64_t>(h) * (nb + 1);
    const int32_t* __restrict__ si = sel_idx + static_cast<int64_t>(h) * cap;
    const int e1 = static_cast<int>(min(static_cast<int64_t>(so[i + 1]), cap));
    for (int e = so[i]; e < e1; ++e) {
        const int j = si[e];
        for (int t0 = offs[j]; t0 < offs[j + 1]; t0 += kChunk) {
            __syncthreads();
            for (int x = threadIdx.x; x < kChunk * D; x += 64) {
                const int r = x / D, c = x % D;
                Ks[r][c] = ld_elem(kh + static_cast<int64_t>(t0 + r) * ld + c);
                Vs[r][c] = ld_elem(vh + static_cast<int64_t>(t0 + r) * ld + c);
            }
            __syncthreads();
#pragma unroll 4
            for (int r = 0; r < kChunk; ++r) {
                float s = 0.0f, dp = 0.0f;
#pragma unroll
                for (int c = 0; c < D; ++c) {
                    s = fmaf(qr[c], Ks[r][c], s);
                    dp = fmaf(dor[c], Vs[r][c], dp);
                }
                const float pr = __expf(s - L);
                const float ds = pr * (dp - Dd);
#pragma unroll
                for (int c = 0; c < D; ++c) acc[c] = fmaf(ds, Ks[r][c], acc[c]);
            }
        }
    }
    T* __restrict__ drow = dq + row_offset(om, p, h);
#pragma unroll
    for (int c = 0; c < D; ++c) st_elem(drow + c, acc[c] * scale);
}

template <typename T, int D>
__global__ void __launch_bounds__(64)
attn_dkdv_simt_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                      const T* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ Dq,
                      T* __restrict__ dk, T* __restrict__ dv, int64_t N, int64_t ld, int64_t hs,
                      const int32_t* __restrict__ offs, int nb, const int32_t* __restrict__ tr_off,
                      const int32_t* __restrict__ tr_idx, int64_t cap, const float* __restrict__ dkbar,
                      const float* __restrict__ dvbar, const RowMap om, float scale) {
    __shared__ float Qs[kChunk][D + 1];
    __shared__ float Os[kChunk][D + 1];
    __shared__ float Ls[kChunk], Ds[kChunk];
    const int h = blockIdx.y;
    const int64_t p0 = static_cast<int64_t>(blockIdx.x) * 64;
    const int64_t p = p0 + threadIdx.x;
    const int j = block_of(offs, nb, p0);
    const T* __restrict__ qh = q + h * hs;
    const T* __restrict__ oh = dout + h * hs;
    float kr[D], vr[D], ak[D], av[D];
#pragma unroll
    for (int c = 0; c < D; ++c) {
        kr[c] = ld_elem(k + p * ld + h * hs + c) * scale;
        vr[c] = ld_elem(v + p * ld + h * hs + c);
        ak[c] = 0.0f;
        av[c] = 0.0f;
    }
    const int32_t* __restrict__ to = tr_off + static_cast<int64_t>(h) * (nb + 1);
    const int32_t* __restrict__ ti = tr_idx + static_cast<int64_t>(h) * cap;
    const int e1 = static_cast<int>(min(static_cast<int64_t>(to[j + 1]), cap));
    for (int e = to[j]; e < e1; ++e) {
        const int i = ti[e];
        for (int t0 = offs[i]; t0 < offs[i + 1]; t0 += kChunk) {
            __syncthreads();
            for (int x = threadIdx.x; x < kChunk * D; x += 64) {
                const int r = x / D, c = x % D;
                Qs[r][c] = ld_elem(qh + static_cast<int64_t>(t0 + r) * ld + c);
                Os[r][c] = ld_elem(oh + static_cast<int64_t>(t0 + r) * ld + c);
            }
            if (threadIdx.x < kChunk) {
                Ls[threadIdx.x] = lse[static_cast<int64_t>(h) * N + t0 + threadIdx.x];
                Ds[threadIdx.x] = Dq[static_cast<int64_t>(h) * N + t0 + threadIdx.x];
            }
            __syncthreads();
#pragma unroll 4
            for (int r = 0; r < kChunk; ++r) {
                float s = 0.0f, dp = 0.0f;
#pragma unroll
                for (int c = 0; c < D; ++c) {
                    s = fmaf(kr[c], Qs[r][c], s);
                    dp = fmaf(vr[c], Os[r][c], dp);
                }
                const float pr = __expf(s - Ls[r]);
                const float ds = pr * (dp - Ds[r]);
#pragma unroll
                for (int c = 0; c < D; ++c) {
                    av[c] = fmaf(pr, Os[r][c], av[c]);
                    ak[c] = fmaf(ds, Qs[r][c], ak[c]);
                }
            }
        }
    }
    // routed backward: the block-mean gradients of this key block, shared by its B tokens
    const float invB = 1.0f / static_cast<float>(offs[j + 1] - offs[j]);
    const int64_t jb = (static_cast<int64_t>(h) * nb + j) * D;
    const int64_t orow = row_offset(om, p, h);
#pragma unroll
    for (int c = 0; c < D; ++c) {
        st_elem(dk + orow + c, ak[c] * scale + (dkbar ? dkbar[jb + c] * invB : 0.0f));
        st_elem(dv + orow + c, av[c] + (dvbar ? dvbar[jb + c] * invB : 0.0f));
    }
}

template <typename T, int D>
static hipError_t fwd_simt(const void* q, const void* k, const void* v, void* o, float* lse, int64_t N, int heads,
                           int64_t ld, int64_t hs, const int32_t* offs, int nb, const int32_t* so, const int32_t* si,
                           int64_t cap, const uint8_t* skip, const RowMap& om, float scale, void* ores, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(N / 64), heads);
    hipLaunchKernelGGL((attn_fwd_simt_kernel<T, D>), grid, dim3(64), 0, s, static_cast<const T*>(q),
                       static_cast<const T*>(k), static_cast<const T*>(v), static_cast<T*>(o), lse, N, ld, hs, offs, nb,
                       so, si, cap, skip, om, scale, static_cast<T*>(ores));
    return hipGetLastError();
}

hipError_t launch_attn_fwd_simt(const void* q, const void* k, const void* v, void* o, float* lse, bool bf16, int64_t N,
                                int heads, int d, int64_t ld, int64_t hs, const int32_t* offs, int nb,
                                const int32_t* so, const int32_t* si, int64_t cap, const uint8_t* skip,
                                const RowMap& om, float scale, void* ores, hipStream_t s) {
    if (bf16)
        return d == 128 ? fwd_simt<uint16_t, 128>(q, k, v, o, lse, N, heads, ld, hs, offs, nb, so, si, cap, skip, om, scale,
                                                  ores, s)
                        : fwd_simt<uint16_t, 64>(q, k, v, o, lse, N, heads, ld, hs, offs, nb, so, si, cap, skip, om, scale,
                                                 ores, s);
    return d == 128 ? fwd_simt<float, 128>(q, k, v, o, lse, N, heads, ld, hs, offs, nb, so, si, cap, skip, om, scale,
                                           nullptr, s)
                    : fwd_simt<float, 64>(q, k, v, o, lse, N, heads, ld, hs, offs, nb, so, si, cap, skip, om, scale,
                                          nullptr, s);
}

template <typename T, int D>
static hipError_t dot_launch(const void* o, const void* dout, int64_t N, int heads, int64_t ld, int64_t hs,
                             const RowMap& om, float* Dq, const void* ores, const float* lse, float* lse2,
                             hipStream_t s) {
    hipLaunchKernelGGL((attn_bwd_dot_kernel<T, D>), dim3(static_cast<unsigned>((N + 63) / 64), heads), dim3(256), 0, s,
                       static_cast<const T*>(o), static_cast<const T*>(dout), N, heads, ld, hs, om, Dq,
                       static_cast<const T*>(ores), lse, lse2);
    return hipGetLastError();
}

hipError_t launch_bwd_dot(const void* o, const void* dout, bool bf16, int64_t N, int heads, int d, int64_t ld,
                          int64_t hs, const RowMap& om, float* Dq, const void* ores, const float* lse, float* lse2,
                          hipStream_t s) {
    if (bf16)
        return d == 128 ? dot_launch<uint16_t, 128>(o, dout, N, heads, ld, hs, om, Dq, ores, lse, lse2, s)
                        : dot_launch<uint16_t, 64>(o, dout, N, heads, ld, hs, om, Dq, ores, lse, lse2, s);
    return d == 128 ? dot_launch<float, 128>(o, dout, N, heads, ld, hs, om, Dq, nullptr, lse, lse2, s)
                    : dot_launch<float, 64>(o, dout, N, heads, ld, hs, om, Dq, nullptr, lse, lse2, s);
}

template <typename T, int D>
static hipError_t bwd_simt(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                           const float* Dq, void* dq, void* dk, void* dv, int64_t N, int heads, int64_t ld,
                           int64_t hs, const int32_t* offs, int nb, const int32_t* so, const int32_t* si,
                           const int32_t* to, const int32_t* ti, int64_t cap, const RouteGrad* rg,
                           const RowMap& om, float scale, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(N / 64), heads);
    hipLaunchKernelGGL((attn_dq_simt_kernel<T, D>), grid, dim3(64), 0, s, static_cast<const T*>(q),
                       static_cast<const T*>(k), static_cast<const T*>(v), static_cast<const T*>(dout), lse, Dq,
                       static_cast<T*>(dq), N, ld, hs, offs, nb, so, si, cap, rg ? rg->skip_q : nullptr, om, scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_dkdv_simt_kernel<T, D>), grid, dim3(64), 0, s, static_cast<const T*>(q),
                       static_cast<const T*>(k), static_cast<const T*>(v), static_cast<const T*>(dout), lse, Dq,
                       static_cast<T*>(dk), static_cast<T*>(dv), N, ld, hs, offs, nb, to, ti, cap,
                       rg ? rg->dkbar : nullptr, rg ? rg->dvbar : nullptr, om, scale);
    return hipGetLastError();
}

hipError_t launch_attn_bwd_simt(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                                const float* Dq, void* dq, void* dk, void* dv, bool bf16, int64_t N, int heads, int d,
                                int64_t ld, int64_t hs, const int32_t* offs, int nb, const int32_t* so,
                                const int32_t* si, const int32_t* to, const int32_t* ti, int64_t cap,
                                const RouteGrad* rg, const RowMap& om, float scale, hipStream_t s) {
    if (bf16)
        return d == 128 ? bwd_simt<uint16_t, 128>(q, k, v, dout, lse, Dq, dq, dk, dv, N, heads, ld, hs, offs, nb, so,
                                                   si, to, ti, cap, rg, om, scale, s)
                        : bwd_simt<uint16_t, 64>(q, k, v, dout, lse, Dq, dq, dk, dv, N, heads, ld, hs, offs, nb, so, si,
                                                  to, ti, cap, rg, om, scale, s);
    return d == 128 ? bwd_simt<float, 128>(q, k, v, dout, lse, Dq, dq, dk, dv, N, heads, ld, hs, offs, nb, so, si, to,
                                            ti, cap, rg, om, scale, s)
                    : bwd_simt<float, 64>(q, k, v, dout, lse, Dq, dq, dk, dv, N, heads, ld, hs, offs, nb, so, si, to,
                                           ti, cap, rg, om, scale, s);
}

}  // namespace prism

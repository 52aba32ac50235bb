// flat.hip - sharpness routing and the block-mean ("flat") attention path
// ("In-Context Sparse Attention" article: grouped computation routes query
// blocks by the sharpness M_i of their softmax; flat blocks use a
// zeroth-order Taylor kernel over block-mean keys).
//
//   sharpness_kernel   M_i = variance of softmax(L[i, :]) over the NB key
//                      blocks, float64, two passes as written (max and sum of
//                      exp, then the squared deviations of the probabilities)
//   flat_rank_kernel   flat[i] = rank of (M_i, i) < n_flat
//   block_means_kernel K_bar, V_bar [heads, NB, d] fp32: float64 block sums
//                      divided by B, rounded once
//   attn_flat_kernel   for every 64-row tile of a flat block: per row q,
//                      O = sum_j B_j e^{s q.K_bar_j} V_bar_j / sum_j B_j e^{...}
//                      over the block's selected set, fp32 with an online
//                      softmax; four lanes per row, each owning d/4 channels,
//                      and the selected blocks' means staged through LDS
#include <algorithm>
#include <cmath>

#include "prism_device.hpp"
#include "prism_internal.hpp"

namespace prism {

namespace {

__device__ __forceinline__ float elem_in(const float* p) { return *p; }
__device__ __forceinline__ float elem_in(const uint16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ void elem_out(float* p, float x) { *p = x; }
__device__ __forceinline__ void elem_out(uint16_t* p, float x) { *p = f32_to_bf16(x); }

__device__ __forceinline__ int block_containing(const int32_t* __restrict__ offs, int nb, int64_t p) {
    int a = 0, b = nb;
    while (b - a > 1) {
        const int m = (a + b) >> 1;
        if (offs[m] <= p) a = m;
        else b = m;
    }
    return a;
}

// block-wide reductions over 256 threads, in a fixed order
__device__ __forceinline__ double block_sum256(double v, double* red) {
    red[threadIdx.x] = v;
    __syncthreads();
    for (int s = 128; s >= 1; s >>= 1) {
        if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
        __syncthreads();
    }
    const double r = red[0];
    __syncthreads();
    return r;
}

__device__ __forceinline__ float block_max256(float v, float* red) {
    red[threadIdx.x] = v;
    __syncthreads();
    for (int s = 128; s >= 1; s >>= 1) {
        if (threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
        __syncthreads();
    }
    const float r = red[0];
    __syncthreads();
    return r;
}

}  // namespace

// grid (NB, heads): one workgroup per row of pooled scores
__global__ void __launch_bounds__(256)
sharpness_kernel(const float* __restrict__ logits, int nb, double* __restrict__ M) {
    __shared__ double red[256];
    __shared__ float redf[256];
    const int i = blockIdx.x, h = blockIdx.y;
    const float* __restrict__ row = logits + (static_cast<int64_t>(h) * nb + i) * nb;
    float mx = -INFINITY;
    for (int j = threadIdx.x; j < nb; j += 256) mx = fmaxf(mx, row[j]);
    mx = block_max256(mx, redf);
    const double dmx = static_cast<double>(mx);
    double s1 = 0.0;
    for (int j = threadIdx.x; j < nb; j += 256) s1 += exp(static_cast<double>(row[j]) - dmx);
    s1 = block_sum256(s1, red);
    const double u = 1.0 / static_cast<double>(nb);
    double s2 = 0.0;
    for (int j = threadIdx.x; j < nb; j += 256) {
        const double dv = exp(static_cast<double>(row[j]) - dmx) / s1 - u;
        s2 += dv * dv;
    }
    s2 = block_sum256(s2, red);
    if (threadIdx.x == 0) M[static_cast<int64_t>(h) * nb + i] = s2 / static_cast<double>(nb);
}

// grid (ceil(NB / 256), heads): rank of (M_i, i) among the head's rows
__global__ void __launch_bounds__(256)
flat_rank_kernel(const double* __restrict__ M, int nb, int n_flat, uint8_t* __restrict__ flat) {
    __shared__ double chunk[256];
    const int h = blockIdx.y;
    const int i = blockIdx.x * 256 + threadIdx.x;
    const double* __restrict__ Mh = M + static_cast<int64_t>(h) * nb;
    const double mi = i < nb ? Mh[i] : 0.0;
    int rank = 0;
    for (int base = 0; base < nb; base += 256) {
        chunk[threadIdx.x] = base + threadIdx.x < nb ? Mh[base + threadIdx.x] : 0.0;
        __syncthreads();
        const int lim = min(256, nb - base);
        for (int t = 0; t < lim; ++t) {
            const double mj = chunk[t];
            rank += (mj < mi) || (mj == mi && base + t < i);
        }
        __syncthreads();
    }
    if (i < nb) flat[static_cast<int64_t>(h) * nb + i] = rank < n_flat ? 1 : 0;
}

// grid (NB, heads): block means of K and V, float64 sums, fp32 results
template <typename T>
__global__ void __launch_bounds__(256)
block_means_kernel(const T* __restrict__ k, const T* __restrict__ v, int d, int64_t ld, int64_t hs,
                   const int32_t* __restrict__ offs, int nb, float* __restrict__ kbar, float* __restrict__ vbar) {
    __shared__ double part[2][256];
    const int j = blockIdx.x, h = blockIdx.y;
    const int rs = 256 / d;                       // row slots
    const int c = threadIdx.x % d, slot = threadIdx.x / d;
    const int64_t t0 = offs[j], t1 = offs[j + 1];
    double sk = 0.0, sv = 0.0;
    if (slot < rs)
        for (int64_t t = t0 + slot; t < t1; t += rs) {
            sk += static_cast<double>(elem_in(k + t * ld + h * hs + c));
            sv += static_cast<double>(elem_in(v + t * ld + h * hs + c));
        }
    part[0][threadIdx.x] = sk;
    part[1][threadIdx.x] = sv;
    __syncthreads();
    if (threadIdx.x < d) {
        double a = 0.0, b = 0.0;
        for (int r = 0; r < rs; ++r) {
            a += part[0][r * d + c];
            b += part[1][r * d + c];
        }
        const double B = static_cast<double>(t1 - t0);
        const int64_t o = (static_cast<int64_t>(h) * nb + j) * d + c;
        kbar[o] = static_cast<float>(a / B);
        vbar[o] = static_cast<float>(b / B);
    }
}

// grid (N/64 * heads): one workgroup of 256 threads per 64-row tile
template <typename T, int D>
__global__ void __launch_bounds__(256)
attn_flat_kernel(const T* __restrict__ q, const float* __restrict__ kbar, const float* __restrict__ vbar,
                 T* __restrict__ o, float* __restrict__ lse, int64_t N, int64_t ld, int64_t hs,
                 const int32_t* __restrict__ offs, int nb, const int32_t* __restrict__ sel_off,
                 const int32_t* __restrict__ sel_idx, int64_t cap, const uint8_t* __restrict__ flat, float scale,
                 T* __restrict__ ores) {
    constexpr int PW = D / 4;          // channels per lane
    constexpr int PS = PW + 4;         // padded LDS stride of a lane's slice
    constexpr int CH = 16;             // selected blocks staged per round
    __shared__ float Ks[CH][4][PS], Vs[CH][4][PS];
    __shared__ float lb[CH];
    const int ntiles = static_cast<int>(N / 64);
    const int h = blockIdx.x / ntiles;
    const int64_t p0 = static_cast<int64_t>(blockIdx.x % ntiles) * 64;
    const int i = block_containing(offs, nb, p0);
    if (!flat[static_cast<int64_t>(h) * nb + i]) return;
    const int r = threadIdx.x >> 2, part = threadIdx.x & 3;
    const int64_t p = p0 + r;
    float qr[PW], acc[PW];
    const T* __restrict__ qrow = q + p * ld + h * hs + part * PW;
#pragma unroll
    for (int c = 0; c < PW; ++c) {
        qr[c] = elem_in(qrow + c);
        acc[c] = 0.0f;
    }
    float m = -INFINITY, l = 0.0f;
    const int32_t* __restrict__ so = sel_off + static_cast<int64_t>(h) * (nb + 1);
    const int32_t* __restrict__ si = sel_idx + static_cast<int64_t>(h) * cap;
    const int e0 = so[i];
    const int e1 = static_cast<int>(min(static_cast<int64_t>(so[i + 1]), cap));
    const float* __restrict__ kh = kbar + static_cast<int64_t>(h) * nb * D;
    const float* __restrict__ vh = vbar + static_cast<int64_t>(h) * nb * D;
    for (int e = e0; e < e1; e += CH) {
        const int n = min(CH, e1 - e);
        __syncthreads();
        for (int x = threadIdx.x; x < n * D; x += 256) {
            const int jj = x / D, c = x % D;
            const int64_t j = si[e + jj];
            Ks[jj][c / PW][c % PW] = kh[j * D + c];
            Vs[jj][c / PW][c % PW] = vh[j * D + c];
        }
        if (threadIdx.x < n) {
            const int j = si[e + threadIdx.x];
            lb[threadIdx.x] = logf(static_cast<float>(offs[j + 1] - offs[j]));
        }
        __syncthreads();
        for (int jj = 0; jj < n; ++jj) {
            float dot = 0.0f;
#pragma unroll
            for (int c = 0; c < PW; ++c) dot = fmaf(qr[c], Ks[jj][part][c], dot);
            dot += __shfl_xor(dot, 1, 64);
            dot += __shfl_xor(dot, 2, 64);
            const float s = fmaf(dot, scale, lb[jj]);
            if (s > m) {
                const float a = expf(m - s);
                l *= a;
#pragma unroll
                for (int c = 0; c < PW; ++c) acc[c] *= a;
                m = s;
            }
            const float pj = expf(s - m);
            l += pj;
#pragma unroll
            for (int c = 0; c < PW; ++c) acc[c] = fmaf(pj, Vs[jj][part][c], acc[c]);
        }
    }
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;   // a row with no stored entry: O = 0, lse = -inf
    T* __restrict__ orow = o + p * ld + h * hs + part * PW;
#pragma unroll
    for (int c = 0; c < PW; ++c) {
        elem_out(orow + c, acc[c] * inv);
        if (ores) elem_out(ores + (orow - o) + c, acc[c] * inv - elem_in(orow + c));   // bf16 residual
    }
    if (part == 0) lse[static_cast<int64_t>(h) * N + p] = m + logf(l);
}

// Backward of the flat path (the selection and routing held constant): for a
// flat query row q with forward weights w_j = B_j e^{s q.K_bar_j - lse_q},
// D_q = rowsum(dO * O) and dS_j = w_j (dO_q . V_bar_j - D_q):
//   dq = s sum_j dS_j K_bar_j                         (attn_flat_dq_kernel)
//   dK_bar_j = s sum_q dS_qj q,  dV_bar_j = sum_q w_qj dO_q   (flat_kgrad_kernel,
//   key-major over the flat query blocks that selected j, fixed order)
// and the dK/dV kernel adds dK_bar_j / B_j, dV_bar_j / B_j to every token of j.

template <typename T, int D>
__global__ void __launch_bounds__(256)
attn_flat_dq_kernel(const T* __restrict__ q, const T* __restrict__ dout, const float* __restrict__ kbar,
                    const float* __restrict__ vbar, const float* __restrict__ lse, const float* __restrict__ Dq,
                    T* __restrict__ dq, int64_t N, int64_t ld, int64_t hs, const int32_t* __restrict__ offs, int nb,
                    const int32_t* __restrict__ sel_off, const int32_t* __restrict__ sel_idx, int64_t cap,
                    const uint8_t* __restrict__ flat, float scale) {
    constexpr int PW = D / 4, PS = PW + 4, CH = 16;
    __shared__ float Ks[CH][4][PS], Vs[CH][4][PS];
    __shared__ float lb[CH];
    const int ntiles = static_cast<int>(N / 64);
    const int h = blockIdx.x / ntiles;
    const int64_t p0 = static_cast<int64_t>(blockIdx.x % ntiles) * 64;
    const int i = block_containing(offs, nb, p0);
    if (!flat[static_cast<int64_t>(h) * nb + i]) return;
    const int r = threadIdx.x >> 2, part = threadIdx.x & 3;
    const int64_t p = p0 + r;
    float qr[PW], dr[PW], acc[PW];
    const T* __restrict__ qrow = q + p * ld + h * hs + part * PW;
    const T* __restrict__ drow = dout + p * ld + h * hs + part * PW;
#pragma unroll
    for (int c = 0; c < PW; ++c) {
        qr[c] = elem_in(qrow + c);
        dr[c] = elem_in(drow + c);
        acc[c] = 0.0f;
    }
    const float L = lse[static_cast<int64_t>(h) * N + p];
    const float Dd = Dq[static_cast<int64_t>(h) * N + p];
    const int32_t* __restrict__ so = sel_off + static_cast<int64_t>(h) * (nb + 1);
    const int32_t* __restrict__ si = sel_idx + static_cast<int64_t>(h) * cap;
    const int e0 = so[i];
    const int e1 = static_cast<int>(min(static_cast<int64_t>(so[i + 1]), cap));
    const float* __restrict__ kh = kbar + static_cast<int64_t>(h) * nb * D;
    const float* __restrict__ vh = vbar + static_cast<int64_t>(h) * nb * D;
    for (int e = e0; e < e1; e += CH) {
        const int n = min(CH, e1 - e);
        __syncthreads();
        for (int x = threadIdx.x; x < n * D; x += 256) {
            const int jj = x / D, c = x % D;
            const int64_t j = si[e + jj];
            Ks[jj][c / PW][c % PW] = kh[j * D + c];
            Vs[jj][c / PW][c % PW] = vh[j * D + c];
        }
        if (threadIdx.x < n) {
            const int j = si[e + threadIdx.x];
            lb[threadIdx.x] = logf(static_cast<float>(offs[j + 1] - offs[j]));
        }
        __syncthreads();
        for (int jj = 0; jj < n; ++jj) {
            float d1 = 0.0f, d2 = 0.0f;
#pragma unroll
            for (int c = 0; c < PW; ++c) {
                d1 = fmaf(qr[c], Ks[jj][part][c], d1);
                d2 = fmaf(dr[c], Vs[jj][part][c], d2);
            }
            d1 += __shfl_xor(d1, 1, 64);
            d1 += __shfl_xor(d1, 2, 64);
            d2 += __shfl_xor(d2, 1, 64);
            d2 += __shfl_xor(d2, 2, 64);
            const float w = expf(fmaf(d1, scale, lb[jj]) - L);
            const float ds = w * (d2 - Dd);
#pragma unroll
            for (int c = 0; c < PW; ++c) acc[c] = fmaf(ds, Ks[jj][part][c], acc[c]);
        }
    }
    T* __restrict__ out = dq + p * ld + h * hs + part * PW;
#pragma unroll
    for (int c = 0; c < PW; ++c) elem_out(out + c, acc[c] * scale);
}

// grid (NB, heads): key block j against the rows of every flat query block
// that selected it (ascending), 64 row slots of 4 lanes, reduced over slots in
// slot order
template <typename T, int D>
__global__ void __launch_bounds__(256)
flat_kgrad_kernel(const T* __restrict__ q, const T* __restrict__ dout, const float* __restrict__ kbar,
                  const float* __restrict__ vbar, const float* __restrict__ lse, const float* __restrict__ Dq,
                  int64_t N, int64_t ld, int64_t hs, const int32_t* __restrict__ offs, int nb,
                  const int32_t* __restrict__ fto, const int32_t* __restrict__ fti, int64_t cap, float scale,
                  float* __restrict__ dkbar, float* __restrict__ dvbar) {
    constexpr int PW = D / 4;
    __shared__ float red[64][D];
    const int j = blockIdx.x, h = blockIdx.y;
    const int slot = threadIdx.x >> 2, part = threadIdx.x & 3;
    const int64_t jb = (static_cast<int64_t>(h) * nb + j) * D;
    float kb[PW], vb[PW], ka[PW], va[PW];
#pragma unroll
    for (int c = 0; c < PW; ++c) {
        kb[c] = kbar[jb + part * PW + c];
        vb[c] = vbar[jb + part * PW + c];
        ka[c] = va[c] = 0.0f;
    }
    const float lbj = logf(static_cast<float>(offs[j + 1] - offs[j]));
    const int32_t* __restrict__ to = fto + static_cast<int64_t>(h) * (nb + 1);
    const int32_t* __restrict__ ti = fti + static_cast<int64_t>(h) * cap;
    const int e0 = to[j];
    const int e1 = static_cast<int>(min(static_cast<int64_t>(to[j + 1]), cap));
    for (int e = e0; e < e1; ++e) {
        const int i = ti[e];
        // blocks hold a whole number of 64-token tiles: every slot has a row
        for (int64_t row = offs[i] + slot; row < offs[i + 1]; row += 64) {
            float qr[PW], dr[PW];
            const T* __restrict__ qrow = q + row * ld + h * hs + part * PW;
            const T* __restrict__ drow = dout + row * ld + h * hs + part * PW;
            float d1 = 0.0f, d2 = 0.0f;
#pragma unroll
            for (int c = 0; c < PW; ++c) {
                qr[c] = elem_in(qrow + c);
                dr[c] = elem_in(drow + c);
                d1 = fmaf(qr[c], kb[c], d1);
                d2 = fmaf(dr[c], vb[c], d2);
            }
            d1 += __shfl_xor(d1, 1, 64);
            d1 += __shfl_xor(d1, 2, 64);
            d2 += __shfl_xor(d2, 1, 64);
            d2 += __shfl_xor(d2, 2, 64);
            const float w = expf(fmaf(d1, scale, lbj) - lse[static_cast<int64_t>(h) * N + row]);
            const float ds = w * (d2 - Dq[static_cast<int64_t>(h) * N + row]);
#pragma unroll
            for (int c = 0; c < PW; ++c) {
                ka[c] = fmaf(ds, qr[c], ka[c]);
                va[c] = fmaf(w, dr[c], va[c]);
            }
        }
    }
#pragma unroll
    for (int c = 0; c < PW; ++c) red[slot][part * PW + c] = ka[c];
    __syncthreads();
    for (int c = threadIdx.x; c < D; c += 256) {
        float t = 0.0f;
        for (int s2 = 0; s2 < 64; ++s2) t += red[s2][c];
        dkbar[jb + c] = t * scale;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < PW; ++c) red[slot][part * PW + c] = va[c];
    __syncthreads();
    for (int c = threadIdx.x; c < D; c += 256) {
        float t = 0.0f;
        for (int s2 = 0; s2 < 64; ++s2) t += red[s2][c];
        dvbar[jb + c] = t;
    }
}

hipError_t launch_flat_dq(const void* q, const void* dout, const float* kbar, const float* vbar, const float* lse,
                          const float* Dq, void* dq, bool bf16, int64_t N, int heads, int d, int64_t ld, int64_t hs,
                          const int32_t* offs, int nb, const int32_t* so, const int32_t* si, int64_t cap,
                          const uint8_t* flat, float scale, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(N / 64 * heads));
#define PRISM_FLAT_DQ(T, DD)                                                                                        \
    hipLaunchKernelGGL((attn_flat_dq_kernel<T, DD>), grid, dim3(256), 0, s, static_cast<const T*>(q),              \
                       static_cast<const T*>(dout), kbar, vbar, lse, Dq, static_cast<T*>(dq), N, ld, hs, offs, nb, \
                       so, si, cap, flat, scale)
    if (bf16) {
        if (d == 128) PRISM_FLAT_DQ(uint16_t, 128);
        else PRISM_FLAT_DQ(uint16_t, 64);
    } else {
        if (d == 128) PRISM_FLAT_DQ(float, 128);
        else PRISM_FLAT_DQ(float, 64);
    }
#undef PRISM_FLAT_DQ
    return hipGetLastError();
}

hipError_t launch_flat_kgrad(const void* q, const void* dout, const float* kbar, const float* vbar, const float* lse,
                             const float* Dq, bool bf16, int64_t N, int heads, int d, int64_t ld, int64_t hs,
                             const int32_t* offs, int nb, const int32_t* fto, const int32_t* fti, int64_t cap,
                             float scale, float* dkbar, float* dvbar, hipStream_t s) {
    const dim3 grid(nb, heads);
#define PRISM_FLAT_KG(T, DD)                                                                                       \
    hipLaunchKernelGGL((flat_kgrad_kernel<T, DD>), grid, dim3(256), 0, s, static_cast<const T*>(q),               \
                       static_cast<const T*>(dout), kbar, vbar, lse, Dq, N, ld, hs, offs, nb, fto, fti, cap, scale, \
                       dkbar, dvbar)
    if (bf16) {
        if (d == 128) PRISM_FLAT_KG(uint16_t, 128);
        else PRISM_FLAT_KG(uint16_t, 64);
    } else {
        if (d == 128) PRISM_FLAT_KG(float, 128);
        else PRISM_FLAT_KG(float, 64);
    }
#undef PRISM_FLAT_KG
    return hipGetLastError();
}

hipError_t launch_flat_route(const float* logits, int heads, int nb, int n_flat, double* sharpness, uint8_t* flat,
                             hipStream_t s) {
    hipLaunchKernelGGL(sharpness_kernel, dim3(nb, heads), dim3(256), 0, s, logits, nb, sharpness);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(flat_rank_kernel, dim3((nb + 255) / 256, heads), dim3(256), 0, s, sharpness, nb, n_flat, flat);
    return hipGetLastError();
}

hipError_t launch_block_means(const void* k, const void* v, bool bf16, int heads, int d, int64_t ld, int64_t hs,
                              const int32_t* offs, int nb, float* kbar, float* vbar, hipStream_t s) {
    if (bf16)
        hipLaunchKernelGGL(block_means_kernel<uint16_t>, dim3(nb, heads), dim3(256), 0, s,
                           static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), d, ld, hs, offs, nb, kbar,
                           vbar);
    else
        hipLaunchKernelGGL(block_means_kernel<float>, dim3(nb, heads), dim3(256), 0, s, static_cast<const float*>(k),
                           static_cast<const float*>(v), d, ld, hs, offs, nb, kbar, vbar);
    return hipGetLastError();
}

hipError_t launch_attn_flat(const void* q, const float* kbar, const float* vbar, void* o, float* lse, bool bf16,
                            int64_t N, int heads, int d, int64_t ld, int64_t hs, const int32_t* offs, int nb,
                            const int32_t* so, const int32_t* si, int64_t cap, const uint8_t* flat, float scale,
                            void* ores, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(N / 64 * heads));
    if (bf16) {
        const uint16_t* Q = static_cast<const uint16_t*>(q);
        uint16_t* O = static_cast<uint16_t*>(o);
        if (d == 128)
            hipLaunchKernelGGL((attn_flat_kernel<uint16_t, 128>), grid, dim3(256), 0, s, Q, kbar, vbar, O, lse, N, ld,
                               hs, offs, nb, so, si, cap, flat, scale, static_cast<uint16_t*>(ores));
        else
            hipLaunchKernelGGL((attn_flat_kernel<uint16_t, 64>), grid, dim3(256), 0, s, Q, kbar, vbar, O, lse, N, ld, hs,
                               offs, nb, so, si, cap, flat, scale, static_cast<uint16_t*>(ores));
    } else {
        const float* Q = static_cast<const float*>(q);
        float* O = static_cast<float*>(o);
        if (d == 128)
            hipLaunchKernelGGL((attn_flat_kernel<float, 128>), grid, dim3(256), 0, s, Q, kbar, vbar, O, lse, N, ld, hs,
                               offs, nb, so, si, cap, flat, scale, static_cast<float*>(nullptr));
        else
            hipLaunchKernelGGL((attn_flat_kernel<float, 64>), grid, dim3(256), 0, s, Q, kbar, vbar, O, lse, N, ld, hs,
                               offs, nb, so, si, cap, flat, scale, static_cast<float*>(nullptr));
    }
    return hipGetLastError();
}

}  // namespace prism

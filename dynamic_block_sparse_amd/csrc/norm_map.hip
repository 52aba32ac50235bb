// norm_map.hip - the audio-to-video norm map (Prism reading guide, "Phương
// pháp" §1: a at each token is the 2-norm of the audio-to-video cross-attention
// output cached from the layer before), divided by its clip-wide maximum so
// that it lies in [0, 1].
//
// Pass 1: one wave per token row at a time reads the row with 16-byte loads
// (4-byte loads for rows that are not 16-byte aligned) and sums the squares in
// float64: a bf16 or fp32 value squared is exact in float64, each lane sums its
// elements in order, the 64 lane sums are added in a fixed butterfly, and the
// square root is the correctly rounded float64 one.  Each workgroup records
// the largest norm it saw.
// Pass 2: every workgroup takes the maximum of those per-workgroup maxima and
// writes a = float(norm / max) for its rows (0 when every norm is 0).
#include <algorithm>

#include "prism_device.hpp"
#include "prism_internal.hpp"

namespace prism {

namespace {

template <typename TIn>
__device__ __forceinline__ double sq(TIn x);
template <>
__device__ __forceinline__ double sq<uint16_t>(uint16_t x) {
    const double v = static_cast<double>(bf16_to_f32(x));
    return v * v;
}
template <>
__device__ __forceinline__ double sq<float>(float x) {
    const double v = static_cast<double>(x);
    return v * v;
}

// sum of squares of the EPV elements held in a 16-byte word
template <typename TIn>
__device__ __forceinline__ double sq16(const uint4& w) {
    double s = 0.0;
    if constexpr (sizeof(TIn) == 2) {
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s += sq<uint16_t>(static_cast<uint16_t>(u[i] & 0xffffu));
            s += sq<uint16_t>(static_cast<uint16_t>(u[i] >> 16));
        }
    } else {
        s += sq<float>(__uint_as_float(w.x));
        s += sq<float>(__uint_as_float(w.y));
        s += sq<float>(__uint_as_float(w.z));
        s += sq<float>(__uint_as_float(w.w));
    }
    return s;
}

}  // namespace

template <typename TIn, bool VEC>
__global__ void __launch_bounds__(256)
norm_rows_kernel(const TIn* __restrict__ h, int64_t N, int64_t C, int64_t ld, double* __restrict__ norms,
                 double* __restrict__ block_max) {
    constexpr int EPV = 16 / static_cast<int>(sizeof(TIn));
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t nw = static_cast<int64_t>(gridDim.x) * 4;
    double mx = 0.0;
    for (int64_t n = static_cast<int64_t>(blockIdx.x) * 4 + wave; n < N; n += nw) {
        const TIn* __restrict__ row = h + n * ld;
        double acc = 0.0;
        int64_t c0 = 0;
        if constexpr (VEC) {
            const int64_t nv = C / EPV;
            const uint4* __restrict__ rv = reinterpret_cast<const uint4*>(row);
#pragma unroll 4
            for (int64_t j = lane; j < nv; j += 64) acc += sq16<TIn>(rv[j]);
            c0 = nv * EPV;
        }
        for (int64_t c = c0 + lane; c < C; c += 64) acc += sq<TIn>(row[c]);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
        const double nr = sqrt(acc);
        if (lane == 0) norms[n] = nr;
        mx = fmax(mx, nr);
    }
    __shared__ double wm[4];
    if (lane == 0) wm[wave] = mx;
    __syncthreads();
    if (threadIdx.x == 0) block_max[blockIdx.x] = fmax(fmax(wm[0], wm[1]), fmax(wm[2], wm[3]));
}

__global__ void __launch_bounds__(256)
norm_scale_kernel(const double* __restrict__ norms, const double* __restrict__ block_max, int nblk, int64_t N,
                  float* __restrict__ a) {
    __shared__ double red[256];
    double m = 0.0;
    for (int i = threadIdx.x; i < nblk; i += 256) m = fmax(m, block_max[i]);
    red[threadIdx.x] = m;
    __syncthreads();
    for (int s = 128; s >= 1; s >>= 1) {
        if (threadIdx.x < s) red[threadIdx.x] = fmax(red[threadIdx.x], red[threadIdx.x + s]);
        __syncthreads();
    }
    const double top = red[0];
    for (int64_t n = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; n < N;
         n += static_cast<int64_t>(gridDim.x) * 256)
        a[n] = top > 0.0 ? static_cast<float>(norms[n] / top) : 0.0f;
}

int norm_map_blocks(int64_t N) { return static_cast<int>(std::min<int64_t>((N + 3) / 4, kNormMapMaxBlocks)); }

hipError_t launch_norm_map(const void* h, bool bf16, int64_t N, int64_t C, int64_t ld, float* a, double* norms,
                           double* block_max, hipStream_t s) {
    const int g1 = norm_map_blocks(N);
    const size_t es = bf16 ? 2 : 4;
    const bool vec = (reinterpret_cast<uintptr_t>(h) & 15) == 0 && (ld * static_cast<int64_t>(es)) % 16 == 0;
    if (bf16) {
        const uint16_t* p = static_cast<const uint16_t*>(h);
        if (vec) hipLaunchKernelGGL((norm_rows_kernel<uint16_t, true>), dim3(g1), dim3(256), 0, s, p, N, C, ld, norms, block_max);
        else hipLaunchKernelGGL((norm_rows_kernel<uint16_t, false>), dim3(g1), dim3(256), 0, s, p, N, C, ld, norms, block_max);
    } else {
        const float* p = static_cast<const float*>(h);
        if (vec) hipLaunchKernelGGL((norm_rows_kernel<float, true>), dim3(g1), dim3(256), 0, s, p, N, C, ld, norms, block_max);
        else hipLaunchKernelGGL((norm_rows_kernel<float, false>), dim3(g1), dim3(256), 0, s, p, N, C, ld, norms, block_max);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned g2 = static_cast<unsigned>(std::min<int64_t>((N + 255) / 256, 1024));
    hipLaunchKernelGGL(norm_scale_kernel, dim3(g2), dim3(256), 0, s, norms, block_max, g1, N, a);
    return hipGetLastError();
}

}  // namespace prism

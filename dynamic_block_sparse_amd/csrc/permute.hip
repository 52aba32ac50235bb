// permute.hip - block-major gather and its inverse scatter.
//
// The pages reorganise the token sequence into zone-shaped blocks (news article
// at ailog.hnlab.kr, "핵심 내용" steps 1-2) and pool and attend whole blocks
// (Prism reading guide, "Phương pháp" §3); after this permutation every block
// is one contiguous run of 64, 128 or 256 rows, which is what the selection and
// attention kernels stream.  The order inside a zone is computed from the
// zone's shape index in-kernel; no index array is read.
//
// One wave moves one token row at a time with 16-byte loads and stores; a
// workgroup of 4 waves walks a contiguous range of block-major positions, so
// the block-major side is written (gather) or read (scatter) sequentially.
// permute_heads_kernel moves all heads of a token in one pass, with separate
// token and head strides on each side: a raster row of every head is read (or
// written) as one contiguous run, and each head's block-major rows go to (or
// come from) their own head-major plane.
#include "prism_device.hpp"
#include "prism_internal.hpp"

namespace prism {

constexpr int kPermThreads = 256;
constexpr int kPermRowsPerWave = 8;

// A wave moves `sub` rows at a time (sub = 64 / vectors-per-row for short rows,
// e.g. one head of 128 bf16 = 16 vectors -> 4 rows; 1 for long rows).
template <typename V>
__global__ void __launch_bounds__(kPermThreads)
permute_rows_kernel(const V* __restrict__ x, V* __restrict__ y, const uint8_t* __restrict__ zone_shape, ZoneGrid g,
                    int64_t N, int64_t vec_per_row, int64_t x_ld_vec, int64_t y_ld_vec, int inverse, int sub) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    const int rsub = sub > 1 ? lane / static_cast<int>(vec_per_row) : 0;
    const int c0 = sub > 1 ? lane % static_cast<int>(vec_per_row) : lane;
    const int cstep = sub > 1 ? static_cast<int>(vec_per_row) : kWave;
    if (rsub >= sub) return;
    const int64_t first =
        (static_cast<int64_t>(blockIdx.x) * (kPermThreads / kWave) + wid) * kPermRowsPerWave * sub;
#pragma unroll 1
    for (int r = 0; r < kPermRowsPerWave; ++r) {
        const int64_t p = first + static_cast<int64_t>(r) * sub + rsub;
        if (p >= N) return;
        const int64_t n = block_major_to_raster(p, zone_shape, g);
        const int64_t src = inverse ? p : n;
        const int64_t dst = inverse ? n : p;
        const V* __restrict__ xs = x + src * x_ld_vec;
        V* __restrict__ yd = y + dst * y_ld_vec;
        for (int64_t c = c0; c < vec_per_row; c += cstep) yd[c] = xs[c];
    }
}

hipError_t launch_block_permute(const void* x, void* y, int elem_bytes, int64_t row_elems, int64_t x_ld,
                                int64_t y_ld, const uint8_t* zone_shape, ZoneGrid g, int64_t N, int inverse,
                                hipStream_t s) {
    const int64_t row_bytes = row_elems * elem_bytes;
    int64_t vec = 2;
    if ((row_bytes % 16) == 0 && ((x_ld * elem_bytes) % 16) == 0 && ((y_ld * elem_bytes) % 16) == 0 &&
        ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) % 16) == 0)
        vec = 16;
    else if ((row_bytes % 4) == 0 && ((x_ld * elem_bytes) % 4) == 0 && ((y_ld * elem_bytes) % 4) == 0 &&
             ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) % 4) == 0)
        vec = 4;
    const int64_t vpr = row_bytes / vec;
    const int sub = vpr < kWave ? static_cast<int>(kWave / vpr) : 1;
    const int64_t rows_per_block = (kPermThreads / kWave) * kPermRowsPerWave * sub;
    const dim3 grid(static_cast<unsigned>((N + rows_per_block - 1) / rows_per_block));
    const int64_t xb = x_ld * elem_bytes, yb = y_ld * elem_bytes;
    if (vec == 16) {
        hipLaunchKernelGGL(permute_rows_kernel<uint4>, grid, dim3(kPermThreads), 0, s,
                           static_cast<const uint4*>(x), static_cast<uint4*>(y), zone_shape, g, N, vpr, xb / 16,
                           yb / 16, inverse, sub);
    } else if (vec == 4) {
        hipLaunchKernelGGL(permute_rows_kernel<uint32_t>, grid, dim3(kPermThreads), 0, s,
                           static_cast<const uint32_t*>(x), static_cast<uint32_t*>(y), zone_shape, g, N, vpr, xb / 4,
                           yb / 4, inverse, sub);
    } else {
        hipLaunchKernelGGL(permute_rows_kernel<uint16_t>, grid, dim3(kPermThreads), 0, s,
                           static_cast<const uint16_t*>(x), static_cast<uint16_t*>(y), zone_shape, g, N, vpr, xb / 2,
                           yb / 2, inverse, sub);
    }
    return hipGetLastError();
}

// All heads of one token per wave step: vector v of the row is head v / vph,
// vector v % vph of that head.  Strides are in vectors.
template <typename V>
__global__ void __launch_bounds__(kPermThreads)
permute_heads_kernel(const V* __restrict__ x, V* __restrict__ y, const uint8_t* __restrict__ zone_shape, ZoneGrid g,
                     int64_t N, int heads, int vph, int64_t x_ld, int64_t x_hs, int64_t y_ld, int64_t y_hs,
                     int inverse) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    const int nv = heads * vph;
    const int64_t first = (static_cast<int64_t>(blockIdx.x) * (kPermThreads / kWave) + wid) * kPermRowsPerWave;
#pragma unroll 1
    for (int r = 0; r < kPermRowsPerWave; ++r) {
        const int64_t p = first + r;
        if (p >= N) return;
        const int64_t n = block_major_to_raster(p, zone_shape, g);
        const V* __restrict__ xs = x + (inverse ? p : n) * x_ld;
        V* __restrict__ yd = y + (inverse ? n : p) * y_ld;
#pragma unroll 4
        for (int v = lane; v < nv; v += kWave) {
            const int hh = v / vph, c = v - hh * vph;
            yd[hh * y_hs + c] = xs[hh * x_hs + c];
        }
    }
}

hipError_t launch_block_permute_heads(const void* x, void* y, int elem_bytes, int heads, int d, int64_t x_ld,
                                      int64_t x_hs, int64_t y_ld, int64_t y_hs, const uint8_t* zone_shape, ZoneGrid g,
                                      int64_t N, int inverse, hipStream_t s) {
    // the caller has checked 16-byte alignment of the pointers, strides and rows
    const int per = 16 / elem_bytes;
    const int64_t rows_per_block = (kPermThreads / kWave) * kPermRowsPerWave;
    const dim3 grid(static_cast<unsigned>((N + rows_per_block - 1) / rows_per_block));
    hipLaunchKernelGGL(permute_heads_kernel<uint4>, grid, dim3(kPermThreads), 0, s, static_cast<const uint4*>(x),
                       static_cast<uint4*>(y), zone_shape, g, N, heads, d / per, x_ld / per, x_hs / per, y_ld / per,
                       y_hs / per, inverse);
    return hipGetLastError();
}

}  // namespace prism

// prism_device.hpp - device-side helpers shared by the gfx950 kernels of the
// Prism block-sparse attention library.  Wave size is 64 throughout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace prism {

constexpr int kWave = 64;
constexpr int kZone = 8;
constexpr int kZoneTokens = 512;
constexpr float kLog2e = 1.4426950408889634f;   // log2(e), for exp(x) = exp2(x log2(e))

// Candidate block shapes (b_T, b_H, b_W), 16 entries: every box with edges in
// {2, 4, 8} and volume 64, 128 or 256, by volume then lexicographically.  The
// index is what zone_shape stores and what breaks ties between equidistant
// shapes.
__host__ __device__ inline void shape_of(int idx, int& bt, int& bh, int& bw) {
    // packed as 2-bit log2 edges: (lt << 4) | (lh << 2) | lw
    constexpr uint8_t kPacked[16] = {
        (1 << 4) | (2 << 2) | 3, (1 << 4) | (3 << 2) | 2, (2 << 4) | (1 << 2) | 3,
        (2 << 4) | (2 << 2) | 2, (2 << 4) | (3 << 2) | 1, (3 << 4) | (1 << 2) | 2,
        (3 << 4) | (2 << 2) | 1,                                      // volume 64
        (1 << 4) | (3 << 2) | 3, (2 << 4) | (2 << 2) | 3, (2 << 4) | (3 << 2) | 2,
        (3 << 4) | (1 << 2) | 3, (3 << 4) | (2 << 2) | 2, (3 << 4) | (3 << 2) | 1,   // 128
        (2 << 4) | (3 << 2) | 3, (3 << 4) | (2 << 2) | 3, (3 << 4) | (3 << 2) | 2    // 256
    };
    const uint8_t p = kPacked[idx & 15];
    bt = 1 << ((p >> 4) & 3);
    bh = 1 << ((p >> 2) & 3);
    bw = 1 << (p & 3);
}

// bf16 <-> fp32 (round to nearest even; inputs here are finite)
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// wave-level reductions (fixed butterfly order, hence deterministic)
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}
template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        T o = __shfl_xor(v, off, kWave);
        v = o > v ? o : v;
    }
    return v;
}

// Block-wide sum in a fixed order: butterfly inside each wave, then the wave
// totals in wave order.  `scratch` holds at least blockDim.x / 64 values.
template <typename T>
__device__ __forceinline__ T block_sum(T v, T* scratch) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    const int nw = blockDim.x / kWave;
    v = wave_sum(v);
    __syncthreads();
    if (lane == 0) scratch[wid] = v;
    __syncthreads();
    T t = scratch[0];
    for (int w = 1; w < nw; ++w) t += scratch[w];
    return t;
}
template <typename T>
__device__ __forceinline__ T block_max(T v, T* scratch) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    const int nw = blockDim.x / kWave;
    v = wave_max(v);
    __syncthreads();
    if (lane == 0) scratch[wid] = v;
    __syncthreads();
    T t = scratch[0];
    for (int w = 1; w < nw; ++w) t = scratch[w] > t ? scratch[w] : t;
    return t;
}

// Map block-major position p to its raster token index for the zone shapes.
struct ZoneGrid {
    int T, H, W, nH, nW;
    const int32_t* order;   // order[pos] = raster zone at block-major zone position pos (NULL: raster)
};
__device__ __forceinline__ int64_t block_major_to_raster(int64_t p, const uint8_t* __restrict__ zone_shape,
                                                         const ZoneGrid g) {
    const int64_t m = g.order ? static_cast<int64_t>(g.order[p >> 9]) : (p >> 9);
    const int q = static_cast<int>(p & 511);
    int bt, bh, bw;
    shape_of(zone_shape[m], bt, bh, bw);
    const int vol = bt * bh * bw;
    const int j = q / vol;
    const int r = q - j * vol;
    const int nbh = kZone / bh, nbw = kZone / bw;
    const int jt = j / (nbh * nbw);
    const int jh = (j / nbw) % nbh;
    const int jw = j % nbw;
    const int rt = r / (bh * bw);
    const int rh = (r / bw) % bh;
    const int rw = r % bw;
    const int64_t zt = m / (g.nH * g.nW);
    const int64_t zh = (m / g.nW) % g.nH;
    const int64_t zw = m % g.nW;
    const int64_t t = zt * kZone + jt * bt + rt;
    const int64_t h = zh * kZone + jh * bh + rh;
    const int64_t w = zw * kZone + jw * bw + rw;
    return (t * g.H + h) * g.W + w;
}

// Where the attention kernels write their output rows (and where the backward
// reads O): the row at block-major position p goes to raster token pi(p) of the
// grid, at element offset pi(p) * ld + h * hs, when zone_shape is set; with
// zone_shape NULL it stays at p (ld and hs are then the inputs' strides).
struct RowMap {
    const uint8_t* zone_shape;
    ZoneGrid g;
    int64_t ld, hs;
};
__device__ __forceinline__ int64_t row_offset(const RowMap& m, int64_t p, int h) {
    const int64_t r = m.zone_shape ? block_major_to_raster(p, m.zone_shape, m.g) : p;
    return r * m.ld + static_cast<int64_t>(h) * m.hs;
}

// ---------------------------------------------------------------- direct global->LDS loads

typedef __attribute__((address_space(1))) void gvoid_t;
typedef __attribute__((address_space(3))) void lvoid_t;

// LDS byte address of a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lvoid_t*)p));
}

// One direct global->LDS load: lane l fetches BYTES bytes at gbase + voff[l]
// (voff an unsigned 32-bit byte offset) and they land at LDS address
// lds + BYTES * l.  It is written in asm so that the compiler does not see an
// LDS store in flight: it would otherwise make every later LDS read that it
// cannot tell apart (the transposing reads in particular) wait for all
// outstanding loads, including those into another buffer.  Completion is
// awaited explicitly (dma_join) before the buffer is read.  One wait state
// separates the M0 write from the load that uses it.
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gbase), "s"(lds)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* gbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(gbase), "s"(lds)
                 : "memory", "m0");
}

// wait for this wave's direct loads, then for every wave's
__device__ __forceinline__ void dma_join() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
}

}  // namespace prism

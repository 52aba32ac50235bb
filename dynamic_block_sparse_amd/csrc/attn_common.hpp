// attn_common.hpp - shared pieces of the bf16 MFMA attention kernels.
//
// Exact attention over the selected key blocks only, with an online softmax
// (Prism reading guide, xyznot.com paper 2610.05416, "Phương pháp" §3), and
// its gradient with the selection held constant.
//
// Every block is 1, 2 or 4 64-token tiles after the block-major permutation,
// and all rows of a block share its selected set, so the unit of work is a
// 64-row tile against the 64-key tiles of the selected blocks.  A workgroup
// has 2 waves; each wave owns 32 rows (forward, dQ) or 32 keys (dK/dV) and
// streams the other side's tiles through LDS.
//
// MFMA shape v_mfma_f32_32x32x16_bf16 (lane l, half h = l / 32):
//   A (32x16): lane holds row l%32, k = 8h .. 8h+7
//   B (16x32): lane holds k = 8h .. 8h+7, column l%32
//   C (32x32): lane holds column l%32, rows 8*(v/4) + 4h + v%4, v = 0..15
// Products whose reduction runs over tokens (P V, dS K, dO^T P, Q^T dS) take
// their B operand straight from a C tile in registers.  The 16-token k-step s2
// of a 32-token C tile then holds tokens 16*s2 + 4h + {0..3} and
// 16*s2 + 8 + 4h + {0..3}; the A operand is read in that same order from a
// row-major LDS tile with two transposing reads (ds_read_b64_tr_b16): in each
// group of 16 lanes, lane i receives element i%4 of the 8-byte chunks
// addressed by lanes i/4, 4 + i/4, 8 + i/4 and 12 + i/4 of the group, so
// pointing lane s at (row R + s/4, column C + 4*(s%4)) hands lane i rows
// R .. R+3 of column C + i.
//
// LDS tiles are 64 rows x D bf16, unpadded, with the 16-byte chunk c of row r
// stored at chunk position c ^ swz(r): swz(r) = 4*(r & 3) + ((r >> 2) & 3) for
// D = 128 and 2*(r & 3) + ((r >> 2) & 1) for D = 64.  Both the 16-byte row
// reads and the transposing reads are then free of LDS bank conflicts
// (measured with the bank-conflict counter on gfx950; the unswizzled layout
// and other XOR patterns conflict on one or the other).  Tiles are filled by direct global->LDS
// loads (global_load_lds_dwordx4: lane l's 16 bytes land at base + 16 l), each
// lane fetching the global chunk its LDS slot holds, so that the loads overlap
// the compute of this or another resident workgroup.
#pragma once
#include "prism_device.hpp"
#include "prism_internal.hpp"

namespace prism {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((__vector_size__(8)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.6931471805599453f;


__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
}

// two fp32 -> packed bf16 pair (round to nearest even), one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// bf16 residual of four fp32 values r against their rounded pair hi:
// r - float(hi), rounded to bf16.  hi + residual carries r to about 16 bits.
__device__ __forceinline__ u32x2_t residual4(const float (&r)[4], const u32x2_t& hi) {
    return u32x2_t{pack2(r[0] - __uint_as_float(hi.x << 16), r[1] - __uint_as_float(hi.x & 0xffff0000u)),
                   pack2(r[2] - __uint_as_float(hi.y << 16), r[3] - __uint_as_float(hi.y & 0xffff0000u))};
}

// acc + lo + hi of a packed bf16 pair, one v_dot2 against (1, 1)
__device__ __forceinline__ float sum_bf16_pair(uint32_t w, float acc) {
    const bf16x2_t one = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), one, acc, false);
}

// 2^x on the transcendental unit; results below the normal range flush to 0,
// which is what the softmax wants for scores far below the row maximum
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max(a, b, c) in one v_max3_f32 on the raw values.  fmaxf keeps IEEE NaN
// semantics, so the compiler first canonicalises every MFMA result with a
// v_max_f32 x, x of its own (two instructions per value instead of half of
// one); the scores here are never NaN, and the maximum is the same.
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// max of x and the x of lane ^ 32 (never NaN), through v_permlane32_swap (a register
// exchange between the two 32-lane halves, no LDS round trip): with both
// operands x, one result holds the lower half's values in both halves and the
// other the upper half's
__device__ __forceinline__ float max_across_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return max3_raw(__uint_as_float(r[0]), __uint_as_float(r[1]), __uint_as_float(r[1]));
}

// B operand of k-step s2 built from C-tile registers 8*s2 .. 8*s2+7
__device__ __forceinline__ u32x4_t pack_kstep(const f32x16_t& x, int s2) {
    return u32x4_t{pack2(x[8 * s2 + 0], x[8 * s2 + 1]), pack2(x[8 * s2 + 2], x[8 * s2 + 3]),
                   pack2(x[8 * s2 + 4], x[8 * s2 + 5]), pack2(x[8 * s2 + 6], x[8 * s2 + 7])};
}

// Scheduling hint for an unrolled run of STEPS steps that each issue NR LDS
// reads feeding NM MFMAs: keep the reads AHEAD steps ahead of the MFMAs that
// consume them, so LDS latency hides behind matrix work instead of the wave
// waiting on every step.
template <int NR, int NM, int STEPS, int AHEAD>
__device__ __forceinline__ void sched_reads_ahead() {
    __builtin_amdgcn_sched_group_barrier(0x100, NR * AHEAD, 0);
#pragma unroll
    for (int i = 0; i < STEPS - AHEAD; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NM * AHEAD, 0);
}

// ---------------------------------------------------------------- swizzled LDS tiles

template <int D>
__device__ __forceinline__ u32x4_t sw_read16(const uint16_t* tile, int r, int c);

// c0, c1 += A B over the D channels, where the A operands are the 16-byte rows
// (col and 32 + col) of a swizzled 64 x D tile and B the k-steps held in b:
// the two 32-row halves of the product of the tile with a 32-column operand.
// The tile fragments are read two k-steps ahead of the MFMAs that use them
// (left to itself the compiler reads each one just before its MFMA and waits
// the whole LDS latency every step); a schedule barrier keeps each step's
// reads and MFMAs in that order.
template <int D>
__device__ __forceinline__ void rows_x_ksteps(const uint16_t* tile, int col, int hl, const u32x4_t (&b)[D / 16],
                                              f32x16_t& c0, f32x16_t& c1) {
    constexpr int KS = D / 16;
    u32x4_t a[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        a[s][0] = sw_read16<D>(tile, col, 16 * s + 8 * hl);
        a[s][1] = sw_read16<D>(tile, 32 + col, 16 * s + 8 * hl);
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        u32x4_t n0, n1;
        if (s + 2 < KS) {
            n0 = sw_read16<D>(tile, col, 16 * (s + 2) + 8 * hl);
            n1 = sw_read16<D>(tile, 32 + col, 16 * (s + 2) + 8 * hl);
        }
        c0 = mfma32(a[s & 1][0], b[s], c0);
        c1 = mfma32(a[s & 1][1], b[s], c1);
        if (s + 2 < KS) {
            a[s & 1][0] = n0;
            a[s & 1][1] = n1;
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int D>
__device__ __forceinline__ int swz(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return ((r & 3) << 1) | ((r >> 2) & 1);
}

// element offset of (row r, column c) in a swizzled tile, c a multiple of 4
template <int D>
__device__ __forceinline__ int sw_off(int r, int c) {
    return r * D + ((((c >> 3) ^ swz<D>(r))) << 3) + (c & 7);
}

// 16-byte read of columns c .. c+7 (c a multiple of 8) of row r
template <int D>
__device__ __forceinline__ u32x4_t sw_read16(const uint16_t* tile, int r, int c) {
    return *reinterpret_cast<const u32x4_t*>(tile + sw_off<D>(r, c));
}

// A operand for a reduction over the rows of a swizzled tile: output rows are
// the tile's columns col0 .. col0+31, and the 16-row k-step starting at `base`
// is read in the permuted order that matches pack_kstep.
template <int D>
__device__ __forceinline__ u32x4_t tr_operand(const uint16_t* tile, int base, int col0, int lane) {
    const int g = lane >> 4, sl = lane & 15;
    const int row = base + 4 * (g >> 1) + (sl >> 2);
    const int col = col0 + 16 * (g & 1) + 4 * (sl & 3);
    const s16x4_t r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tile + sw_off<D>(row, col)));
    const s16x4_t r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tile + sw_off<D>(row + 8, col)));
    const u32x2_t a = __builtin_bit_cast(u32x2_t, r1);
    const u32x2_t b = __builtin_bit_cast(u32x2_t, r2);
    return u32x4_t{a.x, a.y, b.x, b.y};
}

// acc[m] += tile^T(rows row0 + 16 ks .. +15, columns 32 m .. +31) b[ks] for
// ks < KST and m < D / 32, in (ks, m) order: the DM accumulators are
// independent chains, and the transposed operands are read AHEAD products
// ahead of their MFMA (a schedule barrier keeps that order, as in
// rows_x_ksteps; 4 VGPRs per product read ahead).
template <int D, int KST, int AHEAD = 4>
__device__ __forceinline__ void tr_accumulate(const uint16_t* tile, int row0, const u32x4_t (&b)[KST],
                                              f32x16_t (&acc)[D / 32], int lane) {
    constexpr int DM = D / 32, N = KST * DM, kAhead = AHEAD;
    u32x4_t a[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead && i < N; ++i) a[i] = tr_operand<D>(tile, row0 + 16 * (i / DM), 32 * (i % DM), lane);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        u32x4_t nx;
        if (i + kAhead < N) nx = tr_operand<D>(tile, row0 + 16 * ((i + kAhead) / DM), 32 * ((i + kAhead) % DM), lane);
        acc[i % DM] = mfma32(a[i % kAhead], b[i / DM], acc[i % DM]);
        if (i + kAhead < N) a[i % kAhead] = nx;
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Per-lane byte offsets for loading a 64-row tile (token stride ld elements)
// into a swizzled LDS tile, shared by the NW waves of the workgroup: wave w
// issues instructions w, w + NW, ...; one instruction fills 1 KB of LDS
// (64 lanes x 16 bytes), i.e. 64 / (D / 8) consecutive rows.  Each lane loads
// the global chunk that its LDS slot holds under the swizzle.
template <int D, int NW>
struct TileDma {
    static constexpr int CPR = D / 8;       // 16-byte chunks per row
    static constexpr int RPI = 64 / CPR;    // rows per instruction
    static constexpr int NI = 64 / RPI;     // instructions per tile
    static constexpr int PER = NI / NW;     // instructions per wave
    uint32_t voff[PER];
    __device__ void init(int64_t ld, int wave, int lane) {
        const int pc = lane % CPR;
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int r = (u * NW + wave) * RPI + lane / CPR;
            voff[u] = static_cast<uint32_t>((r * ld + ((pc ^ swz<D>(r)) << 3)) * 2);
        }
    }
    __device__ void load(uint16_t* dst, const uint16_t* src, int wave) const {
        const uint32_t base = lds_addr(dst);
#pragma unroll
        for (int u = 0; u < PER; ++u) dma16(src, voff[u], base + (u * NW + wave) * 1024);
    }
};

// An empty use of x: the compiler waits here for the global load that
// produced x.  Operands loaded before the tile loop are settled this way;
// otherwise the compiler would place that wait at their first use inside the
// loop, in every iteration, where the direct loads in flight (which it does
// not see) would make it wait for the next tile as well.
__device__ __forceinline__ void settle(const u32x4_t& x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void settle(float x) { asm volatile("" ::"v"(x)); }

// Cursor over the 64-token tiles of a list of blocks (uniform across the workgroup).
struct TileCursor {
    const int32_t* __restrict__ sel;
    const int32_t* __restrict__ offs;
    int e, e_end, pos, end;
    __device__ void init(const int32_t* s, const int32_t* o, int e0, int e1) {
        sel = s;
        offs = o;
        e = e0;
        e_end = e1;
        pos = end = 0;
        if (e < e_end) {
            const int j = sel[e];
            pos = offs[j];
            end = offs[j + 1];
        }
    }
    __device__ int next() {   // next tile's first token, or -1
        if (e >= e_end) return -1;
        const int t = pos;
        pos += 64;
        if (pos >= end) {
            ++e;
            if (e < e_end) {
                const int j = sel[e];
                pos = offs[j];
                end = offs[j + 1];
            }
        }
        return t;
    }
};

// Double-buffered walk over the tiles of `cur`: tile t+1 is loaded into
// buffer b^1 while tile t, in buffer b, is used.  (The dK/dV kernel; the
// forward and dQ kernels keep one tile of each operand and a second resident
// workgroup per SIMD instead, loading by phase.)
template <class Issue, class Compute>
__device__ __forceinline__ void tile_pipeline(TileCursor& cur, Issue&& issue, Compute&& compute) {
    int t = cur.next();
    if (t < 0) return;
    issue(t, 0);
    dma_join();
    for (int b = 0;; b ^= 1) {
        t = cur.next();
        if (t >= 0) issue(t, b ^ 1);
        compute(b);
        dma_join();
        if (t < 0) return;
    }
}

// XCD-aware mapping.  Workgroups are dispatched in id order and dealt
// round-robin to the 8 XCDs; each XCD gets a contiguous range of the
// (head, tile) grid, so neighbouring tiles of a head, which select overlapping
// key blocks, meet in that XCD's L2.  (Measured at 2K: giving every XCD a
// slice of the same head instead was 1.2-1.8x slower.)
__device__ __forceinline__ int xcd_remap(int w) {
    const int G = static_cast<int>(gridDim.x);
    if (G % 8) return w;
    return (w % 8) * (G / 8) + w / 8;
}

// tile visited by workgroup wg (an entry outside the head's range, which a
// consistent set of block offsets never leaves, falls back to raster order)
__device__ __forceinline__ int tile_of(const int32_t* __restrict__ order, int wg, int ntiles) {
    const int t = order[wg];
    return static_cast<unsigned>(t) < static_cast<unsigned>(ntiles) ? t : wg % ntiles;
}

__device__ __forceinline__ int find_block(const int32_t* __restrict__ offs, int nb, int64_t p) {
    int a = 0, b = nb;
    while (b - a > 1) {
        const int m = (a + b) >> 1;
        if (offs[m] <= p) a = m;
        else b = m;
    }
    return a;
}

}  // namespace prism

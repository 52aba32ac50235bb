// attn_mfma.hip - block-sparse flash attention on gfx950 bf16 MFMA.
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
// lane fetching the global chunk its LDS slot holds, double-buffered so the
// next tile loads while the current one is used.
#include "prism_device.hpp"
#include "prism_internal.hpp"

namespace prism {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((__vector_size__(8)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(1))) void gvoid_t;
typedef __attribute__((address_space(3))) void lvoid_t;
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;


__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
}

// two fp32 -> packed bf16 pair (round to nearest even), one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// 2^x on the transcendental unit; results below the normal range flush to 0,
// which is what the softmax wants for scores far below the row maximum
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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

// LDS byte address of a __shared__ object
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lvoid_t*)p));
}

// One direct global->LDS load: lane l fetches BYTES bytes at gbase + voff[l]
// and they land at LDS address lds + BYTES * l.  It is written in asm so that
// the compiler does not see an LDS store in flight: it would otherwise make
// every later transposing LDS read wait for all outstanding loads, including
// those into the other buffer.  Completion is awaited explicitly (dma_join)
// before the buffer is read.  One wait state separates the M0 write from the
// load that uses it.
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gbase), "s"(lds)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* gbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(gbase), "s"(lds)
                 : "memory", "m0");
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

// wait for this wave's direct loads, then for every wave's
__device__ __forceinline__ void dma_join() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
}

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
// buffer b^1 while tile t, in buffer b, is used.
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

__device__ __forceinline__ int find_block(const int32_t* __restrict__ offs, int nb, int64_t p) {
    int a = 0, b = nb;
    while (b - a > 1) {
        const int m = (a + b) >> 1;
        if (offs[m] <= p) a = m;
        else b = m;
    }
    return a;
}

// ---------------------------------------------------------------- forward
//
// 2 waves per 64-row query tile; wave w owns rows 32*w .. +31 and streams
// every selected 64-key tile.  Scores are computed transposed, S^T = K Q^T,
// so a lane owns one query row: its max and sum need one cross-lane swap and
// the O^T rescale is a per-lane scalar.  The running maximum is raised only
// when a tile's maximum exceeds it by more than 8 (log2 units), so O is
// rescaled rarely; exponents stay below 2^8 in between.

template <int D>
__global__ void __launch_bounds__(128, 1)
attn_fwd_mfma_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                     uint16_t* __restrict__ o, float* __restrict__ lse, int64_t N, int64_t ld, int64_t hs,
                     const int32_t* __restrict__ offs, int nb, const int32_t* __restrict__ sel_off,
                     const int32_t* __restrict__ sel_idx, int64_t cap, float scale_log2) {
    __shared__ uint16_t kbuf[2][64 * D], vbuf[2][64 * D];
    const int ntiles = static_cast<int>(N / 64);
    const int wg = xcd_remap(blockIdx.x);
    const int h = wg / ntiles;
    const int64_t p0 = static_cast<int64_t>(wg % ntiles) * 64;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hl = lane >> 5, col = lane & 31;
    const int i = find_block(offs, nb, p0);
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
    float mrow = -INFINITY, lrow = 0.0f;

    TileDma<D, 2> dma;
    dma.init(ld, wave, lane);
    auto issue = [&](int t, int b) {
        dma.load(kbuf[b], kh_ + static_cast<int64_t>(t) * ld, wave);
        dma.load(vbuf[b], vh_ + static_cast<int64_t>(t) * ld, wave);
    };
    auto compute = [&](int b) {
        const uint16_t* kt = kbuf[b];
        const uint16_t* vt = vbuf[b];
        f32x16_t s0, s1;
#pragma unroll
        for (int x = 0; x < 16; ++x) s0[x] = s1[x] = 0.0f;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            s0 = mfma32(sw_read16<D>(kt, col, 16 * s + 8 * hl), qb[s], s0);
            s1 = mfma32(sw_read16<D>(kt, 32 + col, 16 * s + 8 * hl), qb[s], s1);
        }
        sched_reads_ahead<2, 2, KS, 2>();
        float mx = -INFINITY;
#pragma unroll
        for (int x = 0; x < 16; ++x) mx = fmaxf(mx, fmaxf(s0[x], s1[x]));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * scale_log2;
        if (__any(mx > mrow + 8.0f)) {
            const float mnew = fmaxf(mrow, mx);
            const float alpha = fast_exp2(mrow - mnew);
            mrow = mnew;
            lrow *= alpha;
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
        const u32x4_t pb[4] = {pack_kstep(s0, 0), pack_kstep(s0, 1), pack_kstep(s1, 0), pack_kstep(s1, 1)};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int m = 0; m < DM; ++m) oacc[m] = mfma32(tr_operand<D>(vt, 16 * ks, 32 * m, lane), pb[ks], oacc[m]);
    };

    TileCursor cur;
    cur.init(si, offs, e0, e1);
    tile_pipeline(cur, issue, compute);
    // lanes l and l^32 hold the two halves of a row's sum
    const float lt = lrow + __shfl_xor(lrow, 32, 64);
    const float inv = 1.0f / lt;
    uint16_t* orow = o + row * ld + h * hs;
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

// ---------------------------------------------------------------- backward
//
// dQ kernel (query-major): 2 waves per 64-row query tile, wave w owns rows
// 32*w .. +31 and streams every selected 64-key tile:
//   S^T = K Q^T, P^T = exp2(S^T - lse), dP^T = V dO^T, dS^T = P^T (dP^T - D),
//   dQ^T += K^T dS^T
// dK/dV kernel (key-major): 2 waves per 64-key tile, wave w owns keys
// 32*w .. +31 and streams the 64-row tiles of every query block that selected
// the tile's block (transposed CSR, ascending):
//   S = Q K^T, P = exp2(S - lse), dP = dO V^T, dS = P (dP - D),
//   dV^T += dO^T P, dK^T += Q^T dS
// Each output element is accumulated by one lane in a fixed order: the
// backward is deterministic.

template <int D>
__global__ void __launch_bounds__(128, 1)
attn_dq_mfma_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ Dq,
                    uint16_t* __restrict__ dq, int64_t N, int64_t ld, int64_t hs, const int32_t* __restrict__ offs,
                    int nb, const int32_t* __restrict__ sel_off, const int32_t* __restrict__ sel_idx, int64_t cap,
                    float scale_log2, float scale) {
    __shared__ uint16_t kbuf[2][64 * D], vbuf[2][64 * D];
    const int ntiles = static_cast<int>(N / 64);
    const int wg = xcd_remap(blockIdx.x);
    const int h = wg / ntiles;
    const int64_t p0 = static_cast<int64_t>(wg % ntiles) * 64;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hl = lane >> 5, col = lane & 31;
    const int i = find_block(offs, nb, p0);
    const int32_t* __restrict__ so = sel_off + static_cast<int64_t>(h) * (nb + 1);
    const int32_t* __restrict__ si = sel_idx + static_cast<int64_t>(h) * cap;
    const int e0 = so[i];
    const int e1 = static_cast<int>(min(static_cast<int64_t>(so[i + 1]), cap));
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
    f32x16_t acc[DM];
#pragma unroll
    for (int m = 0; m < DM; ++m)
#pragma unroll
        for (int x = 0; x < 16; ++x) acc[m][x] = 0.0f;
    const uint16_t* __restrict__ kh_ = k + h * hs;
    const uint16_t* __restrict__ vh_ = v + h * hs;

    TileDma<D, 2> dma;
    dma.init(ld, wave, lane);
    auto issue = [&](int t, int b) {
        dma.load(kbuf[b], kh_ + static_cast<int64_t>(t) * ld, wave);
        dma.load(vbuf[b], vh_ + static_cast<int64_t>(t) * ld, wave);
    };
    auto compute = [&](int b) {
        const uint16_t* kt = kbuf[b];
        const uint16_t* vt = vbuf[b];
        f32x16_t sa[2], pa[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int x = 0; x < 16; ++x) sa[mt][x] = pa[mt][x] = 0.0f;
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                sa[mt] = mfma32(sw_read16<D>(kt, 32 * mt + col, 16 * s + 8 * hl), qb[s], sa[mt]);
                pa[mt] = mfma32(sw_read16<D>(vt, 32 * mt + col, 16 * s + 8 * hl), db[s], pa[mt]);
            }
        sched_reads_ahead<4, 4, KS, 2>();
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int x = 0; x < 16; ++x) {
                const float p = fast_exp2(fmaf(sa[mt][x], scale_log2, -lrow));
                sa[mt][x] = p * (pa[mt][x] - drow);     // dS^T
            }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const u32x4_t bs = pack_kstep(sa[ks >> 1], ks & 1);
#pragma unroll
            for (int m = 0; m < DM; ++m) acc[m] = mfma32(tr_operand<D>(kt, 16 * ks, 32 * m, lane), bs, acc[m]);
        }
    };

    TileCursor cur;
    cur.init(si, offs, e0, e1);
    tile_pipeline(cur, issue, compute);
    uint16_t* out = dq + row * ld + h * hs;
#pragma unroll
    for (int m = 0; m < DM; ++m)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x16_t& a = acc[m];
            *reinterpret_cast<u32x2_t*>(out + 32 * m + 8 * g + 4 * hl) =
                u32x2_t{pack2(a[4 * g] * scale, a[4 * g + 1] * scale), pack2(a[4 * g + 2] * scale, a[4 * g + 3] * scale)};
        }
}

template <int D>
__global__ void __launch_bounds__(128)
attn_dkdv_mfma_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                      const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ Dq,
                      uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int64_t N, int64_t ld, int64_t hs,
                      const int32_t* __restrict__ offs, int nb, const int32_t* __restrict__ tr_off,
                      const int32_t* __restrict__ tr_idx, int64_t cap, float scale_log2, float scale) {
    // Q and dO tiles, lse (natural log) and D = rowsum(dO * O) of their rows
    __shared__ uint16_t qbuf[2][64 * D], obuf[2][64 * D];
    __shared__ float lbuf[2][64], dbuf[2][64];
    const int ntiles = static_cast<int>(N / 64);
    const int wg = xcd_remap(blockIdx.x);
    const int h = wg / ntiles;
    const int64_t k0 = static_cast<int64_t>(wg % ntiles) * 64;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hl = lane >> 5, col = lane & 31;
    const int j = find_block(offs, nb, k0);
    const int32_t* __restrict__ to = tr_off + static_cast<int64_t>(h) * (nb + 1);
    const int32_t* __restrict__ ti = tr_idx + static_cast<int64_t>(h) * cap;
    const int e0 = to[j];
    const int e1 = static_cast<int>(min(static_cast<int64_t>(to[j + 1]), cap));
    constexpr int KS = D / 16, DM = D / 32;
    const int64_t key = k0 + 32 * wave + col;
    u32x4_t kb[KS], vb[KS];
    {
        const uint16_t* kp = k + key * ld + h * hs;
        const uint16_t* vp = v + key * ld + h * hs;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            kb[s] = *reinterpret_cast<const u32x4_t*>(kp + 16 * s + 8 * hl);
            vb[s] = *reinterpret_cast<const u32x4_t*>(vp + 16 * s + 8 * hl);
        }
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            settle(kb[s]);
            settle(vb[s]);
        }
    }
    f32x16_t ak[DM], av[DM];
#pragma unroll
    for (int m = 0; m < DM; ++m)
#pragma unroll
        for (int x = 0; x < 16; ++x) ak[m][x] = av[m][x] = 0.0f;
    const uint16_t* __restrict__ qh_ = q + h * hs;
    const uint16_t* __restrict__ oh_ = dout + h * hs;
    const float* __restrict__ lh = lse + static_cast<int64_t>(h) * N;
    const float* __restrict__ dh = Dq + static_cast<int64_t>(h) * N;

    TileDma<D, 2> dma;
    dma.init(ld, wave, lane);
    const uint32_t loff = 4 * lane;
    auto issue = [&](int t, int b) {
        dma.load(qbuf[b], qh_ + static_cast<int64_t>(t) * ld, wave);
        dma.load(obuf[b], oh_ + static_cast<int64_t>(t) * ld, wave);
        if (wave == 0) dma4(lh + t, loff, lds_addr(lbuf[b]));
        else dma4(dh + t, loff, lds_addr(dbuf[b]));
    };
    auto compute = [&](int b) {
        const uint16_t* qt = qbuf[b];
        const uint16_t* ot = obuf[b];
        const float* lt = lbuf[b];
        const float* dt = dbuf[b];
        f32x16_t sa[2], pa[2];
#pragma unroll
        for (int mr = 0; mr < 2; ++mr)
#pragma unroll
            for (int x = 0; x < 16; ++x) sa[mr][x] = pa[mr][x] = 0.0f;
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int mr = 0; mr < 2; ++mr) {
                sa[mr] = mfma32(sw_read16<D>(qt, 32 * mr + col, 16 * s + 8 * hl), kb[s], sa[mr]);
                pa[mr] = mfma32(sw_read16<D>(ot, 32 * mr + col, 16 * s + 8 * hl), vb[s], pa[mr]);
            }
        sched_reads_ahead<4, 4, KS, 2>();
        // register x of row tile mr holds query row 32*mr + 8*(x/4) + 4*hl + x%4
#pragma unroll
        for (int mr = 0; mr < 2; ++mr)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 l4 = *reinterpret_cast<const float4*>(&lt[32 * mr + 8 * g + 4 * hl]);
                const float4 d4 = *reinterpret_cast<const float4*>(&dt[32 * mr + 8 * g + 4 * hl]);
                const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
                const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float p = fast_exp2(fmaf(sa[mr][4 * g + r], scale_log2, -lv[r] * kLog2e));
                    sa[mr][4 * g + r] = p;
                    pa[mr][4 * g + r] = p * (pa[mr][4 * g + r] - dv4[r]);   // dS
                }
            }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const u32x4_t bp = pack_kstep(sa[ks >> 1], ks & 1);
            const u32x4_t bs = pack_kstep(pa[ks >> 1], ks & 1);
#pragma unroll
            for (int m = 0; m < DM; ++m) {
                av[m] = mfma32(tr_operand<D>(ot, 16 * ks, 32 * m, lane), bp, av[m]);
                ak[m] = mfma32(tr_operand<D>(qt, 16 * ks, 32 * m, lane), bs, ak[m]);
            }
        }
    };

    TileCursor cur;
    cur.init(ti, offs, e0, e1);
    tile_pipeline(cur, issue, compute);
    uint16_t* ko = dk + key * ld + h * hs;
    uint16_t* vo = dv + key * ld + h * hs;
#pragma unroll
    for (int m = 0; m < DM; ++m)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x16_t& a = ak[m];
            const f32x16_t& c = av[m];
            const int dcol = 32 * m + 8 * g + 4 * hl;
            *reinterpret_cast<u32x2_t*>(ko + dcol) =
                u32x2_t{pack2(a[4 * g] * scale, a[4 * g + 1] * scale), pack2(a[4 * g + 2] * scale, a[4 * g + 3] * scale)};
            *reinterpret_cast<u32x2_t*>(vo + dcol) =
                u32x2_t{pack2(c[4 * g], c[4 * g + 1]), pack2(c[4 * g + 2], c[4 * g + 3])};
        }
}

// ---------------------------------------------------------------- launchers

hipError_t launch_attn_fwd_mfma(const void* q, const void* k, const void* v, void* o, float* lse, int64_t N, int heads,
                                int d, int64_t ld, int64_t hs, const int32_t* offs, int nb, const int32_t* so,
                                const int32_t* si, int64_t cap, float scale, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(N / 64 * heads));
    const float sl2 = scale * kLog2e;
    const uint16_t* Q = static_cast<const uint16_t*>(q);
    const uint16_t* K = static_cast<const uint16_t*>(k);
    const uint16_t* V = static_cast<const uint16_t*>(v);
    uint16_t* O = static_cast<uint16_t*>(o);
    if (d == 128)
        hipLaunchKernelGGL(attn_fwd_mfma_kernel<128>, grid, dim3(128), 0, s, Q, K, V, O, lse, N, ld, hs, offs, nb, so,
                           si, cap, sl2);
    else
        hipLaunchKernelGGL(attn_fwd_mfma_kernel<64>, grid, dim3(128), 0, s, Q, K, V, O, lse, N, ld, hs, offs, nb, so,
                           si, cap, sl2);
    return hipGetLastError();
}

hipError_t launch_attn_bwd_mfma(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                                const float* Dq, void* dq, void* dk, void* dv, int64_t N, int heads, int d, int64_t ld,
                                int64_t hs, const int32_t* offs, int nb, const int32_t* so, const int32_t* si,
                                const int32_t* to, const int32_t* ti, int64_t cap, float scale, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(N / 64 * heads));
    const float sl2 = scale * kLog2e;
    const uint16_t* Q = static_cast<const uint16_t*>(q);
    const uint16_t* K = static_cast<const uint16_t*>(k);
    const uint16_t* V = static_cast<const uint16_t*>(v);
    const uint16_t* O = static_cast<const uint16_t*>(dout);
    uint16_t* dQ = static_cast<uint16_t*>(dq);
    uint16_t* dK = static_cast<uint16_t*>(dk);
    uint16_t* dV = static_cast<uint16_t*>(dv);
    if (d == 128) {
        hipLaunchKernelGGL(attn_dq_mfma_kernel<128>, grid, dim3(128), 0, s, Q, K, V, O, lse, Dq, dQ, N, ld, hs, offs,
                           nb, so, si, cap, sl2, scale);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(attn_dkdv_mfma_kernel<128>, grid, dim3(128), 0, s, Q, K, V, O, lse, Dq, dK, dV, N, ld, hs,
                           offs, nb, to, ti, cap, sl2, scale);
    } else {
        hipLaunchKernelGGL(attn_dq_mfma_kernel<64>, grid, dim3(128), 0, s, Q, K, V, O, lse, Dq, dQ, N, ld, hs, offs,
                           nb, so, si, cap, sl2, scale);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(attn_dkdv_mfma_kernel<64>, grid, dim3(128), 0, s, Q, K, V, O, lse, Dq, dK, dV, N, ld, hs,
                           offs, nb, to, ti, cap, sl2, scale);
    }
    return hipGetLastError();
}

}  // namespace prism

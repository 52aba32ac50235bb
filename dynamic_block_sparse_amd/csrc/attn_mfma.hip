// attn_mfma.hip - block-sparse flash attention on gfx950 bf16 MFMA.
//
// Exact attention over the selected key blocks only, with an online softmax
// (Prism reading guide, xyznot.com paper 2610.05416, "Phương pháp" §3).
//
// Layout of the work.  A workgroup of 4 waves owns one 64-row query tile of
// one head (every block is 1, 2 or 4 such tiles after the block-major
// permutation, and all rows of a block share its selected set).  The tile's
// key stream is the concatenation of the selected blocks' 64-key tiles;
// each iteration stages two key tiles in LDS.  Wave w takes query rows
// 32*(w & 1) .. +31 against key tile (w >> 1) of the pair, keeps its own
// online-softmax state, and the two key halves are merged at the end.
//
// MFMA shapes (v_mfma_f32_32x32x16_bf16; lane l, half h = l / 32):
//   A (32x16): lane holds row l%32, columns 8h..8h+7
//   B (16x32): lane holds rows 8h..8h+7, column l%32
//   C (32x32): lane holds column l%32, rows 8*(v/4) + 4h + v%4, v = 0..15
// Scores are computed transposed, S^T = K Q^T (A = K from LDS, B = Q from
// registers), so a lane owns one query row (column l%32) and 32 of the tile's
// keys; P^T then already sits in the B-operand layout of O^T = V^T P^T up to a
// permutation of the 16 keys of each k-step, which the V^T operand reads in
// the same order.  V is stored transposed in LDS for that operand.
#include "prism_device.hpp"
#include "prism_internal.hpp"

namespace prism {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    const __bf16 a = static_cast<__bf16>(lo);
    const __bf16 b = static_cast<__bf16>(hi);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Cursor over the 64-key tiles of a selected set (uniform across the workgroup).
struct TileCursor {
    const int32_t* __restrict__ sel;   // selected block indices
    const int32_t* __restrict__ offs;  // block offsets
    int e, e_end;                      // position in sel
    int pos, end;                      // token range of the current block
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
    // next tile's first token, or -1
    __device__ int next() {
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

template <int D>
struct FwdSmem {
    static constexpr int KS = D + 8;    // K row stride (bf16): 16-byte aligned, conflict-free A reads
    static constexpr int VS = 64 + 4;   // V^T row stride (bf16)
    uint16_t k[2][64][KS];
    uint16_t vt[2][D][VS];
};

// Global -> register staging of a key tile pair.  K: 16-byte chunks, row-major
// coalesced; V: each thread takes two adjacent keys of one 8-column chunk so
// that the transposed LDS store writes whole dwords.
template <int D>
struct PairRegs {
    static constexpr int KCH = 2 * 64 * D / 8 / 256;   // K chunks per thread
    static constexpr int VPR = 2 * 32 * D / 8 / 256;   // V key-pair chunks per thread
    u32x4_t k[KCH];
    u32x4_t v0[VPR], v1[VPR];
};

template <int D>
__device__ __forceinline__ void load_pair(PairRegs<D>& r, const uint16_t* __restrict__ kh, const uint16_t* __restrict__ vh,
                                          int64_t ld, int t0, int t1) {
    constexpr int CPR = D / 8;  // 16-byte chunks per row
#pragma unroll
    for (int e = 0; e < PairRegs<D>::KCH; ++e) {
        const int c = threadIdx.x + 256 * e;
        const int tile = c / (64 * CPR);
        const int rr = c % (64 * CPR);
        const int key = rr / CPR, col = rr % CPR;
        const int t = tile ? t1 : t0;
        if (t >= 0) r.k[e] = *reinterpret_cast<const u32x4_t*>(kh + static_cast<int64_t>(t + key) * ld + col * 8);
    }
#pragma unroll
    for (int e = 0; e < PairRegs<D>::VPR; ++e) {
        const int c = threadIdx.x + 256 * e;
        const int tile = c / (32 * CPR);
        const int rr = c % (32 * CPR);
        const int kp = rr % 32, col = rr / 32;
        const int t = tile ? t1 : t0;
        if (t >= 0) {
            r.v0[e] = *reinterpret_cast<const u32x4_t*>(vh + static_cast<int64_t>(t + 2 * kp) * ld + col * 8);
            r.v1[e] = *reinterpret_cast<const u32x4_t*>(vh + static_cast<int64_t>(t + 2 * kp + 1) * ld + col * 8);
        }
    }
}

template <int D>
__device__ __forceinline__ void store_pair(const PairRegs<D>& r, FwdSmem<D>& sm, bool has1) {
    constexpr int CPR = D / 8;
#pragma unroll
    for (int e = 0; e < PairRegs<D>::KCH; ++e) {
        const int c = threadIdx.x + 256 * e;
        const int tile = c / (64 * CPR);
        const int rr = c % (64 * CPR);
        const int key = rr / CPR, col = rr % CPR;
        if (tile == 0 || has1) *reinterpret_cast<u32x4_t*>(&sm.k[tile][key][col * 8]) = r.k[e];
    }
#pragma unroll
    for (int e = 0; e < PairRegs<D>::VPR; ++e) {
        const int c = threadIdx.x + 256 * e;
        const int tile = c / (32 * CPR);
        const int rr = c % (32 * CPR);
        const int kp = rr % 32, col = rr / 32;
        if (tile == 0 || has1) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t a = r.v0[e][q], b = r.v1[e][q];
                // column 8*col + 2q from both keys, then column 8*col + 2q + 1
                *reinterpret_cast<uint32_t*>(&sm.vt[tile][col * 8 + 2 * q][2 * kp]) = (a & 0xFFFFu) | (b << 16);
                *reinterpret_cast<uint32_t*>(&sm.vt[tile][col * 8 + 2 * q + 1][2 * kp]) = (a >> 16) | (b & 0xFFFF0000u);
            }
        }
    }
}

// XCD-aware mapping.  Workgroups are dispatched in id order and dealt
// round-robin to the 8 XCDs; each XCD gets a contiguous range of the
// (head, tile) grid, so neighbouring tiles of a head, which select overlapping
// key blocks, meet in that XCD's L2.  (Measured at 2K: giving every XCD a
// slice of the same head instead was 1.2-1.8x slower.)
__device__ __forceinline__ int xcd_remap(int w, int ntiles) {
    const int G = static_cast<int>(gridDim.x);
    (void)ntiles;
    if (G % 8) return w;
    return (w % 8) * (G / 8) + w / 8;
}

template <int D>
__global__ void __launch_bounds__(256, 2)
attn_fwd_mfma_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                     uint16_t* __restrict__ o, float* __restrict__ lse, int64_t N, int heads, int64_t ld, int64_t hs,
                     const int32_t* __restrict__ offs, int nb, const int32_t* __restrict__ sel_off,
                     const int32_t* __restrict__ sel_idx, int64_t cap, float scale_log2) {
    __shared__ FwdSmem<D> sm;
    const int ntiles = static_cast<int>(N / 64);
    const int G = ntiles * heads;
    const int wg = xcd_remap(blockIdx.x, ntiles);
    const int h = wg / ntiles;
    const int qt = wg % ntiles;
    const int64_t p0 = static_cast<int64_t>(qt) * 64;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int rh = wave & 1, kh = wave >> 1;
    const int hl = lane >> 5, col = lane & 31;

    // block of this tile
    int i;
    {
        int a = 0, b = nb;
        while (b - a > 1) {
            const int m = (a + b) >> 1;
            if (offs[m] <= p0) a = m;
            else b = m;
        }
        i = a;
    }
    const uint16_t* __restrict__ kh_ = k + h * hs;
    const uint16_t* __restrict__ vh_ = v + h * hs;
    const int32_t* __restrict__ so = sel_off + static_cast<int64_t>(h) * (nb + 1);
    const int32_t* __restrict__ si = sel_idx + static_cast<int64_t>(h) * cap;
    const int e0 = so[i];
    const int e1 = static_cast<int>(min(static_cast<int64_t>(so[i + 1]), cap));

    // Q^T operand: this lane's query row, columns 16s + 8h .. +7
    constexpr int KS = D / 16;
    u32x4_t qb[KS];
    {
        const uint16_t* qrow = q + (p0 + 32 * rh + col) * ld + h * hs;
#pragma unroll
        for (int s = 0; s < KS; ++s) qb[s] = *reinterpret_cast<const u32x4_t*>(qrow + 16 * s + 8 * hl);
    }
    constexpr int DM = D / 32;
    f32x16_t oacc[DM];
#pragma unroll
    for (int m = 0; m < DM; ++m)
#pragma unroll
        for (int v2 = 0; v2 < 16; ++v2) oacc[m][v2] = 0.0f;
    float mrow = -INFINITY, lrow = 0.0f;

    TileCursor cur;
    cur.init(si, offs, e0, e1);
    PairRegs<D> regs;
    int t0 = cur.next();
    int t1 = cur.next();
    load_pair<D>(regs, kh_, vh_, ld, t0, t1);
    while (t0 >= 0) {
        const bool has1 = t1 >= 0;
        __syncthreads();
        store_pair<D>(regs, sm, has1);
        __syncthreads();
        const int n0 = cur.next();
        const int n1 = n0 >= 0 ? cur.next() : -1;
        if (n0 >= 0) load_pair<D>(regs, kh_, vh_, ld, n0, n1);
        if (kh == 0 || has1) {
            // S^T for 64 keys (two 32-key M tiles) x 32 rows
            f32x16_t s0, s1;
#pragma unroll
            for (int v2 = 0; v2 < 16; ++v2) s0[v2] = s1[v2] = 0.0f;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const u32x4_t a0 = *reinterpret_cast<const u32x4_t*>(&sm.k[kh][col][16 * s + 8 * hl]);
                const u32x4_t a1 = *reinterpret_cast<const u32x4_t*>(&sm.k[kh][32 + col][16 * s + 8 * hl]);
                s0 = mfma32(a0, qb[s], s0);
                s1 = mfma32(a1, qb[s], s1);
            }
            float mx = -INFINITY;
#pragma unroll
            for (int v2 = 0; v2 < 16; ++v2) {
                s0[v2] *= scale_log2;
                s1[v2] *= scale_log2;
                mx = fmaxf(mx, fmaxf(s0[v2], s1[v2]));
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float mnew = fmaxf(mrow, mx);
            const float alpha = exp2f(mrow - mnew);
            mrow = mnew;
            float ls = 0.0f;
#pragma unroll
            for (int v2 = 0; v2 < 16; ++v2) {
                s0[v2] = exp2f(s0[v2] - mnew);
                s1[v2] = exp2f(s1[v2] - mnew);
                ls += s0[v2] + s1[v2];
            }
            lrow = lrow * alpha + ls;
#pragma unroll
            for (int m = 0; m < DM; ++m)
#pragma unroll
                for (int v2 = 0; v2 < 16; ++v2) oacc[m][v2] *= alpha;
            // P^T operands: k-step (mt, s2) takes registers 8*s2 .. 8*s2+7 of M tile mt
            u32x4_t pb[4];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                pb[s2] = u32x4_t{pack2(s0[8 * s2 + 0], s0[8 * s2 + 1]), pack2(s0[8 * s2 + 2], s0[8 * s2 + 3]),
                                 pack2(s0[8 * s2 + 4], s0[8 * s2 + 5]), pack2(s0[8 * s2 + 6], s0[8 * s2 + 7])};
                pb[2 + s2] = u32x4_t{pack2(s1[8 * s2 + 0], s1[8 * s2 + 1]), pack2(s1[8 * s2 + 2], s1[8 * s2 + 3]),
                                     pack2(s1[8 * s2 + 4], s1[8 * s2 + 5]), pack2(s1[8 * s2 + 6], s1[8 * s2 + 7])};
            }
            // O^T += V^T P^T; the V^T operand reads keys base + 4h + 0..3 and base + 8 + 4h + 0..3
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int base = 16 * ks + 4 * hl;
#pragma unroll
                for (int m = 0; m < DM; ++m) {
                    const uint16_t* vrow = &sm.vt[kh][32 * m + col][0];
                    const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(vrow + base);
                    const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(vrow + base + 8);
                    oacc[m] = mfma32(u32x4_t{lo.x, lo.y, hi.x, hi.y}, pb[ks], oacc[m]);
                }
            }
        }
        t0 = n0;
        t1 = n1;
    }
    // merge the two key halves (waves kh = 1 hand their state to kh = 0)
    __syncthreads();
    float* red = reinterpret_cast<float*>(&sm);   // reuses the staging area
    const int slot = rh * 64 + lane;
    constexpr int PER = 3 + 16 * DM;   // odd stride: lanes land in distinct banks
    if (kh == 1) {
        float* dst = red + slot * PER;
        dst[0] = mrow;
        dst[1] = lrow;
#pragma unroll
        for (int m = 0; m < DM; ++m)
#pragma unroll
            for (int v2 = 0; v2 < 16; ++v2) dst[2 + 16 * m + v2] = oacc[m][v2];
    }
    __syncthreads();
    if (kh == 0) {
        const float* src = red + slot * PER;
        const float m1 = src[0], l1 = src[1];
        const float mt = fmaxf(mrow, m1);
        const float a0 = exp2f(mrow - mt);
        const float a1 = (m1 == -INFINITY) ? 0.0f : exp2f(m1 - mt);
        float lt = lrow * a0 + l1 * a1;
        lt += __shfl_xor(lt, 32, 64);
        const float inv = 1.0f / lt;
        const int64_t row = p0 + 32 * rh + col;
        uint16_t* orow = o + row * ld + h * hs;
#pragma unroll
        for (int m = 0; m < DM; ++m)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float x[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) x[r] = (oacc[m][4 * g + r] * a0 + src[2 + 16 * m + 4 * g + r] * a1) * inv;
                const int dcol = 32 * m + 8 * g + 4 * hl;
                *reinterpret_cast<u32x2_t*>(orow + dcol) = u32x2_t{pack2(x[0], x[1]), pack2(x[2], x[3])};
            }
        if (hl == 0) lse[static_cast<int64_t>(h) * N + row] = (mt + __log2f(lt)) * kLn2;
    }
}

// ---------------------------------------------------------------- backward
//
// dQ kernel (query-major): a workgroup owns a 64-row query tile and streams the
// selected 64-key tiles one at a time; wave w takes rows 32*(w & 1) and keys
// 32*(w >> 1) of the tile:
//   S^T = K Q^T, P^T = exp2(S^T - lse), dP^T = V dO^T, dS^T = P^T (dP^T - D),
//   dQ^T += K^T dS^T
// dK/dV kernel (key-major): a workgroup owns a 64-key tile and streams the
// 64-row tiles of every query block that selected its block (transposed CSR,
// ascending); wave w takes keys 32*(w & 1) and rows 32*(w >> 1):
//   S = Q K^T, P = exp2(S - lse), dP = dO V^T, dS = P (dP - D),
//   dV^T += dO^T P, dK^T += Q^T dS
// The two halves of each workgroup are summed in a fixed order at the end, so
// every output element is accumulated in the same order on every run.

template <int D>
struct Tile2 {                       // one 64-row tile: natural and transposed copies
    static constexpr int NS = D + 8;
    static constexpr int TS = 64 + 4;
    uint16_t nat[64][NS];
    uint16_t tr[D][TS];
};

// Stage rows t .. t+63 of x (token stride ld) into `nat` (and `tr` if TR).
// Each thread takes two adjacent rows of an 8-column chunk.
template <int D, bool TR>
__device__ __forceinline__ void stage_tile(Tile2<D>& tl, const uint16_t* __restrict__ x, int64_t ld, int t) {
    constexpr int CPR = D / 8;
    constexpr int PER = 32 * CPR / 256;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const int c = threadIdx.x + 256 * e;
        const int rp = c % 32, cc = c / 32;
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(x + static_cast<int64_t>(t + 2 * rp) * ld + cc * 8);
        const u32x4_t b = *reinterpret_cast<const u32x4_t*>(x + static_cast<int64_t>(t + 2 * rp + 1) * ld + cc * 8);
        *reinterpret_cast<u32x4_t*>(&tl.nat[2 * rp][cc * 8]) = a;
        *reinterpret_cast<u32x4_t*>(&tl.nat[2 * rp + 1][cc * 8]) = b;
        if (TR) {
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                *reinterpret_cast<uint32_t*>(&tl.tr[cc * 8 + 2 * qq][2 * rp]) = (a[qq] & 0xFFFFu) | (b[qq] << 16);
                *reinterpret_cast<uint32_t*>(&tl.tr[cc * 8 + 2 * qq + 1][2 * rp]) =
                    (a[qq] >> 16) | (b[qq] & 0xFFFF0000u);
            }
        }
    }
}

// B operand of a 16-row k-step built from accumulator registers 8*s2 .. 8*s2+7
__device__ __forceinline__ u32x4_t pack_kstep(const f32x16_t& x, int s2) {
    return u32x4_t{pack2(x[8 * s2 + 0], x[8 * s2 + 1]), pack2(x[8 * s2 + 2], x[8 * s2 + 3]),
                   pack2(x[8 * s2 + 4], x[8 * s2 + 5]), pack2(x[8 * s2 + 6], x[8 * s2 + 7])};
}

// A operand from a transposed tile: row r of tr, the 16-column k-step at
// column offset c0, in the permuted order (c0 + 4h + 0..3, c0 + 8 + 4h + 0..3)
template <int D>
__device__ __forceinline__ u32x4_t tr_operand(const Tile2<D>& tl, int r, int c0, int hl) {
    const uint16_t* p = &tl.tr[r][c0 + 4 * hl];
    const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(p);
    const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(p + 8);
    return u32x4_t{lo.x, lo.y, hi.x, hi.y};
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

template <int D>
struct DqSmem {
    Tile2<D> k;
    uint16_t v[64][D + 8];
};

template <int D>
__global__ void __launch_bounds__(256, 2)
attn_dq_mfma_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ Dq,
                    uint16_t* __restrict__ dq, int64_t N, int heads, int64_t ld, int64_t hs,
                    const int32_t* __restrict__ offs, int nb, const int32_t* __restrict__ sel_off,
                    const int32_t* __restrict__ sel_idx, int64_t cap, float scale_log2, float scale) {
    __shared__ DqSmem<D> sm;
    const int ntiles = static_cast<int>(N / 64);
    const int wg = xcd_remap(blockIdx.x, ntiles);
    const int h = wg / ntiles;
    const int qt = wg % ntiles;
    const int64_t p0 = static_cast<int64_t>(qt) * 64;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int rh = wave & 1, kq = wave >> 1;
    const int hl = lane >> 5, col = lane & 31;
    const int i = find_block(offs, nb, p0);
    const int32_t* __restrict__ so = sel_off + static_cast<int64_t>(h) * (nb + 1);
    const int32_t* __restrict__ si = sel_idx + static_cast<int64_t>(h) * cap;
    const int e0 = so[i];
    const int e1 = static_cast<int>(min(static_cast<int64_t>(so[i + 1]), cap));
    constexpr int KS = D / 16, DM = D / 32;
    const int64_t row = p0 + 32 * rh + col;
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
    f32x16_t acc[DM];
#pragma unroll
    for (int m = 0; m < DM; ++m)
#pragma unroll
        for (int v2 = 0; v2 < 16; ++v2) acc[m][v2] = 0.0f;
    const uint16_t* __restrict__ kh_ = k + h * hs;
    const uint16_t* __restrict__ vh_ = v + h * hs;
    TileCursor cur;
    cur.init(si, offs, e0, e1);
    for (int t = cur.next(); t >= 0; t = cur.next()) {
        __syncthreads();
        stage_tile<D, true>(sm.k, kh_, ld, t);
        {
            constexpr int CPR = D / 8;
#pragma unroll
            for (int e = 0; e < 64 * CPR / 256; ++e) {
                const int c = threadIdx.x + 256 * e;
                const int r = c / CPR, cc = c % CPR;
                *reinterpret_cast<u32x4_t*>(&sm.v[r][cc * 8]) =
                    *reinterpret_cast<const u32x4_t*>(vh_ + static_cast<int64_t>(t + r) * ld + cc * 8);
            }
        }
        __syncthreads();
        f32x16_t sa, pa;
#pragma unroll
        for (int v2 = 0; v2 < 16; ++v2) sa[v2] = pa[v2] = 0.0f;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const u32x4_t ak = *reinterpret_cast<const u32x4_t*>(&sm.k.nat[32 * kq + col][16 * s + 8 * hl]);
            const u32x4_t av = *reinterpret_cast<const u32x4_t*>(&sm.v[32 * kq + col][16 * s + 8 * hl]);
            sa = mfma32(ak, qb[s], sa);
            pa = mfma32(av, db[s], pa);
        }
#pragma unroll
        for (int v2 = 0; v2 < 16; ++v2) {
            const float p = exp2f(sa[v2] * scale_log2 - lrow);
            sa[v2] = p * (pa[v2] - drow);          // dS^T
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const u32x4_t b = pack_kstep(sa, s2);
#pragma unroll
            for (int m = 0; m < DM; ++m) acc[m] = mfma32(tr_operand<D>(sm.k, 32 * m + col, 32 * kq + 16 * s2, hl), b, acc[m]);
        }
    }
    // sum the two key halves: kq = 1 hands its partial to kq = 0
    __syncthreads();
    float* red = reinterpret_cast<float*>(&sm);
    const int slot = rh * 64 + lane;
    if (kq == 1) {
#pragma unroll
        for (int m = 0; m < DM; ++m)
#pragma unroll
            for (int v2 = 0; v2 < 16; ++v2) red[slot * (16 * DM + 1) + 16 * m + v2] = acc[m][v2];
    }
    __syncthreads();
    if (kq == 0) {
        uint16_t* out = dq + row * ld + h * hs;
#pragma unroll
        for (int m = 0; m < DM; ++m)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float x[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    x[r] = (acc[m][4 * g + r] + red[slot * (16 * DM + 1) + 16 * m + 4 * g + r]) * scale;
                *reinterpret_cast<u32x2_t*>(out + 32 * m + 8 * g + 4 * hl) = u32x2_t{pack2(x[0], x[1]), pack2(x[2], x[3])};
            }
    }
}

template <int D>
struct DkvSmem {
    Tile2<D> q;
    Tile2<D> o;       // dO
    float l2[64];     // lse in log2 units
    float dd[64];     // D = rowsum(dO * O)
};

template <int D>
__global__ void __launch_bounds__(256, 2)
attn_dkdv_mfma_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                      const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ Dq,
                      uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int64_t N, int heads, int64_t ld,
                      int64_t hs, const int32_t* __restrict__ offs, int nb, const int32_t* __restrict__ tr_off,
                      const int32_t* __restrict__ tr_idx, int64_t cap, float scale_log2, float scale) {
    __shared__ DkvSmem<D> sm;
    const int ntiles = static_cast<int>(N / 64);
    const int wg = xcd_remap(blockIdx.x, ntiles);
    const int h = wg / ntiles;
    const int kt = wg % ntiles;
    const int64_t k0 = static_cast<int64_t>(kt) * 64;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int kr = wave & 1, qr = wave >> 1;
    const int hl = lane >> 5, col = lane & 31;
    const int j = find_block(offs, nb, k0);
    const int32_t* __restrict__ to = tr_off + static_cast<int64_t>(h) * (nb + 1);
    const int32_t* __restrict__ ti = tr_idx + static_cast<int64_t>(h) * cap;
    const int e0 = to[j];
    const int e1 = static_cast<int>(min(static_cast<int64_t>(to[j + 1]), cap));
    constexpr int KS = D / 16, DM = D / 32;
    const int64_t key = k0 + 32 * kr + col;
    u32x4_t kb[KS], vb[KS];
    {
        const uint16_t* kp = k + key * ld + h * hs;
        const uint16_t* vp = v + key * ld + h * hs;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            kb[s] = *reinterpret_cast<const u32x4_t*>(kp + 16 * s + 8 * hl);
            vb[s] = *reinterpret_cast<const u32x4_t*>(vp + 16 * s + 8 * hl);
        }
    }
    f32x16_t ak[DM], av[DM];
#pragma unroll
    for (int m = 0; m < DM; ++m)
#pragma unroll
        for (int v2 = 0; v2 < 16; ++v2) ak[m][v2] = av[m][v2] = 0.0f;
    const uint16_t* __restrict__ qh_ = q + h * hs;
    const uint16_t* __restrict__ oh_ = dout + h * hs;
    const float* __restrict__ lh = lse + static_cast<int64_t>(h) * N;
    const float* __restrict__ dh = Dq + static_cast<int64_t>(h) * N;
    TileCursor cur;
    cur.init(ti, offs, e0, e1);
    for (int t = cur.next(); t >= 0; t = cur.next()) {
        __syncthreads();
        stage_tile<D, true>(sm.q, qh_, ld, t);
        stage_tile<D, true>(sm.o, oh_, ld, t);
        if (threadIdx.x < 64) sm.l2[threadIdx.x] = lh[t + threadIdx.x] * kLog2e;
        else if (threadIdx.x < 128) sm.dd[threadIdx.x - 64] = dh[t + threadIdx.x - 64];
        __syncthreads();
        f32x16_t sa, pa;
#pragma unroll
        for (int v2 = 0; v2 < 16; ++v2) sa[v2] = pa[v2] = 0.0f;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const u32x4_t aq = *reinterpret_cast<const u32x4_t*>(&sm.q.nat[32 * qr + col][16 * s + 8 * hl]);
            const u32x4_t ao = *reinterpret_cast<const u32x4_t*>(&sm.o.nat[32 * qr + col][16 * s + 8 * hl]);
            sa = mfma32(aq, kb[s], sa);
            pa = mfma32(ao, vb[s], pa);
        }
        // rows of register v: 32*qr + 8*(v/4) + 4*hl + v%4
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4 l4 = *reinterpret_cast<const float4*>(&sm.l2[32 * qr + 8 * g + 4 * hl]);
            const float4 d4 = *reinterpret_cast<const float4*>(&sm.dd[32 * qr + 8 * g + 4 * hl]);
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
            const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = exp2f(sa[4 * g + r] * scale_log2 - lv[r]);
                sa[4 * g + r] = p;
                pa[4 * g + r] = p * (pa[4 * g + r] - dv4[r]);   // dS
            }
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const u32x4_t bp = pack_kstep(sa, s2);
            const u32x4_t bs = pack_kstep(pa, s2);
#pragma unroll
            for (int m = 0; m < DM; ++m) {
                av[m] = mfma32(tr_operand<D>(sm.o, 32 * m + col, 32 * qr + 16 * s2, hl), bp, av[m]);
                ak[m] = mfma32(tr_operand<D>(sm.q, 32 * m + col, 32 * qr + 16 * s2, hl), bs, ak[m]);
            }
        }
    }
    // sum the two row halves: qr = 1 hands its partials to qr = 0
    __syncthreads();
    float* red = reinterpret_cast<float*>(&sm);
    const int slot = kr * 64 + lane;
    constexpr int PER = 32 * DM + 1;   // odd stride: lanes land in distinct banks
    if (qr == 1) {
#pragma unroll
        for (int m = 0; m < DM; ++m)
#pragma unroll
            for (int v2 = 0; v2 < 16; ++v2) {
                red[slot * PER + 16 * m + v2] = ak[m][v2];
                red[slot * PER + 16 * DM + 16 * m + v2] = av[m][v2];
            }
    }
    __syncthreads();
    if (qr == 0) {
        uint16_t* ko = dk + key * ld + h * hs;
        uint16_t* vo = dv + key * ld + h * hs;
#pragma unroll
        for (int m = 0; m < DM; ++m)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float xk[4], xv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    xk[r] = (ak[m][4 * g + r] + red[slot * PER + 16 * m + 4 * g + r]) * scale;
                    xv[r] = av[m][4 * g + r] + red[slot * PER + 16 * DM + 16 * m + 4 * g + r];
                }
                const int dcol = 32 * m + 8 * g + 4 * hl;
                *reinterpret_cast<u32x2_t*>(ko + dcol) = u32x2_t{pack2(xk[0], xk[1]), pack2(xk[2], xk[3])};
                *reinterpret_cast<u32x2_t*>(vo + dcol) = u32x2_t{pack2(xv[0], xv[1]), pack2(xv[2], xv[3])};
            }
    }
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
    if (d == 128) {
        hipLaunchKernelGGL(attn_dq_mfma_kernel<128>, grid, dim3(256), 0, s, Q, K, V, O, lse, Dq,
                           static_cast<uint16_t*>(dq), N, heads, ld, hs, offs, nb, so, si, cap, sl2, scale);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(attn_dkdv_mfma_kernel<128>, grid, dim3(256), 0, s, Q, K, V, O, lse, Dq,
                           static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), N, heads, ld, hs, offs, nb, to, ti,
                           cap, sl2, scale);
    } else {
        hipLaunchKernelGGL(attn_dq_mfma_kernel<64>, grid, dim3(256), 0, s, Q, K, V, O, lse, Dq,
                           static_cast<uint16_t*>(dq), N, heads, ld, hs, offs, nb, so, si, cap, sl2, scale);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(attn_dkdv_mfma_kernel<64>, grid, dim3(256), 0, s, Q, K, V, O, lse, Dq,
                           static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), N, heads, ld, hs, offs, nb, to, ti,
                           cap, sl2, scale);
    }
    return hipGetLastError();
}

hipError_t launch_attn_fwd_mfma(const void* q, const void* k, const void* v, void* o, float* lse, int64_t N, int heads,
                                int d, int64_t ld, int64_t hs, const int32_t* offs, int nb, const int32_t* so,
                                const int32_t* si, int64_t cap, float scale, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(N / 64 * heads));
    const float sl2 = scale * kLog2e;
    if (d == 128)
        hipLaunchKernelGGL(attn_fwd_mfma_kernel<128>, grid, dim3(256), 0, s, static_cast<const uint16_t*>(q),
                           static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o),
                           lse, N, heads, ld, hs, offs, nb, so, si, cap, sl2);
    else
        hipLaunchKernelGGL(attn_fwd_mfma_kernel<64>, grid, dim3(256), 0, s, static_cast<const uint16_t*>(q),
                           static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o),
                           lse, N, heads, ld, hs, offs, nb, so, si, cap, sl2);
    return hipGetLastError();
}

}  // namespace prism

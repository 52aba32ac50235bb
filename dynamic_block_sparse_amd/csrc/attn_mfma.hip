// attn_mfma.hip - block-sparse flash attention on gfx950 bf16 MFMA.
//
// Exact attention over the selected key blocks only, with an online softmax
// (Prism reading guide, xyznot.com paper 2610.05416, "Phương pháp" §3), and
// its gradient with the selection held constant.
//
// Every block is 1, 2 or 4 64-token tiles after the block-major permutation,
// and all rows of a block share its selected set, so the unit of work is a
// 64-row tile against the 64-key tiles of the selected blocks.
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
#include "prism_device.hpp"
#include "prism_internal.hpp"

namespace prism {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((__vector_size__(8)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

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

__device__ __forceinline__ u32x4_t lds_read16(const uint16_t* p) { return *reinterpret_cast<const u32x4_t*>(p); }

// A operand for a reduction over the rows of a row-major LDS tile `nat`
// (row stride NS elements): output rows are the tile's columns col0 .. col0+31,
// and the 16-row k-step starting at `base` is read in the permuted order that
// matches pack_kstep (rows base + 4h + 0..3, then base + 8 + 4h + 0..3).
template <int NS>
__device__ __forceinline__ u32x4_t tr_operand(const uint16_t* nat, int base, int col0, int lane) {
    const int g = lane >> 4, sl = lane & 15;
    const int row = base + 4 * (g >> 1) + (sl >> 2);
    const int col = col0 + 16 * (g & 1) + 4 * (sl & 3);
    const uint16_t* p = nat + row * NS + col;
    const s16x4_t r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
    const s16x4_t r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p + 8 * NS));
    const u32x2_t a = __builtin_bit_cast(u32x2_t, r1);
    const u32x2_t b = __builtin_bit_cast(u32x2_t, r2);
    return u32x4_t{a.x, a.y, b.x, b.y};
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
// 4 waves per 64-row query tile.  Each iteration stages two 64-key tiles of K
// and V (row-major) in LDS; wave w takes query rows 32*(w & 1) against key
// tile w >> 1 with its own online-softmax state; the two key halves are
// merged at the end.  Scores are computed transposed, S^T = K Q^T, so a lane
// owns one query row: its max and sum need one cross-lane swap and the O^T
// rescale is a per-lane scalar.

template <int D>
struct FwdSmem {
    static constexpr int NS = D + 8;   // row stride: 16-byte aligned, conflict-free 16-byte row reads
    uint16_t k[2][64][NS];
    uint16_t v[2][64][NS];
};

template <int D>
struct FwdStage {
    static constexpr int CPR = D / 8;                // 16-byte chunks per row
    static constexpr int RPP = 256 / CPR;            // rows covered per pass by the 256 threads
    static constexpr int PASSES = 64 / RPP;          // passes per tile
    u32x4_t r[4 * PASSES];                           // [tensor K/V][tile 0/1][pass]
};

template <int D>
__global__ void __launch_bounds__(256, 2)
attn_fwd_mfma_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                     uint16_t* __restrict__ o, float* __restrict__ lse, int64_t N, int64_t ld, int64_t hs,
                     const int32_t* __restrict__ offs, int nb, const int32_t* __restrict__ sel_off,
                     const int32_t* __restrict__ sel_idx, int64_t cap, float scale_log2) {
    using S = FwdStage<D>;
    constexpr int NS = FwdSmem<D>::NS;
    __shared__ FwdSmem<D> sm;
    const int ntiles = static_cast<int>(N / 64);
    const int wg = xcd_remap(blockIdx.x);
    const int h = wg / ntiles;
    const int64_t p0 = static_cast<int64_t>(wg % ntiles) * 64;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int rh = wave & 1, kh = wave >> 1;
    const int hl = lane >> 5, col = lane & 31;
    const int i = find_block(offs, nb, p0);
    const uint16_t* __restrict__ kh_ = k + h * hs;
    const uint16_t* __restrict__ vh_ = v + h * hs;
    const int32_t* __restrict__ so = sel_off + static_cast<int64_t>(h) * (nb + 1);
    const int32_t* __restrict__ si = sel_idx + static_cast<int64_t>(h) * cap;
    const int e0 = so[i];
    const int e1 = static_cast<int>(min(static_cast<int64_t>(so[i + 1]), cap));

    // staging: thread owns 16-byte column chunk sc of rows sr + RPP*pass
    const int sc = threadIdx.x % S::CPR, sr = threadIdx.x / S::CPR;
    int64_t goff[S::PASSES];
#pragma unroll
    for (int ps = 0; ps < S::PASSES; ++ps) goff[ps] = static_cast<int64_t>(sr + S::RPP * ps) * ld + sc * 8;

    constexpr int KS = D / 16, DM = D / 32;
    u32x4_t qb[KS];
    {
        const uint16_t* qrow = q + (p0 + 32 * rh + col) * ld + h * hs;
#pragma unroll
        for (int s = 0; s < KS; ++s) qb[s] = *reinterpret_cast<const u32x4_t*>(qrow + 16 * s + 8 * hl);
    }
    f32x16_t oacc[DM];
#pragma unroll
    for (int m = 0; m < DM; ++m)
#pragma unroll
        for (int x = 0; x < 16; ++x) oacc[m][x] = 0.0f;
    float mrow = -INFINITY, lrow = 0.0f;

    TileCursor cur;
    cur.init(si, offs, e0, e1);
    S st;
    auto load = [&](int t0, int t1) {
#pragma unroll
        for (int tl = 0; tl < 2; ++tl) {
            const int t = tl ? t1 : t0;
            if (t < 0) continue;
            const uint16_t* kb = kh_ + static_cast<int64_t>(t) * ld;
            const uint16_t* vb = vh_ + static_cast<int64_t>(t) * ld;
#pragma unroll
            for (int ps = 0; ps < S::PASSES; ++ps) {
                st.r[(0 * 2 + tl) * S::PASSES + ps] = *reinterpret_cast<const u32x4_t*>(kb + goff[ps]);
                st.r[(1 * 2 + tl) * S::PASSES + ps] = *reinterpret_cast<const u32x4_t*>(vb + goff[ps]);
            }
        }
    };
    int t0 = cur.next();
    int t1 = cur.next();
    load(t0, t1);
    while (t0 >= 0) {
        const bool has1 = t1 >= 0;
        __syncthreads();
#pragma unroll
        for (int tl = 0; tl < 2; ++tl) {
            if (tl == 1 && !has1) continue;
#pragma unroll
            for (int ps = 0; ps < S::PASSES; ++ps) {
                *reinterpret_cast<u32x4_t*>(&sm.k[tl][sr + S::RPP * ps][sc * 8]) = st.r[(0 * 2 + tl) * S::PASSES + ps];
                *reinterpret_cast<u32x4_t*>(&sm.v[tl][sr + S::RPP * ps][sc * 8]) = st.r[(1 * 2 + tl) * S::PASSES + ps];
            }
        }
        __syncthreads();
        const int n0 = cur.next();
        const int n1 = n0 >= 0 ? cur.next() : -1;
        if (n0 >= 0) load(n0, n1);
        if (kh == 0 || has1) {
            const uint16_t* kt = &sm.k[kh][0][0];
            const uint16_t* vt = &sm.v[kh][0][0];
            f32x16_t s0, s1;
#pragma unroll
            for (int x = 0; x < 16; ++x) s0[x] = s1[x] = 0.0f;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                s0 = mfma32(lds_read16(kt + col * NS + 16 * s + 8 * hl), qb[s], s0);
                s1 = mfma32(lds_read16(kt + (32 + col) * NS + 16 * s + 8 * hl), qb[s], s1);
            }
            float mx = -INFINITY;
#pragma unroll
            for (int x = 0; x < 16; ++x) mx = fmaxf(mx, fmaxf(s0[x], s1[x]));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * scale_log2;
            const float mnew = fmaxf(mrow, mx);
            const float alpha = fast_exp2(mrow - mnew);
            mrow = mnew;
            float ls = 0.0f;
#pragma unroll
            for (int x = 0; x < 16; ++x) {
                s0[x] = fast_exp2(fmaf(s0[x], scale_log2, -mnew));
                s1[x] = fast_exp2(fmaf(s1[x], scale_log2, -mnew));
                ls += s0[x] + s1[x];
            }
            lrow = fmaf(lrow, alpha, ls);
#pragma unroll
            for (int m = 0; m < DM; ++m)
#pragma unroll
                for (int x = 0; x < 16; ++x) oacc[m][x] *= alpha;
            const u32x4_t pb[4] = {pack_kstep(s0, 0), pack_kstep(s0, 1), pack_kstep(s1, 0), pack_kstep(s1, 1)};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int m = 0; m < DM; ++m) oacc[m] = mfma32(tr_operand<NS>(vt, 16 * ks, 32 * m, lane), pb[ks], oacc[m]);
        }
        t0 = n0;
        t1 = n1;
    }
    // merge the two key halves (waves kh = 1 hand their state to kh = 0)
    __syncthreads();
    float* red = reinterpret_cast<float*>(&sm);
    constexpr int PER = 3 + 16 * DM;   // odd stride: lanes land in distinct banks
    const int slot = rh * 64 + lane;
    if (kh == 1) {
        float* dst = red + slot * PER;
        dst[0] = mrow;
        dst[1] = lrow;
#pragma unroll
        for (int m = 0; m < DM; ++m)
#pragma unroll
            for (int x = 0; x < 16; ++x) dst[2 + 16 * m + x] = oacc[m][x];
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
                *reinterpret_cast<u32x2_t*>(orow + 32 * m + 8 * g + 4 * hl) = u32x2_t{pack2(x[0], x[1]), pack2(x[2], x[3])};
            }
        if (hl == 0) lse[static_cast<int64_t>(h) * N + row] = (mt + __log2f(lt)) * kLn2;
    }
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
struct BwdTile {
    static constexpr int NS = D + 8;
    uint16_t a[64][NS];
    uint16_t b[64][NS];
};

// Stage rows t .. t+63 of x and y (same strides) into tile.a / tile.b with the
// 128 threads of the workgroup, 16-byte chunks, consecutive threads on
// consecutive chunks of a row.
template <int D>
__device__ __forceinline__ void stage2(BwdTile<D>& tl, const uint16_t* __restrict__ x, const uint16_t* __restrict__ y,
                                       int64_t ld, int t) {
    constexpr int CPR = D / 8, RPP = 128 / CPR, PASSES = 64 / RPP;
    const int sc = threadIdx.x % CPR, sr = threadIdx.x / CPR;
    u32x4_t ra[PASSES], rb[PASSES];
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
        const int64_t off = static_cast<int64_t>(t + sr + RPP * ps) * ld + sc * 8;
        ra[ps] = *reinterpret_cast<const u32x4_t*>(x + off);
        rb[ps] = *reinterpret_cast<const u32x4_t*>(y + off);
    }
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
        *reinterpret_cast<u32x4_t*>(&tl.a[sr + RPP * ps][sc * 8]) = ra[ps];
        *reinterpret_cast<u32x4_t*>(&tl.b[sr + RPP * ps][sc * 8]) = rb[ps];
    }
}

template <int D>
__global__ void __launch_bounds__(128, 2)
attn_dq_mfma_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ Dq,
                    uint16_t* __restrict__ dq, int64_t N, int64_t ld, int64_t hs, const int32_t* __restrict__ offs,
                    int nb, const int32_t* __restrict__ sel_off, const int32_t* __restrict__ sel_idx, int64_t cap,
                    float scale_log2, float scale) {
    constexpr int NS = BwdTile<D>::NS;
    __shared__ BwdTile<D> sm;     // a = K, b = V
    const int ntiles = static_cast<int>(N / 64);
    const int wg = xcd_remap(blockIdx.x);
    const int h = wg / ntiles;
    const int64_t p0 = static_cast<int64_t>(wg % ntiles) * 64;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
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
    f32x16_t acc[DM];
#pragma unroll
    for (int m = 0; m < DM; ++m)
#pragma unroll
        for (int x = 0; x < 16; ++x) acc[m][x] = 0.0f;
    const uint16_t* __restrict__ kh_ = k + h * hs;
    const uint16_t* __restrict__ vh_ = v + h * hs;
    TileCursor cur;
    cur.init(si, offs, e0, e1);
    for (int t = cur.next(); t >= 0; t = cur.next()) {
        __syncthreads();
        stage2<D>(sm, kh_, vh_, ld, t);
        __syncthreads();
        f32x16_t sa[2], pa[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int x = 0; x < 16; ++x) sa[mt][x] = pa[mt][x] = 0.0f;
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                sa[mt] = mfma32(lds_read16(&sm.a[32 * mt + col][16 * s + 8 * hl]), qb[s], sa[mt]);
                pa[mt] = mfma32(lds_read16(&sm.b[32 * mt + col][16 * s + 8 * hl]), db[s], pa[mt]);
            }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int x = 0; x < 16; ++x) {
                const float p = fast_exp2(fmaf(sa[mt][x], scale_log2, -lrow));
                sa[mt][x] = p * (pa[mt][x] - drow);     // dS^T
            }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const u32x4_t b = pack_kstep(sa[ks >> 1], ks & 1);
#pragma unroll
            for (int m = 0; m < DM; ++m) acc[m] = mfma32(tr_operand<NS>(&sm.a[0][0], 16 * ks, 32 * m, lane), b, acc[m]);
        }
    }
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
struct DkvSmem {
    BwdTile<D> t;      // a = Q, b = dO
    float l2[64];      // lse in log2 units
    float dd[64];      // D = rowsum(dO * O)
};

template <int D>
__global__ void __launch_bounds__(128)
attn_dkdv_mfma_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                      const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ Dq,
                      uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int64_t N, int64_t ld, int64_t hs,
                      const int32_t* __restrict__ offs, int nb, const int32_t* __restrict__ tr_off,
                      const int32_t* __restrict__ tr_idx, int64_t cap, float scale_log2, float scale) {
    constexpr int NS = BwdTile<D>::NS;
    __shared__ DkvSmem<D> sm;
    const int ntiles = static_cast<int>(N / 64);
    const int wg = xcd_remap(blockIdx.x);
    const int h = wg / ntiles;
    const int64_t k0 = static_cast<int64_t>(wg % ntiles) * 64;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
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
    TileCursor cur;
    cur.init(ti, offs, e0, e1);
    for (int t = cur.next(); t >= 0; t = cur.next()) {
        __syncthreads();
        stage2<D>(sm.t, qh_, oh_, ld, t);
        if (threadIdx.x < 64) sm.l2[threadIdx.x] = lh[t + threadIdx.x] * kLog2e;
        else sm.dd[threadIdx.x - 64] = dh[t + threadIdx.x - 64];
        __syncthreads();
        f32x16_t sa[2], pa[2];
#pragma unroll
        for (int mr = 0; mr < 2; ++mr)
#pragma unroll
            for (int x = 0; x < 16; ++x) sa[mr][x] = pa[mr][x] = 0.0f;
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int mr = 0; mr < 2; ++mr) {
                sa[mr] = mfma32(lds_read16(&sm.t.a[32 * mr + col][16 * s + 8 * hl]), kb[s], sa[mr]);
                pa[mr] = mfma32(lds_read16(&sm.t.b[32 * mr + col][16 * s + 8 * hl]), vb[s], pa[mr]);
            }
        // register x of row tile mr holds query row 32*mr + 8*(x/4) + 4*hl + x%4
#pragma unroll
        for (int mr = 0; mr < 2; ++mr)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 l4 = *reinterpret_cast<const float4*>(&sm.l2[32 * mr + 8 * g + 4 * hl]);
                const float4 d4 = *reinterpret_cast<const float4*>(&sm.dd[32 * mr + 8 * g + 4 * hl]);
                const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
                const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float p = fast_exp2(fmaf(sa[mr][4 * g + r], scale_log2, -lv[r]));
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
                av[m] = mfma32(tr_operand<NS>(&sm.t.b[0][0], 16 * ks, 32 * m, lane), bp, av[m]);
                ak[m] = mfma32(tr_operand<NS>(&sm.t.a[0][0], 16 * ks, 32 * m, lane), bs, ak[m]);
            }
        }
    }
    uint16_t* ko = dk + key * ld + h * hs;
    uint16_t* vo = dv + key * ld + h * hs;
#pragma unroll
    for (int m = 0; m < DM; ++m)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x16_t& a = ak[m];
            const f32x16_t& b = av[m];
            const int dcol = 32 * m + 8 * g + 4 * hl;
            *reinterpret_cast<u32x2_t*>(ko + dcol) =
                u32x2_t{pack2(a[4 * g] * scale, a[4 * g + 1] * scale), pack2(a[4 * g + 2] * scale, a[4 * g + 3] * scale)};
            *reinterpret_cast<u32x2_t*>(vo + dcol) =
                u32x2_t{pack2(b[4 * g], b[4 * g + 1]), pack2(b[4 * g + 2], b[4 * g + 3])};
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
        hipLaunchKernelGGL(attn_fwd_mfma_kernel<128>, grid, dim3(256), 0, s, Q, K, V, O, lse, N, ld, hs, offs, nb, so,
                           si, cap, sl2);
    else
        hipLaunchKernelGGL(attn_fwd_mfma_kernel<64>, grid, dim3(256), 0, s, Q, K, V, O, lse, N, ld, hs, offs, nb, so,
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

// select.hip - pooled block scores and hybrid Top-k U Top-p key-block
// selection (Prism reading guide, xyznot.com paper 2610.05416, "Phương pháp"
// §3: key blocks are mean-pooled, scored against query blocks into block
// probabilities P_i, and S_i = Top-k(P_i, k) U Top-p(P_i, p)).
//
// Kernels, in launch order:
//   pool_kernel          float64 block means of Q and K per head (16-byte
//                        loads; sums of at most 256 bf16 values of moderate
//                        range are exact in float64, whatever the order)
//   logits_kernel        L[h][i][j] = fl32(scale * (Q_bar_i . K_bar_j)), the dot in
//                        float64 on MFMA: the scores are rounded once, so they
//                        equal the float64 definition's nearest float up to
//                        rare one-ulp differences from the summation order
//   select_reg_kernel    per row (up to 16384 blocks): the row's order-
//                        preserving 32-bit score keys and their softmax masses
//                        (float64 exp, as 2^-48 fixed-point integers) are held
//                        in registers; a (count, mass) histogram over 256
//                        score buckets finds the bucket of the boundary of the
//                        first max(k, n_p) ranked blocks, and a binary search
//                        over that bucket's keys finds the boundary; ties at
//                        it are resolved by index.
//                        No sort: the union of the two prefixes is one prefix
//                        of the ranking, so only its boundary matters.
//   select_count_kernel  the same result for longer rows, keys in LDS, by a
//                        4-pass radix select over (count, mass) histograms.
//   csr_scan_kernel      per head exclusive scan of the row counts
//   select_write_kernel  per row: ordered compaction of the selected indices
// and, for the backward, the transposed CSR (key block -> query blocks):
//   tr_count_kernel, csr_scan_kernel, tr_fill_kernel, tr_sort_kernel.
#include <algorithm>
#include <cstdlib>

#include "prism_device.hpp"
#include "prism_internal.hpp"

namespace prism {

// ---------------------------------------------------------------- pooling

template <typename TIn>
__device__ __forceinline__ double load_as_double(const TIn* p);
template <>
__device__ __forceinline__ double load_as_double<uint16_t>(const uint16_t* p) {
    return static_cast<double>(bf16_to_f32(*p));
}
template <>
__device__ __forceinline__ double load_as_double<float>(const float* p) {
    return static_cast<double>(*p);
}

// grid (nb, heads, 2): z = 0 pools q, z = 1 pools k.  Each lane loads 16
// bytes (EPV channels) of a row; the 256 threads cover RPS rows at a time and
// keep float64 partial sums, which are then added over the RPS row slots in
// slot order.
template <typename TIn, int D>
__global__ void __launch_bounds__(256)
pool_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k, int64_t ld, int64_t hs,
            const int32_t* __restrict__ offs, int nb, int heads, double* __restrict__ pooled) {
    constexpr int EPV = 16 / static_cast<int>(sizeof(TIn));   // channels per lane
    constexpr int LPR = D / EPV;                                // lanes per row
    constexpr int RPS = 256 / LPR;                              // rows per step
    __shared__ double part[RPS][D];
    const int i = blockIdx.x, h = blockIdx.y, which = blockIdx.z;
    const TIn* __restrict__ x = (which == 0 ? q : k) + static_cast<int64_t>(h) * hs;
    const int slot = threadIdx.x / LPR, cv = threadIdx.x % LPR;
    const int r0 = offs[i], r1 = offs[i + 1];
    double acc[EPV];
#pragma unroll
    for (int e = 0; e < EPV; ++e) acc[e] = 0.0;
    for (int r = r0 + slot; r < r1; r += RPS) {
        const uint4 u = *reinterpret_cast<const uint4*>(x + static_cast<int64_t>(r) * ld + cv * EPV);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
        if constexpr (EPV == 8) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] += static_cast<double>(bf16_to_f32(static_cast<uint16_t>(w[e] & 0xFFFFu)));
                acc[2 * e + 1] += static_cast<double>(bf16_to_f32(static_cast<uint16_t>(w[e] >> 16)));
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += static_cast<double>(__uint_as_float(w[e]));
        }
    }
#pragma unroll
    for (int e = 0; e < EPV; ++e) part[slot][cv * EPV + e] = acc[e];
    __syncthreads();
    for (int c = threadIdx.x; c < D; c += 256) {
        double t = part[0][c];
        for (int g = 1; g < RPS; ++g) t += part[g][c];
        pooled[((static_cast<int64_t>(which) * heads + h) * nb + i) * D + c] = t / static_cast<double>(r1 - r0);
    }
}

// ---------------------------------------------------------------- scores

constexpr int kLT = 128;  // output tile (rows and columns)
constexpr int kLC = 16;   // channels per LDS chunk

typedef double d4_t __attribute__((ext_vector_type(4)));

// One workgroup per 128 x 128 tile of one head's scores, on float64 MFMA
// (v_mfma_f64_16x16x4f64; lane l holds A[l % 16][l / 16] and B[l / 16][l % 16],
// and register r of the result D[4 r + l / 16][l % 16], checked with a probe).
// Wave (wi, wj) computes the 64 x 64 sub-tile at (64 wi, 64 wj) as 4 x 4 MFMA
// tiles.  The pooled means are staged in LDS channel-major, 16 channels at a
// time.  Each score is rounded once to fp32 after the scale (TOut = float), or
// kept in float64 (TOut = double, the run-pair scores of sub-block scoring).
//
// Tiles are visited XCD-aware and grouped: the 1D grid is dealt to the 8 XCDs
// in contiguous ranges, and inside a head kLGroup rows of query tiles sweep the
// key tiles together, so each key tile's pooled means are read from L2 by the
// kLGroup workgroups that use it while it is resident.  (In plain row order,
// dealt round-robin, the 2K scores fetched 10.7 GB beyond L2 for 4.6 GB of
// output.)
constexpr int kLGroup = 8;
template <int D, typename TOut>
__global__ void __launch_bounds__(256, 2)
logits_kernel(const double* __restrict__ pq, const double* __restrict__ pk, int nb, double scale,
              TOut* __restrict__ logits) {
    __shared__ double Qs[kLC][kLT + 2];
    __shared__ double Ks[kLC][kLT + 2];
    const int nt = (nb + kLT - 1) / kLT;
    const int G = static_cast<int>(gridDim.x);
    const int w = G % 8 ? static_cast<int>(blockIdx.x)
                        : static_cast<int>(blockIdx.x % 8) * (G / 8) + static_cast<int>(blockIdx.x / 8);
    const int h = w / (nt * nt);
    const int u = w - h * nt * nt;
    const int per_group = kLGroup * nt;
    const int first = (u / per_group) * kLGroup;
    const int gsize = min(nt - first, kLGroup);
    const int ti = first + (u % per_group) % gsize;
    const int tj = (u % per_group) / gsize;
    const int i0 = ti * kLT, j0 = tj * kLT;
    const double* __restrict__ Qb = pq + static_cast<int64_t>(h) * nb * D;
    const double* __restrict__ Kb = pk + static_cast<int64_t>(h) * nb * D;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int wi = wave >> 1, wj = wave & 1;
    const int lr = lane & 15, lk = lane >> 4;
    d4_t acc[4][4];
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = d4_t{0.0, 0.0, 0.0, 0.0};
    // staging: thread t brings 8 channels (sc .. sc+7) of row t / 2 of each
    // operand; the next chunk's global loads are in flight while this one is used
    const int srow = threadIdx.x >> 1, sc = (threadIdx.x & 1) * 8;
    const int gi = i0 + srow, gj = j0 + srow;
    double qv[8], kv[8];
    auto fetch = [&](int c0) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const double2 q2 = gi < nb ? *reinterpret_cast<const double2*>(Qb + static_cast<int64_t>(gi) * D + c0 + sc + e)
                                       : double2{0.0, 0.0};
            const double2 k2 = gj < nb ? *reinterpret_cast<const double2*>(Kb + static_cast<int64_t>(gj) * D + c0 + sc + e)
                                       : double2{0.0, 0.0};
            qv[e] = q2.x;
            qv[e + 1] = q2.y;
            kv[e] = k2.x;
            kv[e + 1] = k2.y;
        }
    };
    fetch(0);
    for (int c0 = 0; c0 < D; c0 += kLC) {
        __syncthreads();   // the previous chunk has been read
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            Qs[sc + e][srow] = qv[e];
            Ks[sc + e][srow] = kv[e];
        }
        __syncthreads();
        if (c0 + kLC < D) fetch(c0 + kLC);
#pragma unroll
        for (int kk = 0; kk < kLC; kk += 4) {
            double av[4], bv[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) av[x] = Qs[kk + lk][64 * wi + 16 * x + lr];
#pragma unroll
            for (int y = 0; y < 4; ++y) bv[y] = Ks[kk + lk][64 * wj + 16 * y + lr];
#pragma unroll
            for (int x = 0; x < 4; ++x)
#pragma unroll
                for (int y = 0; y < 4; ++y) acc[x][y] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[x], bv[y], acc[x][y], 0, 0, 0);
        }
    }
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int oi = i0 + 64 * wi + 16 * x + 4 * r + lk;
            if (oi >= nb) continue;
#pragma unroll
            for (int y = 0; y < 4; ++y) {
                const int oj = j0 + 64 * wj + 16 * y + lr;
                if (oj < nb) logits[(static_cast<int64_t>(h) * nb + oi) * nb + oj] = static_cast<TOut>(scale * acc[x][y][r]);
            }
        }
}

// ---------------------------------------------------------------- sub-block scores
//
// Scoring variant (DFSAttn article, sub-block scoring): every block is cut
// into its consecutive 64-token runs (a block holds 1, 2 or 4 of them and
// starts at a multiple of 64 tokens), the runs are pooled like blocks and
// scored pairwise in float64 by logits_kernel<D, double>, and the score of
// block pair (i, j) is the log of the mean of exp over its run pairs.

__global__ void __launch_bounds__(256) run_offsets_kernel(int32_t* __restrict__ run_offs, int64_t nr) {
    const int64_t r = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (r <= nr) run_offs[r] = static_cast<int32_t>(r * 64);
}

// grid (nb, heads): one workgroup per query block, a thread per key block at a
// time.  S[h][a][b] holds scale * (Q_bar_a . K_bar_b) for runs a, b (nr x nr
// per head).  The pair maximum m is factored out; the exponentials are added
// over the key runs in order, each of them first over the query runs in order;
// the mean divides by the pair count; m + log(mean) is rounded once to fp32.
__global__ void __launch_bounds__(256)
subblock_reduce_kernel(const double* __restrict__ S, int64_t nr, const int32_t* __restrict__ offs, int nb,
                       float* __restrict__ logits) {
    const int i = blockIdx.x, h = blockIdx.y;
    const int a0 = offs[i] >> 6;
    const int na = (offs[i + 1] >> 6) - a0;
    const double* __restrict__ Sh = S + (static_cast<int64_t>(h) * nr + a0) * nr;
    float* __restrict__ out = logits + (static_cast<int64_t>(h) * nb + i) * nb;
    for (int j = threadIdx.x; j < nb; j += 256) {
        const int b0 = offs[j] >> 6;
        const int nbj = (offs[j + 1] >> 6) - b0;
        double m = -INFINITY;
        for (int b = 0; b < nbj; ++b)
            for (int a = 0; a < na; ++a) m = fmax(m, Sh[static_cast<int64_t>(a) * nr + b0 + b]);
        double tot = 0.0;
        for (int b = 0; b < nbj; ++b) {
            double cs = 0.0;
            for (int a = 0; a < na; ++a) cs += exp(Sh[static_cast<int64_t>(a) * nr + b0 + b] - m);
            tot += cs;
        }
        out[j] = static_cast<float>(m + log(tot / static_cast<double>(na * nbj)));
    }
}

// ---------------------------------------------------------------- selection

// Order-preserving key of a finite float (-0 is folded onto +0 so that equal
// scores compare equal); every finite value maps to a key >= 0x00800000.
__device__ __forceinline__ uint32_t score_key(float x) {
    uint32_t u = __float_as_uint(x == 0.0f ? 0.0f : x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Softmax mass of a score in fixed point: round(exp(L - M) * 2^48).  Each
// value is at most 2^48, so the sum of a row (at most 32768 blocks) fits in 64
// bits, and integer sums are exact in any order: histograms built with LDS
// atomics are deterministic.  The rounding moves a row's cumulative mass by at
// most nb * 2^-49 (< 6e-11 of the total).
__device__ __forceinline__ uint64_t mass_fixed(uint32_t key, double M) {
    return __double2ull_rn(exp(static_cast<double>(key_score(key)) - M) * 281474976710656.0);
}

constexpr int kSelThreads = 256;
constexpr int kBuckets = kSelThreads;   // score buckets of select_reg_kernel
constexpr float kBucketSpan = 40.0f;    // their span below the row maximum at most:
                                        // mass below max - 34.7 rounds to 0 (2^-48 units)

// One workgroup per (row i, head h).  The row's keys live in LDS; the boundary
// key of the kept prefix is found by a 4-pass radix select (8-bit digits, most
// significant first) over (count, mass) histograms: at each pass the boundary
// lies in the highest digit bucket b whose inclusive suffix (everything at or
// above b, plus everything above the current prefix) satisfies
//   count >= max(k, 1)  and  mass >= p * Z.
__global__ void __launch_bounds__(kSelThreads)
select_count_kernel(const float* __restrict__ logits, int nb, int top_k, double top_p, int32_t* __restrict__ row_count,
                    uint32_t* __restrict__ row_thr, int32_t* __restrict__ row_tie) {
    extern __shared__ uint32_t skey[];                 // nb keys
    __shared__ uint32_t hcnt[256];
    __shared__ unsigned long long hmass[256];
    __shared__ unsigned long long red64[kSelThreads / kWave];
    __shared__ uint32_t red32[kSelThreads / kWave];
    __shared__ uint32_t s_digit;
    __shared__ uint32_t s_cabove;
    __shared__ unsigned long long s_mabove;
    const int i = blockIdx.x, h = blockIdx.y;
    const int64_t row = static_cast<int64_t>(h) * nb + i;
    const float* __restrict__ L = logits + row * nb;
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;

    uint32_t kmax = 0;
    for (int j = threadIdx.x; j < nb; j += kSelThreads) {
        const uint32_t kk = score_key(L[j]);
        skey[j] = kk;
        kmax = kk > kmax ? kk : kmax;
    }
    kmax = block_max(kmax, red32);
    const double M = static_cast<double>(key_score(kmax));
    uint64_t z = 0;
    for (int j = threadIdx.x; j < nb; j += kSelThreads) z += mass_fixed(skey[j], M);
    z = block_sum(static_cast<unsigned long long>(z), red64);
    const double target = top_p * static_cast<double>(z);
    const int kk = top_k > 1 ? top_k : 1;    // the Top-p prefix holds at least one block

    int count;
    uint32_t thr;
    int tie;
    if (!(nb >= kk && static_cast<double>(z) >= target)) {
        count = nb;                            // no prefix qualifies: keep every block
        thr = 0u;
        tie = 0;
    } else {
        uint32_t prefix = 0, cabove = 0;
        uint64_t mabove = 0;
        uint32_t ceq = 0;
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            hcnt[threadIdx.x] = 0;             // 256 threads, 256 buckets
            hmass[threadIdx.x] = 0;
            __syncthreads();
            for (int j0 = 0; j0 < nb; j0 += kSelThreads) {
                const int j = j0 + threadIdx.x;
                uint32_t key = 0;
                bool act = false;
                if (j < nb) {
                    key = skey[j];
                    act = pass == 0 || (key >> (shift + 8)) == prefix;
                }
                const uint32_t dig = (key >> shift) & 255u;
                const uint64_t mf = act ? mass_fixed(key, M) : 0;
                if (pass == 0) {
                    // scores share few leading digits: sum equal digits across the
                    // wave first, one atomic per distinct digit
                    bool left = act;
                    while (true) {
                        const uint64_t bal = __ballot(left);
                        if (!bal) break;
                        const int leader = __ffsll(static_cast<unsigned long long>(bal)) - 1;
                        const uint32_t dl = __shfl(dig, leader, kWave);
                        const bool mine = left && dig == dl;
                        const unsigned long long sum = wave_sum(static_cast<unsigned long long>(mine ? mf : 0));
                        const int cnt = __popcll(__ballot(mine));
                        if (lane == leader) {
                            atomicAdd(&hcnt[dl], static_cast<uint32_t>(cnt));
                            atomicAdd(&hmass[dl], sum);
                        }
                        left = left && !mine;
                    }
                } else if (act) {
                    atomicAdd(&hcnt[dig], 1u);
                    atomicAdd(&hmass[dig], static_cast<unsigned long long>(mf));
                }
            }
            __syncthreads();
            if (wid == 0) {
                // lane l owns buckets 4l .. 4l+3; inclusive suffix sums from the top
                uint32_t c[4];
                unsigned long long m4[4];
                uint32_t tc = 0;
                unsigned long long tm = 0;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    c[r] = hcnt[4 * lane + r];
                    m4[r] = hmass[4 * lane + r];
                    tc += c[r];
                    tm += m4[r];
                }
                uint32_t sc = tc;
                unsigned long long sm = tm;
#pragma unroll
                for (int off = 1; off < kWave; off <<= 1) {
                    const uint32_t oc = __shfl_down(sc, off, kWave);
                    const unsigned long long om = __shfl_down(sm, off, kWave);
                    if (lane + off < kWave) {
                        sc += oc;
                        sm += om;
                    }
                }
                // sc, sm: everything in lanes >= this lane; walk down this lane's buckets
                uint32_t ec = sc - tc;
                unsigned long long em = sm - tm;
                int ntrue = 0;
#pragma unroll
                for (int r = 3; r >= 0; --r) {
                    const uint32_t ic = ec + c[r];
                    const unsigned long long im = em + m4[r];
                    const bool ok = cabove + ic >= static_cast<uint32_t>(kk) &&
                                    static_cast<double>(mabove + im) >= target;
                    ntrue += ok ? 1 : 0;
                    ec = ic;
                    em = im;
                }
                const int b = wave_sum(ntrue) - 1;   // predicate holds exactly on buckets 0..b
                if (lane == (b >> 2)) {
                    // everything strictly above bucket b
                    uint32_t xc = sc - tc;
                    unsigned long long xm = sm - tm;
                    for (int r = 3; r > (b & 3); --r) {
                        xc += c[r];
                        xm += m4[r];
                    }
                    s_digit = static_cast<uint32_t>(b);
                    s_cabove = xc;
                    s_mabove = xm;
                }
            }
            __syncthreads();
            const uint32_t b = s_digit;
            prefix = (prefix << 8) | b;
            cabove += s_cabove;
            mabove += s_mabove;
            ceq = hcnt[b];
            __syncthreads();
        }
        thr = prefix;
        // the boundary lies among the ceq ties of key thr, taken in index order
        const uint64_t eb = mass_fixed(thr, M);
        uint32_t m = 0;
        uint64_t acc = mabove;
        do {
            ++m;
            acc += eb;
        } while (m < ceq && !(cabove + m >= static_cast<uint32_t>(kk) && static_cast<double>(acc) >= target));
        count = static_cast<int>(cabove + m);
        tie = static_cast<int>(m);   // the first m ties in index order (select_write_kernel)
    }
    if (threadIdx.x == 0) {
        row_count[row] = count;
        row_thr[row] = thr;
        row_tie[row] = tie;
    }
}

// Wave-wide sums with DPP lane exchanges instead of LDS shuffles: two quad
// permutes and the half-row and row mirrors leave every lane holding the sum
// of its 16-lane row; the four row sums are then read out as scalars.  The
// 64-bit sum adds the 32-bit halves with carry, so it is exact.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_add_u64(unsigned long long v) {
    const uint32_t lo = dpp_u32<CTRL>(static_cast<uint32_t>(v));
    const uint32_t hi = dpp_u32<CTRL>(static_cast<uint32_t>(v >> 32));
    return v + ((static_cast<unsigned long long>(hi) << 32) | lo);
}
__device__ __forceinline__ uint32_t wave_sum_dpp(uint32_t v) {
    v += dpp_u32<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp_u32<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp_u32<0x141>(v);   // row_half_mirror
    v += dpp_u32<0x140>(v);   // row_mirror
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 0)) +
           static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 16)) +
           static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 32)) +
           static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 48));
}
__device__ __forceinline__ unsigned long long wave_sum_dpp(unsigned long long v) {
    v = dpp_add_u64<0xB1>(v);
    v = dpp_add_u64<0x4E>(v);
    v = dpp_add_u64<0x141>(v);
    v = dpp_add_u64<0x140>(v);
    unsigned long long t = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), 16 * r));
        const uint32_t hi =
            static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v >> 32)), 16 * r));
        t += (static_cast<unsigned long long>(hi) << 32) | lo;
    }
    return t;
}

// Sums over the workgroup of a (count, mass) pair; every thread gets the
// totals.  `slot` alternates between calls so that one barrier per call
// suffices: a slot is rewritten only after every thread has passed the
// barrier of the call in between, i.e. after it read the slot.
__device__ __forceinline__ void block_sum_cm(uint32_t& c, unsigned long long& m, uint32_t (*rc)[kSelThreads / kWave],
                                             unsigned long long (*rm)[kSelThreads / kWave], int& slot) {
    c = wave_sum_dpp(c);
    m = wave_sum_dpp(m);
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    if (lane == 0) {
        rc[slot][wid] = c;
        rm[slot][wid] = m;
    }
    __syncthreads();
    c = 0;
    m = 0;
#pragma unroll
    for (int w = 0; w < kSelThreads / kWave; ++w) {
        c += rc[slot][w];
        m += rm[slot][w];
    }
    slot ^= 1;
}

// Single-value forms of block_sum_cm (same slot discipline).
__device__ __forceinline__ uint32_t block_sum_c(uint32_t c, uint32_t (*rc)[kSelThreads / kWave], int& slot) {
    c = wave_sum_dpp(c);
    if ((threadIdx.x & (kWave - 1)) == 0) rc[slot][threadIdx.x / kWave] = c;
    __syncthreads();
    c = 0;
#pragma unroll
    for (int w = 0; w < kSelThreads / kWave; ++w) c += rc[slot][w];
    slot ^= 1;
    return c;
}
__device__ __forceinline__ unsigned long long block_sum_m(unsigned long long m,
                                                          unsigned long long (*rm)[kSelThreads / kWave], int& slot) {
    m = wave_sum_dpp(m);
    if ((threadIdx.x & (kWave - 1)) == 0) rm[slot][threadIdx.x / kWave] = m;
    __syncthreads();
    m = 0;
#pragma unroll
    for (int w = 0; w < kSelThreads / kWave; ++w) m += rm[slot][w];
    slot ^= 1;
    return m;
}

// One workgroup per (row i, head h); thread t holds blocks t + 256 e, e < E.
// The kept prefix is {key > u} plus the first ties of key u in index order,
// where u is the largest key value with count(key >= u) >= max(k, 1) and
// mass(key >= u) >= p * Z.  Both sums only grow as u falls: a histogram over
// score buckets finds the bucket that holds u, and a bisection over that
// bucket's keys alone finds u.
// (Registers capped so that four workgroups share a CU up to E = 32.)
template <int E>
__global__ void __launch_bounds__(kSelThreads, E <= 32 ? 4 : 2)
select_reg_kernel(const float* __restrict__ logits, int nb, int top_k, double top_p, int32_t* __restrict__ row_count,
                  uint32_t* __restrict__ row_thr, int32_t* __restrict__ row_tie) {
    __shared__ uint32_t red32[kSelThreads / kWave];
    __shared__ unsigned long long red64[kSelThreads / kWave];
    __shared__ uint32_t rc[2][kSelThreads / kWave];
    __shared__ unsigned long long rm[2][kSelThreads / kWave];
    __shared__ uint32_t ckey[kSelThreads];            // compacted undecided keys
    __shared__ unsigned long long cms[kSelThreads];   // and their masses
    __shared__ uint32_t ccnt, cres;
    __shared__ uint32_t hcnt[kBuckets];               // per score bucket: keys
    __shared__ unsigned long long hmass[kBuckets];    // and their mass
    __shared__ uint32_t s_bc, s_bn;
    __shared__ unsigned long long s_bm;
    const int i = blockIdx.x, h = blockIdx.y;
    const int64_t row = static_cast<int64_t>(h) * nb + i;
    const float* __restrict__ L = logits + row * nb;
    uint32_t key[E];
    hcnt[threadIdx.x] = 0u;   // kBuckets == kSelThreads: thread t owns bucket t
    hmass[threadIdx.x] = 0ull;
    uint32_t kmax = 0, nkmin = 0;   // nkmin = ~(smallest key)
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int j = threadIdx.x + kSelThreads * e;
        // padding key 0 lies below every finite score's key and is never counted
        key[e] = j < nb ? score_key(L[j]) : 0u;
        kmax = key[e] > kmax ? key[e] : kmax;
        nkmin = (j < nb && ~key[e] > nkmin) ? ~key[e] : nkmin;
    }
    kmax = block_max(kmax, red32);
    const uint32_t kmin = ~block_max(nkmin, red32);
    const double M = static_cast<double>(key_score(kmax));
    // Score buckets counted down from the maximum, of width span /
    // (kBuckets - 1), span = min(max - min, kBucketSpan); the last bucket also
    // takes everything deeper.  A bucket is an interval of keys (the map only
    // falls as the score grows).  Each key's mass goes to Z and to its
    // bucket's (count, mass); the masses are not kept.
    const float smax = key_score(kmax);
    const float span = fminf(smax - key_score(kmin), kBucketSpan);
    const float inv = span > 0.0f ? static_cast<float>(kBuckets - 1) / span : 0.0f;
    auto bucket_of = [&](uint32_t kv) -> int {
        const float t = (smax - key_score(kv)) * inv;
        return t < static_cast<float>(kBuckets - 1) ? static_cast<int>(t) : kBuckets - 1;
    };
    unsigned long long z = 0;
#pragma unroll
    for (int e = 0; e < E; ++e)
        if (key[e]) {
            const unsigned long long m = mass_fixed(key[e], M);
            const int b = bucket_of(key[e]);
            z += m;
            atomicAdd(&hcnt[b], 1u);
            if (m) atomicAdd(&hmass[b], m);
        }
    z = block_sum(z, red64);   // its barriers also complete the histogram
    const double target = top_p * static_cast<double>(z);
    const uint32_t kk = top_k > 1 ? static_cast<uint32_t>(top_k) : 1u;
    int count, tie;
    uint32_t thr;
    if (!(static_cast<uint32_t>(nb) >= kk && static_cast<double>(z) >= target)) {
        count = nb;                    // no prefix qualifies: keep every block
        thr = 0u;
        tie = 0;
    } else {
        int slot = 0;
        // Largest u in [lo, hi) whose suffix (keys >= u) satisfies the count
        // condition (by_count) or the mass condition, given that it holds at lo
        // and fails at hi.  Each step of the bisection sums over the whole row;
        // once at most kSelThreads keys lie in [lo, hi), they are compacted into
        // LDS and wave 0 finishes the search on them alone, adding the exact
        // (count, mass) of the keys at or above hi.  The sums are integers, so
        // the result does not depend on the order of the compacted keys.
        auto finish = [&](uint32_t lo, uint32_t hi, uint32_t bc, unsigned long long bm, bool by_count) -> uint32_t {
            if (threadIdx.x == 0) ccnt = 0u;
            __syncthreads();
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (key[e] >= lo && key[e] < hi) ckey[atomicAdd(&ccnt, 1u)] = key[e];
            __syncthreads();
            if (threadIdx.x < kWave) {
                // the candidates' masses are evaluated here, CPL per lane (not
                // in the compaction, whose per-key branches a whole wave runs)
                constexpr int CPL = kSelThreads / kWave;   // candidates per lane
                const uint32_t n = ccnt;
                uint32_t ck[CPL];
                unsigned long long cm[CPL];
#pragma unroll
                for (int x = 0; x < CPL; ++x) {
                    const uint32_t j = threadIdx.x + kWave * x;
                    ck[x] = j < n ? ckey[j] : 0u;   // key 0 lies below every finite score's key
                    cm[x] = (j < n && !by_count) ? mass_fixed(ck[x], M) : 0ull;
                }
                while (hi - lo > 1u) {
                    const uint32_t mid = lo + (hi - lo) / 2u;
                    bool ok;
                    if (by_count) {
                        uint32_t c = 0;
#pragma unroll
                        for (int x = 0; x < CPL; ++x) c += ck[x] >= mid ? 1u : 0u;
                        ok = bc + wave_sum_dpp(c) >= kk;
                    } else {
                        unsigned long long m = 0;
#pragma unroll
                        for (int x = 0; x < CPL; ++x) m += ck[x] >= mid ? cm[x] : 0ull;
                        ok = static_cast<double>(bm + wave_sum_dpp(m)) >= target;
                    }
                    if (ok) lo = mid;
                    else hi = mid;
                }
                if (threadIdx.x == 0) cres = lo;
            }
            __syncthreads();
            return cres;
        };
        // c_lo = count(key >= lo) and c_hi = count(key >= hi) are carried along,
        // so the number of keys still undecided is known without another pass;
        // m_hi = mass(key >= hi) when the mass condition is searched.
        auto search = [&](uint32_t lo, uint32_t hi, uint32_t c_lo, uint32_t c_hi, unsigned long long m_hi,
                          bool by_count) -> uint32_t {
            while (hi - lo > 1u) {
                if (c_lo - c_hi <= static_cast<uint32_t>(kSelThreads)) return finish(lo, hi, c_hi, m_hi, by_count);
                const uint32_t mid = lo + (hi - lo) / 2u;
                uint32_t c = 0;
                unsigned long long m = 0;
                bool ok;
                if (by_count) {
#pragma unroll
                    for (int e = 0; e < E; ++e) c += key[e] >= mid ? 1u : 0u;
                    c = block_sum_c(c, rc, slot);
                    ok = c >= kk;
                } else {
                    // the mass at or above hi is m_hi; the masses of the keys in
                    // [mid, hi) are evaluated again
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        c += key[e] >= mid ? 1u : 0u;
                        if (key[e] >= mid && key[e] < hi) m += mass_fixed(key[e], M);
                    }
                    block_sum_cm(c, m, rc, rm, slot);
                    m += m_hi;
                    ok = static_cast<double>(m) >= target;
                }
                if (ok) {
                    lo = mid;
                    c_lo = c;
                } else {
                    hi = mid;
                    c_hi = c;
                    m_hi = m;
                }
            }
            return lo;
        };
        // The boundary's bucket: the count and the mass of keys at or above a
        // bucket's lowest key are prefix sums over the buckets from the top.
        // The boundary u = min(u_count, u_mass) lies in the bucket b* where
        // the later of the two conditions first holds; keys in earlier buckets
        // are kept, keys in later ones are not, and the bisection runs only
        // over the keys of b* (search() starts with the counts at its ends).
        // inclusive prefix over the buckets: a wave scan, then the totals of
        // the waves below
        const int lane = threadIdx.x & (kWave - 1);
        const int wid = threadIdx.x / kWave;
        const uint32_t own_c = hcnt[threadIdx.x];
        const unsigned long long own_m = hmass[threadIdx.x];
        uint32_t pc = own_c;
        unsigned long long pm = own_m;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const uint32_t c = __shfl_up(pc, off, kWave);
            const unsigned long long m = __shfl_up(pm, off, kWave);
            if (lane >= off) {
                pc += c;
                pm += m;
            }
        }
        if (lane == kWave - 1) {
            rc[slot][wid] = pc;
            rm[slot][wid] = pm;
        }
        __syncthreads();
#pragma unroll
        for (int w = 0; w < kSelThreads / kWave; ++w)
            if (w < wid) {
                pc += rc[slot][w];
                pm += rm[slot][w];
            }
        slot ^= 1;
        // first bucket meeting each condition = the number of buckets that
        // miss it (both only become true along the buckets, and both hold at
        // the last bucket, which ends the row)
        uint32_t miss_c = pc >= kk ? 0u : 1u;
        unsigned long long miss_m = static_cast<double>(pm) >= target ? 0ull : 1ull;
        block_sum_cm(miss_c, miss_m, rc, rm, slot);
        const int b_c = static_cast<int>(miss_c), b_m = static_cast<int>(miss_m);
        const int bs = b_c > b_m ? b_c : b_m;
        if (static_cast<int>(threadIdx.x) == bs) {
            s_bc = pc - own_c;   // count and mass of the keys above the bucket
            s_bm = pm - own_m;
            s_bn = own_c;
        }
        // the bucket's lowest and highest keys
        uint32_t bmax = 0u, bnmin = 0u;
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (key[e] && bucket_of(key[e]) == bs) {
                bmax = key[e] > bmax ? key[e] : bmax;
                bnmin = ~key[e] > bnmin ? ~key[e] : bnmin;
            }
        bmax = block_max(bmax, red32);
        bnmin = block_max(bnmin, red32);   // its barriers also publish s_bc, s_bm, s_bn
        const uint32_t blo = ~bnmin, bhi = bmax + 1u;
        const uint32_t c_above = s_bc, n_b = s_bn;
        const unsigned long long m_above = s_bm;
        uint32_t lo = 0xFFFFFFFFu;
        if (b_c == bs) lo = search(blo, bhi, c_above + n_b, c_above, m_above, true);
        if (b_m == bs) {
            const uint32_t um = search(blo, bhi, c_above + n_b, c_above, m_above, false);
            lo = um < lo ? um : lo;
        }
        thr = lo;
        // blocks strictly above the boundary key, and the ties at it.  The
        // keys above b* hold m_above; the masses of the keys of b* above thr
        // are evaluated again, by wave 0 on the compacted keys when they fit.
        uint32_t cabove = 0, ceq = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            cabove += key[e] > thr ? 1u : 0u;
            ceq += key[e] == thr ? 1u : 0u;
        }
        {
            unsigned long long c64 = ceq;
            block_sum_cm(cabove, c64, rc, rm, slot);
            ceq = static_cast<uint32_t>(c64);
        }
        unsigned long long mabove = 0;
        if (cabove - c_above <= static_cast<uint32_t>(kSelThreads)) {
            if (threadIdx.x == 0) ccnt = 0u;
            __syncthreads();
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (key[e] > thr && key[e] < bhi) ckey[atomicAdd(&ccnt, 1u)] = key[e];
            __syncthreads();
            if (threadIdx.x < kWave) {
                const uint32_t n = ccnt;
                unsigned long long m = 0;
#pragma unroll
                for (int x = 0; x < kSelThreads / kWave; ++x) {
                    const uint32_t j = threadIdx.x + kWave * x;
                    m += j < n ? mass_fixed(ckey[j], M) : 0ull;
                }
                m = wave_sum_dpp(m);
                if (threadIdx.x == 0) cms[0] = m;
            }
            __syncthreads();
            mabove = cms[0];
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (key[e] > thr && key[e] < bhi) mabove += mass_fixed(key[e], M);
            mabove = block_sum_m(mabove, rm, slot);
        }
        mabove += m_above;
        const uint64_t eb = mass_fixed(thr, M);
        uint32_t m = 0;
        uint64_t acc = mabove;
        do {
            ++m;
            acc += eb;
        } while (m < ceq && !(cabove + m >= kk && static_cast<double>(acc) >= target));
        count = static_cast<int>(cabove + m);
        tie = static_cast<int>(m);   // the first m ties in index order (select_write_kernel)
    }
    if (threadIdx.x == 0) {
        row_count[row] = count;
        row_thr[row] = thr;
        row_tie[row] = tie;
    }
}

// exclusive scan of counts[h][0..n) into offsets[h][0..n]; totals[h] = sum
__global__ void __launch_bounds__(1024)
csr_scan_kernel(const int32_t* __restrict__ counts, int n, int32_t* __restrict__ offsets, int64_t* __restrict__ totals) {
    __shared__ int32_t buf[1024];
    __shared__ int64_t carry;
    const int h = blockIdx.x;
    const int32_t* __restrict__ c = counts + static_cast<int64_t>(h) * n;
    int32_t* __restrict__ o = offsets + static_cast<int64_t>(h) * (n + 1);
    if (threadIdx.x == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < n; base += 1024) {
        const int idx = base + threadIdx.x;
        const int32_t v = idx < n ? c[idx] : 0;
        buf[threadIdx.x] = v;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {
            const int32_t t = threadIdx.x >= off ? buf[threadIdx.x - off] : 0;
            __syncthreads();
            buf[threadIdx.x] += t;
            __syncthreads();
        }
        if (idx < n) o[idx] = static_cast<int32_t>(carry + buf[threadIdx.x] - v);
        __syncthreads();
        if (threadIdx.x == 1023) carry += buf[1023];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        o[n] = static_cast<int32_t>(carry);
        if (totals) totals[h] = carry;
    }
}

// The row is taken kWriteChunks chunks of NW*64 keys at a time: each thread
// has that many independent loads in flight, and one barrier per pass orders
// the chunks (the per-wave counts are double-buffered, so the next pass can
// write its counts while a slower wave still reads this pass's).  A block is
// kept if its key is above the row's boundary key, or equal to it and among
// the first `tie` such blocks in index order; the ties' ranks come from the
// same per-wave counts.
constexpr int kWriteChunks = 4;
template <int NW>
__global__ void __launch_bounds__(NW * 64)
select_write_kernel(const float* __restrict__ logits, int nb, const uint32_t* __restrict__ row_thr,
                    const int32_t* __restrict__ row_tie, const int32_t* __restrict__ sel_offsets,
                    int32_t* __restrict__ sel_idx, int64_t cap) {
    constexpr int NT = NW * 64;
    constexpr int U = kWriteChunks;
    __shared__ int sg[2][U * NW];   // keys above the boundary, per chunk and wave
    __shared__ int st[2][U * NW];   // keys equal to it
    const int i = blockIdx.x, h = blockIdx.y;
    const int64_t row = static_cast<int64_t>(h) * nb + i;
    const float* __restrict__ L = logits + row * nb;
    const uint32_t thr = row_thr[row];
    const int tie = row_tie[row];
    int64_t pos = sel_offsets[static_cast<int64_t>(h) * (nb + 1) + i];
    int32_t* __restrict__ out = sel_idx + static_cast<int64_t>(h) * cap;
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));   // lanes under this one
    int buf = 0;
    int tbase = 0;   // ties in earlier passes
    for (int base = 0; base < nb; base += U * NT) {
        float v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = base + u * NT + static_cast<int>(threadIdx.x);
            v[u] = j < nb ? L[j] : 0.0f;
        }
        bool g[U], t[U];
        uint64_t bt[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = base + u * NT + static_cast<int>(threadIdx.x);
            const uint32_t kk = score_key(v[u]);
            g[u] = j < nb && kk > thr;
            t[u] = j < nb && kk == thr;
            bt[u] = __ballot(t[u]);
            const uint64_t bg = __ballot(g[u]);
            if (lane == 0) {
                sg[buf][u * NW + wid] = __popcll(bg);
                st[buf][u * NW + wid] = __popcll(bt[u]);
            }
        }
        __syncthreads();
        // chunk u of wave w starts after every chunk before u and, inside u,
        // after the waves below w; of the ties of (u, w), those ranked below
        // `tie` in the row are kept
        int acc = 0, tacc = tbase, woff[U], toff[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const int ng = sg[buf][u * NW + w], nt = st[buf][u * NW + w];
                if (w == wid) {
                    woff[u] = acc;
                    toff[u] = tacc;
                }
                acc += ng + min(max(tie - tacc, 0), nt);
                tacc += nt;
            }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool f = g[u] || (t[u] && toff[u] + __popcll(bt[u] & below) < tie);
            const int before = __popcll(__ballot(f) & below);
            if (f) {
                const int64_t p = pos + woff[u] + before;
                if (p < cap) out[p] = base + u * NT + static_cast<int>(threadIdx.x);
            }
        }
        pos += acc;
        tbase = tacc;
        buf ^= 1;
    }
}

// ---------------------------------------------------------------- transposed CSR

__global__ void __launch_bounds__(256)
tr_count_kernel(const int32_t* __restrict__ sel_offsets, const int32_t* __restrict__ sel_idx, int nb, int64_t cap,
                const uint8_t* __restrict__ rowmask, int want, int32_t* __restrict__ tcount) {
    const int i = blockIdx.x, h = blockIdx.y;
    if (rowmask && (rowmask[static_cast<int64_t>(h) * nb + i] != 0) != (want != 0)) return;
    const int32_t* __restrict__ so = sel_offsets + static_cast<int64_t>(h) * (nb + 1);
    const int32_t* __restrict__ si = sel_idx + static_cast<int64_t>(h) * cap;
    const int64_t e1 = min(static_cast<int64_t>(so[i + 1]), cap);   // a truncated list stops at cap
    for (int64_t e = so[i] + threadIdx.x; e < e1; e += blockDim.x)
        atomicAdd(&tcount[static_cast<int64_t>(h) * nb + si[e]], 1);
}

__global__ void __launch_bounds__(256)
tr_fill_kernel(const int32_t* __restrict__ sel_offsets, const int32_t* __restrict__ sel_idx, int nb, int64_t cap,
               const uint8_t* __restrict__ rowmask, int want, const int32_t* __restrict__ tr_offsets,
               int32_t* __restrict__ tcursor, int32_t* __restrict__ tr_idx) {
    const int i = blockIdx.x, h = blockIdx.y;
    if (rowmask && (rowmask[static_cast<int64_t>(h) * nb + i] != 0) != (want != 0)) return;
    const int32_t* __restrict__ so = sel_offsets + static_cast<int64_t>(h) * (nb + 1);
    const int32_t* __restrict__ si = sel_idx + static_cast<int64_t>(h) * cap;
    const int32_t* __restrict__ to = tr_offsets + static_cast<int64_t>(h) * (nb + 1);
    const int64_t e1 = min(static_cast<int64_t>(so[i + 1]), cap);
    for (int64_t e = so[i] + threadIdx.x; e < e1; e += blockDim.x) {
        const int j = si[e];
        const int slot = atomicAdd(&tcursor[static_cast<int64_t>(h) * nb + j], 1);
        tr_idx[static_cast<int64_t>(h) * cap + to[j] + slot] = i;
    }
}

// Sort one key block's list of query blocks ascending (the fill order depends
// on atomics; the backward reads the lists in ascending order so that its
// sums are deterministic).  Entries are distinct, so the rank of an entry is
// the number of smaller entries.
constexpr int kSortLds = 8192;
__global__ void __launch_bounds__(256)
tr_sort_kernel(const int32_t* __restrict__ tr_offsets, int nb, int64_t cap, int32_t* __restrict__ tr_idx,
               int32_t* __restrict__ scratch) {
    __shared__ int32_t seg[kSortLds];
    const int j = blockIdx.x, h = blockIdx.y;
    const int32_t* __restrict__ to = tr_offsets + static_cast<int64_t>(h) * (nb + 1);
    const int64_t b = to[j], n = to[j + 1] - to[j];
    if (n <= 1) return;
    int32_t* __restrict__ list = tr_idx + static_cast<int64_t>(h) * cap + b;
    if (n <= kSortLds) {
        for (int64_t e = threadIdx.x; e < n; e += blockDim.x) seg[e] = list[e];
        __syncthreads();
        for (int64_t e = threadIdx.x; e < n; e += blockDim.x) {
            const int32_t v = seg[e];
            int r = 0;
            for (int64_t f = 0; f < n; ++f) r += seg[f] < v ? 1 : 0;
            list[r] = v;
        }
    } else {
        // long list: rank against a copy in the scratch area (same offsets)
        int32_t* __restrict__ cp = scratch + static_cast<int64_t>(h) * cap + b;
        for (int64_t e = threadIdx.x; e < n; e += blockDim.x) cp[e] = list[e];
        __syncthreads();
        for (int64_t e = threadIdx.x; e < n; e += blockDim.x) {
            const int32_t v = cp[e];
            int r = 0;
            for (int64_t f = 0; f < n; ++f) r += cp[f] < v ? 1 : 0;
            list[r] = v;
        }
    }
}

// ---------------------------------------------------------------- tile visiting order
//
// The attention kernels stream, per 64-row tile, the key tiles that its block
// selected, in ascending block order.  Visiting the query tiles grouped by
// the first block they select lets the workgroups that run at the same time
// on one XCD start on the same key tiles and share them in L2 (at 2K the
// forward gains 6%).  The order only changes timing: every tile's result is
// accumulated in its own fixed order, so the outputs are the same bits under
// any order.  Tiles of equal key keep their launch order (a stable counting
// sort), so the order itself is deterministic too.

__global__ void __launch_bounds__(256) fill_i32_kernel(int32_t* __restrict__ p, int64_t n, int32_t v) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256)
        p[i] = v;
}

__device__ __forceinline__ int first_selected(const int32_t* __restrict__ so, const int32_t* __restrict__ si,
                                              int64_t cap, int i) {
    const int64_t e0 = so[i], e1 = min(static_cast<int64_t>(so[i + 1]), cap);
    return e0 < e1 ? si[e0] : 0;
}

__device__ __forceinline__ int order_key(const int32_t* __restrict__ so, const int32_t* __restrict__ si, int64_t cap,
                                         int i, int nb) {
    const int key = first_selected(so, si, cap, i);
    return key >= 0 && key < nb ? key : 0;
}

// The sort is done within units: the intersections of a head with one XCD's
// contiguous range of the launch order (the attention kernels deal positions
// [x G/8, (x+1) G/8) to XCD x).  Each XCD therefore keeps the tiles, and so the
// work, that raster order gives it; only their order within its range changes.
// (Sorting a whole head at once moved the selections' heavy, diffuse tiles into
// one XCD's range when a launch held a single head: 2.4x slower on a
// 1,105,920-token clip.)  Along the launch order neither the head nor the range
// index decreases, so unit = head + range index names each unit once.
__device__ __forceinline__ void tile_unit(int h, int t, int64_t ntiles, int64_t seg, int& unit, int64_t& base) {
    const int64_t p = static_cast<int64_t>(h) * ntiles + t;
    const int64_t r = p / seg;
    unit = h + static_cast<int>(r);
    base = max(static_cast<int64_t>(h) * ntiles, r * seg);
}

// bucket[unit][key] += 1 for every tile, key = its block's first selected block
__global__ void __launch_bounds__(256)
order_count_kernel(const int32_t* __restrict__ sel_offsets, const int32_t* __restrict__ sel_idx, int64_t cap,
                   const int32_t* __restrict__ offs, int nb, int64_t ntiles, int64_t seg, int32_t* __restrict__ bucket,
                   int32_t* __restrict__ tkey) {
    const int i = blockIdx.x * 256 + threadIdx.x, h = blockIdx.y;
    if (i >= nb) return;
    const int32_t* so = sel_offsets + static_cast<int64_t>(h) * (nb + 1);
    const int32_t* si = sel_idx + static_cast<int64_t>(h) * cap;
    const int key = order_key(so, si, cap, i, nb);
    for (int t = offs[i] / 64; t < offs[i + 1] / 64; ++t) {
        int u;
        int64_t base;
        tile_unit(h, t, ntiles, seg, u, base);
        atomicAdd(&bucket[static_cast<int64_t>(u) * nb + key], 1);
        tkey[static_cast<int64_t>(h) * ntiles + t] = key;
    }
}

// order[base(unit) + start[unit][key] + slot] = tile, with the slots of one
// key in ascending tile order (a stable counting sort, so the visiting order is
// deterministic and keeps spatial order inside a key).  One workgroup of
// kOrderChunk threads per (range r, head h) pair, i.e. per unit; its tiles are
// placed in chunks of kOrderChunk: a tile's slot is the number of earlier tiles
// of its key in the chunk plus cursor[unit][key], the count left by earlier
// chunks.  The in-chunk rank comes from a bitonic sort of (key, position)
// pairs in LDS: in the sorted chunk a tile's rank is its distance from the
// first entry of its key, found by binary search.  tkey[h * ntiles + t] is
// tile t's key (written by order_count_kernel).
constexpr int kOrderChunk = 1024;
__global__ void __launch_bounds__(kOrderChunk)
order_fill_kernel(const int32_t* __restrict__ tkey, int nb, int64_t ntiles, int64_t seg,
                  const int32_t* __restrict__ start, int32_t* __restrict__ cursor, int32_t* __restrict__ order) {
    __shared__ unsigned long long sk[kOrderChunk];   // (key << 32) | chunk position, sorted in place
    __shared__ int32_t rank_of[kOrderChunk];
    __shared__ uint8_t last_of[kOrderChunk];
    const int r = blockIdx.x, h = blockIdx.y;
    const int64_t lo = max(static_cast<int64_t>(h) * ntiles, static_cast<int64_t>(r) * seg);
    const int64_t hi = min(static_cast<int64_t>(h + 1) * ntiles, static_cast<int64_t>(r + 1) * seg);
    if (lo >= hi) return;   // head h has no tile in range r
    const int u = h + r;
    const int32_t* st = start + static_cast<int64_t>(u) * (nb + 1);
    int32_t* cu = cursor + static_cast<int64_t>(u) * nb;
    const int tid = threadIdx.x;
    for (int64_t c0 = lo; c0 < hi; c0 += kOrderChunk) {
        const int64_t p = c0 + tid;   // launch position h * ntiles + t
        const bool live = p < hi;
        const int key = live ? tkey[p] : -1;
        // dead positions sort after every key
        sk[tid] = (static_cast<unsigned long long>(live ? static_cast<uint32_t>(key) : 0xFFFFFFFFu) << 32) |
                  static_cast<uint32_t>(tid);
        __syncthreads();
        for (int size = 2; size <= kOrderChunk; size <<= 1)
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                const int j = tid ^ stride;
                if (j > tid) {
                    const unsigned long long x = sk[tid], y = sk[j];
                    if ((x > y) == ((tid & size) == 0)) {
                        sk[tid] = y;
                        sk[j] = x;
                    }
                }
                __syncthreads();
            }
        {
            // sorted position tid: rank = distance from the first entry of its key
            const unsigned long long v = sk[tid];
            const uint32_t vk = static_cast<uint32_t>(v >> 32);
            int a = 0, b = tid;   // first position whose key is vk lies in [a, b]
            while (a < b) {
                const int m = (a + b) >> 1;
                if (static_cast<uint32_t>(sk[m] >> 32) < vk) a = m + 1;
                else b = m;
            }
            const int pos = static_cast<int>(v & 0xFFFFFFFFu);
            rank_of[pos] = tid - a;
            last_of[pos] = tid == kOrderChunk - 1 || static_cast<uint32_t>(sk[tid + 1] >> 32) != vk;
        }
        __syncthreads();
        const int rank = rank_of[tid];
        const bool last = last_of[tid] != 0;
        int cur = 0;
        if (live) {
            cur = cu[key];
            order[lo + st[key] + cur + rank] = static_cast<int32_t>(p - static_cast<int64_t>(h) * ntiles);
        }
        __syncthreads();   // every tile of the chunk has read its key's count
        if (live && last) cu[key] = cur + rank + 1;
        __syncthreads();   // counts updated and LDS free before the next chunk
    }
}

// ---------------------------------------------------------------- launchers

namespace {

// float64 means of Q and K over the ranges offs[i] .. offs[i+1] (blocks or runs)
hipError_t launch_pool(const void* q, const void* k, bool bf16, int heads, int d, int64_t ld, int64_t hs,
                       const int32_t* offs, int n, double* pooled, hipStream_t s) {
    const dim3 pg(n, heads, 2);
    if (bf16) {
        if (d == 128)
            hipLaunchKernelGGL((pool_kernel<uint16_t, 128>), pg, dim3(256), 0, s, static_cast<const uint16_t*>(q),
                               static_cast<const uint16_t*>(k), ld, hs, offs, n, heads, pooled);
        else
            hipLaunchKernelGGL((pool_kernel<uint16_t, 64>), pg, dim3(256), 0, s, static_cast<const uint16_t*>(q),
                               static_cast<const uint16_t*>(k), ld, hs, offs, n, heads, pooled);
    } else {
        if (d == 128)
            hipLaunchKernelGGL((pool_kernel<float, 128>), pg, dim3(256), 0, s, static_cast<const float*>(q),
                               static_cast<const float*>(k), ld, hs, offs, n, heads, pooled);
        else
            hipLaunchKernelGGL((pool_kernel<float, 64>), pg, dim3(256), 0, s, static_cast<const float*>(q),
                               static_cast<const float*>(k), ld, hs, offs, n, heads, pooled);
    }
    return hipGetLastError();
}

// scores of `heads` heads whose pooled means of Q and K start at pq and pk
// (n x d doubles per head)
template <typename TOut>
hipError_t launch_scores(const double* pq, const double* pk, int n, int heads, int d, float scale, TOut* out,
                         hipStream_t s) {
    const int nt = (n + kLT - 1) / kLT;
    const dim3 lg(static_cast<unsigned>(nt * nt * heads));
    if (d == 128)
        hipLaunchKernelGGL((logits_kernel<128, TOut>), lg, dim3(256), 0, s, pq, pk, n, static_cast<double>(scale),
                           out);
    else
        hipLaunchKernelGGL((logits_kernel<64, TOut>), lg, dim3(256), 0, s, pq, pk, n, static_cast<double>(scale),
                           out);
    return hipGetLastError();
}

// the selection proper, from the fp32 scores of every row
hipError_t select_rows(const float* logits, int heads, int nb, int top_k, double top_p, int32_t* sel_offsets,
                       int32_t* sel_idx, int64_t cap, int64_t* sel_total, int32_t* row_count, uint32_t* row_thr,
                       int32_t* row_tie, hipStream_t s) {
    const dim3 rg(nb, heads);
    // PRISM_SELECT_RADIX=1 forces the LDS radix kernel (used by the tests to
    // compare the two kernels on rows of any length)
    const char* ev = std::getenv("PRISM_SELECT_RADIX");
    const bool radix = ev && ev[0] == '1';
    hipError_t e;
    if (!radix && nb <= 16 * kSelThreads) {
        if (nb <= 8 * kSelThreads)
            hipLaunchKernelGGL(select_reg_kernel<8>, rg, dim3(kSelThreads), 0, s, logits, nb, top_k, top_p, row_count,
                               row_thr, row_tie);
        else
            hipLaunchKernelGGL(select_reg_kernel<16>, rg, dim3(kSelThreads), 0, s, logits, nb, top_k, top_p,
                               row_count, row_thr, row_tie);
    } else if (!radix && nb <= 64 * kSelThreads) {
        if (nb <= 32 * kSelThreads)
            hipLaunchKernelGGL(select_reg_kernel<32>, rg, dim3(kSelThreads), 0, s, logits, nb, top_k, top_p,
                               row_count, row_thr, row_tie);
        else
            hipLaunchKernelGGL(select_reg_kernel<64>, rg, dim3(kSelThreads), 0, s, logits, nb, top_k, top_p,
                               row_count, row_thr, row_tie);
    } else {
        const size_t lds = static_cast<size_t>(nb) * sizeof(uint32_t);
        if (lds > 48 * 1024) {
            e = hipFuncSetAttribute(reinterpret_cast<const void*>(&select_count_kernel),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(select_count_kernel, rg, dim3(kSelThreads), lds, s, logits, nb, top_k, top_p, row_count,
                           row_thr, row_tie);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(csr_scan_kernel, dim3(heads), dim3(1024), 0, s, row_count, nb, sel_offsets, sel_total);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(select_write_kernel<4>, rg, dim3(256), 0, s, logits, nb, row_thr, row_tie, sel_offsets,
                       sel_idx, cap);
    return hipGetLastError();
}

}  // namespace

// PRISM_SCORE_GROUP_BYTES overrides the group budget (the tests force groups
// of one head on small grids); the workspace size and the launches read it
// alike, so it must not change between the two
int64_t score_group_budget() {
    const char* ev = std::getenv("PRISM_SCORE_GROUP_BYTES");
    const long long v = ev ? std::atoll(ev) : 0;
    return v > 0 ? static_cast<int64_t>(v) : kScoreGroupBytes;
}

int64_t score_group_heads(int heads, int nb) {
    const int64_t per_head = static_cast<int64_t>(nb) * nb * static_cast<int64_t>(sizeof(float));
    return std::max<int64_t>(1, std::min<int64_t>(heads, score_group_budget() / std::max<int64_t>(per_head, 1)));
}

hipError_t launch_select(const void* q, const void* k, bool bf16, int heads, int d, int64_t ld, int64_t hs,
                         const int32_t* offs, int nb, int top_k, double top_p, float scale, int32_t* sel_offsets,
                         int32_t* sel_idx, int64_t cap, int64_t* sel_total, float* logits, bool logits_all,
                         double* pooled, int32_t* row_count, uint32_t* row_thr, int32_t* row_tie, hipStream_t s) {
    hipError_t e = launch_pool(q, k, bf16, heads, d, ld, hs, offs, nb, pooled, s);
    if (e != hipSuccess) return e;
    // heads in groups whose scores fit kScoreGroupBytes; the group's score
    // buffer is reused unless the caller asked for every head's scores
    const int64_t hg = logits_all ? heads : score_group_heads(heads, nb);
    const int64_t nb2 = static_cast<int64_t>(nb) * nb;
    for (int64_t h0 = 0; h0 < heads; h0 += hg) {
        const int g = static_cast<int>(std::min<int64_t>(hg, heads - h0));
        float* L = logits_all ? logits + h0 * nb2 : logits;
        e = launch_scores<float>(pooled + h0 * nb * d, pooled + (heads + h0) * nb * d, nb, g, d, scale, L, s);
        if (e != hipSuccess) return e;
        e = select_rows(L, g, nb, top_k, top_p, sel_offsets + h0 * (nb + 1), sel_idx + h0 * cap, cap, sel_total + h0,
                        row_count + h0 * nb, row_thr + h0 * nb, row_tie + h0 * nb, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

int64_t subblock_group_heads(int heads, int64_t nr, int nb) {
    const int64_t per_head = nr * nr * static_cast<int64_t>(sizeof(double)) +
                             static_cast<int64_t>(nb) * nb * static_cast<int64_t>(sizeof(float));
    return std::max<int64_t>(1, std::min<int64_t>(heads, score_group_budget() / std::max<int64_t>(per_head, 1)));
}

hipError_t launch_select_subblock(const void* q, const void* k, bool bf16, int heads, int d, int64_t ld, int64_t hs,
                                  int64_t N, const int32_t* offs, int nb, int top_k, double top_p, float scale,
                                  int32_t* sel_offsets, int32_t* sel_idx, int64_t cap, int64_t* sel_total,
                                  float* logits, bool logits_all, const SubblockWs& w, int32_t* row_count,
                                  uint32_t* row_thr, int32_t* row_tie, hipStream_t s) {
    const int64_t nr = N / 64;
    hipLaunchKernelGGL(run_offsets_kernel, dim3(static_cast<unsigned>((nr + 1 + 255) / 256)), dim3(256), 0, s,
                       w.run_offs, nr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_pool(q, k, bf16, heads, d, ld, hs, w.run_offs, static_cast<int>(nr), w.run_pooled, s);
    if (e != hipSuccess) return e;
    // heads in groups, as in launch_select: the run-pair scores and the block
    // scores of one group at a time
    const int64_t hg = subblock_group_heads(heads, nr, nb);
    const int64_t nb2 = static_cast<int64_t>(nb) * nb;
    for (int64_t h0 = 0; h0 < heads; h0 += hg) {
        const int g = static_cast<int>(std::min<int64_t>(hg, heads - h0));
        float* L = logits_all ? logits + h0 * nb2 : logits;
        e = launch_scores<double>(w.run_pooled + h0 * nr * d, w.run_pooled + (heads + h0) * nr * d,
                                  static_cast<int>(nr), g, d, scale, w.run_scores, s);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(subblock_reduce_kernel, dim3(nb, g), dim3(256), 0, s, w.run_scores, nr, offs, nb, L);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        e = select_rows(L, g, nb, top_k, top_p, sel_offsets + h0 * (nb + 1), sel_idx + h0 * cap, cap, sel_total + h0,
                        row_count + h0 * nb, row_thr + h0 * nb, row_tie + h0 * nb, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// zeroes n counters with a kernel (not a memset node, so that a captured
// graph replays it like the other launches)
hipError_t fill_zero(int32_t* p, int64_t n, hipStream_t s) {
    const unsigned g = static_cast<unsigned>(std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 4096)));
    hipLaunchKernelGGL(fill_i32_kernel, dim3(g), dim3(256), 0, s, p, n, 0);
    return hipGetLastError();
}

hipError_t launch_csr_scan(const int32_t* counts, int n, int32_t* offsets, int64_t* totals, int heads, hipStream_t s) {
    hipLaunchKernelGGL(csr_scan_kernel, dim3(heads), dim3(1024), 0, s, counts, n, offsets, totals);
    return hipGetLastError();
}

hipError_t launch_transpose_csr(const int32_t* sel_offsets, const int32_t* sel_idx, int nb, int heads, int64_t cap,
                                int32_t* tcount, int32_t* tr_offsets, int32_t* tr_idx, int32_t* scratch,
                                const uint8_t* rowmask, int want, hipStream_t s) {
    hipError_t e = fill_zero(tcount, static_cast<int64_t>(heads) * nb, s);
    if (e != hipSuccess) return e;
    const dim3 rg(nb, heads);
    hipLaunchKernelGGL(tr_count_kernel, rg, dim3(256), 0, s, sel_offsets, sel_idx, nb, cap, rowmask, want, tcount);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(csr_scan_kernel, dim3(heads), dim3(1024), 0, s, tcount, nb, tr_offsets,
                       static_cast<int64_t*>(nullptr));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = fill_zero(tcount, static_cast<int64_t>(heads) * nb, s)) != hipSuccess) return e;
    hipLaunchKernelGGL(tr_fill_kernel, rg, dim3(256), 0, s, sel_offsets, sel_idx, nb, cap, rowmask, want, tr_offsets,
                       tcount, tr_idx);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(tr_sort_kernel, rg, dim3(256), 0, s, tr_offsets, nb, cap, tr_idx, scratch);
    return hipGetLastError();
}

hipError_t launch_tile_order(const int32_t* sel_offsets, const int32_t* sel_idx, int64_t cap, const int32_t* offs,
                             int nb, int heads, int64_t ntiles, int32_t* bucket, int32_t* start, int32_t* order,
                             hipStream_t s) {
    const int64_t G = ntiles * heads;
    const int64_t seg = G % 8 ? G : G / 8;            // one XCD's range of the launch order
    const int units = tile_order_units(heads);
    const int64_t nbk = static_cast<int64_t>(units) * nb;
    hipError_t e = fill_zero(bucket, nbk, s);
    if (e != hipSuccess) return e;
    const dim3 g((nb + 255) / 256, heads);
    int32_t* tkey = order + heads * ntiles;            // second half of the order buffer
    hipLaunchKernelGGL(order_count_kernel, g, dim3(256), 0, s, sel_offsets, sel_idx, cap, offs, nb, ntiles, seg, bucket,
                       tkey);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(csr_scan_kernel, dim3(units), dim3(1024), 0, s, bucket, nb, start,
                       static_cast<int64_t*>(nullptr));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = fill_zero(bucket, nbk, s)) != hipSuccess) return e;
    hipLaunchKernelGGL(order_fill_kernel, dim3(8, heads), dim3(kOrderChunk), 0, s, tkey, nb, ntiles, seg, start,
                       bucket, order);
    return hipGetLastError();
}

}  // namespace prism

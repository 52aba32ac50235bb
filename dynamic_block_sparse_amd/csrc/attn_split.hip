// attn_split.hip - the split plan of the forward and dQ kernels (attn_split.hpp).
//
//   split_cost_kernel   per row: key tiles of its selected list and the number
//                       of key ranges the list touches (its chunks); adds the
//                       partial slots it would need to every threshold of a
//                       ladder that it exceeds
//   split_pick_kernel   the lowest threshold of the ladder whose rows fit the
//                       slot capacity (none: no row is split)
//   split_rows_kernel   marks the rows above it and counts their slots
//   split_count_kernel  per split row and chunk: tiles of the chunk's key range
//   split_fill_kernel   writes every (chunk, tile) item at its key range's place
//                       (the order inside a range is arbitrary: each item owns a
//                       fixed partial slot, so the results do not depend on it)
// Row and range offsets come from the per-head exclusive scan of select.hip.
#include <climits>

#include "attn_split.hpp"
#include "prism_internal.hpp"

namespace prism {

namespace {

constexpr int kLadder = 8;   // thresholds T0, 2 T0, ..., 2^7 T0 key tiles

// one wave per row: key tiles of entries e0..e1 and the number of key-range
// starts (entries whose range differs from the previous entry's)
__device__ __forceinline__ void row_walk(const int32_t* __restrict__ s, const int32_t* __restrict__ offs, int e0, int e1,
                                         int W, int& tiles, int& starts) {
    const int lane = threadIdx.x & 63;
    int t = 0, st = 0, prev = -1;
    for (int b = e0; b < e1; b += 64) {
        const int e = b + lane;
        const bool valid = e < e1;
        const int j = valid ? s[e] : 0;
        const int r = j / W;
        if (valid) t += (offs[j + 1] - offs[j]) >> 6;
        int rp = __shfl_up(r, 1, 64);
        if (lane == 0) rp = prev;
        st += __popcll(__ballot(valid && r != rp));
        const int last = min(63, e1 - 1 - b);
        prev = __shfl(r, last, 64);
    }
    tiles = wave_sum(t);
    starts = st;
}

__global__ void __launch_bounds__(64)
split_cost_kernel(const int32_t* __restrict__ sel_off, const int32_t* __restrict__ sel_idx, int64_t cap,
                  const int32_t* __restrict__ offs, int nb, int W, int T0, int32_t* __restrict__ cost,
                  int32_t* __restrict__ nch, unsigned long long* __restrict__ demand) {
    const int i = blockIdx.x, h = blockIdx.y;
    const int32_t* so = sel_off + static_cast<int64_t>(h) * (nb + 1);
    const int e0 = so[i];
    const int e1 = static_cast<int>(min(static_cast<int64_t>(so[i + 1]), cap));
    int tiles, starts;
    row_walk(sel_idx + static_cast<int64_t>(h) * cap, offs, e0, e1, W, tiles, starts);
    if (threadIdx.x == 0) {
        const int64_t ri = static_cast<int64_t>(h) * nb + i;
        cost[ri] = tiles;
        nch[ri] = starts;
        const unsigned long long slots =
            static_cast<unsigned long long>((offs[i + 1] - offs[i]) >> 6) * static_cast<unsigned long long>(starts);
        for (int k = 0; k < kLadder; ++k)
            if (static_cast<int64_t>(tiles) > (static_cast<int64_t>(T0) << k)) atomicAdd(&demand[k], slots);
    }
}

__global__ void split_pick_kernel(const unsigned long long* __restrict__ demand, int T0, int64_t cap_slots,
                                  int32_t* __restrict__ tsel) {
    if (threadIdx.x != 0) return;
    int t = INT_MAX;
    if (T0 > 0)
        for (int k = 0; k < kLadder; ++k)
            if (demand[k] <= static_cast<unsigned long long>(cap_slots)) {
                t = T0 << k;
                break;
            }
    tsel[0] = t;
}

__global__ void __launch_bounds__(256)
split_rows_kernel(const int32_t* __restrict__ cost, const int32_t* __restrict__ nch, const int32_t* __restrict__ offs,
                  int nb, const int32_t* __restrict__ tsel, uint8_t* __restrict__ heavy, int32_t* __restrict__ pcount) {
    const int i = blockIdx.x * 256 + threadIdx.x, h = blockIdx.y;
    if (i >= nb) return;
    const int64_t ri = static_cast<int64_t>(h) * nb + i;
    const bool hv = cost[ri] > tsel[0];
    heavy[ri] = hv ? 1 : 0;
    pcount[ri] = hv ? ((offs[i + 1] - offs[i]) >> 6) * nch[ri] : 0;
}

__global__ void __launch_bounds__(64)
split_count_kernel(const int32_t* __restrict__ sel_off, const int32_t* __restrict__ sel_idx, int64_t cap,
                   const int32_t* __restrict__ offs, int nb, int W, int nR, const uint8_t* __restrict__ heavy,
                   int32_t* __restrict__ bucket) {
    const int i = blockIdx.x, h = blockIdx.y;
    if (!heavy[static_cast<int64_t>(h) * nb + i]) return;
    const int lane = threadIdx.x & 63;
    const int32_t* so = sel_off + static_cast<int64_t>(h) * (nb + 1);
    const int32_t* s = sel_idx + static_cast<int64_t>(h) * cap;
    const int e0 = so[i];
    const int e1 = static_cast<int>(min(static_cast<int64_t>(so[i + 1]), cap));
    const int nt = (offs[i + 1] - offs[i]) >> 6;
    int prev = -1;
    for (int b = e0; b < e1; b += 64) {
        const int e = b + lane;
        const bool valid = e < e1;
        const int r = valid ? s[e] / W : 0;
        int rp = __shfl_up(r, 1, 64);
        if (lane == 0) rp = prev;
        if (valid && r != rp) atomicAdd(&bucket[static_cast<int64_t>(h) * nR + r], nt);
        prev = __shfl(r, min(63, e1 - 1 - b), 64);
    }
}

// Items of one split row: chunk c (entries a .. z-1, key range r) holds tiles
// tile0 .. tile0+nt-1, in partial slots pslot0 + c nt + t, placed at their
// range's start plus a cursor.
__device__ __forceinline__ void emit_chunk(int4* __restrict__ items, int64_t at, int gt0, int nt, int a, int z,
                                           int64_t pslot) {
    for (int t = 0; t < nt; ++t)
        items[at + t] = make_int4(gt0 + t, a, z, static_cast<int>(pslot + t));
}

__global__ void __launch_bounds__(64)
split_fill_kernel(const int32_t* __restrict__ sel_off, const int32_t* __restrict__ sel_idx, int64_t cap,
                  const int32_t* __restrict__ offs, int nb, int W, int nR, int ntiles,
                  const uint8_t* __restrict__ heavy, const int32_t* __restrict__ pbase,
                  const int64_t* __restrict__ ptot, const int32_t* __restrict__ bstart, int32_t* __restrict__ cursor,
                  int4* __restrict__ items) {
    const int i = blockIdx.x, h = blockIdx.y;
    if (!heavy[static_cast<int64_t>(h) * nb + i]) return;
    const int lane = threadIdx.x & 63;
    const int32_t* so = sel_off + static_cast<int64_t>(h) * (nb + 1);
    const int32_t* s = sel_idx + static_cast<int64_t>(h) * cap;
    const int e0 = so[i];
    const int e1 = static_cast<int>(min(static_cast<int64_t>(so[i + 1]), cap));
    const int nt = (offs[i + 1] - offs[i]) >> 6;
    const int gt0 = h * ntiles + (offs[i] >> 6);
    int64_t base = 0;
    for (int x = 0; x < h; ++x) base += ptot[x];
    const int64_t pslot0 = base + pbase[static_cast<int64_t>(h) * (nb + 1) + i];
    const int32_t* bs = bstart + static_cast<int64_t>(h) * (nR + 1);
    int32_t* cu = cursor + static_cast<int64_t>(h) * nR;
    auto place = [&](int a, int z, int c, int r) {
        const int64_t at = base + bs[r] + atomicAdd(&cu[r], nt);
        emit_chunk(items, at, gt0, nt, a, z, pslot0 + static_cast<int64_t>(c) * nt);
    };
    int c = 0;           // index of the open chunk (or of the next one)
    int open_a = -1;     // first entry of the chunk still open at a group's end, -1 if none
    int open_r = 0;
    int prev = -1;
    for (int b = e0; b < e1; b += 64) {
        const int e = b + lane;
        const bool valid = e < e1;
        const int r = valid ? s[e] / W : 0;
        int rp = __shfl_up(r, 1, 64);
        if (lane == 0) rp = prev;
        const bool st = valid && r != rp;
        const unsigned long long mask = __ballot(st);
        if (mask) {
            // the chunk left open by the previous group ends at this group's first start
            if (open_a >= 0) {
                if (lane == 0) place(open_a, b + __ffsll(mask) - 1, c, open_r);
                ++c;
            }
            // every start but the last ends at the next start of this group
            const unsigned long long above = lane == 63 ? 0ull : (mask & ~((2ull << lane) - 1ull));
            if (st && above) place(e, b + __ffsll(above) - 1, c + __popcll(mask & ((1ull << lane) - 1ull)), r);
            const int last = 63 - __clzll(mask);
            c += __popcll(mask) - 1;
            open_a = b + last;
            open_r = __shfl(r, last, 64);
        }
        prev = __shfl(r, min(63, e1 - 1 - b), 64);
    }
    if (open_a >= 0 && lane == 0) place(open_a, e1, c, open_r);
}

}  // namespace

hipError_t launch_split_plan(const int32_t* sel_off, const int32_t* sel_idx, int64_t cap, const int32_t* offs, int nb,
                             int heads, int64_t ntiles, int W, int T0, const SplitWs& w, hipStream_t s) {
    const int nR = (nb + W - 1) / W;
    hipError_t e = fill_zero(reinterpret_cast<int32_t*>(w.demand), 2 * kLadder, s);
    if (e != hipSuccess) return e;
    const dim3 rows(nb, heads);
    hipLaunchKernelGGL(split_cost_kernel, rows, dim3(64), 0, s, sel_off, sel_idx, cap, offs, nb, W, T0, w.cost, w.nch,
                       w.demand);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(split_pick_kernel, dim3(1), dim3(64), 0, s, w.demand, T0, w.cap_slots, w.tsel);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(split_rows_kernel, dim3((nb + 255) / 256, heads), dim3(256), 0, s, w.cost, w.nch, offs, nb,
                       w.tsel, w.heavy, w.pcount);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = launch_csr_scan(w.pcount, nb, w.pbase, w.ptot, heads, s)) != hipSuccess) return e;
    if ((e = fill_zero(w.bucket, static_cast<int64_t>(heads) * nR, s)) != hipSuccess) return e;
    hipLaunchKernelGGL(split_count_kernel, rows, dim3(64), 0, s, sel_off, sel_idx, cap, offs, nb, W, nR, w.heavy,
                       w.bucket);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = launch_csr_scan(w.bucket, nR, w.bstart, w.btot, heads, s)) != hipSuccess) return e;
    if ((e = fill_zero(w.bucket, static_cast<int64_t>(heads) * nR, s)) != hipSuccess) return e;   // cursors
    hipLaunchKernelGGL(split_fill_kernel, rows, dim3(64), 0, s, sel_off, sel_idx, cap, offs, nb, W, nR,
                       static_cast<int>(ntiles), w.heavy, w.pbase, w.ptot, w.bstart, w.bucket, w.items);
    return hipGetLastError();
}

SplitView split_view(const SplitWs& w, int heads) {
    SplitView v;
    v.items = w.items;
    v.ptotal = w.ptot;
    v.pbase = w.pbase;
    v.nchunk = w.nch;
    v.heavy = w.heavy;
    v.partials = w.partials;
    v.heads = heads;
    v.cap_slots = w.cap_slots;
    return v;
}

}  // namespace prism

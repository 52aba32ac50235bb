// attn_split.hpp - key-range split of long selected lists (the forward and dQ
// kernels' work items).
//
// A query block whose selected list is long (the diffuse rows that Top-p
// expands; reading guide, xyznot.com paper 2610.05416, "Các ý tưởng cốt lõi")
// streams thousands of key tiles that many other long rows also read.  The
// plan cuts such a row's list at fixed key-range boundaries (blocks
// [r W, (r + 1) W) form range r) into chunks; each (chunk, query tile) is one
// work item with its own fp32 partial slot, and a head's items are ordered by
// key range.  Workgroups that run together on one XCD then walk the same key
// ranges and share their tiles in that XCD's L2, and the long rows no longer
// run as a few very long workgroups.  A combine pass merges each tile's
// partials in chunk order, so results do not depend on the run order.
#pragma once
#include "prism_device.hpp"

namespace prism {

// The device view of one launch's split plan (a group of heads).
struct SplitView {
    const int4* items;       // [cap_slots] {h * ntiles + tile, e0, e1, partial slot}, items of head h first
    const int64_t* ptotal;   // [heads] items (= partial slots) of each head
    const int32_t* pbase;    // [heads][nb + 1] first slot of each row within its head's slots
    const int32_t* nchunk;   // [heads][nb] chunks of each row
    const uint8_t* heavy;    // [heads][nb] 1 for rows that were split
    float* partials;         // [cap_slots][split_partial_floats(d)]
    int heads;
    int64_t cap_slots;       // slot capacity, a multiple of 8: the chunk kernels' grid
};

// fp32 values of one partial slot: the 64 x D accumulator tile in the
// kernels' register layout, then three values per lane (forward: running
// maximum and the two row sums; dQ: its part of sum P dP)
__host__ __device__ constexpr int fwd_partial_floats(int D) { return 2 * (D / 32) * 16 * 64 + 3 * 128; }

__device__ __forceinline__ int64_t split_part_base(const SplitView& sv, int h) {
    int64_t b = 0;
    for (int x = 0; x < h; ++x) b += sv.ptotal[x];
    return b;
}

// Item of this chunk workgroup.  Workgroup b runs on XCD b % 8, and XCD x
// takes items [x S, (x + 1) S), S = ceil(G / 8), in order, so each XCD walks
// a contiguous stretch of the key-range order; workgroups beyond the plan's
// G items return false.
__device__ __forceinline__ bool split_item_of(const SplitView& sv, int& idx) {
    const int64_t G = split_part_base(sv, sv.heads);
    const int64_t S = (G + 7) / 8;
    const int64_t x = blockIdx.x % 8, l = blockIdx.x / 8;
    const int64_t i = x * S + l;
    if (l >= S || i >= G) return false;
    idx = static_cast<int>(i);
    return true;
}

inline int64_t split_grid(const SplitView& sv) { return sv.cap_slots; }

}  // namespace prism

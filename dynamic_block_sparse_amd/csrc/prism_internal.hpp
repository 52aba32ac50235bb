// prism_internal.hpp - launchers shared between the kernel files and the host
// ABI layer.  Every launcher is asynchronous on `s` and returns the launch
// status; argument checking is done by the caller (prism_api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace prism {

struct SplitView;   // attn_split.hpp

struct ZoneGrid;

hipError_t launch_zone_shapes(const void* v, bool bf16, int64_t C, int64_t ld, const float* a, ZoneGrid g, int nZ,
                              double tau128, double tau256, double eps, uint8_t* zone_shape, int32_t* block_offsets,
                              int32_t* nb_dev, double* partial, double* rec, hipStream_t s);
size_t zone_partial_doubles(int nZ, int64_t C);

hipError_t launch_block_permute(const void* x, void* y, int elem_bytes, int64_t row_elems, int64_t x_ld,
                                int64_t y_ld, const uint8_t* zone_shape, ZoneGrid g, int64_t N, int inverse,
                                hipStream_t s);
hipError_t launch_block_permute_heads(const void* x, void* y, int elem_bytes, int heads, int d, int64_t x_ld,
                                      int64_t x_hs, int64_t y_ld, int64_t y_hs, const uint8_t* zone_shape, ZoneGrid g,
                                      int64_t N, int inverse, hipStream_t s);

// The selection scores heads in groups: the fp32 score matrices of one group
// ([g, nb, nb]) are written and then read back by the selection, so a group is
// sized to stay within the 256 MB memory-side (Infinity) cache of the MI355X
// (one head at 2K: 6924^2 scores = 192 MB), and no [heads, nb, nb] matrix is
// kept.  logits_all: the caller's buffer holds every head's scores instead.
constexpr int64_t kScoreGroupBytes = int64_t(256) << 20;
int64_t score_group_heads(int heads, int nb);
int64_t subblock_group_heads(int heads, int64_t nr, int nb);

hipError_t launch_select(const void* q, const void* k, bool bf16, int heads, int d, int64_t ld, int64_t hs,
                         const int32_t* offs, int nb, int top_k, double top_p, float scale, int32_t* sel_offsets,
                         int32_t* sel_idx, int64_t cap, int64_t* sel_total, float* logits, bool logits_all,
                         double* pooled, int32_t* row_count, uint32_t* row_thr, int32_t* row_tie, hipStream_t s);

// Sub-block scoring: the runs (64-token pieces) of the N tokens, their float64
// means of Q and K, and their pairwise float64 scores.
struct SubblockWs {
    int32_t* run_offs;     // [N/64 + 1]
    double* run_pooled;    // [2, heads, N/64, d]
    double* run_scores;    // [g, N/64, N/64]: one head group (subblock_group_heads)
};
hipError_t launch_select_subblock(const void* q, const void* k, bool bf16, int heads, int d, int64_t ld, int64_t hs,
                                  int64_t N, const int32_t* offs, int nb, int top_k, double top_p, float scale,
                                  int32_t* sel_offsets, int32_t* sel_idx, int64_t cap, int64_t* sel_total,
                                  float* logits, bool logits_all, const SubblockWs& w, int32_t* row_count,
                                  uint32_t* row_thr, int32_t* row_tie, hipStream_t s);

// rowmask (NULL: every query block) keeps query block i when
// (rowmask[h*nb + i] != 0) == want
hipError_t launch_transpose_csr(const int32_t* sel_offsets, const int32_t* sel_idx, int nb, int heads, int64_t cap,
                                int32_t* tcount, int32_t* tr_offsets, int32_t* tr_idx, int32_t* scratch,
                                const uint8_t* rowmask, int want, hipStream_t s);

// Extras of the routed backward: dQ skips the tiles of flat query blocks, and
// dK/dV add to every token of key block j the block-mean gradients / B_j.
struct RouteGrad {
    const uint8_t* skip_q;   // [heads, nb] or NULL
    const float* dkbar;      // [heads, nb, d] or NULL (already scaled)
    const float* dvbar;      // [heads, nb, d] or NULL
};

hipError_t launch_attn_fwd_simt(const void* q, const void* k, const void* v, void* o, float* lse, bool bf16, int64_t N,
                                int heads, int d, int64_t ld, int64_t hs, const int32_t* offs, int nb,
                                const int32_t* so, const int32_t* si, int64_t cap, const uint8_t* skip,
                                const RowMap& om, float scale, void* ores, hipStream_t s);

hipError_t launch_attn_fwd_mfma(const void* q, const void* k, const void* v, void* o, float* lse, int64_t N, int heads,
                                int d, int64_t ld, int64_t hs, const int32_t* offs, int nb, const int32_t* so,
                                const int32_t* si, int64_t cap, const int32_t* order, const uint8_t* skip,
                                const RowMap& om, float scale, void* ores, hipStream_t s);

// row dots D = rowsum(dO * O) into Dq and, when lse2 is set, lse * log2(e) into lse2
hipError_t launch_bwd_dot(const void* o, const void* dout, bool bf16, int64_t N, int heads, int d, int64_t ld,
                          int64_t hs, const RowMap& om, float* Dq, const void* ores, const float* lse, float* lse2,
                          hipStream_t s);

// dQ of one group of heads (pointers at the group's first head): the tile
// kernel over the tiles not marked in `skip`, then, for a split plan, its
// chunks and combine; dK/dV of all heads after every group's dQ (it reads the
// exact row dots that the dQ kernels leave in Dq)
hipError_t launch_attn_dq_mfma(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                              float* Dq, void* dq, int64_t N, int heads, int d, int64_t ld, int64_t hs,
                              const int32_t* offs, int nb, const int32_t* so, const int32_t* si, int64_t cap,
                              const int32_t* qorder, const uint8_t* skip, const RowMap& om, float scale,
                              hipStream_t s);
hipError_t launch_attn_dq_split(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                                float* Dq, void* dq, int64_t N, int heads, int d, int64_t ld, int64_t hs,
                                const int32_t* offs, int nb, const int32_t* si, int64_t cap, const SplitView& sv,
                                const RowMap& om, float scale, hipStream_t s);
// lse2: lse * log2(e) (launch_bwd_dot)
hipError_t launch_attn_dkdv_mfma(const void* q, const void* k, const void* v, const void* dout, const float* lse2,
                                 const float* Dq, void* dk, void* dv, int64_t N, int heads, int d, int64_t ld,
                                 int64_t hs, const int32_t* offs, int nb, const int32_t* to, const int32_t* ti,
                                 int64_t cap, const int32_t* horder, const RouteGrad* rg, const RowMap& om, float scale,
                                 hipStream_t s);
// The dK/dV launch's head order (order[slot] = head, `heads` entries): runs of
// heads/8 consecutive slots, one per XCD, balanced by each head's count of
// (query tile, key tile) pairs from the transposed CSR; cost holds `heads`
// 64-bit counters.
hipError_t launch_head_order(const int32_t* tr_off, const int32_t* tr_idx, const int32_t* offs, int nb, int heads,
                             int64_t cap, unsigned long long* cost, int32_t* order, hipStream_t s);

hipError_t launch_attn_bwd_simt(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                                const float* Dq, void* dq, void* dk, void* dv, bool bf16, int64_t N, int heads, int d,
                                int64_t ld, int64_t hs, const int32_t* offs, int nb, const int32_t* so,
                                const int32_t* si, const int32_t* to, const int32_t* ti, int64_t cap,
                                const RouteGrad* rg, const RowMap& om, float scale, hipStream_t s);

// visiting order of the query tiles: within each unit (a head's part of one
// XCD's range of the launch order), tile ids grouped by first selected block;
// bucket holds tile_order_units(heads) * nb and start tile_order_units(heads) *
// (nb + 1) ints; order holds 2 * heads * ntiles ints (the second half keeps
// each tile's key while the first is filled)
inline int tile_order_units(int heads) { return heads + 8; }
hipError_t launch_tile_order(const int32_t* sel_offsets, const int32_t* sel_idx, int64_t cap, const int32_t* offs,
                             int nb, int heads, int64_t ntiles, int32_t* bucket, int32_t* start, int32_t* order,
                             hipStream_t s);
// counters cleared by a kernel (not a memset node, so that a captured graph
// replays it like the other launches)
hipError_t fill_zero(int32_t* p, int64_t n, hipStream_t s);
// per-head exclusive scan: offsets[h][0..n] of counts[h][0..n), totals[h] = sum (totals may be NULL)
hipError_t launch_csr_scan(const int32_t* counts, int n, int32_t* offsets, int64_t* totals, int heads, hipStream_t s);

// Key-range split of long selected lists for one launch (a group of heads;
// attn_split.hpp).  Buffers from the call's workspace: cost, nch, heavy,
// pcount [heads][nb]; pbase [heads][nb + 1]; ptot, btot [heads]; bucket
// [heads][nR] (also the fill cursors); bstart [heads][nR + 1]; demand [8];
// tsel [1]; items [cap_slots]; partials [cap_slots][fwd_partial_floats(d)];
// nR = ceil(nb / W).  Rows with more than the chosen threshold of key tiles
// are split into W-block key ranges; the threshold is the lowest of T0,
// 2 T0, ..., 128 T0 whose items fit cap_slots (none: nothing is split; T0 = 0
// disables the split).
struct SplitWs {
    int32_t* cost;
    int32_t* nch;
    uint8_t* heavy;
    int32_t* pcount;
    int32_t* pbase;
    int64_t* ptot;
    int32_t* bucket;
    int32_t* bstart;
    int64_t* btot;
    unsigned long long* demand;
    int32_t* tsel;
    int4* items;
    float* partials;
    int64_t cap_slots;
};
hipError_t launch_split_plan(const int32_t* sel_off, const int32_t* sel_idx, int64_t cap, const int32_t* offs, int nb,
                             int heads, int64_t ntiles, int W, int T0, const SplitWs& w, hipStream_t s);
SplitView split_view(const SplitWs& w, int heads);
// chunk items of a plan (fp32 partials), then the combine that writes O, its
// residual and lse of the split rows
hipError_t launch_attn_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, int64_t N,
                                 int heads, int d, int64_t ld, int64_t hs, const int32_t* offs, int nb,
                                 const int32_t* si, int64_t cap, const SplitView& sv, const RowMap& om, float scale,
                                 void* ores, hipStream_t s);

// audio-to-video norm map: per-token 2-norms (float64) and their clip-wide
// normalisation; block_max holds norm_map_blocks(N) <= kNormMapMaxBlocks doubles
constexpr int kNormMapMaxBlocks = 4096;
int norm_map_blocks(int64_t N);
hipError_t launch_norm_map(const void* h, bool bf16, int64_t N, int64_t C, int64_t ld, float* a, double* norms,
                           double* block_max, hipStream_t s);

// next row f3: sharpness routing and the block-mean flat path
hipError_t launch_flat_route(const float* logits, int heads, int nb, int n_flat, double* sharpness, uint8_t* flat,
                             hipStream_t s);
hipError_t launch_block_means(const void* k, const void* v, bool bf16, int heads, int d, int64_t ld, int64_t hs,
                              const int32_t* offs, int nb, float* kbar, float* vbar, hipStream_t s);
hipError_t launch_flat_dq(const void* q, const void* dout, const float* kbar, const float* vbar, const float* lse,
                          const float* Dq, void* dq, bool bf16, int64_t N, int heads, int d, int64_t ld, int64_t hs,
                          const int32_t* offs, int nb, const int32_t* so, const int32_t* si, int64_t cap,
                          const uint8_t* flat, float scale, hipStream_t s);
hipError_t launch_flat_kgrad(const void* q, const void* dout, const float* kbar, const float* vbar, const float* lse,
                             const float* Dq, bool bf16, int64_t N, int heads, int d, int64_t ld, int64_t hs,
                             const int32_t* offs, int nb, const int32_t* fto, const int32_t* fti, int64_t cap,
                             float scale, float* dkbar, float* dvbar, hipStream_t s);
hipError_t launch_attn_flat(const void* q, const float* kbar, const float* vbar, void* o, float* lse, bool bf16,
                            int64_t N, int heads, int d, int64_t ld, int64_t hs, const int32_t* offs, int nb,
                            const int32_t* so, const int32_t* si, int64_t cap, const uint8_t* flat, float scale,
                            void* ores, hipStream_t s);

}  // namespace prism

/*
 * prism.h - C ABI of the MI355X (gfx950) Prism dynamic block-sparse attention path.
 *
 * The path (Prism reading guide, xyznot.com paper 2610.05416, "Phương pháp" §1-§3;
 * news article at ailog.hnlab.kr, "핵심 내용", three steps):
 *   1. split the T x H x W latent token grid into 8 x 8 x 8 macro-zones;
 *   2. per zone, the directional video variance of mean-pooled V and the audio
 *      terms give the variation indicator g_d; a density gives the block volume
 *      B in {64, 128, 256} and the log2 optimum picks the nearest of 16 shapes;
 *   3. tokens are permuted into block-major order (each block contiguous);
 *   4. Q and K blocks are mean-pooled and scored; per query block a hybrid
 *      Top-k U Top-p set of key blocks is selected;
 *   5. exact attention runs over the selected key blocks only (forward and
 *      backward).
 *
 * Conventions shared by every call:
 *   - Every pointer argument is device memory owned by the caller unless the
 *     argument says "host".  The library allocates nothing, frees nothing and
 *     keeps no pointer after a call returns; scratch comes from the caller's
 *     workspace `ws` of at least prism_workspace_size(...) bytes (16-byte aligned).
 *   - Every call is asynchronous on `stream` (0 = the null stream) unless it
 *     says it synchronises.  The returned status comes from host-side checks
 *     made before anything is launched: on any status other than PRISM_OK
 *     nothing was launched and no output was touched.  A failing launch
 *     returns PRISM_E_HIP (outputs then undefined).
 *   - No C++ exception crosses this boundary.  prism_last_error() returns a
 *     message for the calling thread's last failure.
 *   - The library holds no mutable global state; calls on different streams
 *     may run concurrently as long as their buffers do not overlap.
 *   - Token tensors are [N, heads, d] with element strides `ld` (between tokens)
 *     and `hs` (between heads), d contiguous; every tensor of one call has the
 *     same dtype, ld and hs.  Supported d: 64 and 128.  Vector access needs the
 *     pointers 16-byte aligned and ld, hs multiples of 8 elements (bf16) or 4
 *     (f32), and 64 * ld * element size below 2^32 bytes (tiles are addressed
 *     with 32-bit offsets).
 *   - Block counts: every call that takes `nb` needs 1 <= nb and 64 * nb <= N
 *     (PRISM_E_ARG otherwise) and nb <= 32768 (PRISM_E_UNSUPPORTED above: the
 *     longest selection row, 32768 fp32 keys, is held in one workgroup's LDS).
 *     A 128 x 128 x 128 grid of 64-token blocks reaches the limit exactly.
 *   - Environment variables that switch to alternative kernels or schedules
 *     with the same results, for tests: PRISM_SELECT_RADIX=1 makes
 *     prism_select use its LDS radix-select kernel at every row length (by
 *     default it is used only for rows of more than 16384 blocks);
 *     PRISM_ATTN_SIMT=1 makes the bf16 attention calls use the vector-ALU
 *     kernels instead of the MFMA ones; PRISM_SCORE_GROUP_BYTES=n sets the
 *     per-group budget of the selection's score matrices (default 256 MB);
 *     PRISM_FWD_PAIRS=1 runs the two 64-row tiles of a 128- or 256-token
 *     block in one forward workgroup over their shared list (bit-identical);
 *     PRISM_SPLIT_T, PRISM_SPLIT_W, PRISM_SPLIT_GROUP and PRISM_SPLIT_SLOTS
 *     set the key-range split of long selected lists (first threshold in key
 *     tiles, 0 = never split; range width in blocks; heads per launch group;
 *     partial slots per 64-token tile).  Workspace sizes read the same
 *     variables, so they must not change between prism_workspace_size and
 *     the call.
 *   - Block-major order: zones in raster order (m = (zt*nH + zh)*nW + zw, 512
 *     positions each); inside a zone, its blocks in raster order over the block
 *     grid; inside a block, tokens in raster (t, h, w) order.  Raster token
 *     index n = (t*H + h)*W + w.
 */
#ifndef PRISM_H
#define PRISM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PRISM_OK = 0,
    PRISM_E_ARG = 1,          /* null pointer, negative or inconsistent size, bad k/p */
    PRISM_E_GRID = 2,         /* T, H or W not a positive multiple of 8 */
    PRISM_E_DTYPE = 3,        /* unknown dtype */
    PRISM_E_UNSUPPORTED = 4,  /* d not in {64, 128}, misaligned pointer or stride */
    PRISM_E_WORKSPACE = 5,    /* ws NULL or smaller than prism_workspace_size() */
    PRISM_E_HIP = 6           /* a HIP runtime call or launch failed */
} prism_status;

typedef enum { PRISM_F32 = 0, PRISM_BF16 = 1 } prism_dtype;

/* Thresholds of the volume rule and the indicator's epsilon.  The reading guide
 * ("Phương pháp" §2) gives tau128 = 0.5 and tau256 = 0.25; §1 adds an epsilon
 * without a value (1e-6 is the value used by the tests and benchmark). */
typedef struct { double tau128, tau256, eps; } prism_shape_params;

/* operation codes for prism_workspace_size */
enum { PRISM_OP_ZONE_SHAPES = 0, PRISM_OP_SELECT = 1, PRISM_OP_ATTN_FWD = 2, PRISM_OP_ATTN_BWD = 3,
       PRISM_OP_NORM_MAP = 4, PRISM_OP_FLAT_ROUTE = 5, PRISM_OP_ROUTED_FWD = 6, PRISM_OP_ROUTED_BWD = 7,
       PRISM_OP_SELECT_SUB = 8 };

/* Per-zone record written by prism_zone_shapes when `zone_stats` is not NULL:
 * 16 doubles per zone. */
enum {
    PRISM_ZS_SIGMA2_V = 0,    /* [3] directional video variance, axes T, H, W ("Phương pháp" §1, first display) */
    PRISM_ZS_R = 3,           /* [3] its ratio r_{v,d} (1/3 each for a constant zone) */
    PRISM_ZS_ABAR = 6,        /* audio coupling: zone mean of a */
    PRISM_ZS_SIGMA2_A = 7,    /* [3] variance of a's axis slice means */
    PRISM_ZS_VHAT = 10,       /* [3] its ratio (1/3 each when a is constant on the zone) */
    PRISM_ZS_RHO = 13,        /* density: max(S_v / max over zones of S_v, abar) */
    PRISM_ZS_SV = 14,         /* S_v = sum of the three video variances */
    PRISM_ZS_B = 15,          /* block volume 64, 128 or 256 */
    PRISM_ZS_STRIDE = 16
};

/*
 * prism_audio_norm_map - the audio-to-video norm map that prism_zone_shapes
 * takes as a_map: a at token n is the 2-norm of the audio-to-video
 * cross-attention output cached from the layer before (reading guide,
 * "Phương pháp" §1, definition of a), divided by its largest value over the
 * clip so that it lies in [0, 1] (the pages state the range but give no
 * normalisation; an all-zero clip maps to zeros).
 *
 *   h       device [N, C] rows of the cross-attention output in raster token
 *           order, row stride ld >= C elements, bf16 or fp32
 *   a       out device [N] fp32 map, values in [0, 1]
 *   norms   optional out device [N] float64 raw norms (NULL: kept in ws)
 *   ws, ws_bytes  prism_workspace_size(PRISM_OP_NORM_MAP, N, 0, 0, 0, 0) bytes (depends on N only)
 *
 * Squares are summed in float64 (exact for bf16 and fp32 values), the square
 * root is float64, and a = float(norm / max) is rounded once.  Rows are read
 * with 16-byte loads when h and the row stride are 16-byte aligned, 4- or
 * 2-byte loads otherwise.  Errors: PRISM_E_ARG for a NULL pointer, N <= 0,
 * C <= 0 or ld < C; PRISM_E_DTYPE; PRISM_E_WORKSPACE.
 */
prism_status prism_audio_norm_map(const void* h, prism_dtype dt, int64_t N, int64_t C, int64_t ld,
                                  float* a, double* norms, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * prism_zone_shapes - macro-zones, variation indicator, block volume and shape,
 * block layout ("Phương pháp" §1 and §2 of the reading guide; "Các ý tưởng cốt
 * lõi" for the 8x8x8 zones and the 16 candidate shapes).
 *
 *   T, H, W        grid sides (positive multiples of 8); N = T*H*W, nZ = N/512
 *   v, vdt, C, v_ld  value tensor in raster order: C channels per token
 *                  (all heads: one shape per zone, shared by every head),
 *                  token stride v_ld elements (>= C)
 *   a_map          [N] fp32 audio-to-video norm map in raster order, values in [0, 1]
 *   prm            host pointer to thresholds and epsilon (NULL: 0.5, 0.25, 1e-6)
 *   zone_shape     out [nZ] uint8: index into the candidate table of
 *                  prism_candidate_shapes()
 *   block_offsets  out [8*nZ + 1] int32: token offset of each block in
 *                  block-major order; entries 0..NB are valid, entry NB = N
 *   nb_dev         out device int32: NB, the number of blocks
 *   nb_host        optional host int32*: when not NULL the call synchronises
 *                  `stream` and stores NB there
 *   zone_stats     optional out [nZ * PRISM_ZS_STRIDE] doubles (layout above)
 *   zone_order     optional device [nZ] int32: zone_order[pos] is the raster zone
 *                  placed at block-major zone position pos (NULL: raster order;
 *                  prism_hilbert_zone_order gives the Hilbert order).  The block
 *                  offsets follow it; pass the same array to the permutations.
 *
 * Statistics accumulate in float64.  Decisions: rho < tau256 -> 256, else
 * rho < tau128 -> 128, else 64; the shape is the candidate of that volume
 * nearest to l* (third display of the reading guide's method) in squared log2
 * distance, distances within 1e-9 of the minimum counting as ties and going
 * to the lowest candidate index.
 */
prism_status prism_zone_shapes(int32_t T, int32_t H, int32_t W,
                               const void* v, prism_dtype vdt, int64_t C, int64_t v_ld,
                               const float* a_map, const prism_shape_params* prm,
                               uint8_t* zone_shape, int32_t* block_offsets, int32_t* nb_dev,
                               int32_t* nb_host, double* zone_stats,
                               void* ws, size_t ws_bytes, const int32_t* zone_order, hipStream_t stream);

/*
 * prism_zone_shapes_noalloc - prism_zone_shapes for callers that cannot
 * allocate device memory (code under stream capture into a graph, tight
 * serving loops, harnesses that forbid hipMalloc): the same arguments, checks,
 * kernels and outputs, without `ws` and `ws_bytes`.  Its scratch is a fixed
 * device array of PRISM_ZONE_SCRATCH_BYTES inside the library, one per GPU,
 * held until the process ends; the call allocates nothing (nb_host, when not
 * NULL, still synchronizes the stream).
 *   Limit: the scratch that prism_workspace_size(PRISM_OP_ZONE_SHAPES, N, 0, C,
 *   0, 0) reports must fit in PRISM_ZONE_SCRATCH_BYTES, about
 *   nZ * (3 ceil(C / 256) + 16) * 8 bytes (20,000 zones, 10 million tokens, at
 *   C = 3072); a larger grid returns PRISM_E_WORKSPACE before any launch.
 *   Every call on one GPU shares that GPU's array: calls that overlap on one
 *   GPU (two streams, two threads) race and must be serialized.  Each call
 *   writes every scratch value before it reads it, so nothing left by an
 *   earlier call reaches the outputs.
 * Status: as prism_zone_shapes; PRISM_E_UNSUPPORTED on a device index above 63.
 */
#define PRISM_ZONE_SCRATCH_BYTES (8u << 20)
prism_status prism_zone_shapes_noalloc(int32_t T, int32_t H, int32_t W,
                                       const void* v, prism_dtype vdt, int64_t C, int64_t v_ld,
                                       const float* a_map, const prism_shape_params* prm,
                                       uint8_t* zone_shape, int32_t* block_offsets, int32_t* nb_dev,
                                       int32_t* nb_host, double* zone_stats,
                                       const int32_t* zone_order, hipStream_t stream);

/*
 * prism_block_permute - gather rows from raster into block-major order
 * (inverse = 0: y[p] = x[pi(p)]) or scatter them back (inverse = 1:
 * y[pi(p)] = x[p]), pi being the block-major order defined above for the zone
 * shapes of prism_zone_shapes.  The pages reorganise the token sequence into
 * zone-shaped blocks (news article, "핵심 내용" steps 1-2) and pool and attend
 * whole blocks (reading guide §3); they give no order, so the order above is
 * this library's reading.
 *
 *   row_elems      elements moved per token (e.g. heads*d)
 *   x_ld, y_ld     token strides of x and y in elements (>= row_elems)
 *   x, y           must not overlap
 *   zone_order     the zone order given to prism_zone_shapes (NULL: raster)
 */
prism_status prism_block_permute(int32_t T, int32_t H, int32_t W, const uint8_t* zone_shape,
                                 const void* x, void* y, prism_dtype dt, int64_t row_elems,
                                 int64_t x_ld, int64_t y_ld, int32_t inverse, const int32_t* zone_order,
                                 hipStream_t stream);

/*
 * prism_block_permute_heads - the same permutation for all heads of a token
 * tensor in one call, with separate token and head strides on each side:
 * head hh of token row r of x is x + r*x_ld + hh*x_hs (likewise y), d
 * elements each.  Typical use: a raster [N, heads, d] tensor (x_ld = heads*d,
 * x_hs = d) gathered into head-major block-major storage [heads, N, d]
 * (y_ld = d, y_hs = N*d), and back with inverse = 1.
 *
 *   heads, d       heads per token, elements per head (d * element size a
 *                  multiple of 16 bytes)
 *   x_ld, x_hs     token and head strides of x in elements (16-byte multiples)
 *   y_ld, y_hs     the same for y
 *   x, y           16-byte aligned; the memory spans of x and y must not
 *                  overlap; the head regions of one tensor must not overlap
 *                  each other (not checked)
 * Status: PRISM_E_GRID for a bad grid, PRISM_E_ARG for null pointers,
 * non-positive heads or d, negative strides or overlapping spans,
 * PRISM_E_UNSUPPORTED for sizes, strides or pointers that are not 16-byte
 * multiples.
 */
prism_status prism_block_permute_heads(int32_t T, int32_t H, int32_t W, const uint8_t* zone_shape,
                                       const void* x, void* y, prism_dtype dt, int32_t heads, int32_t d,
                                       int64_t x_ld, int64_t x_hs, int64_t y_ld, int64_t y_hs,
                                       int32_t inverse, const int32_t* zone_order, hipStream_t stream);

/*
 * prism_select - pooled block scores and hybrid Top-k U Top-p key-block
 * selection (reading guide, "Phương pháp" §3, the selected-set display).
 *
 *   q, k           block-major [N, heads, d] (output of prism_block_permute)
 *   block_offsets, nb  as written by prism_zone_shapes (nb on the host)
 *   top_k          k >= 0;  top_p  0 <= p <= 1
 *   scale          score scale (1/sqrt(d) in the tests), a float32 value
 *   sel_offsets    out [heads * (nb + 1)] int32: row i of head h holds
 *                  sel_idx[h*cap + sel_offsets[h*(nb+1) + i] ...
 *                  h*cap + sel_offsets[h*(nb+1) + i + 1] - 1]
 *   sel_idx        out [heads * cap] int32 key-block indices, ascending per row
 *   cap            capacity per head (nb*nb never truncates).  A caller that
 *                  sizes it from the counts passes a guess, reads sel_total,
 *                  and calls again with cap >= max(sel_total) if it was short
 *                  (sel_offsets and sel_total are complete either way).
 *   sel_total      out device [heads] int64: entries head h needed; a value
 *                  above cap means that head's list was truncated at cap
 *                  (its CSR must then not be used)
 *   logits         optional out [heads * nb * nb] fp32: the pooled scores.
 *                  NULL: the scores are computed one group of heads at a
 *                  time in the workspace, each group's [g, nb, nb] matrices
 *                  within 256 MB (the MI355X's memory-side cache), and no
 *                  matrix of every head is kept.
 *   ws, ws_bytes   prism_workspace_size(PRISM_OP_SELECT, N, heads, d, nb, 0)
 *                  bytes (independent of cap)
 *
 * Each block is pooled by its float64 mean; its score with key block j is
 * scale * (Q_bar_i . K_bar_j) evaluated in float64 and rounded once to fp32.
 * Per row the blocks are ranked by score (ties: lower index first); the row
 * keeps the first max(k, n_p) of them (at most nb), n_p being the shortest
 * prefix whose softmax mass, summed in float64, reaches p.
 */
prism_status prism_select(const void* q, const void* k, prism_dtype dt,
                          int64_t N, int32_t heads, int32_t d, int64_t ld, int64_t hs,
                          const int32_t* block_offsets, int32_t nb,
                          int32_t top_k, double top_p, float scale,
                          int32_t* sel_offsets, int32_t* sel_idx, int64_t cap,
                          int64_t* sel_total, float* logits,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * prism_select_subblock - prism_select with sub-block scores (scoring variant
 * of the DFSAttn article, "sub-block scoring": a large block is judged by the
 * finer scores of its parts, added up).  Arguments, outputs and the selection
 * rule are those of prism_select; only the score of block pair (i, j) differs:
 *
 *   every block is cut into its consecutive 64-token runs (blocks from
 *   prism_zone_shapes hold 1, 2 or 4 runs and start at multiples of 64; other
 *   block_offsets must keep that property, which is not checked); runs are
 *   pooled by their float64 means; the score is
 *     m + log( mean over run pairs (a in i, b in j) of exp(s_ab - m) ),
 *   s_ab = scale * (Q_bar_a . K_bar_b) in float64, m the largest s_ab of the
 *   pair, evaluated in float64 and rounded once to fp32.  A pair of 64-token
 *   blocks keeps its prism_select score; a larger pair scores at least the
 *   plain score of its means and at most its best run pair.
 *
 *   N              a multiple of 64
 *   ws, ws_bytes   prism_workspace_size(PRISM_OP_SELECT_SUB, N, heads, d, nb, 0)
 *                  bytes: the run-pair scores of one group of heads at a time,
 *                  g * (N/64)^2 doubles, g as many heads as fit 256 MB with
 *                  their block scores, at least one (680 MB at 589,824 tokens)
 * Status: as prism_select, plus PRISM_E_ARG when N is not a multiple of 64.
 */
prism_status prism_select_subblock(const void* q, const void* k, prism_dtype dt,
                                   int64_t N, int32_t heads, int32_t d, int64_t ld, int64_t hs,
                                   const int32_t* block_offsets, int32_t nb,
                                   int32_t top_k, double top_p, float scale,
                                   int32_t* sel_offsets, int32_t* sel_idx, int64_t cap,
                                   int64_t* sel_total, float* logits,
                                   void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Raster placement of attention outputs: the inverse of the block-major
 * permutation applied as the rows are written, instead of a separate
 * prism_block_permute(..., inverse = 1) pass.  The row at block-major
 * position p goes to raster token pi(p) of the T x H x W grid laid out by
 * zone_shape (and zone_order), at element offset pi(p) * ld + h * hs from the
 * output pointer.  ld > 0 and hs >= 0 are multiples of 16 bytes in elements;
 * the head regions of one output must not overlap each other (not checked).
 */
typedef struct {
    int32_t T, H, W;              /* grid of prism_zone_shapes; T*H*W must equal N */
    const uint8_t* zone_shape;    /* device, from prism_zone_shapes */
    const int32_t* zone_order;    /* device zone order given to prism_zone_shapes, or NULL */
    int64_t ld, hs;               /* token and head strides of the raster tensors, elements */
} prism_raster_layout;

/*
 * prism_sparse_attn_fwd - exact attention restricted to the selected key blocks
 * (reading guide, "Phương pháp" §3: online-softmax attention over S_i only).
 * Non-causal, no dropout, no bias.
 *
 *   q, k, v        block-major [N, heads, d]
 *   o              out [N, heads, d], same dtype: block-major with q's strides when
 *                  `out` is NULL, else raster as `out` describes
 *   lse            out [heads, N] fp32 natural-log log-sum-exp of the scaled scores,
 *                  indexed by block-major position in either case
 *   o_res          optional out (NULL: not written; bf16 only, NULL for fp32): the
 *                  bf16 residual O - bf16(O) of every element, in o's layout and
 *                  strides.  O + o_res carries O to about 16 bits, which the
 *                  backward needs for rowsum(dO * O): that row dot computed from
 *                  the rounded O moves dK by up to 2^-9 |O| |dO| |Q| per user row
 *   sel_offsets, sel_idx, cap  the CSR written by prism_select; it must be complete
 *                  (sel_total <= cap for every head, which cap = nb*nb guarantees).
 *                  Given a truncated one, each row attends over the entries stored
 *                  for it below cap, and a row with none gets O = 0 and lse = -inf
 *   scale          softmax scale, finite and > 0 (1/sqrt(d)); PRISM_E_ARG otherwise
 *   block_offsets  must be the offsets written by prism_zone_shapes for the same
 *                  grid (every block a whole number of 64-token tiles)
 *   out            NULL or the raster placement of o (PRISM_E_GRID / PRISM_E_ARG /
 *                  PRISM_E_UNSUPPORTED for a bad grid, token count or stride)
 *   ws, ws_bytes   prism_workspace_size(PRISM_OP_ATTN_FWD, ...) bytes: the order in
 *                  which the query tiles are visited (grouped by first selected
 *                  block, which shares key tiles in L2); PRISM_E_WORKSPACE if short
 * bf16 runs on bf16 MFMA with fp32 accumulation and an fp32 online softmax;
 * f32 runs on fp32 vector arithmetic.  The outputs do not depend on the
 * visiting order: each row is accumulated over its blocks in ascending order.
 */
prism_status prism_sparse_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                                   void* o_res, prism_dtype dt, int64_t N, int32_t heads, int32_t d,
                                   int64_t ld, int64_t hs,
                                   const int32_t* block_offsets, int32_t nb,
                                   const int32_t* sel_offsets, const int32_t* sel_idx, int64_t cap,
                                   float scale, const prism_raster_layout* out,
                                   void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * prism_sparse_attn_bwd - gradient of prism_sparse_attn_fwd with respect to
 * q, k and v, the selection being a constant.  The pages train with the
 * method but do not describe its backward; this is the chain rule of the
 * masked softmax: P = exp(scale*q.k - lse), dV = P^T dO, dP = dO V^T,
 * dS = P (dP - rowsum(dO * O)), dQ = scale dS K, dK = scale dS^T Q.
 *
 *   o              forward output: block-major with q's strides, or raster as `io`
 *                  describes
 *   o_res          the forward's residual of O (same layout as o), or NULL: then
 *                  rowsum(dO * O) is taken from the rounded O alone
 *   dout           upstream gradient, block-major
 *   lse            forward log-sum-exp
 *   sel_offsets, sel_idx, cap  the CSR given to the forward (complete; with a
 *                  truncated one the gradient is that of the forward over the
 *                  stored entries, and a row with none contributes nothing)
 *   dq, dk, dv     out, same dtype, fully overwritten: block-major with q's strides,
 *                  or raster as `io` describes
 *   io             NULL or the raster placement of o, dq, dk and dv (checks as in
 *                  prism_sparse_attn_fwd)
 *   ws, ws_bytes   prism_workspace_size(PRISM_OP_ATTN_BWD, ...) bytes: row sums,
 *                  lse in base 2, the transposed selection and the dQ tile
 *                  visiting order
 * Deterministic: every output element is accumulated in a fixed order.
 */
prism_status prism_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                                   const void* o_res, const void* dout, const float* lse,
                                   void* dq, void* dk, void* dv,
                                   prism_dtype dt, int64_t N, int32_t heads, int32_t d,
                                   int64_t ld, int64_t hs,
                                   const int32_t* block_offsets, int32_t nb,
                                   const int32_t* sel_offsets, const int32_t* sel_idx, int64_t cap,
                                   float scale, const prism_raster_layout* io,
                                   void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * prism_flat_route - sharpness routing of query blocks (next row after the
 * exact path; "In-Context Sparse Attention" article, grouped computation):
 * M_i is the variance of the softmax of query block i's pooled scores over its
 * NB key blocks, and the floor(flat_ratio * NB) blocks of lowest M_i per head
 * are flat, ties toward the lower index (the article names a flat ratio and a
 * threshold on M_i without values).
 *
 *   logits     device [heads, NB, NB] fp32 pooled scores (prism_select's logits)
 *   flat_ratio in [0, 1]
 *   flat       out device [heads, NB] uint8: 1 flat, 0 sharp
 *   sharpness  optional out device [heads, NB] float64 M_i (NULL: kept in ws,
 *              prism_workspace_size(PRISM_OP_FLAT_ROUTE, 0, heads, 0, nb, 0) bytes)
 * M_i is computed in float64 as written: max, sum of exp, then the squared
 * deviations of the probabilities from 1/NB.  Errors: PRISM_E_ARG for a NULL
 * pointer, heads or nb out of range, flat_ratio outside [0, 1];
 * PRISM_E_WORKSPACE.
 */
prism_status prism_flat_route(const float* logits, int32_t heads, int32_t nb, double flat_ratio, uint8_t* flat,
                              double* sharpness, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * prism_routed_attn_fwd - forward with sharp blocks on the exact path of
 * prism_sparse_attn_fwd and flat blocks (flat[h*NB + i] != 0) on the
 * block-mean path: every selected key block j enters as its mean key and mean
 * value, counted B_j times (the article's zeroth-order Taylor kernel, over the
 * block's selected set):
 *     O_q = sum_j B_j exp(s q.K_bar_j) V_bar_j / sum_j B_j exp(s q.K_bar_j),
 *     lse_q = log sum_j B_j exp(s q.K_bar_j).
 * Arguments as prism_sparse_attn_fwd without `out` (o is block-major), plus `flat` from prism_flat_route;
 * workspace prism_workspace_size(PRISM_OP_ROUTED_FWD, ...) bytes.  Block means
 * are float64 sums rounded once to fp32; the flat path computes in fp32.
 */
prism_status prism_routed_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, void* o_res,
                                   prism_dtype dt, int64_t N, int32_t heads, int32_t d, int64_t ld, int64_t hs,
                                   const int32_t* block_offsets, int32_t nb, const int32_t* sel_offsets,
                                   const int32_t* sel_idx, int64_t cap, const uint8_t* flat, float scale, void* ws,
                                   size_t ws_bytes, hipStream_t stream);

/*
 * prism_routed_attn_bwd - gradient of prism_routed_attn_fwd, the selection
 * and the routing held constant.  Sharp query blocks contribute exactly as in
 * prism_sparse_attn_bwd.  A flat query row q with weights w_j, D_q =
 * rowsum(dO * O) and dS_j = w_j (dO_q . V_bar_j - D_q) contributes
 *     dq = scale sum_j dS_j K_bar_j,
 *     dK_bar_j += scale dS_j q,   dV_bar_j += w_j dO_q,
 * and every token of key block j receives dK_bar_j / B_j and dV_bar_j / B_j
 * (the chain rule through the block means; the article gives no backward).
 * Arguments as prism_sparse_attn_bwd without `io` (o, dq, dk, dv block-major), plus `flat`; workspace
 * prism_workspace_size(PRISM_OP_ROUTED_BWD, ...) bytes.  Deterministic: the
 * block-mean gradients are summed per key block in a fixed order and added to
 * the exact dK/dV before rounding.
 */
prism_status prism_routed_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* o_res,
                                   const void* dout, const float* lse, void* dq, void* dk, void* dv, prism_dtype dt,
                                   int64_t N, int32_t heads, int32_t d, int64_t ld, int64_t hs,
                                   const int32_t* block_offsets, int32_t nb, const int32_t* sel_offsets,
                                   const int32_t* sel_idx, int64_t cap, const uint8_t* flat, float scale, void* ws,
                                   size_t ws_bytes, hipStream_t stream);

/*
 * prism_hilbert_zone_order - host function (next row after the exact path; the
 * DFSAttn article's Hilbert-curve reordering, applied to zones): order[pos] =
 * the raster zone index of the pos-th zone along the 3D Hilbert curve of
 * J. Skilling's transform over the smallest 2^k cube holding the zone grid,
 * axes (t, h, w) with t the most significant, zones outside the grid skipped.
 *
 *   order   out host [nZ] int32 (nZ = T/8 * H/8 * W/8); copy it to the device
 *           for prism_zone_shapes and the permutations
 * Errors: PRISM_E_GRID, PRISM_E_ARG for a NULL pointer.
 */
prism_status prism_hilbert_zone_order(int32_t T, int32_t H, int32_t W, int32_t* order);

/* Workspace bytes for one call.  ZONE_SHAPES: N = T*H*W and d = C (heads, nb,
 * cap ignored).  SELECT, ATTN_FWD, ATTN_BWD: the call's N, heads, d, nb, cap. */
size_t prism_workspace_size(int32_t op, int64_t N, int32_t heads, int32_t d, int32_t nb, int64_t cap);

/* Static description of a status code. */
const char* prism_status_string(prism_status s);

/* Message of the calling thread's last failing call ("" if none). */
const char* prism_last_error(void);

/* The 16 candidate shapes (b_T, b_H, b_W) in the index order used by
 * zone_shape: by volume (64, 128, 256), then lexicographically.  Host memory. */
void prism_candidate_shapes(int32_t out[16][3]);

#ifdef __cplusplus
}
#endif

#endif /* PRISM_H */

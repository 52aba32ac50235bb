// prism_api.cpp - the C ABI declared in include/prism.h: argument checks,
// workspace carving and kernel launches.  Nothing here allocates device
// memory; errors are reported by status code plus a thread-local message.  The
// one piece of state is the per-device address of the fixed scratch array that
// prism_zone_shapes_noalloc uses instead of a workspace.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "attn_split.hpp"
#include "prism.h"
#include "prism_device.hpp"
#include "prism_internal.hpp"

namespace {

thread_local std::string g_last_error;

prism_status fail(prism_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

prism_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return PRISM_OK;
    return fail(PRISM_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Carves consecutive aligned regions out of the caller's workspace.
struct Carver {
    char* base;
    size_t off = 0;
    explicit Carver(void* b) : base(static_cast<char*>(b)) {}
    template <typename T>
    T* take(size_t count) {
        T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
        off += align_up(count * sizeof(T));
        return p;
    }
};

struct SelectWs {
    double* pooled;
    float* logits;
    int32_t* row_count;
    uint32_t* row_thr;
    int32_t* row_tie;
};
SelectWs carve_select(Carver& c, int64_t heads, int64_t d, int64_t nb) {
    SelectWs w;
    w.pooled = c.take<double>(2 * heads * nb * d);
    w.logits = c.take<float>(prism::score_group_heads(static_cast<int>(heads), static_cast<int>(nb)) * nb * nb);
    w.row_count = c.take<int32_t>(heads * nb);
    w.row_thr = c.take<uint32_t>(heads * nb);
    w.row_tie = c.take<int32_t>(heads * nb);
    return w;
}

// sub-block scoring: the selection's per-row buffers and scores, plus the runs
struct SubSelectWs {
    float* logits;
    int32_t* row_count;
    uint32_t* row_thr;
    int32_t* row_tie;
    prism::SubblockWs sub;
};
SubSelectWs carve_select_sub(Carver& c, int64_t N, int64_t heads, int64_t d, int64_t nb) {
    SubSelectWs w;
    const int64_t nr = N / 64;
    const int64_t hg = prism::subblock_group_heads(static_cast<int>(heads), nr, static_cast<int>(nb));
    w.logits = c.take<float>(hg * nb * nb);
    w.row_count = c.take<int32_t>(heads * nb);
    w.row_thr = c.take<uint32_t>(heads * nb);
    w.row_tie = c.take<int32_t>(heads * nb);
    w.sub.run_offs = c.take<int32_t>(nr + 1);
    w.sub.run_pooled = c.take<double>(2 * heads * nr * d);
    w.sub.run_scores = c.take<double>(hg * nr * nr);
    return w;
}

struct BwdWs {
    float* Dq;
    float* lse2;       // lse * log2(e), for dK/dV
    int32_t* tcount;
    int32_t* tr_offsets;
    int32_t* tr_idx;
    int32_t* scratch;
    int32_t* obucket;  // bucket counts of the tile order
    int32_t* ostart;   // bucket starts of the tile order
    int32_t* qorder;   // dQ tile order
    unsigned long long* hcost;   // per-head pair counts of the dK/dV launch
    int32_t* horder;             // its head order
};
// `hg` heads share the per-group buffers (the dQ tile order), all heads the rest
BwdWs carve_bwd(Carver& c, int64_t N, int64_t heads, int64_t hg, int64_t nb, int64_t cap) {
    BwdWs w;
    w.Dq = c.take<float>(heads * N);
    w.lse2 = c.take<float>(heads * N);
    w.tcount = c.take<int32_t>(heads * nb);
    w.tr_offsets = c.take<int32_t>(heads * (nb + 1));
    w.tr_idx = c.take<int32_t>(heads * cap);
    w.scratch = c.take<int32_t>(heads * cap);
    const int64_t units = prism::tile_order_units(static_cast<int>(hg));
    w.obucket = c.take<int32_t>(units * nb);
    w.ostart = c.take<int32_t>(units * (nb + 1));
    w.qorder = c.take<int32_t>(2 * hg * (N / 64));
    w.hcost = c.take<unsigned long long>(heads);
    w.horder = c.take<int32_t>(heads);
    return w;
}

// Visiting order of the 64-token tiles for the attention kernels.
struct OrderWs {
    int32_t* bucket;
    int32_t* start;
    int32_t* order;
};
OrderWs carve_order(Carver& c, int64_t N, int64_t heads, int64_t nb) {
    OrderWs w;
    const int64_t units = prism::tile_order_units(static_cast<int>(heads));
    w.bucket = c.take<int32_t>(units * nb);
    w.start = c.take<int32_t>(units * (nb + 1));
    w.order = c.take<int32_t>(2 * heads * (N / 64));
    return w;
}

// The forward and dQ process heads in groups of at most `group` heads, each
// group with the same per-group buffers (tile order, split plan, partials).
// Rows with more than T0 key tiles (or the lowest multiple 2^k T0 whose items
// fit the slot capacity, `slots` per query tile of the group) are split into
// key ranges of W blocks.  (At 2K one slot per tile runs as fast as two and
// needs 7.6 GB of partials instead of 15.2; groups of 8 or 12 heads took 4-11 ms
// more per step.)  The environment may override the four for
// experiments (PRISM_SPLIT_W, PRISM_SPLIT_T: 0 turns the split off,
// PRISM_SPLIT_GROUP, PRISM_SPLIT_SLOTS); the workspace size and the calls read
// the same values.
struct SplitParams {
    int W, T0, group, slots;   // slots: partial slots per query tile of a group
};
int env_int(const char* name, int dflt, int lo, int hi) {
    const char* e = std::getenv(name);
    if (!e || !*e) return dflt;
    const long v = std::strtol(e, nullptr, 10);
    return v < lo ? lo : (v > hi ? hi : static_cast<int>(v));
}
SplitParams split_params() {
    return SplitParams{env_int("PRISM_SPLIT_W", 128, 1, 1 << 15), env_int("PRISM_SPLIT_T", 256, 0, 1 << 20),
                       env_int("PRISM_SPLIT_GROUP", 64, 1, 1 << 10), env_int("PRISM_SPLIT_SLOTS", 1, 1, 1 << 10)};
}
int64_t group_heads(int64_t heads, const SplitParams& sp) { return std::min<int64_t>(heads, sp.group); }
// partial-slot capacity of one group, a multiple of 8
int64_t split_slots(int64_t N, int64_t hg, const SplitParams& sp) { return (sp.slots * (N / 64) * hg + 7) / 8 * 8; }

prism::SplitWs carve_split(Carver& c, int64_t N, int64_t hg, int64_t nb, int64_t d, const SplitParams& sp) {
    prism::SplitWs w;
    const int64_t nR = (nb + sp.W - 1) / sp.W;
    w.cap_slots = split_slots(N, hg, sp);
    w.cost = c.take<int32_t>(hg * nb);
    w.nch = c.take<int32_t>(hg * nb);
    w.heavy = c.take<uint8_t>(hg * nb);
    w.pcount = c.take<int32_t>(hg * nb);
    w.pbase = c.take<int32_t>(hg * (nb + 1));
    w.ptot = c.take<int64_t>(hg);
    w.bucket = c.take<int32_t>(hg * nR);
    w.bstart = c.take<int32_t>(hg * (nR + 1));
    w.btot = c.take<int64_t>(hg);
    w.demand = c.take<unsigned long long>(8);
    w.tsel = c.take<int32_t>(1);
    w.items = c.take<int4>(w.cap_slots);
    w.partials = c.take<float>(w.cap_slots * prism::fwd_partial_floats(static_cast<int>(d)));
    return w;
}

// Extra workspace of the routed backward: the transposed CSR restricted to
// flat query blocks, the block means and their gradients.
struct RoutedBwdWs {
    int32_t* fto;
    int32_t* fti;
    float* kbar;
    float* vbar;
    float* dkbar;
    float* dvbar;
};
RoutedBwdWs carve_routed_bwd(Carver& c, int64_t heads, int64_t d, int64_t nb, int64_t cap) {
    RoutedBwdWs w;
    w.fto = c.take<int32_t>(heads * (nb + 1));
    w.fti = c.take<int32_t>(heads * cap);
    w.kbar = c.take<float>(heads * nb * d);
    w.vbar = c.take<float>(heads * nb * d);
    w.dkbar = c.take<float>(heads * nb * d);
    w.dvbar = c.take<float>(heads * nb * d);
    return w;
}

size_t zone_ws(int64_t N, int64_t C) {
    const int nZ = static_cast<int>(N / prism::kZoneTokens);
    return align_up(prism::zone_partial_doubles(nZ, C) * sizeof(double)) +
           align_up(static_cast<size_t>(nZ) * PRISM_ZS_STRIDE * sizeof(double));
}

bool use_simt_attention(prism_dtype dt) {
    if (dt == PRISM_F32) return true;
    const char* e = std::getenv("PRISM_ATTN_SIMT");
    return e && e[0] == '1';
}

prism_status check_grid(int32_t T, int32_t H, int32_t W) {
    if (T <= 0 || H <= 0 || W <= 0 || T % 8 || H % 8 || W % 8)
        return fail(PRISM_E_GRID, "grid %d x %d x %d: sides must be positive multiples of 8", T, H, W);
    const int64_t nZ = static_cast<int64_t>(T / 8) * (H / 8) * (W / 8);
    if (nZ > (1 << 22)) return fail(PRISM_E_ARG, "grid too large (%lld zones)", static_cast<long long>(nZ));
    return PRISM_OK;
}

int elem_bytes(prism_dtype dt) { return dt == PRISM_BF16 ? 2 : 4; }

// shared checks of the token-tensor calls
prism_status check_tokens(prism_dtype dt, int64_t N, int32_t heads, int32_t d, int64_t ld, int64_t hs, int32_t nb,
                          int64_t cap) {
    if (dt != PRISM_F32 && dt != PRISM_BF16) return fail(PRISM_E_DTYPE, "unknown dtype %d", static_cast<int>(dt));
    if (N <= 0 || N % 64) return fail(PRISM_E_ARG, "N = %lld must be a positive multiple of 64", static_cast<long long>(N));
    if (heads <= 0) return fail(PRISM_E_ARG, "heads = %d must be positive", heads);
    if (d != 64 && d != 128) return fail(PRISM_E_UNSUPPORTED, "d = %d: supported head sizes are 64 and 128", d);
    if (ld < d || hs < 0) return fail(PRISM_E_ARG, "bad strides ld = %lld, hs = %lld", static_cast<long long>(ld),
                                      static_cast<long long>(hs));
    const int64_t vec = 16 / elem_bytes(dt);
    if (ld % vec || hs % vec)
        return fail(PRISM_E_UNSUPPORTED, "strides must be multiples of %lld elements", static_cast<long long>(vec));
    if (ld * 64 * elem_bytes(dt) >= (int64_t{1} << 32))
        return fail(PRISM_E_UNSUPPORTED, "ld = %lld too large: 64 rows must span less than 4 GiB",
                    static_cast<long long>(ld));
    if (nb <= 0 || static_cast<int64_t>(nb) * 64 > N)
        return fail(PRISM_E_ARG, "nb = %d out of range for N = %lld", nb, static_cast<long long>(N));
    if (nb > 32768) return fail(PRISM_E_UNSUPPORTED, "nb = %d above the 32768-block limit", nb);
    if (cap <= 0) return fail(PRISM_E_ARG, "cap must be positive");
    return PRISM_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

prism::ZoneGrid grid_of(int32_t T, int32_t H, int32_t W, const int32_t* zone_order = nullptr) {
    prism::ZoneGrid g;
    g.T = T;
    g.H = H;
    g.W = W;
    g.nH = H / 8;
    g.nW = W / 8;
    g.order = zone_order;
    return g;
}

// Output rows block-major (layout NULL: the inputs' strides) or scattered to
// raster order through the zone shapes.
prism_status row_map(const prism_raster_layout* L, prism_dtype dt, int64_t N, int64_t ld, int64_t hs,
                     prism::RowMap& m) {
    m.zone_shape = nullptr;
    m.g = grid_of(8, 8, 8);
    m.ld = ld;
    m.hs = hs;
    if (!L) return PRISM_OK;
    prism_status st = check_grid(L->T, L->H, L->W);
    if (st != PRISM_OK) return st;
    if (static_cast<int64_t>(L->T) * L->H * L->W != N)
        return fail(PRISM_E_ARG, "raster layout grid %d x %d x %d does not hold N = %lld tokens", L->T, L->H, L->W,
                    static_cast<long long>(N));
    if (!L->zone_shape) return fail(PRISM_E_ARG, "raster layout needs zone_shape");
    const int64_t vec = dt == PRISM_BF16 ? 8 : 4;   // elements per 16 bytes
    if (L->ld <= 0 || L->hs < 0 || L->ld % vec || L->hs % vec)
        return fail(PRISM_E_UNSUPPORTED, "raster layout strides must be non-negative multiples of 16 bytes "
                                         "(ld = %lld, hs = %lld)",
                    static_cast<long long>(L->ld), static_cast<long long>(L->hs));
    m.zone_shape = L->zone_shape;
    m.g = grid_of(L->T, L->H, L->W, L->zone_order);
    m.ld = L->ld;
    m.hs = L->hs;
    return PRISM_OK;
}

// Index of cell x (3 axes, `bits` bits each) along the 3D Hilbert curve of
// J. Skilling's transform ("Programming the Hilbert curve", AIP Conf. Proc.
// 707, 2004): undo the per-level rotations and reflections, Gray-code the
// axes, then interleave their bits from the top level down, axis 0 first.
uint64_t hilbert_index3(uint32_t x0, uint32_t x1, uint32_t x2, int bits) {
    uint32_t x[3] = {x0, x1, x2};
    const uint32_t top = 1u << (bits - 1);
    for (uint32_t q = top; q > 1; q >>= 1) {
        const uint32_t low = q - 1;
        for (int i = 0; i < 3; ++i) {
            if (x[i] & q) {
                x[0] ^= low;
            } else {
                const uint32_t sw = (x[0] ^ x[i]) & low;
                x[0] ^= sw;
                x[i] ^= sw;
            }
        }
    }
    x[1] ^= x[0];
    x[2] ^= x[1];
    uint32_t flip = 0;
    for (uint32_t q = top; q > 1; q >>= 1)
        if (x[2] & q) flip ^= q - 1;
    for (int i = 0; i < 3; ++i) x[i] ^= flip;
    uint64_t h = 0;
    for (int b = bits - 1; b >= 0; --b)
        for (int i = 0; i < 3; ++i) h = (h << 1) | ((x[i] >> b) & 1u);
    return h;
}

}  // namespace

extern "C" {

const char* prism_status_string(prism_status s) {
    switch (s) {
        case PRISM_OK: return "ok";
        case PRISM_E_ARG: return "invalid argument";
        case PRISM_E_GRID: return "grid sides must be positive multiples of 8";
        case PRISM_E_DTYPE: return "unknown dtype";
        case PRISM_E_UNSUPPORTED: return "unsupported size, stride or alignment";
        case PRISM_E_WORKSPACE: return "workspace missing or too small";
        case PRISM_E_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* prism_last_error(void) { return g_last_error.c_str(); }

prism_status prism_hilbert_zone_order(int32_t T, int32_t H, int32_t W, int32_t* order) {
    prism_status st = check_grid(T, H, W);
    if (st != PRISM_OK) return st;
    if (!order) return fail(PRISM_E_ARG, "null pointer argument");
    const int nT = T / 8, nH = H / 8, nW = W / 8;
    int bits = 1;
    while ((1 << bits) < std::max(nT, std::max(nH, nW))) ++bits;
    if (bits > 21) return fail(PRISM_E_UNSUPPORTED, "zone grid too large for a 63-bit Hilbert index");
    const int64_t nZ = static_cast<int64_t>(nT) * nH * nW;
    std::vector<std::pair<uint64_t, int32_t>> keyed(static_cast<size_t>(nZ));
    for (int64_t m = 0; m < nZ; ++m) {
        const int zt = static_cast<int>(m / (static_cast<int64_t>(nH) * nW));
        const int zh = static_cast<int>((m / nW) % nH), zw = static_cast<int>(m % nW);
        keyed[static_cast<size_t>(m)] = {hilbert_index3(zt, zh, zw, bits), static_cast<int32_t>(m)};
    }
    std::sort(keyed.begin(), keyed.end());
    for (int64_t pos = 0; pos < nZ; ++pos) order[pos] = keyed[static_cast<size_t>(pos)].second;
    return PRISM_OK;
}

void prism_candidate_shapes(int32_t out[16][3]) {
    for (int i = 0; i < 16; ++i) {
        int bt, bh, bw;
        prism::shape_of(i, bt, bh, bw);
        out[i][0] = bt;
        out[i][1] = bh;
        out[i][2] = bw;
    }
}

size_t prism_workspace_size(int32_t op, int64_t N, int32_t heads, int32_t d, int32_t nb, int64_t cap) {
    if (op == PRISM_OP_FLAT_ROUTE)   // no token count: heads x nb sharpness values
        return heads > 0 && nb > 0 ? align_up(static_cast<size_t>(heads) * nb * sizeof(double)) : 0;
    if (N <= 0) return 0;
    switch (op) {
        case PRISM_OP_ZONE_SHAPES: return zone_ws(N, d);
        case PRISM_OP_SELECT: {
            Carver c(nullptr);
            carve_select(c, heads, d, nb);
            return c.off;
        }
        case PRISM_OP_SELECT_SUB: {
            Carver c(nullptr);
            carve_select_sub(c, N, heads, d, nb);
            return c.off;
        }
        case PRISM_OP_ATTN_FWD: {
            const SplitParams sp = split_params();
            const int64_t hg = group_heads(heads, sp);
            Carver c(nullptr);
            carve_order(c, N, hg, nb);
            carve_split(c, N, hg, nb, d, sp);
            return c.off;
        }
        case PRISM_OP_ROUTED_FWD: {
            const int64_t hg = group_heads(heads, split_params());
            Carver c(nullptr);
            carve_order(c, N, hg, nb);
            c.take<float>(static_cast<size_t>(heads) * nb * d);
            c.take<float>(static_cast<size_t>(heads) * nb * d);
            return c.off;
        }
        case PRISM_OP_ROUTED_BWD: {
            const int64_t hg = group_heads(heads, split_params());
            Carver c(nullptr);
            carve_bwd(c, N, heads, hg, nb, cap);
            carve_routed_bwd(c, heads, d, nb, cap);
            return c.off;
        }
        case PRISM_OP_NORM_MAP:
            return align_up(static_cast<size_t>(N) * sizeof(double)) +
                   align_up(static_cast<size_t>(prism::kNormMapMaxBlocks) * sizeof(double));
        case PRISM_OP_ATTN_BWD: {
            const SplitParams sp = split_params();
            const int64_t hg = group_heads(heads, sp);
            Carver c(nullptr);
            carve_bwd(c, N, heads, hg, nb, cap);
            carve_split(c, N, hg, nb, d, sp);
            return c.off;
        }
    }
    return 0;
}

prism_status prism_audio_norm_map(const void* h, prism_dtype dt, int64_t N, int64_t C, int64_t ld, float* a,
                                  double* norms, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (dt != PRISM_F32 && dt != PRISM_BF16) return fail(PRISM_E_DTYPE, "unknown dtype %d", static_cast<int>(dt));
    if (!h || !a) return fail(PRISM_E_ARG, "null pointer argument");
    if (N <= 0 || C <= 0 || ld < C)
        return fail(PRISM_E_ARG, "need N > 0, C > 0 and ld >= C (N = %lld, C = %lld, ld = %lld)",
                    static_cast<long long>(N), static_cast<long long>(C), static_cast<long long>(ld));
    const size_t need = prism_workspace_size(PRISM_OP_NORM_MAP, N, 0, 0, 0, 0);
    if (!ws || ws_bytes < need)
        return fail(PRISM_E_WORKSPACE, "norm map needs %zu workspace bytes, got %zu", need, ws ? ws_bytes : 0);
    Carver c(ws);
    double* own = c.take<double>(static_cast<size_t>(N));
    double* bmax = c.take<double>(static_cast<size_t>(prism::kNormMapMaxBlocks));
    return hip_status(prism::launch_norm_map(h, dt == PRISM_BF16, N, C, ld, a, norms ? norms : own, bmax, stream),
                      "norm map launch");
}

namespace {

prism_status check_zone_args(int32_t T, int32_t H, int32_t W, const void* v, prism_dtype vdt, int64_t C, int64_t v_ld,
                             const float* a_map, const prism_shape_params* prm, uint8_t* zone_shape,
                             int32_t* block_offsets, int32_t* nb_dev, prism_shape_params& p) {
    prism_status st = check_grid(T, H, W);
    if (st != PRISM_OK) return st;
    if (vdt != PRISM_F32 && vdt != PRISM_BF16) return fail(PRISM_E_DTYPE, "unknown dtype %d", static_cast<int>(vdt));
    if (!v || !a_map || !zone_shape || !block_offsets || !nb_dev) return fail(PRISM_E_ARG, "null pointer argument");
    if (C <= 0 || v_ld < C) return fail(PRISM_E_ARG, "bad channel count C = %lld or stride v_ld = %lld",
                                        static_cast<long long>(C), static_cast<long long>(v_ld));
    p = prism_shape_params{0.5, 0.25, 1e-6};
    if (prm) p = *prm;
    if (!(p.tau256 >= 0.0 && p.tau256 <= p.tau128 && p.tau128 <= 1.0) || !(p.eps > 0.0) || !std::isfinite(p.eps))
        return fail(PRISM_E_ARG, "thresholds must satisfy 0 <= tau256 <= tau128 <= 1 and eps > 0");
    return PRISM_OK;
}

// the launches of prism_zone_shapes on checked arguments and a large enough
// scratch (a workspace, or the fixed array of the no-allocation call)
prism_status zone_shapes_launch(int32_t T, int32_t H, int32_t W, const void* v, prism_dtype vdt, int64_t C,
                                int64_t v_ld, const float* a_map, const prism_shape_params& p, uint8_t* zone_shape,
                                int32_t* block_offsets, int32_t* nb_dev, int32_t* nb_host, double* zone_stats,
                                void* ws, const int32_t* zone_order, hipStream_t stream) {
    const int64_t N = static_cast<int64_t>(T) * H * W;
    prism_status st = PRISM_OK;
    Carver c(ws);
    const int nZ = static_cast<int>(N / prism::kZoneTokens);
    double* partial = c.take<double>(prism::zone_partial_doubles(nZ, C));
    double* rec = c.take<double>(static_cast<size_t>(nZ) * PRISM_ZS_STRIDE);
    st = hip_status(prism::launch_zone_shapes(v, vdt == PRISM_BF16, C, v_ld, a_map, grid_of(T, H, W, zone_order), nZ, p.tau128,
                                              p.tau256, p.eps, zone_shape, block_offsets, nb_dev, partial, rec, stream),
                    "zone_shapes launch");
    if (st != PRISM_OK) return st;
    if (zone_stats) {
        st = hip_status(hipMemcpyAsync(zone_stats, rec, static_cast<size_t>(nZ) * PRISM_ZS_STRIDE * sizeof(double),
                                       hipMemcpyDeviceToDevice, stream),
                        "zone_stats copy");
        if (st != PRISM_OK) return st;
    }
    if (nb_host) {
        st = hip_status(hipMemcpyAsync(nb_host, nb_dev, sizeof(int32_t), hipMemcpyDeviceToHost, stream), "NB copy");
        if (st != PRISM_OK) return st;
        st = hip_status(hipStreamSynchronize(stream), "stream synchronize");
    }
    return st;
}

}  // namespace

prism_status prism_zone_shapes(int32_t T, int32_t H, int32_t W, const void* v, prism_dtype vdt, int64_t C,
                               int64_t v_ld, const float* a_map, const prism_shape_params* prm, uint8_t* zone_shape,
                               int32_t* block_offsets, int32_t* nb_dev, int32_t* nb_host, double* zone_stats, void* ws,
                               size_t ws_bytes, const int32_t* zone_order, hipStream_t stream) {
    prism_shape_params p;
    prism_status st = check_zone_args(T, H, W, v, vdt, C, v_ld, a_map, prm, zone_shape, block_offsets, nb_dev, p);
    if (st != PRISM_OK) return st;
    const size_t need = zone_ws(static_cast<int64_t>(T) * H * W, C);
    if (!ws || ws_bytes < need)
        return fail(PRISM_E_WORKSPACE, "zone_shapes needs %zu workspace bytes, got %zu", need, ws ? ws_bytes : 0);
    return zone_shapes_launch(T, H, W, v, vdt, C, v_ld, a_map, p, zone_shape, block_offsets, nb_dev, nb_host,
                              zone_stats, ws, zone_order, stream);
}

// ---------------------------------------------------------------- zone shapes without allocation
//
// prism_zone_shapes_noalloc takes the scratch of prism_zone_shapes (the
// per-slab partial sums and the per-zone records) from this fixed array.
// Each GPU that the library runs on holds its own copy until the process
// ends.  On the host the array's name is only a stand-in, never a device
// address: the address is looked up once per device, with that device
// current, and kept in g_scratch, and only that address reaches a kernel.
// Every scratch value is written before it is read, so nothing is cleared
// between calls; calls that overlap on one GPU share the array and race.

static __device__ __align__(256) unsigned char scratch[PRISM_ZONE_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// the current device's address of `scratch`
prism_status current_scratch(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(PRISM_E_UNSUPPORTED, "device %d: the no-allocation scratch covers devices 0..%d", dev,
                    kMaxDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol, "scratch address");
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return PRISM_OK;
}

}  // namespace

prism_status prism_zone_shapes_noalloc(int32_t T, int32_t H, int32_t W, const void* v, prism_dtype vdt, int64_t C,
                                       int64_t v_ld, const float* a_map, const prism_shape_params* prm,
                                       uint8_t* zone_shape, int32_t* block_offsets, int32_t* nb_dev, int32_t* nb_host,
                                       double* zone_stats, const int32_t* zone_order, hipStream_t stream) {
    prism_shape_params p;
    prism_status st = check_zone_args(T, H, W, v, vdt, C, v_ld, a_map, prm, zone_shape, block_offsets, nb_dev, p);
    if (st != PRISM_OK) return st;
    const size_t need = zone_ws(static_cast<int64_t>(T) * H * W, C);
    if (need > PRISM_ZONE_SCRATCH_BYTES)
        return fail(PRISM_E_WORKSPACE,
                    "zone shapes of this grid need %zu scratch bytes, more than the %zu of the no-allocation call",
                    need, static_cast<size_t>(PRISM_ZONE_SCRATCH_BYTES));
    void* ws = nullptr;
    if ((st = current_scratch(&ws)) != PRISM_OK) return st;
    return zone_shapes_launch(T, H, W, v, vdt, C, v_ld, a_map, p, zone_shape, block_offsets, nb_dev, nb_host,
                              zone_stats, ws, zone_order, stream);
}

prism_status prism_block_permute(int32_t T, int32_t H, int32_t W, const uint8_t* zone_shape, const void* x, void* y,
                                 prism_dtype dt, int64_t row_elems, int64_t x_ld, int64_t y_ld, int32_t inverse,
                                 const int32_t* zone_order, hipStream_t stream) {
    prism_status st = check_grid(T, H, W);
    if (st != PRISM_OK) return st;
    if (dt != PRISM_F32 && dt != PRISM_BF16) return fail(PRISM_E_DTYPE, "unknown dtype %d", static_cast<int>(dt));
    if (!zone_shape || !x || !y) return fail(PRISM_E_ARG, "null pointer argument");
    if (row_elems <= 0 || x_ld < row_elems || y_ld < row_elems)
        return fail(PRISM_E_ARG, "bad row_elems = %lld or strides", static_cast<long long>(row_elems));
    if (inverse != 0 && inverse != 1) return fail(PRISM_E_ARG, "inverse must be 0 or 1");
    const int64_t N = static_cast<int64_t>(T) * H * W;
    const int eb = elem_bytes(dt);
    const char* xb = static_cast<const char*>(x);
    const char* yb = static_cast<const char*>(y);
    const int64_t xspan = ((N - 1) * x_ld + row_elems) * eb, yspan = ((N - 1) * y_ld + row_elems) * eb;
    if (xb < yb + yspan && yb < xb + xspan) return fail(PRISM_E_ARG, "x and y overlap");
    return hip_status(prism::launch_block_permute(x, y, eb, row_elems, x_ld, y_ld, zone_shape, grid_of(T, H, W, zone_order), N,
                                                  inverse, stream),
                      "block_permute launch");
}

prism_status prism_block_permute_heads(int32_t T, int32_t H, int32_t W, const uint8_t* zone_shape, const void* x,
                                       void* y, prism_dtype dt, int32_t heads, int32_t d, int64_t x_ld, int64_t x_hs,
                                       int64_t y_ld, int64_t y_hs, int32_t inverse, const int32_t* zone_order,
                                       hipStream_t stream) {
    prism_status st = check_grid(T, H, W);
    if (st != PRISM_OK) return st;
    if (dt != PRISM_F32 && dt != PRISM_BF16) return fail(PRISM_E_DTYPE, "unknown dtype %d", static_cast<int>(dt));
    if (!zone_shape || !x || !y) return fail(PRISM_E_ARG, "null pointer argument");
    if (heads <= 0 || d <= 0) return fail(PRISM_E_ARG, "heads = %d and d = %d must be positive", heads, d);
    if (x_ld < 0 || x_hs < 0 || y_ld < 0 || y_hs < 0) return fail(PRISM_E_ARG, "strides must be non-negative");
    if (inverse != 0 && inverse != 1) return fail(PRISM_E_ARG, "inverse must be 0 or 1");
    const int eb = elem_bytes(dt);
    const int64_t vec = 16 / eb;
    if (d % vec || x_ld % vec || x_hs % vec || y_ld % vec || y_hs % vec ||
        ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15))
        return fail(PRISM_E_UNSUPPORTED, "d, strides and pointers must be 16-byte multiples");
    const int64_t N = static_cast<int64_t>(T) * H * W;
    const char* xb = static_cast<const char*>(x);
    const char* yb = static_cast<const char*>(y);
    const int64_t xspan = ((N - 1) * x_ld + (heads - 1) * x_hs + d) * eb;
    const int64_t yspan = ((N - 1) * y_ld + (heads - 1) * y_hs + d) * eb;
    if (xb < yb + yspan && yb < xb + xspan) return fail(PRISM_E_ARG, "x and y overlap");
    return hip_status(prism::launch_block_permute_heads(x, y, eb, heads, d, x_ld, x_hs, y_ld, y_hs, zone_shape,
                                                        grid_of(T, H, W, zone_order), N, inverse, stream),
                      "block_permute_heads launch");
}

prism_status prism_select(const void* q, const void* k, prism_dtype dt, int64_t N, int32_t heads, int32_t d,
                          int64_t ld, int64_t hs, const int32_t* block_offsets, int32_t nb, int32_t top_k, double top_p,
                          float scale, int32_t* sel_offsets, int32_t* sel_idx, int64_t cap, int64_t* sel_total,
                          float* logits, void* ws, size_t ws_bytes, hipStream_t stream) {
    prism_status st = check_tokens(dt, N, heads, d, ld, hs, nb, cap);
    if (st != PRISM_OK) return st;
    if (!q || !k || !block_offsets || !sel_offsets || !sel_idx || !sel_total)
        return fail(PRISM_E_ARG, "null pointer argument");
    if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k)) & 15)
        return fail(PRISM_E_UNSUPPORTED, "q and k must be 16-byte aligned");
    if (top_k < 0 || !(top_p >= 0.0 && top_p <= 1.0)) return fail(PRISM_E_ARG, "need k >= 0 and 0 <= p <= 1");
    if (!std::isfinite(scale)) return fail(PRISM_E_ARG, "scale must be finite");
    const size_t need = prism_workspace_size(PRISM_OP_SELECT, N, heads, d, nb, cap);
    if (!ws || ws_bytes < need)
        return fail(PRISM_E_WORKSPACE, "select needs %zu workspace bytes, got %zu", need, ws ? ws_bytes : 0);
    Carver c(ws);
    SelectWs w = carve_select(c, heads, d, nb);
    float* L = logits ? logits : w.logits;
    return hip_status(prism::launch_select(q, k, dt == PRISM_BF16, heads, d, ld, hs, block_offsets, nb, top_k, top_p,
                                           scale, sel_offsets, sel_idx, cap, sel_total, L, logits != nullptr, w.pooled,
                                           w.row_count, w.row_thr, w.row_tie, stream),
                      "select launch");
}

prism_status prism_select_subblock(const void* q, const void* k, prism_dtype dt, int64_t N, int32_t heads, int32_t d,
                                   int64_t ld, int64_t hs, const int32_t* block_offsets, int32_t nb, int32_t top_k,
                                   double top_p, float scale, int32_t* sel_offsets, int32_t* sel_idx, int64_t cap,
                                   int64_t* sel_total, float* logits, void* ws, size_t ws_bytes, hipStream_t stream) {
    prism_status st = check_tokens(dt, N, heads, d, ld, hs, nb, cap);
    if (st != PRISM_OK) return st;
    if (!q || !k || !block_offsets || !sel_offsets || !sel_idx || !sel_total)
        return fail(PRISM_E_ARG, "null pointer argument");
    if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k)) & 15)
        return fail(PRISM_E_UNSUPPORTED, "q and k must be 16-byte aligned");
    if (top_k < 0 || !(top_p >= 0.0 && top_p <= 1.0)) return fail(PRISM_E_ARG, "need k >= 0 and 0 <= p <= 1");
    if (!std::isfinite(scale)) return fail(PRISM_E_ARG, "scale must be finite");
    if (N % 64 != 0) return fail(PRISM_E_ARG, "sub-block scoring needs N a multiple of 64 (N = %lld)",
                                 static_cast<long long>(N));
    if (N / 64 > 0x7FFFFFFF / 256) return fail(PRISM_E_UNSUPPORTED, "too many runs for one launch");
    const size_t need = prism_workspace_size(PRISM_OP_SELECT_SUB, N, heads, d, nb, cap);
    if (!ws || ws_bytes < need)
        return fail(PRISM_E_WORKSPACE, "sub-block select needs %zu workspace bytes, got %zu", need,
                    ws ? ws_bytes : 0);
    Carver c(ws);
    SubSelectWs w = carve_select_sub(c, N, heads, d, nb);
    float* L = logits ? logits : w.logits;
    return hip_status(prism::launch_select_subblock(q, k, dt == PRISM_BF16, heads, d, ld, hs, N, block_offsets, nb,
                                                    top_k, top_p, scale, sel_offsets, sel_idx, cap, sel_total, L,
                                                    logits != nullptr, w.sub, w.row_count, w.row_thr, w.row_tie,
                                                    stream),
                      "sub-block select launch");
}

namespace {

// The optional bf16 residual of O: NULL, or 16-byte aligned storage with o's
// layout; an fp32 O needs none.
prism_status check_residual(const void* o_res, prism_dtype dt) {
    if (!o_res) return PRISM_OK;
    if (dt != PRISM_BF16) return fail(PRISM_E_ARG, "o_res is for bf16 outputs only (pass NULL for fp32)");
    if (!aligned16(o_res)) return fail(PRISM_E_UNSUPPORTED, "o_res must be 16-byte aligned");
    return PRISM_OK;
}

// Checks shared by the exact and the routed forward.
prism_status check_fwd(const void* q, const void* k, const void* v, const void* o, const float* lse, prism_dtype dt,
                       int64_t N, int32_t heads, int32_t d, int64_t ld, int64_t hs, const int32_t* block_offsets,
                       int32_t nb, const int32_t* sel_offsets, const int32_t* sel_idx, int64_t cap, float scale) {
    prism_status st = check_tokens(dt, N, heads, d, ld, hs, nb, cap);
    if (st != PRISM_OK) return st;
    if (!q || !k || !v || !o || !lse || !block_offsets || !sel_offsets || !sel_idx)
        return fail(PRISM_E_ARG, "null pointer argument");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(PRISM_E_UNSUPPORTED, "token tensors must be 16-byte aligned");
    if (!std::isfinite(scale) || !(scale > 0.0f)) return fail(PRISM_E_ARG, "scale must be finite and positive");
    if (static_cast<int64_t>(N / 64) * heads > 0x7FFFFFFF)
        return fail(PRISM_E_UNSUPPORTED, "too many query tiles for one launch");
    return PRISM_OK;
}

// Element offset of head g0 in a bf16 token tensor, as a pointer.
const void* at_head_c(const void* p, int64_t g0, int64_t hs) {
    return p ? static_cast<const void*>(static_cast<const uint16_t*>(p) + g0 * hs) : nullptr;
}
void* at_head(void* p, int64_t g0, int64_t hs) {
    return p ? static_cast<void*>(static_cast<uint16_t*>(p) + g0 * hs) : nullptr;
}

// Exact forward over the tiles whose block is not marked in `skip` (NULL: all).
// The MFMA path takes the heads in groups (split_params); within a group the
// rows with long selected lists are split into key-range chunks (not on the
// routed path, which passes `skip`), the other tiles run in the visiting order
// of launch_tile_order, and a combine merges the chunks.
prism_status exact_fwd(const void* q, const void* k, const void* v, void* o, float* lse, void* o_res, prism_dtype dt,
                       int64_t N, int32_t heads, int32_t d, int64_t ld, int64_t hs, const int32_t* block_offsets,
                       int32_t nb, const int32_t* sel_offsets, const int32_t* sel_idx, int64_t cap,
                       const uint8_t* skip, const prism::RowMap& om, float scale, Carver& c, hipStream_t stream) {
    if (use_simt_attention(dt))
        return hip_status(prism::launch_attn_fwd_simt(q, k, v, o, lse, dt == PRISM_BF16, N, heads, d, ld, hs,
                                                      block_offsets, nb, sel_offsets, sel_idx, cap, skip, om,
                                                      scale, o_res, stream),
                          "attention forward launch");
    const SplitParams sp = split_params();
    const int64_t hg = group_heads(heads, sp);
    OrderWs w = carve_order(c, N, hg, nb);
    const bool split = !skip && sp.T0 > 0;
    prism::SplitWs sw{};
    if (!skip) sw = carve_split(c, N, hg, nb, d, sp);
    for (int64_t g0 = 0; g0 < heads; g0 += hg) {
        const int n = static_cast<int>(std::min<int64_t>(hg, heads - g0));
        const int32_t* so = sel_offsets + g0 * (nb + 1);
        const int32_t* si = sel_idx + g0 * cap;
        const void* qg = at_head_c(q, g0, hs);
        const void* kg = at_head_c(k, g0, hs);
        const void* vg = at_head_c(v, g0, hs);
        void* og = at_head(o, g0, om.hs);
        void* rg = at_head(o_res, g0, om.hs);
        float* lg = lse + g0 * N;
        const uint8_t* sk = skip ? skip + g0 * nb : nullptr;
        prism_status st;
        if (split) {
            st = hip_status(prism::launch_split_plan(so, si, cap, block_offsets, nb, n, N / 64, sp.W, sp.T0, sw, stream),
                            "split plan launch");
            if (st != PRISM_OK) return st;
            sk = sw.heavy;
        }
        st = hip_status(prism::launch_tile_order(so, si, cap, block_offsets, nb, n, N / 64, w.bucket, w.start, w.order,
                                                 stream),
                        "tile order launch");
        if (st != PRISM_OK) return st;
        st = hip_status(prism::launch_attn_fwd_mfma(qg, kg, vg, og, lg, N, n, d, ld, hs, block_offsets, nb, so, si, cap,
                                                    w.order, sk, om, scale, rg, stream),
                        "attention forward launch");
        if (st != PRISM_OK) return st;
        if (split) {
            st = hip_status(prism::launch_attn_fwd_split(qg, kg, vg, og, lg, N, n, d, ld, hs, block_offsets, nb, si, cap,
                                                         prism::split_view(sw, n), om, scale, rg, stream),
                            "split forward launch");
            if (st != PRISM_OK) return st;
        }
    }
    return PRISM_OK;
}

}  // namespace

prism_status prism_sparse_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, void* o_res,
                                   prism_dtype dt, int64_t N, int32_t heads, int32_t d, int64_t ld, int64_t hs,
                                   const int32_t* block_offsets, int32_t nb, const int32_t* sel_offsets,
                                   const int32_t* sel_idx, int64_t cap, float scale, const prism_raster_layout* out,
                                   void* ws, size_t ws_bytes, hipStream_t stream) {
    prism_status st = check_fwd(q, k, v, o, lse, dt, N, heads, d, ld, hs, block_offsets, nb, sel_offsets, sel_idx, cap,
                                scale);
    if (st != PRISM_OK) return st;
    if ((st = check_residual(o_res, dt)) != PRISM_OK) return st;
    prism::RowMap om;
    if ((st = row_map(out, dt, N, ld, hs, om)) != PRISM_OK) return st;
    const size_t need = prism_workspace_size(PRISM_OP_ATTN_FWD, N, heads, d, nb, cap);
    if (!ws || ws_bytes < need)
        return fail(PRISM_E_WORKSPACE, "forward needs %zu workspace bytes, got %zu", need, ws ? ws_bytes : 0);
    Carver c(ws);
    return exact_fwd(q, k, v, o, lse, o_res, dt, N, heads, d, ld, hs, block_offsets, nb, sel_offsets, sel_idx, cap,
                     nullptr, om, scale, c, stream);
}

prism_status prism_flat_route(const float* logits, int32_t heads, int32_t nb, double flat_ratio, uint8_t* flat,
                              double* sharpness, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!logits || !flat) return fail(PRISM_E_ARG, "null pointer argument");
    if (heads <= 0 || nb <= 0 || heads > 65535) return fail(PRISM_E_ARG, "need 0 < heads <= 65535 and nb > 0");
    if (!(flat_ratio >= 0.0 && flat_ratio <= 1.0)) return fail(PRISM_E_ARG, "need 0 <= flat_ratio <= 1");
    double* M = sharpness;
    if (!M) {
        const size_t need = prism_workspace_size(PRISM_OP_FLAT_ROUTE, 0, heads, 0, nb, 0);
        if (!ws || ws_bytes < need)
            return fail(PRISM_E_WORKSPACE, "flat routing needs %zu workspace bytes, got %zu", need, ws ? ws_bytes : 0);
        Carver c(ws);
        M = c.take<double>(static_cast<size_t>(heads) * nb);
    }
    const int n_flat = static_cast<int>(std::floor(flat_ratio * static_cast<double>(nb)));
    return hip_status(prism::launch_flat_route(logits, heads, nb, n_flat, M, flat, stream), "flat routing launch");
}

prism_status prism_routed_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, void* o_res,
                                   prism_dtype dt, int64_t N, int32_t heads, int32_t d, int64_t ld, int64_t hs,
                                   const int32_t* block_offsets, int32_t nb, const int32_t* sel_offsets,
                                   const int32_t* sel_idx, int64_t cap, const uint8_t* flat, float scale, void* ws,
                                   size_t ws_bytes, hipStream_t stream) {
    prism_status st = check_fwd(q, k, v, o, lse, dt, N, heads, d, ld, hs, block_offsets, nb, sel_offsets, sel_idx, cap,
                                scale);
    if (st != PRISM_OK) return st;
    if ((st = check_residual(o_res, dt)) != PRISM_OK) return st;
    if (!flat) return fail(PRISM_E_ARG, "null pointer argument");
    const size_t need = prism_workspace_size(PRISM_OP_ROUTED_FWD, N, heads, d, nb, cap);
    if (!ws || ws_bytes < need)
        return fail(PRISM_E_WORKSPACE, "routed forward needs %zu workspace bytes, got %zu", need, ws ? ws_bytes : 0);
    Carver c(ws);
    prism::RowMap om;
    row_map(nullptr, dt, N, ld, hs, om);
    st = exact_fwd(q, k, v, o, lse, o_res, dt, N, heads, d, ld, hs, block_offsets, nb, sel_offsets, sel_idx, cap, flat,
                   om, scale, c, stream);
    if (st != PRISM_OK) return st;
    float* kbar = c.take<float>(static_cast<size_t>(heads) * nb * d);
    float* vbar = c.take<float>(static_cast<size_t>(heads) * nb * d);
    const bool bf16 = dt == PRISM_BF16;
    st = hip_status(prism::launch_block_means(k, v, bf16, heads, d, ld, hs, block_offsets, nb, kbar, vbar, stream),
                    "block means launch");
    if (st != PRISM_OK) return st;
    return hip_status(prism::launch_attn_flat(q, kbar, vbar, o, lse, bf16, N, heads, d, ld, hs, block_offsets, nb,
                                              sel_offsets, sel_idx, cap, flat, scale, o_res, stream),
                      "flat attention launch");
}

namespace {

prism_status check_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                       const void* dq, const void* dk, const void* dv, prism_dtype dt, int64_t N, int32_t heads,
                       int32_t d, int64_t ld, int64_t hs, const int32_t* block_offsets, int32_t nb,
                       const int32_t* sel_offsets, const int32_t* sel_idx, int64_t cap, float scale) {
    prism_status st = check_tokens(dt, N, heads, d, ld, hs, nb, cap);
    if (st != PRISM_OK) return st;
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !block_offsets || !sel_offsets || !sel_idx)
        return fail(PRISM_E_ARG, "null pointer argument");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
        !aligned16(dk) || !aligned16(dv))
        return fail(PRISM_E_UNSUPPORTED, "token tensors must be 16-byte aligned");
    if (!std::isfinite(scale) || !(scale > 0.0f)) return fail(PRISM_E_ARG, "scale must be finite and positive");
    if (static_cast<int64_t>(N / 64) * heads > 0x7FFFFFFF)
        return fail(PRISM_E_UNSUPPORTED, "too many tiles for one launch");
    return PRISM_OK;
}

// dQ and dK/dV on the exact path, from a transposed CSR already built in w;
// rg (NULL for the plain backward) carries the routed extras.  dQ takes the
// heads in groups like the forward, with the same key-range split of long rows
// (not on the routed path); dK/dV then runs once over all heads.  `c` follows
// carve_bwd in the workspace.
prism_status exact_bwd(const void* q, const void* k, const void* v, const void* dout, const float* lse, void* dq,
                       void* dk, void* dv, prism_dtype dt, int64_t N, int32_t heads, int32_t d, int64_t ld, int64_t hs,
                       const int32_t* block_offsets, int32_t nb, const int32_t* sel_offsets, const int32_t* sel_idx,
                       int64_t cap, float scale, const BwdWs& w, const prism::RouteGrad* rg, const prism::RowMap& om,
                       Carver& c, hipStream_t stream) {
    if (use_simt_attention(dt))
        return hip_status(prism::launch_attn_bwd_simt(q, k, v, dout, lse, w.Dq, dq, dk, dv, dt == PRISM_BF16, N, heads,
                                                      d, ld, hs, block_offsets, nb, sel_offsets, sel_idx, w.tr_offsets,
                                                      w.tr_idx, cap, rg, om, scale, stream),
                          "attention backward launch");
    const SplitParams sp = split_params();
    const int64_t hg = group_heads(heads, sp);
    const bool split = !rg && sp.T0 > 0;
    prism::SplitWs sw{};
    if (!rg) sw = carve_split(c, N, hg, nb, d, sp);
    for (int64_t g0 = 0; g0 < heads; g0 += hg) {
        const int n = static_cast<int>(std::min<int64_t>(hg, heads - g0));
        const int32_t* so = sel_offsets + g0 * (nb + 1);
        const int32_t* si = sel_idx + g0 * cap;
        const void* qg = at_head_c(q, g0, hs);
        const void* kg = at_head_c(k, g0, hs);
        const void* vg = at_head_c(v, g0, hs);
        const void* dog = at_head_c(dout, g0, hs);
        void* dqg = at_head(dq, g0, om.hs);
        const float* lg = lse + g0 * N;
        float* Dg = w.Dq + g0 * N;
        const uint8_t* sk = rg && rg->skip_q ? rg->skip_q + g0 * nb : nullptr;
        prism_status st;
        if (split) {
            st = hip_status(prism::launch_split_plan(so, si, cap, block_offsets, nb, n, N / 64, sp.W, sp.T0, sw, stream),
                            "split plan launch");
            if (st != PRISM_OK) return st;
            sk = sw.heavy;
        }
        st = hip_status(prism::launch_tile_order(so, si, cap, block_offsets, nb, n, N / 64, w.obucket, w.ostart,
                                                 w.qorder, stream),
                        "tile order launch");
        if (st != PRISM_OK) return st;
        st = hip_status(prism::launch_attn_dq_mfma(qg, kg, vg, dog, lg, Dg, dqg, N, n, d, ld, hs, block_offsets, nb, so,
                                                   si, cap, w.qorder, sk, om, scale, stream),
                        "dQ launch");
        if (st != PRISM_OK) return st;
        if (split) {
            st = hip_status(prism::launch_attn_dq_split(qg, kg, vg, dog, lg, Dg, dqg, N, n, d, ld, hs, block_offsets, nb,
                                                        si, cap, prism::split_view(sw, n), om, scale, stream),
                            "split dQ launch");
            if (st != PRISM_OK) return st;
        }
    }
    prism_status st = hip_status(prism::launch_head_order(w.tr_offsets, w.tr_idx, block_offsets, nb, heads, cap,
                                                          w.hcost, w.horder, stream),
                                 "dK/dV head order launch");
    if (st != PRISM_OK) return st;
    return hip_status(prism::launch_attn_dkdv_mfma(q, k, v, dout, w.lse2, w.Dq, dk, dv, N, heads, d, ld, hs,
                                                   block_offsets, nb, w.tr_offsets, w.tr_idx, cap, w.horder, rg, om,
                                                   scale, stream),
                      "dK/dV launch");
}

}  // namespace

prism_status prism_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* o_res,
                                   const void* dout, const float* lse, void* dq, void* dk, void* dv, prism_dtype dt,
                                   int64_t N, int32_t heads, int32_t d, int64_t ld, int64_t hs,
                                   const int32_t* block_offsets, int32_t nb, const int32_t* sel_offsets,
                                   const int32_t* sel_idx, int64_t cap, float scale, const prism_raster_layout* io,
                                   void* ws, size_t ws_bytes, hipStream_t stream) {
    prism_status st = check_bwd(q, k, v, o, dout, lse, dq, dk, dv, dt, N, heads, d, ld, hs, block_offsets, nb,
                                sel_offsets, sel_idx, cap, scale);
    if (st != PRISM_OK) return st;
    if ((st = check_residual(o_res, dt)) != PRISM_OK) return st;
    prism::RowMap om;
    if ((st = row_map(io, dt, N, ld, hs, om)) != PRISM_OK) return st;
    const size_t need = prism_workspace_size(PRISM_OP_ATTN_BWD, N, heads, d, nb, cap);
    if (!ws || ws_bytes < need)
        return fail(PRISM_E_WORKSPACE, "backward needs %zu workspace bytes, got %zu", need, ws ? ws_bytes : 0);
    Carver c(ws);
    BwdWs w = carve_bwd(c, N, heads, group_heads(heads, split_params()), nb, cap);
    st = hip_status(prism::launch_bwd_dot(o, dout, dt == PRISM_BF16, N, heads, d, ld, hs, om, w.Dq, o_res, lse, w.lse2,
                                          stream),
                    "backward dot launch");
    if (st != PRISM_OK) return st;
    st = hip_status(prism::launch_transpose_csr(sel_offsets, sel_idx, nb, heads, cap, w.tcount, w.tr_offsets, w.tr_idx,
                                                w.scratch, nullptr, 0, stream),
                    "transposed selection launch");
    if (st != PRISM_OK) return st;
    return exact_bwd(q, k, v, dout, lse, dq, dk, dv, dt, N, heads, d, ld, hs, block_offsets, nb, sel_offsets, sel_idx,
                     cap, scale, w, nullptr, om, c, stream);
}

prism_status prism_routed_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* o_res,
                                   const void* dout, const float* lse, void* dq, void* dk, void* dv, prism_dtype dt,
                                   int64_t N, int32_t heads, int32_t d, int64_t ld, int64_t hs,
                                   const int32_t* block_offsets, int32_t nb, const int32_t* sel_offsets,
                                   const int32_t* sel_idx, int64_t cap, const uint8_t* flat, float scale, void* ws,
                                   size_t ws_bytes, hipStream_t stream) {
    prism_status st = check_bwd(q, k, v, o, dout, lse, dq, dk, dv, dt, N, heads, d, ld, hs, block_offsets, nb,
                                sel_offsets, sel_idx, cap, scale);
    if (st != PRISM_OK) return st;
    if ((st = check_residual(o_res, dt)) != PRISM_OK) return st;
    if (!flat) return fail(PRISM_E_ARG, "null pointer argument");
    const size_t need = prism_workspace_size(PRISM_OP_ROUTED_BWD, N, heads, d, nb, cap);
    if (!ws || ws_bytes < need)
        return fail(PRISM_E_WORKSPACE, "routed backward needs %zu workspace bytes, got %zu", need, ws ? ws_bytes : 0);
    Carver c(ws);
    BwdWs w = carve_bwd(c, N, heads, group_heads(heads, split_params()), nb, cap);
    RoutedBwdWs r = carve_routed_bwd(c, heads, d, nb, cap);
    const bool bf16 = dt == PRISM_BF16;
    prism::RowMap om;
    row_map(nullptr, dt, N, ld, hs, om);
    st = hip_status(prism::launch_bwd_dot(o, dout, bf16, N, heads, d, ld, hs, om, w.Dq, o_res, lse, w.lse2, stream),
                    "backward dot launch");
    if (st != PRISM_OK) return st;
    // key block -> sharp query blocks (exact dK/dV) and -> flat query blocks (block-mean gradients)
    st = hip_status(prism::launch_transpose_csr(sel_offsets, sel_idx, nb, heads, cap, w.tcount, w.tr_offsets, w.tr_idx,
                                                w.scratch, flat, 0, stream),
                    "transposed selection launch");
    if (st != PRISM_OK) return st;
    st = hip_status(prism::launch_transpose_csr(sel_offsets, sel_idx, nb, heads, cap, w.tcount, r.fto, r.fti,
                                                w.scratch, flat, 1, stream),
                    "transposed selection launch");
    if (st != PRISM_OK) return st;
    st = hip_status(prism::launch_block_means(k, v, bf16, heads, d, ld, hs, block_offsets, nb, r.kbar, r.vbar, stream),
                    "block means launch");
    if (st != PRISM_OK) return st;
    st = hip_status(prism::launch_flat_dq(q, dout, r.kbar, r.vbar, lse, w.Dq, dq, bf16, N, heads, d, ld, hs,
                                          block_offsets, nb, sel_offsets, sel_idx, cap, flat, scale, stream),
                    "flat dQ launch");
    if (st != PRISM_OK) return st;
    st = hip_status(prism::launch_flat_kgrad(q, dout, r.kbar, r.vbar, lse, w.Dq, bf16, N, heads, d, ld, hs,
                                             block_offsets, nb, r.fto, r.fti, cap, scale, r.dkbar, r.dvbar, stream),
                    "flat key-block gradient launch");
    if (st != PRISM_OK) return st;
    const prism::RouteGrad rg{flat, r.dkbar, r.dvbar};
    return exact_bwd(q, k, v, dout, lse, dq, dk, dv, dt, N, heads, d, ld, hs, block_offsets, nb, sel_offsets, sel_idx,
                     cap, scale, w, &rg, om, c, stream);
}

}  // extern "C"

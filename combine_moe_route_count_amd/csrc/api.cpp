// api.cpp - the C ABI of libmoe_route.so: argument checks, workspace carving
// and the launch sequence of each entry point.  Every check runs before the
// first launch, so a call that returns an error has enqueued nothing.
#include <hip/hip_runtime_api.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>

#include "moe_route.h"
#include "internal.hpp"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

constexpr int kTile = 1024;  // entries per routing tile (matches the rank kernel)
constexpr int64_t kMaxRows = INT32_MAX;

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok() { return MOE_OK; }

int hip_fail(hipError_t e, const char* where) {
    return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

int elem_bytes(moe_dtype d) { return d == MOE_F32 ? 4 : (d == MOE_BF16 ? 2 : 1); }

bool quantized(moe_dtype d) { return d == MOE_FP8_E4M3 || d == MOE_FP4_E2M1; }

// Workspace carving.  Sizes depend only on (T, K, E, R).
struct Carve {
    size_t total = 0;
    size_t take(size_t bytes) {
        const size_t at = total;
        total += align256(bytes);
        return at;
    }
};

struct RouteWs {  // one routing level: N entries over NK keys
    size_t local_rank, tile_cnt, tile_flags, off;
    int64_t tiles;
};

RouteWs carve_route(Carve& c, int64_t N, int NK) {
    RouteWs r;
    r.tiles = (N + kTile - 1) / kTile;
    r.local_rank = c.take(sizeof(int32_t) * (size_t)(N > 0 ? N : 1));
    r.tile_cnt = c.take(sizeof(int32_t) * (size_t)(r.tiles > 0 ? r.tiles : 1) * NK);
    r.tile_flags = c.take(sizeof(int32_t) * 2 * (size_t)(r.tiles > 0 ? r.tiles : 1));
    r.off = c.take(sizeof(int32_t) * ((size_t)NK + 1));
    return r;
}

struct Layout {
    RouteWs experts, ranks;
    size_t ticket;  // uint64_t arrival ticket of the one-launch routing
    size_t total;
};

Layout layout(int64_t T, int K, int E, int R) {
    Carve c;
    Layout L;
    L.ticket = c.take(sizeof(uint64_t));
    L.experts = carve_route(c, T * K, E);
    if (R > 0) L.ranks = carve_route(c, T * R, R);
    L.total = c.total;
    return L;
}

template <typename P>
P* at(void* ws, size_t off) {
    return (P*)((char*)ws + off);
}

int check_routing(int64_t T, int K, int E, const int32_t* idx) {
    if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T=%lld must be >= 0", (long long)T);
    if (K < 1 || K > 16) return fail(MOE_ERR_INVALID_ARG, "K=%d must be in [1,16]", K);
    if (E < 1 || E > 1024) return fail(MOE_ERR_INVALID_ARG, "E=%d must be in [1,1024]", E);
    if (T * (int64_t)K >= ((int64_t)1 << 31))
        return fail(MOE_ERR_INVALID_ARG, "T*K=%lld must be < 2^31", (long long)(T * K));
    if (T > 0 && !idx) return fail(MOE_ERR_INVALID_ARG, "idx is NULL");
    if (idx && !aligned(idx, 4)) return fail(MOE_ERR_INVALID_ARG, "idx is not 4-byte aligned");
    return MOE_OK;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
    if (ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                    ws_bytes, need);
    if (need > 0 && !ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
    if (ws && !aligned(ws, 256)) return fail(MOE_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    return MOE_OK;
}

int check_rows_ptr(const void* p, int64_t rows, const char* name) {
    if (rows > 0 && !p) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", name);
    if (p && !aligned(p, 16)) return fail(MOE_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
    return MOE_OK;
}

int check_H(int64_t H, bool fp8) {
    if (H <= 0 || H % 8 != 0)
        return fail(MOE_ERR_INVALID_ARG, "H=%lld must be a positive multiple of 8", (long long)H);
    if (fp8 && H % 128 != 0)
        return fail(MOE_ERR_INVALID_ARG, "H=%lld must be a multiple of 128 for fp8",
                    (long long)H);
    if (H > ((int64_t)1 << 24))
        return fail(MOE_ERR_INVALID_ARG, "H=%lld exceeds 2^24", (long long)H);
    return MOE_OK;
}

#define MOE_TRY(expr)                 \
    do {                              \
        const int st_ = (expr);       \
        if (st_ != MOE_OK) return st_; \
    } while (0)

#define MOE_HIP(expr, where)                  \
    do {                                      \
        const hipError_t e_ = (expr);         \
        if (e_ != hipSuccess) return hip_fail(e_, where); \
    } while (0)

// Rank pass + scan pass for one routing level.
struct LevelOut {
    int32_t* cnt_out = nullptr;
    int32_t* off_out = nullptr;
    int32_t* packed_cnt = nullptr;
    int32_t* packed_off = nullptr;
    int32_t* stats = nullptr;
};

moe::ScanArgs scan_args(void* ws, const RouteWs& L, int NK, int64_t cap, int64_t rows_limit,
                        const LevelOut& o, moe::StatsMode mode) {
    moe::ScanArgs sa;
    sa.tile_cnt = at<int32_t>(ws, L.tile_cnt);
    sa.tile_flags = at<int32_t>(ws, L.tile_flags);
    sa.tiles = (int)L.tiles;
    sa.NK = NK;
    sa.cap = cap;
    sa.rows_limit = rows_limit;
    sa.off_ws = at<int32_t>(ws, L.off);
    sa.cnt_out = o.cnt_out;
    sa.off_out = o.off_out;
    sa.packed_cnt = o.packed_cnt;
    sa.packed_off = o.packed_off;
    sa.stats = o.stats;
    sa.mode = mode;
    return sa;
}

hipError_t route_level(void* ws, const RouteWs& L, size_t ticket, moe::KeyKind kind,
                       const int32_t* idx, const int32_t* rank_slot, int64_t N, int K, int E,
                       int R, int NK, int64_t cap, int64_t rows_limit, const LevelOut& o,
                       moe::StatsMode mode, hipStream_t s) {
    const moe::ScanArgs sa = scan_args(ws, L, NK, cap, rows_limit, o, mode);
    int nbits = 0;
    while ((1 << nbits) < NK) ++nbits;
    if (L.tiles > 0 && NK <= moe::kFusedMaxKeys) {
        moe::RouteFusedArgs fa;
        fa.kind = kind;
        fa.idx = idx;
        fa.rank_slot = rank_slot;
        fa.N = N;
        fa.K = K;
        fa.E = E;
        fa.R = R;
        fa.nbits = nbits;
        fa.local_rank = at<int32_t>(ws, L.local_rank);
        fa.scan = sa;
        fa.ticket = at<uint64_t>(ws, ticket);
        return moe::launch_route_fused(fa, s);
    }
    moe::RankArgs ra;
    ra.kind = kind;
    ra.idx = idx;
    ra.rank_slot = rank_slot;
    ra.N = N;
    ra.K = K;
    ra.E = E;
    ra.R = R;
    ra.NK = NK;
    ra.local_rank = at<int32_t>(ws, L.local_rank);
    ra.tile_cnt = sa.tile_cnt;
    ra.tile_flags = (int32_t*)sa.tile_flags;
    hipError_t e = moe::launch_rank(ra, s);
    if (e != hipSuccess) return e;
    return moe::launch_scan(sa, s);
}

moe::SlotArgs slot_args(void* ws, const RouteWs& L, const int32_t* idx, int K, int E, int64_t cap,
                        int64_t packed_rows) {
    moe::SlotArgs a;
    a.idx = idx;
    a.local_rank = at<int32_t>(ws, L.local_rank);
    a.tile_base = at<int32_t>(ws, L.tile_cnt);
    a.off = at<int32_t>(ws, L.off);
    a.K = K;
    a.E = E;
    a.cap = cap;
    a.packed_rows = packed_rows;
    return a;
}

}  // namespace

MOE_API int moe_version(void) { return (1 << 16) | 2; }

MOE_API const char* moe_geometry(void) { return moe::geometry_text(); }

MOE_API const char* moe_last_error(void) { return g_last_error.c_str(); }

MOE_API size_t moe_workspace_size(int64_t T, int K, int E, int R) {
    if (T < 0 || K < 1 || E < 1 || R < 0) return 0;
    return layout(T, K, E, R).total;
}

MOE_API int moe_route_count(const int32_t* idx, int64_t T, int K, int E, int32_t* cnt,
                            int32_t* off, int32_t* stats, void* ws, size_t ws_bytes,
                            void* stream) {
    MOE_TRY(check_routing(T, K, E, idx));
    if (!cnt || !off) return fail(MOE_ERR_INVALID_ARG, "cnt and off must be non-NULL");
    const Layout L = layout(T, K, E, 0);
    MOE_TRY(check_ws(ws, ws_bytes, L.total));
    LevelOut o;
    o.cnt_out = cnt;
    o.off_out = off;
    o.stats = stats;
    MOE_HIP(route_level(ws, L.experts, L.ticket, moe::KeyKind::Experts, idx, nullptr, T * K, K, E, 0, E, 0,
                        INT64_MAX, o, moe::StatsMode::Plain, (hipStream_t)stream),
            "moe_route_count");
    return ok();
}

namespace {

// Payload checks shared by the dispatch entry points: bf16 -> bf16 or fp8
// (pack), f32 -> f32, pre-quantized fp8 -> fp8 with its scale rows.
int check_payload(const void* x, moe_dtype x_dt, const float* x_scales, int64_t T, int64_t H,
                  int64_t packed_rows, const void* packed_x, moe_dtype packed_dt,
                  const float* packed_scales) {
    if (x_dt != MOE_BF16 && x_dt != MOE_F32 && x_dt != MOE_FP8_E4M3)
        return fail(MOE_ERR_INVALID_ARG, "x dtype must be MOE_BF16, MOE_F32 or MOE_FP8_E4M3");
    if (packed_dt != MOE_BF16 && packed_dt != MOE_F32 && !quantized(packed_dt))
        return fail(MOE_ERR_INVALID_ARG, "unknown packed dtype %d", (int)packed_dt);
    const bool fp8_out = quantized(packed_dt);
    if (packed_dt != x_dt && !fp8_out)
        return fail(MOE_ERR_INVALID_ARG, "packed dtype must equal x dtype or be fp8/fp4");
    if (fp8_out && x_dt == MOE_F32)
        return fail(MOE_ERR_UNSUPPORTED, "fp8/fp4 packing is implemented for bf16 input only");
    if (x_dt == MOE_FP8_E4M3 && packed_dt != MOE_FP8_E4M3)
        return fail(MOE_ERR_INVALID_ARG, "pre-quantized fp8 input goes to fp8 rows");
    MOE_TRY(check_H(H, fp8_out));
    if (packed_rows < 0 || packed_rows > kMaxRows)
        return fail(MOE_ERR_INVALID_ARG, "packed_rows must be in [0, 2^31-1]");
    MOE_TRY(check_rows_ptr(x, T, "x"));
    MOE_TRY(check_rows_ptr(packed_x, packed_rows, "packed_x"));
    if (fp8_out && packed_rows > 0 && !packed_scales)
        return fail(MOE_ERR_INVALID_ARG, "packed_scales is NULL for fp8");
    if (!fp8_out && packed_scales)
        return fail(MOE_ERR_INVALID_ARG, "packed_scales must be NULL unless fp8");
    if (packed_scales && !aligned(packed_scales, 4))
        return fail(MOE_ERR_INVALID_ARG, "packed_scales is not 4-byte aligned");
    if (x_dt == MOE_FP8_E4M3 && T > 0 && !x_scales)
        return fail(MOE_ERR_INVALID_ARG, "x_scales is NULL for pre-quantized input");
    if (x_dt != MOE_FP8_E4M3 && x_scales)
        return fail(MOE_ERR_INVALID_ARG, "x_scales must be NULL unless x is fp8");
    if (x_scales && !aligned(x_scales, 4))
        return fail(MOE_ERR_INVALID_ARG, "x_scales is not 4-byte aligned");
    return MOE_OK;
}

moe::ScatterArgs scatter_args(const void* x, moe_dtype x_dt, const float* x_scales, int64_t T,
                              int64_t H, moe_dtype packed_dt, void* packed_x, float* packed_scales,
                              int32_t* packed_src, int64_t* tok_map) {
    moe::ScatterArgs sa{};
    sa.x = x;
    sa.x_scales = x_dt == MOE_FP8_E4M3 ? x_scales : nullptr;
    sa.T = T;
    sa.H = H;
    sa.x_bytes = elem_bytes(x_dt);
    sa.fp8 = quantized(packed_dt) && x_dt == MOE_BF16;
    sa.fp4 = packed_dt == MOE_FP4_E2M1;
    sa.replay = false;
    sa.packed = packed_x;
    sa.scales = packed_scales;
    sa.packed_src = packed_src;
    sa.tok_map = tok_map;
    return sa;
}

// Every argument check of a routed dispatch except the workspace.
int check_dispatch(const void* x, moe_dtype x_dt, const float* x_scales, int64_t T, int64_t H,
                   const int32_t* idx, int K, int E, int64_t cap, int64_t packed_rows,
                   const void* packed_x, moe_dtype packed_dt, const float* packed_scales,
                   const int32_t* packed_cnt, const int32_t* packed_src, const int64_t* tok_map) {
    MOE_TRY(check_routing(T, K, E, idx));
    MOE_TRY(check_payload(x, x_dt, x_scales, T, H, packed_rows, packed_x, packed_dt,
                          packed_scales));
    if (cap < 0) return fail(MOE_ERR_INVALID_ARG, "cap must be >= 0");
    if (!packed_cnt) return fail(MOE_ERR_INVALID_ARG, "packed_cnt is NULL");
    if (packed_rows > 0 && !packed_src) return fail(MOE_ERR_INVALID_ARG, "packed_src is NULL");
    if (T > 0 && !tok_map) return fail(MOE_ERR_INVALID_ARG, "tok_map is NULL");
    if (tok_map && !aligned(tok_map, 8)) return fail(MOE_ERR_INVALID_ARG, "tok_map is not 8-byte aligned");
    return MOE_OK;
}

int dispatch_impl(const void* x, moe_dtype x_dt, const float* x_scales, int64_t T, int64_t H,
                  const int32_t* idx, int K, int E, int64_t cap, int64_t packed_rows,
                  void* packed_x, moe_dtype packed_dt, float* packed_scales, int32_t* packed_cnt,
                  int32_t* packed_off, int32_t* packed_src, int64_t* tok_map, int32_t* stats,
                  void* ws, size_t ws_bytes, void* stream) {
    MOE_TRY(check_dispatch(x, x_dt, x_scales, T, H, idx, K, E, cap, packed_rows, packed_x,
                           packed_dt, packed_scales, packed_cnt, packed_src, tok_map));
    const Layout L = layout(T, K, E, 0);
    MOE_TRY(check_ws(ws, ws_bytes, L.total));
    hipStream_t s = (hipStream_t)stream;

    moe::ScatterArgs sa = scatter_args(x, x_dt, x_scales, T, H, packed_dt, packed_x,
                                       packed_scales, packed_src, tok_map);
    sa.slot = slot_args(ws, L.experts, idx, K, E, cap, packed_rows);

    LevelOut o;
    o.packed_cnt = packed_cnt;
    o.packed_off = packed_off;
    o.stats = stats;
    if (moe::dispatch_small_fits(T, K, E)) {   // one routing tile: routing and scatter in one launch
        MOE_HIP(moe::launch_dispatch_small(
                    sa, scan_args(ws, L.experts, E, cap, packed_rows, o, moe::StatsMode::Plain), s),
                "dispatch (one launch)");
        return ok();
    }
    MOE_HIP(route_level(ws, L.experts, L.ticket, moe::KeyKind::Experts, idx, nullptr, T * K, K, E,
                        0, E, cap, packed_rows, o, moe::StatsMode::Plain, s),
            "dispatch routing");
    MOE_HIP(moe::launch_scatter(sa, s), "dispatch scatter");
    return ok();
}

}  // namespace

MOE_API int moe_dispatch(const void* x, moe_dtype x_dt, int64_t T, int64_t H, const int32_t* idx,
                         int K, int E, int64_t cap, int64_t packed_rows, void* packed_x,
                         moe_dtype packed_dt, float* packed_scales, int32_t* packed_cnt,
                         int32_t* packed_off, int32_t* packed_src, int64_t* tok_map,
                         int32_t* stats, void* ws, size_t ws_bytes, void* stream) {
    if (x_dt == MOE_FP8_E4M3)
        return fail(MOE_ERR_INVALID_ARG, "fp8 input carries scales: use moe_dispatch_prequant");
    return dispatch_impl(x, x_dt, nullptr, T, H, idx, K, E, cap, packed_rows, packed_x, packed_dt,
                         packed_scales, packed_cnt, packed_off, packed_src, tok_map, stats, ws,
                         ws_bytes, stream);
}

MOE_API int moe_dispatch_noalloc(const void* x, moe_dtype x_dt, int64_t T, int64_t H,
                                 const int32_t* idx, int K, int E, int64_t cap, int64_t packed_rows,
                                 void* packed_x, moe_dtype packed_dt, float* packed_scales,
                                 int32_t* packed_cnt, int32_t* packed_off, int32_t* packed_src,
                                 int64_t* tok_map, int32_t* stats, void* stream) {
    if (x_dt == MOE_FP8_E4M3)
        return fail(MOE_ERR_INVALID_ARG, "fp8 input carries scales: use moe_dispatch_prequant");
    // every argument check runs before the workspace lookup (which may touch
    // the device once) and before any launch
    MOE_TRY(check_dispatch(x, x_dt, nullptr, T, H, idx, K, E, cap, packed_rows, packed_x,
                           packed_dt, packed_scales, packed_cnt, packed_src, tok_map));
    const size_t need = layout(T, K, E, 0).total;
    if (need > moe::kScratchBytes)
        return fail(MOE_ERR_WORKSPACE,
                    "T=%lld K=%d E=%d needs a %zu-byte workspace, more than the %zu bytes of the "
                    "static one: use moe_dispatch with a workspace",
                    (long long)T, K, E, need, moe::kScratchBytes);
    // A call's launches (routing, then the scatter reading the routing's results
    // from the shared array) are enqueued as one unit: two host threads calling
    // on one stream cannot interleave their launches, so the stream orders whole
    // calls.  Only the enqueue is serialized; nothing waits for the device.
    static std::mutex enqueue_mu;
    std::lock_guard<std::mutex> lock(enqueue_mu);
    void* ws = nullptr;
    MOE_HIP(moe::scratch_for_stream((hipStream_t)stream, &ws), "moe_dispatch_noalloc workspace");
    return dispatch_impl(x, x_dt, nullptr, T, H, idx, K, E, cap, packed_rows, packed_x, packed_dt,
                         packed_scales, packed_cnt, packed_off, packed_src, tok_map, stats, ws,
                         moe::kScratchBytes, stream);
}

MOE_API int moe_dispatch_prequant(const uint8_t* x_q, const float* x_scales, int64_t T, int64_t H,
                                  const int32_t* idx, int K, int E, int64_t cap,
                                  int64_t packed_rows, uint8_t* packed_x, float* packed_scales,
                                  int32_t* packed_cnt, int32_t* packed_off, int32_t* packed_src,
                                  int64_t* tok_map, int32_t* stats, void* ws, size_t ws_bytes,
                                  void* stream) {
    return dispatch_impl(x_q, MOE_FP8_E4M3, x_scales, T, H, idx, K, E, cap, packed_rows, packed_x,
                         MOE_FP8_E4M3, packed_scales, packed_cnt, packed_off, packed_src, tok_map,
                         stats, ws, ws_bytes, stream);
}

MOE_API int moe_dispatch_replay(const void* x, moe_dtype x_dt, const float* x_scales, int64_t T,
                                int64_t H, const int64_t* tok_map, int K, int64_t packed_rows,
                                void* packed_x, moe_dtype packed_dt, float* packed_scales,
                                void* stream) {
    if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T=%lld must be >= 0", (long long)T);
    if (K < 1 || K > 16) return fail(MOE_ERR_INVALID_ARG, "K=%d must be in [1,16]", K);
    if (T * (int64_t)K >= ((int64_t)1 << 31))
        return fail(MOE_ERR_INVALID_ARG, "T*K=%lld must be < 2^31", (long long)(T * K));
    MOE_TRY(check_payload(x, x_dt, x_scales, T, H, packed_rows, packed_x, packed_dt,
                          packed_scales));
    if (T > 0 && !tok_map) return fail(MOE_ERR_INVALID_ARG, "tok_map is NULL");
    if (tok_map && !aligned(tok_map, 8)) return fail(MOE_ERR_INVALID_ARG, "tok_map is not 8-byte aligned");
    moe::ScatterArgs sa = scatter_args(x, x_dt, x_scales, T, H, packed_dt, packed_x,
                                       packed_scales, nullptr, const_cast<int64_t*>(tok_map));
    sa.replay = true;
    sa.slot = moe::SlotArgs{};
    sa.slot.K = K;
    sa.slot.packed_rows = packed_rows;
    MOE_HIP(moe::launch_scatter(sa, (hipStream_t)stream), "moe_dispatch_replay");
    return ok();
}

MOE_API int moe_combine(const void* y, moe_dtype y_dt, int64_t y_rows, int64_t H,
                        const int64_t* tok_map, const float* w, int64_t T, int K, int E,
                        const moe_dedup_plan* dd, void* out, moe_dtype out_dt,
                        float* out_weights, void* stream) {
    if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T must be >= 0");
    if (K < 1 || K > 16) return fail(MOE_ERR_INVALID_ARG, "K=%d must be in [1,16]", K);
    if (y_dt != MOE_BF16 && y_dt != MOE_F32)
        return fail(y_dt == MOE_FP8_E4M3 ? MOE_ERR_UNSUPPORTED : MOE_ERR_INVALID_ARG,
                    "y dtype must be MOE_BF16 or MOE_F32");
    if (out_dt != MOE_BF16 && out_dt != MOE_F32)
        return fail(MOE_ERR_INVALID_ARG, "out dtype must be MOE_BF16 or MOE_F32");
    MOE_TRY(check_H(H, false));
    if (y_rows < 0 || y_rows > kMaxRows)
        return fail(MOE_ERR_INVALID_ARG, "y_rows must be in [0, 2^31-1]");
    MOE_TRY(check_rows_ptr(y, y_rows, "y"));
    MOE_TRY(check_rows_ptr(out, T, "out"));
    if (T > 0 && (!tok_map || !w)) return fail(MOE_ERR_INVALID_ARG, "tok_map and w must be non-NULL");
    if (tok_map && !aligned(tok_map, 8)) return fail(MOE_ERR_INVALID_ARG, "tok_map is not 8-byte aligned");
    if (w && !aligned(w, 4)) return fail(MOE_ERR_INVALID_ARG, "w is not 4-byte aligned");
    if (out_weights && !aligned(out_weights, 4))
        return fail(MOE_ERR_INVALID_ARG, "out_weights is not 4-byte aligned");
    moe::CombineArgs a{};
    if (dd) {
        if (E < 1 || E > 1024) return fail(MOE_ERR_INVALID_ARG, "E=%d must be in [1,1024]", E);
        if (dd->R < 1 || dd->R > 32 || E % dd->R != 0)
            return fail(MOE_ERR_INVALID_ARG, "R=%d must be in [1,32] and divide E=%d", dd->R, E);
        if (T > 0 && (!dd->idx || !dd->rank_slot))
            return fail(MOE_ERR_INVALID_ARG, "dedup plan idx and rank_slot must be non-NULL");
        if (dd->recv_rows < 0 || dd->recv_rows > kMaxRows)
            return fail(MOE_ERR_INVALID_ARG, "recv_rows must be in [0, 2^31-1]");
        if (dd->partial && !aligned(dd->partial, 16))
            return fail(MOE_ERR_INVALID_ARG, "partial is not 16-byte aligned");
        a.R = dd->R;
        a.idx = dd->idx;
        a.rank_slot = dd->rank_slot;
        a.recv_rows = dd->recv_rows;
        a.partial = dd->partial;
    }
    a.y = y;
    a.y_f32 = y_dt == MOE_F32;
    a.y_rows = y_rows;
    a.H = H;
    a.tok_map = tok_map;
    a.w = w;
    a.T = T;
    a.K = K;
    a.E = E;
    a.out = out;
    a.out_f32 = out_dt == MOE_F32;
    a.out_weights = out_weights;
    MOE_HIP(moe::launch_combine(a, (hipStream_t)stream), "moe_combine");
    return ok();
}

namespace {

int combine_quant(const uint8_t* q, bool fp4, const float* scales, int64_t y_rows, int64_t H,
                  const int64_t* tok_map, const float* w, int64_t T, int K, void* out,
                  moe_dtype out_dt, float* out_weights, void* stream, const char* name) {
    if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T must be >= 0");
    if (K < 1 || K > 16) return fail(MOE_ERR_INVALID_ARG, "K=%d must be in [1,16]", K);
    if (out_dt != MOE_BF16 && out_dt != MOE_F32)
        return fail(MOE_ERR_INVALID_ARG, "out dtype must be MOE_BF16 or MOE_F32");
    MOE_TRY(check_H(H, true));
    if (y_rows < 0 || y_rows > kMaxRows)
        return fail(MOE_ERR_INVALID_ARG, "y_rows must be in [0, 2^31-1]");
    MOE_TRY(check_rows_ptr(q, y_rows, "q"));
    if (scales && !aligned(scales, 4)) return fail(MOE_ERR_INVALID_ARG, "scales is not 4-byte aligned");
    MOE_TRY(check_rows_ptr(out, T, "out"));
    if (T > 0 && (!tok_map || !w)) return fail(MOE_ERR_INVALID_ARG, "tok_map and w must be non-NULL");
    if (tok_map && !aligned(tok_map, 8)) return fail(MOE_ERR_INVALID_ARG, "tok_map is not 8-byte aligned");
    if (w && !aligned(w, 4)) return fail(MOE_ERR_INVALID_ARG, "w is not 4-byte aligned");
    if (out_weights && !aligned(out_weights, 4))
        return fail(MOE_ERR_INVALID_ARG, "out_weights is not 4-byte aligned");
    moe::CombineArgs a{};
    a.y = q;
    a.y_fp8 = true;
    a.y_fp4 = fp4;
    a.y_scales = scales;
    a.y_rows = y_rows;
    a.H = H;
    a.tok_map = tok_map;
    a.w = w;
    a.T = T;
    a.K = K;
    a.out = out;
    a.out_f32 = out_dt == MOE_F32;
    a.out_weights = out_weights;
    MOE_HIP(moe::launch_combine(a, (hipStream_t)stream), name);
    return ok();
}

}  // namespace

MOE_API int moe_combine_fp8(const uint8_t* q, const float* scales, int64_t y_rows, int64_t H,
                            const int64_t* tok_map, const float* w, int64_t T, int K, void* out,
                            moe_dtype out_dt, float* out_weights, void* stream) {
    return combine_quant(q, false, scales, y_rows, H, tok_map, w, T, K, out, out_dt, out_weights,
                         stream, "moe_combine_fp8");
}

MOE_API int moe_combine_fp4(const uint8_t* q, const float* scales, int64_t y_rows, int64_t H,
                            const int64_t* tok_map, const float* w, int64_t T, int K, void* out,
                            moe_dtype out_dt, float* out_weights, void* stream) {
    return combine_quant(q, true, scales, y_rows, H, tok_map, w, T, K, out, out_dt, out_weights,
                         stream, "moe_combine_fp4");
}

MOE_API int moe_dedup_dispatch(const void* x, moe_dtype x_dt, int64_t T, int64_t H,
                               const int32_t* idx, int K, int E, int R, void* recv_x,
                               int64_t recv_rows, int32_t* recv_cnt, int32_t* recv_off,
                               int32_t* recv_src, int32_t* rank_slot, int64_t cap,
                               int64_t packed_rows, void* packed_x, int32_t* packed_cnt,
                               int32_t* packed_off, int32_t* packed_src, int64_t* tok_map,
                               int32_t* stats, void* ws, size_t ws_bytes, void* stream) {
    MOE_TRY(check_routing(T, K, E, idx));
    if (R < 1 || R > 32 || E % R != 0)
        return fail(MOE_ERR_INVALID_ARG, "R=%d must be in [1,32] and divide E=%d", R, E);
    if (T * (int64_t)R >= ((int64_t)1 << 31))
        return fail(MOE_ERR_INVALID_ARG, "T*R must be < 2^31");
    if (x_dt != MOE_BF16 && x_dt != MOE_F32)
        return fail(MOE_ERR_INVALID_ARG, "x dtype must be MOE_BF16 or MOE_F32");
    MOE_TRY(check_H(H, false));
    if (cap < 0) return fail(MOE_ERR_INVALID_ARG, "cap must be >= 0");
    if (packed_rows < 0 || packed_rows > kMaxRows)
        return fail(MOE_ERR_INVALID_ARG, "packed_rows must be in [0, 2^31-1]");
    if (recv_rows < 0 || recv_rows > kMaxRows)
        return fail(MOE_ERR_INVALID_ARG, "recv_rows must be in [0, 2^31-1]");
    MOE_TRY(check_rows_ptr(x, T, "x"));
    MOE_TRY(check_rows_ptr(recv_x, recv_rows, "recv_x"));
    MOE_TRY(check_rows_ptr(packed_x, packed_rows, "packed_x"));
    if (!recv_cnt || !recv_off || !packed_cnt)
        return fail(MOE_ERR_INVALID_ARG, "recv_cnt, recv_off and packed_cnt must be non-NULL");
    if (recv_rows > 0 && !recv_src) return fail(MOE_ERR_INVALID_ARG, "recv_src is NULL");
    if (packed_rows > 0 && !packed_src) return fail(MOE_ERR_INVALID_ARG, "packed_src is NULL");
    if (T > 0 && (!tok_map || !rank_slot))
        return fail(MOE_ERR_INVALID_ARG, "tok_map and rank_slot must be non-NULL");
    if (tok_map && !aligned(tok_map, 8)) return fail(MOE_ERR_INVALID_ARG, "tok_map is not 8-byte aligned");
    const Layout L = layout(T, K, E, R);
    MOE_TRY(check_ws(ws, ws_bytes, L.total));
    hipStream_t s = (hipStream_t)stream;
    const int xb = elem_bytes(x_dt);

    // stage 1 routing: (token, rank) pairs, one recv row each, in token order per rank
    LevelOut ro;
    ro.cnt_out = recv_cnt;
    ro.off_out = recv_off;
    ro.stats = stats;
    MOE_HIP(route_level(ws, L.ranks, L.ticket, moe::KeyKind::Ranks, idx, nullptr, T * R, K, E, R, R, 0,
                        recv_rows, ro, moe::StatsMode::RecvRows, s),
            "moe_dedup_dispatch rank routing");
    moe::RecvArgs rc;
    rc.x = x;
    rc.T = T;
    rc.H = H;
    rc.x_bytes = xb;
    rc.R = R;
    rc.local_rank = at<int32_t>(ws, L.ranks.local_rank);
    rc.tile_base = at<int32_t>(ws, L.ranks.tile_cnt);
    rc.off = at<int32_t>(ws, L.ranks.off);
    rc.recv_rows = recv_rows;
    rc.recv_x = recv_x;
    rc.recv_src = recv_src;
    rc.rank_slot = rank_slot;
    rc.idx = idx;
    rc.K = K;
    rc.E = E;
    rc.tok_map = tok_map;
    MOE_HIP(moe::launch_recv_copy(rc, s), "moe_dedup_dispatch recv copy");

    // stage 2 routing: surviving entries to expert slots, then local expansion
    LevelOut eo;
    eo.packed_cnt = packed_cnt;
    eo.packed_off = packed_off;
    eo.stats = stats;
    MOE_HIP(route_level(ws, L.experts, L.ticket, moe::KeyKind::Survivors, idx, rank_slot, T * K, K, E, R, E,
                        cap, packed_rows, eo, moe::StatsMode::Experts, s),
            "moe_dedup_dispatch expert routing");
    moe::ExpandArgs ea;
    ea.slot = slot_args(ws, L.experts, idx, K, E, cap, packed_rows);
    ea.T = T;
    ea.H = H;
    ea.x_bytes = xb;
    ea.R = R;
    ea.recv_src = recv_src;
    ea.recv_off = at<int32_t>(ws, L.ranks.off);
    ea.recv_rows = recv_rows;
    ea.recv_x = recv_x;
    ea.packed = packed_x;
    ea.packed_src = packed_src;
    ea.tok_map = tok_map;
    MOE_HIP(moe::launch_expand(ea, s), "moe_dedup_dispatch expansion");
    return ok();
}

MOE_API int moe_fp8_dequant(const uint8_t* q, const float* scales, int64_t rows, int64_t H,
                            void* y, void* stream) {
    if (rows < 0) return fail(MOE_ERR_INVALID_ARG, "rows must be >= 0");
    MOE_TRY(check_H(H, true));
    MOE_TRY(check_rows_ptr(q, rows, "q"));
    MOE_TRY(check_rows_ptr(y, rows, "y"));
    if (rows > 0 && !scales) return fail(MOE_ERR_INVALID_ARG, "scales is NULL");
    if (scales && !aligned(scales, 4)) return fail(MOE_ERR_INVALID_ARG, "scales is not 4-byte aligned");
    MOE_HIP(moe::launch_fp8_dequant(q, scales, rows, H, y, (hipStream_t)stream), "moe_fp8_dequant");
    return ok();
}

MOE_API int moe_copy16(const void* src, void* dst, int64_t bytes, void* stream) {
    if (bytes < 0 || bytes % 16 != 0)
        return fail(MOE_ERR_INVALID_ARG, "bytes=%lld must be a non-negative multiple of 16",
                    (long long)bytes);
    if (bytes > 0 && (!src || !dst)) return fail(MOE_ERR_INVALID_ARG, "src or dst is NULL");
    if ((src && !aligned(src, 16)) || (dst && !aligned(dst, 16)))
        return fail(MOE_ERR_INVALID_ARG, "src and dst must be 16-byte aligned");
    const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
    if (bytes > 0 && a < b + (uintptr_t)bytes && b < a + (uintptr_t)bytes)
        return fail(MOE_ERR_INVALID_ARG, "src and dst overlap");
    MOE_HIP(moe::launch_copy16(src, dst, bytes, (hipStream_t)stream), "moe_copy16");
    return ok();
}

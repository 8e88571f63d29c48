// internal.hpp - host-side launch interface between the C ABI layer (api.cpp)
// and the kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------------------
// routing: per-tile stable ranks, then the scan over tiles and keys
// ---------------------------------------------------------------------------

// Which key function maps a flat entry to its key.
enum class KeyKind {
    Experts,    // f = t*K + k, key = idx[f] when valid
    Ranks,      // f = t*R + r, key = r when r is in token t's rank mask
    Survivors,  // f = t*K + k, key = idx[f] when valid and its recv row exists
};

struct RankArgs {
    KeyKind kind;
    const int32_t* idx;
    const int32_t* rank_slot;  // Survivors only
    int64_t N;                 // entries (T*K or T*R)
    int K, E, R;
    int NK;                    // number of keys (E or R)
    int32_t* local_rank;       // [N]  stable rank inside the tile, -1 for no key
    int32_t* tile_cnt;         // [tiles][NK]
    int32_t* tile_flags;       // [tiles][2]  invalid ids, dropped-before-slot
};
hipError_t launch_rank(const RankArgs& a, hipStream_t s);

enum class StatsMode { Plain = 0, RecvRows = 1, Experts = 2 };

struct ScanArgs {
    int32_t* tile_cnt;          // [tiles][NK] counts in, exclusive per-key tile bases out
    const int32_t* tile_flags;  // [tiles][2]
    int tiles, NK;
    int64_t cap;                // > 0: padded segments of cap rows
    int64_t rows_limit;         // rows available (packed_rows / recv_rows)
    int32_t* off_ws;            // [NK+1] offsets, always written (read by the copy kernels)
    int32_t* cnt_out;           // [NK]   may be null
    int32_t* off_out;           // [NK+1] may be null
    int32_t* packed_cnt;        // [NK]   may be null
    int32_t* packed_off;        // [NK+1] may be null
    int32_t* stats;             // [3]    may be null
    StatsMode mode;
};
hipError_t launch_scan(const ScanArgs& a, hipStream_t s);

// ---------------------------------------------------------------------------
// row movement
// ---------------------------------------------------------------------------

struct SlotArgs {             // how an entry finds its packed row
    const int32_t* idx;
    const int32_t* local_rank;
    const int32_t* tile_base;  // [tiles][E]
    const int32_t* off;        // [E+1]
    int K, E;
    int64_t cap, packed_rows;
};

struct ScatterArgs {
    SlotArgs slot;
    const void* x;             // [T,H]
    const float* x_scales;     // pre-quantized input: [T,H/128] forwarded to scales; else null
    int64_t T, H;
    int x_bytes;               // 2 (bf16), 4 (f32) or 1 (pre-quantized e4m3)
    bool fp8;                  // pack bf16 -> e4m3 (or, with fp4, e2m1) + scales
    bool fp4;                  // with fp8: e2m1 codes, two per byte
    bool replay;               // rows from the cached tok_map; tok_map and packed_src not written
    void* packed;
    float* scales;
    int32_t* packed_src;
    int64_t* tok_map;          // written by the routed dispatch, read by the replay
};
hipError_t launch_scatter(const ScatterArgs& a, hipStream_t s);

// Routing and scatter of a dispatch in one launch when its routing is one tile
// and its keys fit the one-launch routing (dispatch_small_fits); sc is the
// routing's scan description (outputs, limits) as for the two-launch path.
bool dispatch_small_fits(int64_t T, int K, int E);
hipError_t launch_dispatch_small(const ScatterArgs& a, const ScanArgs& sc, hipStream_t s);

struct RecvArgs {             // dedup stage 1: one copy per (token, rank)
    const void* x;
    int64_t T, H;
    int x_bytes;
    int R;
    const int32_t* local_rank;  // rank-level ranks [T*R]
    const int32_t* tile_base;   // [tiles][R]
    const int32_t* off;         // [R+1]
    int64_t recv_rows;
    void* recv_x;
    int32_t* recv_src;
    int32_t* rank_slot;
    const int32_t* idx;         // [T,K] expert ids: entries with no recv row get tok_map -1 here
    int K, E;
    int64_t* tok_map;
};
hipError_t launch_recv_copy(const RecvArgs& a, hipStream_t s);

struct ExpandArgs {           // dedup stage 2: recv rows -> per-expert rows
    SlotArgs slot;
    int64_t T, H;
    int x_bytes;
    int R;
    const int32_t* recv_src;    // [recv_rows] token of each recv row
    const int32_t* recv_off;    // [R+1] rank segments of the recv rows (uncapped counts)
    int64_t recv_rows;
    const void* recv_x;
    void* packed;
    int32_t* packed_src;
    int64_t* tok_map;
};
hipError_t launch_expand(const ExpandArgs& a, hipStream_t s);

// ---------------------------------------------------------------------------
// routing in one launch: ranks, then the scan by the last routing workgroup
// ---------------------------------------------------------------------------

// Key counts up to which the one-launch routing is used: its rank pass keeps
// 16 waves x NK running counts in LDS.
constexpr int kFusedMaxKeys = 512;

// LDS of one gfx950 CU.  Launches that cap their residency reserve
// kLdsPerCu / n bytes of LDS per workgroup (never touched), so that at most n
// of their workgroups share a CU.
constexpr size_t kLdsPerCu = 160 * 1024;

struct RouteFusedArgs {
    KeyKind kind;
    const int32_t* idx;
    const int32_t* rank_slot;  // Survivors only
    int64_t N;          // entries
    int K, E, R;
    int nbits;          // key bits of NK
    int32_t* local_rank;
    ScanArgs scan;      // tiles, NK, tile counts in the workspace, outputs
    uint64_t* ticket;   // in the workspace: (tag << 32) | tiles finished
};
hipError_t launch_route_fused(const RouteFusedArgs& a, hipStream_t s);

hipError_t launch_fp8_dequant(const uint8_t* q, const float* scales, int64_t rows, int64_t H,
                              void* y, hipStream_t s);
hipError_t launch_copy16(const void* src, void* dst, int64_t bytes, hipStream_t s);

// Launch geometry of the row movers and gathers (geometry.cpp): the measured
// defaults, or the overrides of MOE_GEOM, read once.  Only how the work is split
// over workgroups and how many share a CU; never what is computed.
struct Geometry {
    int combine_chunk_units;   // lane-units per combine workgroup (64..256)
    int combine_wgs_per_cu;    // residency cap of the bf16 gather (0: none)
    int fp8_chunks;            // workgroups per token row of the e4m3 pack
    int fp8_wgs_per_cu;
    int copy_chunks;           // bit-copy scatter
    int copy_wgs_per_cu;
    int recv_chunks;           // dedup recv copy
    int recv_wgs_per_cu;
    int expand_chunks;         // dedup expansion
    int expand_wgs_per_cu;
};
const Geometry& geometry();
const char* geometry_text();   // "key=value,..." (and "; ignored: ..." for rejected overrides)

// The static workspace of moe_dispatch_noalloc (scratch.hip): its size, and the
// device address of the copy on the GPU that owns stream s (looked up once per
// GPU, with that GPU current).
constexpr size_t kScratchBytes = (size_t)4 << 20;
hipError_t scratch_for_stream(hipStream_t s, void** out);

// ---------------------------------------------------------------------------
// combine
// ---------------------------------------------------------------------------

struct CombineArgs {
    const void* y;
    bool y_f32;
    bool y_fp8;              // e4m3 codes, dequantized with y_scales (NULL: scale 1)
    bool y_fp4;              // with y_fp8: e2m1 codes, two per byte
    const float* y_scales;   // [y_rows, H/128]
    int64_t y_rows, H;
    const int64_t* tok_map;
    const float* w;
    int64_t T;
    int K, E;
    void* out;
    bool out_f32;
    float* out_weights;
    // dedup (R == 0: plain)
    int R;
    const int32_t* idx;
    const int32_t* rank_slot;
    int64_t recv_rows;
    float* partial;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);

}  // namespace moe

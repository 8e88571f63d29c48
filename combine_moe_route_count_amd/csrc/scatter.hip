// scatter.hip - row movement of the dispatch: token rows into per-expert
// packed rows (bit copies or the fused blockwise fp8 pack), the dedup recv copy
// and local expansion, and the fp8 dequantize helper.
//
// One workgroup per source token (the e4m3 pack: two, half a row each; the
// dedup expansion: one per recv row).  The token row is loaded once into
// registers with 16-byte loads (issued before the routing lookups, whose
// latency they hide), then stored to each of the token's destination rows with
// 16-byte stores, as the byte-generic row copy of "Draft: cco + flydsl
// dispatch/combine" (ROCm/mori pull 448, PR description: 16 B scatter; commit
// log: the dispatch copy is byte-generic, f32 works by element size) does on
// its side.  The fp8 pack follows the coalesced blockwise quantize of the same
// page (commit log, "Replace the lane-serial per-block quantize ..."): a
// 128-element block lives in 8 adjacent lanes of 16 elements each, its amax is
// a three-step DPP max inside the 8 lanes, and each lane stores its 16 fp8
// bytes with one 16-byte store.
#include "device_common.hpp"
#include "internal.hpp"
#include "route_device.hpp"
#include "rows_device.hpp"

namespace moe {

namespace {

constexpr int kCopyThreads = 256;

// ---------------------------------------------------------------------------
// plain dispatch, bit copy (bf16 or f32)
// ---------------------------------------------------------------------------
// Destination rows of token t, broadcast to every lane.  REPLAY: the rows of a
// cached tok_map, taken as they stand when inside [0, packed_rows) (nothing is
// written back); otherwise the routing lookup, which also writes tok_map and
// packed_src.
// meta: this workgroup writes tok_map and packed_src (one workgroup per token
// does when the row is split over several).
template <int DMAX, bool REPLAY>
__device__ __forceinline__ void token_rows(const ScatterArgs& a, int64_t t, int (&rows)[DMAX],
                                           bool meta = true) {
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int K = a.slot.K;
    int my_row = -1;
    if (REPLAY) {
        if (lane < K) {
            const int64_t r = a.tok_map[t * K + lane];
            my_row = (r >= 0 && r < a.slot.packed_rows) ? (int)r : -1;
        }
    } else {
        if (lane < K) my_row = entry_row(a.slot, t * K + lane);
        if (tid < K && meta) {
            a.tok_map[t * K + tid] = my_row;
            if (my_row >= 0) a.packed_src[my_row] = (int32_t)t;
        }
    }
    broadcast_rows<DMAX>(my_row, rows);
}

// Pre-quantized input: the token's row of block scales goes unchanged to every
// destination row.
template <int DMAX>
__device__ __forceinline__ void forward_scales(const ScatterArgs& a, int64_t t, const int (&rows)[DMAX],
                                               int nth) {
    const int64_t nblk = a.H / kFp8Block;
    for (int64_t i = threadIdx.x; i < nblk; i += nth) {
        float v = a.x_scales[t * nblk + i];
        asm volatile("" : "+v"(v));   // one wait for the load, not one per conditional store
#pragma unroll
        for (int d = 0; d < DMAX; ++d) {
            if (d >= a.slot.K) break;
            if (rows[d] >= 0) a.scales[(int64_t)rows[d] * nblk + i] = v;
        }
    }
}

// Destination rows of the routed and replayed scatters: the routing lookup
// (which also writes tok_map and packed_src) or the cached tok_map.
template <int DMAX, bool REPLAY>
struct LookupRows {
    const ScatterArgs& a;
    bool meta = true;   // this workgroup writes the token's tok_map / packed_src
    __device__ __forceinline__ void operator()(int64_t t, int (&rows)[DMAX]) const {
        token_rows<DMAX, REPLAY>(a, t, rows, meta);
    }
};

// The vectors of chunk c of a row of nvec vectors cut into chunks of C.
__device__ __forceinline__ VecRange chunk_range(int c, int C, int nvec) {
    return VecRange{c * C, min(nvec, c * C + C)};
}

// Moves the vectors r of token t's row; get_rows(t, rows) runs after the
// first loads of the row are issued, so their latency overlaps it.  first:
// this workgroup holds the row's first chunk and forwards the scale row.
template <int DMAX, int VPT, bool SC, class RowsFn>
__device__ __forceinline__ void scatter_copy_item(const ScatterArgs& a, int64_t t, int nth,
                                                  VecRange r, bool first, const RowsFn& get_rows) {
    const int tid = threadIdx.x;
    const int64_t row_bytes = a.H * a.x_bytes;
    const char* src = (const char*)a.x + t * row_bytes;

    u32x4 val[VPT];
    load_first_pass<VPT>(src, r, val, tid, nth);

    int rows[DMAX];
    get_rows(t, rows);
    // scales first: loading them after the row stores would reuse registers the
    // stores still read, and the compiler would wait for every store first
    if (SC && first) forward_scales<DMAX>(a, t, rows, nth);
    // SC: pre-quantized fp8 rows; otherwise bf16 / f32 row copies
    store_row_copies<DMAX, VPT, SC ? kStoreThrough : kStorePlain>(src, r, (char*)a.packed,
                                                                   row_bytes, rows, a.slot.K, val,
                                                                   tid, nth);
}

// ---------------------------------------------------------------------------
// plain dispatch, fused blockwise fp8 pack (bf16 in)
// ---------------------------------------------------------------------------

// Units [c*C, c*C + C) of token t's row (C a multiple of the 8 units of a
// scale block); get_rows(t, rows) runs once the first loads are issued.
template <int DMAX, int UPT, bool FP4, class RowsFn>
__device__ __forceinline__ void scatter_fp8_item(const ScatterArgs& a, int64_t t, int nth, int c,
                                                 int C, const RowsFn& get_rows) {
    const int tid = threadIdx.x;
    const int K = a.slot.K;
    const int64_t H = a.H;
    const int u0 = c * C;
    const int nunits = min((int)(H / 16), u0 + C);   // 16 elements per lane-unit; chunk end
    const int64_t nblk = H / kFp8Block;
    const int step = UPT * nth;
    const char* src = (const char*)a.x + t * H * 2;

    // the first pass of the row is in flight while the routing is looked up
    u32x4 lo[UPT], hi[UPT];
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
        const int u = u0 + tid + i * nth;
        lo[i] = u32x4{0, 0, 0, 0};
        hi[i] = u32x4{0, 0, 0, 0};
        if (u < nunits) {
            lo[i] = ld16_stream(src + (int64_t)u * 32);
            hi[i] = ld16_stream(src + (int64_t)u * 32 + 16);
        }
    }

    int rows[DMAX];
    get_rows(t, rows);
    const int64_t prow = FP4 ? H / 2 : H;      // bytes per packed row
    for (int base = u0;;) {
        u32x4 q[UPT];
        u32x2 q4[UPT];
        float s[UPT];
#pragma unroll
        for (int i = 0; i < UPT; ++i) {
            if (FP4) fp4_pack16(lo[i], hi[i], q4[i], s[i]);
            else fp8_pack16(lo[i], hi[i], q[i], s[i]);
        }
#pragma unroll
        for (int d = 0; d < DMAX; ++d) {
            if (d >= K) break;
            if (rows[d] < 0) continue;
            const RowOut<kStoreThrough> out((char*)a.packed + (int64_t)rows[d] * prow, prow);
            float* sc = a.scales + (int64_t)rows[d] * nblk;
#pragma unroll
            for (int i = 0; i < UPT; ++i) {
                const int u = base + tid + i * nth;
                if (u < nunits) {
                    if (FP4) out.st8(u * 8, q4[i]);
                    else out.st16(u * 16, q[i]);
                    if ((u & 7) == 0) sc[u >> 3] = s[i];  // cached: L2 merges the 32-byte pieces of a scale row
                }
            }
        }
        base += step;
        if (base >= nunits) break;
#pragma unroll
        for (int i = 0; i < UPT; ++i) {
            const int u = base + tid + i * nth;
            lo[i] = u32x4{0, 0, 0, 0};
            hi[i] = u32x4{0, 0, 0, 0};
            if (u < nunits) {
                lo[i] = ld16_stream(src + (int64_t)u * 32);
                hi[i] = ld16_stream(src + (int64_t)u * 32 + 16);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// dedup stage 1: one copy of x[t] per (t, r) in the token's rank mask
// ---------------------------------------------------------------------------
template <int DMAX, int VPT>
__device__ __forceinline__ void recv_copy_kernel_item(const RecvArgs& a, int64_t t, int nth,
                                                      VecRange vr, bool meta) {
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int R = a.R;
    const int64_t row_bytes = a.H * a.x_bytes;
    const char* src = (const char*)a.x + t * row_bytes;

    u32x4 val[VPT];
    load_first_pass<VPT>(src, vr, val, tid, nth);

    int my_row = -1;
    if (lane < R) {
        const int64_t f = t * R + lane;
        const int32_t lr = a.local_rank[f];
        if (lr >= 0) {
            const int64_t row = (int64_t)a.off[lane] + a.tile_base[(f / kTile) * R + lane] + lr;
            my_row = row < a.recv_rows ? (int)row : -1;
        }
    }
    if (tid < R && meta) {
        a.rank_slot[t * R + tid] = my_row;
        if (my_row >= 0) a.recv_src[my_row] = (int32_t)t;
    }
    // Entries that no recv row carries (no expert, an invalid id, or a recv row
    // past recv_rows) get their -1 here; the expansion, which walks the recv
    // rows, writes every other entry.  Rank of a valid e: e / (E/R).
    if (meta) {
        int e = -1;
        if (tid < a.K) e = a.idx[t * a.K + tid];
        const bool valid = tid < a.K && e >= 0 && e < a.E;
        const int rk = valid ? e / (a.E / R) : 0;
        const int rs = __shfl(my_row, rk, kWave);
        if (tid < a.K && (!valid || rs < 0)) a.tok_map[t * a.K + tid] = -1;
    }
    int rows[DMAX];
    broadcast_rows<DMAX>(my_row, rows);
    store_row_copies<DMAX, VPT, kStorePlain>(src, vr, (char*)a.recv_x, row_bytes, rows, R, val,
                                             tid, nth);
}

// ---------------------------------------------------------------------------
// dedup stage 2: each recv row expanded to its token's entries on the row's
// rank (the same slots a plain dispatch of the surviving ids gives)
// ---------------------------------------------------------------------------
// One workgroup per recv row, in recv-row order, as the owner of a rank's
// receive buffer walks it: the recv rows are read front to back and the
// writes go to the rank's E/R expert segments only.  The recv row is loaded
// first; its rank (the segment holding it) and its token are looked up
// meanwhile.  Walking the tokens instead (each token's recv rows, then its
// entries) took 552 us against about 525 for this order at T=16384 H=4096 E=64
// K=6 R=8 f32.
template <int KMAX, int VPT>
__device__ __forceinline__ void expand_kernel_item(const ExpandArgs& a, int64_t j, int nth,
                                                   VecRange vr, bool meta) {
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int K = a.slot.K;
    const int R = a.R;
    const int er = a.slot.E / R;
    const int64_t row_bytes = a.H * a.x_bytes;
    const char* src = (const char*)a.recv_x + j * row_bytes;

    u32x4 val[VPT];
    load_first_pass<VPT>(src, vr, val, tid, nth);

    // rank of row j: the last segment starting at or before j (empty segments
    // start where the next one does, so they are never the last)
    const uint64_t starts = ballot64(lane < R && (int64_t)a.recv_off[lane] <= j);
    const int r = starts ? 63 - __builtin_clzll(starts) : -1;   // recv_off[0] = 0: never -1
    const int32_t t = a.recv_src[j];

    int my_row = -1;
    bool on_rank = false;   // this lane's entry belongs to row j's rank
    if (lane < K && r >= 0 && t >= 0 && t < a.T) {
        const int64_t f = (int64_t)t * K + lane;
        const int32_t e = a.slot.idx[f];
        if (e >= 0 && e < a.slot.E && e / er == r) {
            on_rank = true;
            my_row = entry_row(a.slot, f);
        }
    }
    // every wave needs the rows for its broadcast; the first wave of the row's
    // first chunk writes them
    if (tid < K && on_rank && meta) {
        const int64_t f = (int64_t)t * K + tid;
        a.tok_map[f] = my_row;
        if (my_row >= 0) a.packed_src[my_row] = t;
    }
    int rows[KMAX];
    broadcast_rows<KMAX>(my_row, rows);
    store_row_copies<KMAX, VPT, kStoreThrough>(src, vr, (char*)a.packed, row_bytes, rows, K, val,
                                               tid, nth);
}

// ---------------------------------------------------------------------------
// kernels: grid-stride over their work items (tokens, token halves or recv rows)
// ---------------------------------------------------------------------------
// nth is the workgroup size, passed as an argument: blockDim.x comes from a
// 16-bit field that gfx9 can only read with a vector load, which the compiler
// repeats after every store it cannot prove disjoint and then waits for with
// vmcnt(0), i.e. for every store in flight.
// nch workgroups per row (chunks of C vectors); chunk 0 writes the row's
// routing outputs.
template <int DMAX, int VPT, bool REPLAY, bool SC>
__global__ __launch_bounds__(kCopyThreads) void scatter_copy_kernel(ScatterArgs a, int nth, int nch,
                                                                    int C) {
    const int nvec = (int)(a.H * a.x_bytes / 16);
    const int64_t items = a.T * nch;
    for (int64_t wi = blockIdx.x; wi < items; wi += gridDim.x) {
        const int64_t t = wi / nch;
        const int c = (int)(wi - t * nch);
        scatter_copy_item<DMAX, VPT, SC>(a, t, nth, chunk_range(c, C, nvec), c == 0,
                                         LookupRows<DMAX, REPLAY>{a, c == 0});
    }
}
template <int DMAX, int UPT, bool REPLAY, bool FP4>
__global__ __launch_bounds__(kCopyThreads) void scatter_fp8_kernel(ScatterArgs a, int nth, int nch,
                                                                   int C) {
    const int64_t items = a.T * nch;
    for (int64_t wi = blockIdx.x; wi < items; wi += gridDim.x) {
        const int64_t t = wi / nch;
        const int c = (int)(wi - t * nch);
        // chunk 0 writes the token's tok_map and packed_src
        scatter_fp8_item<DMAX, UPT, FP4>(a, t, nth, c, C, LookupRows<DMAX, REPLAY>{a, c == 0});
    }
}
template <int DMAX, int VPT>
__global__ __launch_bounds__(kCopyThreads) void recv_copy_kernel(RecvArgs a, int nth, int nch, int C) {
    const int nvec = (int)(a.H * a.x_bytes / 16);
    const int64_t items = a.T * nch;
    for (int64_t wi = blockIdx.x; wi < items; wi += gridDim.x) {
        const int64_t t = wi / nch;
        const int c = (int)(wi - t * nch);
        recv_copy_kernel_item<DMAX, VPT>(a, t, nth, chunk_range(c, C, nvec), c == 0);
    }
}

// Recv row of work item wi (whole rows, n of them).  Workgroups go to the 8
// XCDs round-robin in launch order; within each group of 64 items, XCD x takes
// 8 consecutive recv rows (the items x, x+8, ..., x+56), so the rows' tokens,
// expert ids and routing entries, neighbours in memory, are read through one
// XCD's L2, and the rank's packed rows that XCD writes lie close together.  The
// last n % 64 rows keep the plain order.  Measured on the dedup workload
// (T=16384 H=4096 E=64 K=6 R=8 f32): dispatch 748-756 -> 733-743 us; with 4
// rows per XCD 764-767 us, with 16 or 32 741-746 us.
__device__ __forceinline__ int64_t expand_row_of(int64_t wi, int64_t n) {
    constexpr int kRowsPerXcd = 8, kGroup = 8 * kRowsPerXcd;
    const int64_t grouped = (n / kGroup) * kGroup;
    if (wi >= grouped) return wi;
    const int64_t g = wi / kGroup;
    const int r = (int)(wi - g * kGroup);
    return g * kGroup + (int64_t)(r % 8) * kRowsPerXcd + r / 8;
}

template <int KMAX, int VPT>
__global__ __launch_bounds__(kCopyThreads) void expand_kernel(ExpandArgs a, int nth, int nch, int C) {
    // rows written by the recv copy: the uncapped total, clipped to recv_rows
    const int64_t total = a.recv_off[a.R];
    const int64_t n = total < a.recv_rows ? total : a.recv_rows;
    const int nvec = (int)(a.H * a.x_bytes / 16);
    const int64_t items = n * nch;
    for (int64_t wi = blockIdx.x; wi < items; wi += gridDim.x) {
        int64_t j;
        int c;
        if (nch == 1) {
            j = expand_row_of(wi, n);
            c = 0;
        } else {
            j = wi / nch;
            c = (int)(wi - j * nch);
        }
        expand_kernel_item<KMAX, VPT>(a, j, nth, chunk_range(c, C, nvec), c == 0);
    }
}

// ---------------------------------------------------------------------------
// dispatch of one routing tile (T*K <= 1024 entries: decode-sized calls) in one
// launch.  Every workgroup ranks the whole tile in its LDS (the rank pass of the
// routing, 16 waves x one 64-entry chunk), scans the key totals there and so
// knows every entry's row without waiting for any other workgroup.  Workgroups
// 0..T-1 then move their token's row as the routed scatter does; one more
// workgroup writes the routing outputs (packed_cnt, packed_off, stats) with the
// routing's own scan, off the token workgroups' path (done by the first token
// workgroup, that scan made the launch 1.3 us longer).  At T=32 H=6144 E=128
// K=8 the dispatch takes 8.8 us this way against 11.5 us as two launches
// (routing, then scatter), launch latency included.
// ---------------------------------------------------------------------------
constexpr int kSmallThreads = kTile;   // one thread per entry of the tile

enum class SmallMode { Copy, CopyScales, Fp8, Fp4 };

// The rows of token t in a one-tile dispatch: the whole tile ranked in LDS, the
// key totals scanned there, then the routing's entry rule with the tile's base
// 0.  Called by every thread of the workgroup, after the token row's first
// loads are issued.
template <int DMAX>
struct SmallRows {
    const ScatterArgs& a;
    int nbits;
    int32_t* run_all;     // LDS [16 waves][E]
    int32_t* rank_lds;    // LDS [kTile]
    int32_t* key_lds;     // LDS [kTile]: each entry's expert (valid where its rank is >= 0)
    int32_t* off_lds;     // LDS [E]
    int32_t* flags_lds;   // LDS [2]
    int32_t* wave_sums;   // LDS [16]
    __device__ __forceinline__ void operator()(int64_t t, int (&rows)[DMAX]) const {
        constexpr int kWaves = kSmallThreads / kWave;
        const int tid = threadIdx.x;
        const int lane = tid % kWave;
        const int K = a.slot.K;
        const int E = a.slot.E;
        rank_tile<kWaves, 1>(ExpertKeys{a.slot.idx, E}, a.T * K, E, nbits, 0, run_all, rank_lds,
                             nullptr, nullptr, flags_lds, key_lds);
        __syncthreads();
        int32_t tot = 0;
        if (tid < E)
            for (int w = 0; w < kWaves; ++w) tot += run_all[w * E + tid];
        const int32_t excl = block_exclusive_scan(tot, wave_sums);
        if (tid < E) off_lds[tid] = excl;
        __syncthreads();
        int my_row = -1;
        if (lane < K) {
            const int64_t f = t * K + lane;
            const int32_t lr = rank_lds[f];
            if (lr >= 0) {
                const int32_t e = key_lds[f];
                const int64_t base = a.slot.cap > 0 ? (int64_t)e * a.slot.cap : (int64_t)off_lds[e];
                const int64_t row = base + lr;
                if (!((a.slot.cap > 0 && lr >= a.slot.cap) || row >= a.slot.packed_rows))
                    my_row = (int)row;
            }
        }
        if (tid < K) {
            a.tok_map[t * K + tid] = my_row;
            if (my_row >= 0) a.packed_src[my_row] = (int32_t)t;
        }
        broadcast_rows<DMAX>(my_row, rows);
    }
};

// One workgroup per token (T <= 1024 here), then the routing outputs' workgroup.
template <int DMAX, SmallMode MODE>
__global__ __launch_bounds__(kSmallThreads) void dispatch_small_kernel(ScatterArgs a, ScanArgs sc,
                                                                       int nbits) {
    extern __shared__ int32_t run_all[];            // [16 waves][E] running counts
    __shared__ int32_t rank_lds[kTile];             // stable rank of each entry, -1: no key
    __shared__ int32_t key_lds[kTile];              // each entry's key
    __shared__ int32_t off_lds[kFusedMaxKeys];      // exclusive offsets of the keys
    __shared__ int32_t flags_lds[2];
    __shared__ int32_t wave_sums[kSmallThreads / kWave];
    const int64_t t = blockIdx.x;
    if (t == a.T) {   // the routing outputs
        constexpr int kWaves = kSmallThreads / kWave;
        rank_tile<kWaves, 1>(ExpertKeys{a.slot.idx, a.slot.E}, a.T * a.slot.K, a.slot.E, nbits, 0,
                             run_all, rank_lds, nullptr, nullptr, flags_lds);
        __syncthreads();
        const OneTileLds lds{run_all, kWaves, flags_lds};
        scan_tiles_body<false>(sc, &lds);
        return;
    }
    const SmallRows<DMAX> rows{a, nbits, run_all, rank_lds, key_lds, off_lds, flags_lds, wave_sums};
    const VecRange whole{0, (int)(a.H * a.x_bytes / 16)};
    if constexpr (MODE == SmallMode::Copy)
        scatter_copy_item<DMAX, 4, false>(a, t, kSmallThreads, whole, true, rows);
    else if constexpr (MODE == SmallMode::CopyScales)
        scatter_copy_item<DMAX, 4, true>(a, t, kSmallThreads, whole, true, rows);
    else
        scatter_fp8_item<DMAX, 2, MODE == SmallMode::Fp4>(a, t, kSmallThreads, 0, (int)(a.H / 16),
                                                          rows);
}

template <SmallMode MODE>
struct SmallLaunch {
    template <int D, int V>
    struct Launch {
        static void go(dim3 g, int, const ScanArgs& sc, const ScatterArgs& a, int nbits,
                       hipStream_t s) {
            const size_t lds = sizeof(int32_t) * (size_t)(kSmallThreads / kWave) * a.slot.E;
            dispatch_small_kernel<D, MODE><<<g, dim3(kSmallThreads), lds, s>>>(a, sc, nbits);
        }
    };
};

template <SmallMode MODE>
hipError_t small_by_dmax(int D, dim3 grid, const ScanArgs& sc, const ScatterArgs& a, int nbits,
                         hipStream_t s) {
    if (D <= 2) SmallLaunch<MODE>::template Launch<2, 0>::go(grid, 0, sc, a, nbits, s);
    else if (D <= 4) SmallLaunch<MODE>::template Launch<4, 0>::go(grid, 0, sc, a, nbits, s);
    else if (D <= 8) SmallLaunch<MODE>::template Launch<8, 0>::go(grid, 0, sc, a, nbits, s);
    else SmallLaunch<MODE>::template Launch<16, 0>::go(grid, 0, sc, a, nbits, s);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp8 dequantize: y = bf16(f32(q) * s[block])
// ---------------------------------------------------------------------------
constexpr int kDequantThreads = 256;

__global__ __launch_bounds__(kDequantThreads) void fp8_dequant_kernel(const uint8_t* __restrict__ q,
                                                          const float* __restrict__ scales,
                                                          int64_t units, int64_t H,
                                                          uint16_t* __restrict__ y) {
    const int64_t upr = H / 16;
    const int64_t nblk = H / kFp8Block;
    const int64_t stride = (int64_t)gridDim.x * kDequantThreads;
    for (int64_t u = (int64_t)blockIdx.x * kDequantThreads + threadIdx.x; u < units; u += stride) {
        const int64_t row = u / upr;
        const int64_t col = (u - row * upr) * 16;
        const u32x4 v = ld16(q + row * H + col);
        const float s = scales[row * nblk + col / kFp8Block];
        u32x4 o0, o1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float a0, a1, b0, b1;
            unpack_e4m3x2<false>(v[j], a0, a1);
            unpack_e4m3x2<true>(v[j], b0, b1);
            const uint32_t p0 = pack_bf16x2(a0 * s, a1 * s);
            const uint32_t p1 = pack_bf16x2(b0 * s, b1 * s);
            if (j < 2) {
                o0[2 * j] = p0;
                o0[2 * j + 1] = p1;
            } else {
                o1[2 * (j - 2)] = p0;
                o1[2 * (j - 2) + 1] = p1;
            }
        }
        st16(y + row * H + col, o0);
        st16(y + row * H + col + 8, o1);
    }
}

// ---------------------------------------------------------------------------
// 16-byte streaming copy: the plain copy the row movers are measured against
// ---------------------------------------------------------------------------
constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 4;   // 16-byte vectors per lane in flight

__global__ __launch_bounds__(kStreamThreads) void copy16_kernel(const u32x4* __restrict__ src,
                                                                u32x4* __restrict__ dst,
                                                                int64_t nvec) {
    const int64_t per_block = (int64_t)kStreamThreads * kStreamUnroll;
    const int64_t stride = (int64_t)gridDim.x * per_block;
    for (int64_t base = (int64_t)blockIdx.x * per_block; base < nvec; base += stride) {
        u32x4 v[kStreamUnroll];
#pragma unroll
        for (int i = 0; i < kStreamUnroll; ++i) {
            const int64_t j = base + i * kStreamThreads + threadIdx.x;
            if (j < nvec) v[i] = ld16_stream(src + j);
        }
#pragma unroll
        for (int i = 0; i < kStreamUnroll; ++i) {
            const int64_t j = base + i * kStreamThreads + threadIdx.x;
            if (j < nvec) st16_stream(dst + j, v[i]);
        }
    }
}

template <int VPT>
int copy_threads(int nvec) {
    int per = (nvec + VPT - 1) / VPT;
    int th = ((per + kWave - 1) / kWave) * kWave;
    if (th > kCopyThreads) th = kCopyThreads;
    if (th < kWave) th = kWave;
    return th;
}

// Launch<DMAX, VPT>::go(a, s) with the smallest DMAX (destinations per source
// row the kernel is compiled for) that holds D; each launch sizes its own grid.
template <template <int, int> class Launch, int VPT, class Args>
hipError_t by_dmax(int D, const Args& a, hipStream_t s) {
    if (D <= 2) Launch<2, VPT>::go(a, s);
    else if (D <= 4) Launch<4, VPT>::go(a, s);
    else if (D <= 8) Launch<8, VPT>::go(a, s);
    else if (D <= 16) Launch<16, VPT>::go(a, s);
    else Launch<32, VPT>::go(a, s);
    return hipGetLastError();
}

// Split of a token row over the workgroups of the quantizing scatter.  The
// e4m3 forms give each token two workgroups (half a row each) and cap the
// launch at 8 workgroups per CU through an LDS reservation: fewer rows are
// being written at any moment, and HBM takes the writes faster (the
// T=8192 H=7168 K=8 skewed dispatch: 123 -> 120 us; one workgroup per token
// capped at 3 per CU 120-122 us; four per token 125-127 us).  The e2m1 form,
// half the bytes per row, lost time under the same cap (79.5 -> 82.5 us) and
// keeps one uncapped workgroup per token.
struct Fp8Split {
    int nch;       // workgroups per token
    int C;         // lane-units per workgroup, a multiple of a scale block's 8
    int threads;
    size_t lds;
};

inline Fp8Split fp8_split(int64_t H, bool fp4) {
    const int nunits = (int)(H / 16);
    const int nblk = nunits / 8;
    Fp8Split sp;
    const int chunks = geometry().fp8_chunks, wpc = geometry().fp8_wgs_per_cu;
    sp.nch = fp4 ? 1 : (nblk < chunks ? nblk : chunks);
    sp.C = ((nblk + sp.nch - 1) / sp.nch) * 8;
    sp.threads = copy_threads<2>(sp.C);
    sp.lds = fp4 || wpc == 0 ? 0 : kLdsPerCu / wpc;
    return sp;
}

// Split of a row over the workgroups of a bit-copy kernel: nch workgroups per
// row of nvec 16-byte vectors, C vectors each, and at most wgs_per_cu of them
// resident on a CU (an LDS reservation; 0: no cap).
struct CopySplit {
    int nch;
    int C;
    int threads;
    size_t lds;
};
inline CopySplit copy_split(int nvec, int chunks, int wgs_per_cu) {
    CopySplit sp;
    sp.nch = chunks < 1 ? 1 : (chunks > nvec ? nvec : chunks);
    sp.C = (nvec + sp.nch - 1) / sp.nch;
    sp.nch = (nvec + sp.C - 1) / sp.C;   // no empty chunk
    sp.threads = copy_threads<4>(sp.C);
    sp.lds = wgs_per_cu > 0 ? kLdsPerCu / wgs_per_cu : 0;
    return sp;
}
// Token-row copies (bf16, f32, pre-quantized fp8): one uncapped workgroup per
// row (two or four chunks, or caps of 4-7 per CU, measured 0-8 us slower on the
// T=8192 H=7168 K=8 bf16 dispatch and the prefill one).  The dedup recv copy:
// two workgroups per 16 KB f32 row.  The dedup expansion: whole recv rows, at
// most 4 workgroups per CU; in recv-row order the resident workgroups then
// write a narrower band of the rank's expert segments (T=16384 H=4096 E=64 K=6
// R=8: dedup dispatch 788 -> 766 us with the cap, 760 us with the split recv
// copy; caps of 3 or 6 per CU, or chunked expansion rows, were slower).

inline dim3 copy_grid(int64_t items) {
    return dim3((unsigned)(items < kMaxGrid ? items : kMaxGrid));
}

template <bool REPLAY, bool SC>
struct CopyMode {
    template <int D, int V>
    struct Launch {
        static void go(const ScatterArgs& a, hipStream_t s) {
            const CopySplit sp = copy_split((int)(a.H * a.x_bytes / 16), geometry().copy_chunks,
                                            geometry().copy_wgs_per_cu);
            scatter_copy_kernel<D, V, REPLAY, SC>
                <<<copy_grid(a.T * sp.nch), dim3(sp.threads), sp.lds, s>>>(a, sp.threads, sp.nch, sp.C);
        }
    };
};
template <bool REPLAY, bool FP4>
struct Fp8Mode {
    template <int D, int V>
    struct Launch {
        static void go(const ScatterArgs& a, hipStream_t s) {
            const Fp8Split sp = fp8_split(a.H, FP4);
            const int64_t items = a.T * sp.nch;
            const dim3 grid((unsigned)(items < kMaxGrid ? items : kMaxGrid));
            scatter_fp8_kernel<D, V, REPLAY, FP4>
                <<<grid, dim3(sp.threads), sp.lds, s>>>(a, sp.threads, sp.nch, sp.C);
        }
    };
};
template <int D, int V>
struct LaunchRecv {
    static void go(const RecvArgs& a, hipStream_t s) {
        const CopySplit sp = copy_split((int)(a.H * a.x_bytes / 16), geometry().recv_chunks, geometry().recv_wgs_per_cu);
        recv_copy_kernel<D, V>
            <<<copy_grid(a.T * sp.nch), dim3(sp.threads), sp.lds, s>>>(a, sp.threads, sp.nch, sp.C);
    }
};
template <int D, int V>
struct LaunchExpand {
    static void go(const ExpandArgs& a, hipStream_t s) {
        const CopySplit sp = copy_split((int)(a.H * a.x_bytes / 16), geometry().expand_chunks,
                                         geometry().expand_wgs_per_cu);
        expand_kernel<D, V><<<copy_grid(a.recv_rows * sp.nch), dim3(sp.threads), sp.lds, s>>>(
            a, sp.threads, sp.nch, sp.C);
    }
};

}  // namespace

hipError_t launch_scatter(const ScatterArgs& a, hipStream_t s) {
    if (a.T == 0) return hipSuccess;
    const int K = a.slot.K;
    if (a.fp8) {
        if (a.fp4)
            return a.replay ? by_dmax<Fp8Mode<true, true>::Launch, 2>(K, a, s)
                            : by_dmax<Fp8Mode<false, true>::Launch, 2>(K, a, s);
        return a.replay ? by_dmax<Fp8Mode<true, false>::Launch, 2>(K, a, s)
                        : by_dmax<Fp8Mode<false, false>::Launch, 2>(K, a, s);
    }
    const bool sc = a.x_scales != nullptr;
    if (a.replay)
        return sc ? by_dmax<CopyMode<true, true>::Launch, 4>(K, a, s)
                  : by_dmax<CopyMode<true, false>::Launch, 4>(K, a, s);
    return sc ? by_dmax<CopyMode<false, true>::Launch, 4>(K, a, s)
              : by_dmax<CopyMode<false, false>::Launch, 4>(K, a, s);
}

bool dispatch_small_fits(int64_t T, int K, int E) {
    return T > 0 && T * K <= kTile && E <= kFusedMaxKeys;
}

hipError_t launch_dispatch_small(const ScatterArgs& a, const ScanArgs& sc, hipStream_t s) {
    if (!dispatch_small_fits(a.T, a.slot.K, a.slot.E) || a.replay || sc.tiles != 1)
        return hipErrorInvalidValue;
    int nbits = 0;
    while ((1 << nbits) < a.slot.E) ++nbits;
    const dim3 grid((unsigned)a.T + 1);   // the tokens, then the routing outputs
    if (a.fp8)
        return a.fp4 ? small_by_dmax<SmallMode::Fp4>(a.slot.K, grid, sc, a, nbits, s)
                     : small_by_dmax<SmallMode::Fp8>(a.slot.K, grid, sc, a, nbits, s);
    return a.x_scales ? small_by_dmax<SmallMode::CopyScales>(a.slot.K, grid, sc, a, nbits, s)
                      : small_by_dmax<SmallMode::Copy>(a.slot.K, grid, sc, a, nbits, s);
}

hipError_t launch_recv_copy(const RecvArgs& a, hipStream_t s) {
    if (a.T == 0) return hipSuccess;
    return by_dmax<LaunchRecv, 4>(a.R, a, s);
}

hipError_t launch_expand(const ExpandArgs& a, hipStream_t s) {
    if (a.T == 0 || a.recv_rows == 0) return hipSuccess;
    return by_dmax<LaunchExpand, 4>(a.slot.K, a, s);
}

hipError_t launch_fp8_dequant(const uint8_t* q, const float* scales, int64_t rows, int64_t H,
                              void* y, hipStream_t s) {
    const int64_t units = rows * (H / 16);
    if (units == 0) return hipSuccess;
    int64_t blocks = (units + kDequantThreads - 1) / kDequantThreads;
    if (blocks > 65536) blocks = 65536;
    fp8_dequant_kernel<<<dim3((unsigned)blocks), dim3(kDequantThreads), 0, s>>>(q, scales, units,
                                                                                H, (uint16_t*)y);
    return hipGetLastError();
}

hipError_t launch_copy16(const void* src, void* dst, int64_t bytes, hipStream_t s) {
    const int64_t nvec = bytes / 16;
    if (nvec == 0) return hipSuccess;
    const int64_t per_block = (int64_t)kStreamThreads * kStreamUnroll;
    int64_t blocks = (nvec + per_block - 1) / per_block;
    if (blocks > kMaxGrid) blocks = kMaxGrid;  // one pass per workgroup up to 64 GiB
    copy16_kernel<<<dim3((unsigned)blocks), dim3(kStreamThreads), 0, s>>>(
        (const u32x4*)src, (u32x4*)dst, nvec);
    return hipGetLastError();
}

}  // namespace moe

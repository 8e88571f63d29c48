// route_device.hpp - device bodies of the routing passes (stable per-tile
// ranks and the tile / key scan), shared by the two-launch routing kernels
// and the one-launch routing kernel.
#pragma once

#include "device_common.hpp"
#include "internal.hpp"

namespace moe {

struct ExpertKeys {
    const int32_t* idx;
    int E;
    __device__ __forceinline__ int operator()(int64_t f) const {
        const int32_t e = idx[f];
        if (e >= 0 && e < E) return e;
        return e == -1 ? kKeySkip : kKeyInvalid;
    }
};

// f = t*R + r.  The rank of a valid expert e is e / (E/R); the division only
// happens after the validity test so the -1 sentinel never lands on rank 0.
struct RankKeys {
    const int32_t* idx;
    int K, E, R, er;
    __device__ __forceinline__ int operator()(int64_t f) const {
        const int t = (int)(f / R);
        const int r = (int)(f - (int64_t)t * R);
        uint32_t mask = 0;
        for (int k = 0; k < K; ++k) {
            const int32_t e = idx[(int64_t)t * K + k];
            if (e >= 0 && e < E) mask |= 1u << (e / er);
        }
        return ((mask >> r) & 1u) ? r : kKeySkip;
    }
};

// f = t*K + k: a valid expert keeps its key only if the recv row of its
// (token, rank) exists; otherwise the entry is dropped before slotting.
struct SurvivorKeys {
    const int32_t* idx;
    const int32_t* rank_slot;
    int K, E, R, er;
    __device__ __forceinline__ int operator()(int64_t f) const {
        const int32_t e = idx[f];
        if (!(e >= 0 && e < E)) return e == -1 ? kKeySkip : kKeyInvalid;
        const int64_t t = f / K;
        return rank_slot[t * R + e / er] >= 0 ? e : kKeyDropped;
    }
};

// Stable ranks of one tile of WAVES*CHUNKS*64 entries.  Each wave owns a
// contiguous run of CHUNKS*64 entries and walks it in 64-entry chunks; equal
// keys are found with one ballot per key bit, a lane's rank is the number of
// equal-key lanes below it (mbcnt) plus the wave's running count in LDS, and
// after a barrier each entry adds the counts of the tile's earlier waves.
// run_all: LDS of WAVES*NK ints.  All threads of the workgroup must call it.
// flags_lds (optional, LDS): the workgroup scans its own tile (a one-tile
// launch), so nothing is published: thread 0 leaves the two flag totals there
// and the counts stay in run_all.  key_out (optional): each entry's key.
template <int WAVES, int CHUNKS, class KeyFn>
__device__ __forceinline__ void rank_tile(const KeyFn& keys, int64_t N, int NK, int nbits,
                                          int64_t tile, int32_t* run_all,
                                          int32_t* __restrict__ local_rank,
                                          int32_t* __restrict__ tile_cnt,
                                          int32_t* __restrict__ tile_flags,
                                          int32_t* flags_lds = nullptr,
                                          int32_t* key_out = nullptr) {
    static_assert(WAVES * CHUNKS * kWave == kTile, "tile size");
    __shared__ int32_t flag_cnt[WAVES][2];
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;

    for (int i = tid; i < WAVES * NK; i += WAVES * kWave) run_all[i] = 0;

    const int64_t f0 = tile * kTile + (int64_t)wave * (CHUNKS * kWave) + lane;
    int key[CHUNKS];
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) {
        const int64_t f = f0 + c * kWave;
        key[c] = f < N ? keys(f) : kKeySkip;
    }
    __syncthreads();

    int32_t* run = run_all + wave * NK;
    int rank[CHUNKS];
    int n_invalid = 0, n_dropped = 0;
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) {
        const uint64_t m = match_key(key[c], nbits);
        const int below = lanes_below(m);
        int r = -1;
        if (key[c] >= 0) r = run[key[c]] + below;
        // the lowest lane of each equal-key group advances the wave's count
        if (key[c] >= 0 && below == 0) run[key[c]] = r + __popcll(m);
        rank[c] = r;
        n_invalid += __popcll(ballot64(key[c] == kKeyInvalid));
        n_dropped += __popcll(ballot64(key[c] == kKeyDropped));
    }
    if (lane == 0) {
        flag_cnt[wave][0] = n_invalid;
        flag_cnt[wave][1] = n_dropped;
    }
    __syncthreads();

#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) {
        const int64_t f = f0 + c * kWave;
        if (f >= N) continue;
        int r = rank[c];
        if (key[c] >= 0)
            for (int w = 0; w < wave; ++w) r += run_all[w * NK + key[c]];
        local_rank[f] = r;
        if (key_out) key_out[f] = key[c];
    }
    // The tile's counts and flags are read by another workgroup (the scan),
    // possibly in the same launch on another XCD: agent-scope stores write
    // them through to the device coherence point, so the publisher only has to
    // wait for their completion instead of writing back its whole L2.
    if (!flags_lds) {
        for (int e = tid; e < NK; e += WAVES * kWave) {
            int s = 0;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) s += run_all[w * NK + e];
            __hip_atomic_store(&tile_cnt[tile * NK + e], s, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (tid == 0) {
        int a = 0, b = 0;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            a += flag_cnt[w][0];
            b += flag_cnt[w][1];
        }
        if (flags_lds) {
            flags_lds[0] = a;
            flags_lds[1] = b;
        } else {
            __hip_atomic_store(&tile_flags[2 * tile], a, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&tile_flags[2 * tile + 1], b, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

constexpr int kScanThreads = 1024;
constexpr int kScanCache = 16;  // tile counts a scan thread keeps in registers

// Exclusive scan of one int per thread over the block (initial value 0).
__device__ __forceinline__ int32_t block_exclusive_scan(int32_t v, int32_t* wave_sums) {
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    int32_t x = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int32_t y = __shfl_up(x, d, kWave);
        if (lane >= d) x += y;
    }
    if (lane == kWave - 1) wave_sums[wave] = x;
    __syncthreads();
    if (wave == 0) {
        int32_t ws = lane < kScanThreads / kWave ? wave_sums[lane] : 0;
#pragma unroll
        for (int d = 1; d < kScanThreads / kWave; d <<= 1) {
            const int32_t y = __shfl_up(ws, d, kWave);
            if (lane >= d) ws += y;
        }
        if (lane < kScanThreads / kWave) wave_sums[lane] = ws;  // inclusive wave totals
    }
    __syncthreads();
    const int32_t before = wave > 0 ? wave_sums[wave - 1] : 0;
    return before + x - v;
}

// A published tile count.  COHERENT: read at agent scope, for counts that
// other workgroups of the same launch stored at agent scope (the one-launch
// routing); otherwise a plain load (counts from an earlier kernel).
template <bool COHERENT>
__device__ __forceinline__ int32_t ld_count(const int32_t* p) {
    if (COHERENT) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return *p;
}

// One workgroup of kScanThreads threads.  Thread (key, part) owns the tiles
// [t0, t1) of one key: it loads their counts once (all loads issued together),
// sums them, takes the prefix of the earlier parts from LDS and writes the
// exclusive tile bases.  The per-key totals are then scanned over keys for the
// offsets.  one_tile (optional): a single-tile launch scanned by the workgroup
// that ranked it, whose counts are still in its LDS (one_tile->run: waves x NK
// running counts; one_tile->flags: the two flag totals), so nothing is read back
// from memory.
struct OneTileLds {
    const int32_t* run;
    int waves;
    const int32_t* flags;
};
template <bool COHERENT>
__device__ __forceinline__ void scan_tiles_body(const ScanArgs& a,
                                                const OneTileLds* one_tile = nullptr) {
    __shared__ int32_t part_sum[kScanThreads];
    __shared__ int32_t key_total[kScanThreads];
    __shared__ int32_t wave_sums[kScanThreads / kWave];
    __shared__ int32_t red[2];
    __shared__ unsigned long long red_drop;
    const int tid = threadIdx.x;
    const int NK = a.NK;
    const int tiles = a.tiles;
    int parts = kScanThreads / NK;
    if (parts > tiles) parts = tiles;
    if (parts < 1) parts = 1;
    const bool active = tid < parts * NK;
    const int key = tid % NK;
    const int part = tid / NK;
    const int tpp = (tiles + parts - 1) / parts;
    const int t0 = part * tpp;
    const int t1 = (t0 + tpp < tiles) ? t0 + tpp : tiles;

    int32_t c[kScanCache];
    int32_t s = 0;
    int32_t fi = 0, fd = 0;
    if (one_tile) {   // tiles == 1, parts == 1: thread key sums its key over the waves
#pragma unroll
        for (int i = 0; i < kScanCache; ++i) c[i] = 0;
        if (active)
            for (int w = 0; w < one_tile->waves; ++w) c[0] += one_tile->run[w * NK + key];
        if (tid == 0) {
            fi = one_tile->flags[0];
            fd = one_tile->flags[1];
        }
    } else {
#pragma unroll
        for (int i = 0; i < kScanCache; ++i) {
            const int tl = t0 + i;
            c[i] = (active && tl < t1) ? ld_count<COHERENT>(&a.tile_cnt[(int64_t)tl * NK + key]) : 0;
        }
        for (int tl = tid; tl < tiles; tl += kScanThreads) {
            fi += ld_count<COHERENT>(&a.tile_flags[2 * (int64_t)tl]);
            fd += ld_count<COHERENT>(&a.tile_flags[2 * (int64_t)tl + 1]);
        }
    }
#pragma unroll
    for (int i = 0; i < kScanCache; ++i) s += c[i];
    if (active)
        for (int tl = t0 + kScanCache; tl < t1; ++tl)
            s += ld_count<COHERENT>(&a.tile_cnt[(int64_t)tl * NK + key]);
    if (tid == 0) {
        red[0] = 0;
        red[1] = 0;
        red_drop = 0;
    }
    part_sum[tid] = s;
    key_total[tid] = 0;
    __syncthreads();

    if (fi) atomicAdd(&red[0], fi);
    if (fd) atomicAdd(&red[1], fd);
    if (active) {
        int32_t run = 0;
        for (int p = 0; p < part; ++p) run += part_sum[p * NK + key];
#pragma unroll
        for (int i = 0; i < kScanCache; ++i) {
            const int tl = t0 + i;
            if (tl < t1) a.tile_cnt[(int64_t)tl * NK + key] = run;
            run += c[i];
        }
        for (int tl = t0 + kScanCache; tl < t1; ++tl) {
            const int64_t j = (int64_t)tl * NK + key;
            const int32_t cc = ld_count<COHERENT>(&a.tile_cnt[j]);
            a.tile_cnt[j] = run;
            run += cc;
        }
        if (part == parts - 1) key_total[key] = run;
    }
    __syncthreads();

    const int32_t mine = key_total[tid];
    const int32_t excl = block_exclusive_scan(mine, wave_sums);
    const int32_t incl = excl + mine;

    if (tid < NK) {
        const int64_t cnt = mine;
        a.off_ws[tid] = excl;
        if (a.cnt_out) a.cnt_out[tid] = mine;
        if (a.off_out) a.off_out[tid] = excl;
        const int64_t base = a.cap > 0 ? (int64_t)tid * a.cap : (int64_t)excl;
        const int64_t seg = a.cap > 0 ? (cnt < a.cap ? cnt : a.cap) : cnt;
        const int64_t lo = base < a.rows_limit ? base : a.rows_limit;
        const int64_t end = base + seg;
        const int64_t hi = end < a.rows_limit ? end : a.rows_limit;
        const int64_t pc = hi > lo ? hi - lo : 0;
        if (a.packed_cnt) a.packed_cnt[tid] = (int32_t)pc;
        if (a.packed_off) a.packed_off[tid] = (int32_t)lo;
        if (tid == NK - 1) {
            a.off_ws[NK] = incl;
            if (a.off_out) a.off_out[NK] = incl;
            const int64_t bend = a.cap > 0 ? (int64_t)NK * a.cap : (int64_t)incl;
            if (a.packed_off) a.packed_off[NK] = (int32_t)(bend < a.rows_limit ? bend : a.rows_limit);
        }
        if (cnt - pc) atomicAdd(&red_drop, (unsigned long long)(cnt - pc));
    }
    __syncthreads();
    if (tid == 0 && a.stats) {
        const int32_t dropped_slots = (int32_t)red_drop;
        switch (a.mode) {
            case StatsMode::Plain:
                a.stats[0] = red[0];
                a.stats[1] = red[1] + dropped_slots;
                a.stats[2] = 0;
                break;
            case StatsMode::RecvRows:
                a.stats[2] = dropped_slots;
                break;
            case StatsMode::Experts:
                a.stats[0] = red[0];
                a.stats[1] = red[1] + dropped_slots;
                break;
        }
    }
}

inline int bits_for(int nk) {
    int b = 0;
    while ((1 << b) < nk) ++b;
    return b;
}

}  // namespace moe

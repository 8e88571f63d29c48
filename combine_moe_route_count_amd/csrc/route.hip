// route.hip - routing histogram, stable slot ranks and exclusive scans.
//
// The pages allocate dispatch slots with remote atomics ("Draft: cco + flydsl
// dispatch/combine", ROCm/mori pull 448, PR description), which makes the slot
// order depend on timing.  Here the slot of an entry is its rank among the
// earlier entries of the same key in flat order (a stable counting sort), found
// in two deterministic passes with no atomics on the result path:
//
//   rank pass  one workgroup per tile of kTile entries.  Each wave owns a
//              contiguous quarter of the tile and walks it in 64-entry chunks.
//              Lanes holding the same key are found with one ballot per key
//              bit; a lane's rank inside its chunk is the count of equal-key
//              lanes below it (mbcnt), plus the wave's running count for that
//              key kept in LDS.  After a barrier each entry adds the counts of
//              the tile's earlier waves.  Output: the rank inside the tile and
//              the per-tile key counts.
//   scan pass  one workgroup: exclusive scan over tiles per key (the tile
//              bases), then over keys (the offsets, initial value 0 as in "Add
//              standalone cuda.coop.cutlass package", NVIDIA/cccl pull 12311),
//              then the per-key segment sizes under the capacity and the
//              statistics.
//
// The wave-level ballot / prefix idea follows the wave64 prefix count that
// "feat(EPv2): [preview] internode dispatch/combine over CCO/GDA" (ROCm/mori
// pull 625, commit log) uses for slot assignment, computed here with mbcnt so
// lane 0 needs no 64-bit shift.
#include "device_common.hpp"
#include "internal.hpp"

#include "route_device.hpp"

namespace moe {

namespace {

template <class KeyFn>
__global__ __launch_bounds__(kRankThreads) void rank_tiles_kernel(
    KeyFn keys, int64_t N, int NK, int nbits, int32_t* __restrict__ local_rank,
    int32_t* __restrict__ tile_cnt, int32_t* __restrict__ tile_flags) {
    extern __shared__ int32_t run_all[];  // [kTileWaves][NK] running counts per wave
    rank_tile<kTileWaves, kTileChunks>(keys, N, NK, nbits, (int64_t)blockIdx.x, run_all,
                                       local_rank, tile_cnt, tile_flags);
}

__global__ __launch_bounds__(kScanThreads) void scan_tiles_kernel(ScanArgs a) {
    scan_tiles_body<false>(a);
}

}  // namespace

hipError_t launch_rank(const RankArgs& a, hipStream_t s) {
    const int64_t tiles = (a.N + kTile - 1) / kTile;
    if (tiles == 0) return hipSuccess;
    const size_t lds = sizeof(int32_t) * (size_t)kTileWaves * a.NK;
    const int nbits = bits_for(a.NK);
    switch (a.kind) {
        case KeyKind::Experts:
            rank_tiles_kernel<<<dim3((unsigned)tiles), dim3(kRankThreads), lds, s>>>(
                ExpertKeys{a.idx, a.E}, a.N, a.NK, nbits, a.local_rank, a.tile_cnt, a.tile_flags);
            break;
        case KeyKind::Ranks:
            rank_tiles_kernel<<<dim3((unsigned)tiles), dim3(kRankThreads), lds, s>>>(
                RankKeys{a.idx, a.K, a.E, a.R, a.E / a.R}, a.N, a.NK, nbits, a.local_rank,
                a.tile_cnt, a.tile_flags);
            break;
        case KeyKind::Survivors:
            rank_tiles_kernel<<<dim3((unsigned)tiles), dim3(kRankThreads), lds, s>>>(
                SurvivorKeys{a.idx, a.rank_slot, a.K, a.E, a.R, a.E / a.R}, a.N, a.NK, nbits,
                a.local_rank, a.tile_cnt, a.tile_flags);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t s) {
    scan_tiles_kernel<<<dim3(1), dim3(kScanThreads), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace moe

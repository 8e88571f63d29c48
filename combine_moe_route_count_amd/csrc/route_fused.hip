// route_fused.hip - one routing level in one launch: stable per-tile ranks,
// then the tile / key scan run by whichever routing workgroup finishes last.
//
// Workgroups of 1024 threads each rank one tile of 1024 entries (16 waves x one
// 64-entry chunk, the pass of route.hip), publish their counts with agent-scope
// stores, and take a ticket.  The workgroup that takes the last ticket runs the
// scan of route.hip on everyone's counts and re-arms the ticket.  Nobody waits for
// anybody: a workgroup either finishes after its tile or, being last, after the
// scan, so the launch needs no co-residency and cannot hang (the CTA-local rule
// of "Drop cooperative launch from the CTA-independent local kernels", MoonEP
// pull 34, "Why it's worth doing").  Compared with two launches this saves one
// kernel boundary on every routing level.
#include "device_common.hpp"
#include "internal.hpp"
#include "route_device.hpp"

namespace moe {

namespace {

constexpr int kFusedThreads = 1024;
constexpr uint32_t kTicketTag = 0x5A17C0DEu;   // no byte-repeat pattern a memset could leave
constexpr int kFusedWaves = kFusedThreads / kWave;

// Arrival on the tagged ticket; returns this launch's count after the arrival.
// The word holds (kTicketTag << 32) | arrivals; the last arrival of every
// launch re-arms it to (kTicketTag << 32) | 0, so each launch after a completed
// one arrives with a single fetch-add.  A word that does not carry the tag
// (a workspace never used, or reused for something else) is repaired once:
// arrivals that find it stale replace it by (tag, 1) with a compare-and-swap,
// or, once another arrival has done so, fetch-add like everyone else; the
// adds that hit the stale word are discarded with it.
__device__ uint32_t arrive_ticket(uint64_t* ticket) {
    const uint64_t old =
        __hip_atomic_fetch_add(ticket, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)(old >> 32) == kTicketTag) return (uint32_t)old + 1u;
    uint64_t cur = __hip_atomic_load(ticket, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t fresh = ((uint64_t)kTicketTag << 32) | 1ull;
    for (;;) {
        if ((uint32_t)(cur >> 32) == kTicketTag) {
            const uint64_t o =
                __hip_atomic_fetch_add(ticket, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return (uint32_t)o + 1u;
        }
        if (__hip_atomic_compare_exchange_strong(ticket, &cur, fresh, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            return 1u;
    }
}

template <class KeyFn>
__global__ __launch_bounds__(kFusedThreads) void route_fused_kernel(KeyFn keys, RouteFusedArgs a) {
    extern __shared__ int32_t run_all[];  // [kFusedWaves][NK] routing counts
    __shared__ uint32_t s_last;
    __shared__ int32_t tile_flags_lds[2];
    const int tid = threadIdx.x;
    // A launch of one tile (up to 1024 entries: the decode-sized calls) is its
    // own last workgroup: it keeps its counts in LDS and scans them there, so
    // nothing is published, no ticket is taken and nothing is read back.
    const bool single = a.scan.tiles == 1;
    rank_tile<kFusedWaves, 1>(keys, a.N, a.scan.NK, a.nbits, (int64_t)blockIdx.x, run_all,
                              a.local_rank, a.scan.tile_cnt, (int32_t*)a.scan.tile_flags,
                              single ? tile_flags_lds : nullptr);
    if (single) {
        __syncthreads();
        const OneTileLds lds{run_all, kFusedWaves, tile_flags_lds};
        scan_tiles_body<true>(a.scan, &lds);
        return;
    }
    // Publication of the tile, and why it needs no release / acquire pair.
    // The LLVM AMDGPU memory model's code sequences for GFX942, which gfx950
    // follows, implement agent scope as: monotonic store = global_store sc1,
    // monotonic load = global_load sc1 (both reach the device coherence point
    // past the XCD's own L2, which is not coherent with the other XCDs' L2s),
    // release fence = buffer_wbl2 sc1 + s_waitcnt vmcnt(0), acquire fence =
    // buffer_inv sc1.  Every value that crosses workgroups here is one of
    // those monotonic accesses (the counts and flags stored in rank_tile, the
    // loads in scan_tiles_body<true>, the ticket's atomics, which the compiler
    // emits with no cache bypass because the device performs them at the
    // coherence point).  The write-back half of a release exists for plain
    // stores left dirty in L2, and none of the published data is such a store,
    // so the part that matters is the wait: vmcnt(0) returns only once every
    // sc1 store of this wave has been acknowledged by the coherence point, and
    // the barrier after it holds the ticket until all 16 waves have waited.
    // On the reading side, the invalidate half of an acquire exists for plain
    // loads that could hit stale L2 lines; the scan reads with sc1 loads
    // issued after its own ticket returned the last count (a control
    // dependence through LDS and a barrier), and each earlier arrival followed
    // its own acknowledged stores, so those loads see every count.  Formally
    // monotonic accesses alone do not order data in the model; the ordering
    // here is the hardware's completion order, which is what the model's
    // release sequence itself relies on.  The regression guards are the GPU
    // tests that run this kernel back to back on two streams, replayed from a
    // graph and 10^4 times with changing sizes.  The fence measured about
    // 10 us per launch: its write-back flushes every dirty line the previous
    // kernel's streaming stores left in this XCD's L2.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) s_last = arrive_ticket(a.ticket) == (uint32_t)a.scan.tiles;
    __syncthreads();
    if (!s_last) return;
    // Every tile's counts are at the coherence point (agent-scope stores that
    // completed before their ticket arrivals, which precede this one); the scan
    // reads them with agent-scope loads, so no cache invalidate is needed.
    scan_tiles_body<true>(a.scan);
    if (tid == 0)
        __hip_atomic_store(a.ticket, (uint64_t)kTicketTag << 32, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

hipError_t launch_route_fused(const RouteFusedArgs& a, hipStream_t s) {
    if (a.scan.tiles <= 0 || a.scan.NK > kFusedMaxKeys) return hipErrorInvalidValue;
    const dim3 grid((unsigned)a.scan.tiles), block(kFusedThreads);
    const size_t lds = sizeof(int32_t) * (size_t)kFusedWaves * a.scan.NK;
    switch (a.kind) {
        case KeyKind::Experts:
            route_fused_kernel<<<grid, block, lds, s>>>(ExpertKeys{a.idx, a.E}, a);
            break;
        case KeyKind::Ranks:
            route_fused_kernel<<<grid, block, lds, s>>>(RankKeys{a.idx, a.K, a.E, a.R, a.E / a.R},
                                                        a);
            break;
        case KeyKind::Survivors:
            route_fused_kernel<<<grid, block, lds, s>>>(
                SurvivorKeys{a.idx, a.rank_slot, a.K, a.E, a.R, a.E / a.R}, a);
            break;
    }
    return hipGetLastError();
}

}  // namespace moe

// device_common.hpp - gfx950 device helpers shared by the MoE route kernels:
// wave64 ballot matching, DPP reductions, bf16 / OCP e4m3 conversions and
// 16-byte vector memory access.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

// Entries per routing tile: 4 waves x 4 chunks x 64 lanes.
constexpr int kTileWaves = 4;
constexpr int kTileChunks = 4;
constexpr int kTile = kTileWaves * kTileChunks * kWave;
constexpr int kRankThreads = kTileWaves * kWave;

// Token-parallel kernels launch at most this many workgroups and loop over the
// rest, which keeps every launch far below the 2^32 work-item limit.
constexpr int64_t kMaxGrid = (int64_t)1 << 22;

constexpr int kFp8Block = 128;
constexpr float kE4m3Max = 448.0f;
constexpr float kE2m1Max = 6.0f;

// Key codes produced by the routing key functions.
constexpr int kKeySkip = -1;     // "no expert": skipped, not counted
constexpr int kKeyInvalid = -2;  // id outside [0, E) other than -1: counted invalid
constexpr int kKeyDropped = -3;  // valid entry dropped before slotting: counted dropped

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// wave64 primitives
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

// Number of set bits of m in the lanes below the calling lane.
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Mask of the lanes whose key equals the calling lane's key (keys >= 0 only;
// lanes with a negative key get an empty mask).  One ballot per key bit, so the
// cost does not depend on how many distinct keys the wave holds.
__device__ __forceinline__ uint64_t match_key(int key, int nbits) {
    uint64_t m = ballot64(key >= 0);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t bm = ballot64(bit);
        m &= bit ? bm : ~bm;
    }
    return key >= 0 ? m : 0ull;
}

template <typename T>
__device__ __forceinline__ T readlane(T v, int lane) {
    static_assert(sizeof(T) == 4, "32-bit readlane");
    int r = __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane);
    return __builtin_bit_cast(T, r);
}

// Max over each aligned group of 8 lanes (DPP quad permutes, then the half-row mirror).
__device__ __forceinline__ float group8_max(float v) {
    int iv = __builtin_bit_cast(int, v);
    float o = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(iv, 0xB1, 0xF, 0xF, true));
    v = fmaxf(v, o);
    iv = __builtin_bit_cast(int, v);
    o = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(iv, 0x4E, 0xF, 0xF, true));
    v = fmaxf(v, o);
    iv = __builtin_bit_cast(int, v);
    o = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(iv, 0x141, 0xF, 0xF, true));
    return fmaxf(v, o);
}

// ---------------------------------------------------------------------------
// number formats
// ---------------------------------------------------------------------------

// Low / high bf16 of a packed pair, widened exactly to f32.
__device__ __forceinline__ float bf16lo(uint32_t d) { return __builtin_bit_cast(float, d << 16); }
__device__ __forceinline__ float bf16hi(uint32_t d) {
    return __builtin_bit_cast(float, d & 0xffff0000u);
}

// Two f32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const uint32_t a = __builtin_bit_cast(uint16_t, (__bf16)lo);
    const uint32_t b = __builtin_bit_cast(uint16_t, (__bf16)hi);
    return a | (b << 16);
}

// Four f32 (each |v| <= 448) -> four OCP e4m3fn bytes, round to nearest even.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
    return (uint32_t)r;
}

// Two e4m3fn bytes (byte pair `hi` of d) -> f32, exact.
template <bool HI>
__device__ __forceinline__ void unpack_e4m3x2(uint32_t d, float& a, float& b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    f2 v = __builtin_amdgcn_cvt_pk_f32_fp8((int)d, HI);
    a = v.x;
    b = v.y;
}

// Eight e2m1 (fp4) codes of d -> f32, exact; element 2i is the low nibble of
// byte i.  The gfx950 scaled converters apply only the exponent of their scale
// operand, so they are given 1.0 and any block scale is applied in f32 apart.
__device__ __forceinline__ void unpack_e2m1x8(uint32_t d, float (&v)[8]) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    const f2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 0);
    const f2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 1);
    const f2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 2);
    const f2 e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 3);
    v[0] = a.x; v[1] = a.y; v[2] = b.x; v[3] = b.y;
    v[4] = c.x; v[5] = c.y; v[6] = e.x; v[7] = e.y;
}

// Eight f32 (|v| <= 6 after the caller's clamp) -> e2m1 codes, round to nearest
// even, sign kept for zero results; byte i holds elements 2i (low) and 2i+1.
__device__ __forceinline__ uint32_t pack_e2m1x8(const float (&v)[8]) {
    uint32_t d = 0;
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, v[0], v[1], 1.0f, 0);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, v[2], v[3], 1.0f, 1);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, v[4], v[5], 1.0f, 2);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, v[6], v[7], 1.0f, 3);
    return d;
}

// ---------------------------------------------------------------------------
// 16-byte memory access
// ---------------------------------------------------------------------------

__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
    return __builtin_nontemporal_load((const u32x4*)p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *(u32x4*)p = v; }
__device__ __forceinline__ void st16_stream(void* p, u32x4 v) {
    __builtin_nontemporal_store(v, (u32x4*)p);
}
__device__ __forceinline__ u32x2 ld8_stream(const void* p) {
    return __builtin_nontemporal_load((const u32x2*)p);
}

// A destination row addressed through a buffer resource.  The row base is
// wave-uniform (a broadcast row index), so it stays in scalar registers and
// each lane adds only its byte offset; an offset outside the row is dropped by
// the hardware range check.  POL is the stores' cache policy, chosen per row
// kind by measurement on 1 GiB-class scatters:
//   kStoreThrough (sc1 nt, agent-scope streaming: written through L2) for the
//     fp8 / fp4 rows (7 KB and less at H=7168), where it beat the plain
//     non-temporal store by about 3% and plain stores lost 10%, and for the
//     dedup expansion, whose source rows are read back from HBM as it goes;
//   kStorePlain (write-back through L2) for the copies of token rows in bf16
//     or f32 (14-16 KB), 3% (bf16 dispatch) to 4% (f32 dedup recv copy) faster;
// the pure-write ceilings are 5.45 TB/s plain, 5.0 sc1 nt, 4.9 nt.
constexpr int kStoreThrough = (1 << 4) | (1 << 1);  // cache policy bits: sc1, nt
constexpr int kStorePlain = 0;
constexpr int kRsrcWord3 = 0x00020000;               // gfx9 descriptor word 3: 32-bit raw data
template <int POL>
struct RowOut {
    __amdgpu_buffer_rsrc_t r;
    __device__ __forceinline__ RowOut(void* row, int64_t bytes)
        : r(__builtin_amdgcn_make_buffer_rsrc(row, 0, (int)bytes, kRsrcWord3)) {}
    __device__ __forceinline__ void st16(int off, u32x4 v) const {
        __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, POL);
    }
    __device__ __forceinline__ void st8(int off, u32x2 v) const {
        __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, POL);
    }
};

}  // namespace moe

// rows_device.hpp - device helpers of the row-moving kernels: the packed row
// of an entry, wave broadcasts of a token's destination rows, the 16-byte
// multi-destination row copy and the blockwise fp8 pack of 16 bf16 values.
#pragma once

#include "device_common.hpp"
#include "internal.hpp"

namespace moe {

// Packed row of entry f, or -1 when the entry has no key or was dropped by the
// capacity / row limit.
__device__ __forceinline__ int entry_row(const SlotArgs& a, int64_t f) {
    // Both loads in flight together (e is only used once lr says it is valid);
    // the empty asm keeps the compiler from sinking the idx load under the
    // branch, which would cost a second memory round trip.
    const int32_t lr = a.local_rank[f];
    int32_t e = a.idx[f];
    asm volatile("" : "+v"(e));
    if (lr < 0) return -1;
    const int64_t slot = (int64_t)a.tile_base[(f / kTile) * a.E + e] + lr;
    const int64_t base = a.cap > 0 ? (int64_t)e * a.cap : (int64_t)a.off[e];
    if ((a.cap > 0 && slot >= a.cap) || base + slot >= a.packed_rows || base + slot < 0) return -1;
    return (int)(base + slot);
}

template <int DMAX>
__device__ __forceinline__ void broadcast_rows(int my_row, int (&rows)[DMAX]) {
#pragma unroll
    for (int d = 0; d < DMAX; ++d) rows[d] = readlane(my_row, d);
}

// Marks loaded registers as settled: the compiler waits for their loads once,
// before the empty asm, and sees plain values afterwards.
template <int N>
__device__ __forceinline__ void settle(u32x4 (&v)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(v[i]));
}

// Copy one row of nvec 16-byte vectors (already holding pass 0 in val) to up
// to D destination rows with store policy POL; passes after the first reload
// from src.
template <int DMAX, int VPT, int POL>
__device__ __forceinline__ void store_row_copies(const char* src, int nvec, char* dst,
                                                 int64_t row_bytes, const int (&rows)[DMAX], int D,
                                                 u32x4 (&val)[VPT], int tid, int nthreads) {
    const int step = VPT * nthreads;
    for (int base = 0;;) {
        // Every store below is conditional and reads loaded registers; without
        // this one explicit use the compiler loses count of the loads at each
        // join and waits for vmcnt(0) before every store, i.e. for the previous
        // stores too.  The empty asm takes the wait once, here.
        settle(val);
#pragma unroll
        for (int d = 0; d < DMAX; ++d) {
            if (d >= D) break;
            if (rows[d] < 0) continue;
            const RowOut<POL> out(dst + (int64_t)rows[d] * row_bytes, row_bytes);
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int v = base + tid + i * nthreads;
                if (v < nvec) out.st16(v * 16, val[i]);
            }
        }
        base += step;
        if (base >= nvec) break;
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int v = base + tid + i * nthreads;
            if (v < nvec) val[i] = ld16_stream(src + (int64_t)v * 16);
        }
    }
}

template <int VPT>
__device__ __forceinline__ void load_first_pass(const char* src, int nvec, u32x4 (&val)[VPT],
                                                int tid, int nthreads) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int v = tid + i * nthreads;
        if (v < nvec) val[i] = ld16_stream(src + (int64_t)v * 16);
    }
}

// Pack 16 bf16 values (two 16-byte vectors) of one lane; the 8 lanes of a
// 128-element block agree on amax and the scale.
__device__ __forceinline__ void fp8_pack16(const u32x4& lo, const u32x4& hi, u32x4& q,
                                           float& scale) {
    float v[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[2 * j] = bf16lo(lo[j]);
        v[2 * j + 1] = bf16hi(lo[j]);
        v[8 + 2 * j] = bf16lo(hi[j]);
        v[8 + 2 * j + 1] = bf16hi(hi[j]);
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(v[j]));
    amax = group8_max(amax);
    scale = 1.0f;
    if (amax > kE4m3Max) {
        // q = e4m3(clamp((x * 448) / amax)); x * 448 is exact for bf16 x and the
        // quotient is a correctly rounded f32 division.
        scale = amax / kE4m3Max;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float n = v[j] * kE4m3Max;
            const float qv = n / amax;
            v[j] = fminf(fmaxf(qv, -kE4m3Max), kE4m3Max);
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
        q[j] = pack_e4m3x4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
}

// The same 16 bf16 values packed to e2m1 (fp4): the fp8 block rule with the
// e2m1 maximum 6 in place of 448; two words of eight codes.
__device__ __forceinline__ void fp4_pack16(const u32x4& lo, const u32x4& hi, u32x2& q,
                                           float& scale) {
    float v[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[2 * j] = bf16lo(lo[j]);
        v[2 * j + 1] = bf16hi(lo[j]);
        v[8 + 2 * j] = bf16lo(hi[j]);
        v[8 + 2 * j + 1] = bf16hi(hi[j]);
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(v[j]));
    amax = group8_max(amax);
    scale = 1.0f;
    if (amax > kE2m1Max) {
        // q = e2m1(clamp((x * 6) / amax)); x * 6 is exact for bf16 x
        scale = amax / kE2m1Max;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float n = v[j] * kE2m1Max;
            const float qv = n / amax;
            v[j] = fminf(fmaxf(qv, -kE2m1Max), kE2m1Max);
        }
    }
    float a[8], b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = v[j];
        b[j] = v[8 + j];
    }
    q[0] = pack_e2m1x8(a);
    q[1] = pack_e2m1x8(b);
}

}  // namespace moe

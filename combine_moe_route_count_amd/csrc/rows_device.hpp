// rows_device.hpp - device helpers of the row-moving kernels: the packed row
// of an entry, wave broadcasts of a token's destination rows, the 16-byte
// multi-destination row copy and the blockwise fp8 / fp4 pack of 16 bf16
// values.
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

// The 16-byte vectors [v0, v1) of a row: the part of it one workgroup moves.
struct VecRange {
    int v0, v1;
};

// Copy the vectors r of one row (already holding pass 0 in val) to up to D
// destination rows with store policy POL; passes after the first reload from
// src.
template <int DMAX, int VPT, int POL>
__device__ __forceinline__ void store_row_copies(const char* src, VecRange r, char* dst,
                                                 int64_t row_bytes, const int (&rows)[DMAX], int D,
                                                 u32x4 (&val)[VPT], int tid, int nthreads) {
    const int step = VPT * nthreads;
    for (int base = r.v0;;) {
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
                if (v < r.v1) out.st16(v * 16, val[i]);
            }
        }
        base += step;
        if (base >= r.v1) break;
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int v = base + tid + i * nthreads;
            if (v < r.v1) val[i] = ld16_stream(src + (int64_t)v * 16);
        }
    }
}

template <int VPT>
__device__ __forceinline__ void load_first_pass(const char* src, VecRange r, u32x4 (&val)[VPT],
                                                int tid, int nthreads) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int v = r.v0 + tid + i * nthreads;
        if (v < r.v1) val[i] = ld16_stream(src + (int64_t)v * 16);
    }
}

// The 16 bf16 values of one lane (two 16-byte vectors), widened exactly to
// f32: element 2j / 2j+1 are the low / high halves of word j.
__device__ __forceinline__ void unpack_bf16x16(const u32x4& lo, const u32x4& hi, float (&v)[16]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[2 * j] = bf16lo(lo[j]);
        v[2 * j + 1] = bf16hi(lo[j]);
        v[8 + 2 * j] = bf16lo(hi[j]);
        v[8 + 2 * j + 1] = bf16hi(hi[j]);
    }
}

// Bit pattern of element j of the lane's 16 bf16 values.
__device__ __forceinline__ uint32_t bf16_bits_at(const u32x4& lo, const u32x4& hi, int j) {
    const uint32_t w = j < 8 ? lo[(j & 7) >> 1] : hi[(j & 7) >> 1];
    return (j & 1) ? w >> 16 : w & 0xffffu;
}

// Largest magnitude among the lane's 16 bf16 values, as bf16 bits with the
// sign cleared (two packed 16-bit maxima per word).  Non-negative floats order
// as their bit patterns, so when every value is finite this is max|x|; a
// result of 0x7F80 or more (exponent all ones) says the lane holds an infinity
// or a NaN.
__device__ __forceinline__ uint32_t bf16x16_max_mag(const u32x4& lo, const u32x4& hi) {
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    u16x2 m = __builtin_bit_cast(u16x2, lo[0] & 0x7fff7fffu);
#pragma unroll
    for (int j = 1; j < 8; ++j) {
        const uint32_t w = j < 4 ? lo[j] : hi[j - 4];
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w & 0x7fff7fffu));
    }
    return m.x > m.y ? m.x : m.y;
}

// max|x| over the finite values only (0 when none is); *has_nan says whether
// one of them is a NaN.  Taken only by a lane that holds a non-finite value.
__device__ __forceinline__ float finite_amax16(const float (&v)[16], bool& has_nan) {
    float amax = 0.0f;
    has_nan = false;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const float a = fabsf(v[j]);
        has_nan |= a != a;
        if (a < __builtin_inff()) amax = fmaxf(amax, a);
    }
    return amax;
}

// In a block with amax > m: v = x*m/amax, the correctly rounded f32 quotient
// of the exact product.  A block near the f32 maximum is first scaled by 2^-64
// (x and amax alike, both exact), so x*m cannot overflow; an element that the
// scaling would make subnormal quotients below 2^-117, whose code is a signed
// zero either way.  Infinities stay infinite and NaNs NaN.
__device__ __forceinline__ void scale_block16(float (&v)[16], float m, float amax) {
    const float pre = amax >= 0x1p64f ? 0x1p-64f : 1.0f;
    const float am = amax * pre;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const float n = (v[j] * pre) * m;
        v[j] = n / am;
    }
}

// Infinities to +-m (saturating conversion, sign kept).
__device__ __forceinline__ void saturate_inf16(float (&v)[16], float m) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
        if (__builtin_isinf(v[j])) v[j] = __builtin_copysignf(m, v[j]);
}

// Pack 16 bf16 values (two 16-byte vectors) of one lane; the 8 lanes of a
// 128-element block agree on amax and the scale.  amax is taken over finite
// values; infinities saturate to +-448 and a NaN gets the NaN code S.1111.111
// with its own sign.  A lane without infinities or NaNs (one integer test)
// takes none of those steps.
__device__ __forceinline__ void fp8_pack16(const u32x4& lo, const u32x4& hi, u32x4& q,
                                           float& scale) {
    const uint32_t mag = bf16x16_max_mag(lo, hi);
    const bool odd = mag >= 0x7f80u;
    // NaN codes, one byte per element (0: not a NaN), taken from the bits
    // before any arithmetic can drop a NaN's sign
    u32x4 nan_code = u32x4{0, 0, 0, 0};
    if (odd) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t b = bf16_bits_at(lo, hi, j);
            if ((b & 0x7fffu) > 0x7f80u)
                nan_code[j >> 2] |= (0x7fu | ((b >> 8) & 0x80u)) << ((j & 3) * 8);
        }
    }
    float v[16];
    unpack_bf16x16(lo, hi, v);
    float amax = __builtin_bit_cast(float, mag << 16);
    if (odd) {
        bool nan;
        amax = finite_amax16(v, nan);
    }
    amax = group8_max(amax);
    scale = 1.0f;
    if (amax > kE4m3Max) {
        // q = e4m3(x * 448 / amax); |quotient| <= 448 for every finite x
        scale = amax / kE4m3Max;
        scale_block16(v, kE4m3Max, amax);
    }
    if (odd) saturate_inf16(v, kE4m3Max);
#pragma unroll
    for (int j = 0; j < 4; ++j)
        q[j] = pack_e4m3x4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
    if (odd) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // bytes of NaN elements: every bit of a NaN code's low seven is set
            const uint32_t m = (nan_code[j] & 0x7f7f7f7fu) | ((nan_code[j] & 0x7f7f7f7fu) << 1);
            q[j] = (q[j] & ~m) | nan_code[j];
        }
    }
}

// The same 16 bf16 values packed to e2m1 (fp4): the fp8 block rule with the
// e2m1 maximum 6 in place of 448; two words of eight codes.  e2m1 has no NaN:
// a block holding one is stored as zero codes with a NaN scale.
__device__ __forceinline__ void fp4_pack16(const u32x4& lo, const u32x4& hi, u32x2& q,
                                           float& scale) {
    float v[16];
    unpack_bf16x16(lo, hi, v);
    const uint32_t mag = bf16x16_max_mag(lo, hi);
    const bool odd = mag >= 0x7f80u;
    float amax = __builtin_bit_cast(float, mag << 16);
    if (odd) {
        bool nan;
        amax = finite_amax16(v, nan);
        if (nan) amax = __builtin_inff();   // finite amax is never infinite: marks the block
    }
    amax = group8_max(amax);
    if (amax == __builtin_inff()) {
        scale = __builtin_bit_cast(float, 0x7fc00000u);
        q = u32x2{0, 0};
        return;
    }
    scale = 1.0f;
    if (amax > kE2m1Max) {
        // q = e2m1(x * 6 / amax)
        scale = amax / kE2m1Max;
        scale_block16(v, kE2m1Max, amax);
    }
    if (odd) saturate_inf16(v, kE2m1Max);
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

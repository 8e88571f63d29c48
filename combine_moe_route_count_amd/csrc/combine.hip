// combine.hip - weighted gather-reduce of each token's expert outputs back to
// token order, plus out_weights.
//
// One workgroup per token.  Lanes below K read the token's tok_map entries and
// weights once and broadcast them to the wave with readlane, so every branch
// on an entry is wave-uniform.  Each lane owns units of 8 elements: it first
// issues the 16-byte loads of all K rows for its units (the load-first gather
// of "feat(EPv2): [preview] internode dispatch/combine over CCO/GDA", ROCm/mori
// pull 625, commit log: 16 B vector gather), then reduces in f32 in ascending
// k with a separately rounded multiply and add (the build disables
// contraction), and stores 16 bytes of bf16 (or 32 bytes of f32).  The weight
// sum is folded in once per token ("Draft: cco + flydsl dispatch/combine",
// ROCm/mori pull 448, commit log: out_weights folded into the gather loop).
//
// The dedup forms keep one partial sum per virtual rank (the local reduce of
// "Drop cooperative launch from the CTA-independent local kernels", MoonEP pull
// 34, "Why it's worth doing") and add the partials in ascending rank order
// (mori pull 448, convert_combine_input followed by the sum across ranks).
#include "device_common.hpp"
#include "internal.hpp"

namespace moe {

namespace {

constexpr int kCombThreads = 512;

// 8 consecutive elements of row `row` starting at element col, as f32.
template <bool YF32>
struct Unit;

template <>
struct Unit<false> {  // bf16: one 16-byte load
    u32x4 a;
    __device__ __forceinline__ void load(const void* y, int64_t row, int64_t H, int64_t col) {
        a = ld16_stream((const uint16_t*)y + row * H + col);
    }
    __device__ __forceinline__ float get(int j) const {
        return (j & 1) ? bf16hi(a[j >> 1]) : bf16lo(a[j >> 1]);
    }
};

template <>
struct Unit<true> {  // f32: two 16-byte loads
    u32x4 a, b;
    __device__ __forceinline__ void load(const void* y, int64_t row, int64_t H, int64_t col) {
        const float* p = (const float*)y + row * H + col;
        a = ld16_stream(p);
        b = ld16_stream(p + 4);
    }
    __device__ __forceinline__ float get(int j) const {
        return __builtin_bit_cast(float, j < 4 ? a[j] : b[j - 4]);
    }
};

template <bool OF32>
__device__ __forceinline__ void store_unit(void* out, int64_t row, int64_t H, int64_t col,
                                           const float (&acc)[8]) {
    if (OF32) {
        float* p = (float*)out + row * H + col;
        u32x4 a, b;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            a[j] = __builtin_bit_cast(uint32_t, acc[j]);
            b[j] = __builtin_bit_cast(uint32_t, acc[4 + j]);
        }
        st16_stream(p, a);
        st16_stream(p + 4, b);
    } else {
        u32x4 a;
#pragma unroll
        for (int j = 0; j < 4; ++j) a[j] = pack_bf16x2(acc[2 * j], acc[2 * j + 1]);
        st16_stream((uint16_t*)out + row * H + col, a);
    }
}

// Entry rows (-1 if absent or outside [0, y_rows)) and weights of token t.
template <int KMAX>
__device__ __forceinline__ void token_entries(const CombineArgs& a, int64_t t, int (&rows)[KMAX],
                                              float (&w)[KMAX]) {
    const int lane = threadIdx.x % kWave;
    int my_row = -1;
    float my_w = 0.0f;
    if (lane < a.K) {
        // both loads in flight together: one memory round trip before the gather
        const int64_t r = a.tok_map[t * a.K + lane];
        const float wk = a.w[t * a.K + lane];
        if (r >= 0 && r < a.y_rows) {
            my_row = (int)r;
            my_w = wk;
        }
    }
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        rows[k] = readlane(my_row, k);
        w[k] = readlane(my_w, k);
    }
}

// ---------------------------------------------------------------------------
// plain combine: acc = 0; acc = acc + w_k * y_k for k ascending
// ---------------------------------------------------------------------------
template <bool YF32, bool OF32, int KMAX, int VPT>
__global__ __launch_bounds__(kCombThreads) void combine_kernel(CombineArgs a) {
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t H = a.H;
    const int units = (int)(H / 8);
    int rows[KMAX];
    float w[KMAX];
    token_entries<KMAX>(a, t, rows, w);

    for (int base = 0; base < units; base += VPT * (int)blockDim.x) {
        Unit<YF32> y[KMAX][VPT];
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (rows[k] < 0) continue;
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int u = base + tid + i * (int)blockDim.x;
                if (u < units) y[k][i].load(a.y, rows[k], H, (int64_t)u * 8);
            }
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int u = base + tid + i * (int)blockDim.x;
            if (u >= units) continue;
            float acc[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                if (rows[k] < 0) continue;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float p = w[k] * y[k][i].get(j);
                    acc[j] = acc[j] + p;
                }
            }
            store_unit<OF32>(a.out, t, H, (int64_t)u * 8, acc);
        }
    }
    if (tid == 0 && a.out_weights) {
        float s = 0.0f;
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (rows[k] >= 0) s = s + w[k];
        a.out_weights[t] = s;
    }
}

// ---------------------------------------------------------------------------
// dedup combine
//   MODE 0: per-rank partials kept in registers, out written (one kernel)
//   MODE 1: per-rank partials written to `partial` (stage A)
// ---------------------------------------------------------------------------
template <int KMAX>
__device__ __forceinline__ void entry_ranks(const CombineArgs& a, int64_t t, int (&ranks)[KMAX]) {
    const int lane = threadIdx.x % kWave;
    const int er = a.E / a.R;
    int my_rank = -1;
    if (lane < a.K) {
        const int32_t e = a.idx[t * a.K + lane];
        if (e >= 0 && e < a.E) my_rank = e / er;
    }
#pragma unroll
    for (int k = 0; k < KMAX; ++k) ranks[k] = readlane(my_rank, k);
}

template <bool YF32, bool OF32, int KMAX, int MODE>
__global__ __launch_bounds__(kCombThreads) void dedup_combine_kernel(CombineArgs a) {
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t H = a.H;
    const int units = (int)(H / 8);
    const int R = a.R;
    int rows[KMAX], ranks[KMAX];
    float w[KMAX];
    token_entries<KMAX>(a, t, rows, w);
    entry_ranks<KMAX>(a, t, ranks);

    for (int u = tid; u < units; u += (int)blockDim.x) {
        float acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
        for (int r = 0; r < R; ++r) {
            const int32_t rs = a.rank_slot[t * R + r];
            if (rs < 0 || rs >= a.recv_rows) continue;
            Unit<YF32> y[KMAX];
#pragma unroll
            for (int k = 0; k < KMAX; ++k)
                if (rows[k] >= 0 && ranks[k] == r) y[k].load(a.y, rows[k], H, (int64_t)u * 8);
            float p[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) p[j] = 0.0f;
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                if (rows[k] < 0 || ranks[k] != r) continue;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float prod = w[k] * y[k].get(j);
                    p[j] = p[j] + prod;
                }
            }
            if (MODE == 1) {
                store_unit<true>(a.partial, rs, H, (int64_t)u * 8, p);
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[j] = acc[j] + p[j];
            }
        }
        if (MODE == 0) store_unit<OF32>(a.out, t, H, (int64_t)u * 8, acc);
    }
    if (MODE == 0 && tid == 0 && a.out_weights) {
        float s = 0.0f;
        for (int r = 0; r < R; ++r) {
            const int32_t rs = a.rank_slot[t * R + r];
            if (rs < 0 || rs >= a.recv_rows) continue;
            float pw = 0.0f;
#pragma unroll
            for (int k = 0; k < KMAX; ++k)
                if (rows[k] >= 0 && ranks[k] == r) pw = pw + w[k];
            s = s + pw;
        }
        a.out_weights[t] = s;
    }
}

// stage B: out[t] = 0 + partial[rank_slot[t][r]] for r ascending
template <bool OF32, int KMAX>
__global__ __launch_bounds__(kCombThreads) void dedup_sum_kernel(CombineArgs a) {
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t H = a.H;
    const int units = (int)(H / 8);
    const int R = a.R;
    for (int u = tid; u < units; u += (int)blockDim.x) {
        float acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
        for (int r = 0; r < R; ++r) {
            const int32_t rs = a.rank_slot[t * R + r];
            if (rs < 0 || rs >= a.recv_rows) continue;
            Unit<true> p;
            p.load(a.partial, rs, H, (int64_t)u * 8);
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] = acc[j] + p.get(j);
        }
        store_unit<OF32>(a.out, t, H, (int64_t)u * 8, acc);
    }
    if (tid == 0 && a.out_weights) {
        int rows[KMAX], ranks[KMAX];
        float w[KMAX];
        // entries are read by lane 0 alone here: no wave-wide broadcast needed
        for (int k = 0; k < KMAX; ++k) {
            rows[k] = -1;
            ranks[k] = -1;
            w[k] = 0.0f;
            if (k >= a.K) continue;
            const int64_t r = a.tok_map[t * a.K + k];
            const int32_t e = a.idx[t * a.K + k];
            if (r >= 0 && r < a.y_rows && e >= 0 && e < a.E) {
                rows[k] = (int)r;
                ranks[k] = e / (a.E / a.R);
                w[k] = a.w[t * a.K + k];
            }
        }
        float s = 0.0f;
        for (int r = 0; r < R; ++r) {
            const int32_t rs = a.rank_slot[t * R + r];
            if (rs < 0 || rs >= a.recv_rows) continue;
            float pw = 0.0f;
            for (int k = 0; k < KMAX; ++k)
                if (rows[k] >= 0 && ranks[k] == r) pw = pw + w[k];
            s = s + pw;
        }
        a.out_weights[t] = s;
    }
}

int comb_threads(int units, int vpt) {
    int per = (units + vpt - 1) / vpt;
    int th = ((per + kWave - 1) / kWave) * kWave;
    if (th > kCombThreads) th = kCombThreads;
    if (th < kWave) th = kWave;
    return th;
}

// One unit per lane and pass: few VGPRs, so four 8-wave workgroups fit on a CU
// and one workgroup's routing latency hides behind the others' gathers.
template <bool YF32, bool OF32, int KMAX>
void plain_go(const CombineArgs& a, hipStream_t s) {
    const int units = (int)(a.H / 8);
    constexpr int VPT = 1;
    combine_kernel<YF32, OF32, KMAX, VPT>
        <<<dim3((unsigned)a.T), dim3(comb_threads(units, VPT)), 0, s>>>(a);
}

template <bool YF32, bool OF32, int KMAX>
void dedup_go(const CombineArgs& a, hipStream_t s) {
    const int units = (int)(a.H / 8);
    const dim3 grid((unsigned)a.T), block(comb_threads(units, 1));
    if (a.partial) {
        dedup_combine_kernel<YF32, OF32, KMAX, 1><<<grid, block, 0, s>>>(a);
        dedup_sum_kernel<OF32, KMAX><<<grid, block, 0, s>>>(a);
    } else {
        dedup_combine_kernel<YF32, OF32, KMAX, 0><<<grid, block, 0, s>>>(a);
    }
}

template <bool YF32, bool OF32>
void by_k(const CombineArgs& a, hipStream_t s) {
    const bool dd = a.R > 0;
#define MOE_K_CASE(KM)                                   \
    if (a.K <= KM) {                                     \
        if (dd) dedup_go<YF32, OF32, KM>(a, s);          \
        else plain_go<YF32, OF32, KM>(a, s);             \
        return;                                          \
    }
    MOE_K_CASE(2)
    MOE_K_CASE(4)
    MOE_K_CASE(8)
    MOE_K_CASE(16)
#undef MOE_K_CASE
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
    if (a.T == 0) return hipSuccess;
    if (a.y_f32) {
        if (a.out_f32) by_k<true, true>(a, s);
        else by_k<true, false>(a, s);
    } else {
        if (a.out_f32) by_k<false, true>(a, s);
        else by_k<false, false>(a, s);
    }
    return hipGetLastError();
}

}  // namespace moe

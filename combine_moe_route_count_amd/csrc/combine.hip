// combine.hip - weighted gather-reduce of each token's expert outputs back to
// token order, plus out_weights.
//
// One workgroup per (token, chunk of the row).  Lanes below K read the token's
// tok_map entries and weights once and broadcast them to the wave with
// readlane, so every branch on an entry is wave-uniform.  Each lane owns a unit
// of 8 bf16 or 4 f32 elements: it first issues the 16-byte loads of all K rows
// for its unit (the load-first gather of "feat(EPv2): [preview] internode
// dispatch/combine over CCO/GDA", ROCm/mori pull 625, commit log: 16 B vector
// gather), then reduces in f32 in ascending k with a separately rounded
// multiply and add (the build disables contraction), and stores the unit as
// bf16 or f32.  The weight
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

constexpr int kCombThreads = 256;

// Elements per lane-unit of the gathers: one 16-byte load per row, 8 bf16 or
// 4 f32.  The 4-element f32 unit keeps the f32 forms under 64 VGPRs (8 waves
// per SIMD) as the bf16 ones are.
constexpr int unit_elems(bool yf32) { return yf32 ? 4 : 8; }

// unit_elems(YF32) consecutive elements of row `row` starting at element col,
// as f32.
template <bool YF32>
struct Unit;

template <>
struct Unit<false> {  // bf16: one 16-byte load
    u32x4 a;
    __device__ __forceinline__ void clear() { a = u32x4{0, 0, 0, 0}; }
    __device__ __forceinline__ void settle() { asm volatile("" : "+v"(a)); }
    __device__ __forceinline__ void load(const void* y, int64_t row, int64_t H, int64_t col) {
        a = ld16_stream((const uint16_t*)y + row * H + col);
    }
    __device__ __forceinline__ float get(int j) const {
        return (j & 1) ? bf16hi(a[j >> 1]) : bf16lo(a[j >> 1]);
    }
    // the same, widened where it is used: inside a loop the compiler would
    // otherwise widen every row once, before the loop, and keep 8 floats per row
    __device__ __forceinline__ float get_here(int j) const {
        uint32_t w = a[j >> 1];
        asm volatile("" : "+v"(w));
        return (j & 1) ? bf16hi(w) : bf16lo(w);
    }
};

template <>
struct Unit<true> {  // f32: one 16-byte load
    u32x4 a;
    __device__ __forceinline__ float get_here(int j) const { return get(j); }
    __device__ __forceinline__ void clear() { a = u32x4{0, 0, 0, 0}; }
    __device__ __forceinline__ void settle() { asm volatile("" : "+v"(a)); }
    __device__ __forceinline__ void load(const void* y, int64_t row, int64_t H, int64_t col) {
        a = ld16_stream((const float*)y + row * H + col);
    }
    __device__ __forceinline__ float get(int j) const {
        // copied to a scalar first: this compiler's __builtin_bit_cast of a
        // vector-element lvalue (a[j] directly) reads element 0 for every j
        const uint32_t v = a[j];
        return __builtin_bit_cast(float, v);
    }
};

// EL (4 or 8) results of one lane-unit, stored as f32 (16-byte stores) or
// bf16 (one 16-byte store of 8, or one 8-byte store of 4).
template <bool OF32, int EL>
__device__ __forceinline__ void store_unit(void* out, int64_t row, int64_t H, int64_t col,
                                           const float (&acc)[EL]) {
    static_assert(EL == 4 || EL == 8, "lane-unit of 4 or 8 elements");
    // if constexpr: the branches index acc up to 7, which must not even be
    // instantiated for a 4-element unit
    if constexpr (OF32) {
        float* p = (float*)out + row * H + col;
#pragma unroll
        for (int h = 0; h < EL / 4; ++h) {
            u32x4 a;
#pragma unroll
            for (int j = 0; j < 4; ++j) a[j] = __builtin_bit_cast(uint32_t, acc[4 * h + j]);
            st16_stream(p + 4 * h, a);
        }
    } else if constexpr (EL == 8) {
        u32x4 a;
#pragma unroll
        for (int j = 0; j < 4; ++j) a[j] = pack_bf16x2(acc[2 * j], acc[2 * j + 1]);
        st16_stream((uint16_t*)out + row * H + col, a);
    } else {
        u32x2 a;
#pragma unroll
        for (int j = 0; j < 2; ++j) a[j] = pack_bf16x2(acc[2 * j], acc[2 * j + 1]);
        __builtin_nontemporal_store(a, (u32x2*)((uint16_t*)out + row * H + col));
    }
}

// EL f32 partial sums into row rs of the two-stage dedup combine's partial
// buffer (16 KB rows at H=4096).  Plain write-back stores: a write-heavy pass
// over large f32 rows, where they beat the non-temporal ones (762 against
// 783 us for the two-stage combine), as for the f32 row copies of the dispatch.
template <int EL>
__device__ __forceinline__ void store_partial(float* partial, int rs, int64_t H, int64_t col,
                                              const float (&p)[EL]) {
    const RowOut<kStorePlain> out(partial + (int64_t)rs * H, H * 4);
#pragma unroll
    for (int h = 0; h < EL / 4; ++h) {
        u32x4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = __builtin_bit_cast(uint32_t, p[4 * h + j]);
        out.st16((int)((col + 4 * h) * 4), v);
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

// Work decomposition: workgroup (c, t) owns units [c*C, c*C + C) of token t,
// one lane-unit per lane, so every lane issues the loads of all K rows at
// once and there is no second pass.  Chunks of at most 256 units (the
// geometry's combine_chunk_units) keep the workgroups small enough that several
// fit on a CU and one workgroup's routing round trip overlaps with the others'
// gathers.

struct Chunking {
    int units;   // 8-element units per row
    int nch;     // chunks per token
    int C;       // units per chunk
};

inline Chunking chunking(int64_t H, int unit_elems = 8) {
    Chunking ch;
    ch.units = (int)(H / unit_elems);
    const int cu = geometry().combine_chunk_units;
    ch.nch = (ch.units + cu - 1) / cu;
    ch.C = (ch.units + ch.nch - 1) / ch.nch;
    return ch;
}

constexpr int kXcds = 8;   // accelerator complex dies of an MI355X, each with its own L2

// Work item wi -> (token t, chunk c).  Workgroups go to the 8 XCDs round-robin
// in launch order, so within each group of 8 tokens the items are laid out
// chunk-major: chunk c of tokens 8g..8g+7 are 8 consecutive items, and every
// chunk of a token runs on the same XCD, where the token's routing entries
// (tok_map, weights, block scales of its rows) stay in that XCD's L2 after
// the first chunk reads them.  Consecutive items still cover neighbouring
// output rows.  The last T % 8 tokens keep the token-major order.  Measured:
// bf16 combine at T=8192 H=7168 K=8 (4 chunks per token) 173.0-173.7 ->
// 170.7-171.9 us; fused dedup combine (T=16384 H=4096 f32, R=8) 322-327 ->
// 305-311 us, two-stage 762-764 -> 747-749 us.  The e4m3 and e2m1 combines keep
// the token-major order: with this one they fetched fewer bytes (their block
// scale rows once per token, 522 -> 493 MB for e4m3) but took 0.3-0.5 us longer.
__device__ __forceinline__ void item_of(int64_t wi, int64_t T, int nch, int64_t& t, int& c) {
    const int64_t grouped = (T / kXcds) * kXcds * nch;
    if (nch > 1 && wi < grouped) {
        const int64_t G = (int64_t)kXcds * nch;
        const int64_t g = wi / G, r = wi - g * G;
        c = (int)(r / kXcds);
        t = g * kXcds + (r - (int64_t)c * kXcds);
    } else {
        t = wi / nch;
        c = (int)(wi - t * nch);
    }
}

// ---------------------------------------------------------------------------
// plain combine: acc = 0; acc = acc + w_k * y_k for k ascending
// ---------------------------------------------------------------------------
template <bool YF32, bool OF32, int KMAX>
__device__ __forceinline__ void combine_item(const CombineArgs& a, int64_t t, int c, int C) {
    constexpr int EL = unit_elems(YF32);
    const int64_t H = a.H;
    const int units = (int)(H / EL);
    int rows[KMAX];
    float w[KMAX];
    token_entries<KMAX>(a, t, rows, w);

    const int u = c * C + (int)threadIdx.x;
    if ((int)threadIdx.x < C && u < units) {
        Unit<YF32> y[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (rows[k] >= 0) y[k].load(a.y, rows[k], H, (int64_t)u * EL);
        float acc[EL];
#pragma unroll
        for (int j = 0; j < EL; ++j) acc[j] = 0.0f;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (rows[k] < 0) continue;
#pragma unroll
            for (int j = 0; j < EL; ++j) {
                const float p = w[k] * y[k].get(j);
                acc[j] = acc[j] + p;
            }
        }
        store_unit<OF32, EL>(a.out, t, H, (int64_t)u * EL, acc);
    }
    if (c == 0 && threadIdx.x == 0 && a.out_weights) {
        float s = 0.0f;
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (rows[k] >= 0) s = s + w[k];
        a.out_weights[t] = s;
    }
}

template <bool YF32, bool OF32, int KMAX>
__global__ __launch_bounds__(kCombThreads) void combine_kernel(CombineArgs a, int C, int nch) {
    const int64_t items = a.T * nch;
    for (int64_t wi = blockIdx.x; wi < items; wi += gridDim.x) {
        int64_t t;
        int c;
        item_of(wi, a.T, nch, t, c);
        combine_item<YF32, OF32, KMAX>(a, t, c, C);
    }
}

// ---------------------------------------------------------------------------
// combine of fp8 expert outputs: v = f32(q) * s (the row's block scale, 1 for
// the direct cast), then acc = acc + w_k * v for k ascending.  Each lane loads
// 8 bytes of codes per row plus the row's scale and dequantizes inside the
// reduce: e4m3, 8 elements per lane-unit, two codes per v_cvt_pk_f32_fp8; FP4,
// e2m1, 16 elements per lane-unit, eight codes per gfx950 scaled conversion
// (scale 1).  Both forms stay under 64 VGPRs (8 waves per SIMD): the e4m3 one
// ran 104 us against 106.6 with 16-element units (88 VGPRs), the e2m1 one 71.1
// against 73.1 with its codes held in the wider array (76 VGPRs); 8-element
// e2m1 units (4-byte loads) took 84 us.
// ---------------------------------------------------------------------------
constexpr int quant_unit_elems(bool fp4) { return fp4 ? 16 : 8; }
template <bool OF32, int KMAX, bool FP4>
__device__ __forceinline__ void combine_fp8_item(const CombineArgs& a, int64_t t, int c, int C) {
    constexpr int EL = quant_unit_elems(FP4);
    const int64_t H = a.H;
    const int units = (int)(H / EL);
    const int64_t nblk = H / kFp8Block;
    const int64_t row_bytes = FP4 ? H / 2 : H;
    int rows[KMAX];
    float w[KMAX];
    token_entries<KMAX>(a, t, rows, w);

    const int u = c * C + (int)threadIdx.x;
    if ((int)threadIdx.x < C && u < units) {
        const uint8_t* q = (const uint8_t*)a.y;
        u32x2 code[KMAX];
        float scl[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (rows[k] < 0) continue;
            code[k] = ld8_stream(q + (int64_t)rows[k] * row_bytes + (int64_t)u * 8);
            scl[k] = a.y_scales ? a.y_scales[(int64_t)rows[k] * nblk + u / (kFp8Block / EL)] : 1.0f;
        }
        float acc[EL];
#pragma unroll
        for (int j = 0; j < EL; ++j) acc[j] = 0.0f;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (rows[k] < 0) continue;
            float v[EL];
            if constexpr (FP4) {
                float h0[8], h1[8];
                unpack_e2m1x8(code[k][0], h0);
                unpack_e2m1x8(code[k][1], h1);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    v[j] = h0[j];
                    v[8 + j] = h1[j];
                }
            } else {
#pragma unroll
                for (int d = 0; d < 2; ++d) {
                    unpack_e4m3x2<false>(code[k][d], v[4 * d], v[4 * d + 1]);
                    unpack_e4m3x2<true>(code[k][d], v[4 * d + 2], v[4 * d + 3]);
                }
            }
            // v * 1.0f == v bitwise, so when every lane's block scale of this row
            // is 1 (all unscaled blocks) the dequantize multiply is skipped; the
            // VALU, not HBM, is what the quantized forms run short of
            if (ballot64(scl[k] != 1.0f) == 0) {
#pragma unroll
                for (int j = 0; j < EL; ++j) {
                    const float p = w[k] * v[j];
                    acc[j] = acc[j] + p;
                }
            } else {
#pragma unroll
                for (int j = 0; j < EL; ++j) {
                    const float dq = v[j] * scl[k];
                    const float p = w[k] * dq;
                    acc[j] = acc[j] + p;
                }
            }
        }
#pragma unroll
        for (int h = 0; h < EL / 8; ++h) {
            float part[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) part[j] = acc[8 * h + j];
            store_unit<OF32, 8>(a.out, t, H, (int64_t)u * EL + 8 * h, part);
        }
    }
    if (c == 0 && threadIdx.x == 0 && a.out_weights) {
        float s = 0.0f;
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (rows[k] >= 0) s = s + w[k];
        a.out_weights[t] = s;
    }
}

template <bool OF32, int KMAX, bool FP4>
__global__ __launch_bounds__(kCombThreads) void combine_fp8_kernel(CombineArgs a, int C, int nch) {
    const int64_t items = a.T * nch;
    for (int64_t wi = blockIdx.x; wi < items; wi += gridDim.x) {
        const int64_t t = wi / nch;   // token-major: see item_of
        combine_fp8_item<OF32, KMAX, FP4>(a, t, (int)(wi - t * nch), C);
    }
}

// ---------------------------------------------------------------------------
// dedup combine
//   MODE 0: per-rank partials kept in registers, out written (one kernel)
//   MODE 1: per-rank partials written to `partial` (stage A)
// ---------------------------------------------------------------------------
// Routing of token t for the dedup forms, every load in flight together:
// lanes below K read tok_map, w and idx, lanes below R read rank_slot.  The
// entries are broadcast to the wave; rank r's recv row stays in lane r and is
// fetched with recv_row(r), so the per-rank loops do no memory access.
template <int KMAX>
struct DedupToken {
    int rows[KMAX];
    float w[KMAX];
    int ranks[KMAX];
    int my_rs;    // lane r: recv row of rank r, or -1
    __device__ __forceinline__ int recv_row(int r) const { return readlane(my_rs, r); }
};

template <int KMAX>
__device__ __forceinline__ void dedup_token(const CombineArgs& a, int64_t t, DedupToken<KMAX>& d) {
    const int lane = threadIdx.x % kWave;
    const int er = a.E / a.R;
    int my_row = -1, my_rank = -1, my_rs = -1;
    float my_w = 0.0f;
    if (lane < a.K) {
        const int64_t r = a.tok_map[t * a.K + lane];
        const float wk = a.w[t * a.K + lane];
        const int32_t e = a.idx[t * a.K + lane];
        if (r >= 0 && r < a.y_rows) {
            my_row = (int)r;
            my_w = wk;
        }
        if (e >= 0 && e < a.E) my_rank = e / er;
    }
    if (lane < a.R) {
        const int32_t rs = a.rank_slot[t * a.R + lane];
        if (rs >= 0 && rs < a.recv_rows) my_rs = rs;
    }
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        d.rows[k] = readlane(my_row, k);
        d.w[k] = readlane(my_w, k);
        d.ranks[k] = readlane(my_rank, k);
    }
    d.my_rs = my_rs;
}

// Sum of the weights of the token's contributing entries, per rank then across
// ranks in ascending order (the grouping of the dedup combine).
template <int KMAX>
__device__ __forceinline__ float dedup_weight_sum(const CombineArgs& a, const DedupToken<KMAX>& d) {
    float s = 0.0f;
    for (int r = 0; r < a.R; ++r) {
        if (d.recv_row(r) < 0) continue;
        float pw = 0.0f;
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (d.rows[k] >= 0 && d.ranks[k] == r) pw = pw + d.w[k];
        s = s + pw;
    }
    return s;
}

template <bool YF32, bool OF32, int KMAX, int MODE>
__device__ __forceinline__ void dedup_item(const CombineArgs& a, int64_t t, int c, int C) {
    constexpr int EL = unit_elems(YF32);
    const int64_t H = a.H;
    const int units = (int)(H / EL);
    DedupToken<KMAX> d;
    dedup_token<KMAX>(a, t, d);

    const int u = c * C + (int)threadIdx.x;
    if ((int)threadIdx.x < C && u < units) {
        Unit<YF32> y[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            y[k].clear();
            if (d.rows[k] >= 0) y[k].load(a.y, d.rows[k], H, (int64_t)u * EL);
        }
        // one wait for all K rows: the per-rank loop below uses them under
        // conditions and, in the two-stage form, stores between the uses
#pragma unroll
        for (int k = 0; k < KMAX; ++k) y[k].settle();
        float acc[EL];
#pragma unroll
        for (int j = 0; j < EL; ++j) acc[j] = 0.0f;
        for (int r = 0; r < a.R; ++r) {
            const int rs = d.recv_row(r);
            if (rs < 0) continue;
            float p[EL];
#pragma unroll
            for (int j = 0; j < EL; ++j) p[j] = 0.0f;
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                if (d.rows[k] < 0 || d.ranks[k] != r) continue;
#pragma unroll
                for (int j = 0; j < EL; ++j) {
                    const float prod = d.w[k] * y[k].get_here(j);
                    p[j] = p[j] + prod;
                }
            }
            if (MODE == 1) {
                store_partial<EL>(a.partial, rs, H, (int64_t)u * EL, p);
            } else {
#pragma unroll
                for (int j = 0; j < EL; ++j) acc[j] = acc[j] + p[j];
            }
        }
        if (MODE == 0) store_unit<OF32, EL>(a.out, t, H, (int64_t)u * EL, acc);
    }
    if (MODE == 0 && c == 0 && threadIdx.x == 0 && a.out_weights)
        a.out_weights[t] = dedup_weight_sum<KMAX>(a, d);
}

template <bool YF32, bool OF32, int KMAX, int MODE>
__global__ __launch_bounds__(kCombThreads) void dedup_combine_kernel(CombineArgs a, int C, int nch) {
    const int64_t items = a.T * nch;
    for (int64_t wi = blockIdx.x; wi < items; wi += gridDim.x) {
        int64_t t;
        int c;
        item_of(wi, a.T, nch, t, c);
        dedup_item<YF32, OF32, KMAX, MODE>(a, t, c, C);
    }
}

// stage B: out[t] = 0 + partial[rank_slot[t][r]] for r ascending.  The partial
// rows of up to kSumBatch ranks are loaded together, then added in rank order.
constexpr int kSumBatch = 8;

template <bool OF32, int KMAX>
__device__ __forceinline__ void dedup_sum_item(const CombineArgs& a, int64_t t, int c, int C) {
    constexpr int EL = unit_elems(true);       // the partial rows are f32
    const int64_t H = a.H;
    const int units = (int)(H / EL);
    DedupToken<KMAX> d;
    dedup_token<KMAX>(a, t, d);
    const int u = c * C + (int)threadIdx.x;
    if ((int)threadIdx.x < C && u < units) {
        float acc[EL];
#pragma unroll
        for (int j = 0; j < EL; ++j) acc[j] = 0.0f;
        for (int r0 = 0; r0 < a.R; r0 += kSumBatch) {
            Unit<true> p[kSumBatch];
            int rs[kSumBatch];
#pragma unroll
            for (int i = 0; i < kSumBatch; ++i) {
                rs[i] = r0 + i < a.R ? d.recv_row(r0 + i) : -1;
                p[i].clear();
                if (rs[i] >= 0) p[i].load(a.partial, rs[i], H, (int64_t)u * EL);
            }
            // one wait for the batch instead of one per conditional use
#pragma unroll
            for (int i = 0; i < kSumBatch; ++i) p[i].settle();
#pragma unroll
            for (int i = 0; i < kSumBatch; ++i) {
                if (rs[i] < 0) continue;
#pragma unroll
                for (int j = 0; j < EL; ++j) acc[j] = acc[j] + p[i].get(j);
            }
        }
        store_unit<OF32, EL>(a.out, t, H, (int64_t)u * EL, acc);
    }
    if (c == 0 && threadIdx.x == 0 && a.out_weights) a.out_weights[t] = dedup_weight_sum<KMAX>(a, d);
}

template <bool OF32, int KMAX>
__global__ __launch_bounds__(kCombThreads) void dedup_sum_kernel(CombineArgs a, int C, int nch) {
    const int64_t items = a.T * nch;
    for (int64_t wi = blockIdx.x; wi < items; wi += gridDim.x) {
        int64_t t;
        int c;
        item_of(wi, a.T, nch, t, c);
        dedup_sum_item<OF32, KMAX>(a, t, c, C);
    }
}

int threads_for(int C) {
    int th = ((C + kWave - 1) / kWave) * kWave;
    return th < kWave ? kWave : th;
}

dim3 item_grid(int64_t items) {
    return dim3((unsigned)(items < kMaxGrid ? items : kMaxGrid));
}

// Residency cap of the bf16 gather.  At the 8 workgroups per CU its registers
// allow, the gather keeps about 64 MB of row loads in flight chip-wide and
// HBM delivers less (181 us for the 1.06 GB combine at T=8192 H=7168 K=8);
// at 4 or 5 per CU (32-40 MB in flight) the same launch takes 173 us, at 3 per
// CU 185 us.  The launch reserves LDS it never touches so that at most
// kGatherWgsPerCu workgroups share a CU's 160 KB.  The f32-row dedup forms
// lost time under the same cap (fused dedup combine 321 -> 356 us), and so did
// the quantized combines, whose dequantize needs the VALU latency hiding of
// full residency (e4m3 104 -> 131 us); those launch uncapped.
// (The cap is the geometry's combine_wgs_per_cu, 5 by default.)
inline size_t gather_lds_reserve() {
    const int n = geometry().combine_wgs_per_cu;
    return n > 0 ? kLdsPerCu / n : 0;
}

template <bool YF32, bool OF32, int KMAX>
void plain_go(const CombineArgs& a, hipStream_t s) {
    const Chunking ch = chunking(a.H, unit_elems(YF32));
    const size_t lds = YF32 ? 0 : gather_lds_reserve();
    combine_kernel<YF32, OF32, KMAX>
        <<<item_grid(a.T * ch.nch), dim3(threads_for(ch.C)), lds, s>>>(a, ch.C, ch.nch);
}

template <bool YF32, bool OF32, int KMAX>
void dedup_go(const CombineArgs& a, hipStream_t s) {
    const Chunking ch = chunking(a.H, unit_elems(YF32));
    const dim3 grid = item_grid(a.T * ch.nch), block(threads_for(ch.C));
    if (a.partial) {
        dedup_combine_kernel<YF32, OF32, KMAX, 1><<<grid, block, 0, s>>>(a, ch.C, ch.nch);
        const Chunking cs = chunking(a.H, unit_elems(true));
        dedup_sum_kernel<OF32, KMAX>
            <<<item_grid(a.T * cs.nch), dim3(threads_for(cs.C)), 0, s>>>(a, cs.C, cs.nch);
    } else {
        dedup_combine_kernel<YF32, OF32, KMAX, 0><<<grid, block, 0, s>>>(a, ch.C, ch.nch);
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
    if (dd) MOE_K_CASE(6)   // the dedup forms hold K f32 rows per lane: fewer registers at K=6
    MOE_K_CASE(8)
    MOE_K_CASE(16)
#undef MOE_K_CASE
}

template <bool OF32, int KMAX, bool FP4>
void fp8_go(const CombineArgs& a, hipStream_t s) {
    const Chunking ch = chunking(a.H, quant_unit_elems(FP4));
    combine_fp8_kernel<OF32, KMAX, FP4>
        <<<item_grid(a.T * ch.nch), dim3(threads_for(ch.C)), 0, s>>>(a, ch.C, ch.nch);
}

template <bool OF32, bool FP4>
void fp8_by_k(const CombineArgs& a, hipStream_t s) {
    if (a.K <= 2) fp8_go<OF32, 2, FP4>(a, s);
    else if (a.K <= 4) fp8_go<OF32, 4, FP4>(a, s);
    else if (a.K <= 8) fp8_go<OF32, 8, FP4>(a, s);
    else fp8_go<OF32, 16, FP4>(a, s);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
    if (a.T == 0) return hipSuccess;
    if (a.y_fp8) {
        if (a.y_fp4) {
            if (a.out_f32) fp8_by_k<true, true>(a, s);
            else fp8_by_k<false, true>(a, s);
        } else {
            if (a.out_f32) fp8_by_k<true, false>(a, s);
            else fp8_by_k<false, false>(a, s);
        }
    } else if (a.y_f32) {
        if (a.out_f32) by_k<true, true>(a, s);
        else by_k<true, false>(a, s);
    } else {
        if (a.out_f32) by_k<false, true>(a, s);
        else by_k<false, false>(a, s);
    }
    return hipGetLastError();
}

}  // namespace moe

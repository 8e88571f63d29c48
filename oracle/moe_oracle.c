/*
 * moe_oracle.c - CPU oracle for the MoE route-count / dispatch / combine path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * statement of what the GPU library computes.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it; the library itself
 * never calls it and shares no code, header or table with it.
 *
 * Sources (pages as titled; sections named):
 *   [mori#448]  "Draft: cco + flydsl dispatch/combine" (ROCm/mori pull 448):
 *               PR description (dispatch, combine gather reducing in f32),
 *               commit "Port mori/FlyDSL StdMoE ..." (convert_dispatch_output:
 *               per-(token,k) repack into packed_x[expert,slot], packed_cnt,
 *               packed_src, int64 tok_map with a -1 sentinel;
 *               convert_combine_input: sum_k wts[k]*packed_x[slot_k]),
 *               commit "Combine now reduces the K forwarded per-token weight
 *               vectors into out_weights",
 *               commit "Port mori's Fp8BlockwiseQuant ..." (128-element blocks,
 *               scale rule, OCP e4m3 maximum 448),
 *               commit "EpDispatchCombineOp gains enable_std_moe ..." (over-cap
 *               entries take the drop path).
 *   [mori#625]  "feat(EPv2): [preview] internode dispatch/combine over CCO/GDA"
 *               (ROCm/mori pull 625), commit log: the -1 expert sentinel must be
 *               tested before dividing by experts-per-rank.
 *   [cccl#12311] "Add standalone cuda.coop.cutlass package": exclusive scans
 *               take an explicit initial value (0 here).
 *   [MoonEP#34] "Drop cooperative launch from the CTA-independent local kernels",
 *               "Why it's worth doing": dedup groups are reduced locally, then
 *               across ranks.
 *
 * Readings taken where the pages are silent or garbled (each one is stated
 * again next to the code that depends on it):
 *   R-slot   slots inside an expert follow the flat entry order f = t*K + k
 *            (a stable counting sort), so the layout is deterministic.
 *   R-valid  an entry is valid iff 0 <= id < E; -1 means "no expert"; any
 *            other id is invalid and counted in stats[0].
 *   R-cap    cap > 0: padded layout, expert e owns rows [e*cap, e*cap+cap);
 *            cap == 0: compact layout, expert e starts at off[e].  Entries past
 *            the capacity, or past packed_rows, are dropped (tok_map = -1) and
 *            counted in stats[1]; the dropped ones are the latest in f.
 *   R-fp8    OCP e4m3fn (bias 7, max 448, no infinities), round to nearest even.
 *            Block of 128: amax = max|x| over the block's finite elements;
 *            amax > 448: s = amax/448 and q = e4m3(x*448/amax), the quotient
 *            of the exact product correctly rounded to f32 (no intermediate
 *            overflow); otherwise s = 1 and q = e4m3(x).
 *   R-nonfinite  the encoders saturate: +-inf (and any magnitude above the
 *            format's maximum) give +-448 (e4m3) or +-6 (e2m1) with the sign
 *            kept; NaN gives the e4m3 NaN code S.1111.111 with the NaN's sign.
 *            e2m1 has no NaN code: a block holding a NaN is stored as all-zero
 *            codes with a NaN block scale, so the whole block decodes to NaN
 *            (the block-scale NaN convention of the OCP microscaling formats).
 *            Infinities never count toward amax, so one infinity does not
 *            flush its block to zero.
 *   R-comb   acc starts at +0.0f and takes, for k ascending, acc = acc + (w*y)
 *            with the product and the sum each rounded to f32 (no fused
 *            multiply-add).  out_weights[t] is the f32 sum of the weights of
 *            the entries that contributed, in the same order.
 *   R-comb8  fp8 expert outputs: v = f32(e4m3(q)) * s with the block's f32
 *            scale (1 when no scales are given), one rounded multiply and no
 *            bf16 step, then the R-comb reduction over v.
 *   R-fp4    fp4 payload: OCP e2m1 (max 6), round to nearest even, two codes
 *            per byte with element 2i in the low nibble; the R-fp8 block rule
 *            with 6 in place of 448 (s = amax/6 when amax > 6, else 1), and
 *            R-nonfinite.
 *   R-comb4  fp4 expert outputs: v = f32(e2m1(q)) * s, then the R-comb
 *            reduction, as R-comb8.
 *   R-prequant  fp8 input (e4m3 codes with one f32 scale per 128-element
 *            block) is dispatched byte for byte and each token's scale row is
 *            forwarded unchanged to every packed row of the token.
 *   R-replay a cached tok_map is reused as it stands: entries inside
 *            [0, packed_rows) get their token's row, nothing else is written.
 *   R-dedup  virtual rank of expert e is e / (E/R), computed only for valid e.
 *            Recv rows: one per (t, r in M[t]) in t order per rank; rows past
 *            recv_rows are dropped with every entry they carry.  Surviving
 *            entries get the same expert slots as a plain dispatch of the
 *            surviving ids.  Combine: per-rank partial sums (R-comb order
 *            restricted to that rank's entries), then out = 0 + partials in
 *            ascending rank order.
 *
 * Parity pins (what checks this file against something other than itself):
 * counts / offsets / slots against numpy bincount, cumsum and stable argsort
 * and exhaustive tiny routings; rows against numpy fancy indexing; the e4m3
 * encoder exhaustively against torch.float8_e4m3fn over every bf16 value; the
 * bf16 encoder against torch's float32->bfloat16 rounding; combine against the
 * identity-expert closed form out = (sum_k w_k) * x, exact dyadic cases and
 * hand-derived order / fusion cases; dedup against python-set rank masks and
 * the plain dispatch of the same ids; the non-finite and near-overflow
 * handling of the block packs against hand-derived codes from the format
 * definitions and against the power-of-two homogeneity of the block rule.
 * The choice of the fp8 scale rule among the readings of the garbled formula
 * is a reading, not a pin.
 *
 * Build: gcc -O2 -std=c99 -ffp-contract=off -fopenmp -shared -fPIC
 * (-ffp-contract=off keeps every multiply and add separately rounded).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_BF16 = 0, ORC_F32 = 1, ORC_FP8 = 2, ORC_FP4 = 3 };

/* ------------------------------------------------------------------ */
/* number formats                                                       */
/* ------------------------------------------------------------------ */

/* bf16 is the upper half of an IEEE binary32.  Widening is exact. */
static float bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Narrow binary32 -> bf16, round to nearest, ties to even.  The 16 discarded
 * bits are compared against half of the last kept bit; a carry out of the
 * mantissa correctly bumps the exponent (up to infinity).  NaN stays NaN. */
static uint16_t f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t kept = u >> 16;
    uint32_t dropped = u & 0xffffu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))
        kept += 1u;
    return (uint16_t)kept;
}

/* OCP e4m3fn: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.
 * Exponent field 0: subnormal m * 2^-9.  Fields 1..15: (1 + m/8) * 2^(E-7),
 * except E=15, m=7 which is NaN.  Largest finite value 448 = 1.75 * 2^8. */
static float e4m3_to_f32(uint8_t b) {
    int E = (b >> 3) & 15, m = b & 7;
    double v;
    if (E == 15 && m == 7)
        return NAN;
    if (E == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, E - 7);
    return (float)((b & 0x80) ? -v : v);
}

/* Encode to e4m3fn, round to nearest, ties to even.  The sign is kept for
 * zero results (-0 and tiny negatives give 0x80).  Saturating (R-nonfinite):
 * a magnitude above 448, infinity included, gives +-448 (S.1111.110; between
 * 448 and 464 that is also the nearest value); NaN gives S.1111.111. */
static uint8_t f32_to_e4m3(float v) {
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v))
        return (uint8_t)(sign | 0x7F);
    double a = fabs((double)v);
    if (a > 448.0)
        return (uint8_t)(sign | 0x7E);
    if (a < 0.015625) {
        /* below 2^-6 the grid is the subnormal step 2^-9; a rounded count of 8
         * is exactly the smallest normal 2^-6, whose code is also 8 */
        double q = nearbyint(a * 512.0);
        return (uint8_t)(sign | (uint8_t)q);
    }
    int e2;
    (void)frexp(a, &e2);          /* a = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1;               /* a = (1 + frac) * 2^E        */
    double frac = ldexp(a, -E) - 1.0;
    double q = nearbyint(frac * 8.0);
    if (q == 8.0) {
        q = 0.0;
        E += 1;
    }
    return (uint8_t)(sign | (uint8_t)(((E + 7) << 3) | (int)q));
}

/* OCP e2m1 (fp4): 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit.
 * Exponent field 0: subnormal m * 0.5.  Fields 1..3: (1 + m/2) * 2^(E-1).
 * Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinities, no NaN. */
static float e2m1_to_f32(uint8_t n) {
    int E = (n >> 1) & 3, m = n & 1;
    double v = E == 0 ? 0.5 * m : ldexp(1.0 + m / 2.0, E - 1);
    return (float)((n & 8) ? -v : v);
}

/* Encode to e2m1, round to nearest, ties to the even code (mantissa bit 0);
 * magnitudes above 6, infinity included, saturate to 6; the sign is kept for
 * zero results.  The format has no NaN: the block rule handles NaN before
 * calling this, which maps it to code 0. */
static uint8_t f32_to_e2m1(float v) {
    uint8_t sign = signbit(v) ? 8 : 0;
    if (isnan(v))
        return 0;
    double a = fabs((double)v);
    uint8_t best = 0;
    double bd = a;                              /* distance to code 0 */
    for (uint8_t c = 1; c < 8; ++c) {
        double d = fabs(a - (double)e2m1_to_f32(c));
        if (d < bd || (d == bd && (c & 1) == 0)) {
            bd = d;
            best = c;
        }
    }
    if (a > 6.0)
        best = 7;
    return sign | best;
}

static float load_elem(const void* base, int dt, int64_t i) {
    if (dt == ORC_BF16)
        return bf16_to_f32(((const uint16_t*)base)[i]);
    return ((const float*)base)[i];
}

static size_t elem_bytes(int dt) { return dt == ORC_F32 ? 4 : (dt == ORC_BF16 ? 2 : 1); }

/* ------------------------------------------------------------------ */
/* blockwise fp8 / fp4 pack of one row                                  */
/* ------------------------------------------------------------------ */

#define FP8_BLOCK 128
#define E4M3_MAX 448.0f

/* Largest magnitude among the finite elements of a 128-element bf16 block (0
 * when none is finite); sets *has_nan when the block holds a NaN. */
static float block_finite_amax(const uint16_t* xb, int* has_nan) {
    float amax = 0.0f;
    *has_nan = 0;
    for (int h = 0; h < FP8_BLOCK; ++h) {
        float x = bf16_to_f32(xb[h]);
        if (isnan(x))
            *has_nan = 1;
        else if (isfinite(x) && fabsf(x) > amax)
            amax = fabsf(x);
    }
    return amax;
}

/* x * m / amax for a bf16 x and a finite amax > m, rounded once to f32: the
 * product is exact in double (8-bit and 3-bit significands, far inside the
 * double range, so a block near the bf16 maximum does not overflow), the
 * double quotient is correctly rounded, and rounding it on to f32 gives the
 * correctly rounded f32 quotient because 53 >= 2*24 + 2 (double rounding is
 * innocuous for division at that precision, S. A. Figueroa, "When is double
 * rounding innocuous?", 1995).  Infinite x gives an infinite quotient and NaN
 * stays NaN; the encoders saturate or keep them (R-nonfinite). */
static float scaled_quotient(float x, float m, float amax) {
    return (float)(((double)x * (double)m) / (double)amax);
}

/* fp8 blockwise pack of one row (readings R-fp8, R-nonfinite) */
static void fp8_pack_row(const uint16_t* xrow, int64_t H, uint8_t* q, float* s) {
    for (int64_t b = 0; b * FP8_BLOCK < H; ++b) {
        const uint16_t* xb = xrow + b * FP8_BLOCK;
        int has_nan;
        float amax = block_finite_amax(xb, &has_nan);
        int scaled = amax > E4M3_MAX;
        s[b] = scaled ? amax / E4M3_MAX : 1.0f;
        for (int h = 0; h < FP8_BLOCK; ++h) {
            float v = bf16_to_f32(xb[h]);
            if (scaled && !isnan(v))                  /* a NaN keeps its sign as it is */
                v = scaled_quotient(v, E4M3_MAX, amax);   /* |v| <= 448 unless x is inf */
            q[b * FP8_BLOCK + h] = f32_to_e4m3(v);
        }
    }
}

/* fp4 blockwise pack of one row (readings R-fp4, R-nonfinite): the R-fp8 rule
 * with the e2m1 maximum 6.  Per 128-element block: amax over the finite
 * elements; amax > 6 gives s = amax/6 and q = e2m1(x*6/amax); otherwise s = 1
 * and q = e2m1(x).  A block holding a NaN gets s = NaN and all-zero codes.
 * Element 2i goes to the low nibble of byte i. */
#define E2M1_MAX 6.0f

static void fp4_pack_row(const uint16_t* xrow, int64_t H, uint8_t* q, float* s) {
    for (int64_t b = 0; b * FP8_BLOCK < H; ++b) {
        const uint16_t* xb = xrow + b * FP8_BLOCK;
        int has_nan;
        float amax = block_finite_amax(xb, &has_nan);
        int scaled = amax > E2M1_MAX;
        uint8_t codes[FP8_BLOCK];
        s[b] = has_nan ? NAN : (scaled ? amax / E2M1_MAX : 1.0f);
        for (int h = 0; h < FP8_BLOCK; ++h) {
            float v = bf16_to_f32(xb[h]);
            if (scaled)
                v = scaled_quotient(v, E2M1_MAX, amax);
            codes[h] = has_nan ? 0 : f32_to_e2m1(v);
        }
        for (int h = 0; h < FP8_BLOCK; h += 2)
            q[(b * FP8_BLOCK + h) / 2] = (uint8_t)(codes[h] | (codes[h + 1] << 4));
    }
}

/* ------------------------------------------------------------------ */
/* route count: histogram and exclusive scan                            */
/* ------------------------------------------------------------------ */

/* cnt[e] = number of valid entries with id e; off[0] = 0 and
 * off[e+1] = off[e] + cnt[e] (exclusive scan, initial value 0).
 * stats[0] = ids outside [0,E) other than -1 (reading R-valid). */
int oracle_route_count(const int32_t* idx, int64_t T, int K, int E,
                       int32_t* cnt, int32_t* off, int32_t* stats) {
    int64_t n_invalid = 0;
    for (int e = 0; e < E; ++e)
        cnt[e] = 0;
    for (int64_t f = 0; f < T * K; ++f) {
        int32_t e = idx[f];
        if (e >= 0 && e < E)
            cnt[e] += 1;
        else if (e != -1)
            n_invalid += 1;
    }
    off[0] = 0;
    for (int e = 0; e < E; ++e)
        off[e + 1] = off[e] + cnt[e];
    if (stats) {
        stats[0] = (int32_t)n_invalid;
        stats[1] = 0;
        stats[2] = 0;
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* slot assignment shared by plain and dedup dispatch                   */
/* ------------------------------------------------------------------ */

/* Assign rows to the entries whose keep[f] is set (plain dispatch: every
 * valid entry; dedup: every valid entry whose recv row survived).  Walks f in
 * increasing order so each expert's entries take slots 0,1,2,... in flat
 * order (reading R-slot).  Rows: base(e) + slot with base = e*cap (padded) or
 * the exclusive scan of the kept counts (compact).  Writes tok_map,
 * packed_src, packed_cnt, packed_off; returns the number of dropped kept
 * entries.  dst_row_of[f] receives the row or -1 for the copy loop. */
static int64_t assign_slots(const int32_t* idx, const uint8_t* keep, int64_t T, int K, int E,
                            int64_t cap, int64_t packed_rows, int32_t* packed_cnt,
                            int32_t* packed_off, int32_t* packed_src, int64_t* tok_map) {
    int64_t N = T * K, dropped = 0;
    int64_t* cntk = (int64_t*)calloc((size_t)E + 1, sizeof(int64_t));
    int64_t* offk = (int64_t*)calloc((size_t)E + 1, sizeof(int64_t));
    int64_t* run = (int64_t*)calloc((size_t)E + 1, sizeof(int64_t));
    for (int64_t f = 0; f < N; ++f)
        if (keep[f])
            cntk[idx[f]] += 1;
    for (int e = 0; e < E; ++e)
        offk[e + 1] = offk[e] + cntk[e];
    for (int e = 0; e < E; ++e)
        packed_cnt[e] = 0;
    for (int64_t f = 0; f < N; ++f) {
        if (!keep[f]) {
            tok_map[f] = -1;
            continue;
        }
        int e = idx[f];
        int64_t slot = run[e]++;
        int64_t base = cap > 0 ? (int64_t)e * cap : offk[e];
        if ((cap > 0 && slot >= cap) || base + slot >= packed_rows) {
            tok_map[f] = -1;
            dropped += 1;
            continue;
        }
        int64_t row = base + slot;
        tok_map[f] = row;
        packed_src[row] = (int32_t)(f / K);
        packed_cnt[e] += 1;
    }
    if (packed_off) {
        for (int e = 0; e <= E; ++e) {
            int64_t base = cap > 0 ? (int64_t)e * cap : offk[e];
            packed_off[e] = (int32_t)(base < packed_rows ? base : packed_rows);
        }
    }
    free(cntk);
    free(offk);
    free(run);
    return dropped;
}

/* Copy (or fp8-pack) the source row of every entry with tok_map >= 0.
 * src_row_of(f) is x[t] for plain dispatch and the recv row for dedup.  An
 * fp8 source (pre-quantized input) is copied byte for byte and its scale row
 * src_scales[s] is forwarded verbatim (reading R-prequant). */
static void copy_rows(const void* src, int src_dt, const float* src_scales, int64_t H,
                      const int64_t* src_row, const int64_t* tok_map, int64_t N, void* packed,
                      int packed_dt, float* scales) {
    int64_t f;
#pragma omp parallel for schedule(dynamic, 16)
    for (f = 0; f < N; ++f) {
        int64_t row = tok_map[f];
        if (row < 0)
            continue;
        int64_t s = src_row[f];
        if (src_dt == ORC_FP8) {
            memcpy((uint8_t*)packed + (size_t)row * H, (const uint8_t*)src + (size_t)s * H,
                   (size_t)H);
            memcpy(scales + row * (H / FP8_BLOCK), src_scales + s * (H / FP8_BLOCK),
                   (size_t)(H / FP8_BLOCK) * sizeof(float));
        } else if (packed_dt == ORC_FP8) {
            fp8_pack_row((const uint16_t*)src + s * H, H, (uint8_t*)packed + row * H,
                         scales + row * (H / FP8_BLOCK));
        } else if (packed_dt == ORC_FP4) {
            fp4_pack_row((const uint16_t*)src + s * H, H, (uint8_t*)packed + row * (H / 2),
                         scales + row * (H / FP8_BLOCK));
        } else {
            size_t eb = elem_bytes(src_dt);
            memcpy((char*)packed + (size_t)row * H * eb, (const char*)src + (size_t)s * H * eb,
                   (size_t)H * eb);
        }
    }
}

/* ------------------------------------------------------------------ */
/* dispatch ([mori#448] convert_dispatch_output)                        */
/* ------------------------------------------------------------------ */

/* x_dt == ORC_FP8 is pre-quantized input: x holds e4m3 codes and x_scales the
 * f32 scale of each 128-element block; both are forwarded unchanged. */
int oracle_dispatch(const void* x, int x_dt, const float* x_scales, int64_t T, int64_t H,
                    const int32_t* idx, int K, int E, int64_t cap, int64_t packed_rows,
                    void* packed, int packed_dt, float* scales, int32_t* packed_cnt,
                    int32_t* packed_off, int32_t* packed_src, int64_t* tok_map, int32_t* stats) {
    int64_t N = T * K, n_invalid = 0;
    uint8_t* keep = (uint8_t*)malloc((size_t)N + 1);
    int64_t* src_row = (int64_t*)malloc(((size_t)N + 1) * sizeof(int64_t));
    for (int64_t f = 0; f < N; ++f) {
        int32_t e = idx[f];
        keep[f] = (e >= 0 && e < E);
        if (!keep[f] && e != -1)
            n_invalid += 1;
        src_row[f] = f / K;
    }
    int64_t dropped = assign_slots(idx, keep, T, K, E, cap, packed_rows, packed_cnt, packed_off,
                                   packed_src, tok_map);
    copy_rows(x, x_dt, x_scales, H, src_row, tok_map, N, packed, packed_dt, scales);
    if (stats) {
        stats[0] = (int32_t)n_invalid;
        stats[1] = (int32_t)dropped;
        stats[2] = 0;
    }
    free(keep);
    free(src_row);
    return 0;
}

/* Replay dispatch (reading R-replay): the routing of an earlier dispatch is
 * reused as it stands ([mori#448] commit "... replay dispatch (make_dispatch
 * replay= reuses cached tok_map, identical layout)"), so only rows move: for
 * every entry f with 0 <= tok_map[f] < packed_rows, packed[tok_map[f]] gets
 * x[f / K] exactly as the dispatch would write it (bit copy, fp8 pack of bf16,
 * or pre-quantized codes with their scale row).  Nothing else is written. */
int oracle_dispatch_replay(const void* x, int x_dt, const float* x_scales, int64_t T, int64_t H,
                           const int64_t* tok_map, int K, int64_t packed_rows, void* packed,
                           int packed_dt, float* scales) {
    int64_t N = T * K;
    int64_t* rows = (int64_t*)malloc(((size_t)N + 1) * sizeof(int64_t));
    int64_t* src_row = (int64_t*)malloc(((size_t)N + 1) * sizeof(int64_t));
    for (int64_t f = 0; f < N; ++f) {
        rows[f] = (tok_map[f] >= 0 && tok_map[f] < packed_rows) ? tok_map[f] : -1;
        src_row[f] = f / K;
    }
    copy_rows(x, x_dt, x_scales, H, src_row, rows, N, packed, packed_dt, scales);
    free(rows);
    free(src_row);
    return 0;
}

/* ------------------------------------------------------------------ */
/* combine ([mori#448] convert_combine_input and the f32 gather)        */
/* ------------------------------------------------------------------ */

/* For token t: acc = 0; for k ascending with 0 <= tok_map[t,k] < y_rows:
 * acc = acc + (w[t,k] * y[row]), product and sum each rounded to f32
 * (reading R-comb).  out[t] = acc (f32) or bf16(acc); out_weights[t] = sum of
 * the same w in the same order.  A token with no entry gives zeros. */
int oracle_combine(const void* y, int y_dt, int64_t y_rows, int64_t H, const int64_t* tok_map,
                   const float* w, int64_t T, int K, void* out, int out_dt, float* out_weights) {
    int64_t t;
#pragma omp parallel for schedule(dynamic, 4)
    for (t = 0; t < T; ++t) {
        float* acc = (float*)malloc((size_t)H * sizeof(float));
        float ws = 0.0f;
        for (int64_t h = 0; h < H; ++h)
            acc[h] = 0.0f;
        for (int k = 0; k < K; ++k) {
            int64_t row = tok_map[t * K + k];
            if (row < 0 || row >= y_rows)
                continue;
            float wk = w[t * K + k];
            for (int64_t h = 0; h < H; ++h) {
                float p = wk * load_elem(y, y_dt, row * H + h);
                acc[h] = acc[h] + p;
            }
            ws = ws + wk;
        }
        for (int64_t h = 0; h < H; ++h) {
            if (out_dt == ORC_BF16)
                ((uint16_t*)out)[t * H + h] = f32_to_bf16(acc[h]);
            else
                ((float*)out)[t * H + h] = acc[h];
        }
        if (out_weights)
            out_weights[t] = ws;
        free(acc);
    }
    return 0;
}

/* Combine of fp8 expert outputs (reading R-comb8): y arrives as e4m3 codes q
 * with one f32 scale per 128-element block of each row ([mori#448] commit
 * "Port mori's Fp8BlockwiseQuant ...": the receiving side dequantizes fp8 times
 * the block's scale and accumulates); scales == NULL is the direct cast
 * ([mori#448] commit "... make_combine_scatter ..."), i.e. every scale 1.
 * Each element is dequantized inside the reduce as v = f32(q) * s, one f32
 * multiply with no bf16 rounding in between, and then combined exactly as in
 * oracle_combine: acc = acc + (w * v) for k ascending. */
int oracle_combine_fp8(const uint8_t* q, const float* scales, int64_t y_rows, int64_t H,
                       const int64_t* tok_map, const float* w, int64_t T, int K, void* out,
                       int out_dt, float* out_weights) {
    const int64_t nblk = H / FP8_BLOCK;
    int64_t t;
#pragma omp parallel for schedule(dynamic, 4)
    for (t = 0; t < T; ++t) {
        float* acc = (float*)malloc((size_t)H * sizeof(float));
        float ws = 0.0f;
        for (int64_t h = 0; h < H; ++h)
            acc[h] = 0.0f;
        for (int k = 0; k < K; ++k) {
            int64_t row = tok_map[t * K + k];
            if (row < 0 || row >= y_rows)
                continue;
            float wk = w[t * K + k];
            for (int64_t h = 0; h < H; ++h) {
                float s = scales ? scales[row * nblk + h / FP8_BLOCK] : 1.0f;
                float v = e4m3_to_f32(q[row * H + h]) * s;
                float p = wk * v;
                acc[h] = acc[h] + p;
            }
            ws = ws + wk;
        }
        for (int64_t h = 0; h < H; ++h) {
            if (out_dt == ORC_BF16)
                ((uint16_t*)out)[t * H + h] = f32_to_bf16(acc[h]);
            else
                ((float*)out)[t * H + h] = acc[h];
        }
        if (out_weights)
            out_weights[t] = ws;
        free(acc);
    }
    return 0;
}

/* Combine of fp4 expert outputs (reading R-comb4): as oracle_combine_fp8 with
 * e2m1 codes, two per byte (element 2i in the low nibble), rows of H/2 bytes
 * ([mori#448] commit "Add the fp4 e2m1 accum path ...": packed fp4 expanded to
 * f32 with the scale, accumulated in f32). */
int oracle_combine_fp4(const uint8_t* q, const float* scales, int64_t y_rows, int64_t H,
                       const int64_t* tok_map, const float* w, int64_t T, int K, void* out,
                       int out_dt, float* out_weights) {
    const int64_t nblk = H / FP8_BLOCK;
    int64_t t;
#pragma omp parallel for schedule(dynamic, 4)
    for (t = 0; t < T; ++t) {
        float* acc = (float*)malloc((size_t)H * sizeof(float));
        float ws = 0.0f;
        for (int64_t h = 0; h < H; ++h)
            acc[h] = 0.0f;
        for (int k = 0; k < K; ++k) {
            int64_t row = tok_map[t * K + k];
            if (row < 0 || row >= y_rows)
                continue;
            float wk = w[t * K + k];
            for (int64_t h = 0; h < H; ++h) {
                uint8_t byte = q[row * (H / 2) + h / 2];
                uint8_t code = (h & 1) ? (byte >> 4) : (byte & 15);
                float s = scales ? scales[row * nblk + h / FP8_BLOCK] : 1.0f;
                float v = e2m1_to_f32(code) * s;
                float p = wk * v;
                acc[h] = acc[h] + p;
            }
            ws = ws + wk;
        }
        for (int64_t h = 0; h < H; ++h) {
            if (out_dt == ORC_BF16)
                ((uint16_t*)out)[t * H + h] = f32_to_bf16(acc[h]);
            else
                ((float*)out)[t * H + h] = acc[h];
        }
        if (out_weights)
            out_weights[t] = ws;
        free(acc);
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* dedup dispatch (virtual ranks)                                       */
/* ------------------------------------------------------------------ */

/* Rank mask M[t] = OR of 1 << (e / (E/R)) over the valid ids of token t; the
 * division happens only after the validity test, so -1 never lands on rank 0
 * ([mori#625] commit log).  recv_cnt[r] = #{t : r in M[t]}, recv_off its
 * exclusive scan.  For t ascending and r ascending in M[t] the pair (t, r)
 * takes row recv_off[r] + (number of earlier tokens with r in M); that row
 * receives a copy of x[t] and recv_src = t, rank_slot[t][r] = row.  All other
 * rank_slot entries are -1.  Rows at or past recv_rows are dropped (stats[2])
 * together with every entry they carry (stats[1]).  Then the surviving entries
 * are expanded locally: each gets the slot a plain dispatch of the surviving
 * ids would give, and its packed row is copied from its recv row. */
int oracle_dedup_dispatch(const void* x, int x_dt, int64_t T, int64_t H, const int32_t* idx,
                          int K, int E, int R, void* recv_x, int64_t recv_rows, int32_t* recv_cnt,
                          int32_t* recv_off, int32_t* recv_src, int32_t* rank_slot, int64_t cap,
                          int64_t packed_rows, void* packed, int32_t* packed_cnt,
                          int32_t* packed_off, int32_t* packed_src, int64_t* tok_map,
                          int32_t* stats) {
    int64_t N = T * K, n_invalid = 0, recv_dropped = 0, entry_dropped = 0;
    int er = E / R;
    uint8_t* keep = (uint8_t*)malloc((size_t)N + 1);
    int64_t* src_row = (int64_t*)malloc(((size_t)N + 1) * sizeof(int64_t));
    uint32_t* mask = (uint32_t*)calloc((size_t)T + 1, sizeof(uint32_t));
    int64_t* run = (int64_t*)calloc((size_t)R + 1, sizeof(int64_t));
    int64_t* tok_of_row = (int64_t*)malloc(((size_t)recv_rows + 1) * sizeof(int64_t));

    for (int64_t t = 0; t < T; ++t)
        for (int k = 0; k < K; ++k) {
            int32_t e = idx[t * K + k];
            if (e >= 0 && e < E)
                mask[t] |= 1u << (e / er);
            else if (e != -1)
                n_invalid += 1;
        }
    for (int r = 0; r < R; ++r)
        recv_cnt[r] = 0;
    for (int64_t t = 0; t < T; ++t)
        for (int r = 0; r < R; ++r)
            if (mask[t] & (1u << r))
                recv_cnt[r] += 1;
    recv_off[0] = 0;
    for (int r = 0; r < R; ++r)
        recv_off[r + 1] = recv_off[r] + recv_cnt[r];
    for (int64_t t = 0; t < T; ++t)
        for (int r = 0; r < R; ++r) {
            rank_slot[t * R + r] = -1;
            if (!(mask[t] & (1u << r)))
                continue;
            int64_t row = recv_off[r] + run[r]++;
            if (row >= recv_rows) {
                recv_dropped += 1;
                continue;
            }
            rank_slot[t * R + r] = (int32_t)row;
            recv_src[row] = (int32_t)t;
            tok_of_row[row] = t;
        }
    /* stage 1: one copy of x[t] per surviving (t, r) */
    {
        int64_t n_rows = recv_off[R] < recv_rows ? recv_off[R] : recv_rows;
        size_t eb = elem_bytes(x_dt);
        int64_t row;
#pragma omp parallel for schedule(dynamic, 16)
        for (row = 0; row < n_rows; ++row)
            memcpy((char*)recv_x + (size_t)row * H * eb,
                   (const char*)x + (size_t)tok_of_row[row] * H * eb, (size_t)H * eb);
    }
    /* stage 2: local expansion of each recv row to the token's experts */
    for (int64_t f = 0; f < N; ++f) {
        int32_t e = idx[f];
        keep[f] = 0;
        src_row[f] = -1;
        if (!(e >= 0 && e < E))
            continue;
        int32_t rs = rank_slot[(f / K) * R + e / er];
        if (rs < 0) {
            entry_dropped += 1;
            continue;
        }
        keep[f] = 1;
        src_row[f] = rs;
    }
    entry_dropped += assign_slots(idx, keep, T, K, E, cap, packed_rows, packed_cnt, packed_off,
                                  packed_src, tok_map);
    copy_rows(recv_x, x_dt, NULL, H, src_row, tok_map, N, packed, x_dt, NULL);
    if (stats) {
        stats[0] = (int32_t)n_invalid;
        stats[1] = (int32_t)entry_dropped;
        stats[2] = (int32_t)recv_dropped;
    }
    free(keep);
    free(src_row);
    free(mask);
    free(run);
    free(tok_of_row);
    return 0;
}

/* ------------------------------------------------------------------ */
/* dedup combine: per rank, then across ranks                           */
/* ------------------------------------------------------------------ */

/* For each recv row (t, r): partial = 0; for k ascending with a valid id on
 * rank r and 0 <= tok_map < y_rows: partial = partial + (w * y[row]).
 * Then out[t] = 0 + partial(r1) + partial(r2) + ... over the token's recv rows
 * in ascending rank order ([MoonEP#34] "Why it's worth doing": local reduce,
 * then the cross-rank combine; [mori#448] convert_combine_input then the sum
 * across destination ranks).  out_weights uses the same grouping.  partial
 * (f32 [recv_rows, H]) is written when non-NULL. */
int oracle_dedup_combine(const void* y, int y_dt, int64_t y_rows, int64_t H,
                         const int64_t* tok_map, const float* w, const int32_t* idx, int64_t T,
                         int K, int E, int R, const int32_t* rank_slot, int64_t recv_rows,
                         float* partial, void* out, int out_dt, float* out_weights) {
    int er = E / R;
    int64_t t;
#pragma omp parallel for schedule(dynamic, 4)
    for (t = 0; t < T; ++t) {
        float* acc = (float*)malloc((size_t)H * sizeof(float));
        float* p = (float*)malloc((size_t)H * sizeof(float));
        float ws = 0.0f;
        for (int64_t h = 0; h < H; ++h)
            acc[h] = 0.0f;
        for (int r = 0; r < R; ++r) {
            int32_t rs = rank_slot[t * R + r];
            if (rs < 0 || rs >= recv_rows)
                continue;
            float pw = 0.0f;
            for (int64_t h = 0; h < H; ++h)
                p[h] = 0.0f;
            for (int k = 0; k < K; ++k) {
                int32_t e = idx[t * K + k];
                if (!(e >= 0 && e < E) || e / er != r)
                    continue;
                int64_t row = tok_map[t * K + k];
                if (row < 0 || row >= y_rows)
                    continue;
                float wk = w[t * K + k];
                for (int64_t h = 0; h < H; ++h) {
                    float prod = wk * load_elem(y, y_dt, row * H + h);
                    p[h] = p[h] + prod;
                }
                pw = pw + wk;
            }
            if (partial)
                memcpy(partial + (size_t)rs * H, p, (size_t)H * sizeof(float));
            for (int64_t h = 0; h < H; ++h)
                acc[h] = acc[h] + p[h];
            ws = ws + pw;
        }
        for (int64_t h = 0; h < H; ++h) {
            if (out_dt == ORC_BF16)
                ((uint16_t*)out)[t * H + h] = f32_to_bf16(acc[h]);
            else
                ((float*)out)[t * H + h] = acc[h];
        }
        if (out_weights)
            out_weights[t] = ws;
        free(acc);
        free(p);
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* expert stand-ins and format helpers (tests and harness)              */
/* ------------------------------------------------------------------ */

/* y = bf16(f32(q) * s[block]), the dequantize step of the blockwise format. */
int oracle_fp8_dequant(const uint8_t* q, const float* scales, int64_t rows, int64_t H,
                       uint16_t* y) {
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r)
        for (int64_t h = 0; h < H; ++h) {
            float v = e4m3_to_f32(q[r * H + h]) * scales[r * (H / FP8_BLOCK) + h / FP8_BLOCK];
            y[r * H + h] = f32_to_bf16(v);
        }
    return 0;
}

/* Decode-workload expert: y[row] = bf16(c[e] * f32(x[row])) for every row of
 * expert e's segment [packed_off[e], packed_off[e] + packed_cnt[e]). */
int oracle_expert_scale(const uint16_t* packed, int64_t H, int E, const int32_t* packed_cnt,
                        const int32_t* packed_off, const float* c, uint16_t* y) {
    for (int e = 0; e < E; ++e)
        for (int64_t row = packed_off[e]; row < (int64_t)packed_off[e] + packed_cnt[e]; ++row)
            for (int64_t h = 0; h < H; ++h)
                y[row * H + h] = f32_to_bf16(c[e] * bf16_to_f32(packed[row * H + h]));
    return 0;
}

void oracle_e2m1_encode(const float* v, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i)
        out[i] = f32_to_e2m1(v[i]);
}

void oracle_e2m1_decode(const uint8_t* c, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i)
        out[i] = e2m1_to_f32(c[i] & 15);
}

void oracle_fp4_pack_rows(const uint16_t* x, int64_t rows, int64_t H, uint8_t* q, float* s) {
    for (int64_t r = 0; r < rows; ++r)
        fp4_pack_row(x + r * H, H, q + r * (H / 2), s + r * (H / FP8_BLOCK));
}

void oracle_bf16_encode(const float* v, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i)
        out[i] = f32_to_bf16(v[i]);
}

void oracle_e4m3_encode(const float* v, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i)
        out[i] = f32_to_e4m3(v[i]);
}

void oracle_e4m3_decode(const uint8_t* b, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i)
        out[i] = e4m3_to_f32(b[i]);
}

void oracle_fp8_pack_rows(const uint16_t* x, int64_t rows, int64_t H, uint8_t* q, float* s) {
    for (int64_t r = 0; r < rows; ++r)
        fp8_pack_row(x + r * H, H, q + r * H, s + r * (H / FP8_BLOCK));
}

/*
 * moe_route.h - C ABI of the MI355X (gfx950) MoE route-count / dispatch /
 * combine library (libmoe_route.so).
 *
 * The operations follow the standard-MoE conversion kernels described in
 * "Draft: cco + flydsl dispatch/combine" (ROCm/mori pull 448), reduced to one
 * GPU:
 *   - convert_dispatch_output (commit log, "Port mori/FlyDSL StdMoE ..."):
 *     repack each (token, k) into per-expert packed rows, recording
 *     packed_cnt, packed_src and an int64 tok_map with -1 as the sentinel;
 *   - convert_combine_input and the f32 gather (PR description; same commit):
 *     out[t] = sum_k w[t,k] * y[tok_map[t,k]] reduced in f32;
 *   - out_weights (commit "Combine now reduces the K forwarded per-token
 *     weight vectors into out_weights"): the sum of the valid weights;
 *   - Fp8BlockwiseQuant (commit "Port mori's Fp8BlockwiseQuant ..."): one f32
 *     scale per 128-element block, OCP e4m3 payload, dequantized inside the
 *     combine's reduction on the receiving side;
 *   - the fp4 e2m1 accumulator path (commit "Add the fp4 e2m1 accum path ..."):
 *     8 codes per 32-bit word, hidden/2 bytes per row;
 *   - replay dispatch and forwarded quant scales (commit "... routing handle,
 *     LEC, reset, replay"): a cached tok_map reused with the identical layout;
 *   - the dispatch dedup (PR description, "ballot dedup"; and "Drop
 *     cooperative launch from the CTA-independent local kernels", MoonEP pull
 *     34, "Why it's worth doing": one copy per dedup group, expanded locally,
 *     reduced locally and then across ranks).
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 * Pointers named x, y, packed_x, recv_x, out, idx, tok_map, ... are DEVICE
 * pointers.  Every buffer is allocated and freed by the caller; the library
 * allocates nothing, keeps no pointer to a caller's buffer after a call
 * returns and holds no state between calls, except the static workspace of
 * moe_dispatch_noalloc (one array per GPU, and its device address once looked
 * up) and the launch geometry, read once (moe_geometry).  Work is enqueued on `stream` (a hipStream_t passed as
 * void*, NULL = the default stream) and the call returns without waiting.
 * Results are deterministic: the same inputs give the same bits, and no
 * output needs clearing between calls.
 *
 * Layouts are row-major.  Expert ids are int32 [T,K]; id e is valid iff
 * 0 <= e < E; -1 means "no expert" and is skipped silently; any other value is
 * skipped and counted as invalid.  Row data: bf16 (uint16 bit patterns) or
 * f32, H elements per row; packed fp8 rows hold H OCP e4m3fn bytes and packed
 * fp4 rows H/2 bytes of OCP e2m1 codes (element 2i in the low nibble of byte
 * i), each with one f32 scale per 128-element block in a separate
 * [rows, H/128] array.
 *
 * Slots.  Within an expert, entries take consecutive slots in flat order
 * f = t*K + k.  With cap > 0 (padded layout) expert e owns rows
 * [e*cap, e*cap + cap); with cap == 0 (compact layout) expert e starts at
 * off[e], the exclusive scan of the counts (initial value 0).  An entry whose
 * slot is >= cap, or whose row is >= packed_rows, is dropped: tok_map = -1.
 * Rows that no entry owns are never written (nor is their packed_src).
 *
 * stats (int32[3], may be NULL): [0] ids outside [0,E) other than -1;
 * [1] valid entries that got no packed row (dropped); [2] dedup recv rows
 * dropped because they did not fit in recv_rows (0 for the plain calls).
 *
 * Errors.  Every argument is checked on the host before anything is
 * enqueued; a call that returns an error has enqueued nothing and changed no
 * buffer.  Data-dependent conditions (bad ids, full capacity, tok_map or
 * rank_slot values outside the row range) never fault: they are skipped and
 * counted as stated.  moe_last_error() gives the text of the calling thread's
 * last error.
 *
 * Limits: 0 <= T, 1 <= K <= 16, 1 <= E <= 1024, T*K < 2^31, H > 0 with
 * H % 8 == 0 (H % 128 == 0 for fp8 and fp4), packed_rows, recv_rows and y_rows <= 2^31-1,
 * row pointers 16-byte aligned, 1 <= R <= 32 with E % R == 0.
 */
#ifndef MOE_ROUTE_H
#define MOE_ROUTE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The two range markers make every int a value of the type (in C++ too, where
 * an enum holds only the values its enumerators span): a caller may pass any
 * code, and an unknown one is rejected with MOE_ERR_INVALID_ARG. */
typedef enum {
    MOE_BF16 = 0,
    MOE_F32 = 1,
    MOE_FP8_E4M3 = 2,
    MOE_FP4_E2M1 = 3,
    MOE_DTYPE_RANGE_MIN_ = -2147483647 - 1,
    MOE_DTYPE_RANGE_MAX_ = 2147483647
} moe_dtype;

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1, /* a pointer, size, dtype or alignment is wrong   */
    MOE_ERR_UNSUPPORTED = -2, /* a valid but unimplemented dtype combination    */
    MOE_ERR_WORKSPACE = -3,   /* ws is NULL or smaller than moe_workspace_size  */
    MOE_ERR_HIP = -4          /* the HIP runtime refused a launch               */
} moe_status;

/* Library version, (major << 16) | minor. */
int moe_version(void);

/* Text of the calling thread's last non-OK status ("" if none). */
const char* moe_last_error(void);

/* The launch geometry in use, as "key=value,..." (a tuning aid for benchmark
 * runs, not part of any result): workgroups per row of each row mover, lane
 * units per combine workgroup, and the per-CU residency caps.  Defaults are the
 * shapes measured fastest on MI355X; the environment variable MOE_GEOM, read
 * once before the first launch, overrides them with pairs in the same form
 * (e.g. "combine_chunk_units=224,combine_wgs_per_cu=4").  An unknown key, a
 * malformed pair or a value outside the key's range is ignored and listed after
 * "; ignored: ".  Results are the same bits under every accepted geometry.
 * The string is owned by the library and lives until the process ends. */
const char* moe_geometry(void);

/* Bytes of device workspace that moe_route_count, moe_dispatch,
 * moe_dispatch_prequant and (with R > 0) moe_dedup_dispatch need for these
 * sizes (moe_dispatch_replay and the combines need none).  The workspace needs no
 * initialisation and may be reused by consecutive calls on one stream, also
 * from a captured graph.  Calls that may run at the same time (other streams)
 * need workspaces of their own: the routing keeps an arrival counter in it,
 * which every completed call leaves re-armed.  After a call that did not run to
 * completion (a device error), clear the workspace before using it again. */
size_t moe_workspace_size(int64_t T, int K, int E, int R);

/* Routing histogram and exclusive scan ("cco + flydsl dispatch/combine",
 * commit log: local_expert_count; the exclusive-scan convention with initial
 * value 0 as in "Add standalone cuda.coop.cutlass package").
 *   idx   int32 [T,K]    expert ids
 *   cnt   int32 [E]      out: valid entries per expert
 *   off   int32 [E+1]    out: off[0] = 0, off[e+1] = off[e] + cnt[e]
 *   stats int32 [3]      out, may be NULL */
int moe_route_count(const int32_t* idx, int64_t T, int K, int E, int32_t* cnt, int32_t* off,
                    int32_t* stats, void* ws, size_t ws_bytes, void* stream);

/* Dispatch: count, scan, assign slots and scatter rows into per-expert packed
 * buffers (convert_dispatch_output), optionally packing bf16 to blockwise fp8.
 *   x            [T,H] x_dt (MOE_BF16 or MOE_F32; fp8 input goes through
 *                moe_dispatch_prequant, which also takes its scales)
 *   cap          > 0: padded layout, rows [e*cap, e*cap+cap); 0: compact layout
 *   packed_rows  rows of packed_x (and packed_src, packed_scales)
 *   packed_x     out [packed_rows,H] packed_dt: x_dt, or MOE_FP8_E4M3 / MOE_FP4_E2M1
 *                from MOE_BF16 (fp4: [packed_rows,H/2] bytes, two codes per byte,
 *                element 2i in the low nibble)
 *   packed_scales out f32 [packed_rows,H/128] iff packed_dt is fp8 or fp4, else NULL.
 *                Per block, with M = 448 (e4m3) or 6 (e2m1): amax = max|x| over
 *                the block's finite values; amax > M gives s = amax/M and
 *                q = enc(x*M/amax), the correctly rounded f32 quotient (no
 *                overflow of x*M); otherwise s = 1 and q = enc(x); enc rounds
 *                to nearest even and saturates (+-inf give +-M, the clamp
 *                before conversion of the pages' fp8 quantizer); a NaN gets the
 *                e4m3 NaN code with its sign; e2m1 has no NaN code, so a block
 *                holding a NaN gets zero codes and the NaN scale 0x7FC00000
 *                (the fp4 rule is the fp8 rule carried to the e2m1 maximum).
 *   packed_cnt   out int32 [E]   rows written per expert
 *   packed_off   out int32 [E+1] first row of each expert's segment,
 *                min(e*cap or off[e], packed_rows); may be NULL
 *   packed_src   out int32 [packed_rows] source token of each written row
 *   tok_map      out int64 [T,K] packed row of entry (t,k), or -1 */
int moe_dispatch(const void* x, moe_dtype x_dt, int64_t T, int64_t H, const int32_t* idx, int K,
                 int E, int64_t cap, int64_t packed_rows, void* packed_x, moe_dtype packed_dt,
                 float* packed_scales, int32_t* packed_cnt, int32_t* packed_off,
                 int32_t* packed_src, int64_t* tok_map, int32_t* stats, void* ws, size_t ws_bytes,
                 void* stream);

/* moe_dispatch for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same arguments, results, checks and errors, without the workspace.  The
 * routing workspace is a static device array of the library, 4 MiB on each
 * GPU the library runs on, held from the first call on that GPU until the
 * process ends; its device address is looked up once per GPU (that first call
 * may briefly make the stream's GPU current).  The call allocates nothing.
 * Limit: moe_workspace_size(T, K, E, 0) <= 4 MiB (T*K up to 837120 entries at
 * E = 256, 523136 at E = 1024); larger sizes return MOE_ERR_WORKSPACE before
 * anything is enqueued.  Every moe_dispatch_noalloc call on one GPU shares the
 * array: calls that may overlap on the device (different streams) race and must
 * be ordered by the caller; calls on one stream are ordered by it, also when
 * several host threads make them (each call's launches are enqueued as one
 * unit, under a lock held only while enqueueing). */
int moe_dispatch_noalloc(const void* x, moe_dtype x_dt, int64_t T, int64_t H, const int32_t* idx,
                         int K, int E, int64_t cap, int64_t packed_rows, void* packed_x,
                         moe_dtype packed_dt, float* packed_scales, int32_t* packed_cnt,
                         int32_t* packed_off, int32_t* packed_src, int64_t* tok_map,
                         int32_t* stats, void* stream);

/* Dispatch of pre-quantized input (the dispatch of "Draft: cco + flydsl
 * dispatch/combine", commit "... routing handle, LEC, reset, replay", forwards
 * the per-token quant scales with the payload): x_q holds e4m3fn codes and
 * x_scales one f32 scale per 128-element block of each token; every packed row
 * of token t receives x_q[t] byte for byte and its scale row receives
 * x_scales[t] unchanged.  The routing outputs (tok_map, packed_*, stats) are
 * those of moe_dispatch on the same ids.
 *   x_q       uint8 [T,H], 16-byte aligned; H % 128 == 0
 *   x_scales  f32 [T,H/128]
 *   packed_x  uint8 [packed_rows,H]; packed_scales f32 [packed_rows,H/128]
 *   the other arguments, limits and errors as for moe_dispatch. */
int moe_dispatch_prequant(const uint8_t* x_q, const float* x_scales, int64_t T, int64_t H,
                          const int32_t* idx, int K, int E, int64_t cap, int64_t packed_rows,
                          uint8_t* packed_x, float* packed_scales, int32_t* packed_cnt,
                          int32_t* packed_off, int32_t* packed_src, int64_t* tok_map,
                          int32_t* stats, void* ws, size_t ws_bytes, void* stream);

/* Replay dispatch (same page and commit: the replay reuses the cached tok_map
 * with the identical layout): no counting, scan or slotting; for every entry
 * with 0 <= tok_map[t,k] < packed_rows, row tok_map[t,k] of packed_x receives
 * token t exactly as moe_dispatch (bf16/f32 bit copy, bf16 -> fp8 or fp4 pack) or
 * moe_dispatch_prequant (fp8 codes plus the scale row) would write it.
 * Nothing else is written: packed_src, packed_cnt and the routing stay as the
 * earlier dispatch left them.  tok_map must hold each row at most once (any
 * dispatch's tok_map does); rows named twice get one of the writers.
 *   x, x_dt, x_scales   payload as for moe_dispatch / moe_dispatch_prequant
 *                       (x_scales only with x_dt == MOE_FP8_E4M3)
 *   tok_map int64 [T,K], 8-byte aligned; K in [1,16]; T*K < 2^31
 *   packed_x, packed_dt, packed_scales as for moe_dispatch.
 * Errors: MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED as for moe_dispatch; a
 * failing call enqueues nothing.  Needs no workspace. */
int moe_dispatch_replay(const void* x, moe_dtype x_dt, const float* x_scales, int64_t T, int64_t H,
                        const int64_t* tok_map, int K, int64_t packed_rows, void* packed_x,
                        moe_dtype packed_dt, float* packed_scales, void* stream);

/* Dedup description for moe_combine: the routing outputs of moe_dedup_dispatch.
 *   idx        int32 [T,K] the ids the dispatch was given (for e / (E/R))
 *   rank_slot  int32 [T,R] recv row of (t, r) or -1
 *   recv_rows  rows of the recv buffer (bound for rank_slot)
 *   partial    f32 [recv_rows,H] or NULL.  Non-NULL: the per-rank partial sums
 *              are written there by one kernel and summed across ranks by a
 *              second one (the two-stage form of a multi-rank combine).  NULL:
 *              one kernel keeps the partials in registers.  The result is the
 *              same bits either way. */
typedef struct moe_dedup_plan {
    int R;
    const int32_t* idx;
    const int32_t* rank_slot;
    int64_t recv_rows;
    float* partial;
} moe_dedup_plan;

/* Combine: weighted gather-reduce back to token order (convert_combine_input
 * and the f32 gather), plus out_weights.
 *   y            [y_rows,H] y_dt (MOE_BF16 or MOE_F32), the expert outputs in
 *                packed-row order (fp8 / fp4 outputs: moe_combine_fp8 /
 *                moe_combine_fp4; y_dt MOE_FP8_E4M3 here is MOE_ERR_UNSUPPORTED)
 *   tok_map      int64 [T,K] from the dispatch; rows outside [0,y_rows) are skipped
 *   w            f32 [T,K] gate weights
 *   dd           NULL: acc = 0, then for k ascending acc = acc + (w * y[row]),
 *                each product and sum rounded to f32 (no fused multiply-add).
 *                Non-NULL: the same sum restricted to each virtual rank's
 *                entries gives one partial per recv row, and
 *                out = 0 + partials in ascending rank order.
 *   out          out [T,H] out_dt (MOE_BF16, rounded to nearest even, or MOE_F32)
 *   out_weights  out f32 [T], the sum of the contributing weights in the same
 *                order and grouping; may be NULL
 *   E            expert count (used with dd only; pass E anyway) */
int moe_combine(const void* y, moe_dtype y_dt, int64_t y_rows, int64_t H, const int64_t* tok_map,
                const float* w, int64_t T, int K, int E, const moe_dedup_plan* dd, void* out,
                moe_dtype out_dt, float* out_weights, void* stream);

/* Dedup dispatch over R virtual ranks of E/R experts each: one row copy per
 * unique (token, rank), then local expansion to the token's experts.
 * Rank of expert e: e / (E/R), taken only for valid e (so -1 never maps to rank 0).
 *   recv_x     out [recv_rows,H] x_dt; row recv_off[r] + j holds the j-th token
 *              (in token order) whose mask contains r
 *   recv_cnt   out int32 [R], recv_off out int32 [R+1] (exclusive scan)
 *   recv_src   out int32 [recv_rows] token of each written recv row
 *   rank_slot  out int32 [T,R] recv row of (t, r), -1 if r is not in the mask
 *              or the row did not fit in recv_rows (then every entry it carries
 *              is dropped)
 *   cap, packed_rows, packed_x (x_dt), packed_cnt, packed_off, packed_src,
 *   tok_map    as in moe_dispatch over the surviving entries; each packed row
 *              is copied from its recv row.  With no recv drop these equal the
 *              outputs of moe_dispatch on the same ids. */
int moe_dedup_dispatch(const void* x, moe_dtype x_dt, int64_t T, int64_t H, const int32_t* idx,
                       int K, int E, int R, void* recv_x, int64_t recv_rows, int32_t* recv_cnt,
                       int32_t* recv_off, int32_t* recv_src, int32_t* rank_slot, int64_t cap,
                       int64_t packed_rows, void* packed_x, int32_t* packed_cnt,
                       int32_t* packed_off, int32_t* packed_src, int64_t* tok_map,
                       int32_t* stats, void* ws, size_t ws_bytes, void* stream);

/* Combine of fp8 expert outputs ("Draft: cco + flydsl dispatch/combine",
 * commit "Port mori's Fp8BlockwiseQuant ...": the receiving side dequantizes
 * fp8 times the block scale and accumulates; commit "... make_combine_scatter
 * ...": the direct-cast variant without scales).  For t, and k ascending with
 * 0 <= tok_map[t,k] < y_rows:
 *   v   = f32(e4m3(q[row][h])) * scales[row][h/128]    (scale 1 if scales NULL;
 *         one rounded f32 multiply, no bf16 step)
 *   acc = acc + w[t,k] * v                             (each op rounded, no FMA)
 *   out[t] = acc as bf16 (nearest even) or f32; out_weights[t] = sum of those w.
 *   q        uint8 [y_rows,H] e4m3fn codes, 16-byte aligned; H % 128 == 0
 *   scales   f32 [y_rows,H/128], or NULL for the direct cast
 *   tok_map, w, T, K, out, out_dt, out_weights as for moe_combine.
 * With scales NULL (or all 1) the result equals moe_combine on the bf16
 * decoding of q.  Errors: MOE_ERR_INVALID_ARG for the checks of moe_combine
 * and H % 128 != 0; enqueues nothing on error.  The dedup plan is not taken. */
int moe_combine_fp8(const uint8_t* q, const float* scales, int64_t y_rows, int64_t H,
                    const int64_t* tok_map, const float* w, int64_t T, int K, void* out,
                    moe_dtype out_dt, float* out_weights, void* stream);

/* Combine of fp4 expert outputs ("Draft: cco + flydsl dispatch/combine",
 * commit adding the fp4 e2m1 accum path: 8 packed codes per i32, expanded to
 * f32 with the gfx950 scaled conversions): as moe_combine_fp8 with q holding
 * e2m1 codes, [y_rows,H/2] bytes, element 2i in the low nibble of byte i;
 * v = f32(e2m1(q)) * scales[row][h/128] (1 if scales NULL). */
int moe_combine_fp4(const uint8_t* q, const float* scales, int64_t y_rows, int64_t H,
                    const int64_t* tok_map, const float* w, int64_t T, int K, void* out,
                    moe_dtype out_dt, float* out_weights, void* stream);

/* Blockwise fp8 dequantize (the inverse step of Fp8BlockwiseQuant):
 * y = bf16(f32(q) * scales[row][h/128]), rounded to nearest even.
 *   q  uint8 [rows,H], scales f32 [rows,H/128], y out bf16 [rows,H]; H % 128 == 0. */
int moe_fp8_dequant(const uint8_t* q, const float* scales, int64_t rows, int64_t H, void* y,
                    void* stream);

/* Plain device copy with 16-byte streaming loads and stores: the copy ceiling
 * the row movers are compared with (a measurement helper, not on the path).
 *   src, dst  device, 16-byte aligned, not overlapping; bytes % 16 == 0. */
int moe_copy16(const void* src, void* dst, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUTE_H */

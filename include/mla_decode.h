/*
 * mla_decode.h -- C ABI of the MI355X (gfx950) single-token MLA decode library.
 *
 * The operation (amd-mixed-mla pages; submission 593653, "Slow fallback"
 * `_bmm_reference`, and its module constants): for every sequence b and each
 * of the 16 query heads h,
 *
 *     s_j      = sm_scale * sum_{d<576} q[b,h,d] * x_j[d]
 *     out[b,h] = sum_j softmax_j(s) * x_j[0:512]
 *     lse[b,h] = log(sum_j exp(s_j))                  (natural log)
 *
 * where x_j = dequant(kv[kv_indices[kv_indptr[b] + j]]) for
 * j < kv_indptr[b+1] - kv_indptr[b]. One latent KV head is shared by all 16
 * query heads; the score dimension is 576 (512 no-RoPE + 64 RoPE) and V is
 * the first 512 columns of the same cache row; one query token per sequence;
 * page size 1. Dequantisation of the cache formats:
 *   - bf16: the value itself.
 *   - fp8 e4m3fn with one per-tensor fp32 scale: code value * scale
 *     (submission 754939, `quantize_fp8`).
 *   - MXFP4: e2m1 nibble value * 2^(e8m0 - 127), one e8m0 scale per 32
 *     consecutive elements, even element in the low nibble (submission
 *     754939, `_dq4` and the V loop of `mla_s1`).
 *
 * Conventions for every entry point:
 *   - Device pointers are caller-owned device memory; the library never
 *     allocates, frees or synchronises. Work is enqueued on `stream` (a
 *     hipStream_t passed as void*, NULL = the null stream); returning means
 *     "launched". Calls that share a workspace must be ordered on one stream.
 *   - Errors are returned as negative status codes (no exceptions, nothing
 *     printed). Arguments are validated on the host before any launch; on an
 *     error nothing is launched and the outputs are untouched.
 *   - Thread-safe and reentrant: no per-call global state.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Fixed shape of the operation. */
#define MLA_NUM_HEADS 16
#define MLA_QK_DIM 576
#define MLA_V_DIM 512
#define MLA_ROPE_DIM 64
#define MLA_MX_BLOCK 32
#define MLA_MX_SCALES_PER_ROW 18 /* 576 / 32 */

/* KV cache formats. */
#define MLA_KV_BF16 0     /* kv: bf16 [rows, 576]; kv_scales: NULL                   */
#define MLA_KV_FP8_E4M3 1 /* kv: uint8 e4m3fn [rows, 576]; kv_scales: device fp32 [1] */
#define MLA_KV_MXFP4 2    /* kv: uint8 [rows, 288] (2 e2m1 per byte, even element in the
                             low nibble); kv_scales: device uint8 e8m0 [rows, 18]       */

/* Status codes. */
#define MLA_OK 0
#define MLA_ERR_INVALID_ARG (-1)       /* null required pointer, negative size, bad format,
                                          misaligned pointer, total_kv out of range */
#define MLA_ERR_UNSUPPORTED (-2)       /* current device is not gfx950 */
#define MLA_ERR_WORKSPACE_TOO_SMALL (-3)
#define MLA_ERR_HIP (-4)               /* a HIP runtime call or kernel launch failed */

/* Flags (bit field). Zero selects the built-in heuristic. */
#define MLA_FLAG_FORCE_SPLIT 0x1       /* split-K grid: (splits x batch) workgroups      */
#define MLA_FLAG_FORCE_PERSISTENT 0x2  /* fixed grid, equal token shares over all batches */
#define MLA_FLAG_MIXED_LENGTHS 0x4     /* hint: sequence lengths differ widely; the heuristic then
                                          picks the persistent grid (ignored by paged and
                                          several-query-token calls, which are split-K)   */
#define MLA_FLAG_COMBINE_LAUNCH 0x8    /* split-K: merge the split partials in a separate
                                          combine launch instead of in the last-arriving
                                          split workgroup of each sequence               */
#define MLA_FLAG_ROW_PER_WG 0x10       /* several-query-token calls: one query row per
                                          workgroup even where the plan would carry two
                                          (bf16 cache, uniform query count); ignored by the
                                          single-token calls                             */
#define MLA_FLAG_SPLITS_SHIFT 8        /* bits 8..15: split count for split-K (1..255)   */
#define MLA_FLAG_GRID_SHIFT 16         /* bits 16..27: workgroups for persistent (1..4095)*/

/*
 * Workspace layout. When a plan has split partials (workspace_bytes > 0), the
 * first MLA_WORKSPACE_COUNTER_BYTES bytes of the workspace hold one 32-bit
 * arrival counter per query row, used by plans with combine = 2 (split-K with
 * 2 to 4 splits, or on the bf16 and fp8 caches 5 to 8 splits, over at most
 * 16384 query rows, unless MLA_FLAG_COMBINE_LAUNCH is set): each split
 * workgroup counts itself in after writing its partial (5 to 8 splits: in
 * bf16, so that the merge loads them all at once),
 * and the one that arrives last merges the row's partials (the log-sum-exp
 * merge of flash-decoding split partials; submission 593653,
 * `_flash_fp8_split_s2`) and sets the counter back to zero.
 * That region must be all zero when a call starts: zero the workspace (at
 * least its first MLA_WORKSPACE_COUNTER_BYTES bytes) once after allocating
 * it. Every call leaves the region all zero again, whatever its plan, so a
 * workspace can be reused across calls and plans without clearing it. Write
 * nothing else into that region. The partials follow it; their contents
 * need no initialisation.
 */
#define MLA_WORKSPACE_COUNTER_BYTES 65536

/* The launch plan the library would use (host-only, deterministic). */
typedef struct mla_plan_info {
    int mode;               /* 0 = split-K, 1 = persistent                              */
    int num_splits;         /* split-K: splits per sequence; persistent: 0              */
    int grid;               /* stage-1 workgroups                                       */
    int num_partials;       /* partial (output, lse) slots held in the workspace        */
    int combine;            /* how the split partials are merged: 0 none (one split),
                               1 a combine launch after stage 1, 2 inside stage 1 by
                               the last-arriving split workgroup of each sequence  */
    int rows_per_wg;        /* query rows each stage-1 workgroup carries: 1, or 2 for
                               mla_decode_mtp on the bf16 cache with a uniform query
                               count of at least 2 (the workgroup gathers the cache
                               once for both rows)                                  */
    size_t workspace_bytes; /* bytes of workspace this plan needs (0 when none)          */
} mla_plan_info;

/*
 * mla_decode_plan: fill `plan` with the launch plan for a call with these
 * sizes. Pure host function (no device query, no HIP call).
 *   batch     number of sequences (>= 0)
 *   total_kv  kv_indptr[batch], host copy (0 <= total_kv <= INT32_MAX)
 *   kv_dtype  MLA_KV_*
 *   flags     MLA_FLAG_* (0 = heuristic)
 * Returns MLA_OK or MLA_ERR_INVALID_ARG.
 * The split count / grid heuristic is this library's own occupancy rule for
 * 256 compute units; the pages' per-shape tables (e.g. submission 754939
 * NSPLITS_SMALL / _MED / _LARGE, submission 703488's 256-program grids) were
 * the prior art for it.
 */
int mla_decode_plan(int batch, int64_t total_kv, int kv_dtype, int flags, mla_plan_info* plan);

/*
 * mla_decode_workspace_size: bytes of device workspace `mla_decode` needs for
 * these sizes (arrival counters and split partials, laid out as described
 * above mla_plan_info). 0 means no workspace is needed. Pure host
 * function. Returns 0 as well for invalid arguments (mla_decode reports them).
 */
size_t mla_decode_workspace_size(int batch, int64_t total_kv, int kv_dtype, int flags);

/*
 * mla_decode: the decode attention defined at the top of this file.
 *   q          device bf16 [batch, 16, 576], contiguous, 16-byte aligned
 *   kv         device cache rows (layout per kv_dtype above), 16-byte aligned;
 *              every kv_indices value must be a valid row (not checked)
 *   kv_scales  per kv_dtype above (device pointer; NULL for bf16)
 *   kv_indptr  device int32 [batch + 1], non-decreasing, kv_indptr[0] = 0,
 *              kv_indptr[batch] = total_kv
 *   kv_indices device int32 [total_kv]: physical row of each logical token
 *              (may be NULL when total_kv = 0)
 *   out        device bf16 [batch, 16, 512], 16-byte aligned (written with RNE)
 *   lse        device fp32 [batch, 16] or NULL to skip; natural-log
 *              log-sum-exp of the scaled scores
 *   batch      number of sequences; 0 is a no-op
 *   total_kv   host copy of kv_indptr[batch] (no device read / sync needed)
 *   kv_dtype   MLA_KV_*
 *   sm_scale   softmax scale; <= 0 (or NaN) selects 1/sqrt(576)
 *   workspace  device scratch of at least mla_decode_workspace_size(...) bytes,
 *              16-byte aligned (NULL allowed when that size is 0); its first
 *              MLA_WORKSPACE_COUNTER_BYTES bytes must be zero (zeroed once
 *              after allocation; every call leaves them zero), the rest need
 *              no initialisation and is clobbered
 *   flags      MLA_FLAG_* (0 = heuristic)
 *   stream     hipStream_t as void*
 * An empty sequence (kv_indptr[b+1] == kv_indptr[b]) yields out = 0 and
 * lse = -inf. Results are deterministic: identical inputs and plan give
 * bitwise-identical outputs.
 * Returns MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED,
 * MLA_ERR_WORKSPACE_TOO_SMALL or MLA_ERR_HIP.
 */
int mla_decode(const void* q, const void* kv, const void* kv_scales, const int32_t* kv_indptr,
               const int32_t* kv_indices, void* out, float* lse, int batch, int64_t total_kv,
               int kv_dtype, float sm_scale, void* workspace, size_t workspace_bytes, int flags,
               void* stream);

/*
 * mla_decode_noalloc: mla_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). It takes no workspace: the arrival counters and split
 * partials of its plan live in a fixed device array inside the library,
 * MLA_NOALLOC_SCRATCH_BYTES bytes per device, which each device holds from its
 * first such call until the process ends. The call itself allocates and frees
 * nothing. The first call on a device looks the array up and enqueues one small
 * fill kernel that zeroes its counter region.
 *   arguments, outputs, results and errors as for mla_decode (without
 *   workspace / workspace_bytes); additionally MLA_ERR_WORKSPACE_TOO_SMALL when
 *   the plan's workspace (mla_decode_workspace_size) exceeds
 *   MLA_NOALLOC_SCRATCH_BYTES, checked on the host before any device call.
 * Every call on one device shares that device's array and leaves the last
 * call's partials in it (its counters zero): calls that may overlap on one
 * device -- two streams, or two host threads -- race and must be ordered by the
 * caller (one stream, or events).
 */
#define MLA_NOALLOC_SCRATCH_BYTES (32u << 20) /* 32 MiB: 64 KiB of counters and up to 1020 partial slots */
int mla_decode_noalloc(const void* q, const void* kv, const void* kv_scales, const int32_t* kv_indptr,
                       const int32_t* kv_indices, void* out, float* lse, int batch, int64_t total_kv, int kv_dtype,
                       float sm_scale, int flags, void* stream);

/*
 * mla_decode_rows: mla_decode with the number of rows the cache buffer holds
 * (for callers that can allocate their cache contiguously per sequence, as
 * the pages' benchmark does with kv_indices = arange; submission 593653,
 * `custom_kernel`).
 *   kv_rows  rows in kv (and in kv_scales for MXFP4); every kv_indices value
 *            must be below it. 0 = unknown, which is exactly mla_decode.
 *   all other arguments, the outputs, the errors and the results as for
 *   mla_decode; MLA_ERR_INVALID_ARG also for kv_rows < 0.
 * With kv_rows known, each stage-1 workgroup requests the first rows of its
 * token range as a contiguous cache would place them (entry t of kv_indices
 * in row t, clamped below kv_rows) together with its query and kv_indices
 * reads, before kv_indices has arrived: on split-K plans when every sequence
 * has the same length (total_kv a multiple of batch, so the range is known
 * before kv_indptr too), on the persistent grid always. It keeps them only when
 * kv_indices names exactly those rows and gathers again otherwise, so the
 * result does not depend on the cache layout; a contiguous cache saves one
 * dependent memory round trip at start-up. The bf16 and fp8 caches do this;
 * on the MXFP4 cache mla_decode_rows is mla_decode (its query split overlaps
 * the first row requests instead).
 */
int mla_decode_rows(const void* q, const void* kv, const void* kv_scales, const int32_t* kv_indptr,
                    const int32_t* kv_indices, void* out, float* lse, int batch, int64_t total_kv, int64_t kv_rows,
                    int kv_dtype, float sm_scale, void* workspace, size_t workspace_bytes, int flags, void* stream);

/*
 * mla_decode_paged: mla_decode over a paged cache (page_size rows per page),
 * the layout the pages' a16w8 path uses with 8-row pages for kv >= 8192
 * (submission 616673, `_run_a16w8`: the fp8 cache viewed as
 * [num_pages, page_size, 1, 576], page indptr = token indptr / page_size,
 * kv_last_page_lens; the paged kv_indptr / kv_indices / kv_last_page_len
 * convention of `mla_decode_fwd` in submission 593653).
 *   kv                cache rows grouped in pages: page p is rows
 *                     p * page_size .. p * page_size + page_size - 1
 *   kv_indptr         device int32 [batch + 1] into kv_indices (pages)
 *   kv_indices        device int32 page ids; sequence b uses pages
 *                     kv_indices[kv_indptr[b] .. kv_indptr[b+1] - 1] in order
 *   kv_last_page_len  device int32 [batch]: tokens in the last page of each
 *                     non-empty sequence (1..page_size); ignored when
 *                     page_size = 1 (may be NULL then)
 *   page_size         1..65536; 1 gives exactly mla_decode
 *   total_kv          host copy of the total number of tokens over the batch
 *                     (sum of (pages_b - 1) * page_size + kv_last_page_len[b])
 * Token j of sequence b is row kv_indices[kv_indptr[b] + j / page_size] *
 * page_size + j % page_size; all other arguments, the outputs and the
 * workspace are as for mla_decode. With page_size > 1 the plan is always
 * split-K (size the workspace with MLA_FLAG_FORCE_SPLIT set) and
 * MLA_FLAG_FORCE_PERSISTENT is rejected with MLA_ERR_INVALID_ARG.
 * Returns as mla_decode; MLA_ERR_INVALID_ARG also for page_size out of range
 * or a NULL / misaligned kv_last_page_len when page_size > 1.
 */
int mla_decode_paged(const void* q, const void* kv, const void* kv_scales, const int32_t* kv_indptr,
                     const int32_t* kv_indices, const int32_t* kv_last_page_len, int page_size, void* out,
                     float* lse, int batch, int64_t total_kv, int kv_dtype, float sm_scale, void* workspace,
                     size_t workspace_bytes, int flags, void* stream);

/* Query scale modes of mla_decode_q8. */
#define MLA_Q_SCALE_STATIC 0  /* *q_scale is read: the caller's per-tensor scale (finite, > 0) */
#define MLA_Q_SCALE_DYNAMIC 1 /* *q_scale is written: max(max |q|, 1e-12) / 448 over the query */

/*
 * mla_decode_q8: the decode attention with an fp8 query (the a8w8 path of
 * submission 593653: `_quantize_q_static_into` / `_quantize_q_dynamic_into`
 * before the attention; submission 754939, `quantize_fp8`). The bf16 query
 * is quantised with one per-tensor fp32 scale,
 *     code[b,h,d] = e4m3fn(clamp(q[b,h,d] / scale, -448, 448))
 * (IEEE binary32 division, round to nearest even), and the attention defined
 * at the top of this file runs with the decoded query code * scale in place
 * of q. The quantisation runs inside the attention kernels; the dynamic scale
 * adds one small reduction launch before them.
 *   q             device bf16 [batch, 16, 576] (as mla_decode)
 *   q_scale       device fp32 [1], 4-byte aligned: read (static) or written
 *                 (dynamic, before the call's kernels finish)
 *   q_scale_mode  MLA_Q_SCALE_STATIC or MLA_Q_SCALE_DYNAMIC
 *   kv .. page_size, out, lse, batch, total_kv, kv_dtype, sm_scale, flags,
 *   stream        as mla_decode_paged (page_size 1 is the layout of
 *                 mla_decode; kv_last_page_len may then be NULL)
 *   workspace     at least mla_decode_q8_workspace_size(...) bytes, 16-byte
 *                 aligned (NULL allowed when that size is 0)
 * Returns as mla_decode_paged; MLA_ERR_INVALID_ARG also for a bad
 * q_scale_mode or a NULL / misaligned q_scale.
 */
int mla_decode_q8(const void* q, float* q_scale, int q_scale_mode, const void* kv, const void* kv_scales,
                  const int32_t* kv_indptr, const int32_t* kv_indices, const int32_t* kv_last_page_len,
                  int page_size, void* out, float* lse, int batch, int64_t total_kv, int kv_dtype, float sm_scale,
                  void* workspace, size_t workspace_bytes, int flags, void* stream);

/*
 * mla_decode_q8_workspace_size: bytes of workspace mla_decode_q8 needs: the
 * split partials of mla_decode_workspace_size(batch, total_kv, kv_dtype,
 * flags), plus, for the dynamic scale, 1 KiB of partial maxima placed after
 * them and never inside the first MLA_WORKSPACE_COUNTER_BYTES bytes (so a
 * dynamic-scale call whose plan has no split partials still needs
 * MLA_WORKSPACE_COUNTER_BYTES + 1 KiB, and leaves the counter region zero).
 * For a paged call (page_size > 1) pass flags with MLA_FLAG_FORCE_SPLIT set.
 * Returns 0 for invalid arguments (mla_decode_q8 reports them).
 */
size_t mla_decode_q8_workspace_size(int batch, int64_t total_kv, int kv_dtype, int flags, int q_scale_mode);

/*
 * mla_quantize_q8_debug: the query quantisation of mla_decode_q8 on its own,
 * through the same scale reduction and code routine (test aid for the
 * bit-exact code check).
 *   q          device bf16 [batch, 16, 576], 16-byte aligned
 *   q_scale    device fp32 [1]: read (static) or written (dynamic)
 *   codes      device uint8 [batch, 16, 576], 8-byte aligned: the e4m3fn codes
 *   workspace  dynamic mode: at least 1 KiB, 16-byte aligned, whose first
 *              1 KiB is overwritten (so not a decode workspace, whose counter
 *              region must stay zero); else unused
 * Returns MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_WORKSPACE_TOO_SMALL,
 * MLA_ERR_UNSUPPORTED or MLA_ERR_HIP.
 */
int mla_quantize_q8_debug(const void* q, int batch, float* q_scale, int q_scale_mode, uint8_t* codes,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_decode_mtp: the decode attention with several query tokens per sequence
 * (multi-token prediction / speculative decoding; the pages' `qo_indptr` with
 * `max_seqlen_qo` / `uni_seqlen_qo`, submission 593653 `_aiter_persistent`).
 * Query row r (of total_q) belongs to sequence b with
 * qo_indptr[b] <= r < qo_indptr[b+1] and is token t = r - qo_indptr[b] of
 * that sequence's n query tokens. It attends
 *   causal = 0: every cache token of sequence b;
 *   causal = 1: the first L_b - n + 1 + t cache tokens (the query tokens are
 *               the sequence's last n positions); none when that count is
 *               <= 0 (out = 0, lse = -inf).
 *   q          device bf16 [total_q, 16, 576]
 *   qo_indptr  device int32 [batch + 1], non-decreasing, qo_indptr[0] = 0,
 *              qo_indptr[batch] = total_q; not read when uni_q_len > 0 (may
 *              then be NULL)
 *   total_q    host copy of qo_indptr[batch]
 *   uni_q_len  > 0: every sequence has exactly uni_q_len query tokens
 *              (total_q must equal batch * uni_q_len); 0: ragged, from qo_indptr
 *   causal     0 or 1 as above
 *   out, lse   device bf16 [total_q, 16, 512] and fp32 [total_q, 16] (or NULL)
 *   kv .. page_size, batch, total_kv, kv_dtype, sm_scale, stream
 *              as mla_decode_paged (page_size 1: the layout of mla_decode)
 *   workspace  at least mla_decode_mtp_workspace_size(...) bytes, 16-byte
 *              aligned (NULL allowed when that size is 0)
 *   flags      MLA_FLAG_FORCE_SPLIT with a split count, or 0 (heuristic);
 *              MLA_FLAG_ROW_PER_WG; the plan (mla_decode_mtp_plan) is always
 *              split-K, and MLA_FLAG_FORCE_PERSISTENT is rejected
 * Returns as mla_decode_paged; MLA_ERR_INVALID_ARG also for a bad causal,
 * total_q or uni_q_len, or a NULL / misaligned qo_indptr when uni_q_len = 0.
 */
int mla_decode_mtp(const void* q, const int32_t* qo_indptr, int total_q, int uni_q_len, int causal, const void* kv,
                   const void* kv_scales, const int32_t* kv_indptr, const int32_t* kv_indices,
                   const int32_t* kv_last_page_len, int page_size, void* out, float* lse, int batch, int64_t total_kv,
                   int kv_dtype, float sm_scale, void* workspace, size_t workspace_bytes, int flags, void* stream);

/*
 * mla_decode_mtp_plan: the launch plan of mla_decode_mtp for these sizes
 * (pure host function). The plan is split-K. On the bf16 cache with a
 * uniform query count n = uni_q_len >= 2 (and without MLA_FLAG_ROW_PER_WG),
 * each workgroup carries two consecutive query rows of one sequence (the
 * last of an odd n alone): grid = splits x batch x ceil(n / 2), and
 * rows_per_wg = 2; both rows' scores run on the rows the workgroup gathers
 * once. Otherwise each workgroup carries one query row: grid = splits x
 * total_q, rows_per_wg = 1. Partials are per query row (num_partials =
 * splits x total_q when splits > 1), merged as for mla_decode.
 * Returns MLA_OK or MLA_ERR_INVALID_ARG.
 */
int mla_decode_mtp_plan(int batch, int total_q, int uni_q_len, int64_t total_kv, int kv_dtype, int flags,
                        mla_plan_info* plan);

/*
 * mla_decode_mtp_workspace_size: bytes of workspace mla_decode_mtp needs
 * (the split partials of mla_decode_mtp_plan's plan). Pure host function; 0
 * for invalid arguments.
 */
size_t mla_decode_mtp_workspace_size(int batch, int total_q, int uni_q_len, int64_t total_kv, int kv_dtype,
                                     int flags);

/*
 * mla_dequant_debug: decode `rows` physical cache rows to fp32 [rows, 576]
 * through the attention kernel's own staging and decode routines (test aid
 * for the bit-exact decoder check). For fp8 the value written is the binary32
 * product (code value) * kv_scale[0]; for MXFP4 it is the e2m1 value times
 * 2^(e8m0 - 127); for bf16 the value itself.
 *   kv, kv_scales  as for mla_decode (row r of the output is physical row r)
 *   path           0: all columns through the score-operand decode (the
 *                     bf16 cache and fp8 scores use it; MXFP4 scores take the
 *                     codes into the MX-scaled MFMA undecoded);
 *                  1: columns 0..511 through the value-operand decode (LDS
 *                     transpose reads), columns 512..575 as path 0
 *   out_f32        device fp32 [rows, 576]
 * Returns MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED or MLA_ERR_HIP.
 */
int mla_dequant_debug(int kv_dtype, const void* kv, const void* kv_scales, int64_t rows, int path,
                      float* out_f32, void* stream);

/*
 * mla_hbm_read_probe: measurement aid, not part of the decode. Streams `bytes`
 * bytes of device memory at `buf` into LDS with the same LDS-DMA loads (and
 * cache hint) that gather the cache rows, two workgroups per compute unit,
 * each reading one contiguous share; nothing is written. Its run time is the
 * practical HBM read ceiling the decode's effective bandwidth is compared with.
 *   buf    device memory, 16-byte aligned, caller-owned
 *   bytes  a multiple of 16 (0 is a no-op)
 * Returns MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED or MLA_ERR_HIP.
 */
int mla_hbm_read_probe(const void* buf, size_t bytes, void* stream);

/*
 * mla_source_digest: identifies the sources this library was compiled from:
 * the first 16 hex digits of SHA-256 over the kernel, planner and this
 * header, as the build computed them ("unrecorded" when built without it).
 * A caller compares it with the digest of the sources it expects, so timings
 * and test results are never attributed to a library left over from other
 * sources. Pure host function; the string is static and owned by the library.
 */
const char* mla_source_digest(void);

/* mla_status_string: static, human-readable text for a status code. */
const char* mla_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */

// Launch planning for MLA decode: split count / grid size and workspace layout.
// Pure host code with no HIP dependency, so it is testable without a GPU.
//
// Two grid shapes are planned:
//   split-K     (splits x batch) workgroups; split s of sequence b covers
//               tokens [s*chunk, min(L_b, (s+1)*chunk)), chunk = ceil(L_b /
//               splits) rounded up to the 32-token workgroup step. One partial
//               slot per (b, s); when splits > 1 the partials of a sequence
//               are merged by its last-arriving split workgroup (up to
//               kMaxMergeSplits splits; up to kMaxMergeSplitsBf16 on the bf16
//               and fp8 caches, from bf16 partials) or by a combine launch.
//               (Flash-decoding split-K: the split partial plus log-sum-exp
//               merge of amd-mixed-mla submission 593653, `_flash_fp8_split_s1`
//               and `_flash_fp8_split_s2`.)
//   persistent  a fixed grid of P workgroups; workgroup p covers the tokens
//               [floor(p*T/P), floor((p+1)*T/P)) of the concatenated sequences
//               and writes one partial per sequence it touches, into slot
//               p + b. The persistent grid of the pages (submission 593653's
//               cached persistent path; submission 616673's a16w8 persistent
//               path) needs a metadata kernel; this partition needs none.
#include "mla_plan.h"

#include <stdint.h>

namespace mla {

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

static size_t partial_bytes(int num_partials) {
    // the arrival counters, then part_o [num_partials][16][512] fp32, then
    // part_lse [num_partials][16] fp32, each section padded to 256 bytes.
    size_t o = (size_t)num_partials * kHeads * kDv * sizeof(float);
    size_t l = (size_t)num_partials * kHeads * sizeof(float);
    return kCounterBytes + ((o + 255) / 256) * 256 + ((l + 255) / 256) * 256;
}

// The partial maxima of the dynamic fp8 query scale follow the plan's bytes,
// and never start inside the arrival-counter region: a plan without split
// partials needs no workspace of its own, but the region must stay zero for
// later calls that reuse the buffer with a merging plan.
size_t q8_amax_offset(size_t plan_bytes) {
    const size_t o = (plan_bytes + 255) & ~(size_t)255;
    return o < kCounterBytes ? kCounterBytes : o;
}

size_t partial_lse_offset(int num_partials) {
    size_t o = (size_t)num_partials * kHeads * kDv * sizeof(float);
    return kCounterBytes + ((o + 255) / 256) * 256;
}

// Split count for split-K, the larger of two rules (each capped at kMaxSplits):
//   fill every workgroup slot of the chip (wgs_per_cu per compute unit) with
//   at least kMinTokensPerWg tokens per workgroup, so that the gather pipeline
//   overlaps (each split also costs a 32 KB partial written and read back);
//   for short sequences, one workgroup per compute unit with at least one
//   32-token step each, since latency rather than bandwidth bounds them.
// A third rule applies when the split partials can be merged by the last-
// arriving split (merge_ok) and the first two rules' split count could not
// be (more than 8 splits on the bf16 and fp8 caches, more than 4 on MXFP4):
// if one workgroup per compute unit fills the chip with at most
// kMaxMergeSplits splits and each split is short, that plan saves the
// combine launch, which costs more than the second workgroup per compute
// unit gains on short splits. Long splits keep two workgroups per compute
// unit to stream.
// Measured optima this reproduces (cold, MI355X): 4 x 1k: 32 splits (bf16
// 14.8 vs 18.1 us at 8 splits; 14.2 against 15.2 at 8 merged); 32 x 1k fp8:
// 8 merged (17.0 us, against 17.6 with the combine launch and 19.4 at 4
// merged); 64 x 1k bf16: 4; 64 x 1k fp8: 8 merged (20.4 us, against 20.9 at
// 4 merged and 23.4 at 8 with the combine launch); 64 x 1k MXFP4: 4 merged
// (equal to 8 with the launch, 23.1 both); 256 x 1k fp8: 2 (39.7 us merged,
// against 41.9 at 1); 64 x 8k fp8: 8 merged (66.1 us, against 79.7 at 4
// merged, when both merged on the VALU); 32 x 8k fp8: 16 (40.4 us, against
// 43.4 at 8 merged); 32 x 8k MXFP4: 16.
int heuristic_splits(int batch, int64_t total_kv, int kv_dtype, bool merge_ok) {
    if (batch <= 0) return 1;
    const int64_t avg = cdiv(total_kv, batch);
    auto rule = [&](int64_t wgs, int64_t min_tokens) {
        int64_t s = cdiv(wgs, batch);
        if (s > avg / min_tokens) s = avg / min_tokens;
        if (s > kMaxSplits) s = kMaxSplits;
        return s < 1 ? (int64_t)1 : s;
    };
    const int64_t fill = rule((int64_t)kNumCUs * wgs_per_cu(kv_dtype), kMinTokensPerWg);
    const int64_t per_cu = rule(kNumCUs, kStepTokens);
    const int64_t s = fill > per_cu ? fill : per_cu;
    if (merge_ok && batch <= kMaxCounterRows && s > max_stage1_merge_splits(kv_dtype) && per_cu > 1 &&
        per_cu <= kMaxMergeSplits &&
        (int64_t)batch * per_cu >= kNumCUs && cdiv(avg, per_cu) <= kShortSplitTokens)
        return (int)per_cu;
    return (int)s;
}

// Persistent grid: one workgroup per compute unit, fewer when there are not
// enough tokens to give each at least kMinTokensPerWg.
int heuristic_grid(int64_t total_kv, int kv_dtype) {
    int64_t g = (int64_t)kNumCUs * wgs_per_cu(kv_dtype);
    int64_t by_len = total_kv / kMinTokensPerWg;
    if (g > by_len) g = by_len;
    if (g < 1) g = 1;
    return (int)g;
}

// The default shape. Split-K when the batch alone fills the chip or when the
// split grid lands on a whole number of workgroups per compute unit; the
// persistent grid for large, uneven shapes where the split grid would leave
// compute units idle.
static bool prefer_persistent(int batch, int64_t total_kv, int kv_dtype, bool merge_ok) {
    if (total_kv < (int64_t)kNumCUs * kPersistentMinTokensPerCU) return false;
    int s = heuristic_splits(batch, total_kv, kv_dtype, merge_ok);
    int64_t wgs = (int64_t)s * batch;
    return (wgs % kNumCUs) != 0;
}

int make_plan(int batch, int64_t total_kv, int kv_dtype, int flags, mla_plan_info* p) {
    if (!p) return MLA_ERR_INVALID_ARG;
    if (batch < 0 || total_kv < 0 || total_kv > INT32_MAX) return MLA_ERR_INVALID_ARG;
    if (kv_dtype < MLA_KV_BF16 || kv_dtype > MLA_KV_MXFP4) return MLA_ERR_INVALID_ARG;
    const bool force_split = (flags & MLA_FLAG_FORCE_SPLIT) != 0;
    const bool force_pers = (flags & MLA_FLAG_FORCE_PERSISTENT) != 0;
    if (force_split && force_pers) return MLA_ERR_INVALID_ARG;
    const int forced_splits = (flags >> MLA_FLAG_SPLITS_SHIFT) & 0xFF;
    const int forced_grid = (flags >> MLA_FLAG_GRID_SHIFT) & 0xFFF;
    if (flags & ~(MLA_FLAG_FORCE_SPLIT | MLA_FLAG_FORCE_PERSISTENT | MLA_FLAG_MIXED_LENGTHS |
                  MLA_FLAG_COMBINE_LAUNCH | MLA_FLAG_ROW_PER_WG | (0xFF << MLA_FLAG_SPLITS_SHIFT) |
                  (0xFFF << MLA_FLAG_GRID_SHIFT)))
        return MLA_ERR_INVALID_ARG;

    p->rows_per_wg = 1;
    if (batch == 0) {
        p->mode = 0;
        p->num_splits = 1;
        p->grid = 0;
        p->num_partials = 0;
        p->combine = 0;
        p->workspace_bytes = 0;
        return MLA_OK;
    }
    // The caller's hint that sequence lengths differ selects the persistent
    // grid: its equal token shares balance mixed lengths, where split-K's
    // per-sequence splits leave the longest sequences on the critical path.
    const bool mixed = (flags & MLA_FLAG_MIXED_LENGTHS) != 0 && total_kv >= kNumCUs;
    const bool merge_ok = (flags & MLA_FLAG_COMBINE_LAUNCH) == 0;
    bool persistent = force_pers || (!force_split && forced_splits == 0 &&
                                     (mixed || prefer_persistent(batch, total_kv, kv_dtype, merge_ok)));
    if (persistent) {
        int g = forced_grid ? forced_grid : heuristic_grid(total_kv, kv_dtype);
        p->mode = 1;
        p->num_splits = 0;
        p->grid = g;
        p->num_partials = g + batch - 1;
        p->combine = 1;
        p->workspace_bytes = partial_bytes(p->num_partials);
    } else {
        int s = forced_splits ? forced_splits : heuristic_splits(batch, total_kv, kv_dtype, merge_ok);
        p->mode = 0;
        p->num_splits = s;
        p->grid = s * batch;
        p->num_partials = (s > 1) ? s * batch : 0;
        // The last-arriving split of a row merges the row's partials alone,
        // so that merge pays only while it reads a few of them; many splits
        // (short batches of long sequences) merge in the wide combine launch.
        // 5..8 splits merge there from bf16 partials on the MFMA: against the
        // combine launch fp8 64 x 8k 60.3 -> 58.8 us (with the merge before
        // it on the VALU 61.8 -> 61.1), fp8 32 x 1k 17.6 -> 17.0, bf16
        // 32 x 1k 20.6 -> 20.2. Not on the MXFP4 cache, bound by instruction
        // issue, where the last arrivals' merge lengthens the tail: 64 x 8k
        // 58.8 -> 59.2 us.
        const bool merge_in_stage1 = s <= max_stage1_merge_splits(kv_dtype) && batch <= kMaxCounterRows && merge_ok;
        p->combine = (s > 1) ? (merge_in_stage1 ? 2 : 1) : 0;
        p->workspace_bytes = (s > 1) ? partial_bytes(p->num_partials) : 0;
    }
    return MLA_OK;
}

int mtp_plan(int batch, int total_q, int uni_q, int64_t total_kv, int kv_dtype, int flags, mla_plan_info* p) {
    if (batch < 0 || total_q < 0 || uni_q < 0 || total_kv < 0 || total_kv > INT32_MAX) return MLA_ERR_INVALID_ARG;
    if (flags & MLA_FLAG_FORCE_PERSISTENT) return MLA_ERR_INVALID_ARG;
    if (uni_q > 0 && (int64_t)uni_q * batch != total_q) return MLA_ERR_INVALID_ARG;
    // On the bf16 cache (one workgroup per CU, registers to spare) a workgroup
    // carries two query rows of a sequence, so the cache is gathered once for
    // both: the plan runs over the row pairs, each seeing its sequence.
    const bool pairs = kv_dtype == MLA_KV_BF16 && uni_q >= 2 && (flags & MLA_FLAG_ROW_PER_WG) == 0;
    const int64_t work_rows = pairs ? (int64_t)batch * ((uni_q + 1) / 2) : total_q;
    // the work rows together see about total_kv * work_rows / batch tokens (capped to the planner's range)
    int64_t tokens = batch > 0 ? total_kv * work_rows / batch : 0;
    if (tokens > INT32_MAX) tokens = INT32_MAX;
    const int rc = make_plan((int)work_rows, tokens, kv_dtype, flags | MLA_FLAG_FORCE_SPLIT, p);
    if (rc != MLA_OK || !pairs) return rc;
    // partials and arrival counters stay per query row
    const int s = p->num_splits;
    const bool merge_ok = (flags & MLA_FLAG_COMBINE_LAUNCH) == 0;
    p->rows_per_wg = 2;
    p->num_partials = (s > 1) ? s * total_q : 0;
    p->combine = (s > 1) ? ((s <= kMaxMergeSplits && total_q <= kMaxCounterRows && merge_ok) ? 2 : 1) : 0;
    p->workspace_bytes = (s > 1) ? partial_bytes(p->num_partials) : 0;
    return MLA_OK;
}

}  // namespace mla

extern "C" int mla_decode_plan(int batch, int64_t total_kv, int kv_dtype, int flags, mla_plan_info* plan) {
    return mla::make_plan(batch, total_kv, kv_dtype, flags, plan);
}

extern "C" size_t mla_decode_workspace_size(int batch, int64_t total_kv, int kv_dtype, int flags) {
    mla_plan_info p;
    if (mla::make_plan(batch, total_kv, kv_dtype, flags, &p) != MLA_OK) return 0;
    return p.workspace_bytes;
}

extern "C" int mla_decode_mtp_plan(int batch, int total_q, int uni_q_len, int64_t total_kv, int kv_dtype, int flags,
                                   mla_plan_info* plan) {
    if (!plan) return MLA_ERR_INVALID_ARG;
    return mla::mtp_plan(batch, total_q, uni_q_len, total_kv, kv_dtype, flags, plan);
}

extern "C" size_t mla_decode_mtp_workspace_size(int batch, int total_q, int uni_q_len, int64_t total_kv, int kv_dtype,
                                                int flags) {
    mla_plan_info p;
    if (mla::mtp_plan(batch, total_q, uni_q_len, total_kv, kv_dtype, flags, &p) != MLA_OK) return 0;
    return p.workspace_bytes;
}

extern "C" size_t mla_decode_q8_workspace_size(int batch, int64_t total_kv, int kv_dtype, int flags,
                                               int q_scale_mode) {
    mla_plan_info p;
    if (q_scale_mode != MLA_Q_SCALE_STATIC && q_scale_mode != MLA_Q_SCALE_DYNAMIC) return 0;
    if (mla::make_plan(batch, total_kv, kv_dtype, flags, &p) != MLA_OK) return 0;
    if (q_scale_mode == MLA_Q_SCALE_STATIC) return p.workspace_bytes;
    return mla::q8_amax_offset(p.workspace_bytes) + mla::kQ8AmaxParts * sizeof(float);
}

extern "C" const char* mla_status_string(int status) {
    switch (status) {
        case MLA_OK: return "ok";
        case MLA_ERR_INVALID_ARG: return "invalid argument";
        case MLA_ERR_UNSUPPORTED: return "unsupported device (gfx950 required)";
        case MLA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case MLA_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

#ifndef MLA_SOURCE_DIGEST
#define MLA_SOURCE_DIGEST "unrecorded"
#endif

extern "C" const char* mla_source_digest(void) { return MLA_SOURCE_DIGEST; }

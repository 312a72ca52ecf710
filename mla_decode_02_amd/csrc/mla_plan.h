// Internal planning constants and helpers shared by the host planner and the
// HIP launch code. No HIP dependency.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "mla_decode.h"

namespace mla {

constexpr int kHeads = MLA_NUM_HEADS;
constexpr int kDqk = MLA_QK_DIM;
constexpr int kDv = MLA_V_DIM;

constexpr int kNumCUs = 256;          // MI355X compute units
constexpr int kWaves = 4;             // waves per stage-1 workgroup
constexpr int kStepTokens = 32;       // tokens per workgroup step (two 16-token MFMA tiles)
constexpr int kMinTokensPerWg = 4 * kStepTokens;  // enough steps for the gather pipeline to overlap
constexpr int kMaxSplits = 64;
constexpr int kPersistentMinTokensPerCU = 1024;
constexpr int kQ8AmaxParts = 256;     // partial maxima of the dynamic fp8 query scale (at most)
constexpr size_t kCounterBytes = MLA_WORKSPACE_COUNTER_BYTES;          // arrival counters ahead of the partials
constexpr int kMaxCounterRows = (int)(kCounterBytes / sizeof(uint32_t));  // query rows with a counter
constexpr int kMaxMergeSplits = 4;    // split-K plans merged by the last-arriving split, fp32 partials
// 5..8 splits are merged there too on the bf16 and fp8 caches, from bf16
// partials, so that one round of loads holds them all (more splits, or
// MXFP4: a combine launch)
constexpr int kMaxMergeSplitsBf16 = 8;
// Most splits the last-arriving split merges on a cache format.
constexpr int max_stage1_merge_splits(int kv_dtype) {
    return kv_dtype == MLA_KV_MXFP4 ? kMaxMergeSplits : kMaxMergeSplitsBf16;
}
constexpr int64_t kShortSplitTokens = 256;  // longest split the one-workgroup-per-CU merged plan is chosen for

// Stage-1 workgroups resident per compute unit (bound by the LDS ring size:
// bf16 one, fp8 and MXFP4 two).
constexpr int wgs_per_cu(int kv_dtype) { return kv_dtype == MLA_KV_BF16 ? 1 : 2; }

int make_plan(int batch, int64_t total_kv, int kv_dtype, int flags, mla_plan_info* p);
int heuristic_splits(int batch, int64_t total_kv, int kv_dtype, bool merge_ok);
int heuristic_grid(int64_t total_kv, int kv_dtype);
size_t partial_lse_offset(int num_partials);
// Plan for total_q query rows over `batch` sequences holding total_kv cache
// tokens (several query tokens per sequence, uni_q each when > 0): always
// split-K, made as for that many sequences of the average length, where a
// "sequence" is a query row, or (bf16 cache, uni_q >= 2) a pair of rows that
// one workgroup carries (rows_per_wg = 2; partials stay per query row).
int mtp_plan(int batch, int total_q, int uni_q, int64_t total_kv, int kv_dtype, int flags, mla_plan_info* p);
// Offset of the dynamic fp8 query scale's partial maxima: after the plan's
// bytes and never inside the arrival-counter region.
size_t q8_amax_offset(size_t plan_bytes);

}  // namespace mla

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
constexpr int kWgsPerCU = 1;          // stage-1 workgroups resident per CU (LDS/VGPR bound)
constexpr int kWaves = 4;             // waves per stage-1 workgroup
constexpr int kStep = 16;             // tokens per wave step (MFMA M dimension)
constexpr int kMinTokensPerWg = kWaves * kStep;
constexpr int kMaxSplits = 64;
constexpr int kPersistentMinTokensPerCU = 1024;

int make_plan(int batch, int64_t total_kv, int kv_dtype, int flags, mla_plan_info* p);
int heuristic_splits(int batch, int64_t total_kv);
int heuristic_grid(int64_t total_kv);
size_t partial_lse_offset(int num_partials);

}  // namespace mla

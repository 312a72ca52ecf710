// MI355X (gfx950) MLA decode: split-K / persistent stage 1, the log-sum-exp
// combine, the fp8-query scale reduction, and decode / quantiser check
// kernels, behind the C ABI declared in include/mla_decode.h.
//
// The operation is the one on the amd-mixed-mla pages (submission 593653,
// `_bmm_reference` and the module constants): 16 query heads share one latent
// KV row per token; scores over 576 dims (512 no-RoPE + 64 RoPE), softmax over
// the tokens, output over the first 512 dims of the same rows.
//
// Stage 1: one workgroup of four waves attends one token range of one query
// row (or, on the bf16 cache with several query tokens, of two rows), in
// 32-token steps (two 16-token tiles). At wave start the query, the first
// window of kv_indices (guessed on split plans with equal lengths, before
// kv_indptr arrives) and, with the cache's row count known, the first steps'
// rows of a contiguous cache are requested together. Per step:
//   1. The step's 32 cache rows are gathered through kv_indices straight from
//      HBM into an LDS ring with LDS-DMA loads (global_load_lds_dwordx4; the
//      MXFP4 scales with two-byte DMAs), kRing - 1 steps ahead of use. Each
//      wave issues one half of one tile. Lane (G, r) of a tile fetches bytes
//      64u + 16G of row r for load u: the MFMA operand layout of the scores.
//   2. Scores S^T[16 tokens x 16 heads] = K . Q^T: wave w computes tile w % 2
//      over half w / 2 of the score dims on v_mfma_f32_16x16x32_bf16 (Q^T in
//      VGPRs), and each tile's two half products are summed through LDS. fp8
//      codes are decoded exactly to bf16 with the gfx950 scaled converts
//      (kv_scale folded into the score scale and the output). On the MXFP4
//      cache the scores run on the MX-scaled fp4 x fp8 MFMA on the raw codes,
//      with the bf16 query split into two e4m3fn code sets (see
//      q_split_quantise). With an fp8 query the scores run on fp8 x fp8 (fp8
//      cache) or MX-scaled fp4 x fp8 (MXFP4 cache) MFMAs on the raw codes.
//   3. Online softmax in the log2 domain with lazy rescaling (the running max
//      only moves when a score exceeds it by 2^8). Every wave runs it on the
//      full step and holds the same max and sum. The S^T accumulator is
//      already the A-operand layout of P for the second product.
//   4. O[16 x 512] += P . V on v_mfma_f32_16x16x32_bf16, each wave for its own
//      128 columns. The token-major V operand comes from LDS transpose reads
//      (ds_read_b64_tr_b8 for fp8 / MXFP4 bytes, ds_read_b64_tr_b16 for bf16)
//      of the same staged rows: V is the first 512 columns of K, so each row is
//      fetched from HBM once.
// The loop is software-pipelined with one barrier per step. The result is the
// final bf16 output + lse, or a split partial (normalised O and its lse;
// fp32, or bf16 on plans of 5 to 8 splits merged in stage 1) that the
// last-arriving split of the row or the combine kernel merges (flash-decoding
// split partials and log-sum-exp merge: submission 593653,
// `_flash_fp8_split_s1` / `_flash_fp8_split_s2`).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "mla_decode.h"
#include "mla_decode_phases.h"
#include "mla_plan.h"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kThreads = 64 * kWaves;

// ---------------------------------------------------------------------------
// Phase timestamps, in the measurement build only (MLA_PHASE_STAMPS=1, the
// library libmla_decode_phases.so; the decode library is built without them
// and contains none of this). Thread 0 of each stage-1 workgroup records the
// 100 MHz real-time counter (s_memrealtime) at the kPhases points below into
// the buffer the host set with mla_phase_buffers, [workgroup][phase]; thread
// 0 of each combine workgroup records its start and end, [workgroup][2].
//   0 kernel entry
//   1 query registers and the first index window in hand
//   2 the first step's rows landed in LDS (after its barrier)
//   3 every step of the range done
//   4 the epilogue's stores complete (every thread)
//   5 the stage-1 merge done (plans that merge in stage 1; else as 4)
// A persistent workgroup attends several sequences: phases 1-4 are those of
// its last one.
// ---------------------------------------------------------------------------
#ifndef MLA_PHASE_STAMPS
#define MLA_PHASE_STAMPS 0
#endif
constexpr int kPhases = 8;
#if MLA_PHASE_STAMPS
__device__ uint64_t* g_phase_stage1;
__device__ uint64_t* g_phase_combine;
#endif
__device__ __forceinline__ void phase_stamp(int k) {
#if MLA_PHASE_STAMPS
    if (threadIdx.x == 0 && g_phase_stage1)
        g_phase_stage1[(size_t)blockIdx.x * kPhases + k] = __builtin_amdgcn_s_memrealtime();
#else
    (void)k;
#endif
}
// Phase 4: in the measurement build, wait for every thread's stores first.
__device__ __forceinline__ void phase_stamp_stores_done() {
#if MLA_PHASE_STAMPS
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    phase_stamp(4);
#endif
}
__device__ __forceinline__ void phase_stamp_combine(int k) {
#if MLA_PHASE_STAMPS
    if (threadIdx.x == 0 && g_phase_combine)
        g_phase_combine[(size_t)blockIdx.x * 2 + k] = __builtin_amdgcn_s_memrealtime();
#else
    (void)k;
#endif
}
constexpr int kTile = 16;                // tokens per MFMA tile
static_assert(kStepTokens == 2 * kTile, "a step is two MFMA tiles");
constexpr int kKSteps = kDqk / 32;       // 18 MFMA k-steps over the 576 score dims
constexpr int kBlocks = kDv / 16;        // 32 output blocks of 16 columns per wave
constexpr float kRescaleThresh = 8.0f;   // log2 units
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct Params {
    const __bf16* q;
    const uint8_t* kv;
    const void* kv_scales;
    const int32_t* indptr;     // [batch + 1] into indices (pages when page_size > 1)
    const int32_t* indices;    // row (page_size 1) or page id of each entry
    const int32_t* last_page;  // [batch] tokens in the last page (page_size > 1)
    int page_size;             // rows per page (1: indices are rows)
    __bf16* out;
    float* lse;
    float* part_o;
    float* part_lse;
    int batch;
    int nsplit;  // split-K: splits per sequence
    int grid;    // persistent: number of workgroups
    int total;   // kv_indptr[batch]
    float sm_scale;
    // fp8 query only: the per-tensor scale (static: read; dynamic: written by
    // workgroup 0) and, for the dynamic scale, the partial maxima of |q|.
    float* q_scale;
    const float* q_amax;
    int q_amax_n;
    // Several query tokens per sequence: query row r of `rows` (q, out, lse
    // rows) belongs to sequence b with qo_indptr[b] <= r < qo_indptr[b+1]
    // (uni_q > 0: every sequence has uni_q rows and qo_indptr is not read).
    // causal: token t of n sees the first L - n + 1 + t cache tokens.
    // qo_indptr NULL and uni_q 0: one row per sequence (rows = batch).
    const int32_t* qo_indptr;
    int uni_q;
    int causal;
    int rows;
    // Split-K with one row per sequence, when total (tokens) is a multiple of
    // batch, the page size a power of two and uni_len = total / batch a
    // multiple of it: uni_len and its split chunk (the length every sequence
    // has when the lengths are equal); else 0.
    int uni_len;
    int uni_chunk;
    // Split-K partials merged by the last-arriving split workgroup of each
    // query row: one arrival counter per row (zero between calls); NULL when a
    // combine launch merges them.
    uint32_t* counters;
    // Rows the cache buffer holds (0: unknown). Known, on batches of equal
    // lengths, it bounds the rows gathered before kv_indices arrives.
    int64_t kv_rows;
};

// ---------------------------------------------------------------------------
// Cache formats: staging layout of one 16-row tile in LDS. The gather of a
// tile is split in two halves (hf = 0, 1), each issued by one wave; every
// LDS-DMA load writes 64 consecutive 16-byte slots of the tile, lane L of load
// v at slot 64 v + L. Chunk c of tile row r (bytes 16 c .. 16 c + 15 of that
// cache row) sits in slot slot(r, c).
//   bf16 and fp8: each group of 8 lanes of a load fetches one whole 128-byte
//     run of cache memory, so the HBM requests of every load are whole lines
//     (a row gather that reads 64-byte pieces of 16 rows per load streams
//     about a third slower); within its run a row's chunks are permuted by an
//     XOR with a function of the row, and the runs are placed so that the 16
//     rows of any chunk lie in 16 different 16-byte bank groups modulo 256
//     bytes (8 different ones in each half of 8 rows): the score operand reads
//     (one chunk of 16 rows) and the transposed value reads stay free of bank
//     conflicts.
//     bf16 (72 chunks per row: 9 runs, the 9 lines of a 1152-byte row): load
//       v = 2k + h brings run k of rows 8h .. 8h + 7, row 8h + (m ^ h) on
//       lanes 8m .. 8m + 7; half hf issues the loads with h = hf, so each lane
//       fetches from one row.
//       slot(r, c) = 64 (2 (c / 8) + r / 8) + 8 ((r % 8) ^ (r / 8)) + ((c % 8) ^ (r % 8))
//     fp8 (36 chunks per row): rows 2p and 2p + 1 form a pair of 72 chunks,
//       pair chunk q = c + 36 (r % 2), i.e. 9 runs that are whole lines when
//       the pair's first row has an even index in a contiguous cache. Load v
//       brings run v of all 8 pairs, pair p on lanes 8 sigma(p) ..,
//       sigma(p) = 2 (p % 4) + p / 4; half hf issues the loads v = hf, hf + 2,
//       .., and each lane fetches from the two rows of its pair.
//       slot(r, c) = 64 (q / 8) + 8 sigma(p) + ((q % 8) ^ (p % 4)),  p = r / 2
//   MXFP4: lane (G, r) = (lane / 16, lane % 16) of code load u (0 <= u < 4)
//     brings bytes 64u + 16G .. +15 of tile row r to tile + 1024u + 16 lane;
//     the 32 RoPE bytes of each row (bytes 256..287) are one 16-byte DMA
//     on lanes 0..31 (lane (c, r) brings bytes 256 + 16c .. +15 of row r
//     to tile + kRopeOff + 16 lane); the 18 e8m0 codes of each row are
//     two-byte DMAs, load v bringing codes 2p, 2p+1, p = 4v + G, of row
//     r into the low half of the dword at tile + kScaleOff + 256 v + 4 lane
//     (load 2 on lanes 0..15 only). Half 0 issues codes 0, 2 and scale
//     loads 0, 2; half 1 codes 1, 3, the RoPE load and scale load 1.
// ---------------------------------------------------------------------------
template <int KV>
struct Fmt;
template <>
struct Fmt<MLA_KV_BF16> {
    static constexpr int kRowBytes = 2 * kDqk;
    static constexpr int kCodeLoads = 18;
    static constexpr int kTileBytes = 18 * 1024;
    static constexpr int kRing = 4;         // steps resident in the workgroup's LDS ring
    static constexpr int kIdxWindow = 2048;  // tokens whose indices are staged in LDS at a time
    static constexpr int kWgsPerCU = 1;     // LDS bound
    static constexpr int ops(int hi) { return 9 + 0 * hi; }  // LDS-DMA instructions of one tile half
};
template <>
struct Fmt<MLA_KV_FP8_E4M3> {
    static constexpr int kRowBytes = kDqk;
    static constexpr int kCodeLoads = 9;
    static constexpr int kTileBytes = 9 * 1024;
    static constexpr int kRing = 3;
    static constexpr int kIdxWindow = 2048;
    static constexpr int kWgsPerCU = 2;
    static constexpr int ops(int hi) { return hi ? 4 : 5; }
};
template <>
struct Fmt<MLA_KV_MXFP4> {
    static constexpr int kRowBytes = kDqk / 2;
    static constexpr int kCodeLoads = 4;
    static constexpr int kRopeOff = 4 * 1024;
    static constexpr int kScaleOff = kRopeOff + 512;
    static constexpr int kTileBytes = kScaleOff + 3 * 256;
    static constexpr int kRing = 4;
    static constexpr int kIdxWindow = 1024;
    static constexpr int kWgsPerCU = 2;
    static constexpr int ops(int hi) { return 4 + 0 * hi; }
};

// LDS of one stage-1 workgroup: the ring of staged steps, the exchange buffer
// for the four waves' partial scores, and the index window.
template <int KV>
struct Layout {
    static constexpr int kStepBytes = 2 * Fmt<KV>::kTileBytes;
    static constexpr int kRingBytes = Fmt<KV>::kRing * kStepBytes;
    static constexpr int kSbufOff = kRingBytes;
    static constexpr int kSbufBytes = kWaves * 64 * 16;  // one step's partial scores; double-buffered
    // MXFP4: the step's value-block scales as fp32, [tile][block 0..15][token], double-buffered
    static constexpr int kFsBytes = KV == MLA_KV_MXFP4 ? 2 * 16 * kTile * 4 : 0;
    static constexpr int kFsOff = kSbufOff + 2 * kSbufBytes;
    static constexpr int kIdxOff = kFsOff + 2 * kFsBytes;
    static constexpr int kBytes = kIdxOff + Fmt<KV>::kIdxWindow * 4;
    static_assert(kBytes * Fmt<KV>::kWgsPerCU <= 160 * 1024, "stage-1 LDS exceeds 160 KiB per CU");
    static_assert(Fmt<KV>::kIdxWindow % kThreads == 0, "index window is loaded by whole workgroups");
    static_assert(Fmt<KV>::kTileBytes % 16 == 0, "tiles stay 16-byte aligned");
    static_assert(kStepBytes >= kHeads * kDqk, "a ring slot holds one sequence's fp8 query codes");
};

// First score dim of the eight held by lane group G in k-step ks. Q^T is
// loaded with the same mapping, so every MFMA contracts exactly those dims.
template <int KV>
__device__ __forceinline__ constexpr int dbase(int ks, int G) {
    if (KV == MLA_KV_BF16) return 32 * ks + 8 * G;
    if (KV == MLA_KV_FP8_E4M3) return 64 * (ks >> 1) + 16 * G + 8 * (ks & 1);
    return ks < 16 ? 128 * (ks >> 2) + 32 * G + 8 * (ks & 3) : 512 + 16 * G + 8 * (ks - 16);
}

// Output column held by lane column r in accumulator block blk.
template <int KV>
__device__ __forceinline__ int dcol(int blk, int r) {
    if (KV == MLA_KV_MXFP4) return 32 * (blk >> 1) + 2 * r + (blk & 1);
    return 16 * blk + r;
}

// Token (0..31 within a step) of k-slot j for lane group G in the P . V
// product: slots 0-3 are tile 0's tokens 4G..4G+3, slots 4-7 tile 1's.
__device__ __forceinline__ int tau(int G, int j) { return j < 4 ? 4 * G + j : 16 + 4 * G + (j - 4); }

// LDS-DMA loads: lane L's `size` bytes from its global address g land at LDS
// byte lds + size * L (size 16), or in the dword at lds + 4 L, zero-extended
// (sizes 2 and 4). Issued from inline assembly so that the compiler, which
// would otherwise drain every outstanding load before each LDS read it cannot
// prove disjoint, leaves the ordering to the explicit waits below. m0 (the
// LDS base operand) is restored before the statement ends.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
    uint32_t save;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(save) : "v"(g), "s"(lds) : "memory");
}
// The same from g + OFF (an immediate, 0 <= OFF < 4096) with the
// non-temporal hint (nt): cache rows are read once per call, so they are
// streamed through the caches rather than kept. The instruction offset of an
// LDS-DMA load moves its LDS destination as well as its global address
// (checked on gfx950), so m0 is set OFF below the destination; every caller's
// destination lies at least OFF bytes into LDS.
template <int OFF>
__device__ __forceinline__ void dma16nt(const void* g, uint32_t lds) {
    static_assert(OFF >= 0 && OFF < 4096, "global load offsets are 12-bit");
    uint32_t save;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off offset:%3 nt\n\ts_mov_b32 m0, %0"
                 : "=&s"(save) : "v"(g), "s"(lds - (uint32_t)OFF), "n"(OFF) : "memory");
}
__device__ __forceinline__ void dma2(const void* g, uint32_t lds) {
    uint32_t save;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_ushort %1, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(save) : "v"(g), "s"(lds) : "memory");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
    uint32_t save;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(save) : "v"(g), "s"(lds) : "memory");
}

// Element i of a read-only int array at a uniform address, as a scalar load
// (through the constant address space). Its wait is on the scalar counter,
// so it never drains the LDS-DMA loads in flight. The same read written as
// an ordinary load after the DMA asm (whose memory clobber rules out the
// scalar form) becomes a vector load whose wait, vmcnt(0), drains them.
__device__ __forceinline__ int32_t ld_scalar(const int32_t* p, int64_t i) {
    return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}
// Wave-uniform 32-bit LDS address of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void*)p);
}

// Wait until at most N vector-memory instructions of this wave are in flight.
// Also a compiler barrier for memory: the compiler does not order LDS reads
// after the LDS-DMA writes by itself.
template <int N>
__device__ __forceinline__ void wait_vmcnt() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// Tile rows whose cache rows lane `lane` fetches when issuing half hf of a
// tile: (first, second) -- the two rows of its pair (fp8), or its one row
// twice (bf16, MXFP4).
template <int KV>
__device__ __forceinline__ int2 lane_tile_rows(int lane, int hf) {
    if constexpr (KV == MLA_KV_BF16) {
        const int r = 8 * hf + ((lane >> 3) ^ hf);
        return make_int2(r, r);
    } else if constexpr (KV == MLA_KV_FP8_E4M3) {
        const int m = lane >> 3, p = (m >> 1) + 4 * (m & 1);
        return make_int2(2 * p, 2 * p + 1);
    } else {
        return make_int2(lane & 15, lane & 15);
    }
}

// The LDS-DMA loads of half HI of one tile (layout above). ra / rb are the
// cache rows of this lane's tile rows lane_tile_rows(lane, HI); `tile` is
// the tile's LDS staging area.
template <int KV, int HI>
__device__ __forceinline__ void issue_half(const Params& P, int64_t ra, int64_t rb, uint8_t* tile, int lane) {
    if constexpr (KV == MLA_KV_BF16) {
        // load 2k + HI: run k (bytes 128k ..) of the lane's row, its chunk 8k + jj
        const int r = 8 * HI + ((lane >> 3) ^ HI), jj = (lane & 7) ^ (r & 7);
        const uint8_t* src = P.kv + ra * Fmt<KV>::kRowBytes + 16 * jj;
        dma16nt<0>(src, lds_addr(tile + 1024 * (0 + HI)));
        dma16nt<128>(src, lds_addr(tile + 1024 * (2 + HI)));
        dma16nt<256>(src, lds_addr(tile + 1024 * (4 + HI)));
        dma16nt<384>(src, lds_addr(tile + 1024 * (6 + HI)));
        dma16nt<512>(src, lds_addr(tile + 1024 * (8 + HI)));
        dma16nt<640>(src, lds_addr(tile + 1024 * (10 + HI)));
        dma16nt<768>(src, lds_addr(tile + 1024 * (12 + HI)));
        dma16nt<896>(src, lds_addr(tile + 1024 * (14 + HI)));
        dma16nt<1024>(src, lds_addr(tile + 1024 * (16 + HI)));
    } else if constexpr (KV == MLA_KV_FP8_E4M3) {
        // load v: pair chunks 8v + jj; below 36 they are chunks of the pair's
        // first row, from 36 on chunks q - 36 of its second row
        const int m = lane >> 3, p = (m >> 1) + 4 * (m & 1), jj = (lane & 7) ^ (p & 3);
        const uint8_t* a = P.kv + ra * Fmt<KV>::kRowBytes + 16 * jj;
        const uint8_t* b = P.kv + rb * Fmt<KV>::kRowBytes + 16 * jj;
        if constexpr (HI == 0) {
            dma16nt<0>(a, lds_addr(tile + 1024 * 0));    // first row, chunk jj
            dma16nt<256>(a, lds_addr(tile + 1024 * 2));  // first row, chunk 16 + jj
            // pair chunk 32 + jj: first row chunk 32 + jj (jj < 4), second row chunk jj - 4 (jj >= 4;
            // jj >= 4 exactly when lane bit 2 is set, the XOR touching only bits 0-1)
            dma16nt<0>((lane & 4) ? b - 64 : a + 512, lds_addr(tile + 1024 * 4));
            dma16nt<192>(b, lds_addr(tile + 1024 * 6));  // second row, chunk 12 + jj
            dma16nt<448>(b, lds_addr(tile + 1024 * 8));  // second row, chunk 28 + jj
        } else {
            dma16nt<128>(a, lds_addr(tile + 1024 * 1));  // first row, chunk 8 + jj
            dma16nt<384>(a, lds_addr(tile + 1024 * 3));  // first row, chunk 24 + jj
            dma16nt<64>(b, lds_addr(tile + 1024 * 5));   // second row, chunk 4 + jj
            dma16nt<320>(b, lds_addr(tile + 1024 * 7));  // second row, chunk 20 + jj
        }
    } else {
        constexpr int RB = Fmt<KV>::kRowBytes;
        const int G = lane >> 4;
        const int64_t row = ra;
        const uint8_t* src = P.kv + row * RB + 16 * G;
        dma16(src + 64 * HI, lds_addr(tile + 1024 * HI));
        dma16(src + 64 * (HI + 2), lds_addr(tile + 1024 * (HI + 2)));
        const uint8_t* sc = reinterpret_cast<const uint8_t*>(P.kv_scales) + row * MLA_MX_SCALES_PER_ROW + 2 * G;
        if (HI == 0) {
            dma2(sc, lds_addr(tile + Fmt<KV>::kScaleOff));
            if (lane < 16) dma2(sc + 16, lds_addr(tile + Fmt<KV>::kScaleOff + 512));
        } else {
            if (lane < 32) dma16(P.kv + row * RB + 256 + 16 * G, lds_addr(tile + Fmt<KV>::kRopeOff));
            dma2(sc + 8, lds_addr(tile + Fmt<KV>::kScaleOff + 256));
        }
    }
}

template <int KV>
__device__ __forceinline__ void issue_half(const Params& P, int64_t ra, int64_t rb, uint8_t* tile, int lane, int hi) {
    if (hi) issue_half<KV, 1>(P, ra, rb, tile, lane);
    else issue_half<KV, 0>(P, ra, rb, tile, lane);
}

// Byte offset, within a tile, of chunk c of tile row r (bf16, fp8; layout above).
template <int KV>
__device__ __forceinline__ int chunk_offset(int r, int c) {
    if constexpr (KV == MLA_KV_BF16) {
        return 16 * (64 * (2 * (c >> 3) + (r >> 3)) + 8 * ((r & 7) ^ (r >> 3)) + ((c & 7) ^ (r & 7)));
    } else {
        const int p = r >> 1, q = c + 36 * (r & 1);
        return 16 * (64 * (q >> 3) + 8 * (2 * (p & 3) + (p >> 2)) + ((q & 7) ^ (p & 3)));
    }
}

// e8m0 code in bits sh..sh+7 of w -> fp32 scale operand of the scaled
// converts (the code is the exponent field: 2^(code - 127)).
__device__ __forceinline__ float e8m0_scale(uint32_t w, int sh) { return __uint_as_float(((w >> sh) & 0xffu) << 23); }

__device__ __forceinline__ bf16x8 join(bf16x2 a, bf16x2 b, bf16x2 c, bf16x2 d) {
    bf16x8 o;
    o[0] = a[0]; o[1] = a[1]; o[2] = b[0]; o[3] = b[1];
    o[4] = c[0]; o[5] = c[1]; o[6] = d[0]; o[7] = d[1];
    return o;
}

// Eight e4m3fn codes (element k in byte k of lo:hi) -> bf16, exactly.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
    return join(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false),
                __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true),
                __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false),
                __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
}

// Eight e2m1 codes of one block (element 2k in the low nibble of byte k) -> bf16.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t dw, float scale) {
    return join(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, scale, 0),
                __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, scale, 1),
                __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, scale, 2),
                __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, scale, 3));
}

// Score operand: k-step ks of tile t (row r = lane % 16, dims dbase(ks, G)..+7).
template <int KV>
__device__ __forceinline__ bf16x8 qk_operand(const uint8_t* step, int t, int ks, int lane) {
    const uint8_t* tile = step + t * Fmt<KV>::kTileBytes;
    if constexpr (KV == MLA_KV_BF16) {
        // dims 8c .. 8c + 7 are chunk c = 4 ks + G of row r
        return *reinterpret_cast<const bf16x8*>(tile + chunk_offset<KV>(lane & 15, 4 * ks + (lane >> 4)));
    } else if constexpr (KV == MLA_KV_FP8_E4M3) {
        // dims 16c + 8 (ks % 2) .. +7 are half ks % 2 of chunk c = 4 (ks / 2) + G of row r
        const u32x4 w =
            *reinterpret_cast<const u32x4*>(tile + chunk_offset<KV>(lane & 15, 4 * (ks >> 1) + (lane >> 4)));
        return (ks & 1) ? fp8x8_to_bf16(w[2], w[3]) : fp8x8_to_bf16(w[0], w[1]);
    } else {
        // e8m0 block k of row r is byte k & 1 of the dword at scale index 16 (k / 2) + r
        const int G = lane >> 4, r = lane & 15;
        const uint32_t* scl = reinterpret_cast<const uint32_t*>(tile + Fmt<KV>::kScaleOff);
        uint32_t dw, sw;
        int sh;
        if (ks < 16) {  // dims 128 (ks / 4) + 32 G + 8 (ks % 4) ..: block 4 (ks / 4) + G
            dw = *reinterpret_cast<const uint32_t*>(tile + 1024 * (ks >> 2) + 16 * lane + 4 * (ks & 3));
            sw = scl[16 * (2 * (ks >> 2) + (G >> 1)) + r];
            sh = 8 * (G & 1);
        } else {        // RoPE dims 512 + 16 G + 8 (ks - 16) ..: block 16 + G / 2
            dw = *reinterpret_cast<const uint32_t*>(tile + Fmt<KV>::kRopeOff + 16 * (16 * (G >> 1) + r) +
                                                    8 * (G & 1) + 4 * (ks - 16));
            sw = scl[16 * 8 + r];
            sh = 8 * (G >> 1);
        }
        return fp4x8_to_bf16(dw, e8m0_scale(sw, sh));
    }
}

// Byte i of dw (two e2m1 codes of one token) scaled by sc[i] -> bf16x2.
__device__ __forceinline__ void cvt_fp4_bytes(uint32_t dw, f32x4 sc, uint32_t* c) {
    c[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, sc[0], 0));
    c[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, sc[1], 1));
    c[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, sc[2], 2));
    c[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, sc[3], 3));
}

// The value-block scales of one staged MXFP4 step as fp32: fs[t][b][r] =
// 2^(e - 127) for block b (< 16) of token r of tile t. Thread i (of 256)
// converts the dword of tile i / 128, block pair (i / 16) % 8, token i % 16.
__device__ __forceinline__ void convert_scales(const uint8_t* step, float* fs, int i) {
    constexpr int TB = Fmt<MLA_KV_MXFP4>::kTileBytes;
    const int t = i >> 7, p = (i >> 4) & 7, r = i & 15;
    const uint32_t dw = *reinterpret_cast<const uint32_t*>(step + t * TB + Fmt<MLA_KV_MXFP4>::kScaleOff + 4 * (16 * p + r));
    fs[(16 * t + 2 * p) * kTile + r] = e8m0_scale(dw, 0);
    fs[(16 * t + 2 * p + 1) * kTile + r] = e8m0_scale(dw, 8);
}

// Max and sum over the four lane groups of column r (lanes r, r+16, r+32, r+48),
// with the gfx950 lane swaps: permlane32_swap pairs lane l with l ^ 32 and
// permlane16_swap lane l with l ^ 16, so two swaps cover the group.
__device__ __forceinline__ float group_max4(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float group_sum4(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// Eight e4m3fn codes per operand (byte k is k-slot 8G + k, as for bf16).
__device__ __forceinline__ f32x4 mfma32(long a, long b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// fp8 query (the a8w8 path; submission 593653, `_quantize_q_static_into` and
// `_quantize_q_dynamic_into`): the bf16 query is quantised with one per-tensor
// fp32 scale, code = e4m3fn(clamp(q / scale, -448, 448)) rounded to nearest
// even, and the attention uses the decoded query code * scale. The kernels
// keep the codes and fold the scale into the score scale. Dynamic scale:
// max(max |q|, 1e-12) / 448, reduced in two steps (q_amax_kernel writes
// partial maxima, every stage-1 workgroup reduces them).
// ---------------------------------------------------------------------------
constexpr float kFp8Max = 448.0f;

// Two fp32 values -> e4m3fn codes (v_cvt_pk_fp8_f32 rounds to nearest even;
// the inputs are already clamped to the finite range) into half HI of w.
template <bool HI>
__device__ __forceinline__ uint32_t q8_pack2(float a, float b, uint32_t w) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)w, HI);
}

// Division by the query scale, rounded like an IEEE binary32 division
// wherever the e4m3fn code can depend on it. Fast form, for
// 2^-80 <= s <= 2^80: x is first clamped to +-1024 s (a quotient beyond
// +-1024 codes to +-448 either way, and the clamp keeps every intermediate
// finite); then y = x * inv with inv = RN(1 / s), followed by two residual
// corrections y += (x - y s) inv, each residual exact by FMA; a zero quotient
// takes the sign of x. This equals RN(x / s) whenever |x / s| >= 2^-12 (below
// that every quotient codes to a zero of x's sign). Other scales take the
// IEEE division itself. The choice is uniform over the launch.
struct Q8Div {
    float s, inv, lim;
    bool fast;
};
__device__ __forceinline__ Q8Div q8_divider(float s) {
    return {s, 1.0f / s, 1024.0f * s, s >= 0x1p-80f && s <= 0x1p80f};
}
template <bool FAST>
__device__ __forceinline__ float q8_div(float x, const Q8Div& d) {
    if constexpr (!FAST) {
        return x / d.s;
    } else {
        x = __builtin_amdgcn_fmed3f(x, -d.lim, d.lim);
        const float y0 = x * d.inv;
        float y = fmaf(fmaf(-y0, d.s, x), d.inv, y0);
        y = fmaf(fmaf(-y, d.s, x), d.inv, y);
        return __uint_as_float(__float_as_uint(y) | (__float_as_uint(x) & 0x80000000u));
    }
}

// Eight bf16 query elements -> eight e4m3fn codes (element k in byte k).
template <bool FAST>
__device__ __forceinline__ u32x2 q8_codes8(bf16x8 x, const Q8Div& d) {
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = __builtin_amdgcn_fmed3f(q8_div<FAST>((float)x[e], d), -kFp8Max, kFp8Max);
    u32x2 c;
    c[0] = q8_pack2<true>(y[2], y[3], q8_pack2<false>(y[0], y[1], 0u));
    c[1] = q8_pack2<true>(y[6], y[7], q8_pack2<false>(y[4], y[5], 0u));
    return c;
}

// Scales outside the fast form's range: the same codes through the IEEE
// division, reading the query from src (global memory) again. Kept out of
// line so that its instructions are never fetched in the common case.
__device__ __noinline__ void q8_quantise_slow(const __bf16* src, int tid, int step, int n, float scale, uint8_t* dst) {
    const Q8Div dv = q8_divider(scale);
    for (int k = tid; k < n; k += step)
        *reinterpret_cast<u32x2*>(dst + 8 * k) = q8_codes8<false>(*reinterpret_cast<const bf16x8*>(src + 8 * k), dv);
}

// Codes of query groups tid, tid + step, ... (< n) into dst (8 bytes per
// group); g holds this thread's groups, src is the query in global memory.
template <int PER>
__device__ __forceinline__ void q8_quantise(const bf16x8 (&g)[PER], const __bf16* src, int tid, int step, int n,
                                            float scale, uint8_t* dst) {
    const Q8Div dv = q8_divider(scale);
    if (__builtin_amdgcn_readfirstlane((int)dv.fast)) {
#pragma unroll
        for (int k = 0; k < PER; ++k)
            if (tid + k * step < n) *reinterpret_cast<u32x2*>(dst + 8 * (tid + k * step)) = q8_codes8<true>(g[k], dv);
    } else {
        q8_quantise_slow(src, tid, step, n, scale, dst);
    }
}

// Dynamic scale from the partial maxima: `part` is this thread's partial
// (0 for threads beyond the count); red is 4 floats of LDS. Contains a
// workgroup barrier.
__device__ __forceinline__ float q8_dynamic_scale(float part, float* red, int tid) {
    float m = part;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    return fmaxf(m, 1e-12f) / kFp8Max;
}

constexpr int kHalfK = kKSteps / 2;            // 9 score k-steps per wave
constexpr int kWaveBlocks = kBlocks / kWaves;  // 8 output blocks (128 columns) per wave

// Partial scores of one wave: tile t, score k-steps kHalfK * HF .. +kHalfK-1.
// Result: lane (G, r) holds S^T[token 4G+i of tile t][head r] over those dims.
// With an fp8 query on the fp8 cache (QOp = long) the cache codes enter the
// MFMA as they are: the eight bytes of row r at dims dbase(ks, G)..+7.
template <int KV, int HF, typename QOp>
__device__ __forceinline__ f32x4 qk_partial(const uint8_t* step, const QOp (&qB)[kHalfK], int t, int lane) {
    f32x4 e0 = {0.f, 0.f, 0.f, 0.f}, e1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kHalfK; ++j) {
        const int ks = kHalfK * HF + j;
        QOp k;
        if constexpr (__is_same(QOp, long)) {
            static_assert(KV == MLA_KV_FP8_E4M3, "fp8 score operands need the fp8 cache");
            k = *reinterpret_cast<const long*>(step + t * Fmt<KV>::kTileBytes +
                                               chunk_offset<KV>(lane & 15, 4 * (ks >> 1) + (lane >> 4)) + 8 * (ks & 1));
        } else {
            k = qk_operand<KV>(step, t, ks, lane);
        }
        if (j & 1) e1 = mfma32(k, qB[j], e1);
        else e0 = mfma32(k, qB[j], e0);
    }
    return e0 + e1;
}

// fp8 query on the MXFP4 cache: the scores run on the MX-scaled MFMA
// v_mfma_scale_f32_16x16x128_f8f6f4 with the cache's e2m1 codes and e8m0
// block scales as operand A and the query's e4m3fn codes (scale 1) as operand
// B, so no cache code is converted. Operand layouts of this instruction on
// gfx950 (16 x 128 per operand, lane group G = lane / 16, row / column
// lane % 16): an e2m1 operand holds k = 32 G .. 32 G + 31, element i in
// nibble i (low nibble first); an e4m3 operand holds k = 16 G + i in bytes
// 0-15 and k = 64 + 16 G + i in bytes 16-31; the A scale of lane (G, r) is
// the e8m0 of (row r, k block G). A score tile is five such products: the
// four 128-dim blocks of the no-RoPE dims (block u is exactly code load u of
// the staged tile, 16 bytes per lane) and the 64 RoPE dims, zero-padded to
// 128. Wave half 0 takes blocks 0-2, half 1 block 3 and the RoPE block.
__device__ __forceinline__ f32x4 mfma_mx(i32x8 a, i32x8 b, int scale_a, f32x4 c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 0, scale_a, 0, 127);
}

// e8m0 scale code of block bi (0..17) of tile row r, from the staged scale
// dwords (codes 2p, 2p + 1 of row r in the low half of the dword at
// kScaleOff + 256 (p / 4) + 4 (16 (p % 4) + r)).
__device__ __forceinline__ int mx_scale_code(const uint8_t* tile, int bi, int r) {
    const int p = bi >> 1;
    return tile[Fmt<MLA_KV_MXFP4>::kScaleOff + 256 * (p >> 2) + 4 * (16 * (p & 3) + r) + (bi & 1)];
}

template <int HF>
__device__ __forceinline__ f32x4 qk_partial_mx(const uint8_t* step, const i32x8 (&qm)[3], int t, int lane) {
    const uint8_t* tile = step + t * Fmt<MLA_KV_MXFP4>::kTileBytes;
    const int G = lane >> 4, r = lane & 15;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < (HF ? 2 : 3); ++j) {
        const int u = HF ? 3 + j : j;
        i32x8 a = {0, 0, 0, 0, 0, 0, 0, 0};
        int sc = 127;
        if (u < 4) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(tile + 1024 * u + 16 * lane);
            a[0] = (int)w[0]; a[1] = (int)w[1]; a[2] = (int)w[2]; a[3] = (int)w[3];
            sc = mx_scale_code(tile, 4 * u + G, r);
        } else if (G < 2) {  // RoPE dims 512 + 32 G ..: lanes 0..31 of the RoPE load
            const u32x4 w = *reinterpret_cast<const u32x4*>(tile + Fmt<MLA_KV_MXFP4>::kRopeOff + 16 * lane);
            a[0] = (int)w[0]; a[1] = (int)w[1]; a[2] = (int)w[2]; a[3] = (int)w[3];
            sc = mx_scale_code(tile, 16 + G, r);
        }
        acc = mfma_mx(a, qm[j], sc, acc);
    }
    return acc;
}

// bf16 query on the MXFP4 cache: the scores also run on the MX-scaled MFMA,
// straight from the staged e2m1 codes, with the query split into two e4m3fn
// code sets that carry their own e8m0 scale per 32-element block:
//     hi = RNE(q / 2^eh),  lo = RNE((q - hi 2^eh) / 2^el),
// eh = floor(log2 max|q|) - 7 over the block and el likewise over the
// residuals (so every scaled value lies below 256, inside the e4m3fn range;
// the residual q - hi 2^eh is exact in fp32). hi 2^eh + lo 2^el equals q
// exactly for the elements within about 2^-10 of their block's largest
// magnitude (four significant bits each, eight together) and differs from
// q by less than 2^-20 of it for the rest, far below the rounding of the
// softmax weights to bf16. No cache code is converted for the scores.
// e8m0 code c of the scale 2^(floor(log2 a) - 7) for a >= 0 (1 for a < 2^-119).
__device__ __forceinline__ int split_scale_code(float a) {
    return max(1, (int)((__float_as_uint(a) >> 23) & 0xffu) - 7);
}
__device__ __forceinline__ float pow2_code(int c) { return __uint_as_float((uint32_t)c << 23); }  // 2^(c - 127)

// The query row's two code sets: thread tid splits the 8-element groups tid,
// tid + 256, ... (< kQGroups) held in g; four consecutive groups (threads 4m
// .. 4m + 3) form one 32-element block. hi_dst / lo_dst receive the codes as
// [16][576] bytes followed by the e8m0 codes [16][18].
template <int PER>
__device__ __forceinline__ void q_split_quantise(const bf16x8 (&g)[PER], int tid, uint8_t* hi_dst, uint8_t* lo_dst) {
    constexpr int kGroups = kHeads * kDqk / 8;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int grp = tid + k * kThreads;
        if (k * kThreads + (tid & ~63) >= kGroups) continue;  // whole waves: the block's four lanes stay together
        float x[8], amax = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            x[e] = (float)g[k][e];
            amax = fmaxf(amax, fabsf(x[e]));
        }
        amax = fmaxf(amax, __shfl_xor(amax, 1));
        amax = fmaxf(amax, __shfl_xor(amax, 2));
        const int ch = split_scale_code(amax);
        const float dh = pow2_code(254 - ch), uh = pow2_code(ch);  // 2^-eh, 2^eh
        u32x2 hc;
        hc[0] = q8_pack2<true>(x[2] * dh, x[3] * dh, q8_pack2<false>(x[0] * dh, x[1] * dh, 0u));
        hc[1] = q8_pack2<true>(x[6] * dh, x[7] * dh, q8_pack2<false>(x[4] * dh, x[5] * dh, 0u));
        float hv[8];
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            hv[4 * w + 0] = __builtin_amdgcn_cvt_f32_fp8((int)hc[w], 0);
            hv[4 * w + 1] = __builtin_amdgcn_cvt_f32_fp8((int)hc[w], 1);
            hv[4 * w + 2] = __builtin_amdgcn_cvt_f32_fp8((int)hc[w], 2);
            hv[4 * w + 3] = __builtin_amdgcn_cvt_f32_fp8((int)hc[w], 3);
        }
        float rr[8], ramax = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            rr[e] = x[e] - hv[e] * uh;  // exact: hi holds the leading bits of x
            ramax = fmaxf(ramax, fabsf(rr[e]));
        }
        ramax = fmaxf(ramax, __shfl_xor(ramax, 1));
        ramax = fmaxf(ramax, __shfl_xor(ramax, 2));
        const int cl = split_scale_code(ramax);
        const float dl = pow2_code(254 - cl);
        u32x2 lc;
        lc[0] = q8_pack2<true>(rr[2] * dl, rr[3] * dl, q8_pack2<false>(rr[0] * dl, rr[1] * dl, 0u));
        lc[1] = q8_pack2<true>(rr[6] * dl, rr[7] * dl, q8_pack2<false>(rr[4] * dl, rr[5] * dl, 0u));
        if (grp < kGroups) {
            *reinterpret_cast<u32x2*>(hi_dst + 8 * grp) = hc;
            *reinterpret_cast<u32x2*>(lo_dst + 8 * grp) = lc;
            if ((tid & 3) == 0) {
                hi_dst[kHeads * kDqk + (grp >> 2)] = (uint8_t)ch;
                lo_dst[kHeads * kDqk + (grp >> 2)] = (uint8_t)cl;
            }
        }
    }
}

__device__ __forceinline__ f32x4 mfma_mx2(i32x8 a, i32x8 b, int scale_a, int scale_b, f32x4 c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 0, scale_a, 0, scale_b);
}

// Partial scores of one wave with the split query: qm[j] / qm[3 + j] are the
// hi / lo B operands of this wave's block j, qs[j] / qs[3 + j] their e8m0
// codes for (head r, k block G). The two pieces accumulate in separate chains.
template <int HF>
__device__ __forceinline__ f32x4 qk_partial_mx2(const uint8_t* step, const i32x8 (&qm)[6], const int (&qs)[6], int t,
                                                int lane) {
    const uint8_t* tile = step + t * Fmt<MLA_KV_MXFP4>::kTileBytes;
    const int G = lane >> 4, r = lane & 15;
    f32x4 ah = {0.f, 0.f, 0.f, 0.f}, al = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < (HF ? 2 : 3); ++j) {
        const int u = HF ? 3 + j : j;
        i32x8 a = {0, 0, 0, 0, 0, 0, 0, 0};
        int sc = 127;
        if (u < 4) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(tile + 1024 * u + 16 * lane);
            a[0] = (int)w[0]; a[1] = (int)w[1]; a[2] = (int)w[2]; a[3] = (int)w[3];
            sc = mx_scale_code(tile, 4 * u + G, r);
        } else if (G < 2) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(tile + Fmt<MLA_KV_MXFP4>::kRopeOff + 16 * lane);
            a[0] = (int)w[0]; a[1] = (int)w[1]; a[2] = (int)w[2]; a[3] = (int)w[3];
            sc = mx_scale_code(tile, 16 + G, r);
        }
        ah = mfma_mx2(a, qm[j], sc, qs[j], ah);
        al = mfma_mx2(a, qm[3 + j], sc, qs[3 + j], al);
    }
    return ah + al;
}

// Query operand type: bf16 (also the decoded fp8 query codes, which bf16
// holds exactly), raw e4m3fn codes when both operands are fp8, or the
// MX-scaled MFMA's e4m3fn operand on the MXFP4 cache (the fp8 query's codes,
// or the two code sets a bf16 query is split into).
template <int KV, int QF>
struct QOperand { using T = bf16x8; };
template <>
struct QOperand<MLA_KV_FP8_E4M3, 1> { using T = long; };
template <>
struct QOperand<MLA_KV_MXFP4, 1> { using T = i32x8; };
template <>
struct QOperand<MLA_KV_MXFP4, 0> { using T = i32x8; };

// NB output blocks of 16 columns: o[j][i] is head 4G+i of block j's column
// r (the wave's blocks: kWaveBlocks * wave + j with one query row per
// workgroup, 2 kWaveBlocks * (wave % 2) + j with two).
template <int NB = kWaveBlocks>
struct WaveAccT {
    f32x4 o[NB];
    float m;  // running max of head r (log2 units), the same in every lane (and wave of the row)
    float l;  // this lane's share of head r's softmax denominator
};
using WaveAcc = WaveAccT<>;

// This wave's value-operand data of one staged step, read from LDS ahead of
// the softmax so that the read latency overlaps it (converted afterwards).
template <int KV>
struct PvRaw;
template <>
struct PvRaw<MLA_KV_BF16> {
    i16x4 lo[kWaveBlocks], hi[kWaveBlocks];
};
template <>
struct PvRaw<MLA_KV_FP8_E4M3> {
    i32x2 w[kWaveBlocks];
};
template <>
struct PvRaw<MLA_KV_MXFP4> {
    i32x2 w[kWaveBlocks / 2];
    f32x4 s0[kWaveBlocks / 2], s1[kWaveBlocks / 2];
};

// Per-lane byte offsets (within a staged step) of this wave's value reads,
// taken once per workgroup; pv_load adds the step base and a compile-time
// per-block part, which the LDS reads take as an immediate offset.
//   fp8 / MXFP4 (ds_read_b64_tr_b8): row i of the transposed 8 x 16-byte block
//     is token tau(G, i); lanes 2i and 2i+1 supply its bytes 0-7 and 8-15.
//     Block c's 16 (fp8) or 32 (MXFP4, two codes a byte) columns are chunk c
//     of the token's row: fp8 a[j] for block 8 wave + j (the row's XOR and
//     pair placement make these 8 separate offsets); MXFP4 a[0] + 256 j.
//   bf16 (ds_read_b64_tr_b16, two reads): row i of each transposed 4 x 16
//     block is token tau(G, i) (first read, tile 0) or tau(G, 4 + i) (second
//     read, the same row of tile 1); lanes 4i..4i+3 supply its 32 bytes, the
//     chunks 2c and 2c + 1 of block c = 8 wave + j: a[j % 4] + 2048 (j / 4).
template <int KV>
struct PvOff {
    int a[KV == MLA_KV_FP8_E4M3 ? 8 : KV == MLA_KV_BF16 ? 4 : 1];
};

template <int KV>
__device__ __forceinline__ PvOff<KV> pv_lane_offsets(int lane, int wave) {
    const int G = lane >> 4, j = lane & 15;
    PvOff<KV> o;
    if constexpr (KV == MLA_KV_FP8_E4M3) {
        const int tk = tau(G, j >> 1), t = tk >> 4, r = tk & 15;
#pragma unroll
        for (int b = 0; b < 8; ++b)
            o.a[b] = t * Fmt<KV>::kTileBytes + chunk_offset<KV>(r, 8 * wave + b) + 8 * (j & 1);
    } else if constexpr (KV == MLA_KV_BF16) {
        const int i = j >> 2, q = j & 3, r = 4 * G + i;
        // chunk 2 (8 wave + b) + q / 2 of row r: 2048 (b / 4) apart for b and b + 4
#pragma unroll
        for (int b = 0; b < 4; ++b) o.a[b] = chunk_offset<KV>(r, 2 * (8 * wave + b) + (q >> 1)) + 8 * (q & 1);
    } else {
        const int tk = tau(G, j >> 1);
        o.a[0] = (tk >> 4) * Fmt<KV>::kTileBytes + 16 * (tk & 15) + 8 * (j & 1) + 1024 * wave;
    }
    return o;
}

template <int KV>
__device__ __forceinline__ void pv_load(const uint8_t* step, const float* fs, const PvOff<KV>& off, int lane,
                                        int wave, PvRaw<KV>& v) {
    if constexpr (KV == MLA_KV_FP8_E4M3) {
#pragma unroll
        for (int j = 0; j < kWaveBlocks; ++j)
            v.w[j] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(step + off.a[j]));
    } else if constexpr (KV == MLA_KV_BF16) {
#pragma unroll
        for (int j = 0; j < kWaveBlocks; ++j) {
            const uint8_t* a0 = step + off.a[j & 3] + 2048 * (j >> 2);
            v.lo[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)a0);
            v.hi[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0 + Fmt<KV>::kTileBytes));
        }
    } else {
        // MX block b = 4 wave + j: codes + 256 j; scales fs[t][b][4G..4G+3] (as f32x4: 4 (16 t + b) + G)
        const uint8_t* vb = step + off.a[0];
        const int G = lane >> 4;
        const f32x4* f = reinterpret_cast<const f32x4*>(fs) + 16 * wave + G;
#pragma unroll
        for (int j = 0; j < kWaveBlocks / 2; ++j) {
            v.w[j] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vb + 256 * j));
            v.s0[j] = f[4 * j];
            v.s1[j] = f[64 + 4 * j];
        }
    }
}

// Value operand of block kWaveBlocks * wave + j (bf16 / fp8): lane (G, n)
// holds column 16 (kWaveBlocks * wave + j) + n of the tokens tau(G, 0..7).
template <int KV>
__device__ __forceinline__ bf16x8 pv_convert(const PvRaw<KV>& v, int j) {
    if constexpr (KV == MLA_KV_FP8_E4M3) return fp8x8_to_bf16((uint32_t)v.w[j][0], (uint32_t)v.w[j][1]);
    else return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v.lo[j], v.hi[j], 0, 1, 2, 3, 4, 5, 6, 7));
}

// Value operands of MX block b = (kWaveBlocks / 2) * wave + j: lane (G, n) holds
// byte n of the block for tokens tau(G, 0..7), i.e. columns 32b + 2n (even)
// and 32b + 2n + 1 (odd), each token scaled by its own e8m0 code.
__device__ __forceinline__ void pv_convert_fp4(const PvRaw<MLA_KV_MXFP4>& v, int j, bf16x8& even, bf16x8& odd) {
    uint32_t c[8];
    cvt_fp4_bytes((uint32_t)v.w[j][0], v.s0[j], c);
    cvt_fp4_bytes((uint32_t)v.w[j][1], v.s1[j], c + 4);
    u32x4 e, o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        e[k] = __builtin_amdgcn_perm(c[2 * k + 1], c[2 * k], 0x05040100u);  // low halves: even columns
        o[k] = __builtin_amdgcn_perm(c[2 * k + 1], c[2 * k], 0x07060302u);  // high halves: odd columns
    }
    even = __builtin_bit_cast(bf16x8, e);
    odd = __builtin_bit_cast(bf16x8, o);
}

// O += P . V for this wave's blocks from the raw operand data.
template <int KV>
__device__ __forceinline__ void pv_mma(const PvRaw<KV>& v, bf16x8 pa, WaveAcc& a) {
    if constexpr (KV == MLA_KV_MXFP4) {
#pragma unroll
        for (int j = 0; j < kWaveBlocks / 2; ++j) {
            bf16x8 ev, od;
            pv_convert_fp4(v, j, ev, od);
            a.o[2 * j] = mfma32(pa, ev, a.o[2 * j]);
            a.o[2 * j + 1] = mfma32(pa, od, a.o[2 * j + 1]);
        }
    } else {
#pragma unroll
        for (int j = 0; j < kWaveBlocks; ++j) a.o[j] = mfma32(pa, pv_convert<KV>(v, j), a.o[j]);
    }
}

// Online softmax of one step's 32 scores; returns P (bf16) in the A-operand
// layout of the P . V product. s[t]: full scores of tile t (the same in all
// four waves, so every wave takes the same rescale decisions and keeps the
// same m and l).
template <int NB = kWaveBlocks>
__device__ __forceinline__ bf16x8 softmax_step(const f32x4 (&s)[2], float qk_scale, int nvalid, int lane,
                                               WaveAccT<NB>& a) {
    const int G = lane >> 4;
    float x[8];  // raw scores; scaled below inside the exponent
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = s[j >> 2][j & 3];
    if (nvalid < kStepTokens) {  // a partial last step: padded tokens carry no weight
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (tau(G, j) >= nvalid) x[j] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    mx = group_max4(mx) * qk_scale;  // qk_scale > 0, so this is the max of the scaled scores
    const float m_new = fmaxf(a.m, mx);
    if (__any(m_new > a.m + kRescaleThresh)) {
        const float alpha = (a.m == -INFINITY) ? 0.f : fast_exp2(a.m - m_new);
        a.m = m_new;
        a.l *= alpha;
        float al[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * G + i);
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) a.o[j][i] *= al[i];
    }
    float p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = fast_exp2(fmaf(x[j], qk_scale, -a.m));
    a.l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    bf16x8 pa;
#pragma unroll
    for (int j = 0; j < 8; ++j) pa[j] = (__bf16)p[j];
    return pa;
}

// Wait until this wave's own LDS-DMA loads of all but the last `groups` issued
// steps have landed. The wave issues half `hi` of one tile per step.
template <int KV, int N = 0>
__device__ __forceinline__ void wait_own(int groups, int hi) {
    constexpr int k0 = Fmt<KV>::ops(0), k1 = Fmt<KV>::ops(1);
    static_assert(N * k0 <= 63 && N * k1 <= 63, "vmcnt holds at most 63");
    if constexpr (N < Fmt<KV>::kRing - 2) {
        if (groups > N) {
            wait_own<KV, N + 1>(groups, hi);
            return;
        }
    }
    if (hi) wait_vmcnt<N * k1>();
    else wait_vmcnt<N * k0>();
}

// Wait until at most X + e ops(hi) of this wave's vector memory operations
// are outstanding: those issued after the ones waited for are X single
// operations and the gathers of e steps (e < kRing).
template <int KV, int X, int E = 0>
__device__ __forceinline__ void wait_behind(int e, int hi) {
    constexpr int k0 = Fmt<KV>::ops(0), k1 = Fmt<KV>::ops(1);
    static_assert(X + E * k0 <= 63 && X + E * k1 <= 63, "vmcnt holds at most 63");
    if constexpr (E < Fmt<KV>::kRing - 1) {
        if (e > E) {
            wait_behind<KV, X, E + 1>(e, hi);
            return;
        }
    }
    if (hi) wait_vmcnt<X + E * k1>();
    else wait_vmcnt<X + E * k0>();
}

constexpr int kQGroups = kHeads * kDqk / 8;                   // 8-element groups of one query row
constexpr int kQPer = (kQGroups + kThreads - 1) / kThreads;  // of them per thread (fp8 query)
template <int KV>
constexpr int kIdxPer = Fmt<KV>::kIdxWindow / kThreads;      // index entries per thread and window
// Byte offset, in the score exchange buffer, of the staged page entries of a
// first index window (dma_pages); its first 64 bytes stay free for the fp8
// query's scale reduction.
constexpr int kPageStageOff = 64;

// Entries [w0, w0 + n) of a sequence whose kv_indices entries start at
// `base`, as cache rows: thread tid takes entry w0 + tid + k * kThreads into
// iv[k] (0 at or beyond n, never used). Token j is row indices[base + j]
// (page size 1), else row indices[base + j / page_size] * page_size +
// j % page_size.
template <int KV>
__device__ __forceinline__ void load_idx(const Params& P, int base, int w0, int n, int32_t (&iv)[kIdxPer<KV>]) {
    const int tid = threadIdx.x, ps = P.page_size;
#pragma unroll
    for (int k = 0; k < kIdxPer<KV>; ++k) {
        const int j = w0 + tid + k * kThreads;
        iv[k] = 0;
        if (tid + k * kThreads < n) {
            if (ps == 1) {
                iv[k] = P.indices[base + j];
            } else {
                const int pg = j / ps;
                iv[k] = P.indices[base + pg] * ps + (j - pg * ps);
            }
        }
    }
}

// Page size 1: entries [first, first + n) of kv_indices (n >= 1) straight
// into the LDS index window idx, entry first + i at idx[i]; the threads past
// n re-read entry first + n - 1 into idx[n..], which is never used.
template <int KV>
__device__ __forceinline__ void dma_idx(const Params& P, int first, int n, int32_t* idx) {
    const int tid = threadIdx.x, wave0 = tid & ~63;
#pragma unroll
    for (int k = 0; k < kIdxPer<KV>; ++k)
        dma4(P.indices + first + min(tid + k * kThreads, n - 1), lds_addr(idx + k * kThreads + wave0));
}

// Page size > 1: the page entries [first, first + np) of kv_indices (1 <=
// np <= 1024) into the page staging area of the score exchange buffer,
// entry first + i at word i; run_wg expands them into the index window. The
// same number of LDS-DMA operations per thread as dma_idx (loads k and k + 4
// write the same words), so the waits that count dma_idx's hold for it.
template <int KV>
__device__ __forceinline__ void dma_pages(const Params& P, int first, int np, uint8_t* smem) {
    static_assert(kIdxPer<KV> == 4 || kIdxPer<KV> == 8, "dma_idx's operation count");
    static_assert(kPageStageOff + 4 * 4 * kThreads <= 2 * Layout<KV>::kSbufBytes,
                  "the page staging fits the exchange buffer");
    int32_t* st = reinterpret_cast<int32_t*>(smem + Layout<KV>::kSbufOff + kPageStageOff);
    const int tid = threadIdx.x, wave0 = tid & ~63;
#pragma unroll
    for (int k = 0; k < kIdxPer<KV>; ++k) {
        const int i = tid + (k & 3) * kThreads;
        dma4(P.indices + first + min(i, np - 1), lds_addr(st + (k & 3) * kThreads + wave0));
    }
}

// Row of prologue token j (< n) of this wave's tile half: the row a
// contiguous cache holds (first + j, tokens past n repeat the last one, as
// issue_step does), clamped below the cache size.
__device__ __forceinline__ int64_t early_row(const Params& P, int64_t first, int j, int n) {
    return min(first + min(j, n - 1), P.kv_rows - 1);
}

// A known cache size: the gathers of the first D steps of a range whose
// kv_indices entries are guessed to be first, first + 1, ... (the rows a
// contiguous cache gives the sequence), issued with the query and index
// requests so that the first rows arrive in the same memory round trip (split
// plans with equal lengths, and every share of the persistent grid). run_wg
// keeps them only where kv_indices confirms every row.
template <int KV>
__device__ __forceinline__ void issue_early(const Params& P, uint8_t* smem, int64_t first, int n) {
    using L = Layout<KV>;
    constexpr int R = Fmt<KV>::kRing, D = R - 1;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int tile = wave & 1, hf = wave >> 1;
    const int2 tr = lane_tile_rows<KV>(lane, hf);
    const int nsteps = (n + kStepTokens - 1) / kStepTokens;
#pragma unroll
    for (int d = 0; d < D; ++d)
        if (d < nsteps)
            issue_half<KV>(P, early_row(P, first, d * kStepTokens + kTile * tile + tr.x, n),
                           early_row(P, first, d * kStepTokens + kTile * tile + tr.y, n),
                           smem + (d % R) * L::kStepBytes + tile * Fmt<KV>::kTileBytes, lane, hf);
}

// The bf16 query row b into ring slot D with LDS-DMA (bf16 and fp8 caches,
// one row per workgroup), laid out in score-operand order: the 16 bytes that
// lane (G, r) of a wave of half hf takes as its k-step kHalfK hf + j operand
// sit at 1024 (kHalfK hf + j) + 16 lane, so run_wg reads Q^T with one linear
// ds_read_b128 per k-step. Issued first at entry, ahead of the index window
// and the early gathers, and waited for with an exact count (run_wg), so that
// the wait for Q leaves those in flight; the compiler's own wait for query
// registers loaded from memory would drain them, as it does not see the DMA
// loads. Waves 0 and 1 issue five loads, waves 2 and 3 four.
template <int KV>
__device__ __forceinline__ void dma_query(const Params& P, int b, uint8_t* smem) {
    constexpr int D = Fmt<KV>::kRing - 1;
    static_assert(Layout<KV>::kStepBytes >= kHeads * kDqk * 2, "a ring slot holds the bf16 query");
    uint8_t* qs = smem + D * Layout<KV>::kStepBytes;
    const int tid = threadIdx.x, lane = tid & 63, G = lane >> 4, r = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const __bf16* qrow = P.q + ((int64_t)b * kHeads + r) * kDqk;
#pragma unroll
    for (int m = 0; m < 5; ++m) {
        const int blk = 4 * m + wave;  // k-step block kHalfK hf + j
        if (blk < 2 * kHalfK) dma16(qrow + dbase<KV>(blk, G), lds_addr(qs + 1024 * blk));
    }
}

// One query row in registers, with the scales read alongside it.
//   bf16 query (bf16 and fp8 caches): this wave's half of Q^T, straight in
//   the score operand layout.
//   fp8 query, and bf16 query on the MXFP4 cache: thread tid holds the
//   8-element groups tid, tid + 256, ... of the row's 16 x 576 query,
//   quantised (fp8 query) or split into two code sets (bf16 query on MXFP4)
//   once per workgroup later on.
// NT = 2 (two query rows per workgroup, bf16 cache and query): wave w holds
// the Q^T operands of row w / 2 over all 18 score k-steps, qB2[h][j] those of
// k-step kHalfK h + j.
template <int KV, int QF, int NT = 1>
struct QueryRegs {
    static_assert(NT == 1 || (NT == 2 && KV == MLA_KV_BF16 && !QF), "two rows per workgroup: bf16 only");
    static constexpr bool kSplit = KV == MLA_KV_MXFP4 && !QF;  // split query on the MX-scaled MFMA
    typename QOperand<KV, QF>::T qB[NT == 2 ? 1 : KV == MLA_KV_MXFP4 ? (QF ? 3 : 6) : kHalfK];
    bf16x8 qB2[NT == 2 ? 2 : 1][NT == 2 ? kHalfK : 1];
    bf16x8 qg[(QF || kSplit) ? kQPer : 1];
    int qsc[kSplit ? 6 : 1];  // split query: e8m0 codes of qB (head r, k block G)
    float kv_scale, q_scale, q_part;
};

// The scales of QueryRegs alone, for a query that comes through LDS
// (dma_query); read as scalar loads.
template <int KV, int QF>
__device__ __forceinline__ void query_scales(const Params& P, QueryRegs<KV, QF>& q) {
    static_assert(!QF, "the fp8 query reads its scale with the query");
    q.kv_scale = 1.0f;
    if constexpr (KV == MLA_KV_FP8_E4M3)
        q.kv_scale = __builtin_bit_cast(float, ld_scalar(reinterpret_cast<const int32_t*>(P.kv_scales), 0));
    q.q_scale = 1.0f;
    q.q_part = 0.0f;
}

template <int KV, int QF>
__device__ __forceinline__ void load_query(const Params& P, int b, QueryRegs<KV, QF>& q) {
    const int tid = threadIdx.x, lane = tid & 63, G = lane >> 4, r = lane & 15;
    const int hf = __builtin_amdgcn_readfirstlane(tid >> 6) >> 1;
    const __bf16* qseq = P.q + (int64_t)b * kHeads * kDqk;
    q.kv_scale = 1.0f;
    if constexpr (KV == MLA_KV_FP8_E4M3) q.kv_scale = *reinterpret_cast<const float*>(P.kv_scales);
    q.q_scale = 1.0f;
    q.q_part = 0.0f;
    if constexpr (QF || QueryRegs<KV, QF>::kSplit) {
#pragma unroll
        for (int k = 0; k < kQPer; ++k) {
            q.qg[k] = bf16x8{};
            if (tid + k * kThreads < kQGroups) q.qg[k] = *reinterpret_cast<const bf16x8*>(qseq + 8 * (tid + k * kThreads));
        }
        if constexpr (QF) {
            if (P.q_amax) q.q_part = tid < P.q_amax_n ? P.q_amax[tid] : 0.0f;
            else q.q_scale = *P.q_scale;
        }
    } else {
        const __bf16* qrow = qseq + r * kDqk;
#pragma unroll
        for (int j = 0; j < kHalfK; ++j)
            q.qB[j] = *reinterpret_cast<const bf16x8*>(qrow + dbase<KV>(kHalfK * hf + j, G));
    }
}

// Two query rows per workgroup: this wave's row is `row` (wave / 2 picks
// which of the pair the caller passes); all 18 k-steps of its Q^T.
__device__ __forceinline__ void load_query_pair(const Params& P, int row, QueryRegs<MLA_KV_BF16, 0, 2>& q) {
    const int lane = threadIdx.x & 63, G = lane >> 4, r = lane & 15;
    const __bf16* qrow = P.q + ((int64_t)row * kHeads + r) * kDqk;
    q.kv_scale = 1.0f;
    q.q_scale = 1.0f;
    q.q_part = 0.0f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < kHalfK; ++j)
            q.qB2[h][j] = *reinterpret_cast<const bf16x8*>(qrow + dbase<MLA_KV_BF16>(kHalfK * h + j, G));
}

// Buffer resource of `bytes` bytes at p for the raw buffer loads of the
// merge (raw buffer, 32-bit data words; loads past the end return 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t merge_rsrc(const float* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), 0, bytes, 0x00020000);
}
// Cache-policy bits of the merge's loads: sc0 | sc1, the system-coherent
// load, which is not served from a possibly stale line of this XCD's L2 (the
// partials were written by workgroups on other XCDs).
constexpr int kCoherentLoad = 0x11;

// The last-arriving split's merge of S = 5..8 bf16 partials [column][head]
// (the formula of merge_if_last) on the MFMA. For 16 output columns the sum
// over slots s of w_s,h x_s[c][h] is a matrix product: the partials' chunks
// as a [column] x [slot, head'] matrix (one 16-byte chunk, 8 heads' of one
// slot, is the A-operand k-block of a lane) times the [slot, head'] x [head]
// matrix that holds w_s,h where head' = h and zero elsewhere
// (v_mfma_f32_16x16x32_bf16: two slots per k-step, four k-steps). The products
// are exact and summed in fp32; each weight enters as two bf16 terms, hi = w
// rounded and lo = w - hi rounded, which carry it to about 2^-17 relative.
// Every lane forms the weights of its head from that head's lse values itself
// (no LDS, no barrier), and all loads are issued in one round, lse first.
// Lane (G, r) of wave w holds row r of the A tiles, column
// 128 w + 32 (r / 4) + 4 t + r % 4 of tile t, chunk half G % 2 of slot
// 2 ks + G / 2 at k-step ks; the products then leave it output columns
// 128 w + 32 G .. +31 of head r, written as four 16-byte pieces.
__device__ void merge_bf16(const Params& P, int row, int S) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int G = lane >> 4, r = lane & 15;
    // Every load is issued, without a branch on S: the slots sl >= S lie past
    // the end of either buffer, so theirs return zero without touching memory
    // (their lse is taken as -inf below). A load under a branch on S would
    // sit behind a wait for the loads before it.
    // l[k] is the lse of slot k ^ s1 (s1 = G / 2), so that e[2 ks] below is
    // always the weight of this lane's slot 2 ks + s1 (no lane-dependent index)
    const int s1 = G >> 1;
    const __amdgpu_buffer_rsrc_t rl = merge_rsrc(P.part_lse + (int64_t)row * S * kHeads, S * kHeads * 4);
    float l[kMaxMergeSplitsBf16];
#pragma unroll
    for (int k = 0; k < kMaxMergeSplitsBf16; ++k)
        l[k] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rl, 4 * ((k ^ s1) * kHeads + r), 0, kCoherentLoad));
    const __amdgpu_buffer_rsrc_t ro = merge_rsrc(P.part_o + (int64_t)row * S * kHeads * kDv, S * kHeads * kDv * 4);
    const int cA = 128 * wave + 32 * (r >> 2) + (r & 3);  // this lane's A column in tile 0
    bf16x8 x[8][4];                                         // [tile][k-step]
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            x[t][ks] = __builtin_bit_cast(
                bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                            ro, 4 * (2 * ks + s1) * kHeads * kDv + 16 * (2 * (cA + 4 * t) + (G & 1)), 0,
                            kCoherentLoad));
    // w_s,r = exp(lse_s - M) / sum_s exp(lse_s - M); empty splits (lse = -inf)
    // and absent slots weigh 0. The sum adds slot pairs (2 j, 2 j + 1) first,
    // which gives every lane of head r the same W whichever order it holds
    // the pair in.
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < kMaxMergeSplitsBf16; ++k) {
        if ((k ^ s1) >= S) l[k] = -INFINITY;
        M = fmaxf(M, l[k]);
    }
    float e[kMaxMergeSplitsBf16], W = 0.f;
#pragma unroll
    for (int k = 0; k < kMaxMergeSplitsBf16; ++k) e[k] = l[k] == -INFINITY ? 0.f : __expf(l[k] - M);
#pragma unroll
    for (int j = 0; j < kMaxMergeSplitsBf16 / 2; ++j) W += e[2 * j] + e[2 * j + 1];
    const float inv = (W > 0.f) ? 1.f / W : 0.f;
    if (wave == 0 && G == 0 && P.lse) P.lse[(int64_t)row * kHeads + r] = (W > 0.f) ? M + logf(W) : -INFINITY;
    // B operands: lane (G, r) holds k-slots 8 G .. +7, i.e. heads' 8 (G % 2) .. +7 of
    // slot 2 ks + G / 2; its one nonzero is head' = r, when r lies in that half
    const bool own = (r >> 3) == (G & 1);
    bf16x8 bh[4], bl[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const float w = e[2 * ks] * inv;
        const __bf16 hi = (__bf16)w;
        const __bf16 lo = (__bf16)(w - (float)hi);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const bool at = own && k == (r & 7);
            bh[ks][k] = at ? hi : (__bf16)0.f;
            bl[ks][k] = at ? lo : (__bf16)0.f;
        }
    }
    f32x4 acc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            acc[t] = mfma32(x[t][ks], bh[ks], acc[t]);
            acc[t] = mfma32(x[t][ks], bl[ks], acc[t]);
        }
    }
    // tile t, row 4 G + i is column 128 w + 32 G + 4 t + i of head r
    __bf16* out = P.out + ((int64_t)row * kHeads + r) * kDv + 128 * wave + 32 * G;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        bf16x8 pk;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pk[i] = (__bf16)acc[2 * p][i];
            pk[4 + i] = (__bf16)acc[2 * p + 1][i];
        }
        *reinterpret_cast<bf16x8*>(out + 8 * p) = pk;
    }
}

// Split-K with the merge in stage 1: the partial of this workgroup (slot
// `slot` of query row `row`) has been written with device-coherent stores.
// Each workgroup waits for its own stores to complete, then counts itself in
// on the row's arrival counter; the one that arrives last sets the counter
// back to zero and merges the row's nsplit partials (the log-sum-exp merge of
// the combine kernel):
//     M = max_s lse_s,  w_s = exp(lse_s - M),
//     out = sum_s w_s O_s / sum_s w_s  (bf16),  lse = M + ln sum_s w_s,
// skipping empty partials (lse_s = -inf). No workgroup waits for another: the
// last to arrive finds every partial complete (their stores completed before
// their counts), so the merge needs no co-residency and no cache flush.
// Thread (h, q) merges head h = tid / 16, columns 4 (q + 16 k) .. +3, k < 8.
__device__ void merge_if_last(const Params& P, int row, uint8_t* smem) {
    wait_vmcnt<0>();  // this thread's partial stores are complete
    __syncthreads();  // ... and every thread's
    int* flag = reinterpret_cast<int*>(smem);
    const int tid = threadIdx.x, S = P.nsplit;
    if (tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(P.counters + row, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = old == (uint32_t)(S - 1);
        if (last) __hip_atomic_store(P.counters + row, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag = last;
    }
    __syncthreads();
    if (!*flag) return;
    if (S > kMaxMergeSplits) {
        merge_bf16(P, row, S);
        return;
    }
    constexpr int kBatch = 4;  // partials whose loads are in flight together
    constexpr int kQuads = kDv / 4 / 16;
    const int h = tid >> 4, q = tid & 15;
    const __amdgpu_buffer_rsrc_t ro = merge_rsrc(P.part_o + (int64_t)row * S * kHeads * kDv, S * kHeads * kDv * 4);
    const __amdgpu_buffer_rsrc_t rl = merge_rsrc(P.part_lse + (int64_t)row * S * kHeads, S * kHeads * 4);
    float m = -INFINITY, W = 0.f;
    f32x4 acc[kQuads];
#pragma unroll
    for (int k = 0; k < kQuads; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < S; s0 += kBatch) {
        float l[kBatch];
        f32x4 o[kBatch][kQuads];
#pragma unroll
        for (int v = 0; v < kBatch; ++v) {
            const int sl = s0 + v;
            l[v] = -INFINITY;
            if (sl < S) {
                l[v] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, 4 * (sl * kHeads + h), 0,
                                                                                      kCoherentLoad));
#pragma unroll
                for (int k = 0; k < kQuads; ++k)
                    o[v][k] = __builtin_bit_cast(
                        f32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, 4 * ((sl * kHeads + h) * kDv + 4 * (q + 16 * k)),
                                                                     0, kCoherentLoad));
            }
        }
        float mb = l[0];
#pragma unroll
        for (int v = 1; v < kBatch; ++v) mb = fmaxf(mb, l[v]);
        if (mb == -INFINITY) continue;
        const float mn = fmaxf(m, mb);
        const float sc = __expf(m - mn);  // m = -inf: 0
        W *= sc;
#pragma unroll
        for (int k = 0; k < kQuads; ++k) acc[k] *= sc;
#pragma unroll
        for (int v = 0; v < kBatch; ++v) {
            if (l[v] == -INFINITY) continue;  // empty or absent: never multiplied
            const float w = __expf(l[v] - mn);
            W += w;
#pragma unroll
            for (int k = 0; k < kQuads; ++k) acc[k] += w * o[v][k];
        }
        m = mn;
    }
    const float inv = (W > 0.f) ? 1.f / W : 0.f;
    __bf16* out = P.out + ((int64_t)row * kHeads + h) * kDv;
#pragma unroll
    for (int k = 0; k < kQuads; ++k) {
        bf16x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) pk[e] = (__bf16)(acc[k][e] * inv);
        *reinterpret_cast<bf16x4*>(out + 4 * (q + 16 * k)) = pk;
    }
    if (q == 0 && P.lse) P.lse[(int64_t)row * kHeads + h] = (W > 0.f) ? m + logf(W) : -INFINITY;
}

// Attend tokens [t0, t1) of one sequence (positions within it; its
// kv_indices entries start at `base`) with query row b, using the whole
// workgroup, and write the result: the final bf16 output row b + lse when
// `final`, else partial slot `slot`. Token j of the sequence is cache row
// indices[base + j] (page size 1), or row
// indices[base + j / page_size] * page_size + j % page_size.
// The four waves work on the same 32-token step: wave w gathers half w / 2 of
// tile w % 2 and computes the scores of tile w % 2 over half w / 2 of the
// score dims (k-steps 9 (w / 2) .. +8, or MX blocks 0-2 / 3 and RoPE), the
// partial scores are summed through LDS in a fixed order, and every wave then
// runs the same softmax and accumulates P . V for its own 128 output columns.
//
// QF = 1: fp8 query. Q is quantised here (static scale read, or the dynamic
// scale reduced from the partial maxima); `scale_out` makes this workgroup
// publish a dynamic scale.
// Two stage-1 workgroups share a compute unit on the fp8 and MXFP4 caches
// (launch indices x and x + 256), and the SIMD arbiter favours older waves,
// so without help the second one finishes last: it runs at priority 2 (MXFP4
// 32 x 8k 38.2 -> 37.8 us, fp8 256 x 8k 213.3 -> 211.5 us when introduced).
// That fixed boost overshoots on long ranges: per-workgroup timestamps
// showed the second workgroups ending about 3.3 us before the first on fp8
// 64 x 8k (MXFP4 32 x 8k 3.6 us, where priority 1 measured the same). The
// fp8 plans with two workgroups per compute unit and long ranges (TURNS)
// therefore let the two take turns at priority 2 step by step instead, which
// brought the two classes within 1.7 us of each other and the last
// workgroup's end 1.3 us earlier. A separate instantiation, because the
// priority switch in the loop costs short ranges about 0.4 us even where it
// is not taken.
template <bool TURNS>
__device__ __forceinline__ void second_wg_priority() {
    if constexpr (!TURNS) {
        if (blockIdx.x >= kNumCUs) __builtin_amdgcn_s_setprio(2);
    }
}
template <bool TURNS>
__device__ __forceinline__ void take_turns_priority(int s) {
    if constexpr (TURNS) {
        if ((s + (blockIdx.x >= kNumCUs ? 1 : 0)) & 1) __builtin_amdgcn_s_setprio(2);
        else __builtin_amdgcn_s_setprio(0);
    }
}
// Tokens per workgroup from which fp8 plans of more than one workgroup per
// compute unit take turns (fp8 64 x 8k has 1024: -1.4 us; 256 x 1k has 512:
// +0.5 us with turns).
constexpr int kTurnsMinTokens = 1024;
// Splits per sequence from which fp8 plans load the bf16 query into registers
// rather than through LDS (launch).
constexpr int kQRegsMinSplits = 32;

// Two query rows per workgroup (NT = 2): row t of the pair sees the sequence's
// positions [0, lim_t); has1 is false when the pair has no second row (the
// last row of an odd count).
struct RowPair {
    int lim0 = 0, lim1 = 0;
    bool has1 = false;
};

template <int KV, int QF, bool MG = false, int NT = 1, bool TURNS = false, bool QL = false>
__device__ void run_wg(const Params& P, uint8_t* smem, int b, int base, int t0, int t1, bool final, int slot,
                       bool scale_out, QueryRegs<KV, QF, NT>& qr, bool idx_dma, bool idx_staged,
                       int64_t early_first = -1, RowPair pr = RowPair{}) {
    using L = Layout<KV>;
    constexpr int R = Fmt<KV>::kRing;
    constexpr int D = R - 1;  // steps issued ahead of the one computed
    static_assert(D >= 2, "ring depth: the pipeline needs the next step landed while one more is in flight");
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, G = lane >> 4, r = lane & 15;
    const int tile = wave & 1, hf = wave >> 1;
    int32_t* idx = reinterpret_cast<int32_t*>(smem + L::kIdxOff);
    f32x4* sbuf = reinterpret_cast<f32x4*>(smem + L::kSbufOff);
    float* fs_buf = reinterpret_cast<float*>(smem + L::kFsOff);
    // One query row per workgroup: the wave's value reads are those of its 8
    // output blocks. Two rows (NT = 2): wave w runs row w / 2 alone, with the
    // 16 blocks of the two block groups 2 (w % 2) and 2 (w % 2) + 1.
    const PvOff<KV> pv_off = pv_lane_offsets<KV>(lane, NT == 2 ? 2 * tile : wave);
    const PvOff<KV> pv_off1 = pv_lane_offsets<KV>(lane, NT == 2 ? 2 * tile + 1 : wave);
    const int2 trows = lane_tile_rows<KV>(lane, hf);  // this lane's tile rows when it issues its half

    // The first index window (unless the caller's LDS-DMA of a guessed window
    // already holds it) and the query are in flight together here.
    constexpr int kIdxWindow = Fmt<KV>::kIdxWindow;
    constexpr int kPer = kIdxPer<KV>;
    int32_t iv[kPer];
    if (!idx_staged) load_idx<KV>(P, base, t0, min(kIdxWindow, t1 - t0), iv);
    using QOp = typename QOperand<KV, QF>::T;
    constexpr bool kMx = QF && KV == MLA_KV_MXFP4;           // fp8 query: scores on the MX-scaled MFMA
    constexpr bool kSplit = QueryRegs<KV, QF, NT>::kSplit;  // bf16 query, MXFP4 cache: split query, same MFMA
    auto& qB = qr.qB;
    auto& qg = qr.qg;
    auto& qsc = qr.qsc;
    const float kv_scale = qr.kv_scale, q_part = qr.q_part;
    float q_scale = qr.q_scale;
    const __bf16* qseq = P.q + (int64_t)b * kHeads * kDqk;
    // The caller's early gathers (the first e_early steps of the first
    // window) when it issued them for the range this workgroup runs, the
    // only case in which they can be kept: the waits up to the first step
    // then leave them in flight. -1: none, or for another range.
    const int e_early = (early_first >= 0 && idx_staged)
                            ? min(D, (min(kIdxWindow, t1 - t0) + kStepTokens - 1) / kStepTokens)
                            : -1;
    // Consume Q and the scales here: the compiler's wait for these loads must
    // not land inside the token loop, where the count it waits for would also
    // drain the gathers in flight (it does not see the LDS-DMA loads).
    if constexpr (QL) {
        // Q^T through ring slot D (dma_query), issued before the caller's
        // index DMA (kIdxPer operations) and early gathers
        static_assert(NT == 1 && !QF && !kSplit, "the query through LDS: bf16 query, one row, bf16 or fp8 cache");
        if (e_early >= 0) wait_behind<KV, kIdxPer<KV>>(e_early, hf);
        else if (idx_dma && early_first < 0) wait_vmcnt<kIdxPer<KV>>();
        else wait_vmcnt<0>();
        __syncthreads();  // every wave's share of Q has landed
        const uint8_t* qs = smem + D * L::kStepBytes;
#pragma unroll
        for (int j = 0; j < kHalfK; ++j)
            qB[j] = *reinterpret_cast<const bf16x8*>(qs + 1024 * (kHalfK * hf + j) + 16 * lane);
    } else if constexpr (NT == 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < kHalfK; ++j) asm volatile("" ::"v"(qr.qB2[h][j]));
    } else if constexpr (QF || kSplit) {
#pragma unroll
        for (int k = 0; k < kQPer; ++k) asm volatile("" ::"v"(qg[k]));
    } else {
#pragma unroll
        for (int j = 0; j < kHalfK; ++j) asm volatile("" ::"v"(qB[j]));
    }
    asm volatile("" ::"v"(kv_scale), "v"(q_part), "v"(q_scale));
    // The caller's index DMA, kept or not, has landed before anything else
    // touches the index window. The early gathers issued after it stay in
    // flight when they may be kept (e_early >= 0, checked below); otherwise
    // they have landed too and no gathers are in flight past this point.
    if (idx_dma) {
        if (e_early >= 0) wait_behind<KV, 0>(e_early, hf);
        else wait_vmcnt<0>();
    }
    phase_stamp(1);
    if constexpr (QF) {
        if (P.q_amax) {
            q_scale = q8_dynamic_scale(q_part, reinterpret_cast<float*>(sbuf), tid);
            if (scale_out && tid == 0) P.q_scale[0] = q_scale;
        }
    }
    const float qk_scale = P.sm_scale * kv_scale * q_scale * kLog2e;

    WaveAccT<kWaveBlocks * NT> acc;
#pragma unroll
    for (int j = 0; j < kWaveBlocks * NT; ++j) acc.o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc.m = -INFINITY;
    acc.l = 0.f;

    for (int w0 = t0; w0 < t1; w0 += kIdxWindow) {
        const int n = min(kIdxWindow, t1 - w0);
        __syncthreads();  // every wave is done with the previous window / previous range
        if (w0 != t0) load_idx<KV>(P, base, w0, n, iv);
        if (w0 != t0 || !idx_staged) {
#pragma unroll
            for (int k = 0; k < kPer; ++k)
                if (tid + k * kThreads < n) idx[tid + k * kThreads] = iv[k];
        } else if (P.page_size > 1) {
            // the caller staged this window's page entries (dma_pages; the page size is then a
            // power of two, ps = 2^sh): token t0 + j is row st[(t0 + j) >> sh - t0 >> sh] << sh
            // plus (t0 + j) & (ps - 1)
            const int sh = __builtin_ctz((unsigned)P.page_size), p0 = t0 >> sh;
            const int32_t* st = reinterpret_cast<const int32_t*>(smem + L::kSbufOff + kPageStageOff);
            // not unrolled: the unrolled form holds every entry's load at once and raised every
            // stage-1 kernel's register count (by 16 VGPRs on the fp8 cache; MXFP4 spilled)
#pragma unroll 1
            for (int k = 0; k < kPer; ++k) {
                const int j = tid + k * kThreads, t = t0 + j;
                if (j < n) idx[j] = (st[(t >> sh) - p0] << sh) | (t & (P.page_size - 1));
            }
        }
        __syncthreads();
        const int nsteps = (n + kStepTokens - 1) / kStepTokens;
        // This wave's half of tile `tile` of step i into ring slot i % R; tokens
        // at or beyond n re-read the last valid row (always in bounds).
        auto issue_step = [&](int i) {
            const int j0 = i * kStepTokens + kTile * tile;
            const int64_t ra = idx[min(j0 + trows.x, n - 1)];
            const int64_t rb = trows.y == trows.x ? ra : (int64_t)idx[min(j0 + trows.y, n - 1)];
            issue_half<KV>(P, ra, rb, smem + (i % R) * L::kStepBytes + tile * Fmt<KV>::kTileBytes, lane, hf);
        };
        // This wave's partial scores of step i, for exchange buffer i % 2.
        // (MXFP4: also converts the step's value-block scales into buffer i % 2.)
        // Two rows per workgroup: the full scores of tile `tile` for row hf.
        auto scores = [&](int i) -> f32x4 {
            const uint8_t* st = smem + (i % R) * L::kStepBytes;
            if constexpr (KV == MLA_KV_MXFP4) convert_scales(st, fs_buf + (i & 1) * (L::kFsBytes / 4), tid);
            if constexpr (NT == 2) {
                return qk_partial<KV, 0>(st, qr.qB2[0], tile, lane) + qk_partial<KV, 1>(st, qr.qB2[1], tile, lane);
            } else if constexpr (kMx) {
                return hf ? qk_partial_mx<1>(st, qB, tile, lane) : qk_partial_mx<0>(st, qB, tile, lane);
            } else if constexpr (kSplit) {
                return hf ? qk_partial_mx2<1>(st, qB, qsc, tile, lane) : qk_partial_mx2<0>(st, qB, qsc, tile, lane);
            } else {
                return hf ? qk_partial<KV, 1>(st, qB, tile, lane) : qk_partial<KV, 0>(st, qB, tile, lane);
            }
        };
        auto put_scores = [&](int i, f32x4 part) { sbuf[(i & 1) * (kWaves * 64) + wave * 64 + lane] = part; };
        // The caller's early gathers of the first D steps (already landed) stand
        // when the guessed range was the true one and kv_indices names exactly
        // the rows this wave fetched; else this wave gathers its steps again.
        bool keep = w0 == t0 && early_first >= 0 && idx_staged;
        if (keep) {
#pragma unroll
            for (int d = 0; d < D; ++d)
                if (d < nsteps) {
                    const int ja = d * kStepTokens + kTile * tile + trows.x;
                    const int jb = d * kStepTokens + kTile * tile + trows.y;
                    keep = keep && (int64_t)idx[min(ja, n - 1)] == early_row(P, early_first, ja, n) &&
                           (int64_t)idx[min(jb, n - 1)] == early_row(P, early_first, jb, n);
                }
            keep = __all(keep);
        }
        if (!keep) {
            // this wave's early gathers into the same slots have landed first
            if (w0 == t0 && e_early >= 0) wait_vmcnt<0>();
#pragma unroll
            for (int d = 0; d < D; ++d)
                if (d < nsteps) issue_step(d);
        }
        // fp8 query, first window: quantise while the first gathers are in
        // flight. The codes ([head][576] bytes) pass through ring slot D, whose
        // step is issued only after the next two barriers.
        uint8_t* qcodes = smem + (D % R) * L::kStepBytes;
        // split query: hi codes in ring slot D, lo codes in the score exchange
        // and value-scale buffers (free until scores(0) and put_scores(0) write
        // them, which every wave does only after a barrier that follows all
        // waves' operand reads below)
        uint8_t* qcodes_lo = smem + L::kSbufOff;
        if constexpr (QF) {
            if (w0 == t0) q8_quantise<kQPer>(qg, qseq, tid, kThreads, kQGroups, q_scale, qcodes);
        } else if constexpr (kSplit) {
            static_assert(L::kIdxOff - L::kSbufOff >= kHeads * kDqk + kHeads * (kDqk / 32),
                          "the exchange and value-scale buffers hold one split-query code set");
            static_assert(L::kStepBytes >= kHeads * kDqk + kHeads * (kDqk / 32), "a ring slot holds one code set");
            if (w0 == t0) q_split_quantise<kQPer>(qg, tid, qcodes, qcodes_lo);
        }
        wait_own<KV>(min(D - 1, nsteps - 1), hf);
        __syncthreads();  // step 0 has landed (and the query codes are written)
        if (w0 == t0) phase_stamp(2);
        if constexpr (kMx) {
            if (w0 == t0) {
                // B operand of block u for head r: dims 128 u + 16 G + (0..15) and 128 u + 64 + 16 G + (0..15);
                // the RoPE block has dims 512 + 16 G + (0..15) and zeros (dims 576.. do not exist)
                const uint8_t* qr = qcodes + r * kDqk;
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    const int u = hf ? 3 + j : j;
                    u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
                    if (u < 4) {
                        lo = *reinterpret_cast<const u32x4*>(qr + 128 * u + 16 * G);
                        hi = *reinterpret_cast<const u32x4*>(qr + 128 * u + 64 + 16 * G);
                    } else if (u == 4) {
                        lo = *reinterpret_cast<const u32x4*>(qr + 512 + 16 * G);
                    }
                    qB[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                  (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                }
            }
        } else if constexpr (kSplit) {
            if (w0 == t0) {
                // as for the fp8 query, once per code set; the e8m0 code of lane (G, r) is that of head r's
                // 32-element block G of the 128-dim block (RoPE: blocks 16, 17, then zero padding)
#pragma unroll
                for (int pc = 0; pc < 2; ++pc) {
                    const uint8_t* cs = pc ? qcodes_lo : qcodes;
                    const uint8_t* crow = cs + r * kDqk;
                    const uint8_t* srow = cs + kHeads * kDqk + r * (kDqk / 32);
#pragma unroll
                    for (int j = 0; j < 3; ++j) {
                        const int u = hf ? 3 + j : j;
                        u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
                        int code = 127;
                        if (u < 4) {
                            lo = *reinterpret_cast<const u32x4*>(crow + 128 * u + 16 * G);
                            hi = *reinterpret_cast<const u32x4*>(crow + 128 * u + 64 + 16 * G);
                            code = srow[4 * u + G];
                        } else if (u == 4) {
                            lo = *reinterpret_cast<const u32x4*>(crow + 512 + 16 * G);
                            if (G < 2) code = srow[16 + G];
                        }
                        qB[3 * pc + j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                               (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                        qsc[3 * pc + j] = code;
                    }
                }
                __syncthreads();  // every wave has read the lo codes before any wave writes the buffers
            }
        } else if constexpr (QF) {
            if (w0 == t0) {
#pragma unroll
                for (int j = 0; j < kHalfK; ++j) {
                    const u32x2 c = *reinterpret_cast<const u32x2*>(qcodes + r * kDqk + dbase<KV>(kHalfK * hf + j, G));
                    if constexpr (__is_same(QOp, long)) qB[j] = __builtin_bit_cast(long, c);
                    else qB[j] = fp8x8_to_bf16(c[0], c[1]);
                }
            }
        }
        put_scores(0, scores(0));
        // Software pipeline: iteration s computes the scores of step s + 1
        // while it runs the softmax and P . V of step s, so the score MFMAs
        // overlap the softmax arithmetic. One barrier per step:
        //   - every wave's partial scores of step s are in buffer s % 2;
        //   - step s + 1 has landed (each wave waited for its own loads);
        //   - every wave is done with step s - 1 (its ring slot and buffer
        //     (s - 1) % 2, which this iteration refills).
        for (int s = 0; s < nsteps; ++s) {
            if (s + 1 < nsteps) wait_own<KV>(min(D - 2, nsteps - 2 - s), hf);
            __syncthreads();
            take_turns_priority<TURNS>(s);
            if (s + D < nsteps) issue_step(s + D);  // into the slot of step s - 1
            const f32x4* sb = sbuf + (s & 1) * (kWaves * 64);
            f32x4 sc[2];
            if constexpr (NT == 2) {  // wave 2 t + u: tile u of row t; this wave's row is hf
                sc[0] = sb[(2 * hf) * 64 + lane];
                sc[1] = sb[(2 * hf + 1) * 64 + lane];
            } else {  // wave 2 h + u: half h of tile u
                sc[0] = sb[0 * 64 + lane] + sb[2 * 64 + lane];
                sc[1] = sb[1 * 64 + lane] + sb[3 * 64 + lane];
            }
            // Program order keeps every long latency behind independent work:
            // the value reads of step s and the score MFMAs of step s + 1 are
            // issued before the softmax, and the scores are stored after P . V.
            PvRaw<KV> v, v1;
            pv_load<KV>(smem + (s % R) * L::kStepBytes, fs_buf + (s & 1) * (L::kFsBytes / 4), pv_off, lane, wave, v);
            if constexpr (NT == 2)
                pv_load<KV>(smem + (s % R) * L::kStepBytes, fs_buf, pv_off1, lane, wave, v1);
            f32x4 next = {0.f, 0.f, 0.f, 0.f};
            if (s + 1 < nsteps) next = scores(s + 1);
            if constexpr (NT == 2) {
                // this wave's row: its valid tokens of the step, none once past
                // its visible prefix (uniform in the wave; no barrier inside)
                const int lim = hf ? (pr.has1 ? pr.lim1 : w0) : pr.lim0;
                const int nv = min(n, lim - w0) - s * kStepTokens;
                if (nv > 0) {
                    const bf16x8 pa = softmax_step(sc, qk_scale, nv, lane, acc);
#pragma unroll
                    for (int j = 0; j < kWaveBlocks; ++j) acc.o[j] = mfma32(pa, pv_convert<KV>(v, j), acc.o[j]);
#pragma unroll
                    for (int j = 0; j < kWaveBlocks; ++j)
                        acc.o[kWaveBlocks + j] = mfma32(pa, pv_convert<KV>(v1, j), acc.o[kWaveBlocks + j]);
                }
            } else {
                const bf16x8 pa = softmax_step(sc, qk_scale, n - s * kStepTokens, lane, acc);
                pv_mma<KV>(v, pa, acc);
            }
            if (s + 1 < nsteps) put_scores(s + 1, next);
        }
    }

    phase_stamp(3);
    // ---- epilogue: every wave of a row holds the same m and l; it writes its own columns ----
    // One row: query row b, the wave's blocks kWaveBlocks * wave + j. Two rows
    // (NT = 2): wave w writes row b + w / 2 (absent: nothing), blocks
    // 2 kWaveBlocks (w % 2) + j; the row's partial slot is slot + (w / 2) nsplit
    // (slots are row-major over the splits).
    const int row = b + (NT == 2 ? hf : 0);
    const bool live = NT == 1 || hf == 0 || pr.has1;
    const int64_t sl = (int64_t)slot + (NT == 2 ? (int64_t)hf * P.nsplit : 0);
    const int vb = NT == 2 ? 2 * kWaveBlocks * tile : kWaveBlocks * wave;  // first output block of this wave
    const bool lse_wave = NT == 2 ? tile == 0 : wave == 0;
    if (live) {
        const float lt = group_sum4(acc.l);
        const float inv_r = (lt > 0.f) ? kv_scale / lt : 0.f;  // head r
        const float lse_r = (lt > 0.f) ? (acc.m + log2f(lt)) * kLn2 : -INFINITY;
        float inv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) inv[i] = __shfl(inv_r, 4 * G + i);  // head 4G+i lives in lane 4G+i
        if (final) {
            __bf16* o = P.out + (int64_t)row * kHeads * kDv;
#pragma unroll
            for (int j = 0; j < kWaveBlocks * NT; ++j) {
                const int col = dcol<KV>(vb + j, r);
#pragma unroll
                for (int i = 0; i < 4; ++i) o[(4 * G + i) * kDv + col] = (__bf16)(acc.o[j][i] * inv[i]);
            }
            if (lse_wave && G == 0 && P.lse) P.lse[(int64_t)row * kHeads + r] = lse_r;
        } else if constexpr (MG) {
            // device-coherent stores (written through to memory), read back by
            // whichever split workgroup of this row arrives last
            float* o = P.part_o + sl * kHeads * kDv;
            if (P.nsplit > kMaxMergeSplits) {
                // 5..8 splits: a bf16 partial [column][head] at the start of the
                // slot, the four heads 4G..4G+3 of a column in one 8-byte store
                uint64_t* ob = reinterpret_cast<uint64_t*>(o);
#pragma unroll
                for (int j = 0; j < kWaveBlocks * NT; ++j) {
                    const int col = dcol<KV>(vb + j, r);
                    bf16x4 pk;
#pragma unroll
                    for (int i = 0; i < 4; ++i) pk[i] = (__bf16)(acc.o[j][i] * inv[i]);
                    __hip_atomic_store(ob + (col * kHeads + 4 * G) / 4, __builtin_bit_cast(uint64_t, pk),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            } else {
#pragma unroll
                for (int j = 0; j < kWaveBlocks * NT; ++j) {
                    const int col = dcol<KV>(vb + j, r);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        __hip_atomic_store(o + (4 * G + i) * kDv + col, acc.o[j][i] * inv[i], __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            if (lse_wave && G == 0)
                __hip_atomic_store(P.part_lse + sl * kHeads + r, lse_r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            float* o = P.part_o + sl * kHeads * kDv;
#pragma unroll
            for (int j = 0; j < kWaveBlocks * NT; ++j) {
                const int col = dcol<KV>(vb + j, r);
#pragma unroll
                for (int i = 0; i < 4; ++i) o[(4 * G + i) * kDv + col] = acc.o[j][i] * inv[i];
            }
            if (lse_wave && G == 0) P.part_lse[sl * kHeads + r] = lse_r;
        }
    }
    phase_stamp_stores_done();
    if constexpr (MG) {
        if (!final) {
            merge_if_last(P, b, smem);
            if (NT == 2 && pr.has1) merge_if_last(P, b + 1, smem);
        }
    }
    phase_stamp(5);
}

// Workgroups are handed to the eight XCDs round-robin (workgroup x to XCD
// x % 8), and each XCD has its own L2. Renumbering the work items so that
// consecutive ones share an XCD keeps the splits of one sequence, which all
// read the same Q row and whose partials one combine workgroup reads back,
// behind one L2. A bijection on [0, n) when n is a multiple of 8, else the
// identity; correctness never depends on where a workgroup runs.
__device__ __forceinline__ int xcd_order(int x, int n) { return (n & 7) ? x : (x & 7) * (n >> 3) + (x >> 3); }

// The number of k in 1..n with ptr[k] <= v, counted by the whole workgroup in
// one pass of loads per 256 entries (wave ballots summed through the 4 ints
// at cnt, in LDS). For a non-decreasing ptr with ptr[0] <= v < ptr[n] this is
// the b with ptr[b] <= v < ptr[b + 1].
__device__ __forceinline__ int count_le(const int32_t* ptr, int n, int v, int* cnt) {
    int b = 0;
    const int tid = threadIdx.x;
    for (int c = 0; c < n; c += kThreads) {
        const int k = c + tid + 1;
        const uint64_t m = __ballot(k <= n && ptr[k] <= v);
        if ((tid & 63) == 0) cnt[tid >> 6] = __popcll(m);
        __syncthreads();
        b += cnt[0] + cnt[1] + cnt[2] + cnt[3];
        __syncthreads();
    }
    return b;
}

// The stage-1 kernels take the fields their first loads need ahead of Params
// as plain arguments: those arrive in SGPRs when the waves start (kernel
// argument preloading, 14 SGPRs), so the query, index and first row requests
// leave without first waiting for the kernel-argument segment to be read.
// kv_rows comes as 32 bits, clamped: a smaller bound on the rows gathered
// before kv_indices arrives stays inside the cache buffer.
// (The launched grid size comes the same way: gridDim is read from the
// kernel-argument segment.)
#define STAGE1_ARGS                                                                                       \
    const __bf16 *q_arg, const int32_t *indices_arg, const void *kv_scales_arg, const uint8_t *kv_arg,          \
        int nsplit_arg, int uni_len_arg, int uni_chunk_arg, int nblocks, int page_size_arg, int kv_rows_arg,       \
        Params P_arg
__device__ __forceinline__ Params stage1_params(const __bf16* q, const int32_t* indices, const void* kv_scales,
                                                const uint8_t* kv, int nsplit, int uni_len, int uni_chunk,
                                                int page_size, int kv_rows, const Params& P_arg) {
    Params P = P_arg;
    P.kv = kv;
    P.page_size = page_size;
    P.kv_rows = kv_rows;
    P.q = q;
    P.indices = indices;
    P.kv_scales = kv_scales;
    P.nsplit = nsplit;
    P.uni_len = uni_len;
    P.uni_chunk = uni_chunk;
    return P;
}

// Two query rows of one sequence per workgroup (several query tokens per
// sequence, uniform count n = uni_q >= 2, bf16 cache): work row w is the
// pair of rows b n + 2 g, b n + 2 g + 1 of sequence b = w / ceil(n / 2),
// g = w % ceil(n / 2) (the last of an odd n alone). The split ranges are
// those of the pair's later row, which sees the most tokens; the earlier
// row masks what it does not see.
template <int KV, int QF, bool MG>
__device__ void split_pair(const Params& P, uint8_t* smem, int nblocks) {
    const int item = xcd_order(blockIdx.x, nblocks);
    const int wrow = item / P.nsplit, s = item % P.nsplit;
    const int n = P.uni_q, gq = (n + 1) >> 1;
    const int b = wrow / gq, t0q = 2 * (wrow - b * gq);
    const int row0 = b * n + t0q;
    const bool has1 = t0q + 1 < n;
    const int hf = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) >> 1;
    QueryRegs<KV, QF, 2> qr;
    load_query_pair(P, row0 + (has1 ? hf : 0), qr);
    const int base = P.indptr[b], entries = P.indptr[b + 1] - base;
    const int Ls = P.page_size == 1 ? entries : entries > 0 ? (entries - 1) * P.page_size + P.last_page[b] : 0;
    const int hide0 = P.causal ? n - 1 - t0q : 0;
    const int hide1 = P.causal && has1 ? hide0 - 1 : hide0;
    RowPair pr;
    pr.lim0 = max(0, Ls - hide0);
    pr.lim1 = max(0, Ls - hide1);
    pr.has1 = has1;
    const int L = pr.lim1;
    const int chunk = ((L + P.nsplit - 1) / P.nsplit + kStepTokens - 1) / kStepTokens * kStepTokens;
    const int t0 = min(L, s * chunk);
    const int t1 = min(L, t0 + chunk);
    run_wg<KV, QF, MG, 2>(P, smem, row0, base, t0, t1, P.nsplit == 1, row0 * P.nsplit + s, false, qr, false, false,
                          -1, pr);
}

// MG: the plan merges the split partials here (the last-arriving split of
// each row); a separate instantiation, so that plans merged by the combine
// launch run a kernel without the merge code. NT: query rows per workgroup.
// QL: the bf16 query comes through LDS (dma_query; bf16 and fp8 caches), else
// it is loaded into registers.
template <int KV, int QF, bool MG, int NT = 1, bool TURNS = false, bool QL = (KV != MLA_KV_MXFP4 && QF == 0)>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(Fmt<KV>::kWgsPerCU, Fmt<KV>::kWgsPerCU)))
void split_kernel(STAGE1_ARGS) {
    phase_stamp(0);
    second_wg_priority<TURNS>();
    const Params P = stage1_params(q_arg, indices_arg, kv_scales_arg, kv_arg, nsplit_arg, uni_len_arg, uni_chunk_arg,
                                   page_size_arg, kv_rows_arg, P_arg);
    __shared__ __attribute__((aligned(16))) uint8_t smem[Layout<KV>::kBytes];
    if constexpr (NT == 2) {
        split_pair<KV, QF, MG>(P, smem, nblocks);
        return;
    }
    const int item = xcd_order(blockIdx.x, nblocks);
    const int row = item / P.nsplit, s = item % P.nsplit;
    // The bf16 query through LDS: its DMA first of all (dma_query).
    static_assert(!QL || (KV != MLA_KV_MXFP4 && !QF), "the query through LDS: bf16 query, bf16 or fp8 cache");
    QueryRegs<KV, QF> qr;
    if constexpr (QL) {
        query_scales<KV, QF>(P, qr);
        dma_query<KV>(P, row, smem);
    } else {
        load_query<KV, QF>(P, row, qr);
    }
    // Sequences of one common length Lu (page size 1, one query row each):
    // sequence b's entries would start at b * Lu, so this split's first index
    // window is requested now, with the query, before kv_indptr arrives. It
    // is kept when kv_indptr confirms the guess and read again otherwise; the
    // guessed entries lie within kv_indices [batch * Lu] either way.
    // With pages (page size ps > 1, a power of two dividing Lu) the sequence
    // holds Pu = Lu / ps of them, guessed to start at entry b * Pu: the
    // window's page entries are staged (dma_pages) and expanded into rows by
    // run_wg.
    const int Lu = P.uni_len, ps = P.page_size;
    const int Pu = ps == 1 ? Lu : Lu / ps;  // kv_indices entries of one sequence
    const int t0u = min(Lu, s * P.uni_chunk), t1u = min(Lu, t0u + P.uni_chunk);
    const bool idx_dma = t1u > t0u;  // Lu > 0
    if (idx_dma) {
        const int nu = min(Fmt<KV>::kIdxWindow, t1u - t0u);
        if (ps == 1)
            dma_idx<KV>(P, row * Lu + t0u, nu, reinterpret_cast<int32_t*>(smem + Layout<KV>::kIdxOff));
        else
            dma_pages<KV>(P, row * Pu + t0u / ps, (t0u + nu - 1) / ps - t0u / ps + 1, smem);
    }
    // With the cache size known, the first steps' rows of a contiguous cache
    // are requested as well (kept by run_wg where kv_indices agrees). Not on
    // the MXFP4 cache: the wait for the query registers also drains LDS-DMA
    // loads issued before it, which would put the query split behind the
    // first rows instead of beside them.
    const int64_t early_first =
        (KV != MLA_KV_MXFP4 && idx_dma && ps == 1 && P.kv_rows > 0) ? (int64_t)row * Lu + t0u : -1;
    if (early_first >= 0) issue_early<KV>(P, smem, early_first, min(Fmt<KV>::kIdxWindow, t1u - t0u));
    // the sequence of this query row, and the cache tokens the causal reading hides from it
    // (the reads of kv_indptr, qo_indptr and kv_last_page_len are scalar loads: ld_scalar)
    int b = row, hide = 0;
    if (P.uni_q > 0 || P.qo_indptr) {
        int t, n;
        if (P.uni_q > 0) {
            b = row / P.uni_q;
            n = P.uni_q;
            t = row - b * n;
        } else {
            b = __builtin_amdgcn_readfirstlane(
                count_le(P.qo_indptr, P.batch, row, reinterpret_cast<int*>(smem + Layout<KV>::kIdxOff)));
            const int r0 = ld_scalar(P.qo_indptr, b);
            n = ld_scalar(P.qo_indptr, b + 1) - r0;
            t = row - r0;
        }
        if (P.causal) hide = n - 1 - t;
    }
    const int base = ld_scalar(P.indptr, b), entries = ld_scalar(P.indptr, b + 1) - base;
    // tokens of the sequence: its entries, or (pages - 1) full pages plus the last page's tokens
    const int Ls =
        P.page_size == 1 ? entries : entries > 0 ? (entries - 1) * P.page_size + ld_scalar(P.last_page, b) : 0;
    const int L = max(0, Ls - hide);
    const int chunk = ((L + P.nsplit - 1) / P.nsplit + kStepTokens - 1) / kStepTokens * kStepTokens;
    const int t0 = min(L, s * chunk);
    const int t1 = min(L, t0 + chunk);
    const bool staged = idx_dma && base == row * Pu && L == Lu;  // then t0, t1 are t0u, t1u
    run_wg<KV, QF, MG, 1, TURNS, QL>(P, smem, row, base, t0, t1, P.nsplit == 1, row * P.nsplit + s, blockIdx.x == 0,
                                     qr, idx_dma, staged, early_first);
}

// Largest p whose share [floor(p T / G), floor((p+1) T / G)) starts at or before t.
__device__ __forceinline__ int share_of(int64_t t, int64_t T, int64_t G) { return (int)(((t + 1) * G - 1) / T); }
__device__ __forceinline__ int64_t share_start(int64_t p, int64_t T, int64_t G) { return p * T / G; }

// The persistent grid: workgroup p attends the tokens [floor(p T / G),
// floor((p+1) T / G)) of the concatenated sequences and writes one partial
// per sequence it touches, into slot p + b. TURNS: the two workgroups of a
// compute unit take turns at priority 2 (as the split plans with long ranges
// do). The sequence bounds are scalar loads. On the bf16 and fp8 caches each
// sequence's bf16 query comes through LDS (dma_query), requested together
// with the first index window and, with the cache size known, the first
// steps' rows of a contiguous cache.
template <int KV, int QF, bool TURNS = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(Fmt<KV>::kWgsPerCU, Fmt<KV>::kWgsPerCU)))
void persistent_kernel(STAGE1_ARGS) {
    phase_stamp(0);
    second_wg_priority<TURNS>();
    constexpr bool QLP = KV != MLA_KV_MXFP4 && QF == 0;
    const Params P = stage1_params(q_arg, indices_arg, kv_scales_arg, kv_arg, nsplit_arg, uni_len_arg, uni_chunk_arg,
                                   page_size_arg, kv_rows_arg, P_arg);
    __shared__ __attribute__((aligned(16))) uint8_t smem[Layout<KV>::kBytes];
    const int64_t T = P.total, Gn = P.grid;
    const int p = xcd_order(blockIdx.x, nblocks);
    const int64_t g0 = share_start(p, T, Gn), g1 = share_start(p + 1, T, Gn);
    if (g0 >= g1) {
        // an empty share; workgroup 0 still publishes a dynamic query scale
        if (QF && P.q_amax && blockIdx.x == 0) {
            const int tid = threadIdx.x;
            const float q = q8_dynamic_scale(tid < P.q_amax_n ? P.q_amax[tid] : 0.0f,
                                             reinterpret_cast<float*>(smem), tid);
            if (tid == 0) P.q_scale[0] = q;
        }
        return;
    }
    bool scale_out = blockIdx.x == 0;
    // first sequence b with indptr[b] <= g0 < indptr[b+1]
    const int lo = __builtin_amdgcn_readfirstlane(
        count_le(P.indptr, P.batch, (int)g0, reinterpret_cast<int*>(smem + Layout<KV>::kIdxOff)));
    for (int b = lo; b < P.batch; ++b) {
        const int s = ld_scalar(P.indptr, b), e = ld_scalar(P.indptr, b + 1);
        if (s >= g1) break;
        const int t0 = (int)max<int64_t>(g0, s), t1 = (int)min<int64_t>(g1, e);
        if (t0 >= t1) continue;
        const bool whole = (s >= g0) && (e <= g1);
        __syncthreads();  // the previous sequence's epilogue has finished reading LDS
        QueryRegs<KV, QF> qr;
        // page size 1: entries are tokens; this share holds entries [t0, t1) of sequence b
        bool idx_dma = false;
        int64_t early_first = -1;
        if constexpr (QLP) {
            // the query, the first index window and, with the cache size known, the first
            // steps' rows of a contiguous cache (entry t0 + j in row t0 + j; kept by run_wg
            // where kv_indices agrees) are requested together, as the split plans do
            query_scales<KV, QF>(P, qr);
            dma_query<KV>(P, b, smem);
            const int nu = min(Fmt<KV>::kIdxWindow, t1 - t0);
            dma_idx<KV>(P, t0, nu, reinterpret_cast<int32_t*>(smem + Layout<KV>::kIdxOff));
            idx_dma = true;
            if (P.kv_rows > 0) {
                early_first = t0;
                issue_early<KV>(P, smem, early_first, nu);
            }
        } else {
            load_query<KV, QF>(P, b, qr);
        }
        run_wg<KV, QF, false, 1, TURNS, QLP>(P, smem, b, s, t0 - s, t1 - s, whole, p + b, scale_out, qr, idx_dma,
                                             idx_dma, early_first);
        scale_out = false;
    }
}

// Stage 2: out[b,h] = sum_s w_s O_s / sum_s w_s, w_s = exp(lse_s - max lse),
// lse = max + ln sum w_s; empty partials (lse = -inf) carry no weight.
// (Submission 703488, `_reduce_splitk_parallel_*`; submission 593653,
// `_flash_fp8_split_s2`.)
// A sequence has 64 items (head, 128-column chunk). One workgroup takes
// `items` consecutive items of one sequence (a power of two <= 8, chosen so
// that no thread needs more than 8 partial loads); its 256 threads are 32
// column quads x 8 groups, 8 / items groups per item. Group g' of an item
// merges partials g', g' + 8 / items, ... against its own running max, with
// the lse and O loads of up to kCombBatch partials in flight at once; the
// group results (m_g, W_g, A_g) of an item are merged in LDS in a fixed
// order: M = max m_g, out = sum e^(m_g - M) A_g / sum e^(m_g - M) W_g (the
// same weighted mean with the sum regrouped).
struct CombineParams {
    const float* part_o;
    const float* part_lse;
    const int32_t* indptr;
    __bf16* out;
    float* lse;
    int batch;
    int mode;    // 0 split-K, 1 persistent
    int nsplit;  // split-K
    int grid;    // persistent
    int total;
    int items;   // items per workgroup
};

constexpr int kCombThreads = 256;
constexpr int kCombCols = 128;
constexpr int kCombQuads = kCombCols / 4;                 // 32
constexpr int kCombGroups = kCombThreads / kCombQuads;    // 8
constexpr int kCombBatch = 8;                             // partials in flight per thread

// Items per combine workgroup: as many as keep each thread at <= 8 partial
// loads (one round trip). The persistent plan's per-sequence partial counts
// vary, so it takes one item per workgroup.
// Items per combine workgroup for `parts` partials per sequence (split-K: the
// split count; persistent: about grid / batch + 1 shares touch a sequence, and
// any other count is merged correctly, only with other parallelism).
static int combine_items(int parts) {
    int i = 8;
    while (i > 1 && (parts * i + kCombGroups - 1) / kCombGroups > kCombBatch) i /= 2;
    return i;
}

// (part_o, part_lse, mode, nsplit and items lead as plain arguments, preloaded
// into SGPRs like the stage-1 kernels' first fields.)
__global__ __launch_bounds__(kCombThreads) void combine_kernel(const float* part_o_arg, const float* part_lse_arg,
                                                               int mode_arg, int nsplit_arg, int items_arg,
                                                               int nblocks, CombineParams C_arg) {
    phase_stamp_combine(0);
    CombineParams C = C_arg;
    C.part_o = part_o_arg;
    C.part_lse = part_lse_arg;
    C.mode = mode_arg;
    C.nsplit = nsplit_arg;
    C.items = items_arg;
    __shared__ f32x4 s_acc[kCombGroups][kCombQuads];
    __shared__ float s_m[kCombGroups];
    __shared__ float s_w[kCombGroups];
    const int I = C.items, gpi = kCombGroups / I;  // items per workgroup, groups per item
    const int wpb = 4 * kHeads / I;                // workgroups per sequence
    const int L = xcd_order(blockIdx.x, nblocks);
    const int b = L / wpb, it0 = (L % wpb) * I;
    const int tid = threadIdx.x, quad = tid & (kCombQuads - 1), gi = tid / kCombQuads;
    const int u = gi / gpi, gq = gi % gpi;         // this thread's item and its group within the item
    const int it = it0 + u, h = it >> 2, chunk = it & 3;
    const int d = chunk * kCombCols + quad * 4;
    // partial k of this sequence lives in slot base + first + k, for k < count
    int first = 0, count = 0, base = 0;
    if (C.mode == 0) {
        count = C.nsplit;
        base = b * C.nsplit;
    } else {
        const int s = C.indptr[b], e = C.indptr[b + 1];
        if (e > s) {
            first = share_of(s, C.total, C.grid);
            const int last = share_of(e - 1, C.total, C.grid);
            if (first == last) return;  // one workgroup held the whole sequence and wrote it
            count = last - first + 1;
        }
        base = b;  // slot of workgroup p for sequence b is p + b
    }
    float m = -INFINITY, W = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = gq; k0 < count; k0 += gpi * kCombBatch) {
        float l[kCombBatch];
        f32x4 o[kCombBatch];
#pragma unroll
        for (int v = 0; v < kCombBatch; ++v) {
            const int k = k0 + gpi * v, p = first + k;
            l[v] = -INFINITY;
            o[v] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (k < count) {
                // an empty persistent share (only when there are fewer tokens than
                // workgroups) wrote nothing: its slot holds no partial
                const bool empty = C.mode == 1 && C.total < C.grid &&
                                   share_start(p, C.total, C.grid) == share_start(p + 1, C.total, C.grid);
                if (!empty) {
                    const int64_t slot = base + p;
                    l[v] = C.part_lse[slot * kHeads + h];
                    o[v] = *reinterpret_cast<const f32x4*>(C.part_o + (slot * kHeads + h) * kDv + d);
                }
            }
        }
        float mb = l[0];
#pragma unroll
        for (int v = 1; v < kCombBatch; ++v) mb = fmaxf(mb, l[v]);
        if (mb == -INFINITY) continue;
        const float mn = fmaxf(m, mb);
        const float sc = __expf(m - mn);  // m = -inf: 0
        W *= sc;
        acc *= sc;
#pragma unroll
        for (int v = 0; v < kCombBatch; ++v) {
            if (l[v] == -INFINITY) continue;  // skipped, never multiplied: the slot may hold anything
            const float w = __expf(l[v] - mn);
            W += w;
            acc += w * o[v];
        }
        m = mn;
    }
    s_acc[gi][quad] = acc;
    if (quad == 0) {  // m and W are the same in every thread of a group
        s_m[gi] = m;
        s_w[gi] = W;
    }
    __syncthreads();
    if (gq == 0) {
        const int g0 = u * gpi;
        float M = s_m[g0];
        for (int g = 1; g < gpi; ++g) M = fmaxf(M, s_m[g0 + g]);
        f32x4 t = {0.f, 0.f, 0.f, 0.f};
        float Wt = 0.f;
        if (M != -INFINITY) {
            for (int g = 0; g < gpi; ++g) {
                if (s_m[g0 + g] == -INFINITY) continue;
                const float e = __expf(s_m[g0 + g] - M);
                t += e * s_acc[g0 + g][quad];
                Wt += e * s_w[g0 + g];
            }
        }
        const float inv = (Wt > 0.f) ? 1.f / Wt : 0.f;
        bf16x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) pk[e] = (__bf16)(t[e] * inv);
        *reinterpret_cast<bf16x4*>(C.out + ((int64_t)b * kHeads + h) * kDv + d) = pk;
        if (quad == 0 && chunk == 0 && C.lse) C.lse[(int64_t)b * kHeads + h] = (Wt > 0.f) ? M + logf(Wt) : -INFINITY;
    }
#if MLA_PHASE_STAMPS
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    phase_stamp_combine(1);
#endif
}

// Decode check: rows -> fp32 through the stage-1 staging (issue_half) and the
// two decode routines of the attention kernel. path 0: every column through
// the score operand (qk_operand); path 1: columns 0..511 through the value
// operand (pv_load, pv_convert / pv_convert_fp4), columns 512..575 through path 0.
// One wave per 32 rows; fp8 values are multiplied by kv_scale in fp32.
template <int KV>
__global__ __launch_bounds__(64) void dequant_kernel(Params P, int64_t rows, int path, float* out) {
    __shared__ __attribute__((aligned(16))) uint8_t step[Layout<KV>::kStepBytes];
    const int lane = threadIdx.x, G = lane >> 4, r = lane & 15;
    const int64_t row0 = (int64_t)blockIdx.x * kStepTokens;
    const int n = (int)min<int64_t>(kStepTokens, rows - row0);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int2 tr = lane_tile_rows<KV>(lane, hf);
            const int64_t ra = row0 + min(kTile * t + tr.x, n - 1), rb = row0 + min(kTile * t + tr.y, n - 1);
            if (hf) issue_half<KV, 1>(P, ra, rb, step + t * Fmt<KV>::kTileBytes, lane);
            else issue_half<KV, 0>(P, ra, rb, step + t * Fmt<KV>::kTileBytes, lane);
        }
    }
    wait_vmcnt<0>();
    __syncthreads();
    __shared__ float fs[KV == MLA_KV_MXFP4 ? 2 * 16 * kTile : 1];
    if constexpr (KV == MLA_KV_MXFP4) {
#pragma unroll
        for (int k = 0; k < 4; ++k) convert_scales(step, fs, 64 * k + lane);
        __syncthreads();
    }
    float mul = 1.0f;
    if constexpr (KV == MLA_KV_FP8_E4M3) mul = *reinterpret_cast<const float*>(P.kv_scales);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int64_t row = row0 + kTile * t + r;
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) {
            const int d0 = dbase<KV>(ks, G);
            if (path == 1 && d0 < kDv) continue;
            const bf16x8 v = qk_operand<KV>(step, t, ks, lane);
            if (kTile * t + r < n)
#pragma unroll
                for (int e = 0; e < 8; ++e) out[row * kDqk + d0 + e] = (float)v[e] * mul;
        }
    }
    if (path == 1) {
        // The value reads of each of the four attention waves (pv_load, pv_convert):
        // lane (G, n) holds column n of block c for tokens tau(G, 0..7).
        for (int w = 0; w < kWaves; ++w) {
            PvRaw<KV> v;
            pv_load<KV>(step, fs, pv_lane_offsets<KV>(lane, w), lane, w, v);
#pragma unroll
            for (int j = 0; j < (KV == MLA_KV_MXFP4 ? kWaveBlocks / 2 : kWaveBlocks); ++j) {
                const int c = (KV == MLA_KV_MXFP4 ? kWaveBlocks / 2 : kWaveBlocks) * w + j;
                bf16x8 v0, v1;
                if constexpr (KV == MLA_KV_MXFP4) pv_convert_fp4(v, j, v0, v1);
                else v0 = pv_convert<KV>(v, j);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int tk = tau(G, e);
                    if (tk >= n) continue;
                    float* o = out + (row0 + tk) * kDqk;
                    if constexpr (KV == MLA_KV_MXFP4) {
                        o[32 * c + 2 * r] = (float)v0[e];
                        o[32 * c + 2 * r + 1] = (float)v1[e];
                    } else {
                        o[16 * c + r] = (float)v0[e] * mul;
                    }
                }
            }
        }
    }
}

// Streaming read of a buffer through the attention kernels' LDS-DMA loads
// (measurement aid for the practical HBM read ceiling): workgroup w reads the
// 16-byte vectors [w n / G, (w + 1) n / G) into an LDS ring, each wave one
// 1 KiB contiguous piece per load, kStreamInFlight loads in flight per wave,
// with the non-temporal hint the cache-row gathers use. Nothing is written.
constexpr int kStreamInFlight = 8;
__global__ __launch_bounds__(256) void stream_read_kernel(const uint8_t* p, int64_t n16) {
    __shared__ __attribute__((aligned(16))) uint8_t ring[kStreamInFlight * 4096];
    const int64_t b0 = (int64_t)blockIdx.x * n16 / gridDim.x, b1 = (int64_t)(blockIdx.x + 1) * n16 / gridDim.x;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int it = 0;
    for (int64_t base = b0; base < b1; base += 256, ++it) {
        const int64_t k = min(base + (int64_t)threadIdx.x, b1 - 1);
        dma16nt<0>(p + 16 * k, lds_addr(ring + (it % kStreamInFlight) * 4096 + 1024 * wave));
        wait_vmcnt<kStreamInFlight - 1>();
    }
    wait_vmcnt<0>();
}

// Dynamic fp8 query scale, first step: part[i] = max |q| over the query rows
// of sequences [i B / n, (i + 1) B / n), n = gridDim.x (at most 256). The
// magnitude of a bf16 value orders like its low 15 bits, so the maximum is
// taken on those bits; it is exact in fp32.
__global__ __launch_bounds__(256) void q_amax_kernel(const __bf16* q, int batch, float* part) {
    __shared__ uint32_t red[4];
    const int n = gridDim.x, i = blockIdx.x, tid = threadIdx.x;
    const int64_t b0 = (int64_t)i * batch / n, b1 = (int64_t)(i + 1) * batch / n;
    const u32x4* v = reinterpret_cast<const u32x4*>(q + b0 * kHeads * kDqk);
    const int64_t cnt = (b1 - b0) * (kHeads * kDqk / 8);  // 16-byte vectors
    constexpr int kInFlight = 8;                           // loads per thread issued together
    uint32_t m = 0;
    for (int64_t base = 0; base < cnt; base += 256 * kInFlight) {
        u32x4 w[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) {
            const int64_t k = base + tid + 256 * u;
            w[u] = u32x4{0u, 0u, 0u, 0u};
            if (k < cnt) w[u] = v[k];
        }
#pragma unroll
        for (int u = 0; u < kInFlight; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) m = max(m, max(w[u][e] & 0x7fffu, (w[u][e] >> 16) & 0x7fffu));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    if (tid == 0) part[i] = __uint_as_float(max(max(red[0], red[1]), max(red[2], red[3])) << 16);
}

// Quantiser check: the e4m3fn codes of every query element, through the same
// scale reduction and code routine as the attention kernels. Workgroup b
// writes sequence b's 16 x 576 codes; workgroup 0 publishes a dynamic scale.
__global__ __launch_bounds__(256) void q8_debug_kernel(Params P, uint8_t* codes) {
    __shared__ float red[4];
    const int tid = threadIdx.x, b = blockIdx.x;
    float q_scale;
    if (P.q_amax) {
        q_scale = q8_dynamic_scale(tid < P.q_amax_n ? P.q_amax[tid] : 0.0f, red, tid);
        if (b == 0 && tid == 0) P.q_scale[0] = q_scale;
    } else {
        q_scale = *P.q_scale;
    }
    constexpr int kGroups = kHeads * kDqk / 8, kPer = (kGroups + 255) / 256;
    const bf16x8* src = reinterpret_cast<const bf16x8*>(P.q + (int64_t)b * kHeads * kDqk);
    bf16x8 g[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        g[k] = bf16x8{};
        if (tid + 256 * k < kGroups) g[k] = src[tid + 256 * k];
    }
    q8_quantise<kPer>(g, P.q + (int64_t)b * kHeads * kDqk, tid, 256, kGroups, q_scale,
                      codes + (int64_t)b * kHeads * kDqk);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

static int check_device() {
    static std::atomic<int> cache[64];  // 0 unknown, 1 gfx950, 2 other
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
    if (dev >= 0 && dev < 64) {
        int c = cache[dev].load(std::memory_order_relaxed);
        if (c == 1) return MLA_OK;
        if (c == 2) return MLA_ERR_UNSUPPORTED;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MLA_ERR_HIP;
    const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev >= 0 && dev < 64) cache[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok ? MLA_OK : MLA_ERR_UNSUPPORTED;
}

// Partial-maximum workgroups of the dynamic query scale for `batch` sequences.
static int q_amax_parts(int batch) { return batch < kQ8AmaxParts ? batch : kQ8AmaxParts; }

template <int KV, int QF>
static int launch(const mla_plan_info& plan, const Params& P, hipStream_t stream) {
    if (QF && P.q_amax) {
        hipLaunchKernelGGL(q_amax_kernel, dim3(P.q_amax_n), dim3(256), 0, stream, P.q, P.batch,
                           const_cast<float*>(P.q_amax));
        if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;
    }
    const bool turns = KV == MLA_KV_FP8_E4M3 && plan.mode == 0 && plan.rows_per_wg == 1 && plan.grid > kNumCUs &&
                       (int64_t)P.total >= (int64_t)kTurnsMinTokens * plan.grid;
    // fp8 plans of many splits per sequence load the bf16 query into registers
    // (with it through LDS, 4 x 1k at 32 splits measured 12.8 -> 13.2 us and
    // 4 x 8k at 64 splits 18.2 -> 18.9, against the same library with the
    // register query; every other shape measured 0.3 to 1.6 us faster)
    const bool q_regs = KV == MLA_KV_FP8_E4M3 && QF == 0 && plan.num_splits >= kQRegsMinSplits && !P.counters;
#define MLA_SPLIT_ARGS                                                                                             \
    dim3(plan.grid), dim3(kThreads), 0, stream, P.q, P.indices, P.kv_scales, P.kv, P.nsplit, P.uni_len,       \
        P.uni_chunk, plan.grid, P.page_size, (int)std::min<int64_t>(P.kv_rows, INT32_MAX), P
    if (plan.rows_per_wg == 2) {
        if constexpr (KV == MLA_KV_BF16 && QF == 0) {
            if (plan.mode != 0 || P.uni_q < 2) return MLA_ERR_INVALID_ARG;
            if (P.counters) hipLaunchKernelGGL((split_kernel<KV, QF, true, 2>), MLA_SPLIT_ARGS);
            else hipLaunchKernelGGL((split_kernel<KV, QF, false, 2>), MLA_SPLIT_ARGS);
        } else {
            return MLA_ERR_INVALID_ARG;  // the planner pairs rows on the bf16 cache only
        }
    } else if (turns) {
        // fp8, two workgroups per compute unit, long ranges: the two take turns at priority 2
        if constexpr (KV == MLA_KV_FP8_E4M3) {
            if (P.counters) hipLaunchKernelGGL((split_kernel<KV, QF, true, 1, true>), MLA_SPLIT_ARGS);
            else if (q_regs) hipLaunchKernelGGL((split_kernel<KV, QF, false, 1, true, false>), MLA_SPLIT_ARGS);
            else hipLaunchKernelGGL((split_kernel<KV, QF, false, 1, true>), MLA_SPLIT_ARGS);
        }
    } else if (plan.mode == 0 && P.counters) {
        hipLaunchKernelGGL((split_kernel<KV, QF, true>), MLA_SPLIT_ARGS);
    } else if (plan.mode == 0) {
        if (q_regs) {
            if constexpr (KV == MLA_KV_FP8_E4M3)
                hipLaunchKernelGGL((split_kernel<KV, QF, false, 1, false, false>), MLA_SPLIT_ARGS);
        } else {
            hipLaunchKernelGGL((split_kernel<KV, QF, false>), MLA_SPLIT_ARGS);
        }
    } else {
        // the persistent grid's shares take turns at priority 2 on the same terms as the split plans
        // (fp8 64 mixed lengths, 512 workgroups of about 1100 tokens: 79.8 -> 77.2 us together with the
        // bf16 query through LDS and the scalar kv_indptr reads)
        const bool pturns = KV == MLA_KV_FP8_E4M3 && plan.grid > kNumCUs &&
                            (int64_t)P.total >= (int64_t)kTurnsMinTokens * plan.grid;
        if (pturns) {
            if constexpr (KV == MLA_KV_FP8_E4M3) hipLaunchKernelGGL((persistent_kernel<KV, QF, true>), MLA_SPLIT_ARGS);
        } else {
            hipLaunchKernelGGL((persistent_kernel<KV, QF>), MLA_SPLIT_ARGS);
        }
    }
#undef MLA_SPLIT_ARGS
    if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;
    if (plan.combine == 1) {
        CombineParams C;
        C.part_o = P.part_o;
        C.part_lse = P.part_lse;
        C.indptr = P.indptr;
        C.out = P.out;
        C.lse = P.lse;
        C.batch = P.rows;
        C.mode = plan.mode;
        C.nsplit = plan.num_splits;
        C.grid = plan.grid;
        C.total = P.total;
        C.items = combine_items(plan.mode == 0 ? plan.num_splits : (plan.grid + P.rows - 1) / P.rows + 1);
        const int nblocks = kHeads * 4 * P.rows / C.items;
        hipLaunchKernelGGL(combine_kernel, dim3(nblocks), dim3(kCombThreads), 0, stream, C.part_o, C.part_lse, C.mode,
                           C.nsplit, C.items, nblocks, C);
        if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;
    }
    return MLA_OK;
}

}  // namespace mla

namespace mla {

// ---------------------------------------------------------------------------
// Scratch for mla_decode_noalloc: the arrival counters and split partials of
// its plans live in this file-scope device array instead of a caller
// workspace. Each device the library runs on holds its own copy (zero when
// the code object loads) until the process ends. In host code the array's
// name only stands in for the symbol: its device address is taken once per
// device with hipGetSymbolAddress (that device current) and cached, and only
// that address is ever passed to kernels.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0 && kScratchBytes > kCounterBytes, "scratch holds the counters and partials");
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex scratch_mu;
static void* scratch_ptr[kMaxDevices];  // device address of `scratch` per device (nullptr: not set up yet)

__global__ __launch_bounds__(256) void clear_u32_kernel(uint32_t* p, int n) {
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0u;
}

// The current device's scratch address. The first call on a device looks the
// symbol up and clears the arrival-counter region with a fill kernel on
// `stream` (the array starts zero; this makes that explicit, and every call
// leaves the region zero again). Returns MLA_OK or MLA_ERR_HIP.
static int scratch_for_current_device(hipStream_t stream, void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_HIP;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MLA_ERR_HIP;
        hipLaunchKernelGGL(clear_u32_kernel, dim3(16), dim3(256), 0, stream, reinterpret_cast<uint32_t*>(p),
                           (int)(kCounterBytes / sizeof(uint32_t)));
        if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return MLA_OK;
}

}  // namespace mla

namespace mla {

// Shared body of mla_decode (page size 1), mla_decode_paged and mla_decode_q8
// (q_mode < 0: bf16 query; else MLA_Q_SCALE_*, with q_scale).
// Several query tokens per sequence (mla_decode_mtp): qo_indptr / uni_q /
// causal as in Params, total_q query rows; the plan is made over the rows.
struct MtpArgs {
    const int32_t* qo_indptr = nullptr;
    int total_q = 0;
    int uni_q = 0;
    int causal = 0;
};

static int decode_impl(const void* q, const void* kv, const void* kv_scales, const int32_t* kv_indptr,
                       const int32_t* kv_indices, const int32_t* kv_last_page_len, int page_size, void* out,
                       float* lse, int batch, int64_t total_kv, int kv_dtype, float sm_scale, void* workspace,
                       size_t workspace_bytes, int flags, void* stream, int q_mode = -1, float* q_scale = nullptr,
                       const MtpArgs* mtp = nullptr, int64_t kv_rows = 0) {
    mla_plan_info plan;
    const int rows = mtp ? mtp->total_q : batch;
    int rc = mtp ? mtp_plan(batch, mtp->total_q, mtp->uni_q, total_kv, kv_dtype, flags, &plan)
                 : make_plan(batch, total_kv, kv_dtype, flags, &plan);
    if (rc != MLA_OK) return rc;
    const bool dyn = q_mode == MLA_Q_SCALE_DYNAMIC;
    const size_t need = dyn ? q8_amax_offset(plan.workspace_bytes) + kQ8AmaxParts * sizeof(float)
                            : plan.workspace_bytes;
    if (batch == 0 || rows == 0) return MLA_OK;
    if (q_mode >= 0 && (!q_scale || !aligned(q_scale, 4))) return MLA_ERR_INVALID_ARG;
    if (mtp && mtp->uni_q == 0 && (!mtp->qo_indptr || !aligned(mtp->qo_indptr, 4))) return MLA_ERR_INVALID_ARG;
    if (!q || !kv || !kv_indptr || !out || kv_rows < 0) return MLA_ERR_INVALID_ARG;
    if (total_kv > 0 && !kv_indices) return MLA_ERR_INVALID_ARG;
    if (kv_dtype != MLA_KV_BF16 && !kv_scales) return MLA_ERR_INVALID_ARG;
    if (page_size > 1 && (!kv_last_page_len || !aligned(kv_last_page_len, 4))) return MLA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(out, 16) || !aligned(kv_indptr, 4) ||
        (kv_indices && !aligned(kv_indices, 4)) || (lse && !aligned(lse, 4)) ||
        (kv_dtype == MLA_KV_FP8_E4M3 && !aligned(kv_scales, 4)))
        return MLA_ERR_INVALID_ARG;
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return MLA_ERR_WORKSPACE_TOO_SMALL;
        if (!aligned(workspace, 16)) return MLA_ERR_INVALID_ARG;
    }
    rc = check_device();
    if (rc != MLA_OK) return rc;

    Params P;
    P.q = reinterpret_cast<const __bf16*>(q);
    P.kv = reinterpret_cast<const uint8_t*>(kv);
    P.kv_scales = kv_scales;
    P.indptr = kv_indptr;
    P.indices = kv_indices;
    P.last_page = kv_last_page_len;
    P.page_size = page_size;
    P.out = reinterpret_cast<__bf16*>(out);
    P.lse = lse;
    // workspace: arrival counters, then the partials (O, then lse)
    P.part_o = plan.num_partials ? reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + kCounterBytes)
                                 : nullptr;
    P.part_lse = plan.num_partials ? reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                                             partial_lse_offset(plan.num_partials))
                                   : nullptr;
    P.counters = plan.combine == 2 ? reinterpret_cast<uint32_t*>(workspace) : nullptr;
    P.kv_rows = kv_rows;
    P.batch = batch;
    P.nsplit = plan.num_splits;
    P.grid = plan.grid;
    P.total = (int)total_kv;
    P.sm_scale = (sm_scale > 0.f) ? sm_scale : 1.0f / 24.0f;  // NaN compares false -> default
    P.q_scale = q_scale;
    P.q_amax = dyn ? reinterpret_cast<const float*>(reinterpret_cast<char*>(workspace) +
                                                    q8_amax_offset(plan.workspace_bytes))
                   : nullptr;
    P.q_amax_n = dyn ? q_amax_parts(batch) : 0;
    P.qo_indptr = mtp ? mtp->qo_indptr : nullptr;
    P.uni_q = mtp ? mtp->uni_q : 0;
    P.causal = mtp ? mtp->causal : 0;
    P.rows = rows;
    P.uni_len = 0;
    P.uni_chunk = 0;
    // With pages, only for a power-of-two page size (run_wg expands the
    // staged page entries with shifts) and a common length that is a whole
    // number of pages: then the batch holds at least batch * Lu / page_size
    // page entries whatever its lengths, so the guessed window never reads
    // past kv_indices.
    if (plan.mode == 0 && !mtp && total_kv > 0 && total_kv % batch == 0 && (page_size & (page_size - 1)) == 0 &&
        (total_kv / batch) % page_size == 0) {
        const int Lu = (int)(total_kv / batch), ns = plan.num_splits;
        P.uni_len = Lu;
        P.uni_chunk = ((Lu + ns - 1) / ns + kStepTokens - 1) / kStepTokens * kStepTokens;  // as the kernel splits
    }

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (q_mode >= 0) {
        switch (kv_dtype) {
            case MLA_KV_BF16: return launch<MLA_KV_BF16, 1>(plan, P, s);
            case MLA_KV_FP8_E4M3: return launch<MLA_KV_FP8_E4M3, 1>(plan, P, s);
            default: return launch<MLA_KV_MXFP4, 1>(plan, P, s);
        }
    }
    switch (kv_dtype) {
        case MLA_KV_BF16: return launch<MLA_KV_BF16, 0>(plan, P, s);
        case MLA_KV_FP8_E4M3: return launch<MLA_KV_FP8_E4M3, 0>(plan, P, s);
        default: return launch<MLA_KV_MXFP4, 0>(plan, P, s);
    }
}

}  // namespace mla

extern "C" int mla_decode(const void* q, const void* kv, const void* kv_scales, const int32_t* kv_indptr,
                          const int32_t* kv_indices, void* out, float* lse, int batch, int64_t total_kv,
                          int kv_dtype, float sm_scale, void* workspace, size_t workspace_bytes, int flags,
                          void* stream) {
    return mla::decode_impl(q, kv, kv_scales, kv_indptr, kv_indices, nullptr, 1, out, lse, batch, total_kv, kv_dtype,
                            sm_scale, workspace, workspace_bytes, flags, stream);
}

extern "C" int mla_decode_noalloc(const void* q, const void* kv, const void* kv_scales, const int32_t* kv_indptr,
                                  const int32_t* kv_indices, void* out, float* lse, int batch, int64_t total_kv,
                                  int kv_dtype, float sm_scale, int flags, void* stream) {
    using namespace mla;
    mla_plan_info plan;
    int rc = make_plan(batch, total_kv, kv_dtype, flags, &plan);
    if (rc != MLA_OK) return rc;
    if (plan.workspace_bytes > kScratchBytes) return MLA_ERR_WORKSPACE_TOO_SMALL;  // before any device call
    void* ws = nullptr;
    if (plan.workspace_bytes > 0 && batch > 0) {
        rc = check_device();
        if (rc != MLA_OK) return rc;
        rc = scratch_for_current_device(reinterpret_cast<hipStream_t>(stream), &ws);
        if (rc != MLA_OK) return rc;
    }
    return decode_impl(q, kv, kv_scales, kv_indptr, kv_indices, nullptr, 1, out, lse, batch, total_kv, kv_dtype,
                       sm_scale, ws, ws ? kScratchBytes : 0, flags, stream);
}

extern "C" int mla_decode_rows(const void* q, const void* kv, const void* kv_scales, const int32_t* kv_indptr,
                               const int32_t* kv_indices, void* out, float* lse, int batch, int64_t total_kv,
                               int64_t kv_rows, int kv_dtype, float sm_scale, void* workspace, size_t workspace_bytes,
                               int flags, void* stream) {
    return mla::decode_impl(q, kv, kv_scales, kv_indptr, kv_indices, nullptr, 1, out, lse, batch, total_kv, kv_dtype,
                            sm_scale, workspace, workspace_bytes, flags, stream, -1, nullptr, nullptr, kv_rows);
}

extern "C" int mla_decode_paged(const void* q, const void* kv, const void* kv_scales, const int32_t* kv_indptr,
                                const int32_t* kv_indices, const int32_t* kv_last_page_len, int page_size, void* out,
                                float* lse, int batch, int64_t total_kv, int kv_dtype, float sm_scale,
                                void* workspace, size_t workspace_bytes, int flags, void* stream) {
    if (page_size < 1 || page_size > (1 << 16)) return MLA_ERR_INVALID_ARG;
    if (page_size > 1) {
        // the persistent partition needs token offsets of every sequence, which
        // paged caches do not carry: paged calls always plan split-K
        if (flags & MLA_FLAG_FORCE_PERSISTENT) return MLA_ERR_INVALID_ARG;
        flags |= MLA_FLAG_FORCE_SPLIT;
    }
    return mla::decode_impl(q, kv, kv_scales, kv_indptr, kv_indices, kv_last_page_len, page_size, out, lse, batch,
                            total_kv, kv_dtype, sm_scale, workspace, workspace_bytes, flags, stream);
}

extern "C" int mla_decode_q8(const void* q, float* q_scale, int q_scale_mode, const void* kv, const void* kv_scales,
                             const int32_t* kv_indptr, const int32_t* kv_indices, const int32_t* kv_last_page_len,
                             int page_size, void* out, float* lse, int batch, int64_t total_kv, int kv_dtype,
                             float sm_scale, void* workspace, size_t workspace_bytes, int flags, void* stream) {
    if (q_scale_mode != MLA_Q_SCALE_STATIC && q_scale_mode != MLA_Q_SCALE_DYNAMIC) return MLA_ERR_INVALID_ARG;
    if (page_size < 1 || page_size > (1 << 16)) return MLA_ERR_INVALID_ARG;
    if (page_size > 1) {
        if (flags & MLA_FLAG_FORCE_PERSISTENT) return MLA_ERR_INVALID_ARG;
        flags |= MLA_FLAG_FORCE_SPLIT;
    }
    return mla::decode_impl(q, kv, kv_scales, kv_indptr, kv_indices, kv_last_page_len, page_size, out, lse, batch,
                            total_kv, kv_dtype, sm_scale, workspace, workspace_bytes, flags, stream, q_scale_mode,
                            q_scale);
}

extern "C" int mla_decode_mtp(const void* q, const int32_t* qo_indptr, int total_q, int uni_q_len, int causal,
                              const void* kv, const void* kv_scales, const int32_t* kv_indptr,
                              const int32_t* kv_indices, const int32_t* kv_last_page_len, int page_size, void* out,
                              float* lse, int batch, int64_t total_kv, int kv_dtype, float sm_scale, void* workspace,
                              size_t workspace_bytes, int flags, void* stream) {
    if (page_size < 1 || page_size > (1 << 16) || total_q < 0 || uni_q_len < 0 || causal < 0 || causal > 1)
        return MLA_ERR_INVALID_ARG;
    if (uni_q_len > 0 && (int64_t)uni_q_len * batch != total_q) return MLA_ERR_INVALID_ARG;
    if (flags & MLA_FLAG_FORCE_PERSISTENT) return MLA_ERR_INVALID_ARG;
    mla::MtpArgs m;
    m.qo_indptr = qo_indptr;
    m.total_q = total_q;
    m.uni_q = uni_q_len;
    m.causal = causal;
    return mla::decode_impl(q, kv, kv_scales, kv_indptr, kv_indices, kv_last_page_len, page_size, out, lse, batch,
                            total_kv, kv_dtype, sm_scale, workspace, workspace_bytes, flags, stream, -1, nullptr, &m);
}

extern "C" int mla_quantize_q8_debug(const void* q, int batch, float* q_scale, int q_scale_mode, uint8_t* codes,
                                     void* workspace, size_t workspace_bytes, void* stream) {
    using namespace mla;
    if (q_scale_mode != MLA_Q_SCALE_STATIC && q_scale_mode != MLA_Q_SCALE_DYNAMIC) return MLA_ERR_INVALID_ARG;
    if (batch < 0) return MLA_ERR_INVALID_ARG;
    if (batch == 0) return MLA_OK;
    if (!q || !q_scale || !codes || !aligned(q, 16) || !aligned(q_scale, 4) || !aligned(codes, 8))
        return MLA_ERR_INVALID_ARG;
    const bool dyn = q_scale_mode == MLA_Q_SCALE_DYNAMIC;
    if (dyn && (!workspace || workspace_bytes < kQ8AmaxParts * sizeof(float))) return MLA_ERR_WORKSPACE_TOO_SMALL;
    if (dyn && !aligned(workspace, 16)) return MLA_ERR_INVALID_ARG;
    int rc = check_device();
    if (rc != MLA_OK) return rc;
    Params P;
    memset(&P, 0, sizeof P);
    P.q = reinterpret_cast<const __bf16*>(q);
    P.batch = batch;
    P.q_scale = q_scale;
    P.q_amax = dyn ? reinterpret_cast<const float*>(workspace) : nullptr;
    P.q_amax_n = dyn ? q_amax_parts(batch) : 0;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (dyn) {
        hipLaunchKernelGGL(q_amax_kernel, dim3(P.q_amax_n), dim3(256), 0, s, P.q, batch,
                           reinterpret_cast<float*>(workspace));
        if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;
    }
    hipLaunchKernelGGL(q8_debug_kernel, dim3(batch), dim3(256), 0, s, P, codes);
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

#if MLA_PHASE_STAMPS
// Measurement build only (include/mla_decode_phases.h).
extern "C" int mla_phase_buffers(uint64_t* stage1, uint64_t* combine) {
    using namespace mla;
    int rc = check_device();
    if (rc != MLA_OK) return rc;
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_phase_stage1), &stage1, sizeof stage1) != hipSuccess) return MLA_ERR_HIP;
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_phase_combine), &combine, sizeof combine) != hipSuccess) return MLA_ERR_HIP;
    return MLA_OK;
}
#endif

extern "C" int mla_hbm_read_probe(const void* buf, size_t bytes, void* stream) {
    using namespace mla;
    if (bytes == 0) return MLA_OK;
    if (!buf || !aligned(buf, 16) || bytes % 16 != 0) return MLA_ERR_INVALID_ARG;
    int rc = check_device();
    if (rc != MLA_OK) return rc;
    const int64_t n16 = (int64_t)(bytes / 16);
    const int grid = n16 < 2 * kNumCUs ? (int)n16 : 2 * kNumCUs;  // two workgroups per compute unit
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                       reinterpret_cast<const uint8_t*>(buf), n16);
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

extern "C" int mla_dequant_debug(int kv_dtype, const void* kv, const void* kv_scales, int64_t rows, int path,
                                 float* out_f32, void* stream) {
    using namespace mla;
    if (kv_dtype < MLA_KV_BF16 || kv_dtype > MLA_KV_MXFP4 || rows < 0 || rows > INT32_MAX || path < 0 || path > 1)
        return MLA_ERR_INVALID_ARG;
    if (rows == 0) return MLA_OK;
    if (!kv || !out_f32 || (kv_dtype != MLA_KV_BF16 && !kv_scales)) return MLA_ERR_INVALID_ARG;
    if (!aligned(kv, 16) || !aligned(out_f32, 4)) return MLA_ERR_INVALID_ARG;
    int rc = check_device();
    if (rc != MLA_OK) return rc;
    Params P;
    memset(&P, 0, sizeof P);
    P.kv = reinterpret_cast<const uint8_t*>(kv);
    P.kv_scales = kv_scales;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)((rows + kStepTokens - 1) / kStepTokens));
    switch (kv_dtype) {
        case MLA_KV_BF16: hipLaunchKernelGGL(dequant_kernel<MLA_KV_BF16>, grid, dim3(64), 0, s, P, rows, path, out_f32); break;
        case MLA_KV_FP8_E4M3: hipLaunchKernelGGL(dequant_kernel<MLA_KV_FP8_E4M3>, grid, dim3(64), 0, s, P, rows, path, out_f32); break;
        default: hipLaunchKernelGGL(dequant_kernel<MLA_KV_MXFP4>, grid, dim3(64), 0, s, P, rows, path, out_f32); break;
    }
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

/*
 * Phase timestamps of the MLA decode kernels: a measurement aid, not part of
 * the decode. Only the measurement build of the library
 * (mla_decode_02_amd/libmla_decode_phases.so, the same sources compiled with
 * MLA_PHASE_STAMPS=1) exports this; the decode library libmla_decode.so does
 * not, and its kernels record nothing.
 *
 * In the measurement build, thread 0 of every stage-1 workgroup writes the
 * 100 MHz real-time counter (s_memrealtime, one tick = 10 ns) at eight phase
 * slots, stage1[workgroup * 8 + phase]:
 *   0 kernel entry
 *   1 the query registers and the first index window in hand
 *   2 the first step's cache rows landed in LDS
 *   3 every step of the workgroup's token range done
 *   4 the epilogue's stores complete (all threads)
 *   5 the stage-1 merge done (plans merged in stage 1; otherwise as 4)
 *   6, 7 unused
 * A persistent workgroup attends several sequences; phases 1-4 are those of
 * its last one. Thread 0 of every combine workgroup writes its start and end
 * (after its stores), combine[workgroup * 2 + {0, 1}]. Workgroup indices are
 * launch order (blockIdx.x).
 */
#ifndef MLA_DECODE_PHASES_H
#define MLA_DECODE_PHASES_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * mla_phase_buffers: set the device buffers the next launches write their
 * stamps into (NULL: record nothing). stage1 holds at least grid * 8 and
 * combine at least (combine workgroups) * 2 uint64 for every launch that
 * follows; the caller owns both. A blocking copy to two device symbols; call
 * it before enqueueing the calls to be measured.
 * Returns MLA_OK, MLA_ERR_UNSUPPORTED or MLA_ERR_HIP.
 */
int mla_phase_buffers(uint64_t* stage1, uint64_t* combine);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_PHASES_H */

/*
 * bwa_diag.h -- diagnostic entry point of the bwa library (include/bwa.h).
 *
 * The library can be built a second time with BWA_SLOT_TIMERS=1
 * (libbwa_slot_timers.so, built beside libbwa.so).  In that build the bf16
 * forward kernel (the block-pair kernel behind bwa_partial_fwd and
 * bwa_ring_fwd) reads the shader clock around the phases of its per-tile
 * loop, so that the time a tile spends in its VALU phase, its staging step,
 * its MFMA phase and the two barriers between them can be read back.  It
 * computes the same results as the default build; reading the clock makes it
 * slightly slower.  In the default build the kernel carries no clock reads
 * and the entry point below reports BWA_ERR_UNSUPPORTED.
 */
#ifndef BWA_DIAG_H_
#define BWA_DIAG_H_

#include <stdint.h>

#include "bwa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Number of int64 fields per record, and the number of records the
 * diagnostic build keeps (workgroups past it do not record). */
#define BWA_SLOT_FIELDS 6
#define BWA_SLOT_RECORDS 4096

/*
 * bwa_fwd_slot_timers -- copy the phase clocks of the most recent bf16
 * forward launch on the current device to host memory.
 *   out         HOST buffer of max_records * 2 * BWA_SLOT_FIELDS int64, owned
 *               by the caller.  Record w (workgroup w of the launch, in launch
 *               order) holds two rows of BWA_SLOT_FIELDS values, wave 0 (the
 *               first wave group) then wave 4 (the second): cycles summed over
 *               the workgroup's KV tiles in [0] the VALU phase (mask,
 *               exponentials, row sums, bf16 probabilities), [1] the staging
 *               step (wait for the landed tile, issue the next tile's loads),
 *               [2] the barrier opening the MFMA slot, [3] the MFMA phase,
 *               [4] the barrier closing it; [5] is the number of tiles.  A
 *               workgroup with no visible tile reports zeros.
 *   max_records records to copy (at most BWA_SLOT_RECORDS are copied).
 *   n_records   out: BWA_SLOT_RECORDS in the diagnostic build, 0 otherwise.
 * Synchronizes the device first.  Returns BWA_ERR_INVALID_ARG for a null
 * pointer or a negative count, BWA_ERR_UNSUPPORTED in the default build,
 * BWA_ERR_HIP if the copy fails.  The clocks are cleared at every forward
 * launch, so in a ring of several launches (ROUNDS mode) the last one's are
 * read.
 */
int bwa_fwd_slot_timers(long long* out, int64_t max_records, int64_t* n_records);

#ifdef __cplusplus
}
#endif

#endif /* BWA_DIAG_H_ */

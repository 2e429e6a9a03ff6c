/*
 * lgm_probe.h — measurement support for liblgm: the read-only streaming
 * ceiling that decode bandwidth is reported against.  The mainarch README's
 * decode-attention section measures a pure streaming read of device memory
 * and grades every decode kernel against that ceiling as well as against the
 * HBM peak; this entry point is that read.  It is not part of the attention
 * path and shares its error conventions (lgm.h): every argument is checked
 * before any HIP call, a violation returns a nonzero lgm_status with
 * lgm_last_error() naming the argument, and nothing is enqueued.
 */
#ifndef LGM_PROBE_H
#define LGM_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "lgm.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read `bytes` bytes of device memory at `src` once, with 16-byte loads.
 * Workgroup w of `num_workgroups` reads the contiguous chunk
 * [w * bytes / num_workgroups, (w + 1) * bytes / num_workgroups).
 *   src           device pointer, 16-byte aligned; only read.
 *   bytes         a positive multiple of num_workgroups * 16384; each chunk
 *                 at most INT32_MAX bytes.
 *   num_workgroups in [1, 65536].
 *   nontemporal   nonzero: loads carry the non-temporal cache hint (the hint
 *                 the whole-row decode kernel uses for K/V); zero: default.
 *   sink          device pointer to one uint32; written only if the XOR of
 *                 the words a workgroup read equals 0x9E3779B9 (keeps the
 *                 loads live; its value means nothing).
 *   stream        hipStream_t as void*; asynchronous.
 * Errors: LGM_ERR_INVALID_ARGUMENT for a NULL or misaligned pointer, a size
 * that is not such a multiple, or an overlap of src and sink; LGM_ERR_HIP if
 * the launch fails.
 */
lgm_status lgm_stream_read_probe(const void* src, size_t bytes, int32_t num_workgroups, int32_t nontemporal,
                                 uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LGM_PROBE_H */

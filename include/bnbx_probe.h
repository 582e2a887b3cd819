/*
 * bnbx_probe.h -- measurement aid of libbnbx (gfx950).
 *
 * A plain streaming read: the rate at which this GPU can stream a given
 * number of bytes from HBM in one launch, with nothing else to do.  The
 * decode GEMV reads its packed weights and their block codes once per launch
 * (mlqm.cn bitsandbytes article, sec. 3.4: the 4-bit weights are what the
 * layer streams), so timing this read over the same two buffers, back to
 * back like the GEMV launches, gives the achievable ceiling that the GEMV's
 * fraction of the HBM peak is read against.  Not part of the method.
 *
 * Conventions as in bnbx.h (device pointers, caller-owned buffers, work
 * enqueued on `stream`, host-side argument checks before any launch).
 */
#ifndef BNBX_PROBE_H
#define BNBX_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "bnbx.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Words of `sink` that bnbx_probe_stream_read may write (one per
 * workgroup). */
#define BNBX_PROBE_SINK_WORDS 1024

/* Reads a_bytes at a, then b_bytes at b, once each with 16-byte loads, and
 * writes to sink[w] the XOR of all 32-bit words that workgroup w read (so
 * the XOR of the written sink words is the XOR of every word of both
 * buffers; unwritten sink words are left as they were).
 *   a, b     device, 16-byte aligned; b may be NULL when b_bytes is 0
 *   a_bytes, b_bytes  multiples of 16; a_bytes + b_bytes > 0
 *   sink     device, uint32[BNBX_PROBE_SINK_WORDS]
 * Errors: BNBX_E_INVAL (a NULL with a_bytes > 0, b NULL with b_bytes > 0,
 * sink NULL, both sizes 0, a size not a multiple of 16), BNBX_E_ALIGN,
 * BNBX_E_HIP. */
BNBX_API int bnbx_probe_stream_read(const void* a, size_t a_bytes, const void* b, size_t b_bytes,
                                    uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BNBX_PROBE_H */

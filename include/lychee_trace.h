/*
 * lychee_trace.h -- phase timestamps of the attention kernel, exported only
 * by the LYCHEE_TRACE build of the library (liblychee_trace.so, built with
 * `python -m hybrid_head_sparse_amd.build --trace`).  A measuring aid, not
 * part of the decode path: the timestamps show where a layer's time goes
 * (prologue, streaming, selection hand-off, record merge, top-k resolve).
 */
#ifndef LYCHEE_TRACE_H
#define LYCHEE_TRACE_H

#include <stdint.h>

#include "lychee.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Route the phase timestamps of the following attention launches on this
 * handle into `buffer` (device memory, caller-owned; NULL stops), as 32
 * 64-bit words per workgroup at ((launch * grid) + workgroup) * 32, grid =
 * the compute units of the device.  Words 0-10 are s_memrealtime stamps
 * (100 MHz) of: entry, prologue done, first head start, streaming done,
 * selection arrival, record complete, record arrival, merge done, resolve
 * start, resolve end, exit (0 where a phase did not occur); word 11 holds
 * flags (1 retrieval head, 2 sparse head, 4 merger, 8 resolver as last
 * arrival, 32 full-scan resolve), word 12 the heads the range touched,
 * words 13-15 the candidate resolver's sizes (units | T << 32, threshold
 * group | count above T << 32, k_eff | workgroups << 32), words 16-26
 * stamps of its phases, word 27 a sparse head's S entries staged and words
 * 28-31 phases of the prologue (read by hybrid_head_sparse_amd/timeline.py).  The buffer must hold (launch + 1) * grid * 256
 * bytes. */
lychee_status lychee_set_trace(lychee_handle* h, void* buffer, uint32_t launch);

#ifdef __cplusplus
}
#endif

#endif /* LYCHEE_TRACE_H */

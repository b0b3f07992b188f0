/*
 * ssd_probe.h -- HBM stream probes of the MI355X SSD library (measurement only).
 *
 * These calls are not part of the method; they measure the DRAM rate that plain streaming
 * kernels reach on the same chip, so that the SSD kernels' achieved bandwidth can be set
 * against a measured ceiling as well as against the 8 TB/s HBM3E peak. Each launches one
 * grid-stride kernel on `stream` (a hipStream_t; NULL means the null stream) and returns
 * without synchronising; time them with events on that stream.
 *
 *   ssd_probe_read   reads `bytes` from src and folds them into one 16-byte value that is
 *                    written to sink only if it equals an impossible pattern (so the loads
 *                    cannot be dropped); sink must hold 16 bytes.
 *   ssd_probe_write  writes `bytes` of a constant pattern to dst.
 *   ssd_probe_copy   copies `bytes` from src to dst (the buffers must not overlap).
 *   ssd_probe_mix    reads `read_bytes` from src and writes `write_bytes` to dst in one pass,
 *                    loads and stores in that proportion all along the run (the stream mix
 *                    of a kernel that reads R and writes W bytes); either size may be 0.
 *
 * `bytes` (for ssd_probe_mix the larger of the two sizes) must be a positive multiple of 16 and every pointer 16-byte aligned (else
 * SSD_ERR_SHAPE or SSD_ERR_ALIGN from ssd.h's status codes, nothing enqueued). `mode` 0 uses
 * ordinary vector loads and stores, 1 non-temporal ones (others: SSD_ERR_UNSUPPORTED).
 * `workgroups` sets the grid (256 threads each; 0 picks 8 per compute unit).
 * The caller owns every buffer; nothing is allocated.
 */
#ifndef SSD_MI355X_PROBE_H
#define SSD_MI355X_PROBE_H

#include <stddef.h>

#include "ssd.h"

#ifdef __cplusplus
extern "C" {
#endif

ssd_status ssd_probe_read(const void* src, size_t bytes, void* sink, int mode, int workgroups,
                          void* stream);
ssd_status ssd_probe_write(void* dst, size_t bytes, int mode, int workgroups, void* stream);
ssd_status ssd_probe_copy(const void* src, void* dst, size_t bytes, int mode, int workgroups,
                          void* stream);
ssd_status ssd_probe_mix(const void* src, size_t read_bytes, void* dst, size_t write_bytes,
                         int mode, int workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SSD_MI355X_PROBE_H */

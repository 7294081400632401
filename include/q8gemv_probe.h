/*
 * Measurement helpers that ship with q8gemv (not part of the GEMV path).
 *
 * The pure-read probe gives the measured ceiling of the HBM read path in the
 * same session as the GEMV timings, as "One level down: #002 the same compiler
 * on a GPU" does in section "Decode: memory decides" (a matvec is compared
 * with a pure-read probe on the same card). The flush evicts the last-level
 * cache before a cold-cache timing.
 *
 * Pointers are device pointers owned by the caller; `stream` is a hipStream_t.
 * Nothing is allocated or synchronized. Status codes are those of q8gemv.h.
 */
#ifndef Q8GEMV_PROBE_H
#define Q8GEMV_PROBE_H

#include <stdint.h>

#include "q8gemv.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Number of uint32 words `sink` must hold for q8g_probe_read. */
#define Q8G_PROBE_SINK_WORDS 16384

/* Read `bytes` of `src` once with 16-byte loads (bytes % 16 == 0, src 16-byte
 * aligned), with nontemporal loads, and write one xor digest per workgroup
 * into sink[0..16383], so the loads cannot be dropped. The grid is sized to
 * the buffer (about eight loads per thread, at most 16384 workgroups). */
q8g_status q8g_probe_read(const void *src, int64_t bytes, uint32_t *sink, void *stream);

/* The same read with plain (cached) loads, the kind the kernels use for data
 * that other workgroups reuse; with the nontemporal probe it calibrates the
 * hardware read counters for both kinds of load. */
q8g_status q8g_probe_read_cached(const void *src, int64_t bytes, uint32_t *sink, void *stream);

/* Overwrite `bytes` of `buf` (bytes % 16 == 0, 16-byte aligned) with `value`
 * in every 32-bit word. */
q8g_status q8g_flush(void *buf, int64_t bytes, uint32_t value, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* Q8GEMV_PROBE_H */

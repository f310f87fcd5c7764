/*
 * probe.h -- measurement kernels in libcfc.so (gfx950): a measured
 * denominator for the VALU roofline of the recurrence kernels.
 *
 * The recurrence of one sample runs on one compute unit, as plain
 * (non-packed) fp32 FMAs on the vector ALUs.  The datasheet fp32 vector peak
 * counts packed FMAs on every compute unit, so it is not the rate such a
 * kernel can reach.  cfc_probe_fma runs independent FMA chains on a chosen
 * number of workgroups and threads, so the rate that `blocks` compute units
 * sustain for this instruction mix can be timed on the device itself.
 *
 * Conventions shared with cfc.h: `out` is a DEVICE pointer owned by the
 * caller; `stream` is a hipStream_t (NULL = null stream); the call only
 * enqueues; it returns CFC_OK or a negative cfc_status with cfc_last_error()
 * set.
 */
#ifndef CFC_PROBE_H
#define CFC_PROBE_H

#include <stddef.h>

#include "cfc.h"

#ifdef __cplusplus
extern "C" {
#endif

/* FMA-rate probe.  Launches `blocks` workgroups of `threads` lanes; every
 * lane runs 8 independent chains x <- fma(x, m, c) (non-packed fp32,
 * v_fma_f32), 8 links per chain per iteration, for `iters` iterations, so
 * the launch performs 2 * 64 * iters * blocks * threads flops.  With
 * one_per_cu != 0 each workgroup reserves 96 KiB of LDS, so no compute unit
 * holds two of them (the persistent K-loop kernel's residency).  Lane i of
 * workgroup w writes the sum of its chains to out[w * threads + i].
 *   blocks in [1, 65536]; threads a multiple of 64 in [64, 1024];
 *   iters in [1, 2^20]; out [blocks * threads] floats.
 * Errors: CFC_EINVAL for sizes out of range or out == NULL. */
int cfc_probe_fma(int blocks, int threads, int one_per_cu, int iters, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CFC_PROBE_H */

/*
 * kq_tune.h -- launch-shape controls of libkq, for benchmark sweeps only.
 *
 * Not part of the operational ABI in kq.h: production callers never need
 * these.  They change how a matvec is split over the GPU, never what it
 * computes (results stay within the documented tolerance and remain
 * deterministic for a fixed shape).
 */
#ifndef KQ_TUNE_H
#define KQ_TUNE_H

#include <stdint.h>

#include "kq.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Process-wide override of the launch shape of the M = 1 matvec of `qtype`
 * (KQ_QTYPE_Q4K or KQ_QTYPE_Q6K): `lanes` lanes per weight row (4, 8, 16, 32
 * or 64), `waves` wavefronts per workgroup (1..16), `grid` workgroups.  A zero
 * field keeps the automatic choice for that field; all zeros restores it.
 * Not thread-safe against concurrent matvec calls.
 * Errors: KQ_ERR_SHAPE for an unknown qtype or an out-of-range field.
 */
kq_status kq_tune_set_shape(int qtype, int lanes, int waves, int grid);

/*
 * The launch shape the current settings give a matvec of n_rows x k on the
 * current device.  Outputs are host pointers.
 * Errors: KQ_ERR_SHAPE, KQ_ERR_NULL, KQ_ERR_UNSUPPORTED, KQ_ERR_DEVICE.
 */
kq_status kq_tune_get_shape(int qtype, int64_t n_rows, int64_t k, int *lanes, int *waves,
                            int *grid);

#ifdef __cplusplus
}
#endif

#endif /* KQ_TUNE_H */

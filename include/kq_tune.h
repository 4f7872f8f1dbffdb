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
 * (KQ_QTYPE_Q4K, KQ_QTYPE_Q5K or KQ_QTYPE_Q6K): `lanes` lanes per weight row (4, 8, 16, 32
 * or 64), `waves` wavefronts per workgroup (1..16), `grid` workgroups,
 * `depth` half-superblock units kept in flight per lane (1..3).  A zero field
 * keeps the automatic choice for that field; all zeros restores it.
 * Not thread-safe against concurrent matvec calls.
 * Errors: KQ_ERR_SHAPE for an unknown qtype or an out-of-range field.
 */
kq_status kq_tune_set_shape(int qtype, int lanes, int waves, int grid, int depth);

/*
 * The launch shape the current settings give a matvec of n_rows x k on the
 * current device.  Outputs are host pointers.
 * Errors: KQ_ERR_SHAPE, KQ_ERR_NULL, KQ_ERR_UNSUPPORTED, KQ_ERR_DEVICE.
 */
kq_status kq_tune_get_shape(int qtype, int64_t n_rows, int64_t k, int *lanes, int *waves,
                            int *grid, int *depth);

/*
 * The automatic launch shape of an M = 1 matvec of n_rows x k (staged != 0:
 * on a staged input) on a device of `cus` compute units, ignoring any
 * kq_tune_set_shape override (host arithmetic only; no device is touched),
 * written to the host array out[6]: lanes per row, waves per workgroup,
 * workgroups, depth, LDS bytes per workgroup (the activation staging), and
 * workgroups per CU the grid is sized for.
 *   n_rows >= 1, 1 <= cus <= 4096; qtype and k as for the matvecs.
 * Errors: KQ_ERR_SHAPE, KQ_ERR_UNSUPPORTED, KQ_ERR_NULL.
 */
kq_status kq_tune_matvec_plan(int qtype, int64_t n_rows, int64_t k, int staged, int cus,
                              int64_t *out);

/*
 * The launch plan kq_matmul_small_m would use for this shape on a device of
 * `cus` compute units (host arithmetic only; no device is touched), written
 * to the host array out[6]: workgroups, superblocks in a workgroup's staged
 * activation window, LDS bytes per workgroup, workspace bytes (as
 * kq_matmul_small_m_workspace_bytes on such a device), threads per
 * workgroup, tiles (256-row groups x superblocks per row).
 *   n_rows >= 1, 2 <= m <= KQ_MAX_M, 1 <= cus <= 4096; qtype and k as for
 *   kq_matmul_small_m.
 * Errors: KQ_ERR_SHAPE, KQ_ERR_UNSUPPORTED, KQ_ERR_NULL.
 */
kq_status kq_tune_small_m_plan(int qtype, int64_t n_rows, int64_t k, int m, int cus, int64_t *out);

/*
 * Process-wide choice between the two kernels of kq_matmul_small_m (and of
 * kq_matmul_small_m_noalloc and kq_ffn_gate_up_q4k_small_m): activation
 * counts 2 <= M <= max_m of `qtype` (KQ_QTYPE_Q4K or KQ_QTYPE_Q6K) run the
 * matvec's integer dot path (each workgroup stages all M rows into LDS and
 * applies every weight unit to each; no workspace), where the staged rows fit
 * the LDS; larger M the matrix-core kernel.  The default max_m is 2 for
 * Q4_K and 0 for Q6_K; max_m 0 sends every M >= 2 to the matrix-core kernel;
 * -1 restores the default.  Both give results within the matvec tolerance,
 * and each row of the dot path equals the 8-lane matvec of that row bit for
 * bit.  The workspace size follows the choice.  Not thread-safe against
 * concurrent calls.
 * Errors: KQ_ERR_SHAPE for an unknown qtype or max_m outside -1..4.
 */
kq_status kq_tune_set_small_m_rows(int qtype, int max_m);

/*
 * Process-wide choice for kq_ffn_gate_up_q4k_small_m: activation counts
 * 2 <= M <= max_m (where the staged rows fit the LDS) run gate and up through
 * the matvec's integer dot path in one launch (each row task streams its gate
 * row's units, then its up row's; no workspace), and each output row then
 * equals kq_ffn_gate_up_q4k of that activation row bit for bit.  Larger M run
 * the two small-M launches.  max_m 0 disables it; -1 restores the default (3).
 * Not thread-safe against concurrent calls.
 * Errors: KQ_ERR_SHAPE for max_m outside -1..4.
 */
kq_status kq_tune_set_gate_up_rows(int max_m);

/*
 * Read-stream probe (benchmark only): reads every byte of the device buffer
 * `buf` once with 16-byte loads over `grid` workgroups of `block` threads and
 * writes grid*block/64 xor-folded words to the device buffer `out` (so the
 * loads cannot be dropped).  Its duration gives the measured HBM read ceiling
 * the matvec bandwidths are compared with.
 *   bytes   multiple of 16; buf 16-byte aligned; out [grid*block/64] uint32.
 *   block   64..1024, a multiple of 64.
 *   unroll  1, 4, 8 or 16 loads in flight per thread.
 *   flags   bit 0: non-temporal loads; bit 1: each workgroup reads one
 *           contiguous chunk (else the grid strides over the buffer).
 * Errors: KQ_ERR_NULL, KQ_ERR_SHAPE, KQ_ERR_ALIGN, KQ_ERR_ALIAS, KQ_ERR_LAUNCH,
 * KQ_ERR_DEVICE.
 */
kq_status kq_probe_read_bw(const void *buf, int64_t bytes, uint32_t *out, int grid, int block,
                           int unroll, int flags, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KQ_TUNE_H */

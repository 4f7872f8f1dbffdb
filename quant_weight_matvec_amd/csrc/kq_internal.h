// kq_internal.h -- declarations shared by the C-ABI shim (kq_abi.cpp) and
// the kernel launchers (kq_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace kqi {

// Process-wide per-device state covers devices 0 .. kMaxDevices - 1.
constexpr int kMaxDevices = 64;
// The current device's compute-unit count (256 if it cannot be read), cached
// per device; safe from several host threads.
int device_cus();
// Raise `kernel`'s dynamic-LDS limit to `bytes` on the current device, once
// per device (`done` holds one bit per device and belongs to that kernel);
// safe from several host threads (two may both set the same attribute).
hipError_t raise_lds_limit(const void *kernel, std::atomic<uint64_t> &done, int bytes);

// Launch shape of a matvec: `lanes` lanes cooperate on one weight row, a
// workgroup has `waves` wavefronts, and `grid` workgroups split the rows into
// contiguous ranges.  Zero fields mean "choose automatically".
// `depth` = units in flight per lane, 1..3 (the one being computed plus a
// look-ahead of depth-1).
struct MatvecShape {
    int lanes;
    int waves;
    int grid;
    int depth;
};

// Tuning override, process-wide (used by sweeps; 0 = automatic).
void set_shape_override(int qtype, MatvecShape s);
MatvecShape get_shape_override(int qtype);

// Each launcher assumes the arguments were validated by the ABI shim.
// The matvec launchers take the activation either as f32 (x) or in the staged
// form (xs, non-null: copied into LDS instead of encoded).
hipError_t launch_matvec_q4k(const uint8_t *W, const float *x, const uint8_t *xs, float *y,
                             int n_rows, int k, const float *silu_gate, hipStream_t stream);
// The previous layer's dual-eps tail, run in the gate+up kernel's prologue in
// place of a given input (k = the tail's row width).
struct TailArgs {
    const float *res_in, *proj, *g_post, *g_next;  // proj null: zero; gains null: unit
    float *res_out, *x_out;                        // each nullable (not written)
    float eps_post, eps_next;
};
// mid_s (nullable): also write mid staged with scale groups of mid_group (16 or 32).
// tail (nullable): compute x as that tail (x and xs are then unused).
hipError_t launch_gate_up_q4k(const uint8_t *Wg, const uint8_t *Wu, const float *x,
                              const uint8_t *xs, float *mid, uint8_t *mid_s, int mid_group,
                              int n_rows, int k, const TailArgs *tail, hipStream_t stream);
// Up to 4 matrices of one type and k sharing x (or its staged form xs) in one
// launch: matrix i has rows[i] rows and writes y[i] (counts validated).
hipError_t launch_matvec_group(int qtype, int count, const uint8_t *const *W, float *const *y,
                               const int *rows, const float *x, const uint8_t *xs, int k,
                               hipStream_t stream);
hipError_t launch_matvec_q5k(const uint8_t *W, const float *x, const uint8_t *xs, float *y,
                             int n_rows, int k, const float *silu_gate, hipStream_t stream);
// Embedding rows: qtype 1 (Q4_K) or 3 (Q5_K); one workgroup per token.
hipError_t launch_embedding(int qtype, const uint8_t *E, const int32_t *tokens, int n_tokens,
                            float *out, int vocab, int hidden, hipStream_t stream);
hipError_t launch_matvec_q6k(const uint8_t *W, const float *x, const uint8_t *xs, float *y,
                             int n_rows, int k, hipStream_t stream);
// staged form of x with scale groups of `group` (16 or 32)
hipError_t launch_stage(const float *x, uint8_t *xs, int k, int group, hipStream_t stream);
// Batched small-m kernel (kq_small_m.hip), m = 2..16.
size_t small_m_workspace_bytes(int qtype, int n_rows, int k, int m);
// The launch plan for a device of `cus` CUs: out = {workgroups, staged window
// in superblocks, LDS bytes, workspace bytes, threads per workgroup, tiles}.
void small_m_plan(int qtype, int n_rows, int k, int m, int cus, int64_t *out);
// kq_matmul_small_m_noalloc: the plan fits the library's scratch array, and
// the launch with the partial tiles and counters there (m = 2..16).
bool small_m_noalloc_fits(int qtype, int n_rows, int k, int m);
hipError_t launch_small_m_noalloc(int qtype, const uint8_t *W, const float *X, int64_t ldx,
                                  float *Y, int64_t ldy, int n_rows, int k, int m,
                                  hipStream_t stream);
// Small M through the matvec's integer dot path (rows_kernel, kq_kernels.hip):
// each workgroup stages the m rows into LDS, then dots each weight unit with
// every row; no workspace.  rows_path says whether (qtype, n_rows, k, m) takes
// it (the default or overridden largest M per qtype, and the rows fit the
// LDS).  With gate, Y = silu(gate) * (W X) row by row (gate may be Y).
int rows_max_m(int qtype);
bool set_rows_max_m(int qtype, int max_m);  // -1 restores the default
bool rows_path(int qtype, int n_rows, int k, int m);
hipError_t launch_rows(int qtype, const uint8_t *W, const float *X, int64_t ldx, float *Y,
                       int64_t ldy, int n_rows, int k, int m, const float *gate, int64_t ldg,
                       hipStream_t stream);
// The verify gate+up through the dot path in one launch: each row task
// streams its gate row's units, then its up row's, and Mid = silu(gate X) *
// (up X); gate_up_rows_path says whether (n_rows, k, m) takes it.
int gate_up_rows_max_m();
bool set_gate_up_rows_max_m(int max_m);  // -1 restores the default
bool gate_up_rows_path(int n_rows, int k, int m);
hipError_t launch_rows_gate_up(const uint8_t *Wg, const uint8_t *Wu, const float *X, int64_t ldx,
                               float *Mid, int64_t ldm, int n_rows, int k, int m,
                               hipStream_t stream);
// Small M (2..16): the dot path where rows_path says so, else the
// matrix-core kernel.
// gate (nullable): Y = silu(gate) * (W X), gate [m][ldg]; it may be Y itself.
hipError_t launch_small_m(int qtype, const uint8_t *W, const float *X, int64_t ldx, float *Y,
                          int64_t ldy, int n_rows, int k, int m, void *workspace,
                          int64_t workspace_bytes, hipStream_t stream,
                          const float *gate = nullptr, int64_t ldg = 0);
// xs_out (nullable): also write next_in staged, groups of xs_group, per row
hipError_t launch_tail(float *residual, const float *projected, float *next_in,
                       const float *g_post, const float *g_next, int rows, int n,
                       float eps_post, float eps_next, uint8_t *xs_out, int xs_group,
                       hipStream_t stream);

hipError_t launch_read_probe(const void *buf, int64_t bytes, uint32_t *out, int grid, int block,
                             int unroll, int flags, hipStream_t stream);

// The shape the automatic choice would use (for reports and tests).
MatvecShape auto_shape(int qtype, int64_t n_rows, int64_t k, int m);
// The automatic matvec launch shape on a device of `cus` CUs, without the
// process-wide override: out = {lanes, waves, grid, depth, LDS bytes per
// workgroup, workgroups per CU}.
void matvec_plan(int qtype, int64_t n_rows, int k, bool staged, int cus, int64_t *out);

const char *variant_names();

}  // namespace kqi

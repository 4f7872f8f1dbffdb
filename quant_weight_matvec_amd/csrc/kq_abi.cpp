// kq_abi.cpp -- the C ABI of libkq: argument validation, status strings,
// build identity.  Every check runs on the host before anything is enqueued,
// so a call that fails leaves its outputs untouched and the stream unchanged
// (the pages' engine fails closed in the same way rather than falling back:
// Ch 4 "Pipeline state objects and the three kernel sources", section 4.7).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include <string>

#include "kq.h"
#include "kq_tune.h"
#include "kq_internal.h"

namespace {

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// [a, a+an) and [b, b+bn) overlap (byte ranges; empty ranges never overlap)
bool overlap(const void *a, int64_t an, const void *b, int64_t bn)
{
    if (!a || !b || an <= 0 || bn <= 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)bn && b0 < a0 + (uintptr_t)an;
}

kq_status check_k(int64_t k)
{
    if (k < KQ_QK || k % KQ_QK) return KQ_ERR_SHAPE;
    if (k > KQ_MAX_K) return KQ_ERR_UNSUPPORTED;
    return KQ_OK;
}

// the HIP error behind this thread's last KQ_ERR_LAUNCH
thread_local hipError_t g_last_hip_error = hipSuccess;

kq_status from_hip(hipError_t e)
{
    if (e == hipSuccess) return KQ_OK;
    g_last_hip_error = e;
    return KQ_ERR_LAUNCH;
}

kq_status check_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return KQ_ERR_DEVICE;
    return KQ_OK;
}

kq_status check_matvec(const void *W, int64_t wbytes_per_row, uintptr_t walign, const float *x,
                       float *y, int64_t n_rows, int64_t k, const float *gate)
{
    if (!W || !x || !y) return KQ_ERR_NULL;
    if (n_rows < 0 || n_rows > INT32_MAX) return KQ_ERR_SHAPE;
    kq_status s = check_k(k);
    if (s != KQ_OK) return s;
    if (!aligned(W, walign) || !aligned(x, 16) || !aligned(y, 4) || (gate && !aligned(gate, 4)))
        return KQ_ERR_ALIGN;
    const int64_t wbytes = n_rows * wbytes_per_row;
    const int64_t ybytes = n_rows * 4;
    if (overlap(y, ybytes, W, wbytes) || overlap(y, ybytes, x, k * 4) ||
        overlap(y, ybytes, gate, gate ? ybytes : 0))
        return KQ_ERR_ALIAS;
    return KQ_OK;
}

}  // namespace

extern "C" {

kq_status kq_matvec_q4k(const void *W, const float *x, float *y, int64_t n_rows, int64_t k,
                        const float *silu_gate, void *stream)
{
    const int64_t rowb = (k / KQ_QK) * KQ_Q4K_BLOCK_BYTES;
    kq_status s = check_matvec(W, rowb, 16, x, y, n_rows, k, silu_gate);
    if (s != KQ_OK) return s;
    if (n_rows == 0) return KQ_OK;
    if ((s = check_device()) != KQ_OK) return s;
    return from_hip(kqi::launch_matvec_q4k((const uint8_t *)W, x, nullptr, y, (int)n_rows, (int)k,
                                           silu_gate, (hipStream_t)stream));
}

kq_status kq_matvec_q5k(const void *W, const float *x, float *y, int64_t n_rows, int64_t k,
                        const float *silu_gate, void *stream)
{
    const int64_t rowb = (k / KQ_QK) * KQ_Q5K_BLOCK_BYTES;
    kq_status s = check_matvec(W, rowb, 16, x, y, n_rows, k, silu_gate);
    if (s != KQ_OK) return s;
    if (n_rows == 0) return KQ_OK;
    if ((s = check_device()) != KQ_OK) return s;
    return from_hip(kqi::launch_matvec_q5k((const uint8_t *)W, x, nullptr, y, (int)n_rows, (int)k,
                                           silu_gate, (hipStream_t)stream));
}

kq_status kq_embedding(int qtype, const void *E, int64_t vocab, int64_t hidden,
                       const int32_t *tokens, int64_t n_tokens, float *out, void *stream)
{
    if (qtype != KQ_QTYPE_Q4K && qtype != KQ_QTYPE_Q5K) return KQ_ERR_SHAPE;
    if (!E || !tokens || !out) return KQ_ERR_NULL;
    if (vocab < 1 || vocab > INT32_MAX || n_tokens < 0 || n_tokens > INT32_MAX)
        return KQ_ERR_SHAPE;
    kq_status s = check_k(hidden);
    if (s != KQ_OK) return s;
    if (!aligned(E, 16) || !aligned(tokens, 4) || !aligned(out, 16)) return KQ_ERR_ALIGN;
    const int64_t blk = qtype == KQ_QTYPE_Q4K ? KQ_Q4K_BLOCK_BYTES : KQ_Q5K_BLOCK_BYTES;
    const int64_t ob = n_tokens * hidden * 4;
    if (overlap(out, ob, E, vocab * (hidden / KQ_QK) * blk) || overlap(out, ob, tokens, n_tokens * 4))
        return KQ_ERR_ALIAS;
    if (n_tokens == 0) return KQ_OK;
    if ((s = check_device()) != KQ_OK) return s;
    return from_hip(kqi::launch_embedding(qtype, (const uint8_t *)E, tokens, (int)n_tokens, out,
                                          (int)vocab, (int)hidden, (hipStream_t)stream));
}

kq_status kq_ffn_gate_up_q4k(const void *W_gate, const void *W_up, const float *x, float *mid,
                             int64_t n_rows, int64_t k, void *stream)
{
    if (!W_gate || !W_up || !x || !mid) return KQ_ERR_NULL;
    if (n_rows < 0 || n_rows > INT32_MAX) return KQ_ERR_SHAPE;
    kq_status s = check_k(k);
    if (s != KQ_OK) return s;
    if (!aligned(W_gate, 16) || !aligned(W_up, 16) || !aligned(x, 16) || !aligned(mid, 4))
        return KQ_ERR_ALIGN;
    const int64_t wbytes = n_rows * (k / KQ_QK) * KQ_Q4K_BLOCK_BYTES;
    if (overlap(mid, n_rows * 4, W_gate, wbytes) || overlap(mid, n_rows * 4, W_up, wbytes) ||
        overlap(mid, n_rows * 4, x, k * 4))
        return KQ_ERR_ALIAS;
    if (n_rows == 0) return KQ_OK;
    if ((s = check_device()) != KQ_OK) return s;
    return from_hip(kqi::launch_gate_up_q4k((const uint8_t *)W_gate, (const uint8_t *)W_up, x,
                                            nullptr, mid, nullptr, 0, (int)n_rows, (int)k,
                                            nullptr, (hipStream_t)stream));
}

kq_status kq_matvec_q6k(const void *W, const float *x, float *y, int64_t n_rows, int64_t k,
                        void *stream)
{
    const int64_t rowb = (k / KQ_QK) * KQ_Q6K_BLOCK_BYTES;
    kq_status s = check_matvec(W, rowb, 4, x, y, n_rows, k, nullptr);
    if (s != KQ_OK) return s;
    if (n_rows == 0) return KQ_OK;
    if ((s = check_device()) != KQ_OK) return s;
    return from_hip(kqi::launch_matvec_q6k((const uint8_t *)W, x, nullptr, y, (int)n_rows, (int)k,
                                           (hipStream_t)stream));
}

// Shared checks of kq_matvec_group and kq_matvec_group_staged; xbytes is the
// size of the input (f32 or staged).
static kq_status check_group(int qtype, int count, const void *const *W, float *const *y,
                             const int64_t *n_rows, const void *x, int64_t xbytes, int64_t k,
                             int64_t *total)
{
    if (qtype != KQ_QTYPE_Q4K && qtype != KQ_QTYPE_Q6K && qtype != KQ_QTYPE_Q5K)
        return KQ_ERR_SHAPE;
    if (count < 1 || count > KQ_MAX_GROUP) return KQ_ERR_SHAPE;
    if (!W || !y || !n_rows || !x) return KQ_ERR_NULL;
    kq_status s = check_k(k);
    if (s != KQ_OK) return s;
    const bool q4 = qtype != KQ_QTYPE_Q6K;  // Q4_K and Q5_K: 16-byte aligned superblocks
    const int64_t rowb = (k / KQ_QK) * (qtype == KQ_QTYPE_Q4K   ? KQ_Q4K_BLOCK_BYTES
                                        : qtype == KQ_QTYPE_Q5K ? KQ_Q5K_BLOCK_BYTES
                                                                : KQ_Q6K_BLOCK_BYTES);
    int64_t t = 0;
    for (int i = 0; i < count; ++i) {
        if (n_rows[i] < 0 || n_rows[i] > INT32_MAX) return KQ_ERR_SHAPE;
        if (n_rows[i] == 0) continue;  // an empty member's pointers are never used
        if (!W[i] || !y[i]) return KQ_ERR_NULL;
        t += n_rows[i];
        if (t > INT32_MAX) return KQ_ERR_SHAPE;
        if (!aligned(W[i], q4 ? 16 : 4) || !aligned(y[i], 4)) return KQ_ERR_ALIGN;
    }
    if (!aligned(x, 16)) return KQ_ERR_ALIGN;
    for (int i = 0; i < count; ++i) {
        const int64_t yb = n_rows[i] * 4;
        if (overlap(y[i], yb, x, xbytes)) return KQ_ERR_ALIAS;
        for (int j = 0; j < count; ++j) {
            if (overlap(y[i], yb, W[j], n_rows[j] * rowb)) return KQ_ERR_ALIAS;
            if (j > i && overlap(y[i], yb, y[j], n_rows[j] * 4)) return KQ_ERR_ALIAS;
        }
    }
    *total = t;
    return KQ_OK;
}

static kq_status run_group(int qtype, int count, const void *const *W, float *const *y,
                           const int64_t *n_rows, const float *x, const void *xs, int64_t k,
                           void *stream)
{
    const uint8_t *w[KQ_MAX_GROUP];
    float *o[KQ_MAX_GROUP];
    int rows[KQ_MAX_GROUP];
    int c = 0;
    for (int i = 0; i < count; ++i) {
        if (n_rows[i] == 0) continue;  // an empty matrix takes no segment
        w[c] = (const uint8_t *)W[i];
        o[c] = y[i];
        rows[c] = (int)n_rows[i];
        ++c;
    }
    if (c == 0) return KQ_OK;
    kq_status s = check_device();
    if (s != KQ_OK) return s;
    return from_hip(kqi::launch_matvec_group(qtype, c, w, o, rows, x, (const uint8_t *)xs,
                                             (int)k, (hipStream_t)stream));
}

kq_status kq_matvec_group(int qtype, int count, const void *const *W, float *const *y,
                          const int64_t *n_rows, const float *x, int64_t k, void *stream)
{
    int64_t total = 0;
    kq_status s = check_group(qtype, count, W, y, n_rows, x, k * 4, k, &total);
    if (s != KQ_OK) return s;
    return run_group(qtype, count, W, y, n_rows, x, nullptr, k, stream);
}

static int64_t staged_size(int qtype, int64_t k);

kq_status kq_matvec_group_staged(int qtype, int count, const void *const *W, float *const *y,
                                 const int64_t *n_rows, const void *xs, int64_t k, void *stream)
{
    if (qtype != KQ_QTYPE_Q4K && qtype != KQ_QTYPE_Q6K && qtype != KQ_QTYPE_Q5K)
        return KQ_ERR_SHAPE;
    const kq_status sk = check_k(k);
    if (sk != KQ_OK) return sk;
    int64_t total = 0;
    kq_status s = check_group(qtype, count, W, y, n_rows, xs, staged_size(qtype, k), k, &total);
    if (s != KQ_OK) return s;
    return run_group(qtype, count, W, y, n_rows, nullptr, xs, k, stream);
}

static kq_status check_small_m(int qtype, int64_t n_rows, int64_t k, int m)
{
    if (qtype == KQ_QTYPE_Q5K) return KQ_ERR_UNSUPPORTED;  // matrix-core path: Q4_K, Q6_K
    if (qtype != KQ_QTYPE_Q4K && qtype != KQ_QTYPE_Q6K) return KQ_ERR_SHAPE;
    if (m < 1 || n_rows < 0 || n_rows > INT32_MAX) return KQ_ERR_SHAPE;
    if (m > KQ_MAX_M) return KQ_ERR_UNSUPPORTED;
    return check_k(k);
}

int64_t kq_matmul_small_m_workspace_bytes(int qtype, int64_t n_rows, int64_t k, int m)
{
    kq_status s = check_small_m(qtype, n_rows, k, m);
    if (s != KQ_OK) return s;
    if (n_rows == 0 || m == 1) return 0;
    if ((s = check_device()) != KQ_OK) return s;
    return (int64_t)kqi::small_m_workspace_bytes(qtype, (int)n_rows, (int)k, m);
}

kq_status kq_matmul_small_m(int qtype, const void *W, const float *X, int64_t ldx, float *Y,
                            int64_t ldy, int64_t n_rows, int64_t k, int m, void *workspace,
                            int64_t workspace_bytes, void *stream)
{
    if (qtype == KQ_QTYPE_Q5K) return KQ_ERR_UNSUPPORTED;
    if (qtype != KQ_QTYPE_Q4K && qtype != KQ_QTYPE_Q6K) return KQ_ERR_SHAPE;
    if (!W || !X || !Y) return KQ_ERR_NULL;
    kq_status s = check_small_m(qtype, n_rows, k, m);
    if (s != KQ_OK) return s;
    if (ldx < k || ldx % 4 || ldy < n_rows || ldy < 1 || workspace_bytes < 0) return KQ_ERR_SHAPE;
    const uintptr_t walign = qtype == KQ_QTYPE_Q4K ? 16 : 4;
    if (!aligned(W, walign) || !aligned(X, 16) || !aligned(Y, 4) || !aligned(workspace, 256))
        return KQ_ERR_ALIGN;
    const int64_t blk = qtype == KQ_QTYPE_Q4K ? KQ_Q4K_BLOCK_BYTES : KQ_Q6K_BLOCK_BYTES;
    const int64_t wbytes = n_rows * (k / KQ_QK) * blk;
    const int64_t ybytes = ((int64_t)(m - 1) * ldy + n_rows) * 4;
    const int64_t xbytes = ((int64_t)(m - 1) * ldx + k) * 4;
    if (overlap(Y, ybytes, W, wbytes) || overlap(Y, ybytes, X, xbytes)) return KQ_ERR_ALIAS;
    if (n_rows == 0) return KQ_OK;
    if ((s = check_device()) != KQ_OK) return s;
    if (m == 1)
        return from_hip(qtype == KQ_QTYPE_Q4K
                            ? kqi::launch_matvec_q4k((const uint8_t *)W, X, nullptr, Y,
                                                     (int)n_rows, (int)k, nullptr,
                                                     (hipStream_t)stream)
                            : kqi::launch_matvec_q6k((const uint8_t *)W, X, nullptr, Y,
                                                     (int)n_rows, (int)k, (hipStream_t)stream));
    const int64_t need =
        (int64_t)kqi::small_m_workspace_bytes(qtype, (int)n_rows, (int)k, m);
    if (need > 0) {
        if (!workspace) return KQ_ERR_NULL;
        if (workspace_bytes < need) return KQ_ERR_SHAPE;
        if (overlap(workspace, need, Y, ybytes) || overlap(workspace, need, X, xbytes) ||
            overlap(workspace, need, W, wbytes))
            return KQ_ERR_ALIAS;
    }
    return from_hip(kqi::launch_small_m(qtype, (const uint8_t *)W, X, ldx, Y, ldy, (int)n_rows,
                                        (int)k, m, workspace, workspace_bytes,
                                        (hipStream_t)stream));
}

kq_status kq_ffn_gate_up_q4k_small_m(const void *W_gate, const void *W_up, const float *X,
                                     int64_t ldx, float *Mid, int64_t ldm, int64_t n_rows,
                                     int64_t k, int m, void *workspace, int64_t workspace_bytes,
                                     void *stream)
{
    if (!W_gate || !W_up || !X || !Mid) return KQ_ERR_NULL;
    kq_status s = check_small_m(KQ_QTYPE_Q4K, n_rows, k, m);
    if (s != KQ_OK) return s;
    if (ldx < k || ldx % 4 || ldm < n_rows || ldm < 1 || workspace_bytes < 0) return KQ_ERR_SHAPE;
    if (!aligned(W_gate, 16) || !aligned(W_up, 16) || !aligned(X, 16) || !aligned(Mid, 4) ||
        !aligned(workspace, 256))
        return KQ_ERR_ALIGN;
    const int64_t wbytes = n_rows * (k / KQ_QK) * KQ_Q4K_BLOCK_BYTES;
    const int64_t mbytes = ((int64_t)(m - 1) * ldm + n_rows) * 4;
    const int64_t xbytes = ((int64_t)(m - 1) * ldx + k) * 4;
    if (overlap(Mid, mbytes, W_gate, wbytes) || overlap(Mid, mbytes, W_up, wbytes) ||
        overlap(Mid, mbytes, X, xbytes))
        return KQ_ERR_ALIAS;
    if (n_rows == 0) return KQ_OK;
    if ((s = check_device()) != KQ_OK) return s;
    const hipStream_t st = (hipStream_t)stream;
    if (m == 1)
        return from_hip(kqi::launch_gate_up_q4k((const uint8_t *)W_gate, (const uint8_t *)W_up, X,
                                                nullptr, Mid, nullptr, 0, (int)n_rows, (int)k,
                                                nullptr, st));
    if (kqi::gate_up_rows_path((int)n_rows, (int)k, m))  // one launch, no workspace
        return from_hip(kqi::launch_rows_gate_up((const uint8_t *)W_gate, (const uint8_t *)W_up, X,
                                                 ldx, Mid, ldm, (int)n_rows, (int)k, m, st));
    const int64_t need = (int64_t)kqi::small_m_workspace_bytes(KQ_QTYPE_Q4K, (int)n_rows, (int)k, m);
    if (need > 0) {
        if (!workspace) return KQ_ERR_NULL;
        if (workspace_bytes < need) return KQ_ERR_SHAPE;
        if (overlap(workspace, need, Mid, mbytes) || overlap(workspace, need, X, xbytes) ||
            overlap(workspace, need, W_gate, wbytes) || overlap(workspace, need, W_up, wbytes))
            return KQ_ERR_ALIAS;
    }
    // gate into Mid, then up with the SiLU of the gate values it overwrites
    hipError_t e = kqi::launch_small_m(KQ_QTYPE_Q4K, (const uint8_t *)W_gate, X, ldx, Mid, ldm,
                                       (int)n_rows, (int)k, m, workspace, workspace_bytes, st);
    if (e != hipSuccess) return from_hip(e);
    return from_hip(kqi::launch_small_m(KQ_QTYPE_Q4K, (const uint8_t *)W_up, X, ldx, Mid, ldm,
                                        (int)n_rows, (int)k, m, workspace, workspace_bytes, st,
                                        Mid, ldm));
}

kq_status kq_matmul_small_m_noalloc(int qtype, const void *W, const float *X, int64_t ldx,
                                    float *Y, int64_t ldy, int64_t n_rows, int64_t k, int m,
                                    void *stream)
{
    if (qtype == KQ_QTYPE_Q5K) return KQ_ERR_UNSUPPORTED;
    if (qtype != KQ_QTYPE_Q4K && qtype != KQ_QTYPE_Q6K) return KQ_ERR_SHAPE;
    if (!W || !X || !Y) return KQ_ERR_NULL;
    kq_status s = check_small_m(qtype, n_rows, k, m);
    if (s != KQ_OK) return s;
    if (ldx < k || ldx % 4 || ldy < n_rows || ldy < 1) return KQ_ERR_SHAPE;
    const uintptr_t walign = qtype == KQ_QTYPE_Q4K ? 16 : 4;
    if (!aligned(W, walign) || !aligned(X, 16) || !aligned(Y, 4)) return KQ_ERR_ALIGN;
    const int64_t blk = qtype == KQ_QTYPE_Q4K ? KQ_Q4K_BLOCK_BYTES : KQ_Q6K_BLOCK_BYTES;
    const int64_t wbytes = n_rows * (k / KQ_QK) * blk;
    const int64_t ybytes = ((int64_t)(m - 1) * ldy + n_rows) * 4;
    const int64_t xbytes = ((int64_t)(m - 1) * ldx + k) * 4;
    if (overlap(Y, ybytes, W, wbytes) || overlap(Y, ybytes, X, xbytes)) return KQ_ERR_ALIAS;
    if (n_rows == 0) return KQ_OK;
    // host arithmetic on the launch plan: a shape the scratch array cannot
    // hold is rejected before any device call
    if (!kqi::small_m_noalloc_fits(qtype, (int)n_rows, (int)k, m)) return KQ_ERR_UNSUPPORTED;
    if ((s = check_device()) != KQ_OK) return s;
    if (m == 1)
        return from_hip(qtype == KQ_QTYPE_Q4K
                            ? kqi::launch_matvec_q4k((const uint8_t *)W, X, nullptr, Y,
                                                     (int)n_rows, (int)k, nullptr,
                                                     (hipStream_t)stream)
                            : kqi::launch_matvec_q6k((const uint8_t *)W, X, nullptr, Y,
                                                     (int)n_rows, (int)k, (hipStream_t)stream));
    const hipError_t e = kqi::launch_small_m_noalloc(qtype, (const uint8_t *)W, X, ldx, Y, ldy,
                                                     (int)n_rows, (int)k, m, (hipStream_t)stream);
    if (e == hipErrorInvalidSymbol || e == hipErrorInvalidDevice) return KQ_ERR_DEVICE;
    return from_hip(e);
}

kq_status kq_fused_residual_norm(float *residual, const float *projected, float *next_in,
                                 const float *g_post, const float *g_next, int64_t rows,
                                 int64_t n, float eps_post, float eps_next, void *stream)
{
    if (!residual || !projected || !next_in || !g_post || !g_next) return KQ_ERR_NULL;
    if (rows < 0 || rows > INT32_MAX || n < 4 || n % 4) return KQ_ERR_SHAPE;
    if (n > KQ_MAX_TAIL_N) return KQ_ERR_UNSUPPORTED;
    if (!(eps_post >= 0.0f) || !(eps_next >= 0.0f) || !isfinite(eps_post) || !isfinite(eps_next))
        return KQ_ERR_SHAPE;
    if (!aligned(residual, 16) || !aligned(projected, 16) || !aligned(next_in, 16) ||
        !aligned(g_post, 16) || !aligned(g_next, 16))
        return KQ_ERR_ALIGN;
    const int64_t b = rows * n * 4;
    if (overlap(next_in, b, residual, b) || overlap(next_in, b, projected, b) ||
        overlap(next_in, b, g_post, n * 4) || overlap(next_in, b, g_next, n * 4) ||
        overlap(residual, b, projected, b) || overlap(residual, b, g_post, n * 4) ||
        overlap(residual, b, g_next, n * 4))
        return KQ_ERR_ALIAS;
    if (rows == 0) return KQ_OK;
    kq_status s = check_device();
    if (s != KQ_OK) return s;
    return from_hip(kqi::launch_tail(residual, projected, next_in, g_post, g_next, (int)rows,
                                     (int)n, eps_post, eps_next, nullptr, 0,
                                     (hipStream_t)stream));
}

// ---------------------------------------------------------------------------
// Staged activations.  The group size follows the consuming weight type:
// 32 inputs for Q4_K, 16 for Q6_K.
static int staged_group(int qtype)
{
    // Q4_K and Q5_K: sub-blocks of 32 inputs; Q6_K: 16
    return (qtype == KQ_QTYPE_Q4K || qtype == KQ_QTYPE_Q5K) ? 32 : (qtype == KQ_QTYPE_Q6K ? 16 : 0);
}

static int64_t staged_size(int qtype, int64_t k)
{
    // limb planes of k + k/8 bytes (16 bytes of padding per 128 inputs), then
    // a scale and a sum per group
    return KQ_STAGED_LIMBS * (k + k / 8) + 8 * (k / staged_group(qtype));
}

int64_t kq_staged_bytes(int qtype, int64_t k)
{
    if (!staged_group(qtype)) return KQ_ERR_SHAPE;
    kq_status s = check_k(k);
    if (s != KQ_OK) return s;
    return staged_size(qtype, k);
}

kq_status kq_stage_activation(int qtype, const float *x, void *xs, int64_t k, void *stream)
{
    if (!staged_group(qtype)) return KQ_ERR_SHAPE;
    if (!x || !xs) return KQ_ERR_NULL;
    kq_status s = check_k(k);
    if (s != KQ_OK) return s;
    if (!aligned(x, 16) || !aligned(xs, 16)) return KQ_ERR_ALIGN;
    if (overlap(xs, staged_size(qtype, k), x, k * 4)) return KQ_ERR_ALIAS;
    if ((s = check_device()) != KQ_OK) return s;
    return from_hip(kqi::launch_stage(x, (uint8_t *)xs, (int)k, staged_group(qtype),
                                      (hipStream_t)stream));
}

kq_status kq_matvec_staged(int qtype, const void *W, const void *xs, float *y, int64_t n_rows,
                           int64_t k, const float *silu_gate, void *stream)
{
    if (!staged_group(qtype)) return KQ_ERR_SHAPE;
    if (!W || !xs || !y) return KQ_ERR_NULL;
    if (qtype == KQ_QTYPE_Q6K && silu_gate) return KQ_ERR_UNSUPPORTED;
    if (n_rows < 0 || n_rows > INT32_MAX) return KQ_ERR_SHAPE;
    kq_status s = check_k(k);
    if (s != KQ_OK) return s;
    const bool q6 = qtype == KQ_QTYPE_Q6K;
    if (!aligned(W, q6 ? 4 : 16) || !aligned(xs, 16) || !aligned(y, 4) ||
        (silu_gate && !aligned(silu_gate, 4)))
        return KQ_ERR_ALIGN;
    const int64_t blk = qtype == KQ_QTYPE_Q4K   ? KQ_Q4K_BLOCK_BYTES
                        : qtype == KQ_QTYPE_Q5K ? KQ_Q5K_BLOCK_BYTES
                                                : KQ_Q6K_BLOCK_BYTES;
    const int64_t wbytes = n_rows * (k / KQ_QK) * blk;
    const int64_t ybytes = n_rows * 4;
    if (overlap(y, ybytes, W, wbytes) || overlap(y, ybytes, xs, staged_size(qtype, k)) ||
        overlap(y, ybytes, silu_gate, silu_gate ? ybytes : 0))
        return KQ_ERR_ALIAS;
    if (n_rows == 0) return KQ_OK;
    if ((s = check_device()) != KQ_OK) return s;
    const uint8_t *w = (const uint8_t *)W, *xsb = (const uint8_t *)xs;
    const hipStream_t st = (hipStream_t)stream;
    if (qtype == KQ_QTYPE_Q4K)
        return from_hip(kqi::launch_matvec_q4k(w, nullptr, xsb, y, (int)n_rows, (int)k, silu_gate, st));
    if (qtype == KQ_QTYPE_Q5K)
        return from_hip(kqi::launch_matvec_q5k(w, nullptr, xsb, y, (int)n_rows, (int)k, silu_gate, st));
    return from_hip(kqi::launch_matvec_q6k(w, nullptr, xsb, y, (int)n_rows, (int)k, st));
}

kq_status kq_ffn_gate_up_q4k_staged(const void *W_gate, const void *W_up, const void *xs,
                                    float *mid, void *mid_s, int mid_qtype, int64_t n_rows,
                                    int64_t k, void *stream)
{
    if (!W_gate || !W_up || !xs || !mid) return KQ_ERR_NULL;
    if (mid_s && !staged_group(mid_qtype)) return KQ_ERR_SHAPE;
    if (n_rows < 0 || n_rows > INT32_MAX) return KQ_ERR_SHAPE;
    if (mid_s && n_rows % KQ_QK) return KQ_ERR_SHAPE;  // mid is the next matvec's input
    kq_status s = check_k(k);
    if (s != KQ_OK) return s;
    if (!aligned(W_gate, 16) || !aligned(W_up, 16) || !aligned(xs, 16) || !aligned(mid, 4) ||
        !aligned(mid_s, 16))
        return KQ_ERR_ALIGN;
    const int64_t wbytes = n_rows * (k / KQ_QK) * KQ_Q4K_BLOCK_BYTES;
    const int64_t xsb = staged_size(KQ_QTYPE_Q4K, k);
    const int64_t mb = n_rows * 4, msb = mid_s ? staged_size(mid_qtype, n_rows) : 0;
    if (overlap(mid, mb, W_gate, wbytes) || overlap(mid, mb, W_up, wbytes) ||
        overlap(mid, mb, xs, xsb) || overlap(mid_s, msb, W_gate, wbytes) ||
        overlap(mid_s, msb, W_up, wbytes) || overlap(mid_s, msb, xs, xsb) ||
        overlap(mid_s, msb, mid, mb))
        return KQ_ERR_ALIAS;
    if (n_rows == 0) return KQ_OK;
    if ((s = check_device()) != KQ_OK) return s;
    return from_hip(kqi::launch_gate_up_q4k(
        (const uint8_t *)W_gate, (const uint8_t *)W_up, nullptr, (const uint8_t *)xs, mid,
        (uint8_t *)mid_s, mid_s ? staged_group(mid_qtype) : 0, (int)n_rows, (int)k, nullptr,
        (hipStream_t)stream));
}

kq_status kq_ffn_tail_gate_up_q4k(const float *residual_in, const float *projected,
                                  const float *g_post, const float *g_next, float *residual_out,
                                  float *next_in, const void *W_gate, const void *W_up, float *mid,
                                  void *mid_s, int mid_qtype, int64_t n_rows, int64_t k,
                                  float eps_post, float eps_next, void *stream)
{
    if (!residual_in || !projected || !g_post || !g_next || !residual_out || !W_gate || !W_up ||
        !mid)
        return KQ_ERR_NULL;
    if (mid_s && !staged_group(mid_qtype)) return KQ_ERR_SHAPE;
    if (n_rows < 1 || n_rows > INT32_MAX) return KQ_ERR_SHAPE;  // the tail needs a launch
    if (mid_s && n_rows % KQ_QK) return KQ_ERR_SHAPE;
    kq_status s = check_k(k);
    if (s != KQ_OK) return s;
    if (k > KQ_MAX_FUSED_TAIL_K) return KQ_ERR_UNSUPPORTED;
    if (!(eps_post >= 0.0f) || !(eps_next >= 0.0f) || !isfinite(eps_post) || !isfinite(eps_next))
        return KQ_ERR_SHAPE;
    if (!aligned(residual_in, 16) || !aligned(projected, 16) || !aligned(g_post, 16) ||
        !aligned(g_next, 16) || !aligned(residual_out, 16) || !aligned(next_in, 16) ||
        !aligned(W_gate, 16) || !aligned(W_up, 16) || !aligned(mid, 4) || !aligned(mid_s, 16))
        return KQ_ERR_ALIGN;
    const int64_t vb = k * 4, wbytes = n_rows * (k / KQ_QK) * KQ_Q4K_BLOCK_BYTES;
    const int64_t mb = n_rows * 4, msb = mid_s ? staged_size(mid_qtype, n_rows) : 0;
    const void *ins[] = {residual_in, projected, g_post, g_next, W_gate, W_up};
    const int64_t inb[] = {vb, vb, vb, vb, wbytes, wbytes};
    void *outs[] = {residual_out, next_in, mid, mid_s};
    const int64_t outb[] = {vb, next_in ? vb : 0, mb, msb};
    for (int o = 0; o < 4; ++o) {
        for (int i = 0; i < 6; ++i)
            if (overlap(outs[o], outb[o], ins[i], inb[i])) return KQ_ERR_ALIAS;
        for (int o2 = o + 1; o2 < 4; ++o2)
            if (overlap(outs[o], outb[o], outs[o2], outb[o2])) return KQ_ERR_ALIAS;
    }
    if ((s = check_device()) != KQ_OK) return s;
    const kqi::TailArgs tail{residual_in, projected, g_post, g_next, residual_out, next_in,
                             eps_post, eps_next};
    return from_hip(kqi::launch_gate_up_q4k(
        (const uint8_t *)W_gate, (const uint8_t *)W_up, nullptr, nullptr, mid, (uint8_t *)mid_s,
        mid_s ? staged_group(mid_qtype) : 0, (int)n_rows, (int)k, &tail, (hipStream_t)stream));
}

kq_status kq_fused_residual_norm_staged(float *residual, const float *projected, float *next_in,
                                        void *next_in_s, int next_qtype, const float *g_post,
                                        const float *g_next, int64_t rows, int64_t n,
                                        float eps_post, float eps_next, void *stream)
{
    if (!next_in_s) return KQ_ERR_NULL;
    if (!staged_group(next_qtype)) return KQ_ERR_SHAPE;
    if (n % KQ_QK) return KQ_ERR_SHAPE;  // next_in is a matvec input
    if (!aligned(next_in_s, 16)) return KQ_ERR_ALIGN;
    if (!residual || !projected || !next_in || !g_post || !g_next) return KQ_ERR_NULL;
    if (rows < 0 || rows > INT32_MAX || n < 4) return KQ_ERR_SHAPE;
    if (n > KQ_MAX_TAIL_N) return KQ_ERR_UNSUPPORTED;
    if (!(eps_post >= 0.0f) || !(eps_next >= 0.0f) || !isfinite(eps_post) || !isfinite(eps_next))
        return KQ_ERR_SHAPE;
    if (!aligned(residual, 16) || !aligned(projected, 16) || !aligned(next_in, 16) ||
        !aligned(g_post, 16) || !aligned(g_next, 16))
        return KQ_ERR_ALIGN;
    const int64_t b = rows * n * 4;
    const int64_t sb = rows * staged_size(next_qtype, n);
    if (overlap(next_in, b, residual, b) || overlap(next_in, b, projected, b) ||
        overlap(next_in, b, g_post, n * 4) || overlap(next_in, b, g_next, n * 4) ||
        overlap(residual, b, projected, b) || overlap(residual, b, g_post, n * 4) ||
        overlap(residual, b, g_next, n * 4) || overlap(next_in_s, sb, residual, b) ||
        overlap(next_in_s, sb, projected, b) || overlap(next_in_s, sb, next_in, b) ||
        overlap(next_in_s, sb, g_post, n * 4) || overlap(next_in_s, sb, g_next, n * 4))
        return KQ_ERR_ALIAS;
    if (rows == 0) return KQ_OK;
    kq_status s = check_device();
    if (s != KQ_OK) return s;
    return from_hip(kqi::launch_tail(residual, projected, next_in, g_post, g_next, (int)rows,
                                     (int)n, eps_post, eps_next, (uint8_t *)next_in_s,
                                     staged_group(next_qtype), (hipStream_t)stream));
}

const char *kq_last_hip_error(void) { return hipGetErrorName(g_last_hip_error); }

const char *kq_status_string(kq_status s)
{
    switch (s) {
    case KQ_OK: return "KQ_OK";
    case KQ_ERR_NULL: return "KQ_ERR_NULL: a required pointer is NULL";
    case KQ_ERR_SHAPE: return "KQ_ERR_SHAPE: a size is out of range or inconsistent";
    case KQ_ERR_ALIGN: return "KQ_ERR_ALIGN: a pointer is not aligned as required";
    case KQ_ERR_ALIAS: return "KQ_ERR_ALIAS: an output overlaps an input";
    case KQ_ERR_UNSUPPORTED: return "KQ_ERR_UNSUPPORTED: valid but unsupported arguments";
    case KQ_ERR_LAUNCH: return "KQ_ERR_LAUNCH: the HIP runtime refused the launch";
    case KQ_ERR_DEVICE: return "KQ_ERR_DEVICE: no usable current device";
    default: return "KQ_ERR_UNKNOWN";
    }
}

#ifndef KQ_GIT_SHA
#define KQ_GIT_SHA "unknown"
#endif

const char *kq_build_info(void)
{
    // built once, thread-safely (function-local static initialisation)
    static const std::string info = [] {
        char buf[512];
        snprintf(buf, sizeof buf, "libkq target=gfx950 hip=%d.%d.%d git=%s variants: %s",
                 HIP_VERSION_MAJOR, HIP_VERSION_MINOR, HIP_VERSION_PATCH, KQ_GIT_SHA,
                 kqi::variant_names());
        return std::string(buf);
    }();
    return info.c_str();
}

namespace {

// Relay buffers of kq_ffn_pass_q4k_q6k in its workspace (byte offsets).
struct PassWs {
    int64_t res_alt, p, mid_s, mid, total;
};

PassWs pass_ws_layout(int64_t hidden, int64_t ffn)
{
    auto up = [](int64_t b) { return (b + 255) / 256 * 256; };
    PassWs w;
    w.res_alt = 0;
    w.p = up(4 * hidden);
    w.mid_s = w.p + up(4 * hidden);
    w.mid = w.mid_s + up(staged_size(KQ_QTYPE_Q6K, ffn));
    w.total = w.mid + up(4 * ffn);
    return w;
}

}  // namespace

int64_t kq_ffn_pass_workspace_bytes(int64_t hidden, int64_t ffn)
{
    kq_status s = check_k(hidden);
    if (s != KQ_OK) return s;
    if ((s = check_k(ffn)) != KQ_OK) return s;
    if (hidden > KQ_MAX_FUSED_TAIL_K) return KQ_ERR_UNSUPPORTED;
    return pass_ws_layout(hidden, ffn).total;
}

kq_status kq_ffn_pass_q4k_q6k(const kq_ffn_layer *layers, int n_layers, float *residual,
                              float *x_out, const float *g_entry, void *workspace,
                              int64_t workspace_bytes, int64_t hidden, int64_t ffn,
                              float eps_post, float eps_next, void *stream)
{
    if (!layers || !residual || !x_out || !workspace) return KQ_ERR_NULL;
    if (n_layers < 1) return KQ_ERR_SHAPE;
    const int64_t need = kq_ffn_pass_workspace_bytes(hidden, ffn);
    if (need < 0) return (kq_status)need;
    if (workspace_bytes < need) return KQ_ERR_SHAPE;
    if (!(eps_post >= 0.0f) || !(eps_next >= 0.0f) || !isfinite(eps_post) || !isfinite(eps_next))
        return KQ_ERR_SHAPE;
    if (!aligned(residual, 16) || !aligned(x_out, 16) || !aligned(g_entry, 16) ||
        !aligned(workspace, 256))
        return KQ_ERR_ALIGN;
    const int64_t vb = hidden * 4;
    const int64_t q4b = ffn * (hidden / KQ_QK) * KQ_Q4K_BLOCK_BYTES;
    const int64_t q6b = hidden * (ffn / KQ_QK) * KQ_Q6K_BLOCK_BYTES;
    void *outs[] = {residual, x_out, workspace};
    const int64_t outb[] = {vb, vb, workspace_bytes};
    for (int o = 0; o < 3; ++o) {
        for (int o2 = o + 1; o2 < 3; ++o2)
            if (overlap(outs[o], outb[o], outs[o2], outb[o2])) return KQ_ERR_ALIAS;
        if (overlap(outs[o], outb[o], g_entry, g_entry ? vb : 0)) return KQ_ERR_ALIAS;
    }
    for (int l = 0; l < n_layers; ++l) {
        const kq_ffn_layer &L = layers[l];
        if (!L.W_gate || !L.W_up || !L.W_down || !L.g_post || !L.g_next) return KQ_ERR_NULL;
        if (!aligned(L.W_gate, 16) || !aligned(L.W_up, 16) || !aligned(L.W_down, 4) ||
            !aligned(L.g_post, 16) || !aligned(L.g_next, 16))
            return KQ_ERR_ALIGN;
        const void *ins[] = {L.W_gate, L.W_up, L.W_down, L.g_post, L.g_next};
        const int64_t inb[] = {q4b, q4b, q6b, vb, vb};
        for (int o = 0; o < 3; ++o)
            for (int i = 0; i < 5; ++i)
                if (overlap(outs[o], outb[o], ins[i], inb[i])) return KQ_ERR_ALIAS;
    }
    kq_status s = check_device();
    if (s != KQ_OK) return s;
    const PassWs w = pass_ws_layout(hidden, ffn);
    uint8_t *ws = (uint8_t *)workspace;
    float *alt = (float *)(ws + w.res_alt);
    float *p = (float *)(ws + w.p);
    uint8_t *mid_s = ws + w.mid_s;
    float *mid = (float *)(ws + w.mid);
    const hipStream_t st = (hipStream_t)stream;
    const int h = (int)hidden, f = (int)ffn;
    // Layer l's tail reads the current residual buffer and writes the other
    // one (every workgroup reads the first while one writes the second).
    // Layer 0's tail is the entry norm, which leaves the residual unchanged:
    // with an odd layer count it writes nothing, so that the residual after
    // the last layer sits in `residual`, where the last tail updates it.
    float *cur = residual, *other = alt;
    for (int l = 0; l < n_layers; ++l) {
        const bool skip_write = l == 0 && (n_layers & 1);
        const kqi::TailArgs t{cur,
                              l ? p : nullptr,
                              l ? layers[l - 1].g_post : nullptr,
                              l ? layers[l - 1].g_next : g_entry,
                              skip_write ? nullptr : other,
                              nullptr,
                              eps_post,
                              eps_next};
        s = from_hip(kqi::launch_gate_up_q4k((const uint8_t *)layers[l].W_gate,
                                             (const uint8_t *)layers[l].W_up, nullptr, nullptr,
                                             mid, mid_s, 16, f, h, &t, st));
        if (s != KQ_OK) return s;
        if (!skip_write) {
            float *tmp = cur;
            cur = other;
            other = tmp;
        }
        s = from_hip(kqi::launch_matvec_q6k((const uint8_t *)layers[l].W_down, nullptr, mid_s, p,
                                            h, f, st));
        if (s != KQ_OK) return s;
    }
    return from_hip(kqi::launch_tail(cur, p, x_out, layers[n_layers - 1].g_post,
                                     layers[n_layers - 1].g_next, 1, h, eps_post, eps_next,
                                     nullptr, 0, st));
}

kq_status kq_tune_set_small_m_rows(int qtype, int max_m)
{
    return kqi::set_rows_max_m(qtype, max_m) ? KQ_OK : KQ_ERR_SHAPE;
}

kq_status kq_tune_set_gate_up_rows(int max_m)
{
    return kqi::set_gate_up_rows_max_m(max_m) ? KQ_OK : KQ_ERR_SHAPE;
}

kq_status kq_tune_set_shape(int qtype, int lanes, int waves, int grid, int depth)
{
    if (qtype != KQ_QTYPE_Q4K && qtype != KQ_QTYPE_Q6K && qtype != KQ_QTYPE_Q5K) return KQ_ERR_SHAPE;
    if (lanes && lanes != 4 && lanes != 8 && lanes != 16 && lanes != 32 && lanes != 64)
        return KQ_ERR_SHAPE;
    if (waves < 0 || waves > 16 || grid < 0 || depth < 0 || depth > 3) return KQ_ERR_SHAPE;
    kqi::set_shape_override(qtype, kqi::MatvecShape{lanes, waves, grid, depth});
    return KQ_OK;
}

kq_status kq_tune_get_shape(int qtype, int64_t n_rows, int64_t k, int *lanes, int *waves,
                            int *grid, int *depth)
{
    if (qtype != KQ_QTYPE_Q4K && qtype != KQ_QTYPE_Q6K && qtype != KQ_QTYPE_Q5K) return KQ_ERR_SHAPE;
    if (!lanes || !waves || !grid || !depth) return KQ_ERR_NULL;
    kq_status s = check_k(k);
    if (s != KQ_OK) return s;
    if (n_rows < 1) return KQ_ERR_SHAPE;
    if ((s = check_device()) != KQ_OK) return s;
    const kqi::MatvecShape sh = kqi::auto_shape(qtype, n_rows, k, 1);
    *lanes = sh.lanes;
    *waves = sh.waves;
    *grid = sh.grid;
    *depth = sh.depth;
    return KQ_OK;
}

kq_status kq_tune_matvec_plan(int qtype, int64_t n_rows, int64_t k, int staged, int cus,
                              int64_t *out)
{
    if (qtype != KQ_QTYPE_Q4K && qtype != KQ_QTYPE_Q6K && qtype != KQ_QTYPE_Q5K) return KQ_ERR_SHAPE;
    kq_status s = check_k(k);
    if (s != KQ_OK) return s;
    if (!out) return KQ_ERR_NULL;
    if (n_rows < 1 || n_rows > INT32_MAX || cus < 1 || cus > 4096) return KQ_ERR_SHAPE;
    kqi::matvec_plan(qtype, n_rows, (int)k, staged != 0, cus, out);
    return KQ_OK;
}

kq_status kq_tune_small_m_plan(int qtype, int64_t n_rows, int64_t k, int m, int cus,
                               int64_t *out)
{
    kq_status s = check_small_m(qtype, n_rows, k, m);
    if (s != KQ_OK) return s;
    if (!out) return KQ_ERR_NULL;
    if (n_rows < 1 || m < 2 || cus < 1 || cus > 4096) return KQ_ERR_SHAPE;
    kqi::small_m_plan(qtype, (int)n_rows, (int)k, m, cus, out);
    return KQ_OK;
}

kq_status kq_probe_read_bw(const void *buf, int64_t bytes, uint32_t *out, int grid, int block,
                           int unroll, int flags, void *stream)
{
    if (!buf || !out) return KQ_ERR_NULL;
    if (bytes < 16 || bytes % 16 || grid < 1) return KQ_ERR_SHAPE;
    if (block < 64 || block > 1024 || block % 64) return KQ_ERR_SHAPE;
    if ((unroll != 1 && unroll != 4 && unroll != 8 && unroll != 16) || flags < 0 || flags > 3)
        return KQ_ERR_SHAPE;
    if (!aligned(buf, 16) || !aligned(out, 4)) return KQ_ERR_ALIGN;
    if (overlap(out, (int64_t)grid * (block / 64) * 4, buf, bytes)) return KQ_ERR_ALIAS;
    kq_status s = check_device();
    if (s != KQ_OK) return s;
    return from_hip(kqi::launch_read_probe(buf, bytes, out, grid, block, unroll, flags,
                                           (hipStream_t)stream));
}

}  // extern "C"

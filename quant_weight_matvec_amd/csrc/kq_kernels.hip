// kq_kernels.hip -- gfx950 kernels of the k-quant decode path.
//
// What is computed comes from "How to Write an Inference Engine -- the Muser
// book": the decode matvec over 256-weight Q4_K / Q6_K superblocks (Ch 19 "The
// down projection + residual", sections 19.1 and 19.3), the SiLU-gated FFN
// product (Ch 10 "The forward pass at a glance", section 10.3, box 11) and the
// fused dual-epsilon tail (Ch 19, section 19.4).  The kernels are designed for
// CDNA4 and follow none of the pages' Metal geometry.
//
// Matvec design (M = 1):
//  * The weight stream is the whole cost (Ch 19, section 19.6: weights are
//    about 700x the activation traffic), so every weight byte is read from HBM
//    exactly once, with 16-byte vector loads, and nothing but the activation
//    vector goes through LDS.
//  * Activation staging: each workgroup converts x once into LDS as block
//    floating point.  Per group of inputs that shares one quant scale (32 for
//    Q4_K, 16 for Q6_K) it keeps a power-of-two exponent, the f32 sum of the
//    group (for the Q4_K min term and the Q6_K -32 offset), and each input as
//    a signed integer of LIMBS*8-1 bits stored as LIMBS signed bytes in
//    separate planes.  The inner loop is then v_dot4_i32_i8 of raw quant
//    bytes against each byte plane: four multiply-adds per instruction and no
//    per-weight float conversion.  With three limbs an input is rounded to a
//    multiple of 2^(e-22), e the group exponent (max|x| < 2^e), so its error
//    is at most 2^-22 times the group's largest magnitude.
//  * Work split: `lanes` lanes share a row and walk its half-superblock units
//    (128 weights) in stride; a wave holds 64/lanes rows; a workgroup owns a
//    contiguous row range.  Per-lane partial sums are folded with a fixed
//    xor-butterfly, so results are bitwise reproducible.
//  * The next unit's loads are issued before the current unit is computed.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kq_device.h"
#include "kq_internal.h"

namespace {

using namespace kqd;

// float4 of x per thread loaded ahead of the weights, times the waves per
// workgroup: 80 / WMAX float4 per thread cover k = 20480 in one round trip.
constexpr int kXPre = 80;

// The previous layer's tail, fused into the gate+up kernel's prologue
// (Ch 10 "The forward pass at a glance", section 10.3: the tail's second
// output is the next layer's input).
struct TailIn {
    const float *res_in, *proj, *g_post, *g_next;  // proj null: zero; gains null: unit
    float *res_out, *x_out;  // written by workgroup 0 unless null
    float eps_post, eps_next;
};

// One wave holds RPT = 64/LANES rows; lane `sub` of a row takes units sub,
// sub+LANES, ...  Each lane keeps DEPTH units of look-ahead in flight: the
// first DEPTH loads are issued before the activation staging (so HBM is busy
// while x is converted), and every step issues the load DEPTH units ahead
// before computing the current one.  DEPTH = 0 loads and computes in turn.
// The rows are those of up to kMaxSegs matrices sharing x (MatSegs); a plain
// matvec is one segment.  n_rows counts the rows of all segments.  FMT is the
// superblock format: 4 = Q4_K, 5 = Q5_K (the same scales, mins and 32-input
// sub-blocks, one more bit per quant).
template <int FMT, int LANES, int LIMBS, int DEPTH, int WMAX, bool SILU>
__global__ __launch_bounds__(64 * WMAX) void q45k_matvec_kernel(const MatSegs segs,
                                                                const float *__restrict__ x,
                                                                const uint8_t *__restrict__ xs,
                                                                const float *__restrict__ gate,
                                                                int n_rows, int k)
{
    using F = KFmt<FMT>;
    extern __shared__ __align__(16) uint8_t smem[];
    const int nsb = k >> 8;
    const int units = 2 * nsb;
    const int64_t row_bytes = (int64_t)nsb * F::kBytes;
    const int r_lo = (int)((int64_t)blockIdx.x * n_rows / gridDim.x);
    const int r_hi = (int)((int64_t)(blockIdx.x + 1) * n_rows / gridDim.x);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    constexpr int RPT = 64 / LANES;
    const int sub = lane % LANES;
    const int h = sub & 1;  // LANES is even: a lane always takes the same half
    const int steps = (units + LANES - 1) / LANES;
    const XPre<kXPre / WMAX> xpre =  // ahead of any weight load
        x_preload<kXPre / WMAX>(xs ? (const void *)xs : (const void *)x, x_pieces<32, LIMBS>(xs, k));

    int t0 = r_lo + wave * RPT;
    int r = t0 + lane / LANES;
    bool rv = r < r_hi;
    const uint8_t *rowp = seg_row(segs, rv ? r : r_lo, row_bytes);
    // Loads are unconditional: a lane past the row's last unit re-reads that
    // unit, a lane without a row reads the workgroup's first row (its result
    // is dropped), so every wave issues the same loads in the same order and
    // waits only for the unit it is about to use.
    auto load = [&](int st) {
        const int u = min(sub + LANES * st, units - 1);
        return F::load(rowp + (int64_t)(u >> 1) * F::kBytes, h);
    };
    constexpr int R = DEPTH + 1;
    typename F::Unit ring[R];
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) {  // slot by slot, as the loop issues them
        ring[j] = load(j);
        __builtin_amdgcn_sched_barrier(0);
    }

    stage_activation<32, LIMBS>(xpre, x, xs, k, smem);
    __syncthreads();
    const uint8_t *planes = smem;
    const float *tscale = reinterpret_cast<const float *>(smem + LIMBS * plane_bytes(k));
    const float *tsum = tscale + (k >> 5);

    while (t0 < r_hi) {
        float acc = 0.0f;
        // step st computes ring slot st % R and first refills the slot freed
        // by the previous step with unit st + DEPTH
        auto step = [&](int j, int st, bool prefetch) __attribute__((always_inline)) {
            // keep each step's arithmetic inside the step: hoisted into an
            // earlier step it would wait there for loads still in flight
            __builtin_amdgcn_sched_barrier(0);
            if (prefetch) ring[(j + DEPTH) % R] = load(st + DEPTH);
            __builtin_amdgcn_sched_barrier(0);
            const int u = sub + LANES * st;
            const int uc = min(u, units - 1);  // the unit that was loaded
            const float d = F::template dot<LIMBS>(ring[j], h, 256 * (uc >> 1) + 128 * h, k,
                                                   planes, tscale, tsum);
            acc += (rv && u < units) ? d : 0.0f;
        };
        // whole passes of R steps: constant slot indices and no branch between
        // a load and its use, so each wait covers exactly the unit needed
        int s0 = 0;
        for (; s0 + R <= steps; s0 += R) {
#pragma unroll
            for (int j = 0; j < R; ++j) step(j, s0 + j, true);
        }
        // the last steps - s0 < R steps: their units are already in flight
#pragma unroll
        for (int j = 0; j + 1 < R; ++j)
            if (s0 + j < steps) step(j, s0 + j, false);
        acc = lane_group_sum<LANES>(acc);
        if (sub == 0 && rv) {
            if constexpr (SILU) {
                const float g = gate[r];
                acc = (g / (1.0f + __expf(-g))) * acc;
            }
            *seg_out(segs, r) = acc;
        }
        t0 += nwaves * RPT;
        r = t0 + lane / LANES;
        rv = r < r_hi;
        rowp = seg_row(segs, rv ? r : r_lo, row_bytes);
        if (t0 < r_hi) {
#pragma unroll
            for (int j = 0; j < DEPTH; ++j) {
                ring[j] = load(j);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
}

// Gate and up projections in one pass: the lanes of a row task stream the
// gate row's units and then the up row's units for the same ffn index (one
// activation staging, one launch) and store mid = silu(gate x) * (up x)
// (Ch 10 "The forward pass at a glance", section 10.3: gate and up read the
// same normed input; the SiLU product follows them).
//
// With TAIL the input is not given: every workgroup first runs the previous
// layer's dual-eps tail on (tl.res_in, tl.proj) itself, in the thread layout
// and summation order of the standalone tail (so its values are bit for bit
// the standalone tail's), and encodes the result straight into LDS; workgroup
// 0 also stores the post-add residual (tl.res_out) and next_in (tl.x_out).
template <int LANES, int LIMBS, int DEPTH, int WMAX, bool TAIL>
__global__ __launch_bounds__(64 * WMAX) void q4k_gate_up_kernel(const uint8_t *__restrict__ Wg,
                                                                const uint8_t *__restrict__ Wu,
                                                                const float *__restrict__ x,
                                                                const uint8_t *__restrict__ xs,
                                                                float *__restrict__ mid,
                                                                uint8_t *__restrict__ mid_s,
                                                                int mid_group, int n_rows, int k,
                                                                TailIn tl)
{
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ float red[2][16];  // one buffer per reduction
    const int nsb = k >> 8;
    const int units = 2 * nsb;      // half-superblock units per row
    const int units2 = 2 * units;   // gate units, then up units
    const int64_t row_bytes = (int64_t)nsb * kQ4Bytes;
    // With a staged mid output every workgroup owns whole scale groups of
    // mid_group rows (it encodes them itself); otherwise an even row split.
    const int rg = mid_s ? mid_group : 1;
    const int ngr = n_rows / rg;
    // Workgroup b runs on XCD b mod 8.  An uneven split of the groups gives
    // the shorter ranges to fixed slots mod 8, which would put them all on one
    // XCD; each block of 8 workgroups takes its 8 ranges rotated by the block
    // index instead, so every XCD gets its share of short ranges (the ranges
    // stay contiguous and in place within the block).
    const int slot = (gridDim.x & 7) ? (int)blockIdx.x
                                     : (int)((blockIdx.x & ~7u) | ((blockIdx.x + (blockIdx.x >> 3)) & 7u));
    const int r_lo = rg * (int)((int64_t)slot * ngr / gridDim.x);
    const int r_hi = rg * (int)((int64_t)(slot + 1) * ngr / gridDim.x);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    constexpr int RPT = 64 / LANES;
    const int sub = lane % LANES;
    const int h = sub & 1;  // LANES and units are even: a lane always takes the same half
    float *midl = reinterpret_cast<float *>(smem + staged_bytes<32, LIMBS>(k));  // this group's mid
    const int steps = (units2 + LANES - 1) / LANES;
    // the activation (or the tail's operands) ahead of any weight load
    XPre<TAIL ? 1 : kXPre / WMAX> xpre;
    const int tt = tail_threads(k), n4 = k >> 2;
    const int tid = threadIdx.x;
    f32x4 tp[kTailVec], tr[kTailVec], tg[kTailVec], tn[kTailVec];
    const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (TAIL) {
        // Only the waves of the standalone tail's layout load (a wave-uniform
        // branch); within them the loads are unconditional (index clamped into
        // the row; slots outside the layout are zeroed at first use), p first:
        // the first sum needs only p.
        // a null projection is a zero one, a null gain a unit one (the
        // entry norm of a layer stack); their loads read res_in instead, so
        // the loads stay unconditional, and the values are replaced below
        const f32x4 *pp4 = reinterpret_cast<const f32x4 *>(tl.proj ? tl.proj : tl.res_in);
        const f32x4 *gp4 = reinterpret_cast<const f32x4 *>(tl.g_post ? tl.g_post : tl.res_in);
        const f32x4 *gn4 = reinterpret_cast<const f32x4 *>(tl.g_next ? tl.g_next : tl.res_in);
        if (tid < tt) {
#pragma unroll
            for (int j = 0; j < kTailVec; ++j) tp[j] = pp4[min(tid + j * tt, n4 - 1)];
#pragma unroll
            for (int j = 0; j < kTailVec; ++j)
                tr[j] = reinterpret_cast<const f32x4 *>(tl.res_in)[min(tid + j * tt, n4 - 1)];
#pragma unroll
            for (int j = 0; j < kTailVec; ++j) tg[j] = gp4[min(tid + j * tt, n4 - 1)];
#pragma unroll
            for (int j = 0; j < kTailVec; ++j) tn[j] = gn4[min(tid + j * tt, n4 - 1)];
        } else {
#pragma unroll
            for (int j = 0; j < kTailVec; ++j) tp[j] = tr[j] = tg[j] = tn[j] = z;
        }
    } else {
        xpre = x_preload<kXPre / WMAX>(xs ? (const void *)xs : (const void *)x,
                                       x_pieces<32, LIMBS>(xs, k));
    }

    int t0 = r_lo + wave * RPT;
    int r = t0 + lane / LANES;
    bool rv = r < r_hi;
    const uint8_t *gp = Wg + (int64_t)(rv ? r : r_lo) * row_bytes;
    const uint8_t *up = Wu + (int64_t)(rv ? r : r_lo) * row_bytes;
    // unconditional loads, as in q4k_matvec_kernel
    auto load = [&](int st) {
        const int u = min(sub + LANES * st, units2 - 1);
        const uint8_t *p = u < units ? gp + (int64_t)(u >> 1) * kQ4Bytes
                                     : up + (int64_t)((u - units) >> 1) * kQ4Bytes;
        return q4_load(p, h);
    };
    constexpr int R = DEPTH + 1;
    Q4Unit ring[R];
    auto ring_prologue = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < DEPTH; ++j) {  // slot by slot, as the loop issues them
            ring[j] = load(j);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // the first weight loads go out before the activation staging; with TAIL
    // right behind the tail's operand loads (issued before them, they delay
    // the tail's first-touch reads behind the whole chip's weight requests;
    // issued after the tail's sums, as they once were, the pass measured
    // 0.3 % slower)
    ring_prologue();

    if constexpr (TAIL) {
        // the standalone tail's arithmetic, in its order; threads past its
        // block add exact zeros to the (non-negative) sums
        const float inv_n = 1.0f / (float)k;
        const f32x4 one = {1.0f, 1.0f, 1.0f, 1.0f};
#pragma unroll
        for (int j = 0; j < kTailVec; ++j) {
            const bool ok = tid < tt && tid + j * tt < n4;
            tp[j] = ok && tl.proj ? tp[j] : z;
            tr[j] = ok ? tr[j] : z;
            tg[j] = ok ? (tl.g_post ? tg[j] : one) : z;
            tn[j] = ok ? (tl.g_next ? tn[j] : one) : z;
        }
        float ss = 0.0f;
#pragma unroll
        for (int j = 0; j < kTailVec; ++j) ss += sumsq4(tp[j]);
        ss = block_sum_fresh(ss, red[0]);
        const float inv_p = rsqrtf(__builtin_fmaf(ss, inv_n, tl.eps_post));
        float sr = 0.0f;
#pragma unroll
        for (int j = 0; j < kTailVec; ++j) {
            const int i = tid + j * tt;
            tr[j] = tail_add(tr[j], tp[j], inv_p, tg[j]);
            if (blockIdx.x == 0 && tl.res_out && tid < tt && i < n4)
                reinterpret_cast<f32x4 *>(tl.res_out)[i] = tr[j];
            sr += sumsq4(tr[j]);
        }
        sr = block_sum_fresh(sr, red[1]);
        const float inv_r = rsqrtf(__builtin_fmaf(sr, inv_n, tl.eps_next));
        uint32_t *plane = reinterpret_cast<uint32_t *>(smem);
        float *tsc = reinterpret_cast<float *>(smem + LIMBS * plane_bytes(k));
#pragma unroll
        for (int j = 0; j < kTailVec; ++j) {
            const int i = tid + j * tt;
            if (tid < tt && i < n4) {  // whole scale groups of lanes
                const f32x4 o = tail_next(tr[j], inv_r, tn[j]);
                if (blockIdx.x == 0 && tl.x_out) reinterpret_cast<f32x4 *>(tl.x_out)[i] = o;
                stage_group<32, LIMBS>(o, i, plane, n4, tsc, tsc + (k >> 5));
            }
        }
    } else {
        stage_activation<32, LIMBS>(xpre, x, xs, k, smem);
    }
    __syncthreads();
    const uint8_t *planes = smem;
    const float *tscale = reinterpret_cast<const float *>(smem + LIMBS * plane_bytes(k));
    const float *tsum = tscale + (k >> 5);

    while (t0 < r_hi) {
        float acc_g = 0.0f, acc_u = 0.0f;
        auto step = [&](int j, int st, bool prefetch) __attribute__((always_inline)) {
            // keep each step's arithmetic inside the step: hoisted into an
            // earlier step it would wait there for loads still in flight
            __builtin_amdgcn_sched_barrier(0);
            if (prefetch) ring[(j + DEPTH) % R] = load(st + DEPTH);
            __builtin_amdgcn_sched_barrier(0);
            const int u = sub + LANES * st;
            const int uc = min(u, units2 - 1);  // the unit that was loaded
            const int uu = uc < units ? uc : uc - units;
            const float d = q4_unit_dot<LIMBS>(ring[j], h, 256 * (uu >> 1) + 128 * h, k, planes,
                                               tscale, tsum);
            acc_g += (rv && u < units) ? d : 0.0f;
            acc_u += (rv && u >= units && u < units2) ? d : 0.0f;
        };
        int s0 = 0;
        for (; s0 + R <= steps; s0 += R) {
#pragma unroll
            for (int j = 0; j < R; ++j) step(j, s0 + j, true);
        }
#pragma unroll
        for (int j = 0; j + 1 < R; ++j)
            if (s0 + j < steps) step(j, s0 + j, false);
        acc_g = lane_group_sum<LANES>(acc_g);
        acc_u = lane_group_sum<LANES>(acc_u);
        if (sub == 0 && rv) {
            const float m = (acc_g / (1.0f + __expf(-acc_g))) * acc_u;
            mid[r] = m;  // (unconditional: a branch on mid here made the kernel 10 % slower)
            if (mid_s) midl[r - r_lo] = m;
        }
        t0 += nwaves * RPT;
        r = t0 + lane / LANES;
        rv = r < r_hi;
        gp = Wg + (int64_t)(rv ? r : r_lo) * row_bytes;
        up = Wu + (int64_t)(rv ? r : r_lo) * row_bytes;
        if (t0 < r_hi) {
#pragma unroll
            for (int j = 0; j < DEPTH; ++j) {
                ring[j] = load(j);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    if (mid_s) {
        // staged form of this workgroup's rows of mid for the next matvec:
        // consecutive lanes hold consecutive float4, whole groups of lanes
        __syncthreads();
        const int n4w = (r_hi - r_lo) >> 2;
        for (int t = threadIdx.x; t < n4w; t += blockDim.x) {
            const f32x4 v = reinterpret_cast<const f32x4 *>(midl)[t];
            const int i = (r_lo >> 2) + t;
            if (mid_group == 16)
                stage_group_global<16, LIMBS>(v, i, mid_s, n_rows);
            else
                stage_group_global<32, LIMBS>(v, i, mid_s, n_rows);
        }
    }
}

template <int LANES, int LIMBS, int DEPTH, int WMAX>
__global__ __launch_bounds__(64 * WMAX) void q6k_matvec_kernel(const MatSegs segs,
                                                               const float *__restrict__ x,
                                                               const uint8_t *__restrict__ xs,
                                                               int n_rows, int k)
{
    extern __shared__ __align__(16) uint8_t smem[];
    const int nsb = k >> 8;
    const int units = 2 * nsb;
    const int64_t row_bytes = (int64_t)nsb * kQ6Bytes;
    const int r_lo = (int)((int64_t)blockIdx.x * n_rows / gridDim.x);
    const int r_hi = (int)((int64_t)(blockIdx.x + 1) * n_rows / gridDim.x);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    constexpr int RPT = 64 / LANES;
    const int sub = lane % LANES;
    const int h = sub & 1;
    const int steps = (units + LANES - 1) / LANES;
    const XPre<kXPre / WMAX> xpre =  // ahead of any weight load
        x_preload<kXPre / WMAX>(xs ? (const void *)xs : (const void *)x, x_pieces<16, LIMBS>(xs, k));

    int t0 = r_lo + wave * RPT;
    int r = t0 + lane / LANES;
    bool rv = r < r_hi;
    const uint8_t *rowp = seg_row(segs, rv ? r : r_lo, row_bytes);
    // unconditional loads, as in q4k_matvec_kernel
    auto load = [&](int st) {
        const int u = min(sub + LANES * st, units - 1);
        return q6_load(rowp + (int64_t)(u >> 1) * kQ6Bytes, h);
    };
    constexpr int R = DEPTH + 1;
    Q6Unit ring[R];
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) {  // slot by slot, as the loop issues them
        ring[j] = load(j);
        __builtin_amdgcn_sched_barrier(0);
    }

    stage_activation<16, LIMBS>(xpre, x, xs, k, smem);
    __syncthreads();
    const uint8_t *planes = smem;
    const float *tscale = reinterpret_cast<const float *>(smem + LIMBS * plane_bytes(k));
    const float *tsum = tscale + (k >> 4);

    while (t0 < r_hi) {
        float acc = 0.0f;
        auto step = [&](int j, int st, bool prefetch) __attribute__((always_inline)) {
            // keep each step's arithmetic inside the step: hoisted into an
            // earlier step it would wait there for loads still in flight
            __builtin_amdgcn_sched_barrier(0);
            if (prefetch) ring[(j + DEPTH) % R] = load(st + DEPTH);
            __builtin_amdgcn_sched_barrier(0);
            const int u = sub + LANES * st;
            const int uc = min(u, units - 1);  // the unit that was loaded
            const float d = q6_unit_dot<LIMBS>(ring[j], 256 * (uc >> 1) + 128 * h, k, planes,
                                               tscale, tsum);
            acc += (rv && u < units) ? d : 0.0f;
        };
        int s0 = 0;
        for (; s0 + R <= steps; s0 += R) {
#pragma unroll
            for (int j = 0; j < R; ++j) step(j, s0 + j, true);
        }
#pragma unroll
        for (int j = 0; j + 1 < R; ++j)
            if (s0 + j < steps) step(j, s0 + j, false);
        acc = lane_group_sum<LANES>(acc);
        if (sub == 0 && rv) *seg_out(segs, r) = acc;
        t0 += nwaves * RPT;
        r = t0 + lane / LANES;
        rv = r < r_hi;
        rowp = seg_row(segs, rv ? r : r_lo, row_bytes);
        if (t0 < r_hi) {
#pragma unroll
            for (int j = 0; j < DEPTH; ++j) {
                ring[j] = load(j);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
}

// Q4_K and Q6_K as seen by rows_kernel: unit load, unit dot, scale group.
template <int FMT> struct RowsFmt;
template <> struct RowsFmt<4> {
    using Unit = Q4Unit;
    static constexpr int kBytes = kQ4Bytes, kGroup = 32;
    static __device__ __forceinline__ Unit load(const uint8_t *sb, int h) { return q4_load(sb, h); }
    template <int LIMBS>
    static __device__ __forceinline__ float dot(const Unit &u, int h, int base, int k,
                                                const uint8_t *planes, const float *tscale,
                                                const float *tsum)
    {
        return q4_unit_dot<LIMBS>(u, h, base, k, planes, tscale, tsum);
    }
};
template <> struct RowsFmt<6> {
    using Unit = Q6Unit;
    static constexpr int kBytes = kQ6Bytes, kGroup = 16;
    static __device__ __forceinline__ Unit load(const uint8_t *sb, int h) { return q6_load(sb, h); }
    template <int LIMBS>
    static __device__ __forceinline__ float dot(const Unit &u, int, int base, int k,
                                                const uint8_t *planes, const float *tscale,
                                                const float *tsum)
    {
        return q6_unit_dot<LIMBS>(u, base, k, planes, tscale, tsum);
    }
};

// MR activation rows through the matvec's integer dot path (Ch 36 "Prefill vs
// decode", section 36.4: each weight row is read once and applied to every
// input column).  Each workgroup stages all MR rows of X (row m at
// X + m * ldx) into LDS with the matvec's encoding, then loads each weight
// unit once and dots it with every row.  Per row the arithmetic is that of
// the 8-lane matvec on the same row, so a row's result does not depend on
// MR, and the call needs no memory beyond its operands.  The matvec is bound
// by its weight stream with the VALU partly idle, so a second row costs
// little time; every further row adds its own integer dots (about 150 VALU
// instructions per Q4_K unit, the bound) and LDS reads of the staged planes,
// which is why the matrix-core path wins from three rows on.
// MODE kRowsPlain: Y = W X.  kRowsSilu: Y = silu(gate) * (W X) row by row;
// gate may be Y itself (each element is read before it is overwritten).
// kRowsGateUp (Q4_K): W is the gate matrix and W2 the up matrix; a row task
// streams the gate row's units, then the up row's, as q4k_gate_up_kernel
// does (Ch 10 "The forward pass at a glance", section 10.3: gate and up read
// the same normed input), and Y = silu(W X) * (W2 X): each output row equals
// that one-launch kernel's at 8 lanes per row bit for bit.
constexpr int kRowsPlain = 0, kRowsSilu = 1, kRowsGateUp = 2;
template <int FMT, int LIMBS, int DEPTH, int WMAX, int MR, int MODE>
__global__ __launch_bounds__(64 * WMAX) void rows_kernel(const uint8_t *__restrict__ W,
                                                         const uint8_t *__restrict__ W2,
                                                         const float *__restrict__ X, int64_t ldx,
                                                         float *Y, int64_t ldy,
                                                         const float *gate, int64_t ldg,
                                                         int n_rows, int k)
{
    static_assert(MODE != kRowsGateUp || FMT == 4, "gate and up are Q4_K");
    using F = RowsFmt<FMT>;
    constexpr int LANES = 8, RPT = 64 / LANES;
    extern __shared__ __align__(16) uint8_t smem[];
    const int nsb = k >> 8;
    const int units = 2 * nsb;
    const int units2 = MODE == kRowsGateUp ? 2 * units : units;  // gate units, then up units
    const int64_t row_bytes = (int64_t)nsb * F::kBytes;
    const int r_lo = (int)((int64_t)blockIdx.x * n_rows / gridDim.x);
    const int r_hi = (int)((int64_t)(blockIdx.x + 1) * n_rows / gridDim.x);
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x >> 6;
    const int sub = lane % LANES;
    const int h = sub & 1;
    const int steps = (units2 + LANES - 1) / LANES;
    const int sb = (int)staged_bytes<F::kGroup, LIMBS>(k);  // one staged row (a multiple of 16)
    // row 0 of X ahead of any weight load (one round trip)
    constexpr int B = kXPre / WMAX;
    XPre<B> pre = x_preload<B>(X, k >> 2);
    int t0 = r_lo + wave * RPT;
    int r = t0 + lane / LANES;
    bool rv = r < r_hi;
    int64_t rowoff = (int64_t)(rv ? r : r_lo) * row_bytes;
    auto load = [&](int st) {
        const int u = min(sub + LANES * st, units2 - 1);
        if constexpr (MODE == kRowsGateUp)
            return F::load(u < units ? W + rowoff + (int64_t)(u >> 1) * F::kBytes
                                     : W2 + rowoff + (int64_t)((u - units) >> 1) * F::kBytes,
                           h);
        else
            return F::load(W + rowoff + (int64_t)(u >> 1) * F::kBytes, h);
    };
    constexpr int R = DEPTH + 1;
    typename F::Unit ring[R];
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) {
        ring[j] = load(j);
        __builtin_amdgcn_sched_barrier(0);
    }
    // every row staged as the matvec stages x, row m at smem + m * sb; the
    // next row's loads go out before the current row is encoded
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        XPre<B> nxt;
        if (m + 1 < MR) nxt = x_preload<B>(X + (m + 1) * ldx, k >> 2);
        stage_activation<F::kGroup, LIMBS, B>(pre, X + m * ldx, nullptr, k, smem + m * sb);
        if (m + 1 < MR) pre = nxt;
    }
    __syncthreads();
    const int P = (int)plane_bytes(k);

    while (t0 < r_hi) {
        float acc[MR], acc_u[MR];  // acc_u: the up sums (kRowsGateUp)
#pragma unroll
        for (int m = 0; m < MR; ++m) acc[m] = acc_u[m] = 0.0f;
        auto step = [&](int j, int st, bool prefetch) __attribute__((always_inline)) {
            __builtin_amdgcn_sched_barrier(0);
            if (prefetch) ring[(j + DEPTH) % R] = load(st + DEPTH);
            __builtin_amdgcn_sched_barrier(0);
            const int u = sub + LANES * st;
            const int uc = min(u, units2 - 1);
            const int uu = uc < units ? uc : uc - units;  // the unit within its row
            const bool ok = rv && u < units;
            const bool ok_u = rv && u >= units && u < units2;
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const uint8_t *planes = smem + m * sb;
                const float *tscale = reinterpret_cast<const float *>(planes + LIMBS * P);
                const float *tsum = tscale + k / F::kGroup;
                const float d = F::template dot<LIMBS>(ring[j], h, 256 * (uu >> 1) + 128 * h, k,
                                                       planes, tscale, tsum);
                acc[m] += ok ? d : 0.0f;
                if constexpr (MODE == kRowsGateUp) acc_u[m] += ok_u ? d : 0.0f;
            }
        };
        int s0 = 0;
        for (; s0 + R <= steps; s0 += R) {
#pragma unroll
            for (int j = 0; j < R; ++j) step(j, s0 + j, true);
        }
#pragma unroll
        for (int j = 0; j + 1 < R; ++j)
            if (s0 + j < steps) step(j, s0 + j, false);
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            acc[m] = lane_group_sum<LANES>(acc[m]);
            if constexpr (MODE == kRowsGateUp) acc_u[m] = lane_group_sum<LANES>(acc_u[m]);
        }
        if (sub == 0 && rv) {
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                float y = acc[m];
                if constexpr (MODE == kRowsSilu) {
                    const float g = gate[m * ldg + r];
                    y = (g / (1.0f + __expf(-g))) * y;
                } else if constexpr (MODE == kRowsGateUp) {
                    y = (y / (1.0f + __expf(-y))) * acc_u[m];
                }
                Y[m * ldy + r] = y;
            }
        }
        t0 += nwaves * RPT;
        r = t0 + lane / LANES;
        rv = r < r_hi;
        rowoff = (int64_t)(rv ? r : r_lo) * row_bytes;
        if (t0 < r_hi) {
#pragma unroll
            for (int j = 0; j < DEPTH; ++j) {
                ring[j] = load(j);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
}

// Staged form of a plain activation vector (the encoding the matvec kernels
// otherwise apply per workgroup), for callers that hand the same x to several
// matvecs.  One float4 per thread; k is a multiple of 256, so the blocks hold
// whole scale groups.
template <int GROUP>
__global__ __launch_bounds__(256) void stage_kernel(const float *__restrict__ x,
                                                    uint8_t *__restrict__ xs, int k)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < (k >> 2))
        stage_group_global<GROUP, KQ_LIMBS>(reinterpret_cast<const f32x4 *>(x)[i], i, xs, k);
}

// Staged output of the tail (the next layer's input in the form its matvec
// consumes; groups of 32 for Q4_K, 16 for Q6_K).  Callers pass whole groups
// of consecutive lanes: n is a multiple of the group, the block a multiple of
// 64 threads.
__device__ __forceinline__ int64_t tail_staged_bytes(int n, int group)
{
    return group == 16 ? staged_bytes<16, KQ_LIMBS>(n) : staged_bytes<32, KQ_LIMBS>(n);
}

__device__ __forceinline__ void stage_tail_out(f32x4 o, int i, uint8_t *xs, int n, int group)
{
    if (group == 16)
        stage_group_global<16, KQ_LIMBS>(o, i, xs, n);
    else
        stage_group_global<32, KQ_LIMBS>(o, i, xs, n);
}

// ---------------------------------------------------------------------------
// Fused dual-epsilon tail: one workgroup per row, float4 slots strided over
// the threads.  Three passes as the operation is defined: the sum of squares
// of the projection; the residual add, written to memory, with the sum of
// squares of the stored f32 sums; the next norm, computed from the stored
// residual.  The row (26 KB at n = 6656) stays in L2 between passes.  Both
// block reductions run in a fixed order (per thread in slot order, an
// xor-butterfly within a wave, then the per-wave partials in wave order), so
// the result is reproducible bit for bit.
__global__ __launch_bounds__(1024) void tail_kernel(float *__restrict__ residual,
                                                    const float *__restrict__ projected,
                                                    float *__restrict__ next_in,
                                                    const float *__restrict__ g_post,
                                                    const float *__restrict__ g_next, int n,
                                                    float eps_post, float eps_next,
                                                    uint8_t *__restrict__ xs_out, int xs_group)
{
    __shared__ float red[2][16];  // one buffer per reduction
    const int64_t off = (int64_t)blockIdx.x * n;
    f32x4 *r4 = reinterpret_cast<f32x4 *>(residual + off);
    const f32x4 *p4 = reinterpret_cast<const f32x4 *>(projected + off);
    f32x4 *o4 = reinterpret_cast<f32x4 *>(next_in + off);
    const f32x4 *gp4 = reinterpret_cast<const f32x4 *>(g_post);
    const f32x4 *gn4 = reinterpret_cast<const f32x4 *>(g_next);
    const int n4 = n >> 2;
    const float inv_n = 1.0f / (float)n;

    float ss = 0.0f;
    for (int i = threadIdx.x; i < n4; i += blockDim.x) ss += sumsq4(p4[i]);
    ss = block_sum_fresh(ss, red[0]);
    const float inv_p = rsqrtf(__builtin_fmaf(ss, inv_n, eps_post));

    float sr = 0.0f;
    for (int i = threadIdx.x; i < n4; i += blockDim.x) {
        const f32x4 v = r4[i] + (p4[i] * inv_p) * gp4[i];
        r4[i] = v;
        sr += sumsq4(v);
    }
    sr = block_sum_fresh(sr, red[1]);
    const float inv_r = rsqrtf(__builtin_fmaf(sr, inv_n, eps_next));

    uint8_t *xs = xs_out ? xs_out + (int64_t)blockIdx.x * tail_staged_bytes(n, xs_group) : nullptr;
    for (int i = threadIdx.x; i < n4; i += blockDim.x) {
        const f32x4 o = (r4[i] * inv_r) * gn4[i];
        o4[i] = o;
        if (xs) stage_tail_out(o, i, xs, n, xs_group);
    }
}

// Register form of the tail for rows up to kTailRegMax wide: every operand is
// loaded once, up front (one memory round trip instead of three); the post-add
// residual is stored and the next norm uses the same f32 values that were
// stored.  Same reduction order as tail_kernel.

__global__ __launch_bounds__(kTailThreads) void tail_reg_kernel(
    float *__restrict__ residual, const float *__restrict__ projected, float *__restrict__ next_in,
    const float *__restrict__ g_post, const float *__restrict__ g_next, int n, float eps_post,
    float eps_next, uint8_t *__restrict__ xs_out, int xs_group)
{
    __shared__ float red[2][kTailThreads / 64];  // one buffer per reduction
    const int64_t off = (int64_t)blockIdx.x * n;
    f32x4 *r4 = reinterpret_cast<f32x4 *>(residual + off);
    const f32x4 *p4 = reinterpret_cast<const f32x4 *>(projected + off);
    f32x4 *o4 = reinterpret_cast<f32x4 *>(next_in + off);
    const f32x4 *gp4 = reinterpret_cast<const f32x4 *>(g_post);
    const f32x4 *gn4 = reinterpret_cast<const f32x4 *>(g_next);
    const int n4 = n >> 2;
    const float inv_n = 1.0f / (float)n;
    const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};

    f32x4 pv[kTailVec], rv[kTailVec], gp[kTailVec], gn[kTailVec];
#pragma unroll
    for (int j = 0; j < kTailVec; ++j) {
        const int i = threadIdx.x + j * blockDim.x;
        const bool ok = i < n4;
        pv[j] = ok ? p4[i] : z;
        rv[j] = ok ? r4[i] : z;
        gp[j] = ok ? gp4[i] : z;
        gn[j] = ok ? gn4[i] : z;
    }
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < kTailVec; ++j) ss += sumsq4(pv[j]);
    ss = block_sum_fresh(ss, red[0]);
    const float inv_p = rsqrtf(__builtin_fmaf(ss, inv_n, eps_post));

    float sr = 0.0f;
#pragma unroll
    for (int j = 0; j < kTailVec; ++j) {
        const int i = threadIdx.x + j * blockDim.x;
        rv[j] = tail_add(rv[j], pv[j], inv_p, gp[j]);
        if (i < n4) r4[i] = rv[j];
        sr += sumsq4(rv[j]);
    }
    sr = block_sum_fresh(sr, red[1]);
    const float inv_r = rsqrtf(__builtin_fmaf(sr, inv_n, eps_next));
    uint8_t *xs = xs_out ? xs_out + (int64_t)blockIdx.x * tail_staged_bytes(n, xs_group) : nullptr;
#pragma unroll
    for (int j = 0; j < kTailVec; ++j) {
        const int i = threadIdx.x + j * blockDim.x;
        if (i < n4) {
            const f32x4 o = tail_next(rv[j], inv_r, gn[j]);
            o4[i] = o;
            if (xs) stage_tail_out(o, i, xs, n, xs_group);
        }
    }
}

// ---------------------------------------------------------------------------
// Embedding lookup (Ch 10 "The forward pass at a glance", section 10.3, box 1:
// one row of the token table turned into the residual stream): out[t] is row
// tokens[t] of E dequantized.  One workgroup per token, one thread per
// 32-weight sub-block: its scale and min from the superblock header, its 32
// quants (Q5_K: and their fifth bits), 32 floats out.  Each weight is
// (d * sc) * q - dmin * m, products exact in f32, so the one rounding is that
// of the subtraction: the f32 value nearest the exact weight.  A token outside
// [0, vocab) gives a row of NaN and reads nothing.
template <int FMT>
__global__ __launch_bounds__(256) void embedding_kernel(const uint8_t *__restrict__ E,
                                                        const int32_t *__restrict__ tokens,
                                                        float *__restrict__ out, int vocab,
                                                        int hidden)
{
    const int t = blockIdx.x;
    const int tok = tokens[t];
    const int nsb = hidden >> 8;
    f32x4 *o = reinterpret_cast<f32x4 *>(out + (int64_t)t * hidden);
    if (tok < 0 || tok >= vocab) {  // uniform across the workgroup
        const float nan = __builtin_nanf("");
        for (int i = threadIdx.x; i < (hidden >> 2); i += blockDim.x) o[i] = (f32x4){nan, nan, nan, nan};
        return;
    }
    constexpr int B = KFmt<FMT>::kBytes;
    const uint8_t *row = E + (int64_t)tok * nsb * B;
    for (int i = threadIdx.x; i < nsb * 8; i += blockDim.x) {
        const int b = i >> 3, s = i & 7, c = s >> 1, hn = s & 1;
        const uint8_t *sb = row + (int64_t)b * B;
        const u32x4 hdr = *reinterpret_cast<const u32x4 *>(sb);
        // the 12 bytes of packed 6-bit fields are hdr.y, hdr.z, hdr.w
        auto byte = [&](int j) -> uint32_t {
            const uint32_t w = j < 4 ? hdr.y : (j < 8 ? hdr.z : hdr.w);
            return (w >> (8 * (j & 3))) & 0xFFu;
        };
        const uint32_t sc = s < 4 ? (byte(s) & 63u) : ((byte(s + 4) & 15u) | ((byte(s - 4) >> 6) << 4));
        const uint32_t mn = s < 4 ? (byte(s + 4) & 63u) : ((byte(s + 4) >> 4) | ((byte(s) >> 6) << 4));
        const float dsc = half_lo(hdr.x) * (float)sc, dm = half_hi(hdr.x) * (float)mn;
        const u32x4 *qp = reinterpret_cast<const u32x4 *>(sb + (FMT == 5 ? 48 : 16) + 32 * c);
        const u32x4 q[2] = {qp[0], qp[1]};
        u32x4 qh[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
        if constexpr (FMT == 5) {
            qh[0] = *reinterpret_cast<const u32x4 *>(sb + 16);
            qh[1] = *reinterpret_cast<const u32x4 *>(sb + 32);
        }
        f32x4 *dst = o + 64 * b + 8 * s;  // inputs 256 b + 32 s ..
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const uint32_t qw = q[w >> 2][w & 3];
            uint32_t v = hn ? (qw >> 4) & 0x0F0F0F0Fu : qw & 0x0F0F0F0Fu;
            if constexpr (FMT == 5) v |= ((qh[w >> 2][w & 3] >> s) & 0x01010101u) << 4;
            f32x4 r;
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = dsc * (float)((v >> (8 * e)) & 0xFFu) - dm;
            dst[w] = r;
        }
    }
}

// ---------------------------------------------------------------------------
// Read-stream probe: every byte of a buffer read once with 16-byte loads,
// folded with xor so the loads stay live.  It measures the HBM read ceiling
// that the matvecs are compared with; it is not on the decode path.
// Variants: U loads in flight per thread; NT non-temporal loads; CHUNK: each
// workgroup reads one contiguous chunk of the buffer (as a matvec workgroup
// reads its own rows) instead of the whole grid striding over it together
// (each wave instruction then covers 1 KB of consecutive bytes either way).
template <int U, bool NT, bool CHUNK>
__global__ void read_probe_kernel(const u32x4 *__restrict__ p, int64_t n16,
                                  uint32_t *__restrict__ out)
{
    int64_t i, end, stride;
    if constexpr (CHUNK) {
        const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
        const int64_t lo = (int64_t)blockIdx.x * per;
        end = min(lo + per, n16);
        i = lo + threadIdx.x;
        stride = blockDim.x;
    } else {
        end = n16;
        i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
        stride = (int64_t)gridDim.x * blockDim.x;
    }
    uint32_t acc = 0;
    for (; i + (U - 1) * stride < end; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int j = 0; j < U; ++j)
            v[j] = NT ? __builtin_nontemporal_load(p + i + j * stride) : p[i + j * stride];
#pragma unroll
        for (int j = 0; j < U; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
    for (; i < end; i += stride) {
        const u32x4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o);
    if ((threadIdx.x & 63) == 0) out[(int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)] = acc;
}

// ---------------------------------------------------------------------------
// Host side: launch shapes.
kqi::MatvecShape g_override[4] = {};

int device_cus() { return kqi::device_cus(); }

// Pick lanes-per-row, waves per workgroup, grid and depth for a matvec from
// the shapes measured best on MI355X at the FFN sizes (below).  Depth 2 (one
// unit in flight ahead of the one computed) is best everywhere: deeper rings
// cost registers and measured slower.
kqi::MatvecShape choose_shape(int qtype, int64_t n_rows, int units, int cus, bool staged)
{
    // Measured on MI355X (sweeps of lanes 8..64, waves 4..16, a quarter to two
    // workgroups per CU, look-ahead 0..2 units, each shape timed as a graph of
    // launches over >= 1 GiB of rotated copies):
    //   Q4_K 19968 x 6656: 8 lanes, 8 waves, 2 workgroups per CU, 1 unit ahead
    //   Q4_K 6656 x 19968: 32 lanes, 16 waves, 1 workgroup per CU (staged x:
    //                      8 waves, 2 workgroups per CU), 1 unit ahead
    //   Q6_K 6656 x 19968: 8 lanes, 8 waves, 1 workgroup per CU, 1 unit ahead
    //   Q6_K, k <= 8192 and many rows per CU (202048 x 6656): no look-ahead
    //     (201 us against 219: the one-slot ring leaves registers for waves);
    //     at 19968 x 6656 also 32 lanes and two workgroups per CU
    //   few rows per CU (the attention projections: 256, 4096 and 8704 rows
    //     over k = 6656, 6656 rows over k = 4096): the time is the latency of
    //     a few units per lane, so a row takes 16..64 lanes (one unit or two
    //     each) and the rows spread over all CUs: K or V alone 7.8 -> 4.5 us
    //     (Q4_K), 9.3 -> 5.1 us (Q6_K); Q 8.4 -> 6.5 us; the four projections
    //     in one group 11.1 -> 9.8 us; o_proj 7.0 -> 6.3 us.
    // 8 lanes per row keep a row's loads contiguous and the lane reduction to
    // DPP moves; a long Q4_K row (k > 8192) is better split 32 ways (9-13 %
    // faster at k = 19968).  Waves without rows still share the conversion of
    // an f32 x, so a long k takes the widest workgroup the registers allow
    // (Q6_K's ring needs more than 128 VGPRs, which caps it at 8 waves); a
    // staged x is only copied, and then 8 waves are best.
    const bool q6 = qtype == 2;
    const int64_t k = 128 * (int64_t)units;
    const int64_t rpc = n_rows / (cus > 0 ? cus : 1);  // rows per CU
    auto fit = [&](int lanes, int waves, int64_t per_cu, int depth) {
        // grid: per_cu workgroups per CU, but no more than there are wave-sized
        // row groups to hand out
        const int64_t rows_per_wave = 64 / lanes;
        const int64_t row_groups = (n_rows + rows_per_wave - 1) / rows_per_wave;
        int64_t g = per_cu * cus;
        if (g > row_groups) g = row_groups;
        return kqi::MatvecShape{lanes, waves, (int)(g > 0 ? g : 1), depth};
    };
    if (k <= 8192 && rpc < 48) {
        if (rpc < 8) return fit(64, 16, 1, q6 ? 1 : 2);
        if (units >= 48) return q6 ? fit(64, 8, 2, 1) : (rpc < 24 ? fit(32, 8, 1, 2) : fit(64, 16, 1, 2));
        return q6 ? fit(8, 4, 1, 2) : fit(16, 8, 1, 2);
    }
    if (q6 && k <= 8192 && rpc < 100) return fit(32, 8, 2, 1);  // 28.2 -> 25.7 us at 19968 x 6656
    const int64_t tiles = (n_rows + 7) / 8;
    const bool long_q4 = !q6 && k > 8192;
    // two workgroups per CU: short rows with many of them, or long rows on a
    // staged x where both stagings fit in the CU's LDS (32 lanes per row: a
    // workgroup needs only a few rows to keep its 8 waves busy)
    const bool two_per_cu =
        !q6 && ((k <= 8192 && n_rows >= 32 * 2 * (int64_t)cus) ||
                (long_q4 && staged && n_rows >= 8 * 2 * (int64_t)cus &&
                 2 * staged_bytes<32, KQ_LIMBS>(k) <= 160 * 1024));
    // very many rows per CU (the LM head, 789 rows per CU): one 16-wave
    // workgroup per CU streams 4-5 % faster than two 8-wave ones
    const bool huge = !q6 && k <= 8192 && rpc >= 256;
    const int64_t gmax = (two_per_cu && !huge) ? 2 * (int64_t)cus : (int64_t)cus;
    const int grid = (int)(tiles < gmax ? (tiles > 0 ? tiles : 1) : gmax);
    const int waves = huge ? 16 : ((q6 || two_per_cu || staged) ? 8 : 16);
    const int depth = (q6 && k <= 8192 && rpc >= 100) ? 1 : 2;
    return kqi::MatvecShape{long_q4 ? 32 : 8, waves, grid, depth};
}

// Raise a kernel's dynamic-LDS limit once to the largest staging size any
// accepted k needs (the attribute is per function, so the flag is per
// kernel instantiation).
template <auto KERN>
hipError_t allow_lds(size_t bytes)
{
    static std::atomic<uint64_t> done{0};
    if (bytes <= 65536) return hipSuccess;
    return kqi::raise_lds_limit(reinterpret_cast<const void *>(KERN), done, 160 * 1024);
}

template <int GROUP>
size_t staging_bytes(int k)
{
    return (size_t)staged_bytes<GROUP, KQ_LIMBS>(k);
}

kqi::MatvecShape resolve_shape(int qtype, int64_t n_rows, int k, bool staged = false)
{
    kqi::MatvecShape s = choose_shape(qtype, n_rows, 2 * (k >> 8), device_cus(), staged);
    const kqi::MatvecShape o = g_override[qtype];
    if (o.lanes) s.lanes = o.lanes;
    if (o.waves) s.waves = o.waves;
    if (o.grid) s.grid = o.grid;
    if (o.depth) s.depth = o.depth;
    return s;
}

template <int FMT, int LANES, int DEPTH, int WMAX>
hipError_t launch_q45k_cfg(const MatSegs &segs, const float *x, const uint8_t *xs, int n_rows,
                           int k, const float *gate, kqi::MatvecShape s, hipStream_t stream)
{
    const size_t lds = staging_bytes<32>(k);
    hipError_t e;
    if (gate) {
        constexpr auto kern = q45k_matvec_kernel<FMT, LANES, KQ_LIMBS, DEPTH, WMAX, true>;
        if ((e = allow_lds<kern>(lds)) != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(s.grid), dim3(64 * s.waves), lds, stream, segs, x, xs,
                           gate, n_rows, k);
    } else {
        constexpr auto kern = q45k_matvec_kernel<FMT, LANES, KQ_LIMBS, DEPTH, WMAX, false>;
        if ((e = allow_lds<kern>(lds)) != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(s.grid), dim3(64 * s.waves), lds, stream, segs, x, xs,
                           gate, n_rows, k);
    }
    return hipGetLastError();
}

template <int LANES, int DEPTH, int WMAX>
hipError_t launch_q6k_cfg(const MatSegs &segs, const float *x, const uint8_t *xs, int n_rows,
                          int k, const float *, kqi::MatvecShape s, hipStream_t stream)
{
    const size_t lds = staging_bytes<16>(k);
    constexpr auto kern = q6k_matvec_kernel<LANES, KQ_LIMBS, DEPTH, WMAX>;
    hipError_t e = allow_lds<kern>(lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(s.grid), dim3(64 * s.waves), lds, stream, segs, x, xs, n_rows,
                       k);
    return hipGetLastError();
}

// Dispatch a runtime shape to the kernel instantiation: lanes 4..64, units
// in flight per lane 1..3 (look-ahead 0..2), and a workgroup-size class (up to 8 waves gets the 256-VGPR budget
// of two waves per SIMD; up to 16 waves the 128-VGPR budget).
template <template <int, int, int> class F>
hipError_t dispatch_shape(kqi::MatvecShape s, const MatSegs &segs, const float *x,
                          const uint8_t *xs, int n_rows, int k, const float *gate,
                          hipStream_t stream)
{
    const bool small = s.waves <= 8;
#define KQ_CASE(L, D)                                                                        \
    if (s.lanes == L && s.depth == D)                                                        \
        return small ? F<L, D - 1, 8>::go(segs, x, xs, n_rows, k, gate, s, stream)           \
                     : F<L, D - 1, 16>::go(segs, x, xs, n_rows, k, gate, s, stream);
#define KQ_CASES(L) KQ_CASE(L, 1) KQ_CASE(L, 2) KQ_CASE(L, 3)
    KQ_CASES(4) KQ_CASES(8) KQ_CASES(16) KQ_CASES(32) KQ_CASES(64)
#undef KQ_CASES
#undef KQ_CASE
    return hipErrorInvalidValue;
}

template <int LANES, int DEPTH, int WMAX, bool TAIL>
hipError_t launch_gate_up_cfg(const uint8_t *Wg, const uint8_t *Wu, const float *x,
                              const uint8_t *xs, float *mid, uint8_t *mid_s, int mid_group,
                              int n_rows, int k, const TailIn &tl, kqi::MatvecShape s,
                              hipStream_t stream)
{
    // staging, then (with a staged mid) the workgroup's rows of mid
    size_t lds = staging_bytes<32>(k);
    if (mid_s) {
        const int ngr = n_rows / mid_group;
        lds += sizeof(float) * (size_t)mid_group * (size_t)((ngr + s.grid - 1) / s.grid);
    }
    constexpr auto kern = q4k_gate_up_kernel<LANES, KQ_LIMBS, DEPTH, WMAX, TAIL>;
    hipError_t e = allow_lds<kern>(lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(s.grid), dim3(64 * s.waves), lds, stream, Wg, Wu, x, xs, mid,
                       mid_s, mid_group, n_rows, k, tl);
    return hipGetLastError();
}

template <int L, int D, int WM>
struct Q4Launch {
    static hipError_t go(const MatSegs &segs, const float *x, const uint8_t *xs, int n, int k,
                         const float *g, kqi::MatvecShape s, hipStream_t st)
    {
        return launch_q45k_cfg<4, L, D, WM>(segs, x, xs, n, k, g, s, st);
    }
};

template <int L, int D, int WM>
struct Q5Launch {
    static hipError_t go(const MatSegs &segs, const float *x, const uint8_t *xs, int n, int k,
                         const float *g, kqi::MatvecShape s, hipStream_t st)
    {
        return launch_q45k_cfg<5, L, D, WM>(segs, x, xs, n, k, g, s, st);
    }
};

template <int L, int D, int WM>
struct Q6Launch {
    static hipError_t go(const MatSegs &segs, const float *x, const uint8_t *xs, int n, int k,
                         const float *g, kqi::MatvecShape s, hipStream_t st)
    {
        return launch_q6k_cfg<L, D, WM>(segs, x, xs, n, k, g, s, st);
    }
};

// One matrix as a one-segment table.
MatSegs one_seg(const uint8_t *W, float *y, int n_rows)
{
    MatSegs m;
    for (int i = 0; i < kMaxSegs; ++i) {
        m.W[i] = W;
        m.y[i] = y;
        m.end[i] = i == 0 ? n_rows : INT32_MAX;
    }
    return m;
}

}  // namespace

// ---- small M through the matvec's dot path (rows_kernel) ----

namespace {

constexpr int kRowsMaxMr = 4;
constexpr int kRowsLds = 160 * 1024 - 512;  // beside the kernel's static LDS
// largest M sent to rows_kernel by default, per qtype (1: Q4_K, 2: Q6_K),
// from timings against the matrix-core path at the FFN shapes (graphs of 52
// launches): Q4_K 19968x6656 at M = 2 25.0 against 27.7 us, at M = 3 and 4
// 31.0 and 37.6 against 26.2 and 26.7 us (each row adds its own integer dots,
// whose VALU issue grows with M);
// Q6_K 6656x19968 at M = 2 37.1 against 36.7 us
constexpr int kRowsDefault[3] = {0, 2, 0};
std::atomic<int> g_rows_override[3] = {{-1}, {-1}, {-1}};
// largest M of the verify gate+up (kq_ffn_gate_up_q4k_small_m) sent to the
// fused dot path (gate and up rows in one launch) by default; measured at
// 19968 x 6656 (graphs of 52 launches): M = 2 40.2 us against 45.2 us for the
// two single-matrix dot launches, M = 3 52.2 against 52.6 us on the matrix
// cores, M = 4 61.2 against 53.1 us
constexpr int kGuRowsDefault = 3;
std::atomic<int> g_gu_rows_override{-1};

template <int FMT, int WMAX, int MR, int MODE>
hipError_t launch_rows_cfg(const uint8_t *W, const uint8_t *W2, const float *X, int64_t ldx,
                           float *Y, int64_t ldy, const float *gate, int64_t ldg, int n_rows,
                           int k, int grid, size_t lds, hipStream_t stream)
{
    constexpr auto kern = rows_kernel<FMT, KQ_LIMBS, 1, WMAX, MR, MODE>;
    static std::atomic<uint64_t> done{0};
    if (lds > 65536) {
        const hipError_t e = kqi::raise_lds_limit(reinterpret_cast<const void *>(kern), done,
                                                  kRowsLds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * WMAX), lds, stream, W, W2, X, ldx, Y, ldy,
                       gate, ldg, n_rows, k);
    return hipGetLastError();
}

// one workgroup per CU, 8-row wave tasks
int rows_grid(int n_rows)
{
    const int64_t tasks = ((int64_t)n_rows + 7) / 8;
    int64_t g = kqi::device_cus();
    if (g > tasks) g = tasks;
    return (int)(g > 0 ? g : 1);
}

}  // namespace

namespace kqi {

int rows_max_m(int qtype)
{
    if (qtype != 1 && qtype != 2) return 0;
    const int o = g_rows_override[qtype].load();
    return o >= 0 ? o : kRowsDefault[qtype];
}

bool set_rows_max_m(int qtype, int max_m)
{
    if (qtype != 1 && qtype != 2) return false;
    if (max_m < -1 || max_m > kRowsMaxMr) return false;
    g_rows_override[qtype].store(max_m);
    return true;
}

bool rows_path(int qtype, int n_rows, int k, int m)
{
    if (m < 2 || m > rows_max_m(qtype) || n_rows < 1) return false;
    const int64_t sb = qtype == 1 ? staged_bytes<32, KQ_LIMBS>(k) : staged_bytes<16, KQ_LIMBS>(k);
    return (int64_t)m * sb <= kRowsLds;
}

hipError_t launch_rows(int qtype, const uint8_t *W, const float *X, int64_t ldx, float *Y,
                       int64_t ldy, int n_rows, int k, int m, const float *gate, int64_t ldg,
                       hipStream_t stream)
{
    const size_t lds = (size_t)m * (size_t)(qtype == 1 ? staged_bytes<32, KQ_LIMBS>(k)
                                                       : staged_bytes<16, KQ_LIMBS>(k));
    // one workgroup per CU: Q4_K with 16 waves (within 128 VGPRs), Q6_K with
    // 8 (its unit ring needs more than 128 VGPRs)
    const int grid = rows_grid(n_rows);
    const bool silu = gate != nullptr;
#define KQ_RW(F, WM, MR)                                                                       \
    if (m == MR)                                                                               \
        return silu ? launch_rows_cfg<F, WM, MR, kRowsSilu>(W, nullptr, X, ldx, Y, ldy, gate,  \
                                                            ldg, n_rows, k, grid, lds, stream) \
                    : launch_rows_cfg<F, WM, MR, kRowsPlain>(W, nullptr, X, ldx, Y, ldy, gate, \
                                                             ldg, n_rows, k, grid, lds, stream);
    if (qtype == 1) {
        KQ_RW(4, 16, 2) KQ_RW(4, 16, 3) KQ_RW(4, 16, 4)
    } else if (!silu) {
        KQ_RW(6, 8, 2) KQ_RW(6, 8, 3) KQ_RW(6, 8, 4)
    }
#undef KQ_RW
    return hipErrorInvalidValue;
}

int gate_up_rows_max_m()
{
    const int o = g_gu_rows_override.load();
    return o >= 0 ? o : kGuRowsDefault;
}

bool set_gate_up_rows_max_m(int max_m)
{
    if (max_m < -1 || max_m > kRowsMaxMr) return false;
    g_gu_rows_override.store(max_m);
    return true;
}

bool gate_up_rows_path(int n_rows, int k, int m)
{
    if (m < 2 || m > gate_up_rows_max_m() || n_rows < 1) return false;
    return (int64_t)m * staged_bytes<32, KQ_LIMBS>(k) <= kRowsLds;
}

hipError_t launch_rows_gate_up(const uint8_t *Wg, const uint8_t *Wu, const float *X, int64_t ldx,
                               float *Mid, int64_t ldm, int n_rows, int k, int m,
                               hipStream_t stream)
{
    const size_t lds = (size_t)m * (size_t)staged_bytes<32, KQ_LIMBS>(k);
    const int grid = rows_grid(n_rows);
    // 12 waves: 96 rows per round cover the 78 rows a CU gets at the FFN
    // shape, and the 168-VGPR budget of 3 waves per SIMD holds two sums per
    // activation row without spills (16 waves' 128 spill at M = 3 and 4)
#define KQ_GW(MR)                                                                              \
    if (m == MR)                                                                               \
        return launch_rows_cfg<4, 12, MR, kRowsGateUp>(Wg, Wu, X, ldx, Mid, ldm, nullptr, 0,   \
                                                       n_rows, k, grid, lds, stream);
    KQ_GW(2) KQ_GW(3) KQ_GW(4)
#undef KQ_GW
    return hipErrorInvalidValue;
}

}  // namespace kqi

namespace kqi {

int device_cus()
{
    static std::atomic<int> cus[kMaxDevices];  // static storage: starts at zero
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int c = cus[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            c <= 0)
            c = 256;
        cus[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}

hipError_t raise_lds_limit(const void *kernel, std::atomic<uint64_t> &done, int bytes)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = (dev >= 0 && dev < kMaxDevices) ? (uint64_t)1 << dev : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
    return e;
}

void set_shape_override(int qtype, MatvecShape s)
{
    if (qtype >= 1 && qtype <= 3) g_override[qtype] = s;
}

MatvecShape get_shape_override(int qtype)
{
    return (qtype >= 1 && qtype <= 3) ? g_override[qtype] : MatvecShape{0, 0, 0, 0};
}

MatvecShape auto_shape(int qtype, int64_t n_rows, int64_t k, int m)
{
    (void)m;
    return resolve_shape(qtype, n_rows, (int)k);
}

void matvec_plan(int qtype, int64_t n_rows, int k, bool staged, int cus, int64_t *out)
{
    const MatvecShape s = choose_shape(qtype, n_rows, 2 * (k >> 8), cus, staged);
    out[0] = s.lanes;
    out[1] = s.waves;
    out[2] = s.grid;
    out[3] = s.depth;
    out[4] = (int64_t)(qtype == 2 ? staging_bytes<16>(k) : staging_bytes<32>(k));
    out[5] = s.grid > cus ? 2 : 1;  // workgroups per CU the grid is sized for
}

hipError_t launch_matvec_q4k(const uint8_t *W, const float *x, const uint8_t *xs, float *y,
                             int n_rows, int k, const float *silu_gate, hipStream_t stream)
{
    return dispatch_shape<Q4Launch>(resolve_shape(1, n_rows, k, xs != nullptr),
                                    one_seg(W, y, n_rows), x, xs, n_rows, k, silu_gate, stream);
}

hipError_t launch_matvec_group(int qtype, int count, const uint8_t *const *W, float *const *y,
                               const int *rows, const float *x, const uint8_t *xs, int k,
                               hipStream_t stream)
{
    MatSegs m;
    int total = 0;
    for (int i = 0; i < kMaxSegs; ++i) {
        const int j = i < count ? i : count - 1;
        m.W[i] = W[j];
        m.y[i] = y[j];
        if (i < count) total += rows[i];
        m.end[i] = i < count ? total : INT32_MAX;
    }
    const MatvecShape s = resolve_shape(qtype, total, k, xs != nullptr);
    if (qtype == 1) return dispatch_shape<Q4Launch>(s, m, x, xs, total, k, nullptr, stream);
    if (qtype == 3) return dispatch_shape<Q5Launch>(s, m, x, xs, total, k, nullptr, stream);
    return dispatch_shape<Q6Launch>(s, m, x, xs, total, k, nullptr, stream);
}

hipError_t launch_matvec_q5k(const uint8_t *W, const float *x, const uint8_t *xs, float *y,
                             int n_rows, int k, const float *silu_gate, hipStream_t stream)
{
    return dispatch_shape<Q5Launch>(resolve_shape(3, n_rows, k, xs != nullptr),
                                    one_seg(W, y, n_rows), x, xs, n_rows, k, silu_gate, stream);
}

hipError_t launch_gate_up_q4k(const uint8_t *Wg, const uint8_t *Wu, const float *x,
                              const uint8_t *xs, float *mid, uint8_t *mid_s, int mid_group,
                              int n_rows, int k, const TailArgs *tail, hipStream_t stream)
{
    // Measured on MI355X at 19968 x 6656 (sweep of lanes 4/8, waves 4..16,
    // grid 1-2 per CU, depth 1-3): 8 lanes per row, one workgroup per CU and
    // one unit of look-ahead best (31.4 us, 4.8 TB/s).  Waves: one 8-row task
    // each, so the workgroup's rows take one round (at least 8 waves, which
    // share the staging of x; at least the tail's layout with the fused
    // tail): the 80 rows a CU gets at the FFN shape take 10 waves, and the
    // 52-layer pass measured 2.849 ms with 10 against 2.869 ms with 12 (11:
    // 2.857 ms; six alternating runs on one box).
    const int tiles = (n_rows + 7) / 8;
    MatvecShape s{8, 0, tiles < device_cus() ? tiles : device_cus(), 2};
    const MatvecShape o = g_override[1];
    if (o.lanes) s.lanes = o.lanes;
    if (o.grid) s.grid = o.grid;
    if (o.depth) s.depth = o.depth;
    if (mid_s && s.grid > n_rows / mid_group) s.grid = n_rows / mid_group;  // whole groups each
    if (o.waves) {
        s.waves = o.waves;
    } else {
        const int rows_wg = mid_s ? mid_group * ((n_rows / mid_group + s.grid - 1) / s.grid)
                                  : (n_rows + s.grid - 1) / s.grid;
        const int rpt = 64 / s.lanes;  // rows of a wave's task
        int w = (rows_wg + rpt - 1) / rpt;
        if (tail && w < tail_threads(k) / 64) w = tail_threads(k) / 64;
        s.waves = w < 8 ? 8 : (w > 16 ? 16 : w);
    }
    const bool small = s.waves <= 8;
    if (tail) {
        // the fused tail runs on the first tail_threads(k) threads: 8 lanes per
        // row (the measured best) and a workgroup at least that wide
        if (s.lanes != 8 || 64 * s.waves < tail_threads(k)) return hipErrorInvalidValue;
        const TailIn tl{tail->res_in, tail->proj, tail->g_post, tail->g_next,
                        tail->res_out, tail->x_out, tail->eps_post, tail->eps_next};
#define KQ_GT(D)                                                                              \
        if (s.depth == D)                                                                     \
            return small ? launch_gate_up_cfg<8, D - 1, 8, true>(Wg, Wu, x, xs, mid, mid_s,   \
                                                                 mid_group, n_rows, k, tl, s, \
                                                                 stream)                      \
                         : launch_gate_up_cfg<8, D - 1, 16, true>(Wg, Wu, x, xs, mid, mid_s,  \
                                                                  mid_group, n_rows, k, tl,   \
                                                                  s, stream);
        KQ_GT(1) KQ_GT(2) KQ_GT(3)
#undef KQ_GT
        return hipErrorInvalidValue;
    }
    const TailIn none{};
#define KQ_GU(L, D)                                                                           \
    if (s.lanes == L && s.depth == D)                                                         \
        return small ? launch_gate_up_cfg<L, D - 1, 8, false>(Wg, Wu, x, xs, mid, mid_s,      \
                                                              mid_group, n_rows, k, none, s,  \
                                                              stream)                         \
                     : launch_gate_up_cfg<L, D - 1, 16, false>(Wg, Wu, x, xs, mid, mid_s,     \
                                                               mid_group, n_rows, k, none, s, \
                                                               stream);
#define KQ_GUS(L) KQ_GU(L, 1) KQ_GU(L, 2) KQ_GU(L, 3)
    KQ_GUS(4) KQ_GUS(8) KQ_GUS(16) KQ_GUS(32) KQ_GUS(64)
#undef KQ_GUS
#undef KQ_GU
    return hipErrorInvalidValue;
}

hipError_t launch_matvec_q6k(const uint8_t *W, const float *x, const uint8_t *xs, float *y,
                             int n_rows, int k, hipStream_t stream)
{
    return dispatch_shape<Q6Launch>(resolve_shape(2, n_rows, k, xs != nullptr),
                                    one_seg(W, y, n_rows), x, xs, n_rows, k, nullptr, stream);
}

hipError_t launch_tail(float *residual, const float *projected, float *next_in,
                       const float *g_post, const float *g_next, int rows, int n,
                       float eps_post, float eps_next, uint8_t *xs_out, int xs_group,
                       hipStream_t stream)
{
    const int n4 = n >> 2;
    if (n <= kTailRegMax) {
        // up to kTailVec float4 slots per thread, whole waves
        const int threads = tail_threads(n);
        hipLaunchKernelGGL(tail_reg_kernel, dim3(rows), dim3(threads), 0, stream, residual,
                           projected, next_in, g_post, g_next, n, eps_post, eps_next, xs_out,
                           xs_group);
        return hipGetLastError();
    }
    // wider rows: about 4 float4 slots per thread, between 1 and 16 waves
    int threads = ((n4 + 4 * 64 - 1) / (4 * 64)) * 64;
    if (threads < 64) threads = 64;
    if (threads > 1024) threads = 1024;
    hipLaunchKernelGGL(tail_kernel, dim3(rows), dim3(threads), 0, stream, residual, projected,
                       next_in, g_post, g_next, n, eps_post, eps_next, xs_out, xs_group);
    return hipGetLastError();
}

hipError_t launch_embedding(int qtype, const uint8_t *E, const int32_t *tokens, int n_tokens,
                            float *out, int vocab, int hidden, hipStream_t stream)
{
    if (qtype == 3)
        hipLaunchKernelGGL(embedding_kernel<5>, dim3(n_tokens), dim3(256), 0, stream, E, tokens,
                           out, vocab, hidden);
    else
        hipLaunchKernelGGL(embedding_kernel<4>, dim3(n_tokens), dim3(256), 0, stream, E, tokens,
                           out, vocab, hidden);
    return hipGetLastError();
}

hipError_t launch_stage(const float *x, uint8_t *xs, int k, int group, hipStream_t stream)
{
    const int n4 = k >> 2;
    const int grid = (n4 + 255) / 256;
    if (group == 16)
        hipLaunchKernelGGL(stage_kernel<16>, dim3(grid), dim3(256), 0, stream, x, xs, k);
    else
        hipLaunchKernelGGL(stage_kernel<32>, dim3(grid), dim3(256), 0, stream, x, xs, k);
    return hipGetLastError();
}

hipError_t launch_read_probe(const void *buf, int64_t bytes, uint32_t *out, int grid, int block,
                             int unroll, int flags, hipStream_t stream)
{
    const u32x4 *p = reinterpret_cast<const u32x4 *>(buf);
    const int64_t n16 = bytes / 16;
    const bool nt = flags & 1, chunk = flags & 2;
#define KQ_PROBE(U)                                                                             \
    if (unroll == U) {                                                                          \
        if (nt && chunk)                                                                        \
            hipLaunchKernelGGL((read_probe_kernel<U, true, true>), dim3(grid), dim3(block), 0,  \
                               stream, p, n16, out);                                            \
        else if (nt)                                                                            \
            hipLaunchKernelGGL((read_probe_kernel<U, true, false>), dim3(grid), dim3(block), 0, \
                               stream, p, n16, out);                                            \
        else if (chunk)                                                                         \
            hipLaunchKernelGGL((read_probe_kernel<U, false, true>), dim3(grid), dim3(block), 0, \
                               stream, p, n16, out);                                            \
        else                                                                                    \
            hipLaunchKernelGGL((read_probe_kernel<U, false, false>), dim3(grid), dim3(block),   \
                               0, stream, p, n16, out);                                         \
        return hipGetLastError();                                                               \
    }
    KQ_PROBE(1) KQ_PROBE(4) KQ_PROBE(8) KQ_PROBE(16)
#undef KQ_PROBE
    return hipErrorInvalidValue;
}

const char *variant_names()
{
    return "q4k/q5k_matvec[lanes=4..64,limbs=3,depth=1..3,silu=0/1,x=f32|staged,group<=4] q6k_matvec[lanes=4..64,limbs=3,depth=1..3,x=f32|staged,group<=4] "
           "embedding[q4k,q5k] "
           "gate_up[q4k, mid staged out: 0/16/32] "
           "small_m[m=1: matvec; q4k m=2 (tunable to m<=4): matvec dot path over all rows; other m=2..16: f16 MFMA, x split hi+lo, stream-K over 256-row groups; q4k: per-lane weight loads, sub-block scale folded into B, 16 waves x 1 16-row tile; q6k: weight tiles through LDS, m<=8: 16 waves x 1 tile, m>8: 8 waves x 2] tail[n<=8192: registers, 1 round trip; wider: 3 passes]";
}

}  // namespace kqi

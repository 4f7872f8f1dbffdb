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
//    per-weight float conversion.  With three limbs the value keeps 23 bits
//    relative to the group maximum.
//  * Work split: `lanes` lanes share a row and walk its half-superblock units
//    (128 weights) in stride; a wave holds 64/lanes rows; a workgroup owns a
//    contiguous row range.  Per-lane partial sums are folded with a fixed
//    xor-butterfly, so results are bitwise reproducible.
//  * The next unit's loads are issued before the current unit is computed.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kq_internal.h"

#define KQ_LIMBS 3

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kQ4Bytes = 144;
constexpr int kQ6Bytes = 210;

__device__ __forceinline__ int sdot4(uint32_t a, uint32_t b, int c)
{
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

__device__ __forceinline__ float half_lo(uint32_t v)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}

__device__ __forceinline__ float half_hi(uint32_t v)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

template <int LIMBS>
__device__ __forceinline__ constexpr int limb_bits()
{
    return LIMBS == 3 ? 22 : 14;
}

// ---------------------------------------------------------------------------
// Activation staging into LDS.
// Layout: LIMBS byte planes of k bytes each (plane 0 = most significant limb),
// then k/GROUP f32 back-scale factors 2^(e - QB), then k/GROUP f32 group sums.
template <int GROUP, int LIMBS>
__device__ __forceinline__ void stage_activation(const float *__restrict__ x, int k,
                                                 uint8_t *__restrict__ smem)
{
    constexpr int TPG = GROUP / 4;  // threads per group, one float4 each
    constexpr int QB = limb_bits<LIMBS>();
    const int n4 = k >> 2;          // a multiple of 64: whole waves stay active
    uint32_t *plane = reinterpret_cast<uint32_t *>(smem);
    float *tscale = reinterpret_cast<float *>(smem + LIMBS * k);
    float *tsum = tscale + k / GROUP;
    const f32x4 *x4 = reinterpret_cast<const f32x4 *>(x);
    for (int i = threadIdx.x; i < n4; i += blockDim.x) {
        const f32x4 v = x4[i];
        float mx = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
        float sm = (v.x + v.y) + (v.z + v.w);
#pragma unroll
        for (int o = 1; o < TPG; o <<= 1) {
            mx = fmaxf(mx, __shfl_xor(mx, o));
            sm = sm + __shfl_xor(sm, o);
        }
        const int e = __builtin_amdgcn_frexp_expf(mx);  // mx < 2^e
        const int sh = QB - e;
        int q[4];
        q[0] = (int)rintf(ldexpf(v.x, sh));
        q[1] = (int)rintf(ldexpf(v.y, sh));
        q[2] = (int)rintf(ldexpf(v.z, sh));
        q[3] = (int)rintf(ldexpf(v.w, sh));
        uint32_t pk[LIMBS];
#pragma unroll
        for (int l = 0; l < LIMBS; ++l) pk[l] = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // balanced base-256 digits, each in [-128, 127]
            const int c = (q[j] << 24) >> 24;
            const int t = (q[j] - c) >> 8;
            if constexpr (LIMBS == 3) {
                const int b = (t << 24) >> 24;
                const int a = (t - b) >> 8;
                pk[0] |= (uint32_t)(a & 255) << (8 * j);
                pk[1] |= (uint32_t)(b & 255) << (8 * j);
                pk[2] |= (uint32_t)(c & 255) << (8 * j);
            } else {
                pk[0] |= (uint32_t)(t & 255) << (8 * j);
                pk[1] |= (uint32_t)(c & 255) << (8 * j);
            }
        }
#pragma unroll
        for (int l = 0; l < LIMBS; ++l) plane[l * n4 + i] = pk[l];
        if ((i & (TPG - 1)) == 0) {
            const int g = i / TPG;
            tscale[g] = isfinite(sm) ? ldexpf(1.0f, e - QB) : __builtin_nanf("");
            tsum[g] = sm;
        }
    }
}

template <int LIMBS>
__device__ __forceinline__ float combine_limbs(const int *acc)
{
    if constexpr (LIMBS == 3)
        return (float)acc[0] * 65536.0f + (float)(acc[1] * 256 + acc[2]);
    else
        return (float)(acc[0] * 256 + acc[1]);
}

template <int LANES>
__device__ __forceinline__ float lane_group_sum(float v)
{
#pragma unroll
    for (int o = LANES / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// ---------------------------------------------------------------------------
// Q4_K unit = one half superblock (sub-blocks 4h..4h+3, 128 weights): the
// 16-byte header and 64 contiguous bytes of nibbles.
struct Q4Unit {
    u32x4 hdr;
    u32x4 q[4];
};

__device__ __forceinline__ Q4Unit q4_load(const uint8_t *__restrict__ sb, int h)
{
    Q4Unit u;
    u.hdr = *reinterpret_cast<const u32x4 *>(sb);
    const u32x4 *p = reinterpret_cast<const u32x4 *>(sb + 16 + 64 * h);
    u.q[0] = p[0];
    u.q[1] = p[1];
    u.q[2] = p[2];
    u.q[3] = p[3];
    return u;
}

// Contribution of one unit to the row's dot product.  `base` is the input
// position of the unit's first weight (256 b + 128 h).
template <int LIMBS>
__device__ __forceinline__ float q4_unit_dot(const Q4Unit &u, int h, int base, int k,
                                             const uint8_t *__restrict__ planes,
                                             const float *__restrict__ tscale,
                                             const float *__restrict__ tsum)
{
    // 6-bit scales and mins of sub-blocks 4h..4h+3, one per byte.
    const uint32_t S0 = u.hdr.y, S1 = u.hdr.z, S2 = u.hdr.w;
    uint32_t scb, mnb;
    if (h == 0) {
        scb = S0 & 0x3F3F3F3Fu;
        mnb = S1 & 0x3F3F3F3Fu;
    } else {
        scb = (S2 & 0x0F0F0F0Fu) | ((S0 >> 2) & 0x30303030u);
        mnb = ((S2 >> 4) & 0x0F0F0F0Fu) | ((S1 >> 2) & 0x30303030u);
    }
    const float d = half_lo(u.hdr.x), dmin = half_hi(u.hdr.x);

    int acc[4][LIMBS];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int l = 0; l < LIMBS; ++l) acc[s][l] = 0;

#pragma unroll
    for (int p = 0; p < 4; ++p) {
        // 16 bytes = inputs j0..j0+15 of sub-block 2c (low nibbles) and of
        // sub-block 2c+1 (high nibbles), c = 2h + p/2, j0 = 16 (p & 1).
        const int plo = base + 64 * (p >> 1) + 16 * (p & 1);
        const int slo = 2 * (p >> 1);
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            lo[w] = u.q[p][w] & 0x0F0F0F0Fu;
            hi[w] = (u.q[p][w] >> 4) & 0x0F0F0F0Fu;
        }
#pragma unroll
        for (int l = 0; l < LIMBS; ++l) {
            const u32x4 xl = *reinterpret_cast<const u32x4 *>(planes + l * k + plo);
            const u32x4 xh = *reinterpret_cast<const u32x4 *>(planes + l * k + plo + 32);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                acc[slo][l] = sdot4(lo[w], xl[w], acc[slo][l]);
                acc[slo + 1][l] = sdot4(hi[w], xh[w], acc[slo + 1][l]);
            }
        }
    }

    const int g0 = base >> 5;  // first 32-input group of this unit
    const f32x4 gs = *reinterpret_cast<const f32x4 *>(tscale + g0);
    const f32x4 gm = *reinterpret_cast<const f32x4 *>(tsum + g0);
    float out = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const float sc = (float)((scb >> (8 * s)) & 0xFFu);
        const float mn = (float)((mnb >> (8 * s)) & 0xFFu);
        const float v = combine_limbs<LIMBS>(acc[s]);
        out += (d * sc) * (gs[s] * v) - (dmin * mn) * gm[s];
    }
    return out;
}

template <int LANES, int LIMBS, bool SILU>
__global__ __launch_bounds__(1024) void q4k_matvec_kernel(const uint8_t *__restrict__ W,
                                                          const float *__restrict__ x,
                                                          float *__restrict__ y,
                                                          const float *__restrict__ gate,
                                                          int n_rows, int k)
{
    extern __shared__ __align__(16) uint8_t smem[];
    stage_activation<32, LIMBS>(x, k, smem);
    __syncthreads();

    const uint8_t *planes = smem;
    const float *tscale = reinterpret_cast<const float *>(smem + LIMBS * k);
    const float *tsum = tscale + (k >> 5);

    const int nsb = k >> 8;
    const int units = 2 * nsb;
    const int64_t row_bytes = (int64_t)nsb * kQ4Bytes;
    const int r_lo = (int)((int64_t)blockIdx.x * n_rows / gridDim.x);
    const int r_hi = (int)((int64_t)(blockIdx.x + 1) * n_rows / gridDim.x);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    constexpr int RPT = 64 / LANES;
    const int sub = lane % LANES;
    const int h = sub & 1;  // LANES is even: a lane always takes the same half

    for (int t0 = r_lo + wave * RPT; t0 < r_hi; t0 += nwaves * RPT) {
        const int r = t0 + lane / LANES;
        float acc = 0.0f;
        if (r < r_hi) {
            const uint8_t *rowp = W + (int64_t)r * row_bytes;
            int u = sub;
            Q4Unit cur;
            if (u < units) cur = q4_load(rowp + (int64_t)(u >> 1) * kQ4Bytes, h);
            for (; u < units; u += LANES) {
                const int un = u + LANES;
                Q4Unit nxt;
                if (un < units) nxt = q4_load(rowp + (int64_t)(un >> 1) * kQ4Bytes, h);
                acc += q4_unit_dot<LIMBS>(cur, h, 256 * (u >> 1) + 128 * h, k, planes, tscale,
                                          tsum);
                cur = nxt;
            }
        }
        acc = lane_group_sum<LANES>(acc);
        if (sub == 0 && r < r_hi) {
            if constexpr (SILU) {
                const float g = gate[r];
                acc = (g / (1.0f + __expf(-g))) * acc;
            }
            y[r] = acc;
        }
    }
}

// ---------------------------------------------------------------------------
// Q6_K unit = one half superblock h: ql bytes 64h..64h+63, qh bytes
// 128+32h..128+32h+31, the 8 int8 scales 192+8h.., and d.  A superblock
// starts 2-byte aligned when its index is odd, so each field is read with
// 4-byte aligned loads that start up to 2 bytes early and is re-aligned in
// registers (v_alignbyte).  No load reaches past the superblock's last byte.
struct Q6Unit {
    u32x4 ql[4];
    uint32_t ql_x;
    u32x4 qh[2];
    uint32_t qh_x;
    uint32_t sc[3];
    uint32_t d;
    int shift;
};

__device__ __forceinline__ Q6Unit q6_load(const uint8_t *__restrict__ sb, int h)
{
    Q6Unit u;
    const int shift = (int)((uintptr_t)sb & 3u);
    u.shift = shift;
    const uint8_t *a = sb - shift;
    const u32x4_a4 *pl = reinterpret_cast<const u32x4_a4 *>(a + 64 * h);
    u.ql[0] = pl[0];
    u.ql[1] = pl[1];
    u.ql[2] = pl[2];
    u.ql[3] = pl[3];
    u.ql_x = *reinterpret_cast<const uint32_t *>(a + 64 * h + 64);
    const u32x4_a4 *ph = reinterpret_cast<const u32x4_a4 *>(a + 128 + 32 * h);
    u.qh[0] = ph[0];
    u.qh[1] = ph[1];
    u.qh_x = *reinterpret_cast<const uint32_t *>(a + 128 + 32 * h + 32);
    const uint32_t *ps = reinterpret_cast<const uint32_t *>(a + 192 + 8 * h);
    u.sc[0] = ps[0];
    u.sc[1] = ps[1];
    u.sc[2] = shift ? ps[2] : 0u;
    u.d = *reinterpret_cast<const uint16_t *>(sb + 208);
    return u;
}

__device__ __forceinline__ uint32_t realign(uint32_t hi, uint32_t lo, int shift)
{
    return __builtin_amdgcn_alignbyte(hi, lo, (uint32_t)shift);
}

template <int LIMBS>
__device__ __forceinline__ float q6_unit_dot(const Q6Unit &u, int base, int k,
                                             const uint8_t *__restrict__ planes,
                                             const float *__restrict__ tscale,
                                             const float *__restrict__ tsum)
{
    const int sh = u.shift;
    uint32_t ql[17], qh[9];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int w = 0; w < 4; ++w) ql[4 * i + w] = u.ql[i][w];
    ql[16] = u.ql_x;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int w = 0; w < 4; ++w) qh[4 * i + w] = u.qh[i][w];
    qh[8] = u.qh_x;
    uint32_t L[16], H[8];
#pragma unroll
    for (int i = 0; i < 16; ++i) L[i] = realign(ql[i + 1], ql[i], sh);
#pragma unroll
    for (int i = 0; i < 8; ++i) H[i] = realign(qh[i + 1], qh[i], sh);
    const uint32_t sc0 = realign(u.sc[1], u.sc[0], sh);
    const uint32_t sc1 = realign(u.sc[2], u.sc[1], sh);
    const float d = half_lo(u.d);

    // base = 256 b + 128 h; 16-input groups of this unit: base/16 .. base/16+7
    const int g0 = base >> 4;
    const f32x4 gsA = *reinterpret_cast<const f32x4 *>(tscale + g0);
    const f32x4 gsB = *reinterpret_cast<const f32x4 *>(tscale + g0 + 4);
    const f32x4 gmA = *reinterpret_cast<const f32x4 *>(tsum + g0);
    const f32x4 gmB = *reinterpret_cast<const f32x4 *>(tsum + g0 + 4);
    float out = 0.0f;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        int acc[4][LIMBS];
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int l = 0; l < LIMBS; ++l) acc[g][l] = 0;
        uint32_t q[4][4];  // [g][t]: quants of inputs base + 32g + 16jj + 4t .. +3
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t l0 = L[4 * jj + t], l1 = L[8 + 4 * jj + t], hh = H[4 * jj + t];
            q[0][t] = (l0 & 0x0F0F0F0Fu) | ((hh & 0x03030303u) << 4);
            q[1][t] = (l1 & 0x0F0F0F0Fu) | ((hh & 0x0C0C0C0Cu) << 2);
            q[2][t] = ((l0 >> 4) & 0x0F0F0F0Fu) | (hh & 0x30303030u);
            q[3][t] = ((l1 >> 4) & 0x0F0F0F0Fu) | ((hh >> 2) & 0x30303030u);
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int pos = base + 32 * g + 16 * jj;
#pragma unroll
            for (int l = 0; l < LIMBS; ++l) {
                const u32x4 xv = *reinterpret_cast<const u32x4 *>(planes + l * k + pos);
#pragma unroll
                for (int t = 0; t < 4; ++t) acc[g][l] = sdot4(q[g][t], xv[t], acc[g][l]);
            }
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int li = 2 * g + jj;  // local sub-block (16 inputs) 0..7
            const uint32_t sw = (li < 4) ? sc0 : sc1;
            const int scv = ((int)(sw << (24 - 8 * (li & 3)))) >> 24;
            const float gsc = (li < 4) ? gsA[li] : gsB[li - 4];
            const float gsum = (li < 4) ? gmA[li] : gmB[li - 4];
            const float v = combine_limbs<LIMBS>(acc[g]);
            out += (d * (float)scv) * (gsc * v - 32.0f * gsum);
        }
    }
    return out;
}

template <int LANES, int LIMBS>
__global__ __launch_bounds__(1024) void q6k_matvec_kernel(const uint8_t *__restrict__ W,
                                                          const float *__restrict__ x,
                                                          float *__restrict__ y, int n_rows,
                                                          int k)
{
    extern __shared__ __align__(16) uint8_t smem[];
    stage_activation<16, LIMBS>(x, k, smem);
    __syncthreads();

    const uint8_t *planes = smem;
    const float *tscale = reinterpret_cast<const float *>(smem + LIMBS * k);
    const float *tsum = tscale + (k >> 4);

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

    for (int t0 = r_lo + wave * RPT; t0 < r_hi; t0 += nwaves * RPT) {
        const int r = t0 + lane / LANES;
        float acc = 0.0f;
        if (r < r_hi) {
            const uint8_t *rowp = W + (int64_t)r * row_bytes;
            // A Q6_K unit holds 30 registers of raw bytes, so it is not double
            // buffered: the workgroup's many waves keep the loads in flight.
            for (int u = sub; u < units; u += LANES) {
                const Q6Unit cur = q6_load(rowp + (int64_t)(u >> 1) * kQ6Bytes, h);
                acc += q6_unit_dot<LIMBS>(cur, 256 * (u >> 1) + 128 * h, k, planes, tscale,
                                          tsum);
            }
        }
        acc = lane_group_sum<LANES>(acc);
        if (sub == 0 && r < r_hi) y[r] = acc;
    }
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
__device__ __forceinline__ float block_sum_fixed(float v, float *red)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    __syncthreads();  // `red` may still be read from the previous reduction
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    float t = 0.0f;
    for (int w = 0; w < nw; ++w) t += red[w];
    return t;
}

__device__ __forceinline__ float sumsq4(f32x4 v)
{
    return v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
}

__global__ __launch_bounds__(1024) void tail_kernel(float *__restrict__ residual,
                                                    const float *__restrict__ projected,
                                                    float *__restrict__ next_in,
                                                    const float *__restrict__ g_post,
                                                    const float *__restrict__ g_next, int n,
                                                    float eps_post, float eps_next)
{
    __shared__ float red[16];
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
    ss = block_sum_fixed(ss, red);
    const float inv_p = rsqrtf(ss * inv_n + eps_post);

    float sr = 0.0f;
    for (int i = threadIdx.x; i < n4; i += blockDim.x) {
        const f32x4 v = r4[i] + (p4[i] * inv_p) * gp4[i];
        r4[i] = v;
        sr += sumsq4(v);
    }
    sr = block_sum_fixed(sr, red);
    const float inv_r = rsqrtf(sr * inv_n + eps_next);

    for (int i = threadIdx.x; i < n4; i += blockDim.x) o4[i] = (r4[i] * inv_r) * gn4[i];
}

// ---------------------------------------------------------------------------
// Host side: launch shapes.
struct DevInfo {
    int cus = 0;
};

DevInfo g_dev[64];
kqi::MatvecShape g_override[3] = {};

int device_cus()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (g_dev[dev].cus == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        g_dev[dev].cus = cus;
    }
    return g_dev[dev].cus;
}

// Pick lanes-per-row, waves per workgroup and grid for a matvec.  The score
// favours: every lane busy in every unit step, every wave slot holding a
// row, and at least 8 waves per CU for latency hiding.
kqi::MatvecShape choose_shape(int64_t n_rows, int units, int cus)
{
    static const int kLanes[] = {4, 8, 16, 32, 64};
    kqi::MatvecShape best{8, 1, 1};
    double best_score = -1.0;
    for (int L : kLanes) {
        const int rpt = 64 / L;
        const int64_t tiles_total = (n_rows + rpt - 1) / rpt;
        const int grid = (int)(tiles_total < cus ? (tiles_total > 0 ? tiles_total : 1) : cus);
        const int64_t rows_wg = (n_rows + grid - 1) / grid;
        const int64_t tiles = (rows_wg + rpt - 1) / rpt;
        const int waves = (int)(tiles < 16 ? tiles : 16);
        const int64_t rounds = (tiles + waves - 1) / waves;
        const int steps = (units + L - 1) / L;
        const double lane_eff = (double)units / (double)(L * steps);
        const double slot_eff = (double)rows_wg / (double)(rpt * waves * rounds);
        const double occ = waves >= 8 ? 1.0 : (double)waves / 8.0;
        const double score = lane_eff * slot_eff * occ;
        if (score > best_score + 1e-9) {
            best_score = score;
            best = kqi::MatvecShape{L, waves, grid};
        }
    }
    return best;
}

// Raise a kernel's dynamic-LDS limit once to the largest staging size any
// accepted k needs (the attribute is per function, so the flag is per
// kernel instantiation).
template <auto KERN>
hipError_t allow_lds(size_t bytes)
{
    static int done = 0;
    if (bytes <= 65536 || done) return hipSuccess;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(KERN),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e == hipSuccess) done = 1;
    return e;
}

template <int GROUP>
size_t staging_bytes(int k)
{
    return (size_t)KQ_LIMBS * k + 2 * sizeof(float) * (size_t)(k / GROUP);
}

kqi::MatvecShape resolve_shape(int qtype, int64_t n_rows, int k)
{
    kqi::MatvecShape s = choose_shape(n_rows, 2 * (k >> 8), device_cus());
    const kqi::MatvecShape o = g_override[qtype];
    if (o.lanes) s.lanes = o.lanes;
    if (o.waves) s.waves = o.waves;
    if (o.grid) s.grid = o.grid;
    return s;
}

template <int LANES>
hipError_t launch_q4k_lanes(const uint8_t *W, const float *x, float *y, int n_rows, int k,
                            const float *gate, kqi::MatvecShape s, hipStream_t stream)
{
    const size_t lds = staging_bytes<32>(k);
    hipError_t e;
    if (gate) {
        constexpr auto kern = q4k_matvec_kernel<LANES, KQ_LIMBS, true>;
        if ((e = allow_lds<kern>(lds)) != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(s.grid), dim3(64 * s.waves), lds, stream, W, x, y, gate,
                           n_rows, k);
    } else {
        constexpr auto kern = q4k_matvec_kernel<LANES, KQ_LIMBS, false>;
        if ((e = allow_lds<kern>(lds)) != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(s.grid), dim3(64 * s.waves), lds, stream, W, x, y, gate,
                           n_rows, k);
    }
    return hipGetLastError();
}

template <int LANES>
hipError_t launch_q6k_lanes(const uint8_t *W, const float *x, float *y, int n_rows, int k,
                            kqi::MatvecShape s, hipStream_t stream)
{
    const size_t lds = staging_bytes<16>(k);
    constexpr auto kern = q6k_matvec_kernel<LANES, KQ_LIMBS>;
    hipError_t e = allow_lds<kern>(lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(s.grid), dim3(64 * s.waves), lds, stream, W, x, y, n_rows, k);
    return hipGetLastError();
}

}  // namespace

namespace kqi {

void set_shape_override(int qtype, MatvecShape s)
{
    if (qtype == 1 || qtype == 2) g_override[qtype] = s;
}

MatvecShape get_shape_override(int qtype)
{
    return (qtype == 1 || qtype == 2) ? g_override[qtype] : MatvecShape{0, 0, 0};
}

MatvecShape auto_shape(int qtype, int64_t n_rows, int64_t k, int m)
{
    (void)m;
    return resolve_shape(qtype, n_rows, (int)k);
}

hipError_t launch_matvec_q4k(const uint8_t *W, const float *x, float *y, int n_rows, int k,
                             const float *silu_gate, hipStream_t stream)
{
    const MatvecShape s = resolve_shape(1, n_rows, k);
    switch (s.lanes) {
    case 4: return launch_q4k_lanes<4>(W, x, y, n_rows, k, silu_gate, s, stream);
    case 8: return launch_q4k_lanes<8>(W, x, y, n_rows, k, silu_gate, s, stream);
    case 16: return launch_q4k_lanes<16>(W, x, y, n_rows, k, silu_gate, s, stream);
    case 32: return launch_q4k_lanes<32>(W, x, y, n_rows, k, silu_gate, s, stream);
    case 64: return launch_q4k_lanes<64>(W, x, y, n_rows, k, silu_gate, s, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_matvec_q6k(const uint8_t *W, const float *x, float *y, int n_rows, int k,
                             hipStream_t stream)
{
    const MatvecShape s = resolve_shape(2, n_rows, k);
    switch (s.lanes) {
    case 4: return launch_q6k_lanes<4>(W, x, y, n_rows, k, s, stream);
    case 8: return launch_q6k_lanes<8>(W, x, y, n_rows, k, s, stream);
    case 16: return launch_q6k_lanes<16>(W, x, y, n_rows, k, s, stream);
    case 32: return launch_q6k_lanes<32>(W, x, y, n_rows, k, s, stream);
    case 64: return launch_q6k_lanes<64>(W, x, y, n_rows, k, s, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_small_m(int qtype, const uint8_t *W, const float *X, int64_t ldx, float *Y,
                          int64_t ldy, int n_rows, int k, int m, hipStream_t stream)
{
    // One matvec per activation row.  Correct, but reads the weights m times;
    // the batched kernel replaces this path.
    for (int i = 0; i < m; ++i) {
        hipError_t e = (qtype == 1)
                           ? launch_matvec_q4k(W, X + i * ldx, Y + i * ldy, n_rows, k, nullptr,
                                               stream)
                           : launch_matvec_q6k(W, X + i * ldx, Y + i * ldy, n_rows, k, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_tail(float *residual, const float *projected, float *next_in,
                       const float *g_post, const float *g_next, int rows, int n,
                       float eps_post, float eps_next, hipStream_t stream)
{
    // about 4 float4 slots per thread, between 1 and 16 waves
    const int n4 = n >> 2;
    int threads = ((n4 + 4 * 64 - 1) / (4 * 64)) * 64;
    if (threads < 64) threads = 64;
    if (threads > 1024) threads = 1024;
    hipLaunchKernelGGL(tail_kernel, dim3(rows), dim3(threads), 0, stream, residual, projected,
                       next_in, g_post, g_next, n, eps_post, eps_next);
    return hipGetLastError();
}

const char *variant_names()
{
    return "q4k_matvec[lanes=4..64,limbs=3,silu=0/1,prefetch=1] q6k_matvec[lanes=4..64,limbs=3,prefetch=0] "
           "small_m[per-row matvec] tail[rows x (64..1024) threads, 3 passes]";
}

}  // namespace kqi

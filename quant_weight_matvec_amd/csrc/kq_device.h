// kq_device.h -- device-side building blocks shared by the kernel files of
// libkq: superblock unit loads and dot products, activation staging into LDS,
// fixed-order reductions.  See kq_kernels.hip for the design notes.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#define KQ_LIMBS 3

namespace kqd {


typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kQ4Bytes = 144;
constexpr int kQ6Bytes = 210;
constexpr int kQ5Bytes = 176;

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
// Reductions over aligned groups of 2, 4 or 8 consecutive lanes with DPP moves
// (VALU operations; no LDS round trip).  Steps: swap neighbours, swap pairs
// within a quad, then mirror within the 8-lane half row.  After step s every
// lane holds the reduction over its aligned 2^s-lane group, the same value in
// all of them (each step combines two group values that are uniform within
// their groups, and max and + are commutative).  Every lane of a group must be
// active.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror

template <int N>
__device__ __forceinline__ float group_max(float v)
{
    static_assert(N == 1 || N == 2 || N == 4 || N == 8, "group of 1, 2, 4 or 8 lanes");
    if constexpr (N >= 2) v = fmaxf(v, dpp_mov<kDppXor1>(v));
    if constexpr (N >= 4) v = fmaxf(v, dpp_mov<kDppXor2>(v));
    if constexpr (N >= 8) v = fmaxf(v, dpp_mov<kDppHalfMirror>(v));
    return v;
}

template <int N>
__device__ __forceinline__ float group_sum(float v)
{
    static_assert(N == 1 || N == 2 || N == 4 || N == 8, "group of 1, 2, 4 or 8 lanes");
    if constexpr (N >= 2) v = v + dpp_mov<kDppXor1>(v);
    if constexpr (N >= 4) v = v + dpp_mov<kDppXor2>(v);
    if constexpr (N >= 8) v = v + dpp_mov<kDppHalfMirror>(v);
    return v;
}

// ---------------------------------------------------------------------------
// Activation staging into LDS.
// Layout: LIMBS byte planes (plane 0 = most significant limb) of plane_bytes(k)
// bytes each, then k/GROUP f32 back-scale factors 2^(e - QB), then k/GROUP f32
// group sums.  A plane holds the inputs in order with 16 bytes of padding
// after every 128: the lanes of a row read units 128 inputs apart, which
// without the padding fall on the same LDS banks.
__host__ __device__ constexpr int64_t plane_bytes(int64_t k) { return k + (k >> 3); }

// Byte offset of input j within a plane.
__host__ __device__ constexpr int plane_off(int j) { return j + ((j >> 7) << 4); }

// Smallest group exponent: a group whose largest magnitude is below 2^kMinExp
// is encoded on the grid of 2^(kMinExp - QB) (absolute error at most
// 2^(kMinExp - QB - 1)) instead of its own, so its back-scale stays a normal
// float; with the group's own exponent it would underflow to zero below
// about 2^-127 and drop the group from the dot product.
constexpr int kMinExp = -100;

// Encodes float4 number i of a k-vector (n4 = k/4 float4) into the planes and
// the group tables.  Preconditions: the TPG = GROUP/4 consecutive lanes that
// hold one scale group all call it together with consecutive i (the group max
// and sum are DPP reductions over them), and 0 <= i < n4 for those lanes; a
// call with i >= n4 stores nothing (whole groups are either all in range or
// all out of it, since n4 is a multiple of TPG).  Per input the rounding error
// is at most 2^(e - QB - 1) <= 2^-QB * max|x over the group|, e the exponent
// with max|x| < 2^e.
// With AGENT the stores are agent-scope (coherent across the XCDs' L2s), for
// a staged vector that other workgroups of the same launch read.
template <int GROUP, int LIMBS, bool AGENT = false>
__device__ __forceinline__ void stage_group(f32x4 v, int i, uint32_t *__restrict__ plane, int n4,
                                            float *__restrict__ tscale, float *__restrict__ tsum)
{
    #pragma clang fp contract(off)
    constexpr int TPG = GROUP / 4;  // threads per group, one float4 each
    constexpr int QB = limb_bits<LIMBS>();
    const float mx = group_max<TPG>(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    const float sm = group_sum<TPG>((v.x + v.y) + (v.z + v.w));
    const int e = max(__builtin_amdgcn_frexp_expf(mx), kMinExp);  // mx < 2^e
    const int sh = QB - e;
    // q = x * 2^sh rounded to nearest even, |q| <= 2^QB.  Adding 1.5 * 2^23
    // rounds once and leaves q in the low mantissa bits of a float in
    // [2^23, 2^24], so the float's bit pattern minus 0x4B400000 is q.  The
    // same subtraction adds 0x80 to every limb byte: the bytes of
    // u = q + 0x80...80 are the balanced base-256 digits of q (each in
    // [-128, 127]) with their top bit flipped, carries included.
    constexpr uint32_t kOff = LIMBS == 3 ? 0x808080u : 0x8080u;
    constexpr uint32_t kBias = 0x4B400000u - kOff;
    const float magic = 12582912.0f;  // 1.5 * 2^23
    const uint32_t u0 = __builtin_bit_cast(uint32_t, ldexpf(v.x, sh) + magic) - kBias;
    const uint32_t u1 = __builtin_bit_cast(uint32_t, ldexpf(v.y, sh) + magic) - kBias;
    const uint32_t u2 = __builtin_bit_cast(uint32_t, ldexpf(v.z, sh) + magic) - kBias;
    const uint32_t u3 = __builtin_bit_cast(uint32_t, ldexpf(v.w, sh) + magic) - kBias;
    // byte transpose (v_perm_b32): plane word l holds limb l of the four
    // inputs, input j in byte j; then flip the top bits back
    const uint32_t lo01 = __builtin_amdgcn_perm(u1, u0, 0x05010400u);  // u0.b0 u1.b0 u0.b1 u1.b1
    const uint32_t lo23 = __builtin_amdgcn_perm(u3, u2, 0x05010400u);
    uint32_t pk[LIMBS];
    if constexpr (LIMBS == 3) {
        const uint32_t hi01 = __builtin_amdgcn_perm(u1, u0, 0x07030602u);  // u0.b2 u1.b2 - -
        const uint32_t hi23 = __builtin_amdgcn_perm(u3, u2, 0x07030602u);
        pk[0] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u) ^ 0x80808080u;
        pk[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u) ^ 0x80808080u;
        pk[2] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u) ^ 0x80808080u;
    } else {
        pk[0] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u) ^ 0x80808080u;
        pk[1] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u) ^ 0x80808080u;
    }
    // word i holds inputs 4i..4i+3; a plane is n4 + n4/8 words.  Past the end
    // (i >= n4) the word index would land in the next plane or, for the last
    // plane, in the scale and sum tables, so nothing is stored.
    if (i >= n4) return;
    const int pw = n4 + (n4 >> 3), wi = i + ((i >> 5) << 2);
    if constexpr (AGENT) {
#pragma unroll
        for (int l = 0; l < LIMBS; ++l)
            __hip_atomic_store(plane + l * pw + wi, pk[l], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((i & (TPG - 1)) == 0) {
            const int g = i / TPG;
            const float sc = isfinite(sm) ? ldexpf(1.0f, e - QB) : __builtin_nanf("");
            __hip_atomic_store(tscale + g, sc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(tsum + g, sm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    } else {
#pragma unroll
        for (int l = 0; l < LIMBS; ++l) plane[l * pw + wi] = pk[l];
        if ((i & (TPG - 1)) == 0) {
            const int g = i / TPG;
            tscale[g] = isfinite(sm) ? ldexpf(1.0f, e - QB) : __builtin_nanf("");
            tsum[g] = sm;
        }
    }
}

// Activation staging into LDS, in the layout above.
// The same bytes in global memory are a "staged" activation: a producer
// kernel that already holds the values writes them in this form once, and
// every consumer workgroup copies them into LDS instead of encoding x again.
template <int GROUP, int LIMBS>
__host__ __device__ constexpr int64_t staged_bytes(int64_t k)
{
    return LIMBS * plane_bytes(k) + 2 * 4 * (k / GROUP);
}

// A kernel issues the first B 16-byte pieces of each thread's share of its
// activation (float4 of x, or pieces of the staged form) before any weight
// load: vector loads of a wave complete in issue order, so the activation
// then arrives after one memory round trip instead of queueing behind the
// weights' look-ahead loads.  stage_activation encodes (or copies) the
// preloaded part and loads the rest in batches of four, each batch one round
// trip.
template <int B>
struct XPre {
    u32x4 v[B];
};

template <int B>
__device__ __forceinline__ XPre<B> x_preload(const void *__restrict__ src, int n16)
{
    XPre<B> p;
    const u32x4 *s4 = reinterpret_cast<const u32x4 *>(src);
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const int i = threadIdx.x + b * blockDim.x;
        if (i < n16) p.v[b] = s4[i];
    }
    return p;
}

// Number of 16-byte pieces x_preload reads: float4 of x, or pieces of xs.
template <int GROUP, int LIMBS>
__device__ __forceinline__ int x_pieces(const uint8_t *xs, int k)
{
    return xs ? (int)(staged_bytes<GROUP, LIMBS>(k) >> 4) : (k >> 2);
}

template <int GROUP, int LIMBS, int B>
__device__ __forceinline__ void stage_activation(const XPre<B> &pre, const float *__restrict__ x,
                                                 const uint8_t *__restrict__ xs, int k,
                                                 uint8_t *__restrict__ smem)
{
    constexpr int BR = 4;
    const int stride = blockDim.x;
    if (xs) {  // staged by the producer: a plain copy
        const int n16 = (int)(staged_bytes<GROUP, LIMBS>(k) >> 4);
        u32x4 *dst = reinterpret_cast<u32x4 *>(smem);
        const u32x4 *s4 = reinterpret_cast<const u32x4 *>(xs);
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const int i = threadIdx.x + b * stride;
            if (i < n16) dst[i] = pre.v[b];
        }
        for (int i0 = threadIdx.x + B * stride; i0 < n16; i0 += BR * stride) {
            u32x4 v[BR];
#pragma unroll
            for (int b = 0; b < BR; ++b) {
                const int i = i0 + b * stride;
                if (i < n16) v[b] = s4[i];
            }
#pragma unroll
            for (int b = 0; b < BR; ++b) {
                const int i = i0 + b * stride;
                if (i < n16) dst[i] = v[b];
            }
        }
        return;
    }
    const int n4 = k >> 2;  // a multiple of 64: whole waves stay active
    uint32_t *plane = reinterpret_cast<uint32_t *>(smem);
    float *tscale = reinterpret_cast<float *>(smem + LIMBS * plane_bytes(k));
    float *tsum = tscale + k / GROUP;
    const f32x4 *x4 = reinterpret_cast<const f32x4 *>(x);
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const int i = threadIdx.x + b * stride;
        if (i < n4)
            stage_group<GROUP, LIMBS>(__builtin_bit_cast(f32x4, pre.v[b]), i, plane, n4, tscale,
                                      tsum);
    }
    for (int i0 = threadIdx.x + B * stride; i0 < n4; i0 += BR * stride) {
        f32x4 v[BR];
#pragma unroll
        for (int b = 0; b < BR; ++b) {
            const int i = i0 + b * stride;
            if (i < n4) v[b] = x4[i];
        }
#pragma unroll
        for (int b = 0; b < BR; ++b) {
            const int i = i0 + b * stride;
            if (i < n4) stage_group<GROUP, LIMBS>(v[b], i, plane, n4, tscale, tsum);
        }
    }
}

// Staging of a plain x without a preload: loaded in batches of four float4.
template <int GROUP, int LIMBS>
__device__ __forceinline__ void stage_activation(const float *__restrict__ x, int k,
                                                 uint8_t *__restrict__ smem)
{
    stage_activation<GROUP, LIMBS, 4>(x_preload<4>(x, k >> 2), x, nullptr, k, smem);
}

// Writes the staged form of values the calling threads hold: thread t of a
// run of consecutive lanes holds float4 number i = i0 + t of the vector (k
// values), and whole scale groups of lanes take part.  Output layout as in
// LDS, at `out` in global memory.
template <int GROUP, int LIMBS, bool AGENT = false>
__device__ __forceinline__ void stage_group_global(f32x4 v, int i, uint8_t *__restrict__ out, int k)
{
    uint32_t *plane = reinterpret_cast<uint32_t *>(out);
    float *tscale = reinterpret_cast<float *>(out + LIMBS * plane_bytes(k));
    float *tsum = tscale + k / GROUP;
    stage_group<GROUP, LIMBS, AGENT>(v, i, plane, k >> 2, tscale, tsum);
}

template <int LIMBS>
__device__ __forceinline__ float combine_limbs(const int *acc)
{
    if constexpr (LIMBS == 3)  // (the product is exact: one rounding either way)
        return __builtin_fmaf((float)acc[0], 65536.0f, (float)(acc[1] * 256 + acc[2]));
    else
        return (float)(acc[0] * 256 + acc[1]);
}

// Sum over the LANES lanes that share a row (aligned groups): DPP for up to 8
// lanes, cross-lane shuffles for the wider steps.
template <int LANES>
__device__ __forceinline__ float lane_group_sum(float v)
{
    if constexpr (LANES <= 8) {
        return group_sum<LANES>(v);
    } else {
#pragma unroll
        for (int o = LANES / 2; o >= 8; o >>= 1) v += __shfl_xor(v, o);
        return group_sum<8>(v);
    }
}

// ---------------------------------------------------------------------------
// Up to kMaxSegs weight matrices of one type and k that share one activation
// vector, launched as one matvec (the pages' concurrent projection group,
// Ch 10 "The forward pass at a glance", section 10.3, box 4): their rows are
// numbered back to back, segment s holding rows [end[s-1], end[s]) of that
// numbering (end[-1] = 0), and row r of the numbering is row r - end[s-1] of
// matrix W[s], written to y[s].  Unused segments have end = INT_MAX.  Lanes
// pick their row's segment with selects (no indexed kernel-argument load).
constexpr int kMaxSegs = 4;
struct MatSegs {
    const uint8_t *W[kMaxSegs];
    float *y[kMaxSegs];
    int end[kMaxSegs];
};

__device__ __forceinline__ int seg_of(const MatSegs &m, int r)
{
    return (r >= m.end[0]) + (r >= m.end[1]) + (r >= m.end[2]);
}

__device__ __forceinline__ int seg_start(const MatSegs &m, int s)
{
    return s == 0 ? 0 : (s == 1 ? m.end[0] : (s == 2 ? m.end[1] : m.end[2]));
}

// First byte of row r (of the joint numbering) in its own matrix.
__device__ __forceinline__ const uint8_t *seg_row(const MatSegs &m, int r, int64_t row_bytes)
{
    const int s = seg_of(m, r);
    const uint8_t *w = s == 0 ? m.W[0] : (s == 1 ? m.W[1] : (s == 2 ? m.W[2] : m.W[3]));
    return w + (int64_t)(r - seg_start(m, s)) * row_bytes;
}

// Output element of row r (of the joint numbering).
__device__ __forceinline__ float *seg_out(const MatSegs &m, int r)
{
    const int s = seg_of(m, r);
    float *y = s == 0 ? m.y[0] : (s == 1 ? m.y[1] : (s == 2 ? m.y[2] : m.y[3]));
    return y + (r - seg_start(m, s));
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
    #pragma clang fp contract(off)
    // 6-bit scales and mins of sub-blocks 4h..4h+3, one per byte.
    const uint32_t S0 = u.hdr.y, S1 = u.hdr.z, S2 = u.hdr.w;
    // both halves' forms, then a per-lane select: a branch on h would split
    // the wave (neighbouring lanes take different halves)
    const uint32_t sc_lo = S0 & 0x3F3F3F3Fu, mn_lo = S1 & 0x3F3F3F3Fu;
    const uint32_t sc_hi = (S2 & 0x0F0F0F0Fu) | ((S0 >> 2) & 0x30303030u);
    const uint32_t mn_hi = ((S2 >> 4) & 0x0F0F0F0Fu) | ((S1 >> 2) & 0x30303030u);
    const uint32_t scb = h ? sc_hi : sc_lo;
    const uint32_t mnb = h ? mn_hi : mn_lo;
    const float d = half_lo(u.hdr.x), dmin = half_hi(u.hdr.x);

    int acc[4][LIMBS];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int l = 0; l < LIMBS; ++l) acc[s][l] = 0;
    // the unit's 128 inputs lie inside one padded 128-input run of each plane
    const int P = (int)plane_bytes(k);
    const uint8_t *xp = planes + (base >> 3);

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
            const u32x4 xl = *reinterpret_cast<const u32x4 *>(xp + l * P + plo);
            const u32x4 xh = *reinterpret_cast<const u32x4 *>(xp + l * P + plo + 32);
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
        // one fused multiply-add per sub-block (gs * v is exact: a power of
        // two times an integer), then a plain add: the rounding does not
        // depend on how the compiler contracts the expression
        out += __builtin_fmaf(d * sc, gs[s] * v, -((dmin * mn) * gm[s]));
    }
    return out;
}

// ---------------------------------------------------------------------------
// Q5_K unit = one half superblock (sub-blocks 4h..4h+3): the 16-byte header
// (d, dmin and the 6-bit scales and mins packed as in Q4_K), all 32 bytes of
// high bits (byte j holds the fifth bit of weight 64c + j in bit 2c and of
// weight 64c + 32 + j in bit 2c + 1), and the unit's 64 bytes of low nibbles
// (laid out as Q4_K's, at byte 48).  A 176-byte superblock keeps 16-byte
// alignment, so every load is a 16-byte vector load.
struct Q5Unit {
    u32x4 hdr;
    u32x4 qh[2];
    u32x4 q[4];
};

__device__ __forceinline__ Q5Unit q5_load(const uint8_t *__restrict__ sb, int h)
{
    Q5Unit u;
    u.hdr = *reinterpret_cast<const u32x4 *>(sb);
    u.qh[0] = *reinterpret_cast<const u32x4 *>(sb + 16);
    u.qh[1] = *reinterpret_cast<const u32x4 *>(sb + 32);
    const u32x4 *p = reinterpret_cast<const u32x4 *>(sb + 48 + 64 * h);
    u.q[0] = p[0];
    u.q[1] = p[1];
    u.q[2] = p[2];
    u.q[3] = p[3];
    return u;
}

// Contribution of one Q5_K unit; as q4_unit_dot with each quant byte
// completed by its fifth bit (values 0..31, still a signed byte operand).
template <int LIMBS>
__device__ __forceinline__ float q5_unit_dot(const Q5Unit &u, int h, int base, int k,
                                             const uint8_t *__restrict__ planes,
                                             const float *__restrict__ tscale,
                                             const float *__restrict__ tsum)
{
    #pragma clang fp contract(off)
    const uint32_t S0 = u.hdr.y, S1 = u.hdr.z, S2 = u.hdr.w;
    const uint32_t sc_lo = S0 & 0x3F3F3F3Fu, mn_lo = S1 & 0x3F3F3F3Fu;
    const uint32_t sc_hi = (S2 & 0x0F0F0F0Fu) | ((S0 >> 2) & 0x30303030u);
    const uint32_t mn_hi = ((S2 >> 4) & 0x0F0F0F0Fu) | ((S1 >> 2) & 0x30303030u);
    const uint32_t scb = h ? sc_hi : sc_lo;
    const uint32_t mnb = h ? mn_hi : mn_lo;
    const float d = half_lo(u.hdr.x), dmin = half_hi(u.hdr.x);

    int acc[4][LIMBS];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int l = 0; l < LIMBS; ++l) acc[s][l] = 0;
    const int P = (int)plane_bytes(k);
    const uint8_t *xp = planes + (base >> 3);

#pragma unroll
    for (int p = 0; p < 4; ++p) {
        // 16 bytes = inputs j0..j0+15 of sub-block 2c (low nibbles, fifth bit
        // 2c) and of sub-block 2c+1 (high nibbles, bit 2c+1), c = 2h + p/2,
        // j0 = 16 (p & 1); the fifth bits sit in high-bit bytes j0..j0+15.
        const int plo = base + 64 * (p >> 1) + 16 * (p & 1);
        const int slo = 2 * (p >> 1);
        const int sh = 4 * h + 2 * (p >> 1);  // bit 2c of each high-bit byte
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t qh = u.qh[p & 1][w] >> sh;
            lo[w] = (u.q[p][w] & 0x0F0F0F0Fu) | ((qh << 4) & 0x10101010u);
            hi[w] = ((u.q[p][w] >> 4) & 0x0F0F0F0Fu) | ((qh << 3) & 0x10101010u);
        }
#pragma unroll
        for (int l = 0; l < LIMBS; ++l) {
            const u32x4 xl = *reinterpret_cast<const u32x4 *>(xp + l * P + plo);
            const u32x4 xh = *reinterpret_cast<const u32x4 *>(xp + l * P + plo + 32);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                acc[slo][l] = sdot4(lo[w], xl[w], acc[slo][l]);
                acc[slo + 1][l] = sdot4(hi[w], xh[w], acc[slo + 1][l]);
            }
        }
    }

    const int g0 = base >> 5;
    const f32x4 gs = *reinterpret_cast<const f32x4 *>(tscale + g0);
    const f32x4 gm = *reinterpret_cast<const f32x4 *>(tsum + g0);
    float out = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const float sc = (float)((scb >> (8 * s)) & 0xFFu);
        const float mn = (float)((mnb >> (8 * s)) & 0xFFu);
        const float v = combine_limbs<LIMBS>(acc[s]);
        // one fused multiply-add per sub-block (gs * v is exact: a power of
        // two times an integer), then a plain add: the rounding does not
        // depend on how the compiler contracts the expression
        out += __builtin_fmaf(d * sc, gs[s] * v, -((dmin * mn) * gm[s]));
    }
    return out;
}

// The superblock format of a Q4_K-style matvec: 4 = Q4_K, 5 = Q5_K.
template <int FMT> struct KFmt;
template <> struct KFmt<4> {
    using Unit = Q4Unit;
    static constexpr int kBytes = kQ4Bytes;
    static __device__ __forceinline__ Unit load(const uint8_t *sb, int h) { return q4_load(sb, h); }
    template <int LIMBS>
    static __device__ __forceinline__ float dot(const Unit &u, int h, int base, int k,
                                                const uint8_t *planes, const float *tscale,
                                                const float *tsum)
    {
        return q4_unit_dot<LIMBS>(u, h, base, k, planes, tscale, tsum);
    }
};
template <> struct KFmt<5> {
    using Unit = Q5Unit;
    static constexpr int kBytes = kQ5Bytes;
    static __device__ __forceinline__ Unit load(const uint8_t *sb, int h) { return q5_load(sb, h); }
    template <int LIMBS>
    static __device__ __forceinline__ float dot(const Unit &u, int h, int base, int k,
                                                const uint8_t *planes, const float *tscale,
                                                const float *tsum)
    {
        return q5_unit_dot<LIMBS>(u, h, base, k, planes, tscale, tsum);
    }
};

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
    // third word only needed when shifted; otherwise re-read the second, so
    // the load stays inside the superblock and is not a branch
    u.sc[2] = ps[shift ? 2 : 1];
    u.d = *reinterpret_cast<const uint16_t *>(sb + 208);
    return u;
}

__device__ __forceinline__ uint32_t realign(uint32_t hi, uint32_t lo, int shift)
{
    return __builtin_amdgcn_alignbyte(hi, lo, (uint32_t)shift);
}

// SPLIT keeps the two halves of the unit apart in the schedule (the second
// half's LDS reads are not hoisted into the first), for kernels that cannot
// give the dot product the registers of both halves at once.
template <int LIMBS, bool SPLIT = false>
__device__ __forceinline__ float q6_unit_dot(const Q6Unit &u, int base, int k,
                                             const uint8_t *__restrict__ planes,
                                             const float *__restrict__ tscale,
                                             const float *__restrict__ tsum)
{
    #pragma clang fp contract(off)
    const int sh = u.shift;
    // the unit's 128 inputs lie inside one padded 128-input run of each plane
    const int P = (int)plane_bytes(k);
    const uint8_t *xp = planes + (base >> 3);
    // ql word i (i = 0..15) and qh word i (i = 0..7) of the unit, re-aligned
    // on use so that only the words of one half are live at a time
    auto qlw = [&](int i) -> uint32_t {
        const uint32_t lo = u.ql[i >> 2][i & 3];
        const uint32_t hi = i == 15 ? u.ql_x : u.ql[(i + 1) >> 2][(i + 1) & 3];
        return realign(hi, lo, sh);
    };
    auto qhw = [&](int i) -> uint32_t {
        const uint32_t lo = u.qh[i >> 2][i & 3];
        const uint32_t hi = i == 7 ? u.qh_x : u.qh[(i + 1) >> 2][(i + 1) & 3];
        return realign(hi, lo, sh);
    };
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
        if constexpr (SPLIT) __builtin_amdgcn_sched_barrier(0);
        int acc[4][LIMBS];
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int l = 0; l < LIMBS; ++l) acc[g][l] = 0;
        uint32_t q[4][4];  // [g][t]: quants of inputs base + 32g + 16jj + 4t .. +3
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t l0 = qlw(4 * jj + t), l1 = qlw(8 + 4 * jj + t), hh = qhw(4 * jj + t);
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
                const u32x4 xv = *reinterpret_cast<const u32x4 *>(xp + l * P + pos);
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
            // written as fused multiply-adds (gsc * v is exact, a power of
            // two times an integer), so that the rounding does not depend on
            // how the compiler schedules or contracts the expression
            out = __builtin_fmaf(d * (float)scv, __builtin_fmaf(gsc, v, -32.0f * gsum), out);
        }
    }
    return out;
}


typedef __attribute__((address_space(3))) void lds_void;

// LDS byte address of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(lds_void *)p;
}

// One direct-to-LDS 16-byte load per lane: lane i's 16 bytes from `src` land
// at LDS byte lds + 16 i.  Written as inline assembly on purpose: the compiler
// then does not track these loads as LDS writes, so it does not drain every
// load in flight at each workgroup barrier; the kernel waits for exactly the
// chunk it needs (s_waitcnt vmcnt) before the barrier that publishes it.  The
// compiler's own counter waits can only become more conservative.
__device__ __forceinline__ void lds_dma16(const void *src, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(lds)
                 : "memory");
}

// Sum over the workgroup in a fixed order (lanes, then waves in order); every
// thread returns the same value.  `red` holds one float per wave and is read
// by all threads at the end; block_sum_fresh is for a buffer no thread can
// still be reading (one not used before in the kernel), block_sum_fixed waits
// for earlier readers first.
__device__ __forceinline__ float block_sum_fresh(float v, float *red)
{
    v = group_sum<8>(v);
#pragma unroll
    for (int o = 32; o >= 8; o >>= 1) v += __shfl_xor(v, o);
    const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    float t = 0.0f;
    for (int w = 0; w < nw; ++w) t += red[w];
    return t;
}

__device__ __forceinline__ float block_sum_fixed(float v, float *red)
{
    __syncthreads();  // `red` may still be read from the previous reduction
    return block_sum_fresh(v, red);
}

// The tail's floating-point steps are written as explicit fused
// multiply-adds, with contraction off inside the helpers (as in the dot
// products and the encode), so that every kernel that runs a tail
// (standalone, fused into gate+up, or inside the one-launch pass) rounds the
// same way: a product a helper returns is rounded before any caller adds it
// (the compiler would otherwise fuse it into the caller's next addition where
// it has no other use, and not where it does).
__device__ __forceinline__ float sumsq4(f32x4 v)
{
    #pragma clang fp contract(off)
    return __builtin_fmaf(v.w, v.w, __builtin_fmaf(v.z, v.z, __builtin_fmaf(v.x, v.x, v.y * v.y)));
}

// ---------------------------------------------------------------------------
// The dual-eps tail in registers: up to kTailVec float4 per thread, whole
// waves, rows up to kTailRegMax wide.  tail_threads(n) is the block size of
// the standalone tail; the fused form (q4k_gate_up_kernel with TAIL) lays its
// threads out the same way so that both sum in the same order.  Beyond four
// waves the count is rounded up to a multiple of four, so each of a CU's four
// SIMDs runs the same number of tail waves (the encode at the end is VALU
// work, and the workgroup waits for its busiest SIMD).
constexpr int kTailVec = 4;
constexpr int kTailThreads = 512;
constexpr int kTailRegMax = 4 * kTailVec * kTailThreads;  // 8192

__host__ __device__ constexpr int tail_threads(int n)
{
    const int w = ((n >> 2) + kTailVec * 64 - 1) / (kTailVec * 64);  // waves needed
    return 64 * (w <= 1 ? 1 : (w <= 4 ? w : (w + 3) / 4 * 4));
}

// r + rms-normed p times the post gain, and the next input, one float4 each
__device__ __forceinline__ f32x4 tail_add(f32x4 r, f32x4 p, float inv_p, f32x4 g)
{
    #pragma clang fp contract(off)
    const f32x4 q = p * inv_p;
    return {__builtin_fmaf(q.x, g.x, r.x), __builtin_fmaf(q.y, g.y, r.y),
            __builtin_fmaf(q.z, g.z, r.z), __builtin_fmaf(q.w, g.w, r.w)};
}

__device__ __forceinline__ f32x4 tail_next(f32x4 r, float inv_r, f32x4 g)
{
    #pragma clang fp contract(off)
    return (r * inv_r) * g;
}

}  // namespace kqd

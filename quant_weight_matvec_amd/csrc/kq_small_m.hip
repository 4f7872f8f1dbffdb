// kq_small_m.hip -- Y[m] = W X[m] for up to 16 activation rows over Q4_K /
// Q6_K weights (the pages' verify / small-batch case: Ch 36 "Speculative
// decoding", section 36.4, where one read of each weight row serves every
// verified position; the M = 16 timings of Ch 19, section 19.4).
//
// Design for gfx950 (the pages' kernels use scalar f32 MACs on another GPU):
//
// * Matrix cores.  One 64-lane wave owns a tile of 16 weight rows.  For every
//   scale sub-block it issues f16 MFMAs D[16 x 16] += A[16 x K'] B[K' x 16]
//   with A = the (up to 16) activation rows and B = the sub-block's quants:
//   Q4_K uses 16x16x32 (one 32-weight sub-block), Q6_K 16x16x16 (one
//   16-weight sub-block).  Lane l holds output column l % 16 = its weight row,
//   so the per-row scale d*sc (and the Q4_K min term) is applied in registers
//   right after the MFMA.
// * Exact quant operands.  A quant q is turned into the f16 value 1024 + q by
//   OR-ing it under the exponent of 1024 (0x6400), then 1024 (Q4_K) or 1056
//   (Q6_K, folding the -32 offset) is subtracted: both steps are exact, so B
//   holds the integers q or q - 32 exactly.
// * Activations at ~22 bits.  Each (row m, superblock) group of 256 inputs is
//   scaled by a power of two so that its largest magnitude is below 2^15, then
//   split into x_hi = f16(x) and x_lo = f16(x - x_hi); two MFMAs (hi, lo) per
//   sub-block accumulate in f32.  The products q * x_hi and q * x_lo are exact
//   in f32.  The Q4_K min term uses the f32 group sums of the scaled inputs.
//   A group holding a NaN or an infinity is staged as NaN, so the whole output
//   row m becomes NaN.
// * Stream-K split.  The work is the grid of (row group of 128 rows, superblock)
//   tiles; workgroup g takes the contiguous range [g T / G, (g+1) T / G).  A row
//   group covered by one workgroup is stored directly.  Otherwise each
//   contributing workgroup stores its partial tile in the workspace and counts
//   itself in with an agent-scope atomic; the last to arrive sums the partials
//   in workgroup order (deterministic for a given grid) and resets the counter.
//   Nothing ever waits on another workgroup, so a launch always terminates.
// * Activation staging.  The inputs of the superblocks a workgroup is about to
//   use are staged in chunks into LDS (hi and lo planes, each 4-group of
//   inputs stored in the order 0,2,1,3 to match how the quant bytes unpack into
//   f16 pairs).  The weight loads of the next tiles are issued before a chunk
//   is staged, so HBM keeps streaming.

#include <hip/hip_runtime.h>
#include <float.h>
#include <math.h>
#include <stdint.h>

#include "kq_device.h"
#include "kq_internal.h"

namespace {

using namespace kqd;

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kSmWaves = 8;
constexpr int kSmThreads = 64 * kSmWaves;
constexpr int kSmRows = 16 * kSmWaves;  // rows per row group
constexpr uint32_t kBias = 0x64006400u;  // f16 1024.0 in both halves
constexpr int kSmLdsMax = 160 * 1024;

struct SmArgs {
    const uint8_t *W;
    const float *X;
    float *Y;
    uint8_t *ws;        // workspace: counters, then partial tiles
    int64_t ldx, ldy;
    int n_rows, k, m;
    int nb;             // superblocks per row
    int T, G;           // tiles, workgroups
    int CH;             // superblocks per staged chunk
    int RS;             // bytes per activation row in one LDS plane
    int part_off;       // byte offset of the partial tiles in the workspace
    int ws_bytes;
    int flag_off;       // LDS byte offset of the last-arrival flag
};

__device__ __forceinline__ int first_tile(int g, int T, int G)
{
    return (int)(((int64_t)g * T) / G);
}

// the workgroup whose range holds tile t
__device__ __forceinline__ int owner(int t, int T, int G)
{
    return (int)((((int64_t)t + 1) * G - 1) / T);
}

__device__ __forceinline__ void st_agent(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void st_agent(uint32_t *p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Per-lane weight data of one superblock of the lane's row.
// Lane l: kb = l >> 4 selects which quarter of every sub-block the lane
// supplies, r = l & 15 the row of the tile.

struct Q4Sb {
    u32x4 hdr;      // d, dmin, 12 bytes of packed 6-bit scales and mins
    uint32_t q[8];  // chunk c: bytes 16 + 32c + 8kb .. +7 as q[2c], q[2c+1]
};

__device__ __forceinline__ Q4Sb load_sb(const uint8_t *__restrict__ sb, int kb, Q4Sb *)
{
    Q4Sb u;
    u.hdr = *reinterpret_cast<const u32x4 *>(sb);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const u32x2 v = *reinterpret_cast<const u32x2 *>(sb + 16 + 32 * c + 8 * kb);
        u.q[2 * c] = v.x;
        u.q[2 * c + 1] = v.y;
    }
    return u;
}

// Q6_K: a superblock starts 2-byte aligned when its global index is odd.  Each
// needed dword is read as an 8-byte window starting at the 4-byte aligned
// address at or below it and re-aligned in registers; every window stays in
// [sb - 2, sb + 210) and sb - 2 is only used when sb is not the first byte of W.
struct Q6Sb {
    uint32_t w[24];  // ql windows u = 0..7 (w[2u], w[2u+1]); qh windows v = 0..3 (w[16+2v], ..)
    u32x4 hs;        // scale bytes, aligned window
    uint32_t tail;   // shift 2: scales 14, 15 and d; shift 0: d
};

__device__ __forceinline__ Q6Sb load_sb(const uint8_t *__restrict__ sb, int kb, Q6Sb *)
{
    Q6Sb u;
    const int sh = (int)((uintptr_t)sb & 3u);
    const uint8_t *a = sb - sh;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const u32x2_a4 v = *reinterpret_cast<const u32x2_a4 *>(a + 16 * i + 4 * kb);
        u.w[2 * i] = v.x;
        u.w[2 * i + 1] = v.y;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u32x2_a4 v = *reinterpret_cast<const u32x2_a4 *>(a + 128 + 16 * i + 4 * kb);
        u.w[16 + 2 * i] = v.x;
        u.w[17 + 2 * i] = v.y;
    }
    u.hs = *reinterpret_cast<const u32x4_a4 *>(a + 192);
    u.tail = sh ? *reinterpret_cast<const uint32_t *>(a + 208)
                : (uint32_t) * reinterpret_cast<const uint16_t *>(a + 208);
    return u;
}

__device__ __forceinline__ h8 as_h8(u32x4 v) { return __builtin_bit_cast(h8, v); }
__device__ __forceinline__ h4 as_h4(u32x2 v) { return __builtin_bit_cast(h4, v); }

// f16 pairs (1024 + byte0 nibble, 1024 + byte2 nibble) etc. from one dword of
// packed nibbles; `s` selects the nibble (0 low, 4 high) and byte pair (0 or 8).
__device__ __forceinline__ uint32_t nib_pair(uint32_t w, int s)
{
    return ((w >> s) & 0x000F000Fu) | kBias;
}

// Contribution of one Q4_K superblock to the lane's 4 outputs, in units of the
// staged (scaled) activations.  `ah` points at the lane's activation row in the
// hi plane at this superblock's first input + 8 kb; the lo plane is `lo_off`
// bytes further.  `st` = group sums of the superblock at [s][m0..m0+3].
__device__ __forceinline__ f32x4 sb_mma(const Q4Sb &u, const uint8_t *__restrict__ ah,
                                        int lo_off, const float *__restrict__ st)
{
    const uint32_t S0 = u.hdr.y, S1 = u.hdr.z, S2 = u.hdr.w;
    const uint32_t scA = S0 & 0x3F3F3F3Fu, mnA = S1 & 0x3F3F3F3Fu;
    const uint32_t scB = (S2 & 0x0F0F0F0Fu) | ((S0 >> 2) & 0x30303030u);
    const uint32_t mnB = ((S2 >> 4) & 0x0F0F0F0Fu) | ((S1 >> 2) & 0x30303030u);
    const float d = half_lo(u.hdr.x), dmin = half_hi(u.hdr.x);
    const h8 off = {1024, 1024, 1024, 1024, 1024, 1024, 1024, 1024};
    f32x4 ys = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint32_t w0 = u.q[2 * c], w1 = u.q[2 * c + 1];
#pragma unroll
        for (int hn = 0; hn < 2; ++hn) {  // hn 0: low nibbles (sub-block 2c), 1: high (2c+1)
            const int s = 2 * c + hn;
            const u32x4 bq = {nib_pair(w0, 4 * hn), nib_pair(w0, 4 * hn + 8), nib_pair(w1, 4 * hn),
                              nib_pair(w1, 4 * hn + 8)};
            const h8 B = as_h8(bq) - off;
            const h8 Ahi = *reinterpret_cast<const h8 *>(ah + 64 * s);
            const h8 Alo = *reinterpret_cast<const h8 *>(ah + lo_off + 64 * s);
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ahi, B, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Alo, B, acc, 0, 0, 0);
            const uint32_t scw = s < 4 ? scA : scB, mnw = s < 4 ? mnA : mnB;
            const float c1 = d * (float)((scw >> (8 * (s & 3))) & 0xFFu);
            const float c2 = dmin * (float)((mnw >> (8 * (s & 3))) & 0xFFu);
            const f32x4 sm = *reinterpret_cast<const f32x4 *>(st + 16 * s);
            ys += c1 * acc - c2 * sm;
        }
    }
    return ys;
}

// One Q6_K superblock; `ah` = the lane's activation row at the superblock's
// first input + 4 kb.
__device__ __forceinline__ f32x4 sb_mma(const Q6Sb &u, const uint8_t *__restrict__ ah,
                                        int lo_off, const float *__restrict__, int sh)
{
    uint32_t L[8], H[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) L[i] = __builtin_amdgcn_alignbyte(u.w[2 * i + 1], u.w[2 * i], sh);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        H[i] = __builtin_amdgcn_alignbyte(u.w[17 + 2 * i], u.w[16 + 2 * i], sh);
    uint32_t sc[4];
    sc[0] = __builtin_amdgcn_alignbyte(u.hs.y, u.hs.x, sh);
    sc[1] = __builtin_amdgcn_alignbyte(u.hs.z, u.hs.y, sh);
    sc[2] = __builtin_amdgcn_alignbyte(u.hs.w, u.hs.z, sh);
    sc[3] = __builtin_amdgcn_alignbyte(u.tail, u.hs.w, sh);
    const float d = half_lo(sh ? (u.tail >> 16) : u.tail);
    const h4 off = {1056, 1056, 1056, 1056};
    f32x4 ys = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 16; ++s) {
        const int h = s >> 3, g = (s >> 1) & 3, hf = s & 1;
        const uint32_t l = L[4 * h + 2 * (g & 1) + hf], hh = H[2 * h + hf];
        const uint32_t lo4 = (g < 2 ? l : (l >> 4)) & 0x0F0F0F0Fu;
        const uint32_t q = lo4 | (((hh >> (2 * g)) & 0x03030303u) << 4);
        const u32x2 bq = {(q & 0x00FF00FFu) | kBias, ((q >> 8) & 0x00FF00FFu) | kBias};
        const h4 B = as_h4(bq) - off;
        const h4 Ahi = *reinterpret_cast<const h4 *>(ah + 32 * s);
        const h4 Alo = *reinterpret_cast<const h4 *>(ah + lo_off + 32 * s);
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        acc = __builtin_amdgcn_mfma_f32_16x16x16f16(Ahi, B, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x16f16(Alo, B, acc, 0, 0, 0);
        const int scv = ((int)(sc[s >> 2] << (24 - 8 * (s & 3)))) >> 24;
        ys += (d * (float)scv) * acc;
    }
    return ys;
}

template <typename U>
__device__ __forceinline__ constexpr bool is_q4()
{
    return sizeof(U) == sizeof(Q4Sb);
}

// ---------------------------------------------------------------------------
// Staging of the activations of superblocks [cb, cb + n) into LDS.
// LDS: hi plane [M][RS bytes], lo plane [M][RS bytes], etab [CH][16] int
// (back-scale exponents), stab [CH][8][16] f32 (Q4_K: sums of 32-input groups,
// scaled).  One wave converts one (row, superblock) group of 256 inputs.
template <bool Q4>
__device__ __forceinline__ void stage_chunk(const SmArgs &a, int cb, int n, uint8_t *smem)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int M = a.m, RS = a.RS;
    uint8_t *hi = smem, *lo = smem + M * RS;
    int *etab = reinterpret_cast<int *>(smem + 2 * M * RS);
    float *stab = reinterpret_cast<float *>(etab + 16 * a.CH);
    const int ngroups = M * n;
    constexpr int B = 4;
    for (int g0 = wave; g0 < ngroups; g0 += B * kSmWaves) {
        f32x4 v[B];
#pragma unroll
        for (int j = 0; j < B; ++j) {
            const int gi = g0 + j * kSmWaves;
            if (gi < ngroups) {
                const int m = gi / n, bb = gi - m * n;
                v[j] = *reinterpret_cast<const f32x4 *>(a.X + (int64_t)m * a.ldx +
                                                        256 * (int64_t)(cb + bb) + 4 * lane);
            }
        }
#pragma unroll
        for (int j = 0; j < B; ++j) {
            const int gi = g0 + j * kSmWaves;
            if (gi >= ngroups) break;  // wave-uniform
            const int m = gi / n, bb = gi - m * n;
            float mx = fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)), fmaxf(fabsf(v[j].z), fabsf(v[j].w)));
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
            const bool fin = mx <= FLT_MAX;  // false for Inf and NaN
            const int e = __builtin_amdgcn_frexp_expf(mx);  // mx < 2^e
            const int sh = 15 - e;
            const f32x4 s = {ldexpf(v[j].x, sh), ldexpf(v[j].y, sh), ldexpf(v[j].z, sh),
                             ldexpf(v[j].w, sh)};
            _Float16 h[4], l[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                h[i] = (_Float16)s[i];
                l[i] = (_Float16)(s[i] - (float)h[i]);
                if (!fin) {
                    h[i] = (_Float16)__builtin_nanf("");
                    l[i] = h[i];
                }
            }
            // inputs 4 lane .. 4 lane + 3 stored in the order 0, 2, 1, 3
            const int boff = m * RS + 2 * (256 * bb + 4 * lane);
            const u32x2 ph = {__builtin_bit_cast(uint32_t, (h4){h[0], h[2], h[1], h[3]}.xy),
                              __builtin_bit_cast(uint32_t, (h4){h[0], h[2], h[1], h[3]}.zw)};
            const u32x2 pl = {__builtin_bit_cast(uint32_t, (h4){l[0], l[2], l[1], l[3]}.xy),
                              __builtin_bit_cast(uint32_t, (h4){l[0], l[2], l[1], l[3]}.zw)};
            *reinterpret_cast<u32x2 *>(hi + boff) = ph;
            *reinterpret_cast<u32x2 *>(lo + boff) = pl;
            if (lane == 0) etab[16 * bb + m] = e - 15;
            if constexpr (Q4) {
                float sm = (s.x + s.y) + (s.z + s.w);
#pragma unroll
                for (int o = 1; o < 8; o <<= 1) sm += __shfl_xor(sm, o);
                if ((lane & 7) == 0) stab[128 * bb + 16 * (lane >> 3) + m] = fin ? sm : __builtin_nanf("");
            }
        }
    }
}

template <typename U, int DEPTH>
__global__ void __launch_bounds__(kSmThreads) small_m_kernel(SmArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr bool Q4 = is_q4<U>();
    constexpr int BLK = Q4 ? kQ4Bytes : kQ6Bytes;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kb = lane >> 4, r = lane & 15, m0 = 4 * kb;
    const int g = blockIdx.x, nb = a.nb, M = a.m;
    const int t0 = first_tile(g, a.T, a.G), t1 = first_tile(g + 1, a.T, a.G);
    const int64_t row_bytes = (int64_t)nb * BLK;
    const int ma = min(r, M - 1);  // activation row this lane feeds into A
    const int lo_off = M * a.RS;
    const int *etab = reinterpret_cast<const int *>(smem + 2 * M * a.RS);
    const float *stab = reinterpret_cast<const float *>(etab + 16 * a.CH);
    int &last_flag = *reinterpret_cast<int *>(smem + a.flag_off);

    auto tile_ptr = [&](int t) {
        const int rg = t / nb, b = t - rg * nb;
        const int row = min(rg * kSmRows + 16 * wave + r, a.n_rows - 1);
        return a.W + row * row_bytes + (int64_t)b * BLK;
    };

    U ring[DEPTH];
#pragma unroll
    for (int i = 0; i < DEPTH; ++i)
        if (t0 + i < t1) ring[i] = load_sb(tile_ptr(t0 + i), kb, (U *)nullptr);

    int t = t0;
    while (t < t1) {
        const int rg = t / nb, bs = t - rg * nb;
        const int be = min(nb, bs + (t1 - t));
        f32x4 yacc = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int cb = bs; cb < be; cb += a.CH) {
            const int n = min(a.CH, be - cb);
            __syncthreads();  // the previous chunk's LDS reads are done
            stage_chunk<Q4>(a, cb, n, smem);
            __syncthreads();
            for (int bb = 0; bb < n; ++bb, ++t) {
                const U cur = ring[0];
#pragma unroll
                for (int i = 0; i + 1 < DEPTH; ++i) ring[i] = ring[i + 1];
                if (t + DEPTH < t1) ring[DEPTH - 1] = load_sb(tile_ptr(t + DEPTH), kb, (U *)nullptr);
                const uint8_t *ah = smem + ma * a.RS + 2 * (256 * bb + (Q4 ? 8 : 4) * kb);
                f32x4 ys;
                if constexpr (Q4)
                    ys = sb_mma(cur, ah, lo_off, stab + 128 * bb + m0);
                else
                    ys = sb_mma(cur, ah, lo_off, nullptr,
                                (int)((uintptr_t)tile_ptr(t) & 3u));
                const i32x4 ex = *reinterpret_cast<const i32x4 *>(etab + 16 * bb + m0);
#pragma unroll
                for (int i = 0; i < 4; ++i) yacc[i] += ldexpf(ys[i], ex[i]);
            }
        }

        // ---- this workgroup's share of row group rg is complete
        const int gl = owner(rg * nb, a.T, a.G), gh = owner(rg * nb + nb - 1, a.T, a.G);
        const int row0 = rg * kSmRows;
        if (gl == gh) {
            const int row = row0 + 16 * wave + r;
            if (row < a.n_rows) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (m0 + i < M) a.Y[(int64_t)(m0 + i) * a.ldy + row] = yacc[i];
            }
            continue;
        }
        float *part = reinterpret_cast<float *>(a.ws + a.part_off);
        uint32_t *cnt = reinterpret_cast<uint32_t *>(a.ws);
        const int slot = (first_tile(g, a.T, a.G) / nb == rg) ? 0 : 1;
        float *pp = part + (int64_t)(2 * g + slot) * (16 * kSmRows);
#pragma unroll
        for (int i = 0; i < 4; ++i) st_agent(pp + (m0 + i) * kSmRows + 16 * wave + r, yacc[i]);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // this wave's stores have completed
        __syncthreads();
        if (threadIdx.x == 0) {
            const uint32_t old = __hip_atomic_fetch_add(cnt + rg, 1u, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
            last_flag = (old + 1 == (uint32_t)(gh - gl + 1));
        }
        __syncthreads();
        if (last_flag) {
            // sum the contributors' partial tiles in workgroup order
            const __amdgpu_buffer_rsrc_t rs =
                __builtin_amdgcn_make_buffer_rsrc(a.ws, (short)0, a.ws_bytes, 0x00020000);
            for (int e = threadIdx.x; e < M * (kSmRows / 4); e += kSmThreads) {
                const int m = e / (kSmRows / 4), q = e - m * (kSmRows / 4);
                f32x4 s;
                for (int c = gl; c <= gh; ++c) {
                    const int sl = (first_tile(c, a.T, a.G) / nb == rg) ? 0 : 1;
                    const uint32_t off = (uint32_t)a.part_off +
                                         4u * (uint32_t)((2 * c + sl) * (16 * kSmRows) +
                                                         m * kSmRows + 4 * q);
                    const f32x4 v = __builtin_bit_cast(
                        f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 16 /* sc1 */));
                    s = (c == gl) ? v : s + v;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = row0 + 4 * q + i;
                    if (row < a.n_rows) a.Y[(int64_t)m * a.ldy + row] = s[i];
                }
            }
            if (threadIdx.x == 0) st_agent(cnt + rg, 0u);
        }
    }
}

struct SmPlan {
    int nb, T, G, CH, RS, part_off, flag_off;
    size_t lds, ws;
};

int sm_cus()
{
    static int cached = 0;
    if (!cached) {
        int dev = 0, c = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            c > 0)
            cached = c;
        else
            cached = 256;
    }
    return cached;
}

SmPlan make_plan(int qtype, int n_rows, int k, int m)
{
    SmPlan p;
    p.nb = k / 256;
    const int rgs = (n_rows + kSmRows - 1) / kSmRows;
    p.T = rgs * p.nb;
    p.G = p.T < sm_cus() ? p.T : sm_cus();
    const int per_sb = 1024 * m + 64 + (qtype == 1 ? 512 : 0);  // LDS bytes per staged superblock
    int ch = (kSmLdsMax - 16 - 32 * m) / per_sb;
    const int seg = (p.T + p.G - 1) / p.G;  // longest range of a workgroup
    if (ch > seg) ch = seg;
    if (ch > p.nb) ch = p.nb;
    if (ch < 1) ch = 1;
    p.CH = ch;
    p.RS = 512 * ch + 16;
    p.flag_off = 2 * m * p.RS + 64 * ch + (qtype == 1 ? 512 * ch : 0);
    p.lds = (size_t)p.flag_off + 16;
    // workspace: one counter per row group, then two partial tiles per workgroup
    p.part_off = ((rgs * 4 + 255) / 256) * 256;
    bool split = false;
    for (int rg = 0; rg < rgs && !split; ++rg) {
        const int64_t a = (int64_t)rg * p.nb, b = a + p.nb - 1;
        split = ((a + 1) * p.G - 1) / p.T != ((b + 1) * p.G - 1) / p.T;
    }
    p.ws = split ? (size_t)p.part_off + (size_t)p.G * 2 * 16 * kSmRows * 4 : 0;
    return p;
}

template <auto KERN>
hipError_t allow_lds()
{
    static hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(KERN),
                                              hipFuncAttributeMaxDynamicSharedMemorySize,
                                              kSmLdsMax);
    return e;
}

}  // namespace

namespace kqi {

size_t small_m_workspace_bytes(int qtype, int n_rows, int k, int m)
{
    if (m < 2) return 0;  // m = 1 runs as the matvec
    return make_plan(qtype, n_rows, k, m).ws;
}

hipError_t launch_small_m_mfma(int qtype, const uint8_t *W, const float *X, int64_t ldx, float *Y,
                               int64_t ldy, int n_rows, int k, int m, void *workspace,
                               int64_t workspace_bytes, hipStream_t stream)
{
    const SmPlan p = make_plan(qtype, n_rows, k, m);
    if ((int64_t)p.ws > workspace_bytes) return hipErrorInvalidValue;
    SmArgs a;
    a.W = W;
    a.X = X;
    a.Y = Y;
    a.ws = reinterpret_cast<uint8_t *>(workspace);
    a.ldx = ldx;
    a.ldy = ldy;
    a.n_rows = n_rows;
    a.k = k;
    a.m = m;
    a.nb = p.nb;
    a.T = p.T;
    a.G = p.G;
    a.CH = p.CH;
    a.RS = p.RS;
    a.part_off = p.part_off;
    a.ws_bytes = (int)p.ws;
    a.flag_off = p.flag_off;
    hipError_t e;
    if (qtype == 1) {
        constexpr auto K = small_m_kernel<Q4Sb, 4>;
        if ((e = allow_lds<K>()) != hipSuccess) return e;
        hipLaunchKernelGGL(K, dim3(p.G), dim3(kSmThreads), p.lds, stream, a);
    } else {
        constexpr auto K = small_m_kernel<Q6Sb, 3>;
        if ((e = allow_lds<K>()) != hipSuccess) return e;
        hipLaunchKernelGGL(K, dim3(p.G), dim3(kSmThreads), p.lds, stream, a);
    }
    return hipGetLastError();
}

}  // namespace kqi

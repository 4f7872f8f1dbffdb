// kq_small_m.hip -- Y[m] = W X[m] for up to 16 activation rows over Q4_K /
// Q6_K weights: the pages' matvec-to-GEMM step (Ch 36 "Prefill vs decode: the
// two graphs", section 36.4 "Projections: from matvec to GEMM": one read of a
// weight row serves every input column), at the verify batch sizes whose M = 16
// timings Ch 19 "The down projection + residual" gives in section 19.7.
//
// Design for gfx950 (the pages' kernels use scalar f32 MACs on another GPU):
//
// * Matrix cores.  A wave owns one or two tiles of 16 weight rows and issues
//   f16 MFMAs D[16 x 16] += A[16 x K'] B[K' x 16] with A = the (up to 16)
//   activation rows and B = quants of the tile's rows: lane l holds output
//   column l % 16 = its weight row.  Every tile of a wave uses the same A
//   registers.  The Q4_K min term is one more MFMA per tile, of the
//   activation rows' 32-input group sums against the row's mins.
// * Exact quant operands.  A quant q is turned into the f16 value 1024 + q by
//   OR-ing it under the exponent of 1024 (0x6400) and the bias is removed
//   exactly.  Q4_K (16x16x32): each lane loads its own bytes of the
//   superblock (no LDS round trip) and folds its sub-block's 6-bit scale into
//   B with one exact f16 fused multiply-add, q sc <= 945 < 2^11, so one MFMA
//   spans four sub-blocks and d is applied once per superblock.  Q6_K
//   (16x16x16): q sc does not fit f16 exactly (up to 32 * 128), so a tile goes
//   through LDS, each 16-input sub-block gets its own MFMA pair and d sc is
//   applied to its result.
// * Activations at ~22 bits.  Each (row m, superblock) group of 256 inputs is
//   scaled by a power of two so that its largest magnitude is below 2^15, then
//   split into x_hi = f16(x) and x_lo = f16(x - x_hi); a hi and a lo MFMA per
//   step accumulate in f32.  The products q * x_hi and q * x_lo are exact in
//   f32.  The Q4_K group sums (of the scaled inputs, times 2^-5) are split
//   into hi and lo halves the same way.
// * Stream-K split.  The work is the grid of (row group of 256 rows, superblock)
//   tiles; workgroup g takes the contiguous range [g T / G, (g+1) T / G).  A row
//   group covered by one workgroup is stored directly.  Otherwise each
//   contributing workgroup stores its partial tile in the workspace and counts
//   itself in with an agent-scope atomic; the last to arrive sums the partials
//   in workgroup order (deterministic for a given grid) and resets the counter.
//   Nothing ever waits on another workgroup, so a launch always terminates.
// * Activation staging.  A workgroup stages the inputs of every superblock its
//   range touches into LDS once, before its loop (hi and lo planes, each
//   4-group of inputs stored in the order 0,2,1,3 to match how the quant bytes
//   unpack into f16 pairs); the grid is sized so that every range fits.  The
//   first weight loads go out with the staging's first loads (before them with
//   16 waves, right after them with 8), so HBM keeps streaming.

#include <hip/hip_runtime.h>
#include <float.h>
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "kq.h"

#include "kq_device.h"
#include "kq_internal.h"

namespace {

using namespace kqd;

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));
typedef uint32_t u32_a2 __attribute__((aligned(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Q6_K launch shapes, one workgroup per CU, 256-row groups either way:
// * 16 waves of one 16-row tile each (4 waves per SIMD hide more latency; the
//   kernel fits 128 VGPRs) whenever the staged window of a one-round grid fits
//   LDS beside their 16 weight tiles: up to 8 activation rows always, up to 12
//   at the verify shape;
// * otherwise 8 waves of two tiles each, which share every activation operand
//   they read, so a range of 8 superblocks of 16 activation rows still fits
//   LDS beside the weight tiles.
template <int SUB, int WAVES, int DEPTH>
struct SmCfg {
    static constexpr int kSub = SUB;      // 16-row tiles per wave
    static constexpr int kWaves = WAVES;  // waves per workgroup
    static constexpr int kThreads = 64 * WAVES;
    static constexpr int kDepth = DEPTH;  // tile sets in flight ahead
};
using SmNarrow = SmCfg<1, 16, 1>;  // the 16-wave shape
using SmWide = SmCfg<2, 8, 1>;     // the 8-wave shape
constexpr int kSmRows = 256;          // rows per row group: 16 kSub kWaves in every shape
static_assert(16 * SmNarrow::kSub * SmNarrow::kWaves == kSmRows, "row group");
static_assert(16 * SmWide::kSub * SmWide::kWaves == kSmRows, "row group");
constexpr uint32_t kBias = 0x64006400u;  // f16 1024.0 in both halves
constexpr int kSmLdsMax = 160 * 1024;    // per workgroup (one per CU)

struct SmArgs {
    const uint8_t *W;
    const float *X;
    float *Y;
    uint8_t *ws;        // workspace: counters, then partial tiles
    int64_t ldx, ldy;
    int n_rows, k, m;
    int nb;             // superblocks per row
    int T, G;           // tiles, workgroups
    int CH;             // superblocks of the staged window (the longest range)
    int RS;             // bytes per activation row in one LDS plane
    int part_off;       // byte offset of the partial tiles in the workspace
    int ws_bytes;
    int flag_off;       // LDS byte offset of the last-arrival flag
    int xs_off;         // LDS byte offset of the staged activations
    const float *gate;  // nullable: Y = silu(gate) * (W X), gate [M][ldg] (may be Y itself)
    int64_t ldg;
};

// The value stored for output (m, row): the product, or with a gate the
// SiLU-gated product silu(g) * v, silu(g) = g / (1 + e^-g).  The gate element
// is read by the thread that then writes the same position of Y, so Y may be
// the gate's own buffer.
__device__ __forceinline__ float sm_out(const SmArgs &a, int m, int row, float v)
{
    if (a.gate) {
        const float g = a.gate[(int64_t)m * a.ldg + row];
        v = (g / (1.0f + __expf(-g))) * v;
    }
    return v;
}

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
// Weight tiles.  A wave's tile is one superblock of each of its 16 rows.  It is
// read from HBM with coalesced 16-byte loads (consecutive lanes take
// consecutive 16-byte pieces of a row), written to the wave's own LDS slot, and
// every lane then reads the bytes its MFMA operands need from there.  (Reading
// those bytes straight from memory would cost one L1 tag lookup per lane per
// few bytes.)  Slot s of the tile is handled by lane s % 64 in load i = s / 64.

// Q6_K: a superblock starts 2-byte aligned when its global index is odd.  A row
// of the tile is read from the 4-byte aligned address a at or below it: 13
// pieces of 16 bytes cover [a, a + 208) and a tail covers [a + 208, sb + 210)
// (a dword when a = sb - 2, a 16-bit load when a = sb).  Every access stays in
// [sb - 2, sb + 210), and sb - 2 is used only when sb is not the first byte of
// W.  Rows sit 240 bytes apart in LDS so the lanes of different rows hit
// different banks.
constexpr int kQ6Pieces = 13;
constexpr int kQ6Slots = 16 * kQ6Pieces;   // 208
constexpr int kQ6Loads = 4;                // ceil(208 / 64)
constexpr int kQ6RowLds = 240;
constexpr int kQ6TileLds = 16 * kQ6RowLds;

struct Q6Tile {
    u32x4 c[kQ6Loads];
    uint32_t t;  // bytes sb+206..209: the last two scales, then d
    bool sh2;    // the superblock starts 2 bytes past a 4-byte boundary
};

template <typename U> struct TileTraits;
template <> struct TileTraits<Q6Tile> {
    static constexpr int kPieces = kQ6Pieces, kLoads = kQ6Loads,
                         kRowLds = kQ6RowLds, kTileLds = kQ6TileLds, kBlk = kQ6Bytes;
};

// Per-lane addressing of a tile: for each load i, the byte offset in W of the
// row this lane's slot belongs to (row clamped to the matrix), and the piece.
template <typename U>
struct TileAddr {
    int64_t row_off[TileTraits<U>::kLoads];
    int64_t tail_off;  // Q6_K: the row of the tail this lane loads (lanes 0..15)
};

template <typename U>
__device__ __forceinline__ void tile_rows(TileAddr<U> &ta, int rg, int slice, int lane, int n_rows,
                                          int64_t row_bytes)
{
    using T = TileTraits<U>;
#pragma unroll
    for (int i = 0; i < T::kLoads; ++i) {
        const int slot = 64 * i + lane;
        const int tr = min(slot / T::kPieces, 15);
        const int row = min(rg * kSmRows + 16 * slice + tr, n_rows - 1);
        ta.row_off[i] = (int64_t)row * row_bytes;
    }
    const int row = min(rg * kSmRows + 16 * slice + (lane & 15), n_rows - 1);
    ta.tail_off = (int64_t)row * row_bytes;
}

__device__ __forceinline__ Q6Tile load_tile(const uint8_t *__restrict__ W, const TileAddr<Q6Tile> &ta,
                                            int b, int lane)
{
    // Every lane loads (a lane past the tile's last piece re-reads that piece;
    // store_tile drops it): no branch between the loads and their use.  The
    // tail is one dword at sb+206 (2-byte aligned, inside the superblock): the
    // last two scales, needed
    // when a = sb - 2 and already in the pieces when a = sb, then d.
    // store_tile picks the word [a + 208, a + 212) the pieces would have
    // continued with (not here: touching loaded data at load time would wait
    // for the load at once).
    Q6Tile u;
#pragma unroll
    for (int i = 0; i < kQ6Loads; ++i) {
        const int slot = min(64 * i + lane, kQ6Slots - 1);
        const int64_t a = (ta.row_off[i] + (int64_t)b * kQ6Bytes) & ~(int64_t)3;
        u.c[i] = *reinterpret_cast<const u32x4_a4 *>(W + a + 16 * (slot % kQ6Pieces));
    }
    const int64_t sb = ta.tail_off + (int64_t)b * kQ6Bytes;
    u.t = *reinterpret_cast<const u32_a2 *>(W + sb + 206);
    u.sh2 = (sb & 3) != 0;  // combined in store_tile, where the data is needed anyway
    return u;
}

__device__ __forceinline__ void store_tile(const Q6Tile &u, uint8_t *tile, int lane)
{
#pragma unroll
    for (int i = 0; i < kQ6Loads; ++i) {
        const int slot = 64 * i + lane;
        if (slot < kQ6Slots)
            *reinterpret_cast<u32x4 *>(tile + kQ6RowLds * (slot / kQ6Pieces) +
                                       16 * (slot % kQ6Pieces)) = u.c[i];
    }
    if (lane < 16)
        *reinterpret_cast<uint32_t *>(tile + kQ6RowLds * lane + 208) =
            u.sh2 ? u.t : (u.t >> 16);
}

// What one lane needs of its row's superblock, read back from the LDS tile.
struct Q6Sb {
    uint32_t w[24];  // ql windows u = 0..7 (w[2u], w[2u+1]); qh windows v = 0..3 (w[16+2v], ..)
    u32x4 hs;        // scale bytes, aligned window
    uint32_t tail;   // shift 2: scales 14, 15 and d; shift 0: d
    int sh;          // byte offset of the superblock from 4-byte alignment (0 or 2)
};

__device__ __forceinline__ Q6Sb read_sb(const uint8_t *__restrict__ row, int kb, int sh, Q6Sb *)
{
    Q6Sb u;
    const uint32_t *rw = reinterpret_cast<const uint32_t *>(row);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        u.w[2 * i] = rw[4 * i + kb];
        u.w[2 * i + 1] = rw[4 * i + kb + 1];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        u.w[16 + 2 * i] = rw[32 + 4 * i + kb];
        u.w[17 + 2 * i] = rw[32 + 4 * i + kb + 1];
    }
    u.hs = *reinterpret_cast<const u32x4 *>(row + 192);
    u.tail = rw[52];
    u.sh = sh;
    return u;
}

__device__ __forceinline__ h8 as_h8(u32x4 v) { return __builtin_bit_cast(h8, v); }
__device__ __forceinline__ h4 as_h4(u32x2 v) { return __builtin_bit_cast(h4, v); }

// (x & mask) | bias in one VALU instruction.  gfx9 VOP3 encodings read at
// most one scalar or literal operand, so the mask is passed in a VGPR (set once
// per lane) and the bias as the one scalar operand.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t vmask, uint32_t bias)
{
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(vmask), "s"(bias));
    return r;
}

// Contribution of one Q6_K superblock of each of the wave's NS sub-tiles to the
// lane's 4 outputs per sub-tile, in units of the staged (scaled) activations:
// one MFMA per 16-input sub-block and plane, scaled by d sc after it.  `ah` =
// the lane's activation row in the hi plane at the superblock's first input +
// 4 kb; the lo plane is `lo_off` bytes further.
template <int NS>
__device__ __forceinline__ void sb_mma(const Q6Sb (&u)[NS], const uint8_t *__restrict__ ah,
                                       int lo_off, uint32_t vmask, f32x4 (&ys)[NS])
{
    uint32_t L[NS][8], H[NS][4], sc[NS][4];
    float d[NS];
#pragma unroll
    for (int h = 0; h < NS; ++h) {
        const int sh = u[h].sh;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            L[h][i] = __builtin_amdgcn_alignbyte(u[h].w[2 * i + 1], u[h].w[2 * i], sh);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            H[h][i] = __builtin_amdgcn_alignbyte(u[h].w[17 + 2 * i], u[h].w[16 + 2 * i], sh);
        sc[h][0] = __builtin_amdgcn_alignbyte(u[h].hs.y, u[h].hs.x, sh);
        sc[h][1] = __builtin_amdgcn_alignbyte(u[h].hs.z, u[h].hs.y, sh);
        sc[h][2] = __builtin_amdgcn_alignbyte(u[h].hs.w, u[h].hs.z, sh);
        sc[h][3] = __builtin_amdgcn_alignbyte(u[h].tail, u[h].hs.w, sh);
        d[h] = half_lo(sh ? (u[h].tail >> 16) : u[h].tail);
        ys[h] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    }
    const h4 off = {1056, 1056, 1056, 1056};
#pragma unroll
    for (int s0 = 0; s0 < 16; s0 += 4) {
        // four sub-blocks at a time: all hi MFMAs, then all lo MFMAs, so no
        // MFMA waits on the one just issued
        h4 B[NS][4];
        f32x4 acc[NS][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int s = s0 + j;
            const int hv = s >> 3, g = (s >> 1) & 3, hf = s & 1;
            const h4 Ahi = *reinterpret_cast<const h4 *>(ah + 32 * s);
#pragma unroll
            for (int h = 0; h < NS; ++h) {
                const uint32_t l = L[h][4 * hv + 2 * (g & 1) + hf], hh = H[h][2 * hv + hf];
                const uint32_t lo4 = (g < 2 ? l : (l >> 4)) & 0x0F0F0F0Fu;
                const uint32_t q = lo4 | (((hh >> (2 * g)) & 0x03030303u) << 4);
                const u32x2 bq = {and_or(q, vmask, kBias), and_or(q >> 8, vmask, kBias)};
                B[h][j] = as_h4(bq) - off;
                acc[h][j] = __builtin_amdgcn_mfma_f32_16x16x16f16(
                    Ahi, B[h][j], (f32x4){0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const h4 Alo = *reinterpret_cast<const h4 *>(ah + lo_off + 32 * (s0 + j));
#pragma unroll
            for (int h = 0; h < NS; ++h)
                acc[h][j] = __builtin_amdgcn_mfma_f32_16x16x16f16(Alo, B[h][j], acc[h][j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int s = s0 + j;
#pragma unroll
            for (int h = 0; h < NS; ++h) {
                const int scv = ((int)(sc[h][s >> 2] << (24 - 8 * (s & 3)))) >> 24;
                const float c1 = d[h] * (float)scv;
#pragma unroll
                for (int i = 0; i < 4; ++i) ys[h][i] = fmaf(c1, acc[h][j][i], ys[h][i]);
            }
        }
    }
}


// ---------------------------------------------------------------------------
// Staging of the activations of superblocks [cb, cb + n) into LDS slots so, so + 1, ...
// LDS: hi plane [M][RS bytes], lo plane [M][RS bytes], etab [CH][16] int
// (back-scale exponents), then for Q4_K the min-term table [CH][4][16][8] f16:
// for slot c and row m, [c][0][m] and [c][1][m] are the hi and lo f16 halves
// of 2^-5 times the sums of the row's 8 scaled 32-input groups (below 2^15 in
// magnitude), groups in the order 0,2,1,3,4,6,5,7, and [c][2..3][m] are zero:
// lane (r, kb) of the min-term MFMA reads [c][kb][r] as its A fragment.
//
// Eight lanes convert one (row, superblock) group of 256 inputs, 32
// consecutive inputs each: the group maximum is a DPP reduction over the
// eight, and a lane's 32 inputs are one 32-input group of the min-term table,
// summed in the lane.  A wave converts 8 groups at a time and issues the loads
// of BL such rounds before converting any, so that a workgroup's whole window
// usually arrives in one memory round trip.  A group holding a NaN or an
// infinity is staged with a NaN, so the whole output row m becomes NaN.
//
// `after_loads` runs once in every wave, right after the wave's first round of
// loads is issued (the first round's loads are unconditional; a wave without
// groups re-reads the last one).  With 8 waves (Q6_K at 9..16 activation rows,
// a heavy staging) the kernel issues its first weight loads there, behind the
// activations, so that the conversion waits for the activations only and the
// weights stream in meanwhile; with 16 waves the staging is one light round
// and the weights go first.
template <bool Q4, int BL, typename F>
__device__ __forceinline__ void stage_chunk(const SmArgs &a, int cb, int n, uint8_t *smem,
                                            int so, F &&after_loads)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int grp = lane >> 3, j8 = lane & 7;
    const int M = a.m, RS = a.RS;
    uint8_t *hi = smem, *lo = smem + M * RS;
    int *etab = reinterpret_cast<int *>(smem + 2 * M * RS);
    uint8_t *sfrag = reinterpret_cast<uint8_t *>(etab + 16 * a.CH);
    const int ngroups = M * n;
    const int nw = blockDim.x >> 6;
    typedef f32x4 Round[BL][8];
    auto load_round = [&](int r0, Round &v) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < BL; ++b) {
            // a group past the end re-reads the last one (its results are dropped)
            const int gi = min(8 * (r0 + b * nw) + grp, ngroups - 1);
            const int m = gi / n, bb = gi - m * n;
            const f32x4 *src = reinterpret_cast<const f32x4 *>(
                a.X + (int64_t)m * a.ldx + 256 * (int64_t)(cb + bb) + 32 * j8);
#pragma unroll
            for (int i = 0; i < 8; ++i) v[b][i] = src[i];
        }
    };
    auto convert_round = [&](int r0, const Round &v) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < BL; ++b) {
            if (8 * (r0 + b * nw) >= ngroups) break;  // wave-uniform
            const int gi = 8 * (r0 + b * nw) + grp;
            const bool act = gi < ngroups;  // the same for the 8 lanes of a group
            const int gc = min(gi, ngroups - 1);
            const int m = gc / n, bb = gc - m * n;
            float mx = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v[b][i].x), fabsf(v[b][i].y)),
                                     fmaxf(fabsf(v[b][i].z), fabsf(v[b][i].w))));
            mx = group_max<8>(mx);
            const bool fin = mx <= FLT_MAX;  // false for Inf and NaN
            const int e = __builtin_amdgcn_frexp_expf(mx);  // mx < 2^e
            const int sh = 15 - e;
            const int sbb = so + bb;  // LDS slot of this superblock
            const int boff = m * RS + 2 * (256 * sbb + 32 * j8);
            float sm = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t ph[4], pl[4];
#pragma unroll
                for (int i2 = 0; i2 < 2; ++i2) {
                    const f32x4 x = v[b][2 * q + i2];
                    const f32x4 sv = {ldexpf(x.x, sh), ldexpf(x.y, sh), ldexpf(x.z, sh),
                                      ldexpf(x.w, sh)};
                    _Float16 h[4], l[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        h[c] = (_Float16)sv[c];
                        l[c] = (_Float16)(sv[c] - (float)h[c]);
                    }
                    // 4 consecutive inputs stored in the order 0, 2, 1, 3
                    ph[2 * i2] = __builtin_bit_cast(uint32_t, (h2){h[0], h[2]});
                    ph[2 * i2 + 1] = __builtin_bit_cast(uint32_t, (h2){h[1], h[3]});
                    pl[2 * i2] = __builtin_bit_cast(uint32_t, (h2){l[0], l[2]});
                    pl[2 * i2 + 1] = __builtin_bit_cast(uint32_t, (h2){l[1], l[3]});
                    if constexpr (Q4) sm += (sv.x + sv.y) + (sv.z + sv.w);
                }
                if (q == 0 && !fin) ph[0] = 0x7E007E00u;  // f16 NaN pair
                if (act) {
                    *reinterpret_cast<u32x4 *>(hi + boff + 16 * q) = (u32x4){ph[0], ph[1], ph[2], ph[3]};
                    *reinterpret_cast<u32x4 *>(lo + boff + 16 * q) = (u32x4){pl[0], pl[1], pl[2], pl[3]};
                }
            }
            if (act) {
                if (j8 == 0) etab[16 * sbb + m] = e - 15;
                if constexpr (Q4) {
                    const float s5 = 0.03125f * sm;
                    _Float16 *sf = reinterpret_cast<_Float16 *>(sfrag + 1024 * sbb) + 8 * m;
                    const int pos = (j8 & 4) | ((j8 & 1) << 1) | ((j8 >> 1) & 1);  // 0,2,1,3,4,6,5,7
                    const _Float16 hs = fin ? (_Float16)s5 : (_Float16)__builtin_nanf("");
                    sf[pos] = hs;
                    sf[128 + pos] = fin ? (_Float16)(s5 - (float)hs) : hs;
                    if (j8 == 1) {
                        const u32x4 z = {0u, 0u, 0u, 0u};
                        *reinterpret_cast<u32x4 *>(sf + 256) = z;
                        *reinterpret_cast<u32x4 *>(sf + 384) = z;
                    }
                }
            }
        }
    };
    {
        Round v;
        load_round(wave, v);
        after_loads();
        if (8 * wave < ngroups) convert_round(wave, v);
    }
    for (int r0 = wave + BL * nw; 8 * r0 < ngroups; r0 += BL * nw) {
        Round v;
        load_round(r0, v);
        convert_round(r0, v);
    }
}

// This workgroup's share of row group rg is complete: store it, or publish it
// as a partial tile and, if it is the last contributor, sum all of them.
// The lane's outputs of tile h are rows 16 (kSub wave + h) + r of the row
// group, activation rows m0 .. m0 + 3.
template <int kSub>
__device__ __forceinline__ void finish_segment(const SmArgs &a, int rg, int gl, int gh, int g,
                                               const f32x4 (&yacc)[kSub], int wave, int r, int m0,
                                               int &last_flag)
{
    const int nb = a.nb, M = a.m;
    const int row0 = rg * kSmRows;
    if (gl == gh) {
#pragma unroll
        for (int h = 0; h < kSub; ++h) {
            const int row = row0 + 16 * (kSub * wave + h) + r;
            if (row < a.n_rows) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (m0 + i < M)
                        a.Y[(int64_t)(m0 + i) * a.ldy + row] = sm_out(a, m0 + i, row, yacc[h][i]);
            }
        }
        return;
    }
    float *part = reinterpret_cast<float *>(a.ws + a.part_off);
    uint32_t *cnt = reinterpret_cast<uint32_t *>(a.ws);
    const int slot = (first_tile(g, a.T, a.G) / nb == rg) ? 0 : 1;
    float *pp = part + (int64_t)(2 * g + slot) * (16 * kSmRows);
#pragma unroll
    for (int h = 0; h < kSub; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            st_agent(pp + (m0 + i) * kSmRows + 16 * (kSub * wave + h) + r, yacc[h][i]);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // this wave's stores have completed
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t old = __hip_atomic_fetch_add(cnt + rg, 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        last_flag = (old + 1 == (uint32_t)(gh - gl + 1));
    }
    __syncthreads();
    if (last_flag) {
        // Sum the contributors' partial tiles in workgroup order.  A thread
        // takes up to kE quads of 4 rows of one activation row and issues the
        // loads of 4 contributors for all of them before it adds any (loads
        // past the last contributor or quad re-read the last one, in bounds,
        // and are not used), so the sum waits for few memory round trips.
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(a.ws, (short)0, a.ws_bytes, 0x00020000);
        // quads per thread: 16 waves take up to 8 activation rows (512 quads),
        // 8 waves of two tiles up to 16 (1024 quads)
        constexpr int kE = kSub;
        const int nq = M * (kSmRows / 4);
        // every contributor after the first starts its range inside this row
        // group (slot 0); the first one owns the group's first tile and
        // starts in it or in an earlier group (slot 1)
        const int sl_first = first_tile(gl, a.T, a.G) < rg * nb ? 1 : 0;
        for (int e0 = threadIdx.x; e0 < nq; e0 += kE * blockDim.x) {
            f32x4 sum[kE];
            for (int c0 = gl; c0 <= gh; c0 += 4) {
                f32x4 v[4][kE];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int c = min(c0 + j, gh);
                    const int sl = c == gl ? sl_first : 0;
#pragma unroll
                    for (int x = 0; x < kE; ++x) {
                        const int e = min(e0 + x * (int)blockDim.x, nq - 1);
                        const int m = e / (kSmRows / 4), q = e - m * (kSmRows / 4);
                        const uint32_t off = (uint32_t)a.part_off +
                                             4u * (uint32_t)((2 * c + sl) * (16 * kSmRows) +
                                                             m * kSmRows + 4 * q);
                        v[j][x] = __builtin_bit_cast(
                            f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0,
                                                                         16 /* sc1 */));
                    }
                }
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int x = 0; x < kE; ++x)
                        if (c0 + j <= gh) sum[x] = (c0 + j == gl) ? v[j][x] : sum[x] + v[j][x];
            }
#pragma unroll
            for (int x = 0; x < kE; ++x) {
                const int e = e0 + x * (int)blockDim.x;
                if (e < nq) {
                    const int m = e / (kSmRows / 4), q = e - m * (kSmRows / 4);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = row0 + 4 * q + i;
                        if (row < a.n_rows)
                            a.Y[(int64_t)m * a.ldy + row] = sm_out(a, m, row, sum[x][i]);
                    }
                }
            }
        }
        if (threadIdx.x == 0) st_agent(cnt + rg, 0u);
    }
}

// A workgroup's range is at most one row of superblocks long, so it touches at
// most two row groups (segments).
constexpr int kMaxSegs = 2;
// Staging rounds (8 groups of 256 inputs each) a wave loads at once: with 16
// waves one covers 16 rows x 8 superblocks of the verify window, with 8 waves
// (Q6_K, m > 8) two do
constexpr int stage_batch(int waves) { return waves >= 16 ? 1 : 2; }

// The workgroup stages the activations of every superblock its range touches
// once, up front (the host sizes the grid so that they fit in LDS), and keeps
// each segment's sums in registers until after the loop.  The steady-state
// step then holds no memory operation besides the ring's own load, and the
// compiler's waits count only the ring (a load, store or barrier under a
// branch in the loop would make it wait for every load in flight at the next
// merge).
template <typename U, typename C>
__global__ void __launch_bounds__(C::kThreads, C::kWaves / 4) small_m_kernel(SmArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int kSub = C::kSub;
    constexpr int DEPTH = C::kDepth;
    using TT = TileTraits<U>;
    using Sb = Q6Sb;
    constexpr int BLK = TT::kBlk;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kb = lane >> 4, r = lane & 15, m0 = 4 * kb;
    const int g = blockIdx.x, nb = a.nb, M = a.m;
    const int t0 = first_tile(g, a.T, a.G), t1 = first_tile(g + 1, a.T, a.G);
    const int64_t row_bytes = (int64_t)nb * BLK;
    const int ma = min(r, M - 1);  // activation row this lane feeds into A
    uint8_t *xs = smem + a.xs_off;  // staged activations and their tables
    uint8_t *tile = smem + wave * TT::kTileLds;  // this wave's weight tile
    const int lo_off = M * a.RS;
    const int *etab = reinterpret_cast<const int *>(xs + 2 * M * a.RS);
    int &last_flag = *reinterpret_cast<int *>(smem + a.flag_off);
    uint32_t vmask;  // kept in a VGPR for v_and_or_b32
    asm volatile("v_mov_b32 %0, %1" : "=v"(vmask) : "s"(0x00FF00FFu));

    // next tile to load: row group rl, superblock bl; the wave's sub-tile h
    // is slice kSub wave + h of the row group
    int rl = t0 / nb, bl = t0 - rl * nb;
    TileAddr<U> ta[kSub];
#pragma unroll
    for (int h = 0; h < kSub; ++h) tile_rows<U>(ta[h], rl, kSub * wave + h, lane, a.n_rows, row_bytes);
    struct Tiles {
        U t[kSub];
    };
    auto load_next = [&]() {
        Tiles u;
#pragma unroll
        for (int h = 0; h < kSub; ++h) u.t[h] = load_tile(a.W, ta[h], bl, lane);
        if (++bl == nb) {
            bl = 0;
            ++rl;
#pragma unroll
            for (int h = 0; h < kSub; ++h)
                tile_rows<U>(ta[h], rl, kSub * wave + h, lane, a.n_rows, row_bytes);
        }
        return u;
    };

    // ring of R = DEPTH + 1 tile sets, steps unrolled R times so every slot
    // index is a constant: step j issues the loads DEPTH steps ahead into the
    // slot freed by the previous step, then uses slot j.  Loads past the
    // workgroup's last tile read clamped rows (tile_rows) and are never used.
    constexpr int R = DEPTH + 1;
    Tiles ring[R];
    auto ring_prologue = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < DEPTH; ++i) {
            ring[i] = load_next();
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // tile being computed: row group rg, superblock b; the staged window
    // starts at superblock cb
    int t = t0, rg = t0 / nb, b = t0 - rg * nb;
    const int cb = b;
    // byte offsets in W of this lane's own rows (for the Q6_K alignment shift)
    int64_t own_row[kSub];
    auto set_rows = [&]() {
#pragma unroll
        for (int h = 0; h < kSub; ++h)
            own_row[h] = (int64_t)min(rg * kSmRows + 16 * (kSub * wave + h) + r, a.n_rows - 1) *
                         row_bytes;
    };
    set_rows();
    f32x4 yacc[kSub];
#pragma unroll
    for (int h = 0; h < kSub; ++h) yacc[h] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    f32x4 sy[kMaxSegs][kSub];  // finished segments' sums
    int seg = 0;
    // Contributors of the first and last row group this workgroup touches;
    // every row group in between lies wholly inside [t0, t1).
    const int rg_first = t0 / nb, rg_last = (t1 - 1) / nb;
    const int gl_first = owner(rg_first * nb, a.T, a.G);
    const int gh_first = owner(rg_first * nb + nb - 1, a.T, a.G);
    const int gl_last = owner(rg_last * nb, a.T, a.G);
    const int gh_last = owner(rg_last * nb + nb - 1, a.T, a.G);
    // the window of superblocks cb, cb + 1, ... (mod nb) the range touches
    {
        // the host sizes the grid so that every workgroup has tiles (t0 < t1)
        const int w = t1 - t0;  // at most nb
        const int n1 = min(w, nb - cb);
        if constexpr (C::kWaves >= 16) {  // one light staging round: weights first
            ring_prologue();
            stage_chunk<false, stage_batch(C::kWaves)>(a, cb, n1, xs, 0, [] {});
        } else {
            stage_chunk<false, stage_batch(C::kWaves)>(a, cb, n1, xs, 0, ring_prologue);
        }
        if (w > n1) stage_chunk<false, stage_batch(C::kWaves)>(a, 0, w - n1, xs, n1, [] {});
        __syncthreads();
    }
    // One step: compute the tiles in ring slot u.
    auto step = [&](const Tiles &u) __attribute__((always_inline)) {
        Sb sb[kSub];
#pragma unroll
        for (int h = 0; h < kSub; ++h) {
            // The tile slot is private to this wave and LDS executes a wave's
            // accesses in order, so the previous tile's reads are done and
            // this tile's writes are visible to the reads below.
            __builtin_amdgcn_wave_barrier();
            store_tile(u.t[h], tile, lane);
            __builtin_amdgcn_wave_barrier();
            const int sh = (int)((own_row[h] + (int64_t)b * BLK) & 3);
            sb[h] = read_sb(tile + TT::kRowLds * r, kb, sh, (Sb *)nullptr);
        }
        const int bb = b >= cb ? b - cb : b + nb - cb;  // LDS slot of superblock b
        const uint8_t *ah = xs + ma * a.RS + 2 * (256 * bb + 4 * kb);
        f32x4 ys[kSub];
        sb_mma<kSub>(sb, ah, lo_off, vmask, ys);
        const i32x4 ex = *reinterpret_cast<const i32x4 *>(etab + 16 * bb + m0);
#pragma unroll
        for (int h = 0; h < kSub; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) yacc[h][i] += ldexpf(ys[h][i], ex[i]);
        ++t;
        ++b;
        if (b == nb || t == t1) {
            // registers only: a select per finished segment
#pragma unroll
            for (int q = 0; q < kMaxSegs; ++q)
#pragma unroll
                for (int h = 0; h < kSub; ++h) sy[q][h] = (q == seg) ? yacc[h] : sy[q][h];
            ++seg;
#pragma unroll
            for (int h = 0; h < kSub; ++h) yacc[h] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
            if (b == nb) {
                b = 0;
                ++rg;
                set_rows();
            }
        }
    };
    // Whole rounds of R steps, with no exit inside a round: the loop's only
    // way out is its latch, so the loads in flight there are the ring's own
    // and the compiler waits in each step only for that step's tile.  The
    // remaining rem < R tiles already sit in ring slots 0 .. rem - 1 (a step
    // loads DEPTH = R - 1 tiles ahead), so the tail steps load nothing.
    const int rounds = (t1 - t0) / R, rem = (t1 - t0) - R * rounds;
    for (int it = 0; it < rounds; ++it) {
#pragma unroll
        for (int j = 0; j < R; ++j) {
            __builtin_amdgcn_sched_barrier(0);
            ring[(j + DEPTH) % R] = load_next();
            __builtin_amdgcn_sched_barrier(0);
            step(ring[j]);
        }
    }
#pragma unroll
    for (int j = 0; j < R - 1; ++j)
        if (j < rem) step(ring[j]);
    // finish the segments in order (seg and the row groups are the same in
    // every wave, so the barriers inside are reached by all)
#pragma unroll
    for (int q = 0; q < kMaxSegs; ++q) {
        if (q < seg) {
            const int rq = rg_first + q;
            const int gl = rq == rg_first ? gl_first : gl_last;
            const int gh = rq == rg_first ? gh_first : gh_last;
            finish_segment<kSub>(a, rq, gl, gh, g, sy[q], wave, r, m0, last_flag);
        }
    }
}

// ---------------------------------------------------------------------------
// Q4_K with per-lane weight loads (no LDS round trip for the weights).
//
// Lane (r, kb) of a 16-row tile reads, per superblock, its row's 16-byte
// header and the 32 quant bytes of chunk kb (bytes 16 + 32 kb .. 47 + 32 kb of
// the superblock) straight from memory: the low nibbles of that chunk are
// sub-block 2 kb, the high nibbles sub-block 2 kb + 1.  MFMA j = 4 hn + jj of a
// plane takes from lane kb the inputs 64 kb + 32 hn + 8 jj .. + 7 (each 4-group
// in the staged order 0, 2, 1, 3), so the four lanes of a row feed four
// different sub-blocks into one MFMA.  Each lane therefore folds its
// sub-block's scale into its B values, exactly: one fused multiply-add in f16
// turns the biased quant 1024 + q into (1024 + q) sc - 1024 sc = q sc, an
// integer <= 15 * 63 = 945 < 2^11.  A high nibble is used where it sits, as
// 1024 + 16 q, with the factors sc / 16 and -64 sc (both exact), so only the
// odd bytes of a dword need a shift.  The 8 MFMAs of a plane then sum the whole
// superblock and d is applied once.
template <int NS, int WAVES, int DEPTH>
struct SmQ4Cfg {
    static constexpr int kSub = NS;       // 16-row tiles per wave
    static constexpr int kWaves = WAVES;  // waves per workgroup
    static constexpr int kThreads = 64 * WAVES;
    static constexpr int kDepth = DEPTH;  // superblock steps in flight ahead
};
// Every m: 16 waves of one tile.  Q4_K keeps no weights in LDS, so the staged
// window of 16 activation rows fits whatever the wave count, and 16 waves
// stage it in one light round; measured at 19968 x 6656 against 8 waves of
// two tiles (which share each A operand): M = 12 29.0-29.4 us against 31.9,
// M = 16 31.1-31.3 us against 32.8-32.9, M <= 8 the same kernel.
using SmQ4 = SmQ4Cfg<1, 16, 2>;
static_assert(16 * SmQ4::kSub * SmQ4::kWaves == kSmRows, "row group");

struct Q4Own {
    u32x4 hdr;  // d, dmin, 12 bytes of packed 6-bit scales and mins
    u32x4 q0;   // quant bytes 32 kb .. 32 kb + 15 of the superblock's 128
    u32x4 q1;   // quant bytes 32 kb + 16 .. 32 kb + 31
};

// p = the superblock's first byte (16-byte aligned)
__device__ __forceinline__ Q4Own load_own(const uint8_t *__restrict__ p, int kb)
{
    Q4Own u;
    u.hdr = *reinterpret_cast<const u32x4 *>(p);
    u.q0 = *reinterpret_cast<const u32x4 *>(p + 16 + 32 * kb);
    u.q1 = *reinterpret_cast<const u32x4 *>(p + 32 + 32 * kb);
    return u;
}

__device__ __forceinline__ h8 splat8(_Float16 v) { return (h8){v, v, v, v, v, v, v, v}; }

// One superblock of each of the wave's NS tiles: ys[h] = the lane's 4 outputs
// of tile h (activation rows 4 kb .. 4 kb + 3, weight row r), in units of the
// staged (scaled) activations.  `ah` = the lane's activation row in the hi
// plane at the superblock's input 64 kb; the lo plane is `lo_off` bytes
// further; `sf` = the lane's A fragment of the min-term table.
template <int NS>
__device__ __forceinline__ void q4_own_mma(const Q4Own (&u)[NS], const uint8_t *__restrict__ ah,
                                           int lo_off, const uint8_t *__restrict__ sf, int kb,
                                           uint32_t mlo, uint32_t mhi, f32x4 (&ys)[NS])
{
    const h8 off = {1024, 1024, 1024, 1024, 1024, 1024, 1024, 1024};
    const h8 As = *reinterpret_cast<const h8 *>(sf);
    h8 f0[NS], c0[NS], f1[NS], c1[NS];
    float d[NS], dmin[NS];
    f32x4 dm[NS];
#pragma unroll
    for (int h = 0; h < NS; ++h) {
        const uint32_t S0 = u[h].hdr.y, S1 = u[h].hdr.z, S2 = u[h].hdr.w;
        // scales of sub-blocks 0..3 and 4..7; this lane's are 2 kb and 2 kb + 1
        const uint32_t scA = S0 & 0x3F3F3F3Fu;
        const uint32_t scB = (S2 & 0x0F0F0F0Fu) | ((S0 >> 2) & 0x30303030u);
        const uint32_t scw = kb < 2 ? scA : scB;
        const int sh = 16 * (kb & 1);
        const _Float16 s0 = (_Float16)(float)((scw >> sh) & 0xFFu);
        const _Float16 s1 = (_Float16)(float)((scw >> (sh + 8)) & 0xFFu);
        f0[h] = splat8(s0);
        c0[h] = splat8(s0 * (_Float16)-1024.0f);
        f1[h] = splat8(s1 * (_Float16)0.0625f);
        c1[h] = splat8(s1 * (_Float16)-64.0f);
        d[h] = half_lo(u[h].hdr.x);
        dmin[h] = half_hi(u[h].hdr.x);
        // the min term: A = the activation rows' 8 group sums, B = the row's
        // 8 mins in the table's order 0,2,1,3,4,6,5,7
        const uint32_t mnA = S1 & 0x3F3F3F3Fu;
        const uint32_t mnB = ((S2 >> 4) & 0x0F0F0F0Fu) | ((S1 >> 2) & 0x30303030u);
        const u32x4 bq = {(mnA & 0x00FF00FFu) | kBias, ((mnA >> 8) & 0x00FF00FFu) | kBias,
                          (mnB & 0x00FF00FFu) | kBias, ((mnB >> 8) & 0x00FF00FFu) | kBias};
        dm[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(As, as_h8(bq) - off,
                                                       (f32x4){0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
    }
    // two accumulators per tile (even and odd jj), each taking both planes
    f32x4 acc[NS][2];
#pragma unroll
    for (int h = 0; h < NS; ++h)
#pragma unroll
        for (int c = 0; c < 2; ++c) acc[h][c] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int hn = 0; hn < 2; ++hn) {
        const uint32_t msk = hn ? mhi : mlo;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const h8 Ahi = *reinterpret_cast<const h8 *>(ah + 64 * hn + 16 * jj);
            const h8 Alo = *reinterpret_cast<const h8 *>(ah + lo_off + 64 * hn + 16 * jj);
#pragma unroll
            for (int h = 0; h < NS; ++h) {
                const u32x4 &q = jj < 2 ? u[h].q0 : u[h].q1;
                const uint32_t w0 = q[2 * (jj & 1)], w1 = q[2 * (jj & 1) + 1];
                // f16 pairs (bytes 0, 2) and (bytes 1, 3) of each dword
                const u32x4 bq = {and_or(w0, msk, kBias), and_or(w0 >> 8, msk, kBias),
                                  and_or(w1, msk, kBias), and_or(w1 >> 8, msk, kBias)};
                const h8 B = __builtin_elementwise_fma(as_h8(bq), hn ? f1[h] : f0[h],
                                                       hn ? c1[h] : c0[h]);
                acc[h][jj & 1] =
                    __builtin_amdgcn_mfma_f32_16x16x32_f16(Ahi, B, acc[h][jj & 1], 0, 0, 0);
                acc[h][jj & 1] =
                    __builtin_amdgcn_mfma_f32_16x16x32_f16(Alo, B, acc[h][jj & 1], 0, 0, 0);
            }
        }
    }
    // the table holds the group sums times 2^-5
#pragma unroll
    for (int h = 0; h < NS; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            ys[h][i] = fmaf(d[h], acc[h][0][i] + acc[h][1][i], -32.0f * dmin[h] * dm[h][i]);
}

// The same work split, staging and fix-up as small_m_kernel; the steady-state
// step holds only the ring's own loads and the LDS reads of the activations.
template <typename C>
__global__ void __launch_bounds__(C::kThreads, C::kWaves / 4) small_m_q4_kernel(SmArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int NS = C::kSub;
    constexpr int DEPTH = C::kDepth;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kb = lane >> 4, r = lane & 15, m0 = 4 * kb;
    const int g = blockIdx.x, nb = a.nb, M = a.m;
    const int t0 = first_tile(g, a.T, a.G), t1 = first_tile(g + 1, a.T, a.G);
    const int64_t row_bytes = (int64_t)nb * kQ4Bytes;
    const int ma = min(r, M - 1);  // activation row this lane feeds into A
    uint8_t *xs = smem + a.xs_off;
    const int lo_off = M * a.RS;
    const int *etab = reinterpret_cast<const int *>(xs + 2 * M * a.RS);
    const uint8_t *sfrag = reinterpret_cast<const uint8_t *>(etab + 16 * a.CH);
    int &last_flag = *reinterpret_cast<int *>(smem + a.flag_off);
    uint32_t mlo, mhi;  // nibble masks, kept in VGPRs for v_and_or_b32
    asm volatile("v_mov_b32 %0, %1" : "=v"(mlo) : "s"(0x000F000Fu));
    asm volatile("v_mov_b32 %0, %1" : "=v"(mhi) : "s"(0x00F000F0u));

    // next superblock to load: row group rl, superblock bl; lrow[h] = byte
    // offset in W of this lane's row of tile h (clamped to the matrix, so
    // loads past the workgroup's last tile stay inside W and go unused)
    int rl = t0 / nb, bl = t0 - rl * nb;
    int64_t lrow[NS];
    auto set_lrow = [&]() {
#pragma unroll
        for (int h = 0; h < NS; ++h)
            lrow[h] = (int64_t)min(rl * kSmRows + 16 * (NS * wave + h) + r, a.n_rows - 1) *
                      row_bytes;
    };
    set_lrow();
    struct Set {
        Q4Own t[NS];
    };
    auto load_next = [&]() {
        Set u;
#pragma unroll
        for (int h = 0; h < NS; ++h)
            u.t[h] = load_own(a.W + lrow[h] + (int64_t)bl * kQ4Bytes, kb);
        if (++bl == nb) {
            bl = 0;
            ++rl;
            set_lrow();
        }
        return u;
    };
    constexpr int R = DEPTH + 1;
    Set ring[R];
    auto ring_prologue = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < DEPTH; ++i) {
            ring[i] = load_next();
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    int t = t0, rg = t0 / nb, b = t0 - rg * nb;
    const int cb = b;
    f32x4 yacc[NS];
#pragma unroll
    for (int h = 0; h < NS; ++h) yacc[h] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    f32x4 sy[kMaxSegs][NS];
    int seg = 0;
    const int rg_first = t0 / nb, rg_last = (t1 - 1) / nb;
    const int gl_first = owner(rg_first * nb, a.T, a.G);
    const int gh_first = owner(rg_first * nb + nb - 1, a.T, a.G);
    const int gl_last = owner(rg_last * nb, a.T, a.G);
    const int gh_last = owner(rg_last * nb + nb - 1, a.T, a.G);
    {
        // the host sizes the grid so that every workgroup has tiles (t0 < t1)
        const int w = t1 - t0;
        const int n1 = min(w, nb - cb);
        if constexpr (C::kWaves >= 16) {  // one light staging round: weights first
            ring_prologue();
            stage_chunk<true, stage_batch(C::kWaves)>(a, cb, n1, xs, 0, [] {});
        } else {
            stage_chunk<true, stage_batch(C::kWaves)>(a, cb, n1, xs, 0, ring_prologue);
        }
        if (w > n1) stage_chunk<true, stage_batch(C::kWaves)>(a, 0, w - n1, xs, n1, [] {});
        __syncthreads();
    }
    auto step = [&](const Set &u) __attribute__((always_inline)) {
        const int bb = b >= cb ? b - cb : b + nb - cb;  // LDS slot of superblock b
        const uint8_t *ah = xs + ma * a.RS + 2 * 256 * bb + 128 * kb;
        f32x4 ys[NS];
        q4_own_mma<NS>(u.t, ah, lo_off, sfrag + 1024 * bb + 256 * kb + 16 * ma, kb, mlo, mhi, ys);
        const i32x4 ex = *reinterpret_cast<const i32x4 *>(etab + 16 * bb + m0);
#pragma unroll
        for (int h = 0; h < NS; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) yacc[h][i] += ldexpf(ys[h][i], ex[i]);
        ++t;
        ++b;
        if (b == nb || t == t1) {
#pragma unroll
            for (int q = 0; q < kMaxSegs; ++q)
#pragma unroll
                for (int h = 0; h < NS; ++h) sy[q][h] = (q == seg) ? yacc[h] : sy[q][h];
            ++seg;
#pragma unroll
            for (int h = 0; h < NS; ++h) yacc[h] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
            if (b == nb) {
                b = 0;
                ++rg;
            }
        }
    };
    const int rounds = (t1 - t0) / R, rem = (t1 - t0) - R * rounds;
    for (int it = 0; it < rounds; ++it) {
#pragma unroll
        for (int j = 0; j < R; ++j) {
            __builtin_amdgcn_sched_barrier(0);
            ring[(j + DEPTH) % R] = load_next();
            __builtin_amdgcn_sched_barrier(0);
            step(ring[j]);
        }
    }
#pragma unroll
    for (int j = 0; j < R - 1; ++j)
        if (j < rem) step(ring[j]);
#pragma unroll
    for (int q = 0; q < kMaxSegs; ++q) {
        if (q < seg) {
            const int rq = rg_first + q;
            const int gl = rq == rg_first ? gl_first : gl_last;
            const int gh = rq == rg_first ? gh_first : gh_last;
            finish_segment<NS>(a, rq, gl, gh, g, sy[q], wave, r, m0, last_flag);
        }
    }
}

struct SmPlan {
    int nb, T, G, CH, RS, part_off, flag_off, xs_off;
    size_t lds, ws;
    bool narrow;  // the 16-wave launch shape
};

int sm_cus() { return kqi::device_cus(); }

SmPlan make_plan(int qtype, int n_rows, int k, int m, int cus)
{
    SmPlan p;
    p.nb = k / 256;
    const int rgs = (n_rows + kSmRows - 1) / kSmRows;
    p.T = rgs * p.nb;
    const int per_sb = 1024 * m + 64 + (qtype == 1 ? 1024 : 0);  // LDS bytes per staged superblock
    // the 16-wave shape: always for Q4_K; for Q6_K when the window of a
    // one-round grid still fits LDS beside 16 waves' weight tiles (up to
    // m = 12 at the verify shape), else 8 waves of two tiles
    {
        const int64_t g1 = p.T < cus ? p.T : cus;
        const int64_t need = (p.T + g1 - 1) / g1;
        const int64_t fit16 = (kSmLdsMax - SmNarrow::kWaves * kQ6TileLds - 16 - 32 * m) / per_sb;
        p.narrow = qtype == 1 || m <= 8 || fit16 >= (need < p.nb ? need : p.nb);
    }
    // Q6_K: the waves' weight tiles first; Q4_K keeps no weights in LDS
    p.xs_off = qtype == 1 ? 0 : (p.narrow ? SmNarrow::kWaves : SmWide::kWaves) * kQ6TileLds;
    int ch = (kSmLdsMax - p.xs_off - 16 - 32 * m) / per_sb;  // superblocks that fit
    if (ch > p.nb) ch = p.nb;
    if (ch < 1) ch = 1;
    // one workgroup per CU, more when a range would not fit in LDS at once:
    // every range is then at most ch <= nb tiles long
    p.G = p.T < cus ? p.T : cus;
    if ((p.T + p.G - 1) / p.G > ch) p.G = (p.T + ch - 1) / ch;
    ch = (p.T + p.G - 1) / p.G;  // the longest range
    p.CH = ch;
    p.RS = 512 * ch + 16;
    p.flag_off = p.xs_off + 2 * m * p.RS + 64 * ch + (qtype == 1 ? 1024 * ch : 0);
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
    static std::atomic<uint64_t> done{0};
    return kqi::raise_lds_limit(reinterpret_cast<const void *>(KERN), done, kSmLdsMax);
}

// The plan's launch, with the partial tiles at byte part_off of ws (counters
// at its start) and ws_bytes the bytes the kernel may touch there.
hipError_t launch_plan(const SmPlan &p, int qtype, const uint8_t *W, const float *X, int64_t ldx,
                       float *Y, int64_t ldy, int n_rows, int k, int m, uint8_t *ws, int part_off,
                       int64_t ws_bytes, hipStream_t stream, const float *gate = nullptr,
                       int64_t ldg = 0)
{
    SmArgs a;
    a.gate = gate;
    a.ldg = ldg;
    a.W = W;
    a.X = X;
    a.Y = Y;
    a.ws = ws;
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
    a.part_off = part_off;
    a.ws_bytes = (int)ws_bytes;
    a.flag_off = p.flag_off;
    a.xs_off = p.xs_off;
    hipError_t e;
#define KQ_SM_GO(U, C)                                                                         \
    {                                                                                         \
        constexpr auto K = small_m_kernel<U, C>;                                              \
        if ((e = allow_lds<K>()) != hipSuccess) return e;                                     \
        hipLaunchKernelGGL(K, dim3(p.G), dim3(C::kThreads), p.lds, stream, a);                 \
        return hipGetLastError();                                                             \
    }
#define KQ_SM_Q4_GO(C)                                                                        \
    {                                                                                         \
        constexpr auto K = small_m_q4_kernel<C>;                                              \
        if ((e = allow_lds<K>()) != hipSuccess) return e;                                     \
        hipLaunchKernelGGL(K, dim3(p.G), dim3(C::kThreads), p.lds, stream, a);                 \
        return hipGetLastError();                                                             \
    }
    if (qtype == 1) {
        KQ_SM_Q4_GO(SmQ4)
    }
    if (p.narrow) KQ_SM_GO(Q6Tile, SmNarrow)
    KQ_SM_GO(Q6Tile, SmWide)
#undef KQ_SM_Q4_GO
#undef KQ_SM_GO
}

// ---------------------------------------------------------------------------
// Library-owned scratch for kq_matmul_small_m_noalloc: one counter per 256-row
// group in the first kNaCounterBytes, then the partial tiles of up to
// kNaPartBytes / (2 * 16 * kSmRows * 4) workgroups.  Each GPU the library runs
// on holds its own copy of the array until the process ends.  In host code
// `scratch` is a host-side stand-in for the symbol, not a device address: its
// device address comes from hipGetSymbolAddress, once per device.
constexpr int kNaCounterBytes = 16 * 1024;
constexpr size_t kNaPartBytes = (size_t)16 << 20;
static_assert(kNaCounterBytes + kNaPartBytes == KQ_SMALL_M_SCRATCH_BYTES, "kq.h size");
__device__ __align__(256) uint8_t scratch[kNaCounterBytes + kNaPartBytes];

__global__ void zero_words_kernel(uint32_t *p, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
struct NaDev {
    uint8_t *ptr;  // device address of `scratch` on this device
    bool zeroed;   // the counter words have been cleared on this device
};
NaDev g_na[kMaxDevices];
std::mutex g_na_mutex;

}  // namespace

namespace kqi {

size_t small_m_workspace_bytes(int qtype, int n_rows, int k, int m)
{
    if (m < 2) return 0;  // m = 1 runs as the matvec
    if (rows_path(qtype, n_rows, k, m)) return 0;  // the dot path takes no workspace
    return make_plan(qtype, n_rows, k, m, sm_cus()).ws;
}

void small_m_plan(int qtype, int n_rows, int k, int m, int cus, int64_t *out)
{
    const SmPlan p = make_plan(qtype, n_rows, k, m, cus);
    out[0] = p.G;
    out[1] = p.CH;
    out[2] = (int64_t)p.lds;
    out[3] = (int64_t)p.ws;
    out[4] = qtype == 1 ? SmQ4::kThreads : (p.narrow ? SmNarrow::kThreads : SmWide::kThreads);
    out[5] = p.T;
}

hipError_t launch_small_m(int qtype, const uint8_t *W, const float *X, int64_t ldx, float *Y,
                          int64_t ldy, int n_rows, int k, int m, void *workspace,
                          int64_t workspace_bytes, hipStream_t stream, const float *gate,
                          int64_t ldg)
{
    if (rows_path(qtype, n_rows, k, m))
        return launch_rows(qtype, W, X, ldx, Y, ldy, n_rows, k, m, gate, ldg, stream);
    const SmPlan p = make_plan(qtype, n_rows, k, m, sm_cus());
    if ((int64_t)p.ws > workspace_bytes) return hipErrorInvalidValue;
    return launch_plan(p, qtype, W, X, ldx, Y, ldy, n_rows, k, m,
                       reinterpret_cast<uint8_t *>(workspace), p.part_off, (int64_t)p.ws, stream,
                       gate, ldg);
}

bool small_m_noalloc_fits(int qtype, int n_rows, int k, int m)
{
    if (m < 2) return true;
    if (rows_path(qtype, n_rows, k, m)) return true;  // no scratch
    const SmPlan p = make_plan(qtype, n_rows, k, m, sm_cus());
    if (p.ws == 0) return true;  // no row group is split: the scratch is not used
    const int64_t rgs = ((int64_t)n_rows + kSmRows - 1) / kSmRows;
    const int64_t parts = (int64_t)p.G * 2 * 16 * kSmRows * 4;
    return 4 * rgs <= kNaCounterBytes && parts <= (int64_t)kNaPartBytes;
}

hipError_t launch_small_m_noalloc(int qtype, const uint8_t *W, const float *X, int64_t ldx,
                                  float *Y, int64_t ldy, int n_rows, int k, int m,
                                  hipStream_t stream)
{
    if (rows_path(qtype, n_rows, k, m))  // the dot path uses no scratch
        return launch_rows(qtype, W, X, ldx, Y, ldy, n_rows, k, m, nullptr, 0, stream);
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    const SmPlan p = make_plan(qtype, n_rows, k, m, sm_cus());
    uint8_t *base;
    bool clear = false;
    {
        std::lock_guard<std::mutex> lock(g_na_mutex);
        if (!g_na[dev].ptr) {
            void *ptr = nullptr;
            e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!ptr) return hipErrorInvalidSymbol;
            g_na[dev].ptr = reinterpret_cast<uint8_t *>(ptr);
        }
        base = g_na[dev].ptr;
        if (p.ws > 0 && !g_na[dev].zeroed) {  // the first call that uses the counters
            clear = true;
            g_na[dev].zeroed = true;
        }
    }
    if (p.ws > 0) {
        // every call leaves the counters it used at zero; they start at zero
        // from the first call's clear (a fill kernel, not a memset, so that
        // a call under graph capture records a kernel node)
        if (clear) {
            const int words = kNaCounterBytes / 4;
            hipLaunchKernelGGL(zero_words_kernel, dim3((words + 255) / 256), dim3(256), 0, stream,
                               reinterpret_cast<uint32_t *>(base), words);
            if ((e = hipGetLastError()) != hipSuccess) {
                std::lock_guard<std::mutex> lock(g_na_mutex);
                g_na[dev].zeroed = false;
                return e;
            }
        }
        const int64_t need = kNaCounterBytes + (int64_t)p.G * 2 * 16 * kSmRows * 4;
        if (need > (int64_t)sizeof(scratch)) return hipErrorInvalidValue;
        return launch_plan(p, qtype, W, X, ldx, Y, ldy, n_rows, k, m, base, kNaCounterBytes, need,
                           stream);
    }
    return launch_plan(p, qtype, W, X, ldx, Y, ldy, n_rows, k, m, base, kNaCounterBytes, 0, stream);
}

}  // namespace kqi

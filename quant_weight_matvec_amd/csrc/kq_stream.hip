// kq_stream.hip -- the M = 1 matvec as an in-order byte stream through LDS.
//
// A workgroup owns a contiguous range of weight rows, i.e. one contiguous run
// of superblocks in memory (each row is its k/256 superblocks back to back and
// rows follow one another; Ch 19 "The down projection + residual", section
// 19.3, gives the 78 superblocks per 19,968-wide row, and section 19.1 the
// decode matvec itself).  It reads that run in address order,
// chunk after chunk, with direct-to-LDS 16-byte loads (global_load_lds_dwordx4:
// no registers held while in flight), keeping NBUF chunks in flight.  Every
// DRAM page is thus read whole while it is open, and the number of bytes in
// flight does not depend on how the arithmetic is mapped to lanes.
//
// Compute: four lanes per superblock, lane q taking the 32 quant bytes of
// sub-blocks 2q (low nibbles) and 2q+1 (high nibbles) against the activation,
// staged once per workgroup as three signed byte limbs per input with one
// exponent per 32-input group (the matvec's staging).  The four partial sums
// of a superblock are added in a fixed order and stored in LDS; a row's
// superblock sums are added in order at the end.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kq_device.h"
#include "kq_internal.h"

namespace {

using namespace kqd;

constexpr int kStThreads = 512;
constexpr int kStWaves = kStThreads / 64;
constexpr int kQ4ChunkSb = 112;                        // superblocks per chunk
constexpr int kQ4ChunkBytes = kQ4ChunkSb * kQ4Bytes;   // 16128
constexpr int kChunkStride = 16384;                    // LDS bytes per ring slot
constexpr int kPiecesPerThread = kChunkStride / 16 / kStThreads;  // 2
constexpr int kStLdsMax = 160 * 1024;

struct StArgs {
    const uint8_t *W;
    const float *x;
    float *y;
    const float *silu_gate;
    int n_rows, k, nb;
    int rows_per_wg;
    int nbuf;          // ring slots
    int x_bytes;       // LDS bytes of the staged activation
    int part_off;      // LDS offset of the per-superblock sums
    int ring_off;      // LDS offset of the ring
};

// Issue the loads of chunk c (superblocks [112 c, 112 c + 112) of this
// workgroup's run) into ring slot `slot`.  Every thread issues exactly
// kPiecesPerThread loads per chunk, in the same order for every chunk, so a
// wait on the vector-memory counter can name a chunk.  Pieces past the end of
// the run re-read the run's first piece and land in the slot's padding or in
// bytes the compute never reads.
__device__ __forceinline__ void issue_chunk(const uint8_t *__restrict__ run, int64_t run_bytes,
                                            int c, uint32_t slot)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < kPiecesPerThread; ++j) {
        // each wave fills one contiguous 1 KB block of the slot
        const int blk = j * kStWaves + wave;
        const int in = 1024 * blk + 16 * lane;  // byte within the chunk
        const int64_t off = (int64_t)c * kQ4ChunkBytes + in;
        const int64_t o = (off + 16 <= run_bytes && in < kQ4ChunkBytes) ? off : 0;
        // the LDS address is the same for the whole wave: make that explicit
        lds_dma16(run + o, __builtin_amdgcn_readfirstlane(slot + 1024 * blk));
    }
}

// s_waitcnt immediate: vmcnt = loads of the NBUF-1 younger chunks (gfx9
// encoding: vmcnt[3:0] in bits 3:0 and vmcnt[5:4] in bits 15:14; expcnt and
// lgkmcnt left at their no-wait maxima)
template <int NBUF>
constexpr int kWaitRing = 0x0F70 | ((kPiecesPerThread * (NBUF - 1)) & 15) |
                          (((kPiecesPerThread * (NBUF - 1)) >> 4) << 14);

template <int NBUF>
__global__ void __launch_bounds__(kStThreads) q4k_stream_kernel(StArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63;
    const int g = blockIdx.x;
    const int r0 = g * a.rows_per_wg;
    const int r1 = min(r0 + a.rows_per_wg, a.n_rows);
    if (r0 >= r1) return;
    const int nsb = (r1 - r0) * a.nb;  // superblocks of this workgroup
    const int64_t run_bytes = (int64_t)nsb * kQ4Bytes;
    const uint8_t *run = a.W + (int64_t)r0 * a.nb * kQ4Bytes;
    const int nchunks = (nsb + kQ4ChunkSb - 1) / kQ4ChunkSb;
    uint8_t *ring = smem + a.ring_off;
    const uint32_t ring_lds = lds_addr(ring);
    float *part = reinterpret_cast<float *>(smem + a.part_off);

    // start the stream before anything else
#pragma unroll
    for (int c = 0; c < NBUF; ++c)
        if (c < nchunks) issue_chunk(run, run_bytes, c, ring_lds + c * kChunkStride);

    stage_activation<32, KQ_LIMBS>(a.x, a.k, smem);
    const uint8_t *planes = smem;
    const float *tscale = reinterpret_cast<const float *>(smem + KQ_LIMBS * plane_bytes(a.k));
    const float *tsum = tscale + (a.k >> 5);

    const int sbl = threadIdx.x >> 2;  // superblock of this lane within a chunk
    const int q = threadIdx.x & 3;     // quarter: sub-blocks 2q and 2q+1
    for (int c = 0; c < nchunks; ++c) {
        // wait for this thread's loads of chunk c (the NBUF-1 later chunks may
        // still be in flight), then for every thread's
        if (c + NBUF - 1 < nchunks)
            __builtin_amdgcn_s_waitcnt(kWaitRing<NBUF>);
        else
            __builtin_amdgcn_s_waitcnt(0x0F70);  // near the end: wait for all
        __syncthreads();
        const uint8_t *slot = ring + (c % NBUF) * kChunkStride;
        const int s = c * kQ4ChunkSb + sbl;  // superblock index within the run
        if (sbl < kQ4ChunkSb && s < nsb) {
            const uint8_t *sb = slot + sbl * kQ4Bytes;
            const u32x4 hdr = *reinterpret_cast<const u32x4 *>(sb);
            const u32x4 qa = *reinterpret_cast<const u32x4 *>(sb + 16 + 32 * q);
            const u32x4 qb = *reinterpret_cast<const u32x4 *>(sb + 32 + 32 * q);
            const int b = s % a.nb;
            const int base = 256 * b + 64 * q;  // first input of sub-block 2q
            // 6-bit scale and min of sub-blocks 2q (low) and 2q+1 (high)
            const uint32_t S0 = hdr.y, S1 = hdr.z, S2 = hdr.w;
            int sc[2], mn[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int j = 2 * q + h;
                if (j < 4) {
                    sc[h] = (S0 >> (8 * j)) & 63;
                    mn[h] = (S1 >> (8 * j)) & 63;
                } else {
                    sc[h] = ((S2 >> (8 * (j - 4))) & 15) | (((S0 >> (8 * (j - 4) + 6)) & 3) << 4);
                    mn[h] = ((S2 >> (8 * (j - 4) + 4)) & 15) | (((S1 >> (8 * (j - 4) + 6)) & 3) << 4);
                }
            }
            int acc[2][KQ_LIMBS];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int l = 0; l < KQ_LIMBS; ++l) acc[h][l] = 0;
            const uint32_t qw[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
#pragma unroll
            for (int l = 0; l < KQ_LIMBS; ++l) {
                const uint8_t *pl = planes + l * (int)plane_bytes(a.k) + plane_off(base);
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const u32x4 xl = *reinterpret_cast<const u32x4 *>(pl + 16 * p);
                    const u32x4 xh = *reinterpret_cast<const u32x4 *>(pl + 32 + 16 * p);
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const uint32_t v = qw[4 * p + w];
                        acc[0][l] = sdot4(v & 0x0F0F0F0Fu, xl[w], acc[0][l]);
                        acc[1][l] = sdot4((v >> 4) & 0x0F0F0F0Fu, xh[w], acc[1][l]);
                    }
                }
            }
            const float d = half_lo(hdr.x), dmin = half_hi(hdr.x);
            const int g0 = base >> 5;
            float out = 0.0f;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float v = combine_limbs<KQ_LIMBS>(acc[h]);
                out += (d * (float)sc[h]) * (tscale[g0 + h] * v) - (dmin * (float)mn[h]) * tsum[g0 + h];
            }
            out = group_sum<4>(out);
            if (q == 0) part[s] = out;
        }
        __syncthreads();  // slot c is free again
        if (c + NBUF < nchunks)
            issue_chunk(run, run_bytes, c + NBUF, ring_lds + (c % NBUF) * kChunkStride);
    }
    __syncthreads();
    // y: each row's superblock sums in order
    for (int i = threadIdx.x; i < r1 - r0; i += kStThreads) {
        float v = 0.0f;
        for (int b = 0; b < a.nb; ++b) v += part[i * a.nb + b];
        if (a.silu_gate) {
            const float gt = a.silu_gate[r0 + i];
            v = (gt / (1.0f + __expf(-gt))) * v;
        }
        a.y[r0 + i] = v;
    }
    (void)lane;
}

}  // namespace

namespace kqi {

static int g_matvec_impl[3] = {0, 0, 0};
int matvec_impl(int qtype) { return (qtype == 1 || qtype == 2) ? g_matvec_impl[qtype] : 0; }
void set_matvec_impl(int qtype, int impl)
{
    if (qtype == 1 || qtype == 2) g_matvec_impl[qtype] = impl;
}

size_t q4k_stream_lds(int n_rows, int k, int grid, int nbuf, int *rows_per_wg, int *x_bytes,
                      int *part_off, int *ring_off)
{
    const int nb = k / 256;
    const int rpw = (n_rows + grid - 1) / grid;
    const int xb = (int)staged_bytes<32, KQ_LIMBS>(k);
    const int po = (xb + 15) & ~15;
    const int ro = (po + 4 * rpw * nb + 1023) & ~1023;
    if (rows_per_wg) *rows_per_wg = rpw;
    if (x_bytes) *x_bytes = xb;
    if (part_off) *part_off = po;
    if (ring_off) *ring_off = ro;
    return (size_t)ro + (size_t)nbuf * kChunkStride;
}

hipError_t launch_matvec_q4k_stream(const uint8_t *W, const float *x, float *y, int n_rows, int k,
                                    const float *silu_gate, int grid, int nbuf, hipStream_t stream)
{
    StArgs a;
    a.W = W;
    a.x = x;
    a.y = y;
    a.silu_gate = silu_gate;
    a.n_rows = n_rows;
    a.k = k;
    a.nb = k / 256;
    const size_t lds = q4k_stream_lds(n_rows, k, grid, nbuf, &a.rows_per_wg, &a.x_bytes,
                                      &a.part_off, &a.ring_off);
    a.nbuf = nbuf;
    if (lds > (size_t)kStLdsMax) return hipErrorInvalidValue;
    const int g = (n_rows + a.rows_per_wg - 1) / a.rows_per_wg;
#define KQ_ST(NB)                                                                              \
    if (nbuf == NB) {                                                                          \
        static hipError_t e = hipFuncSetAttribute(                                             \
            reinterpret_cast<const void *>(q4k_stream_kernel<NB>),                              \
            hipFuncAttributeMaxDynamicSharedMemorySize, kStLdsMax);                            \
        if (e != hipSuccess) return e;                                                         \
        hipLaunchKernelGGL(q4k_stream_kernel<NB>, dim3(g), dim3(kStThreads), lds, stream, a);  \
        return hipGetLastError();                                                              \
    }
    KQ_ST(2)
    KQ_ST(3)
    KQ_ST(4)
    KQ_ST(5)
    KQ_ST(6)
    KQ_ST(7)
#undef KQ_ST
    return hipErrorInvalidValue;
}

}  // namespace kqi

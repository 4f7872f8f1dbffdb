// kq_chain.hip -- one decode token through a stack of FFN layers as a single
// persistent kernel.
//
// Each layer is the FFN block of the pages' decode graph (Ch 10 "The forward
// pass at a glance", section 10.3, boxes 11-13; Ch 19 "The down projection +
// residual", section 19.1):
//   mid      = silu(W_gate x) * (W_up x)                    (Q4_K, ffn x hidden)
//   p        = W_down mid                                   (Q6_K or Q4_K, hidden x ffn)
//   residual = residual + rms_norm(p, eps_post) * g_post
//   x        = rms_norm(residual, eps_next) * g_next        (next layer's input)
// The pages record a whole token on one command buffer and press play once
// (Ch 10, section 10.3); on gfx950 the analogue is one cooperative launch that
// streams every layer's weights with grid-wide barriers only where the data
// really depends on all workgroups:
//   phase A  each workgroup computes mid for its own rows of gate/up (whole
//            16- or 32-row scale groups) and publishes them already encoded for
//            the down projection (byte limbs, exponent, group sum);
//   barrier
//   phase B  each workgroup copies the encoded mid into LDS and computes its
//            rows of p;
//   barrier
//   phase C  every workgroup computes the tail for the whole row itself (same
//            inputs, same order, hence bitwise-identical copies) and encodes the
//            next layer's x straight into LDS, so no third barrier is needed.
// Before each barrier a workgroup issues the loads of its first weight units of
// the next phase, so HBM keeps streaming while the barrier completes.
//
// Cross-workgroup data (encoded mid, p, barrier counters) is written and read
// with agent-scope (sc1) accesses, which are coherent across the per-XCD L2
// caches without invalidating them; a workgroup waits for its own stores to
// complete before it arrives.  Barrier waits are bounded: after
// kSpinLimit polls a workgroup records an error flag and leaves, so a launch
// always terminates.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "kq_device.h"
#include "kq_internal.h"

namespace {

using namespace kqd;

constexpr int kChainWaves = 8;  // 256-VGPR budget: Q6_K keeps 3 units in flight
constexpr int kChainThreads = 64 * kChainWaves;
constexpr int kSpinLimit = 1 << 21;
constexpr int kPhaseBLanes = 8;
constexpr int kQ4Look = 1;  // units looked ahead in phase A (2 in flight)
constexpr int kQ6Look = 2;  // units looked ahead in phase B (3 in flight)
constexpr int kPv = 8;      // float4 slots of p per thread in the tail: hidden <= 16384

struct ChainArgs {
    const uint8_t *const *wg;   // [layers] device pointers
    const uint8_t *const *wu;
    const uint8_t *const *wd;
    const float *const *gpost;  // [layers] -> [hidden]
    const float *const *gnext;
    const float *x_in;          // [hidden]
    float *residual;            // [hidden] in/out
    float *x_out;               // [hidden]
    uint32_t *enc;              // workspace: encoded mid (planes, scales, sums)
    float *p;                   // workspace: [hidden]
    uint32_t *bar;              // workspace: [0] arrivals, [1] exits, [2] error
    uint8_t *ws;                // workspace base (bar, enc and p live inside)
    uint32_t ws_bytes;
    int layers, hidden, ffn;
    float eps_post, eps_next;
};

__device__ __forceinline__ void st_agent(uint32_t *p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_agent(const uint32_t *p)
{
    return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

// Coherent 16-byte loads of workspace data written by other workgroups: a
// buffer load with the agent-scope (sc1) cache policy.  Unlike scalar atomic
// loads these are issued back to back, and the descriptor's size bounds every
// access (an out-of-range offset reads zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ws_rsrc(const ChainArgs &a)
{
    return __builtin_amdgcn_make_buffer_rsrc(a.ws, (short)0, (int)a.ws_bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 ld_agent16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 16 /* sc1 */);
}

// Workspace control block, 32-bit words, every counter on its own 128-byte
// line: word 0 the release flag (last completed barrier epoch), word 1 the
// exit count, word 2 the error code; word 32*(1+g) the arrivals of group g
// (kBarGroup workgroups each); word kCtlTop the arrivals of group leaders.
constexpr int kBarGroup = 16;
constexpr int kMaxGroups = 64;  // up to 1024 workgroups
constexpr int kCtlTop = 32 * (1 + kMaxGroups);
constexpr int kCtlWords = kCtlTop + 32;

// Wait until this wave's stores have completed (vmcnt only; the LDS and
// export counters are left alone).  Cross-workgroup data is stored with
// agent-scope (sc1) stores, so once complete it is visible to the sc1 loads of
// every other workgroup; no L2 write-back is needed.
__device__ __forceinline__ void stores_done() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Grid barrier number `epoch` (1, 2, ...), two-level: a workgroup arrives on
// its group's counter; the last arrival of a group arrives on the top counter;
// the last arrival overall publishes the epoch in the release flag, which all
// poll.  At most kBarGroup (or kMaxGroups) atomics meet on one address.  The
// caller has completed its cross-workgroup stores (stores_done) and may have
// loads in flight.  Returns false if the wait timed out (error flag set).
__device__ bool grid_barrier(uint32_t *ctl, uint32_t epoch, int *ok_lds)
{
    __syncthreads();
    if (threadIdx.x == 0) {
        int ok = 1;
        const int G = gridDim.x, w = blockIdx.x;
        const int ngroups = (G + kBarGroup - 1) / kBarGroup;
        const int g = w / kBarGroup;
        const int members = min(kBarGroup, G - g * kBarGroup);
        const uint32_t old = __hip_atomic_fetch_add(ctl + 32 * (1 + g), 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        if (old + 1 == epoch * (uint32_t)members) {
            const uint32_t t = __hip_atomic_fetch_add(ctl + kCtlTop, 1u, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
            if (t + 1 == epoch * (uint32_t)ngroups) st_agent(ctl, epoch);
        }
        int spins = 0;
        while (ld_agent(ctl) < epoch) {
            __builtin_amdgcn_s_sleep(1);
            if (++spins > kSpinLimit) {
                st_agent(ctl + 2, 1u);
                ok = 0;
                break;
            }
        }
        *ok_lds = ok;
    }
    __syncthreads();
    return *ok_lds != 0;
}

// Encode 4 consecutive values of a scale group (GROUP inputs) into the
// down projection's staging format, in global memory: LIMBS byte planes of
// plane_bytes(ffn) bytes (16 bytes of padding after every 128 inputs), then
// ffn/GROUP back-scales, then ffn/GROUP group sums (the same layout the
// matvec kernels build in LDS).
template <int GROUP>
__device__ __forceinline__ void encode_group_global(f32x4 v, int i, uint32_t *enc, int ffn)
{
    constexpr int TPG = GROUP / 4;
    constexpr int QB = limb_bits<KQ_LIMBS>();
    const int n4 = ffn >> 2;
    const float mx = group_max<TPG>(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    const float sm = group_sum<TPG>((v.x + v.y) + (v.z + v.w));
    const int e = __builtin_amdgcn_frexp_expf(mx);
    const int sh = QB - e;
    int q[4];
    q[0] = (int)rintf(ldexpf(v.x, sh));
    q[1] = (int)rintf(ldexpf(v.y, sh));
    q[2] = (int)rintf(ldexpf(v.z, sh));
    q[3] = (int)rintf(ldexpf(v.w, sh));
    uint32_t pk[KQ_LIMBS];
#pragma unroll
    for (int l = 0; l < KQ_LIMBS; ++l) pk[l] = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = (q[j] << 24) >> 24;
        const int t = (q[j] - c) >> 8;
        const int b = (t << 24) >> 24;
        const int a = (t - b) >> 8;
        pk[0] |= (uint32_t)(a & 255) << (8 * j);
        pk[1] |= (uint32_t)(b & 255) << (8 * j);
        pk[2] |= (uint32_t)(c & 255) << (8 * j);
    }
    const int pw = n4 + (n4 >> 3), wi = i + ((i >> 5) << 2);  // padded plane words
#pragma unroll
    for (int l = 0; l < KQ_LIMBS; ++l) st_agent(enc + l * pw + wi, pk[l]);
    if ((i & (TPG - 1)) == 0) {
        float *tscale = reinterpret_cast<float *>(enc + KQ_LIMBS * pw);
        float *tsum = tscale + ffn / GROUP;
        const int g = i / TPG;
        st_agent(tscale + g, isfinite(sm) ? ldexpf(1.0f, e - QB) : __builtin_nanf(""));
        st_agent(tsum + g, sm);
    }
}

// One lane's share of a row: `units` half-superblock units, lane `sub` takes
// sub, sub+LANES, ...; ring[] holds the look-ahead (already issued).
template <int LANES, int LOOK, class U, class LD, class DOT>
__device__ __forceinline__ float row_share(U (&ring)[LOOK > 0 ? LOOK : 1], int sub, int units,
                                           bool rv, LD load, DOT dot)
{
    const int steps = (units + LANES - 1) / LANES;
    float acc = 0.0f;
    for (int st = 0; st < steps; ++st) {
        const int u = sub + LANES * st;
        const int un = u + LANES * LOOK;
        U nxt;
        if (rv && un < units) nxt = load(un);
        if (rv && u < units) {
            const U &cur = LOOK > 0 ? ring[0] : nxt;
            acc += dot(cur, u);
        }
        if constexpr (LOOK > 0) {
#pragma unroll
            for (int j = 0; j + 1 < LOOK; ++j) ring[j] = ring[j + 1];
            ring[LOOK - 1] = nxt;
        }
    }
    return acc;
}

// Issue the first LOOK units of a row.  Every slot is assigned on every path
// (zero when the lane has no row), so the previous phase's ring is dead here
// and does not occupy registers through the other phases.
template <int LANES, int LOOK, class U, class LD>
__device__ __forceinline__ void prefill(U (&ring)[LOOK > 0 ? LOOK : 1], int sub, int units, bool rv,
                                        LD load)
{
#pragma unroll
    for (int j = 0; j < LOOK; ++j) {
        const int u = sub + LANES * j;
        U v = {};
        if (rv && u < units) v = load(u);
        ring[j] = v;
    }
}

// LDS: [0, stage_bytes) staging area (x for phase A or encoded mid for phase
// B), then the residual f32 [hidden], the gate/up results [2 * max rows],
// reduction scratch.
struct ChainLds {
    uint8_t *stage;
    float *res;
    float *gu;
    float *red;
    int *flag;
};

template <int LA, int DOWN_QT>
__global__ __launch_bounds__(kChainThreads) void ffn_chain_kernel(ChainArgs a, int stage_bytes,
                                                                  int max_rows_a)
{
    extern __shared__ __align__(16) uint8_t smem[];
    ChainLds L;
    L.stage = smem;
    L.res = reinterpret_cast<float *>(smem + stage_bytes);
    L.gu = L.res + a.hidden;
    L.red = L.gu + 2 * max_rows_a;
    L.flag = reinterpret_cast<int *>(L.red + 16);

    const __amdgpu_buffer_rsrc_t rs = ws_rsrc(a);
    constexpr int GD = DOWN_QT == 2 ? 16 : 32;  // down projection's scale group
    const int H = a.hidden, F = a.ffn;
    const int G = gridDim.x, w = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h4 = H >> 2;

    // phase A rows: whole GD-row groups of mid, split evenly over workgroups
    const int ngrp = F / GD;
    const int ra = (int)((int64_t)w * ngrp / G) * GD;
    const int rb = (int)((int64_t)(w + 1) * ngrp / G) * GD;
    const int na = rb - ra;
    // phase B rows of the down projection
    const int pa = (int)((int64_t)w * H / G), pb = (int)((int64_t)(w + 1) * H / G);

    const int nsb_a = H >> 8, units_a = 2 * nsb_a;
    const int64_t rowb_a = (int64_t)nsb_a * 144;
    const int nsb_b = F >> 8, units_b = 2 * nsb_b;
    constexpr int BB = DOWN_QT == 2 ? 210 : 144;
    const int64_t rowb_b = (int64_t)nsb_b * BB;

    // this lane's phase-A task (tile = wave, tiles stride kChainWaves)
    constexpr int RPTA = 64 / LA;
    const int sub_a = lane % LA, ha = sub_a & 1;
    constexpr int RPTB = 64 / kPhaseBLanes;
    const int sub_b = lane % kPhaseBLanes, hb = sub_b & 1;

    // ---- the per-layer pointer tables live in device memory, so they are
    // checked here: every workgroup reads the same table and takes the same
    // decision, so a bad table makes all of them leave before any barrier.
    if (threadIdx.x == 0) {
        int good = 1;
        for (int l = 0; l < a.layers; ++l) {
            const uintptr_t g = (uintptr_t)a.wg[l], u = (uintptr_t)a.wu[l], d = (uintptr_t)a.wd[l];
            const uintptr_t p = (uintptr_t)a.gpost[l], n = (uintptr_t)a.gnext[l];
            good &= g && u && d && p && n && !(g & 15) && !(u & 15) &&
                    !(d & (DOWN_QT == 2 ? 3 : 15)) && !(p & 15) && !(n & 15);
        }
        *L.flag = good;
        if (!good && w == 0) st_agent(a.bar + 2, 2u);
    }
    __syncthreads();
    if (!*L.flag) return;

    // ---- prologue: residual and x_0 into LDS
    for (int i = threadIdx.x; i < H; i += blockDim.x) L.res[i] = a.residual[i];
    stage_activation<32, KQ_LIMBS>(a.x_in, H, L.stage);
    __syncthreads();

    uint32_t epoch = 0;
    bool ok = true;
    Q4Unit ringA[kQ4Look];
    using UB = typename std::conditional<DOWN_QT == 2, Q6Unit, Q4Unit>::type;
    UB ringB[kQ6Look];

    auto task_row = [&](int tile, int &which, int &row) -> bool {
        const int t = tile * RPTA + lane / LA;
        which = t < na ? 0 : 1;
        row = ra + (t < na ? t : t - na);
        return t < 2 * na;
    };
    auto loadA_for = [&](int layer, int tile, bool enable = true) {
        int which, row;
        const bool rv = task_row(tile, which, row) && enable;
        const uint8_t *base = which ? a.wu[layer] : a.wg[layer];
        const uint8_t *rowp = base + (int64_t)(rv ? row : ra) * rowb_a;
        prefill<LA, kQ4Look>(ringA, sub_a, units_a, rv, [&](int u) {
            return q4_load(rowp + (int64_t)(u >> 1) * 144, ha);
        });
    };
    auto loadB_for = [&](int layer, int tile) {
        const int r = pa + tile * RPTB + lane / kPhaseBLanes;
        const bool rv = r < pb;
        const uint8_t *rowp = a.wd[layer] + (int64_t)(rv ? r : pa) * rowb_b;
        prefill<kPhaseBLanes, kQ6Look>(ringB, sub_b, units_b, rv, [&](int u) {
            if constexpr (DOWN_QT == 2)
                return q6_load(rowp + (int64_t)(u >> 1) * 210, hb);
            else
                return q4_load(rowp + (int64_t)(u >> 1) * 144, hb);
        });
    };

    const int tiles_a = (2 * na + RPTA - 1) / RPTA;
    const int tiles_b = (pb - pa + RPTB - 1) / RPTB;
    loadA_for(0, wave);

    for (int l = 0; l < a.layers && ok; ++l) {
        // ---------------- phase A: gate and up rows, mid for [ra, rb)
        {
            const uint8_t *planes = L.stage;
            const float *tscale = reinterpret_cast<const float *>(L.stage + KQ_LIMBS * plane_bytes(H));
            const float *tsum = tscale + (H >> 5);
            for (int tile = wave; tile < tiles_a; tile += kChainWaves) {
                if (tile != wave) loadA_for(l, tile);
                int which, row;
                const bool rv = task_row(tile, which, row);
                const uint8_t *base = which ? a.wu[l] : a.wg[l];
                const uint8_t *rowp = base + (int64_t)(rv ? row : ra) * rowb_a;
                float acc = row_share<LA, kQ4Look>(
                    ringA, sub_a, units_a, rv,
                    [&](int u) { return q4_load(rowp + (int64_t)(u >> 1) * 144, ha); },
                    [&](const Q4Unit &un, int u) {
                        return q4_unit_dot<KQ_LIMBS>(un, ha, 256 * (u >> 1) + 128 * ha, H, planes,
                                                     tscale, tsum);
                    });
                acc = lane_group_sum<LA>(acc);
                if (sub_a == 0 && rv) L.gu[which * max_rows_a + (row - ra)] = acc;
            }
            __syncthreads();
            // mid = silu(g) * u for this workgroup's rows, encoded for phase B
            for (int i = threadIdx.x; i < (na >> 2); i += blockDim.x) {
                f32x4 m;
                float *mm = reinterpret_cast<float *>(&m);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float g = L.gu[4 * i + j], u = L.gu[max_rows_a + 4 * i + j];
                    mm[j] = (g / (1.0f + __expf(-g))) * u;
                }
                encode_group_global<GD>(m, (ra >> 2) + i, a.enc, F);
            }
            stores_done();
            loadB_for(l, wave);
            ok = grid_barrier(a.bar, ++epoch, L.flag);
            if (!ok) break;
        }
        // ---------------- phase B: copy the encoded mid, rows [pa, pb) of p
        {
            const int enc16 = (int)((KQ_LIMBS * plane_bytes(F) + 8 * (F / GD)) >> 4);
            const uint32_t enc_off = (uint32_t)((uint8_t *)a.enc - a.ws);
            u32x4 *dst = reinterpret_cast<u32x4 *>(L.stage);
            for (int i0 = threadIdx.x; i0 < enc16; i0 += 4 * kChainThreads) {
                u32x4 v[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int i = i0 + j * kChainThreads;
                    if (i < enc16) v[j] = ld_agent16(rs, enc_off + 16u * i);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int i = i0 + j * kChainThreads;
                    if (i < enc16) dst[i] = v[j];
                }
            }
            __syncthreads();
            const uint8_t *planes = L.stage;
            const float *tscale = reinterpret_cast<const float *>(L.stage + KQ_LIMBS * plane_bytes(F));
            const float *tsum = tscale + F / GD;
            for (int tile = wave; tile < tiles_b; tile += kChainWaves) {
                if (tile != wave) loadB_for(l, tile);
                const int r = pa + tile * RPTB + lane / kPhaseBLanes;
                const bool rv = r < pb;
                const uint8_t *rowp = a.wd[l] + (int64_t)(rv ? r : pa) * rowb_b;
                float acc = row_share<kPhaseBLanes, kQ6Look>(
                    ringB, sub_b, units_b, rv,
                    [&](int u) {
                        if constexpr (DOWN_QT == 2)
                            return q6_load(rowp + (int64_t)(u >> 1) * 210, hb);
                        else
                            return q4_load(rowp + (int64_t)(u >> 1) * 144, hb);
                    },
                    [&](const UB &un, int u) {
                        if constexpr (DOWN_QT == 2)
                            return q6_unit_dot<KQ_LIMBS>(un, 256 * (u >> 1) + 128 * hb, F, planes,
                                                         tscale, tsum);
                        else
                            return q4_unit_dot<KQ_LIMBS>(un, hb, 256 * (u >> 1) + 128 * hb, F,
                                                         planes, tscale, tsum);
                    });
                acc = lane_group_sum<kPhaseBLanes>(acc);
                if (sub_b == 0 && rv) st_agent(a.p + r, acc);
            }
            stores_done();
            // unconditional (loads disabled after the last layer): keeps the
            // ring's live range inside phase A
            loadA_for(l + 1 < a.layers ? l + 1 : l, wave, l + 1 < a.layers);
            ok = grid_barrier(a.bar, ++epoch, L.flag);
            if (!ok) break;
        }
        // ---------------- phase C: the tail, whole row, in every workgroup
        {
            const f32x4 *gp4 = reinterpret_cast<const f32x4 *>(a.gpost[l]);
            const f32x4 *gn4 = reinterpret_cast<const f32x4 *>(a.gnext[l]);
            f32x4 *res4 = reinterpret_cast<f32x4 *>(L.res);
            const float inv_n = 1.0f / (float)H;
            const uint32_t p_off = (uint32_t)((uint8_t *)a.p - a.ws);
            f32x4 pv[kPv];
#pragma unroll
            for (int j = 0; j < kPv; ++j) {
                const int i = threadIdx.x + j * kChainThreads;
                const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
                pv[j] = i < h4 ? __builtin_bit_cast(f32x4, ld_agent16(rs, p_off + 16u * i)) : z;
            }
            float ss = 0.0f;
#pragma unroll
            for (int j = 0; j < kPv; ++j)
                ss += pv[j].x * pv[j].x + pv[j].y * pv[j].y + pv[j].z * pv[j].z + pv[j].w * pv[j].w;
            ss = block_sum_fixed(ss, L.red);
            const float inv_p = rsqrtf(ss * inv_n + a.eps_post);
            float sr = 0.0f;
#pragma unroll
            for (int j = 0; j < kPv; ++j) {
                const int i = threadIdx.x + j * kChainThreads;
                if (i < h4) {
                    const f32x4 v = res4[i] + (pv[j] * inv_p) * gp4[i];
                    res4[i] = v;
                    sr += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
                }
            }
            sr = block_sum_fixed(sr, L.red);
            const float inv_r = rsqrtf(sr * inv_n + a.eps_next);
            uint32_t *plane = reinterpret_cast<uint32_t *>(L.stage);
            float *tscale = reinterpret_cast<float *>(L.stage + KQ_LIMBS * plane_bytes(H));
            float *tsum = tscale + (H >> 5);
            const bool last = l + 1 == a.layers;
            for (int i = threadIdx.x; i < h4; i += blockDim.x) {
                const f32x4 xv = (res4[i] * inv_r) * gn4[i];
                if (last) {
                    if (w == 0) reinterpret_cast<f32x4 *>(a.x_out)[i] = xv;
                } else {
                    stage_group<32, KQ_LIMBS>(xv, i, plane, h4, tscale, tsum);
                }
            }
            __syncthreads();
        }
    }

    if (w == 0 && ok)
        for (int i = threadIdx.x; i < H; i += blockDim.x) a.residual[i] = L.res[i];
    // exit: the last workgroup out resets the control block for the next launch
    if (threadIdx.x == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const uint32_t prev =
            __hip_atomic_fetch_add(a.bar + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (prev + 1 == gridDim.x) {
            st_agent(a.bar, 0u);
            st_agent(a.bar + 1, 0u);
            st_agent(a.bar + kCtlTop, 0u);
            for (int g = 0; g < kMaxGroups; ++g) st_agent(a.bar + 32 * (1 + g), 0u);
        }
    }
}

size_t chain_stage_bytes(int hidden, int ffn, int down_qt)
{
    const int gd = down_qt == 2 ? 16 : 32;
    const size_t sa = (size_t)KQ_LIMBS * plane_bytes(hidden) + 8 * (size_t)(hidden / 32);
    const size_t sb = (size_t)KQ_LIMBS * plane_bytes(ffn) + 8 * (size_t)(ffn / gd);
    return ((sa > sb ? sa : sb) + 15) & ~(size_t)15;
}

template <int LA, int DQ>
hipError_t launch_chain_cfg(const ChainArgs &a, int grid, size_t lds, int stage, int max_rows_a,
                            hipStream_t stream)
{
    constexpr auto kern = ffn_chain_kernel<LA, DQ>;
    static int attr_done = 0;
    if (!attr_done) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
        attr_done = 1;
    }
    ChainArgs args = a;
    void *params[] = {&args, &stage, &max_rows_a};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void *>(kern), dim3(grid),
                                      dim3(kChainThreads), params, (unsigned)lds, stream);
}

int g_chain_lanes_a = 4;

}  // namespace

namespace kqi {

constexpr size_t kCtlBytes = ((size_t)4 * kCtlWords + 255) & ~(size_t)255;

size_t chain_workspace_bytes(int64_t hidden, int64_t ffn, int down_qtype)
{
    const int gd = down_qtype == 2 ? 16 : 32;
    const size_t enc = (size_t)KQ_LIMBS * plane_bytes(ffn) + 8 * (size_t)(ffn / gd);
    return kCtlBytes + ((enc + 255) & ~(size_t)255) + (((size_t)hidden * 4 + 255) & ~(size_t)255);
}

size_t chain_lds_bytes(int64_t hidden, int64_t ffn, int down_qtype, int grid)
{
    const int gd = down_qtype == 2 ? 16 : 32;
    const int64_t ngrp = ffn / gd;
    const int64_t max_rows_a = ((ngrp + grid - 1) / grid) * gd;
    return chain_stage_bytes((int)hidden, (int)ffn, down_qtype) + 4 * (size_t)hidden +
           8 * (size_t)max_rows_a + 64 + 16;
}

int chain_grid()
{
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    return cus > 0 ? cus : 256;
}

void set_chain_lanes(int lanes) { g_chain_lanes_a = lanes; }

hipError_t launch_ffn_chain(const uint8_t *const *wg, const uint8_t *const *wu,
                            const uint8_t *const *wd, int down_qtype, const float *const *gpost,
                            const float *const *gnext, int layers, int hidden, int ffn,
                            const float *x_in, float *residual, float *x_out, float eps_post,
                            float eps_next, void *workspace, hipStream_t stream)
{
    const int grid = chain_grid();
    if (grid > kBarGroup * kMaxGroups) return hipErrorInvalidValue;
    const int gd = down_qtype == 2 ? 16 : 32;
    const int ngrp = ffn / gd;
    const int max_rows_a = ((ngrp + grid - 1) / grid) * gd;
    const int stage = (int)chain_stage_bytes(hidden, ffn, down_qtype);
    const size_t lds = chain_lds_bytes(hidden, ffn, down_qtype, grid);
    if (lds > 160 * 1024) return hipErrorInvalidValue;
    const size_t enc = (size_t)KQ_LIMBS * plane_bytes(ffn) + 8 * (size_t)(ffn / gd);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    ChainArgs a;
    a.wg = wg;
    a.wu = wu;
    a.wd = wd;
    a.gpost = gpost;
    a.gnext = gnext;
    a.x_in = x_in;
    a.residual = residual;
    a.x_out = x_out;
    a.bar = reinterpret_cast<uint32_t *>(ws);
    a.ws = ws;
    a.ws_bytes = (uint32_t)chain_workspace_bytes(hidden, ffn, down_qtype);
    a.enc = reinterpret_cast<uint32_t *>(ws + kCtlBytes);
    a.p = reinterpret_cast<float *>(ws + kCtlBytes + ((enc + 255) & ~(size_t)255));
    a.layers = layers;
    a.hidden = hidden;
    a.ffn = ffn;
    a.eps_post = eps_post;
    a.eps_next = eps_next;
    const int la = g_chain_lanes_a;
#define KQ_CH(LA)                                                                             \
    if (la == LA)                                                                             \
        return down_qtype == 2 ? launch_chain_cfg<LA, 2>(a, grid, lds, stage, max_rows_a, stream) \
                               : launch_chain_cfg<LA, 1>(a, grid, lds, stage, max_rows_a, stream);
    KQ_CH(2)
    KQ_CH(4)
    KQ_CH(8)
#undef KQ_CH
    return hipErrorInvalidValue;
}

}  // namespace kqi

/*
 * kq_oracle.c -- CPU oracle for the k-quant decode matvec path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The product path
 * (the HIP library under quant_weight_matvec_amd/) never calls it, and this
 * file shares no code, header, table or constant with that library.
 *
 * Source: "How to Write an Inference Engine -- the Muser book".  Everything is
 * computed in IEEE binary64 with plain loops in the order the definitions
 * state it; there is no blocking, fusion or reordering.  Each function names
 * the passage it follows.
 *
 * Reading of the superblock layouts.  The chapter that defines the Q4_K and
 * Q6_K bit packing (Ch 6) is not among the pages.  The pages fix only the sizes
 * (Ch 19 "The down projection + residual", section 19.3: 256 weights in 144 B
 * for Q4_K and in 210 B for Q6_K), the block idea "scale x index (+ min)"
 * (Ch 5 "Quantization from scratch", section 5.5) and integer codebooks
 * (Ch 5, section 5.3).  The packing used here is the common k-quant one:
 *
 *   Q4_K: d f16 | dmin f16 | 12 B of packed 6-bit (scale, min) pairs for
 *         8 sub-blocks of 32 | 128 B of nibbles.
 *         weight = d * scale_s * q - dmin * min_s   (the min is subtracted).
 *   Q6_K: 128 B low 4 bits | 64 B high 2 bits | 16 int8 scales (sub-blocks of
 *         16) | d f16.   weight = d * scale_s * (q - 32).
 *   Q5_K: d f16 | dmin f16 | 12 B of 6-bit (scale, min) pairs packed as in
 *         Q4_K | 32 B of high bits | 128 B of low nibbles (176 B; the pages
 *         name the type, in the pinned decode kernels of Ch 4 "Pipeline state
 *         objects and the three kernel sources", section 4.4, but give no
 *         layout).  Weight i of chunk c = i / 64: low 4 bits as the Q4_K
 *         nibble of the same position, high bit = bit 2c (first 32 of the
 *         chunk) or 2c+1 (last 32) of high-bit byte i mod 32; q = 0..31.
 *         weight = d * scale_s * q - dmin * min_s.
 *
 * Parity against external k-quant producers is unpinned (no external file or
 * decoder is available); the tests pin this reading by one-hot brute force,
 * closed forms and exact integer arithmetic.
 *
 * Planted mistakes: compiling with -DORC_PLANT=n (n > 0) swaps in one
 * deliberate error so a CPU test can show that the pins catch it.  The
 * default build (ORC_PLANT == 0) contains none of them.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORC_PLANT
#define ORC_PLANT 0
#endif

#define ORC_QK 256
#define ORC_Q4K_BYTES 144
#define ORC_Q6K_BYTES 210
#define ORC_Q5K_BYTES 176
#define ORC_QTYPE_Q4K 1
#define ORC_QTYPE_Q6K 2
#define ORC_QTYPE_Q5K 3

/* ------------------------------------------------------------------------ */
/* binary16 decode.  IEEE 754 half: 1 sign bit, 5 exponent bits with bias 15,
 * 10 fraction bits; exponent 0 = zero/subnormal, 31 = inf/NaN.  Ch 5
 * "Quantization from scratch", section 5.2 (Figure 5.3, the f16 layout). */
double orc_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
#if ORC_PLANT == 10
    const int bias = 16;
#else
    const int bias = 15;
#endif
    if (e == 0)
        v = ldexp((double)f, 1 - bias - 10);          /* 0.f * 2^(1-bias) */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - bias - 10); /* 1.f * 2^(e-bias) */
    return sign ? -v : v;
}

static double rd_f16(const uint8_t *p)
{
    return orc_f16_to_f64((uint16_t)(p[0] | (p[1] << 8)));
}

/* ------------------------------------------------------------------------ */
/* Q4_K superblock -> 256 weights.  Block semantics "scale x index + min"
 * (Ch 5, section 5.5, asymmetric form), 144-byte superblock (Ch 19, section
 * 19.3); field packing as stated in the header comment. */
void orc_dequant_q4k(const uint8_t *blk, double *w)
{
    const double d = rd_f16(blk + 0);
    const double dmin = rd_f16(blk + 2);
    const uint8_t *S = blk + 4;    /* 12 bytes of packed 6-bit fields */
    const uint8_t *qs = blk + 16;  /* 128 bytes of nibbles */
    int sc[8], mn[8];
    for (int s = 0; s < 4; ++s) {
        sc[s] = S[s] & 63;
        mn[s] = S[s + 4] & 63;
    }
    for (int s = 4; s < 8; ++s) {
#if ORC_PLANT == 3
        sc[s] = (S[s + 4] & 15) | ((S[s] >> 6) << 4);
#else
        sc[s] = (S[s + 4] & 15) | ((S[s - 4] >> 6) << 4);
#endif
        mn[s] = (S[s + 4] >> 4) | ((S[s] >> 6) << 4);
    }
    for (int i = 0; i < ORC_QK; ++i) {
        int c = i / 64, t = i % 64;
        int byte = qs[32 * c + (t % 32)];
        int q = (t < 32) ? (byte & 15) : (byte >> 4);
#if ORC_PLANT == 2
        int s = 2 * c;             /* high nibbles wrongly on the low sub-block */
#else
        int s = i / 32;
#endif
#if ORC_PLANT == 1
        w[i] = d * sc[s] * q + dmin * mn[s];
#else
        w[i] = d * sc[s] * q - dmin * mn[s];
#endif
    }
}

/* ------------------------------------------------------------------------ */
/* Q6_K superblock -> 256 weights.  Symmetric "scale x index" with the 6-bit
 * index centred by 32 (Ch 5, section 5.5; 210-byte superblock, Ch 19, section
 * 19.3); field packing as stated in the header comment. */
void orc_dequant_q6k(const uint8_t *blk, double *w)
{
    const uint8_t *ql = blk;
    const uint8_t *qh = blk + 128;
    const int8_t *sc = (const int8_t *)(blk + 192);
    const double d = rd_f16(blk + 208);
    for (int i = 0; i < ORC_QK; ++i) {
        int h = i / 128, t = i % 128;
        int j = t % 32, g = t / 32;
        int lob = ql[64 * h + 32 * (g % 2) + j];
        int lo = (g < 2) ? (lob & 15) : (lob >> 4);
#if ORC_PLANT == 4
        int hi = (qh[32 * h + j] >> g) & 3;
#else
        int hi = (qh[32 * h + j] >> (2 * g)) & 3;
#endif
        int q = lo | (hi << 4);
#if ORC_PLANT == 5
        w[i] = d * sc[i / 16] * q;
#elif ORC_PLANT == 6
        w[i] = d * sc[i / 32] * (q - 32);
#else
        w[i] = d * sc[i / 16] * (q - 32);
#endif
    }
}

/* ------------------------------------------------------------------------ */
/* Q5_K superblock -> 256 weights.  The asymmetric "scale x index - min" of
 * Q4_K with a 5-bit index (Ch 5, section 5.5); field packing as stated in the
 * header comment. */
void orc_dequant_q5k(const uint8_t *blk, double *w)
{
    const double d = rd_f16(blk + 0);
    const double dmin = rd_f16(blk + 2);
    const uint8_t *S = blk + 4;    /* 12 bytes of packed 6-bit fields */
    const uint8_t *qh = blk + 16;  /* 32 bytes of high bits */
#if ORC_PLANT == 16
    const uint8_t *qs = blk + 32;  /* low nibbles read from the wrong offset */
#else
    const uint8_t *qs = blk + 48;  /* 128 bytes of low nibbles */
#endif
    int sc[8], mn[8];
    for (int s = 0; s < 4; ++s) {
        sc[s] = S[s] & 63;
        mn[s] = S[s + 4] & 63;
    }
    for (int s = 4; s < 8; ++s) {
        sc[s] = (S[s + 4] & 15) | ((S[s - 4] >> 6) << 4);
        mn[s] = (S[s + 4] >> 4) | ((S[s] >> 6) << 4);
    }
    for (int i = 0; i < ORC_QK; ++i) {
        int c = i / 64, t = i % 64, j = t % 32;
        int byte = qs[32 * c + j];
        int lo = (t < 32) ? (byte & 15) : (byte >> 4);
#if ORC_PLANT == 14
        int bit = c;                          /* one bit per chunk, not two */
#else
        int bit = 2 * c + (t >= 32 ? 1 : 0);
#endif
        int hi = (qh[j] >> bit) & 1;
#if ORC_PLANT == 15
        int q = lo | (hi << 5);
#else
        int q = lo | (hi << 4);
#endif
        int s = i / 32;
        w[i] = d * sc[s] * q - dmin * mn[s];
    }
}

static int64_t orc_block_bytes(int qtype)
{
    return qtype == ORC_QTYPE_Q4K ? ORC_Q4K_BYTES
         : qtype == ORC_QTYPE_Q6K ? ORC_Q6K_BYTES
         : qtype == ORC_QTYPE_Q5K ? ORC_Q5K_BYTES : 0;
}

static void orc_dequant_block(int qtype, const uint8_t *blk, double *w)
{
    if (qtype == ORC_QTYPE_Q4K) orc_dequant_q4k(blk, w);
    else if (qtype == ORC_QTYPE_Q6K) orc_dequant_q6k(blk, w);
    else orc_dequant_q5k(blk, w);
}

int orc_dequant_rows(int qtype, const uint8_t *W, int64_t n_rows, int64_t k, double *out)
{
    if (k % ORC_QK) return -2;
    int64_t nsb = k / ORC_QK;
    int64_t bb = orc_block_bytes(qtype);
    if (!bb) return -5;
    for (int64_t r = 0; r < n_rows; ++r)
        for (int64_t b = 0; b < nsb; ++b) {
            const uint8_t *blk = W + (r * nsb + b) * bb;
            double *dst = out + r * k + b * ORC_QK;
            orc_dequant_block(qtype, blk, dst);
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Matvec and small-M matmul.  y = W x with one output per weight row (Ch 1
 * "The problem: why inference is a memory problem", section 1.3 step 4; Ch 19,
 * section 19.1 operation 1).  W has n_rows outputs and k inputs; row r is
 * k/256 consecutive superblocks and superblock b covers inputs 256b..256b+255.
 * For M rows of activations, Y[m] = W X[m] (Ch 36 "Prefill vs decode",
 * section 36.4: each weight row used once per activation row).  Alongside y
 * the oracle returns S = sum_i |w_i x_i|, the scale of the tolerance. */
typedef struct {
    int qtype;
    const uint8_t *W;
    const double *X;
    int64_t ldx, n_rows, k, m;
    double *Y, *S;
    int64_t r0, r1;
} orc_mm_job;

static void *orc_mm_worker(void *arg)
{
    orc_mm_job *J = (orc_mm_job *)arg;
    const int64_t nsb = J->k / ORC_QK;
    const int64_t bb = orc_block_bytes(J->qtype);
    double w[ORC_QK];
    for (int64_t r = J->r0; r < J->r1; ++r) {
        for (int64_t mm = 0; mm < J->m; ++mm) {
            J->Y[mm * J->n_rows + r] = 0.0;
            J->S[mm * J->n_rows + r] = 0.0;
        }
#if ORC_PLANT == 11
        for (int64_t b = 0; b + 1 < nsb || (nsb == 1 && b < 1); ++b) {
#else
        for (int64_t b = 0; b < nsb; ++b) {
#endif
            const uint8_t *blk = J->W + (r * nsb + b) * bb;
            orc_dequant_block(J->qtype, blk, w);
            for (int64_t mm = 0; mm < J->m; ++mm) {
                const double *x = J->X + mm * J->ldx + b * ORC_QK;
                double acc = J->Y[mm * J->n_rows + r];
                double sab = J->S[mm * J->n_rows + r];
                for (int i = 0; i < ORC_QK; ++i) {
#if ORC_PLANT == 12
                    double p = w[i] * x[ORC_QK - 1 - i];
#else
                    double p = w[i] * x[i];
#endif
                    acc += p;
                    sab += fabs(p);
                }
                J->Y[mm * J->n_rows + r] = acc;
                J->S[mm * J->n_rows + r] = sab;
            }
        }
    }
    return NULL;
}

/* Y is [m][n_rows], S is [m][n_rows].  Returns 0, or a negative code on bad
 * arguments.  nthreads <= 1 runs on the calling thread. */
int orc_matmul(int qtype, const uint8_t *W, const double *X, int64_t ldx,
               int64_t n_rows, int64_t k, int64_t m, double *Y, double *S, int nthreads)
{
    if (!orc_block_bytes(qtype)) return -5;
    if (k <= 0 || k % ORC_QK || n_rows < 0 || m < 1 || ldx < k) return -2;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (n_rows < nthreads) nthreads = n_rows > 0 ? (int)n_rows : 1;
    orc_mm_job jobs[256];
    pthread_t th[256];
    int started[256];
    /* Rows are split into contiguous ranges, one per thread.  Every row is
     * computed by exactly one job in the same order whatever the thread
     * count, so the results do not depend on it. */
    for (int t = 0; t < nthreads; ++t) {
#if ORC_PLANT == 13
        int64_t r1 = n_rows * (t + 1) / nthreads;
        if (t + 1 < nthreads && r1 > n_rows * t / nthreads) --r1; /* drops a row per range */
        jobs[t] = (orc_mm_job){qtype, W, X, ldx, n_rows, k, m, Y, S, n_rows * t / nthreads, r1};
#else
        jobs[t] = (orc_mm_job){qtype, W, X, ldx, n_rows, k, m, Y, S,
                               n_rows * t / nthreads, n_rows * (t + 1) / nthreads};
#endif
    }
    if (nthreads == 1) {
        orc_mm_worker(&jobs[0]);
        return 0;
    }
    /* a job whose thread cannot be started runs on the calling thread */
    for (int t = 0; t < nthreads; ++t)
        started[t] = pthread_create(&th[t], NULL, orc_mm_worker, &jobs[t]) == 0;
    for (int t = 0; t < nthreads; ++t)
        if (!started[t]) orc_mm_worker(&jobs[t]);
    for (int t = 0; t < nthreads; ++t)
        if (started[t]) pthread_join(th[t], NULL);
    return 0;
}

int orc_matvec(int qtype, const uint8_t *W, const double *x, int64_t n_rows, int64_t k,
               double *y, double *S, int nthreads)
{
    return orc_matmul(qtype, W, x, k, n_rows, k, 1, y, S, nthreads);
}

/* ------------------------------------------------------------------------ */
/* SiLU-gated product: mid = silu(gate) * up with silu(z) = z * sigma(z) and
 * sigma(z) = 1 / (1 + e^-z) (the logistic function as Ch 2 "The Metal compute
 * model", section 2.7 writes it for the attention-output gate; silu-times-up is the
 * FFN step of Ch 10 "The forward pass at a glance", section 10.3, box 11).
 * For z very negative, e^-z overflows to +inf and sigma becomes 0. */
void orc_silu_mul(const double *gate, const double *up, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i) {
        double z = gate[i];
        double sig = 1.0 / (1.0 + exp(-z));
#if ORC_PLANT == 9
        (void)sig;
        out[i] = z * up[i];
#else
        out[i] = z * sig * up[i];
#endif
    }
}

/* ------------------------------------------------------------------------ */
/* RMSNorm: out_i = x_i / sqrt(mean(x^2) + eps) * gain_i (gain NULL = ones).
 * The epsilon is added to the mean inside the root and the gain multiplies
 * after normalising (Ch 19, section 19.4, passes 1 and 3; the weightless entry
 * norm with eps 1e-5 is box 2 of Ch 10, section 10.3). */
void orc_rms_norm(const double *x, int64_t n, double eps, const double *gain, double *out)
{
    double ss = 0.0;
    for (int64_t i = 0; i < n; ++i) ss += x[i] * x[i];
#if ORC_PLANT == 7
    double inv = 1.0 / (sqrt(ss / (double)n) + eps);
#else
    double inv = 1.0 / sqrt(ss / (double)n + eps);
#endif
    for (int64_t i = 0; i < n; ++i) out[i] = x[i] * inv * (gain ? gain[i] : 1.0);
}

/* ------------------------------------------------------------------------ */
/* Dual-epsilon residual tail, rows independent (Ch 19, section 19.1
 * operation 2 and section 19.4; Ch 10, section 10.4, Figure 10.2):
 *   residual += rms_norm(projected, eps_post) * g_post
 *   next_in   = rms_norm(residual, eps_next) * g_next
 * The second norm sees the residual after the add.  residual is [rows][n],
 * updated in place; g_post and g_next are [n], shared by all rows. */
void orc_dual_eps_tail(double *residual, const double *projected, const double *g_post,
                       const double *g_next, int64_t rows, int64_t n, double eps_post,
                       double eps_next, double *next_in)
{
    double *a = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (int64_t r = 0; r < rows; ++r) {
        double *res = residual + r * n;
        orc_rms_norm(projected + r * n, n, eps_post, g_post, a);
#if ORC_PLANT == 8
        orc_rms_norm(res, n, eps_next, g_next, next_in + r * n);
        for (int64_t i = 0; i < n; ++i) res[i] += a[i];
#else
        for (int64_t i = 0; i < n; ++i) res[i] += a[i];
        orc_rms_norm(res, n, eps_next, g_next, next_in + r * n);
#endif
    }
    free(a);
}

/* ------------------------------------------------------------------------ */
/* One FFN layer of the decode chain (Ch 10, section 10.3, boxes 11-13; Ch 19,
 * section 19.1): g = Wg x, u = Wu x, mid = silu(g) * u, p = Wd mid, then the
 * dual-eps tail with this layer's gains.  x is [hidden], residual [hidden]
 * (in/out), next_in [hidden]; g, u, mid are [ffn], p is [hidden].  The
 * optional outputs (g, u, mid, p, and the S of each matvec) may be NULL. */
int orc_ffn_layer(int qt_gate, const uint8_t *Wg, int qt_up, const uint8_t *Wu,
                  int qt_down, const uint8_t *Wd, int64_t hidden, int64_t ffn,
                  const double *x, double *residual, const double *g_post,
                  const double *g_next, double eps_post, double eps_next, double *next_in,
                  double *g_out, double *u_out, double *mid_out, double *p_out,
                  double *sg_out, double *su_out, double *sp_out, int nthreads)
{
    double *g = (double *)malloc(sizeof(double) * (size_t)ffn);
    double *u = (double *)malloc(sizeof(double) * (size_t)ffn);
    double *mid = (double *)malloc(sizeof(double) * (size_t)ffn);
    double *p = (double *)malloc(sizeof(double) * (size_t)hidden);
    double *s1 = (double *)malloc(sizeof(double) * (size_t)ffn);
    double *s2 = (double *)malloc(sizeof(double) * (size_t)ffn);
    double *s3 = (double *)malloc(sizeof(double) * (size_t)hidden);
    int rc = orc_matvec(qt_gate, Wg, x, ffn, hidden, g, s1, nthreads);
    if (!rc) rc = orc_matvec(qt_up, Wu, x, ffn, hidden, u, s2, nthreads);
    if (!rc) {
        orc_silu_mul(g, u, ffn, mid);
        rc = orc_matvec(qt_down, Wd, mid, hidden, ffn, p, s3, nthreads);
    }
    if (!rc) {
        orc_dual_eps_tail(residual, p, g_post, g_next, 1, hidden, eps_post, eps_next, next_in);
        if (g_out) memcpy(g_out, g, sizeof(double) * (size_t)ffn);
        if (u_out) memcpy(u_out, u, sizeof(double) * (size_t)ffn);
        if (mid_out) memcpy(mid_out, mid, sizeof(double) * (size_t)ffn);
        if (p_out) memcpy(p_out, p, sizeof(double) * (size_t)hidden);
        if (sg_out) memcpy(sg_out, s1, sizeof(double) * (size_t)ffn);
        if (su_out) memcpy(su_out, s2, sizeof(double) * (size_t)ffn);
        if (sp_out) memcpy(sp_out, s3, sizeof(double) * (size_t)hidden);
    }
    free(g); free(u); free(mid); free(p); free(s1); free(s2); free(s3);
    return rc;
}

int orc_plant(void) { return ORC_PLANT; }

/*
 * starkv_oracle.c -- plain fp64 CPU oracle for STAR-KV decode attention over a low-rank latent
 * KV cache, and for the cache's optional rotation + mixed 4/3-bit quantisation.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test-suite, the smoke check and the benchmark's CPU-baseline
 * leg load this library. It shares no code, header, table or helper with the HIP library under
 * rank_kv_cache_amd/; the two only ever see the same seeded input arrays.
 *
 * What it computes, and from which passage of the STAR-KV pages (cited by page title + section):
 *
 *  - Latent caches: keys are stored per head as pre-RoPE latents Z_k[h] (T x r_h) with a constant
 *    up factor B_k[h] (r_h x d); values are one joint latent Z_v (T x r_v) shared by all heads,
 *    with up factor B_v (r_v x H*d) whose columns [h*d, (h+1)*d) belong to head h.
 *    (Zhou, "STAR-KV reading notes", sections 2.2, 5.1 and 5.3; gist.science explainer,
 *    "Technisches Resuemee", Methodik 2.)
 *  - Decode attention (same notes, Algorithm 2 steps 4-7): for every cached position n the key
 *    K~_n = Z_k[h][n] B_k[h] is rebuilt, rotated with LLaMA rotate-half RoPE at position n, scored
 *    against the (already rotated) query, softmax-normalised over n, and the value side is summed
 *    in latent space first and projected by B_v^h afterwards (section 5.3: the exact reordering
 *    P_h (Z_v B_v^h) = (P_h Z_v) B_v^h). Both orders are implemented (form 0 latent, 1 explicit).
 *  - Dense exempt layers (same notes, section 4 / Algorithm 1 step 2): ordinary RoPE attention on
 *    full-width pre-RoPE K and V; the identity-factor special case of the above.
 *  - Blockwise Hadamard rotation (same notes, section 6.1 / Fig. 5; gist.science Methodik 3):
 *    latent channels split into a high-magnitude block and the rest, each rotated by an orthogonal
 *    block-diagonal Sylvester-Hadamard matrix; Z B = (Z H)(H^T B).
 *  - Mixed-precision quantisation (same notes, section 6.1; model card "calibration recipe":
 *    top fraction 0.25 at 4 bits, the rest at 3 bits): asymmetric, per channel, per 64-token group,
 *    fp16 scale and zero point.
 *
 * Readings where the pages are silent (RoPE convention, query position, softmax scale, the
 * quantiser's rounding rule, the packed byte layout, the Hadamard block size) are each stated
 * next to the function that implements it.
 *
 * Parity pins (tests/test_oracle_pins.py): every function here is checked against something
 * other than itself -- closed forms, library routines, brute force in 40-digit arithmetic,
 * identities, printed values of the pages, or hand-derived byte fixtures.
 *
 * Precision: every arithmetic step of attention, RoPE and rotation runs in IEEE fp64. The
 * quantiser runs in the precision its definition fixes (fp32 steps, fp16 results), because there a
 * floating-point value decides an integer code.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F64 0
#define ORC_F32 1
#define ORC_F16 2
#define ORC_BF16 3

/* ------------------------------------------------------------------------------------------ */
/* IEEE binary16 / bfloat16 scalar conversions (written from the IEEE 754 encoding).           */
/* ------------------------------------------------------------------------------------------ */

double orc_f16_to_f64(uint16_t h)
{
    int s = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m | 0x400), e - 25);    /* (1024 + m) * 2^(e - 15 - 10) */
    return s ? -v : v;
}

/* Round any double to the nearest binary16, ties to even; overflow goes to infinity. */
uint16_t orc_f64_to_f16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x))
        return 0x7e00;
    if (a >= 65520.0)                              /* 65504 + half an ulp ties to even -> inf */
        return sign | 0x7c00;
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);                                  /* a in [2^(e-1), 2^e) */
    int q = e - 11;                                /* binary16 keeps 11 significant bits */
    if (q < -24)
        q = -24;                                   /* subnormal spacing */
    double r = nearbyint(ldexp(a, -q));            /* default rounding mode: nearest-even */
    double v = ldexp(r, q);
    if (v == 0.0)
        return sign;
    int e2;
    frexp(v, &e2);
    int E = e2 + 14;                               /* biased exponent of v */
    if (E >= 1)
        return sign | (uint16_t)(E << 10) | (uint16_t)((uint32_t)ldexp(v, 11 - e2) - 1024u);
    return sign | (uint16_t)ldexp(v, 24);
}

double orc_bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round any double to the nearest bfloat16 (8 significant bits, the binary32 exponent range),
 * ties to even; overflow goes to infinity. Rounded directly from the double, never through
 * binary32, so no second rounding. */
uint16_t orc_f64_to_bf16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x))
        return 0x7fc0;
    if (a >= ldexp(2.0 - ldexp(1.0, -8), 127))   /* max finite + half an ulp ties to even -> inf */
        return sign | 0x7f80;
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);                                  /* a in [2^(e-1), 2^e) */
    int q = e - 8;                                 /* bfloat16 keeps 8 significant bits */
    if (q < -133)
        q = -133;                                  /* subnormal spacing 2^-133 */
    double v = ldexp(nearbyint(ldexp(a, -q)), q);
    if (v == 0.0)
        return sign;
    int e2;
    frexp(v, &e2);
    int E = e2 + 126;                              /* biased exponent of v */
    if (E >= 1)
        return sign | (uint16_t)(E << 7) | (uint16_t)((uint32_t)ldexp(v, 8 - e2) - 128u);
    return sign | (uint16_t)ldexp(v, 133);
}

/* Round n doubles once to the storage type dt (F32: binary32 nearest-even, F16, BF16). */
void orc_round_array(long n, const double *x, int dt, void *out)
{
    for (long i = 0; i < n; ++i) {
        if (dt == ORC_F32)
            ((float *)out)[i] = (float)x[i];
        else if (dt == ORC_F16)
            ((uint16_t *)out)[i] = orc_f64_to_f16(x[i]);
        else
            ((uint16_t *)out)[i] = orc_f64_to_bf16(x[i]);
    }
}

static double load_elem(const void *p, int dt, size_t i)
{
    switch (dt) {
    case ORC_F64: return ((const double *)p)[i];
    case ORC_F32: return (double)((const float *)p)[i];
    case ORC_F16: return orc_f16_to_f64(((const uint16_t *)p)[i]);
    default:      return orc_bf16_to_f64(((const uint16_t *)p)[i]);
    }
}

/* ------------------------------------------------------------------------------------------ */
/* RoPE (LLaMA rotate-half). theta_i = base^(-2i/d), i < d/2; position n rotates the pair      */
/* (x_i, x_{i+d/2}) by the angle n*theta_i. Angles are formed and evaluated in fp64.           */
/* (Zhou notes, section 5.3 and Algorithm 2 step 4c: RoPE at each cached position.)            */
/* ------------------------------------------------------------------------------------------ */

double orc_rope_theta(int i, int d, double base)
{
    return pow(base, (-2.0 * (double)i) / (double)d);
}

void orc_rope(const double *x, int d, double pos, double base, double *out)
{
    int half = d / 2;
    for (int i = 0; i < half; ++i) {
        double ang = pos * orc_rope_theta(i, d, base);
        double c = cos(ang), s = sin(ang);
        double a = x[i], b = x[i + half];
        out[i] = a * c - b * s;
        out[i + half] = b * c + a * s;
    }
}

/* cos/sin of n*theta_i for n < T, i < d/2 (memoised per call; same fp64 values as orc_rope). */
static double *rope_table(long T, int d, double base)
{
    int half = d / 2;
    double *tab = (double *)malloc(sizeof(double) * 2 * (size_t)T * half);
    if (!tab)
        return NULL;
    double *theta = (double *)malloc(sizeof(double) * half);
    for (int i = 0; i < half; ++i)
        theta[i] = orc_rope_theta(i, d, base);
    for (long n = 0; n < T; ++n)
        for (int i = 0; i < half; ++i) {
            double ang = (double)n * theta[i];
            tab[2 * ((size_t)n * half + i)] = cos(ang);
            tab[2 * ((size_t)n * half + i) + 1] = sin(ang);
        }
    free(theta);
    return tab;
}

/* ------------------------------------------------------------------------------------------ */
/* Decode attention for one (b, h): softmax over n < T of scale * q . RoPE_n(k~_n), then the   */
/* value side. k~_n and the value rows are produced by the caller-selected layer kind below.   */
/* ------------------------------------------------------------------------------------------ */

typedef struct {
    int B, H, d, rv, Rk;
    long T;
    const int *koff;          /* [H+1] prefix sums of key ranks */
    const void *zk; int zdt;  /* latent: [B][T][Rk]; dense: K [B][T][H*d] */
    const void *zv;           /* latent: [B][T][rv]; dense: V [B][T][H*d] */
    const double *bk;         /* [Rk][d] */
    const double *bv;         /* [rv][H*d] */
    const double *q;          /* [B][H][d], post-RoPE */
    double scale;
    const double *tab;        /* rope table */
    int dense, form;
} job_t;

static void decode_one(const job_t *J, int b, int h, double *out)
{
    int d = J->d, half = d / 2, Hd = J->H * J->d;
    long T = J->T;
    double *s = (double *)malloc(sizeof(double) * (size_t)T);
    double *kt = (double *)malloc(sizeof(double) * d);
    const double *qv = J->q + ((size_t)b * J->H + h) * d;

    /* scores */
    for (long n = 0; n < T; ++n) {
        if (J->dense) {
            size_t row = ((size_t)b * T + n) * Hd + (size_t)h * d;
            for (int j = 0; j < d; ++j)
                kt[j] = load_elem(J->zk, J->zdt, row + j);
        } else {
            int r0 = J->koff[h], r1 = J->koff[h + 1];
            size_t row = ((size_t)b * T + n) * J->Rk;
            for (int j = 0; j < d; ++j)
                kt[j] = 0.0;
            for (int c = r0; c < r1; ++c) {           /* k~ = Z_k[h][n] . B_k[h] */
                double z = load_elem(J->zk, J->zdt, row + c);
                const double *brow = J->bk + (size_t)c * d;
                for (int j = 0; j < d; ++j)
                    kt[j] += z * brow[j];
            }
        }
        double acc = 0.0;
        const double *cs = J->tab + 2 * (size_t)n * half;
        for (int i = 0; i < half; ++i) {              /* rotate-half RoPE at position n */
            double c = cs[2 * i], sn = cs[2 * i + 1];
            double a = kt[i], bb = kt[i + half];
            acc += qv[i] * (a * c - bb * sn) + qv[i + half] * (bb * c + a * sn);
        }
        s[n] = J->scale * acc;
    }

    /* softmax */
    double m = -INFINITY;
    for (long n = 0; n < T; ++n)
        if (s[n] > m)
            m = s[n];
    double L = 0.0;
    for (long n = 0; n < T; ++n) {
        s[n] = exp(s[n] - m);
        L += s[n];
    }

    for (int j = 0; j < d; ++j)
        out[j] = 0.0;
    if (J->dense) {
        for (long n = 0; n < T; ++n) {
            size_t row = ((size_t)b * T + n) * Hd + (size_t)h * d;
            for (int j = 0; j < d; ++j)
                out[j] += s[n] * load_elem(J->zv, J->zdt, row + j);
        }
    } else if (J->form == 0) {
        /* latent form: a = sum_n p_n Z_v[n]; o = a . B_v[:, h*d:(h+1)*d] */
        int rv = J->rv;
        double *a = (double *)calloc((size_t)rv, sizeof(double));
        for (long n = 0; n < T; ++n) {
            size_t row = ((size_t)b * T + n) * rv;
            for (int c = 0; c < rv; ++c)
                a[c] += s[n] * load_elem(J->zv, J->zdt, row + c);
        }
        for (int c = 0; c < rv; ++c) {
            const double *brow = J->bv + (size_t)c * Hd + (size_t)h * d;
            for (int j = 0; j < d; ++j)
                out[j] += a[c] * brow[j];
        }
        free(a);
    } else {
        /* explicit form: V_h[n] = Z_v[n] . B_v^h, o = sum_n p_n V_h[n] */
        int rv = J->rv;
        double *vrow = (double *)malloc(sizeof(double) * d);
        for (long n = 0; n < T; ++n) {
            size_t row = ((size_t)b * T + n) * rv;
            for (int j = 0; j < d; ++j)
                vrow[j] = 0.0;
            for (int c = 0; c < rv; ++c) {
                double z = load_elem(J->zv, J->zdt, row + c);
                const double *brow = J->bv + (size_t)c * Hd + (size_t)h * d;
                for (int j = 0; j < d; ++j)
                    vrow[j] += z * brow[j];
            }
            for (int j = 0; j < d; ++j)
                out[j] += s[n] * vrow[j];
        }
        free(vrow);
    }
    for (int j = 0; j < d; ++j)
        out[j] /= L;
    free(kt);
    free(s);
}

/*
 * Latent decode attention. zk [B][T][Rk] and zv [B][T][rv] in dtype zdt (ORC_*); bk [Rk][d],
 * bv [rv][H*d] and q [B][H][d] in fp64. key_ranks [H]. form 0 = latent order, 1 = explicit order.
 * pairs: npairs (b,h) pairs to evaluate, or NULL for all B*H in (b,h) order; out [npairs][d].
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int orc_decode_latent(int B, int H, int d, long T, const int *key_ranks, int rv, int zdt,
                      const void *zk, const void *zv, const double *bk, const double *bv,
                      const double *q, double rope_base, double scale, int npairs,
                      const int *pairs, int form, double *out)
{
    if (B < 0 || H <= 0 || d <= 0 || (d & 1) || T <= 0 || rv <= 0)
        return -1;
    int *koff = (int *)malloc(sizeof(int) * (H + 1));
    koff[0] = 0;
    for (int h = 0; h < H; ++h)
        koff[h + 1] = koff[h] + key_ranks[h];
    job_t J = {B, H, d, rv, koff[H], T, koff, zk, zdt, zv, bk, bv, q, scale, NULL, 0, form};
    J.tab = rope_table(T, d, rope_base);
    if (!J.tab) {
        free(koff);
        return -1;
    }
    int n = pairs ? npairs : B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < n; ++i) {
        int b = pairs ? pairs[2 * i] : i / H;
        int h = pairs ? pairs[2 * i + 1] : i % H;
        decode_one(&J, b, h, out + (size_t)i * d);
    }
    free((void *)J.tab);
    free(koff);
    return 0;
}

/* Dense exempt layer: K, V [B][T][H*d] (pre-RoPE keys), q [B][H][d] fp64. */
int orc_decode_dense(int B, int H, int d, long T, int kvdt, const void *k, const void *v,
                     const double *q, double rope_base, double scale, int npairs,
                     const int *pairs, double *out)
{
    if (B < 0 || H <= 0 || d <= 0 || (d & 1) || T <= 0)
        return -1;
    job_t J = {B, H, d, 0, 0, T, NULL, k, kvdt, v, NULL, NULL, q, scale, NULL, 1, 0};
    J.tab = rope_table(T, d, rope_base);
    if (!J.tab)
        return -1;
    int n = pairs ? npairs : B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < n; ++i) {
        int b = pairs ? pairs[2 * i] : i / H;
        int h = pairs ? pairs[2 * i + 1] : i % H;
        decode_one(&J, b, h, out + (size_t)i * d);
    }
    free((void *)J.tab);
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Blockwise Hadamard rotation (Zhou notes, section 6.1 / Fig. 5).                              */
/* Reading: a latent of width r is split into its first n_hi channels (the high-magnitude      */
/* block, which the 4-bit budget protects) and the remaining r - n_hi channels; each segment   */
/* of width w is rotated by blockdiag(H_b, ..., H_b) with b = min(64, largest power of two    */
/* dividing w), H_b the normalised Sylvester matrix H_b[i][j] = (-1)^popcount(i&j) / sqrt(b). */
/* ------------------------------------------------------------------------------------------ */

static int popcount_u32(uint32_t x)
{
    int c = 0;
    while (x) {
        c += (int)(x & 1u);
        x >>= 1;
    }
    return c;
}

/* n must be a power of two; out is n x n, row-major. */
int orc_hadamard(int n, double *out)
{
    if (n <= 0 || (n & (n - 1)))
        return -1;
    double s = 1.0 / sqrt((double)n);
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < n; ++j)
            out[(size_t)i * n + j] = (popcount_u32((uint32_t)(i & j)) & 1) ? -s : s;
    return 0;
}

int orc_hadamard_block(int width)
{
    if (width <= 0)
        return 0;
    int b = 1;
    while (b < 64 && (width % (2 * b)) == 0)
        b *= 2;
    return b;
}

/* Number of high-precision ("hi") channels of a latent of width r: ceil(frac * r). Reading: the
 * fraction is a decimal such as 0.25 or 0.2 that reaches the library as a binary32 parameter, so
 * products within 1e-4 of an integer are taken as that integer (0.2f * 80 = 16.0000002 -> 16);
 * any product farther from an integer is rounded up. */
int orc_n_hi(int r, double frac)
{
    if (r <= 0)
        return 0;
    double x = frac * (double)r;
    int n = (int)ceil(x - 1e-4);
    if (n < 0)
        n = 0;
    if (n > r)
        n = r;
    return n;
}

/*
 * Rotate row vectors: out[row][c] for c in a segment list. x and out are [rows][ld] in fp64.
 * seg: nseg pairs (start, width). Channels outside every segment are copied unchanged.
 */
int orc_rotate_rows_f64(long rows, int ld, int nseg, const int *seg, const double *x, double *out)
{
    for (long t = 0; t < rows; ++t)
        memcpy(out + (size_t)t * ld, x + (size_t)t * ld, sizeof(double) * ld);
    for (int g = 0; g < nseg; ++g) {
        int s0 = seg[2 * g], w = seg[2 * g + 1];
        int bsz = orc_hadamard_block(w);
        double *Hm = (double *)malloc(sizeof(double) * bsz * bsz);
        orc_hadamard(bsz, Hm);
        for (long t = 0; t < rows; ++t) {
            const double *xr = x + (size_t)t * ld;
            double *orow = out + (size_t)t * ld;
            for (int j0 = s0; j0 < s0 + w; j0 += bsz)
                for (int i = 0; i < bsz; ++i) {          /* (x H)_i = sum_j x_j H[j][i] */
                    double acc = 0.0;
                    for (int j = 0; j < bsz; ++j)
                        acc += xr[j0 + j] * Hm[(size_t)j * bsz + i];
                    orow[j0 + i] = acc;
                }
        }
        free(Hm);
    }
    return 0;
}

/*
 * Rotate the rows of a factor (left multiplication by blockdiag(H)^T): B'[j0+i][:] =
 * sum_j H[j][i] B[j0+j][:]. b and out are [C][ncols] fp64; seg as above (over the C rows).
 */
int orc_rotate_factor_f64(int C, int ncols, int nseg, const int *seg, const double *bsrc,
                          double *out)
{
    memcpy(out, bsrc, sizeof(double) * (size_t)C * ncols);
    for (int g = 0; g < nseg; ++g) {
        int s0 = seg[2 * g], w = seg[2 * g + 1];
        int bsz = orc_hadamard_block(w);
        double *Hm = (double *)malloc(sizeof(double) * bsz * bsz);
        orc_hadamard(bsz, Hm);
        for (int j0 = s0; j0 < s0 + w; j0 += bsz)
            for (int i = 0; i < bsz; ++i)
                for (int col = 0; col < ncols; ++col) {
                    double acc = 0.0;
                    for (int j = 0; j < bsz; ++j)
                        acc += Hm[(size_t)j * bsz + i] * bsrc[(size_t)(j0 + j) * ncols + col];
                    out[(size_t)(j0 + i) * ncols + col] = acc;
                }
        free(Hm);
    }
    return 0;
}

/*
 * fp16 storage of a rotation. Reading of how a rotated fp16 latent is stored: the signed sum
 * sum_j (+-x_j) is formed exactly (every binary16 is k*2^-24 with |k| < 2^40, so a sum of at most
 * 64 of them is exact in fp64), multiplied in fp64 by the fp64 value of 1/sqrt(b), and rounded
 * once more to binary16 (nearest-even). Same rule for latent rows and for factor rows.
 */
static uint16_t rot_round(double signed_sum, double inv_sqrt_b)
{
    return orc_f64_to_f16(signed_sum * inv_sqrt_b);
}

int orc_rotate_rows_f16(long rows, int ld, int nseg, const int *seg, const uint16_t *x,
                        uint16_t *out)
{
    for (long t = 0; t < rows; ++t)
        memcpy(out + (size_t)t * ld, x + (size_t)t * ld, sizeof(uint16_t) * ld);
    for (int g = 0; g < nseg; ++g) {
        int s0 = seg[2 * g], w = seg[2 * g + 1];
        int bsz = orc_hadamard_block(w);
        double inv = 1.0 / sqrt((double)bsz);
#pragma omp parallel for schedule(static)
        for (long t = 0; t < rows; ++t) {
            const uint16_t *xr = x + (size_t)t * ld;
            uint16_t *orow = out + (size_t)t * ld;
            for (int j0 = s0; j0 < s0 + w; j0 += bsz)
                for (int i = 0; i < bsz; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < bsz; ++j) {
                        double v = orc_f16_to_f64(xr[j0 + j]);
                        acc += (popcount_u32((uint32_t)(i & j)) & 1) ? -v : v;
                    }
                    orow[j0 + i] = rot_round(acc, inv);
                }
        }
    }
    return 0;
}

int orc_rotate_factor_f16(int C, int ncols, int nseg, const int *seg, const uint16_t *bsrc,
                          uint16_t *out)
{
    memcpy(out, bsrc, sizeof(uint16_t) * (size_t)C * ncols);
    for (int g = 0; g < nseg; ++g) {
        int s0 = seg[2 * g], w = seg[2 * g + 1];
        int bsz = orc_hadamard_block(w);
        double inv = 1.0 / sqrt((double)bsz);
#pragma omp parallel for collapse(2) schedule(static)
        for (int j0 = s0; j0 < s0 + w; j0 += bsz)
            for (int i = 0; i < bsz; ++i)
                for (int col = 0; col < ncols; ++col) {
                    double acc = 0.0;
                    for (int j = 0; j < bsz; ++j) {
                        double v = orc_f16_to_f64(bsrc[(size_t)(j0 + j) * ncols + col]);
                        acc += (popcount_u32((uint32_t)(i & j)) & 1) ? -v : v;
                    }
                    out[(size_t)(j0 + i) * ncols + col] = rot_round(acc, inv);
                }
    }
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Mixed 4/3-bit quantisation (Zhou notes, section 6.1; model card calibration recipe).         */
/*                                                                                              */
/* Reading of the quantiser, per channel and per group of 64 consecutive tokens (x: binary16): */
/*   mn, mx   = min, max of the group                                                           */
/*   s        = (float(mx) - float(mn)) / float(2^bits - 1)        fp32 arithmetic              */
/*   s16      = binary16(s) (nearest-even);   z16 = binary16(mn), -0 stored as +0               */
/*   code     = 0 if s16 == 0, else clamp(rint((float(x) - z) / s), 0, 2^bits - 1) with z, s    */
/*              the fp32 values of z16, s16; fp32 subtract and divide, rint ties to even        */
/*   dequant  = binary16(code * s + z), the exact value rounded once (nearest-even). Every   */
/*              binary16 is an integer multiple of 2^-24 and |code * s + z| < 2^21, so the     */
/*              exact value is an integer times 2^-24 below 2^45 and fp64 holds it exactly.    */
/*                                                                                              */
/* Packed layout of one channel's 64 codes (little-endian 32-bit words; in every word the even */
/* tokens of its span fill the low 16 bits and the odd tokens the high 16 bits, so that tokens   */
/* 2i and 2i+1 sit 16 bits apart):                                                              */
/*   4 bits: 8 words; word t/8 holds tokens 8*(t/8) .. +7; token t at bit 16*(t%2) + 4*((t/2)%4). */
/*   3 bits: 6 words; words 0..3 the low two bits (word t/16, bit 16*(t%2) + 2*((t/2)%8)),      */
/*           words 4..5 the third bit (word 4 + t/32, bit 16*(t%2) + (t/2)%16).                 */
/* ------------------------------------------------------------------------------------------ */

static float f16_to_f32(uint16_t h) { return (float)orc_f16_to_f64(h); }

/* Bit offset of token t's w-bit field inside its 32-bit word: even tokens from bit 0, odd tokens
 * from bit 16, in token order (one field per token pair). */
static int code_bit(int t, int w)
{
    int per_half = 16 / w;                      /* fields in one 16-bit half */
    return 16 * (t & 1) + w * ((t / 2) % per_half);
}

/* Bit-addressed access to a little-endian byte string (bit i = bit i%8 of byte i/8). */
static void set_code_bits(uint8_t *bytes, int bit, int value, int w)
{
    for (int i = 0; i < w; ++i)
        bytes[(bit + i) / 8] |= (uint8_t)(((value >> i) & 1) << ((bit + i) % 8));
}

static int get_code_bits(const uint8_t *bytes, int bit, int w)
{
    int v = 0;
    for (int i = 0; i < w; ++i)
        v |= ((bytes[(bit + i) / 8] >> ((bit + i) % 8)) & 1) << i;
    return v;
}

void orc_quantize_group(const uint16_t *x, long stride, int bits, uint8_t *codes_out,
                        uint16_t *scale_out, uint16_t *zero_out)
{
    double mn = INFINITY, mx = -INFINITY;
    for (int t = 0; t < 64; ++t) {
        double v = orc_f16_to_f64(x[(size_t)t * stride]);
        if (v < mn)
            mn = v;
        if (v > mx)
            mx = v;
    }
    int qmax = (1 << bits) - 1;
    float diff = (float)mx - (float)mn;
    float s = diff / (float)qmax;
    uint16_t s16 = orc_f64_to_f16((double)s);
    uint16_t z16 = orc_f64_to_f16(mn);
    if (z16 == 0x8000)
        z16 = 0;
    float sf = f16_to_f32(s16), zf = f16_to_f32(z16);
    uint8_t code[64];
    for (int t = 0; t < 64; ++t) {
        if ((s16 & 0x7fff) == 0) {
            code[t] = 0;
            continue;
        }
        float v = (f16_to_f32(x[(size_t)t * stride]) - zf) / sf;
        float r = rintf(v);
        if (r < 0.0f)
            r = 0.0f;
        if (r > (float)qmax)
            r = (float)qmax;
        code[t] = (uint8_t)r;
    }
    memset(codes_out, 0, (size_t)8 * bits);
    for (int t = 0; t < 64; ++t) {
        if (bits == 4) {
            set_code_bits(codes_out, 32 * (t / 8) + code_bit(t, 4), code[t] & 0xf, 4);
        } else {
            set_code_bits(codes_out, 32 * (t / 16) + code_bit(t, 2), code[t] & 3, 2);
            set_code_bits(codes_out, 128 + 32 * (t / 32) + code_bit(t, 1), (code[t] >> 2) & 1, 1);
        }
    }
    *scale_out = s16;
    *zero_out = z16;
}

int orc_unpack_code(const uint8_t *codes, int bits, int t)
{
    if (bits == 4)
        return get_code_bits(codes, 32 * (t / 8) + code_bit(t, 4), 4);
    return get_code_bits(codes, 32 * (t / 16) + code_bit(t, 2), 2) |
           (get_code_bits(codes, 128 + 32 * (t / 32) + code_bit(t, 1), 1) << 2);
}

uint16_t orc_dequant_value(int code, uint16_t s16, uint16_t z16)
{
    double exact = (double)code * orc_f16_to_f64(s16) + orc_f16_to_f64(z16);
    return orc_f64_to_f16(exact);
}

/* Bytes of one 64-token block of a latent whose channel c has bits[c] bits: sum of 8*bits. */
long orc_q43_block_bytes(int C, const uint8_t *bits)
{
    long n = 0;
    for (int c = 0; c < C; ++c)
        n += 8L * bits[c];
    return n;
}

/*
 * Quantise a whole latent cache. x [B][T][C] binary16; channel c packed with bits[c] (3 or 4)
 * bits, channels in order inside each 64-token block. Outputs: codes [B][T_cap/64][block_bytes],
 * meta [B][T_cap/64][C][2] (scale, zero), tail [B][64][C] holding the rows of an unfinished last
 * group (T % 64 of them; rows of complete groups never go through the tail).
 */
int orc_q43_pack(int B, long T, long T_cap, int C, const uint8_t *bits, const uint16_t *x,
                 uint8_t *codes, uint16_t *meta, uint16_t *tail)
{
    if (T_cap % 64 || T > T_cap)
        return -1;
    long bb = orc_q43_block_bytes(C, bits);
    long nblk = T_cap / 64, full = T / 64;
    for (int b = 0; b < B; ++b) {
        for (long g = 0; g < full; ++g) {
            uint8_t *blk = codes + ((size_t)b * nblk + g) * bb;
            long off = 0;
            for (int c = 0; c < C; ++c) {
                const uint16_t *src = x + ((size_t)b * T + g * 64) * C + c;
                uint16_t *m = meta + (((size_t)b * nblk + g) * C + c) * 2;
                orc_quantize_group(src, C, bits[c], blk + off, &m[0], &m[1]);
                off += 8L * bits[c];
            }
        }
        long rem = T - full * 64;
        for (long t = 0; t < rem; ++t)
            memcpy(tail + ((size_t)b * 64 + t) * C, x + ((size_t)b * T + full * 64 + t) * C,
                   sizeof(uint16_t) * C);
    }
    return 0;
}

/* Dequantise tokens [t0, t1) to x [B][t1-t0][C] binary16: complete groups (g < seq_len/64) from
 * codes + meta, the tokens of the unfinished group from the tail. */
int orc_q43_unpack(int B, long seq_len, long T_cap, int C, const uint8_t *bits,
                   const uint8_t *codes, const uint16_t *meta, const uint16_t *tail, long t0,
                   long t1, uint16_t *x)
{
    if (T_cap % 64 || seq_len > T_cap || t0 < 0 || t1 > seq_len || t0 > t1)
        return -1;
    long bb = orc_q43_block_bytes(C, bits);
    long nblk = T_cap / 64, full = seq_len / 64;
    long *off = (long *)malloc(sizeof(long) * (C + 1));
    off[0] = 0;
    for (int c = 0; c < C; ++c)
        off[c + 1] = off[c] + 8L * bits[c];
    for (int b = 0; b < B; ++b)
        for (long t = t0; t < t1; ++t) {
            uint16_t *dst = x + ((size_t)b * (t1 - t0) + (t - t0)) * C;
            long g = t / 64;
            if (g < full) {
                const uint8_t *blk = codes + ((size_t)b * nblk + g) * bb;
                for (int c = 0; c < C; ++c) {
                    const uint16_t *m = meta + (((size_t)b * nblk + g) * C + c) * 2;
                    int code = orc_unpack_code(blk + off[c], bits[c], (int)(t % 64));
                    dst[c] = orc_dequant_value(code, m[0], m[1]);
                }
            } else {
                memcpy(dst, tail + ((size_t)b * 64 + (t % 64)) * C, sizeof(uint16_t) * C);
            }
        }
    free(off);
    return 0;
}

#ifdef _OPENMP
#include <omp.h>
#endif
/* Threads the attention loops use (OpenMP over independent (b, h) pairs). */
/* Thread count for later parallel regions (timing only; results do not depend on it). */
void orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

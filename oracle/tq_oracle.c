/*
 * tq_oracle.c -- plain, slow, fp64 CPU oracle for the TurboQuant KV-cache hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark load this file's library.  The GPU library shares no code,
 * header, table or constant generator with it, and neither includes the other.
 *
 * What is computed, and where it is described:
 *   - the five-step key/value compression pipeline (random orthogonal rotation,
 *     Lloyd-Max quantisation against a Beta-distribution codebook, one QJL residual
 *     sign bit per coordinate, 2/4-bit symmetric value quantisation in groups of 32,
 *     bit packing): hotelren.com guide "企业官网建设流程全解析", section 二 (the
 *     5-step pipeline figure and the three bullets under it);
 *   - the unbiased inner-product property E[estimate] = true inner product of the
 *     key path (TurboQuantProd): same section, first bullet;
 *   - the hybrid decode: compressed history plus an exact recent ring buffer of
 *     buffer_size tokens: same guide, section 5.1 (hook installation, items 1-2);
 *   - the magnitude / direction split (norm stored, direction quantised): zingnex.cn
 *     thread "TurboQuant-vLLM：大模型推理的KV缓存量化实战方案", section
 *     "TurboQuant：PolarQuant + Hadamard变换".
 *
 * Readings where the pages are silent (all listed in the design doc of the repository):
 *   rotation = H diag(sigma) / sqrt(d), H the natural-order Sylvester Hadamard matrix;
 *   the key codebook is the Lloyd-Max quantiser of one coordinate of a uniform unit
 *   vector in R^d, whose law is (t+1)/2 ~ Beta((d-1)/2, (d-1)/2);
 *   QJL matrix S: d x d, N(0,1) entries rounded to fp16, drawn from a splitmix64
 *   counter stream through Box-Muller; estimator constant sqrt(pi/2)/d;
 *   value quantiser: bin-centre symmetric, scale fp16(max|v| / 2^(vb-1)).
 *
 * Format choice of the library (not a reading of the pages, which fix no table
 * precision): the stored codebook holds each Lloyd-Max centroid rounded to binary16 and
 * each decision boundary at the exact midpoint of its two stored centroids.  Its cost is
 * pinned by the tests: d times the mean squared error of the stored table stays within
 * 1e-5 (relative) of the fp64 optimum's at d = 64, 128 and 256 for 1 to 4 bits.
 *
 * Everything here runs in double precision on inputs already rounded to their stored
 * type.  No blocking, fusion or reordering: every quantity is computed from its
 * definition (dense Hadamard matrix, dense S r product, direct softmax).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

/* ------------------------------------------------------------------------------ */
/* IEEE binary16 <-> double, written from the format's definition (1 sign bit,     */
/* 5 exponent bits with bias 15, 10 fraction bits), rounding to nearest-even.      */
/* ------------------------------------------------------------------------------ */
double orc_f16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double mag;
    if (e == 0)
        mag = ldexp((double)f, -24); /* subnormal: f * 2^-14 * 2^-10 */
    else if (e == 31)
        mag = f ? NAN : INFINITY;
    else
        mag = ldexp((double)(f + 1024), e - 25); /* (1 + f/1024) * 2^(e-15) */
    return sign ? -mag : mag;
}

uint16_t orc_double_to_f16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x)) return 0x7e00;
    if (a == 0.0) return sign;
    /* quantum of the binary16 grid that a falls into */
    int ex;
    frexp(a, &ex);             /* a = m * 2^ex, m in [0.5, 1) => a in [2^(ex-1), 2^ex) */
    int e_unb = ex - 1;        /* a in [2^e_unb, 2^(e_unb+1)) */
    if (e_unb < -14) e_unb = -14; /* subnormal range shares the quantum 2^-24 */
    double quantum = ldexp(1.0, e_unb - 10);
    double q = a / quantum;    /* exact: division by a power of two */
    double r = nearbyint(q);   /* default rounding mode: nearest, ties to even */
    double val = r * quantum;
    if (val >= 65520.0 || val > 65504.0) return sign | 0x7c00; /* overflow to inf */
    /* re-encode val, which is now exactly representable */
    if (val < ldexp(1.0, -14)) {
        return sign | (uint16_t)r; /* subnormal (or the carry into the smallest normal) */
    }
    int ex2;
    double m2 = frexp(val, &ex2); /* val = m2 * 2^ex2 */
    int e_field = ex2 - 1 + 15;
    int frac = (int)ldexp(m2 * 2.0 - 1.0, 10);
    return sign | (uint16_t)(e_field << 10) | (uint16_t)frac;
}

/* ------------------------------------------------------------------------------ */
/* Seeded tables: sign vector sigma and QJL matrix S.                              */
/* splitmix64 (Steele, Lea and Flood, OOPSLA 2014; the constants of Vigna's        */
/* public-domain reference), used as a counter-based stream: output i is the mix   */
/* of seed + (i+1) * golden-gamma.                                                 */
/* ------------------------------------------------------------------------------ */
uint64_t orc_splitmix64_at(uint64_t seed, uint64_t i)
{
    uint64_t z = seed + (i + 1) * 0x9E3779B97F4A7C15ULL;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/*
 * sigma_j = +1 if the top bit of stream word j is 0, else -1        (j in [0, d))
 * S entries in row-major order, drawn in pairs (2m, 2m+1) by Box-Muller from stream
 * words d + 2m and d + 2m + 1:  u1, u2 = 53-bit uniforms in [0, 1);
 *   R = sqrt(-2 ln(1 - u1)), theta = 2 pi u2, S_2m = R cos theta, S_2m+1 = R sin theta,
 * each rounded to the nearest binary16 value.
 */
void orc_tables(int d, uint64_t seed, int8_t *sigma, uint16_t *S_bits)
{
    for (int j = 0; j < d; ++j)
        sigma[j] = (orc_splitmix64_at(seed, (uint64_t)j) >> 63) ? -1 : 1;
    const double two_pi = 6.283185307179586476925286766559;
    int64_t n = (int64_t)d * d;
    for (int64_t m = 0; 2 * m < n; ++m) {
        uint64_t w1 = orc_splitmix64_at(seed, (uint64_t)(d + 2 * m));
        uint64_t w2 = orc_splitmix64_at(seed, (uint64_t)(d + 2 * m + 1));
        double u1 = (double)(w1 >> 11) * (1.0 / 9007199254740992.0);
        double u2 = (double)(w2 >> 11) * (1.0 / 9007199254740992.0);
        double R = sqrt(-2.0 * log(1.0 - u1));
        double th = two_pi * u2;
        S_bits[2 * m] = orc_double_to_f16(R * cos(th));
        if (2 * m + 1 < n) S_bits[2 * m + 1] = orc_double_to_f16(R * sin(th));
    }
}

/* ------------------------------------------------------------------------------ */
/* Lloyd-Max codebook for one coordinate t of a uniform unit vector in R^d.        */
/* Law: (t+1)/2 ~ Beta(p, p), p = (d-1)/2, i.e. density                            */
/*   f(t) = (1-t^2)^(p-1) / (2^(2p-1) B(p,p))  on (-1, 1).                         */
/* Cell mass uses the regularised incomplete beta function I_x(p,p); the cell's    */
/* first moment has the closed form  int t f = -(1-t^2)^p / (2p 2^(2p-1) B(p,p)).  */
/* ------------------------------------------------------------------------------ */

/* continued fraction of the incomplete beta (DLMF 8.17.22), modified Lentz method */
static double ibeta_cf(double a, double b, double x)
{
    const double tiny = 1e-300;
    double C = 1.0, D = 1.0 - (a + b) * x / (a + 1.0);
    if (fabs(D) < tiny) D = tiny;
    D = 1.0 / D;
    double h = D;
    for (int m = 1; m < 100000; ++m) {
        double m2 = 2.0 * m;
        /* even step: d_{2m} = m (b - m) x / ((a + 2m - 1)(a + 2m)) */
        double num = m * (b - m) * x / ((a + m2 - 1.0) * (a + m2));
        D = 1.0 + num * D; if (fabs(D) < tiny) D = tiny; D = 1.0 / D;
        C = 1.0 + num / C; if (fabs(C) < tiny) C = tiny;
        h *= D * C;
        /* odd step: d_{2m+1} = -(a + m)(a + b + m) x / ((a + 2m)(a + 2m + 1)) */
        num = -(a + m) * (a + b + m) * x / ((a + m2) * (a + m2 + 1.0));
        D = 1.0 + num * D; if (fabs(D) < tiny) D = tiny; D = 1.0 / D;
        C = 1.0 + num / C; if (fabs(C) < tiny) C = tiny;
        double del = D * C;
        h *= del;
        if (fabs(del - 1.0) < 1e-17) break;
    }
    return h;
}

/* regularised incomplete beta I_x(a, b) */
static double ibeta(double a, double b, double x)
{
    if (x <= 0.0) return 0.0;
    if (x >= 1.0) return 1.0;
    double lfront = lgamma(a + b) - lgamma(a) - lgamma(b) + a * log(x) + b * log1p(-x);
    if (x < (a + 1.0) / (a + b + 2.0))
        return exp(lfront) * ibeta_cf(a, b, x) / a;
    double lfront2 = lgamma(a + b) - lgamma(a) - lgamma(b) + b * log1p(-x) + a * log(x);
    return 1.0 - exp(lfront2) * ibeta_cf(b, a, 1.0 - x) / b;
}

/* P(T <= t) for the coordinate law */
static double coord_cdf(double p, double t)
{
    if (t <= -1.0) return 0.0;
    if (t >= 1.0) return 1.0;
    if (t <= 0.0) return ibeta(p, p, 0.5 * (1.0 + t));
    return 1.0 - ibeta(p, p, 0.5 * (1.0 - t)); /* symmetry: keeps the tail accurate */
}

/* int_a^b t f(t) dt, closed form */
static double coord_first_moment(double p, double a, double b)
{
    double lZ = (2.0 * p - 1.0) * log(2.0) + 2.0 * lgamma(p) - lgamma(2.0 * p);
    double fa = (a <= -1.0 || a >= 1.0) ? 0.0 : exp(p * log1p(-a * a) - lZ - log(2.0 * p));
    double fb = (b <= -1.0 || b >= 1.0) ? 0.0 : exp(p * log1p(-b * b) - lZ - log(2.0 * p));
    return fa - fb;
}

/*
 * Lloyd iteration: boundaries are midpoints of adjacent centroids, centroids are the
 * conditional means of their cells; run until no centroid moves by 1e-15, then make
 * the table exactly antisymmetric.  c: 2^kb entries, b: 2^kb - 1 entries (fp64).
 * Returns the number of iterations, or -1 on bad arguments.
 */
int orc_codebook(int d, int kb, double *c, double *b)
{
    if (d < 4 || kb < 1 || kb > 8) return -1;
    int L = 1 << kb;
    double p = 0.5 * (d - 1);
    double sd = 1.0 / sqrt((double)d); /* coordinate standard deviation */
    for (int i = 0; i < L; ++i) c[i] = sd * 3.0 * (-1.0 + (2.0 * i + 1.0) / L);
    int it;
    for (it = 0; it < 200000; ++it) {
        for (int i = 0; i + 1 < L; ++i) b[i] = 0.5 * (c[i] + c[i + 1]);
        double moved = 0.0;
        for (int i = 0; i < L; ++i) {
            double lo = (i == 0) ? -1.0 : b[i - 1];
            double hi = (i == L - 1) ? 1.0 : b[i];
            double mass = coord_cdf(p, hi) - coord_cdf(p, lo);
            double cn = coord_first_moment(p, lo, hi) / mass;
            double dm = fabs(cn - c[i]);
            if (dm > moved) moved = dm;
            c[i] = cn;
        }
        if (moved < 1e-14) break;
    }
    for (int i = 0; i < L / 2; ++i) {
        double m = 0.5 * (c[L - 1 - i] - c[i]);
        c[i] = -m;
        c[L - 1 - i] = m;
    }
    for (int i = 0; i + 1 < L; ++i) b[i] = 0.5 * (c[i] + c[i + 1]);
    return it;
}

/*
 * The table values the library stores and uses (its storage format, see the header):
 * each centroid rounded to the nearest binary16 value, and each decision boundary the
 * exact midpoint of its two stored centroids (representable in binary32).
 */
int orc_stored_codebook(int d, int kb, double *c_store, double *b_store)
{
    int L = 1 << kb;
    double c[256], b[255];
    int it = orc_codebook(d, kb, c, b);
    if (it < 0) return it;
    for (int i = 0; i < L; ++i) c_store[i] = orc_f16_to_double(orc_double_to_f16(c[i]));
    for (int i = 0; i + 1 < L; ++i) b_store[i] = 0.5 * (c_store[i] + c_store[i + 1]);
    return it;
}

/* cell mass and conditional mean, exported so tests can probe the fixed point */
double orc_coord_cdf(int d, double t) { return coord_cdf(0.5 * (d - 1), t); }
double orc_coord_moment(int d, double a, double b) { return coord_first_moment(0.5 * (d - 1), a, b); }

/* ------------------------------------------------------------------------------ */
/* Rotation Pi = H diag(sigma) / sqrt(d), H[i][j] = (-1)^popcount(i & j)           */
/* (Sylvester construction in natural order), applied as a dense matrix.           */
/* ------------------------------------------------------------------------------ */
static int parity_of(unsigned x)
{
    int p = 0;
    while (x) { p ^= 1; x &= x - 1; }
    return p;
}

double orc_hadamard_entry(int i, int j) { return parity_of((unsigned)(i & j)) ? -1.0 : 1.0; }

/* y = Pi x */
void orc_rotate(int d, const int8_t *sigma, const double *x, double *y)
{
    double inv = 1.0 / sqrt((double)d);
    for (int i = 0; i < d; ++i) {
        double acc = 0.0;
        for (int j = 0; j < d; ++j) acc += orc_hadamard_entry(i, j) * sigma[j] * x[j];
        y[i] = acc * inv;
    }
}

/* ------------------------------------------------------------------------------ */
/* Key path, one token-head vector at a time:                                      */
/*   n = |k|, u = Pi k / n, idx_j = #{i : u_j > b_i}, r = u - c[idx], g = |r|,     */
/*   p = S r, z_j = [p_j >= 0].                                                     */
/* c32 / b32 hold the stored single-precision table values.  S is the stored fp16  */
/* matrix, row-major.  Margins: distance of u_j to the nearest boundary and |p_j|, */
/* the quantities whose size decides whether a rounding difference may flip a bit. */
/* force_idx (may be NULL): use these codebook indices instead of the nearest cell   */
/* (a code chosen inside the rounding window changes the residual, and with it      */
/* every sign bit of the row; this re-derives the rest of the row from that choice). */
/* ------------------------------------------------------------------------------ */
void orc_quantize_keys(int d, int kb, const double *c32, const double *b32, const int8_t *sigma,
                       const uint16_t *S_bits, const double *k, int64_t n_rows,
                       uint8_t *idx, uint8_t *z, double *norm, double *rnorm,
                       double *u_margin, double *p_margin, const uint8_t *force_idx)
{
    int L = 1 << kb;
    double *S = (double *)malloc(sizeof(double) * d * d);
    double *u = (double *)malloc(sizeof(double) * d);
    double *r = (double *)malloc(sizeof(double) * d);
    for (int64_t e = 0; e < (int64_t)d * d; ++e) S[e] = orc_f16_to_double(S_bits[e]);
    for (int64_t row = 0; row < n_rows; ++row) {
        const double *kr = k + row * d;
        double ss = 0.0;
        for (int j = 0; j < d; ++j) ss += kr[j] * kr[j];
        double n = sqrt(ss);
        orc_rotate(d, sigma, kr, u);
        for (int j = 0; j < d; ++j) u[j] = (n > 0.0) ? u[j] / n : 0.0;
        double gg = 0.0;
        for (int j = 0; j < d; ++j) {
            int cnt = 0;
            double mg = INFINITY;
            for (int i = 0; i + 1 < L; ++i) {
                if (u[j] > b32[i]) ++cnt;
                double dist = fabs(u[j] - b32[i]);
                if (dist < mg) mg = dist;
            }
            if (force_idx) cnt = force_idx[row * d + j];
            idx[row * d + j] = (uint8_t)cnt;
            if (u_margin) u_margin[row * d + j] = mg;
            r[j] = u[j] - c32[cnt];
            gg += r[j] * r[j];
        }
        norm[row] = n;
        rnorm[row] = sqrt(gg);
        for (int i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int j = 0; j < d; ++j) acc += S[(int64_t)i * d + j] * r[j];
            z[row * d + i] = (acc >= 0.0) ? 1 : 0;
            if (p_margin) p_margin[row * d + i] = fabs(acc);
        }
    }
    free(S); free(u); free(r);
}

/* ------------------------------------------------------------------------------ */
/* Value path: symmetric uniform quantiser per group of 32 consecutive channels.   */
/*   a = max |v|, s = fp16(a / 2^(vb-1)); s == 0 -> every code is 2^(vb-1);         */
/*   else code = clamp(floor(v / s), -2^(vb-1), 2^(vb-1) - 1) + 2^(vb-1).           */
/* Reconstruction is the bin centre (code - 2^(vb-1) + 1/2) s.                      */
/* margin: distance of v/s to the nearest integer step that decides the code.      */
/* ------------------------------------------------------------------------------ */
void orc_quantize_values(int d, int vb, int group, const double *v, int64_t n_rows,
                         uint8_t *code, uint16_t *scale_bits, double *margin)
{
    int half = 1 << (vb - 1);
    int ng = d / group;
    for (int64_t row = 0; row < n_rows; ++row) {
        for (int g = 0; g < ng; ++g) {
            const double *vg = v + row * d + (int64_t)g * group;
            double a = 0.0;
            for (int j = 0; j < group; ++j) if (fabs(vg[j]) > a) a = fabs(vg[j]);
            uint16_t sb = orc_double_to_f16(a / half);
            double s = orc_f16_to_double(sb);
            scale_bits[row * ng + g] = sb;
            for (int j = 0; j < group; ++j) {
                int64_t o = row * d + (int64_t)g * group + j;
                if (s == 0.0) {
                    code[o] = (uint8_t)half;
                    if (margin) margin[o] = INFINITY;
                    continue;
                }
                double x = vg[j] / s;
                double f = floor(x);
                if (f < -half) f = -half;
                if (f > half - 1) f = half - 1;
                code[o] = (uint8_t)((int)f + half);
                if (margin) {
                    double m = INFINITY;
                    for (int t = -half + 1; t <= half - 1; ++t) {
                        double dist = fabs(x - t);
                        if (dist < m) m = dist;
                    }
                    margin[o] = m;
                }
            }
        }
    }
}

/* ------------------------------------------------------------------------------ */
/* Packed record layout (one token-head).  A key record has (kb + 1) d / 32 words.  */
/*   kb = 3: word w (0 <= w < d/8) covers coordinates 8w..8w+7 as eight 4-bit       */
/*   nibbles: nibble k (bits 4k..4k+3) holds the codebook index of coordinate 8w+k  */
/*   in its low three bits and that coordinate's QJL sign bit in its top bit.        */
/*   kb = 1, 2, 4: two planes.  The code plane (words 0 .. kb d/32 - 1) holds the    */
/*   index of coordinate j at bit kb*(j mod (32/kb)) of word floor(j kb / 32); the   */
/*   sign plane (the d/32 words after it) holds the sign bit of coordinate j at bit  */
/*   j mod 32 of its word floor(j / 32).                                             */
/*   Value codes least-significant first: code j sits at bit vb*(j mod (32/vb)) of   */
/*   word floor(j*vb/32)  (four 2-bit codes per byte, as the pages state).           */
/* ------------------------------------------------------------------------------ */
int orc_key_words(int d, int kb) { return (kb + 1) * d / 32; }

void orc_pack_keys(int d, int kb, const uint8_t *idx, const uint8_t *z, int64_t n_rows, uint32_t *words)
{
    int nw = orc_key_words(d, kb);
    for (int64_t row = 0; row < n_rows; ++row) {
        const uint8_t *ir = idx + row * d, *zr = z + row * d;
        uint32_t *wr = words + row * nw;
        for (int w = 0; w < nw; ++w) wr[w] = 0;
        for (int j = 0; j < d; ++j) {
            uint32_t code = (uint32_t)ir[j] & ((1u << kb) - 1u), sign = (uint32_t)zr[j] & 1u;
            if (kb == 3) {
                wr[j / 8] |= (code | (sign << 3)) << (4 * (j % 8));
            } else {
                int per = 32 / kb;
                wr[j / per] |= code << (kb * (j % per));
                wr[kb * d / 32 + j / 32] |= sign << (j % 32);
            }
        }
    }
}

void orc_unpack_keys(int d, int kb, const uint32_t *words, int64_t n_rows, uint8_t *idx, uint8_t *z)
{
    int nw = orc_key_words(d, kb);
    for (int64_t row = 0; row < n_rows; ++row) {
        const uint32_t *wr = words + row * nw;
        for (int j = 0; j < d; ++j) {
            uint32_t code, sign;
            if (kb == 3) {
                uint32_t nib = (wr[j / 8] >> (4 * (j % 8))) & 15u;
                code = nib & 7u;
                sign = nib >> 3;
            } else {
                int per = 32 / kb;
                code = (wr[j / per] >> (kb * (j % per))) & ((1u << kb) - 1u);
                sign = (wr[kb * d / 32 + j / 32] >> (j % 32)) & 1u;
            }
            idx[row * d + j] = (uint8_t)code;
            z[row * d + j] = (uint8_t)sign;
        }
    }
}

void orc_pack_values(int d, int vb, const uint8_t *code, int64_t n_rows, uint32_t *words)
{
    int per = 32 / vb, nw = d * vb / 32;
    for (int64_t row = 0; row < n_rows; ++row)
        for (int w = 0; w < nw; ++w) {
            uint32_t x = 0;
            for (int k = 0; k < per; ++k)
                x |= ((uint32_t)code[row * d + w * per + k] & ((1u << vb) - 1u)) << (vb * k);
            words[row * nw + w] = x;
        }
}

void orc_unpack_values(int d, int vb, const uint32_t *words, int64_t n_rows, uint8_t *code)
{
    int per = 32 / vb, nw = d * vb / 32;
    for (int64_t row = 0; row < n_rows; ++row)
        for (int j = 0; j < d; ++j)
            code[row * d + j] = (uint8_t)((words[row * nw + j / per] >> (vb * (j % per))) & ((1u << vb) - 1u));
}

/* ------------------------------------------------------------------------------ */
/* Hybrid decode attention (compressed history + exact ring), one query head at a  */
/* time.  GQA: query head h reads kv head h / G.  For packed token t:               */
/*   q' = Pi q, w = S q',                                                          */
/*   s_t = n_t ( sum_j q'_j c[idx_tj] + g_t sqrt(pi/2)/d sum_j w_j (2 z_tj - 1) ),  */
/* the unbiased estimate of <q, k_t>; ring token t: s_t = <q, k_t> on fp16 keys.   */
/* Softmax over packed and ring tokens of s * scale, then the weighted sum of the  */
/* bin-centre values (packed) and the exact fp16 values (ring).                    */
/*                                                                                 */
/* Arrays (slice = b * Hkv + kv head; cap = capacity of the packed store,          */
/* buf = ring capacity):                                                           */
/*   kw [slices][cap][(kb+1) d/32] u32, kn [slices][cap][2] f32 (norm, residual   */
/*   norm),                                                                         */
/*   vw [slices][cap][vb d/32] u32, vs [slices][cap][d/32] fp16,                   */
/*   rk, rv [slices][buf][d] fp16, q [B][Hq][d] (double), out [B][Hq][d] (double). */
/* ------------------------------------------------------------------------------ */
void orc_decode(int d, int kb, int vb, int group, const double *c32, const int8_t *sigma,
                const uint16_t *S_bits, int B, int Hq, int Hkv,
                const uint32_t *kw, const float *kn, const uint32_t *vw, const uint16_t *vs,
                int64_t cap, int64_t n_packed,
                const uint16_t *rk, const uint16_t *rv, int buf, int n_ring,
                const double *q, double scale, double *out, double *scores_out)
{
    int G = Hq / Hkv;
    int half = 1 << (vb - 1);
    int ng = d / group;
    int nkw = orc_key_words(d, kb), nvw = d * vb / 32;
    int64_t T = n_packed + n_ring;
    const double kqjl = sqrt(3.14159265358979323846 / 2.0) / d;
    double *S = (double *)malloc(sizeof(double) * d * d);
    double *qr = (double *)malloc(sizeof(double) * d);
    double *w = (double *)malloc(sizeof(double) * d);
    double *s = (double *)malloc(sizeof(double) * (T > 0 ? T : 1));
    double *o = (double *)malloc(sizeof(double) * d);
    uint8_t *idx = (uint8_t *)malloc(d), *z = (uint8_t *)malloc(d), *code = (uint8_t *)malloc(d);
    for (int64_t e = 0; e < (int64_t)d * d; ++e) S[e] = orc_f16_to_double(S_bits[e]);
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hq; ++h) {
            int64_t sl = (int64_t)b * Hkv + h / G;
            const double *qv = q + ((int64_t)b * Hq + h) * d;
            orc_rotate(d, sigma, qv, qr);
            for (int i = 0; i < d; ++i) {
                double acc = 0.0;
                for (int j = 0; j < d; ++j) acc += S[(int64_t)i * d + j] * qr[j];
                w[i] = acc;
            }
            for (int64_t t = 0; t < n_packed; ++t) {
                int64_t rec = sl * cap + t;
                orc_unpack_keys(d, kb, kw + rec * nkw, 1, idx, z);
                double mse = 0.0, sgn = 0.0;
                for (int j = 0; j < d; ++j) {
                    mse += qr[j] * c32[idx[j]];
                    sgn += w[j] * (2.0 * z[j] - 1.0);
                }
                s[t] = (double)kn[rec * 2] * (mse + (double)kn[rec * 2 + 1] * kqjl * sgn);
            }
            for (int t = 0; t < n_ring; ++t) {
                const uint16_t *kr = rk + (sl * buf + t) * d;
                double acc = 0.0;
                for (int j = 0; j < d; ++j) acc += qv[j] * orc_f16_to_double(kr[j]);
                s[n_packed + t] = acc;
            }
            if (scores_out)
                for (int64_t t = 0; t < T; ++t) scores_out[((int64_t)b * Hq + h) * T + t] = s[t];
            double m = -INFINITY;
            for (int64_t t = 0; t < T; ++t) if (s[t] * scale > m) m = s[t] * scale;
            double l = 0.0;
            for (int j = 0; j < d; ++j) o[j] = 0.0;
            for (int64_t t = 0; t < T; ++t) {
                double p = exp(s[t] * scale - m);
                l += p;
                if (t < n_packed) {
                    int64_t rec = sl * cap + t;
                    orc_unpack_values(d, vb, vw + rec * nvw, 1, code);
                    for (int j = 0; j < d; ++j) {
                        double sc = orc_f16_to_double(vs[rec * ng + j / group]);
                        o[j] += p * ((double)code[j] - half + 0.5) * sc;
                    }
                } else {
                    const uint16_t *vr = rv + (sl * buf + (t - n_packed)) * d;
                    for (int j = 0; j < d; ++j) o[j] += p * orc_f16_to_double(vr[j]);
                }
            }
            double *ov = out + ((int64_t)b * Hq + h) * d;
            for (int j = 0; j < d; ++j) ov[j] = (T > 0) ? o[j] / l : 0.0;
        }
    free(S); free(qr); free(w); free(s); free(o); free(idx); free(z); free(code);
}

// tq_host.cpp -- host-side tables of the TurboQuant KV library (no device code).
//
// * Lloyd-Max codebook for one coordinate of a uniform unit vector in R^d (hotelren.com
//   guide "企业官网建设流程全解析", section 二 step 2: Lloyd-Max quantiser with a
//   Beta-distribution codebook, tables per dimension and bit width).  The coordinate
//   density is proportional to (1 - t^2)^((d-3)/2) on (-1, 1); cell masses and first
//   moments are integrated here by composite Gauss-Legendre quadrature.
// * Seeded rotation signs and the fp16 QJL projection (section 二 steps 1 and 3).
// * The device table blob and the size helpers declared in tq.h.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include <hip/hip_runtime.h>

#include "tq.h"
#include "tq_internal.h"

namespace {

// n-point Gauss-Legendre nodes/weights on [-1, 1]: Newton iteration on P_n from the
// Chebyshev-like initial guesses, weights 2 / ((1 - x^2) P_n'(x)^2).
struct GaussLegendre {
    std::vector<double> x, w;
    explicit GaussLegendre(int n) : x(n), w(n) {
        const double pi = 3.14159265358979323846;
        for (int i = 0; i < (n + 1) / 2; ++i) {
            double z = std::cos(pi * (i + 0.75) / (n + 0.5));
            double dp = 0.0;
            for (int it = 0; it < 100; ++it) {
                double p0 = 1.0, p1 = z;
                for (int k = 2; k <= n; ++k) {
                    double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
                    p0 = p1;
                    p1 = p2;
                }
                dp = n * (z * p1 - p0) / (z * z - 1.0);
                double dz = p1 / dp;
                z -= dz;
                if (std::fabs(dz) < 1e-16) break;
            }
            x[i] = -z;
            x[n - 1 - i] = z;
            w[i] = w[n - 1 - i] = 2.0 / ((1.0 - z * z) * dp * dp);
        }
    }
};

// integral over [a, b] of t^m (1 - t^2)^alpha for m = 0, 1 (composite rule)
void cell_moments(const GaussLegendre &gl, double alpha, double a, double b, double &m0, double &m1) {
    const int pieces = 24;
    m0 = m1 = 0.0;
    double h = (b - a) / pieces;
    for (int p = 0; p < pieces; ++p) {
        double lo = a + p * h, mid = lo + 0.5 * h;
        for (size_t i = 0; i < gl.x.size(); ++i) {
            double t = mid + 0.5 * h * gl.x[i];
            double f = std::exp(alpha * std::log1p(-t * t)) * gl.w[i] * 0.5 * h;
            m0 += f;
            m1 += f * t;
        }
    }
}

bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

uint64_t splitmix64_word(uint64_t seed, uint64_t counter) {
    uint64_t z = seed + (counter + 1) * 0x9E3779B97F4A7C15ULL;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint16_t to_half_bits(double x) {
    _Float16 h = (_Float16)x;  // direct double -> binary16, round to nearest even
    uint16_t b;
    std::memcpy(&b, &h, 2);
    return b;
}

}  // namespace

extern "C" tq_status tq_build_codebook(int32_t head_dim, int32_t key_bits, double *c, double *bnd) {
    if (!c || !bnd || !pow2(head_dim) || head_dim < 8 || head_dim > 4096 || key_bits < 1 || key_bits > 4)
        return TQ_ERR_INVALID_ARG;
    const int L = 1 << key_bits;
    const double alpha = 0.5 * (head_dim - 3);
    static const GaussLegendre gl(40);
    const double sd = 1.0 / std::sqrt((double)head_dim);
    for (int i = 0; i < L; ++i) c[i] = 2.0 * sd * (-1.0 + (2.0 * i + 1.0) / L);
    for (int it = 0; it < 200000; ++it) {
        for (int i = 0; i + 1 < L; ++i) bnd[i] = 0.5 * (c[i] + c[i + 1]);
        double moved = 0.0;
        for (int i = 0; i < L; ++i) {
            double lo = i == 0 ? -1.0 : bnd[i - 1];
            double hi = i == L - 1 ? 1.0 : bnd[i];
            double m0, m1;
            cell_moments(gl, alpha, lo, hi, m0, m1);
            double cn = m1 / m0;
            moved = std::fmax(moved, std::fabs(cn - c[i]));
            c[i] = cn;
        }
        if (moved < 1e-14) break;
    }
    for (int i = 0; i < L / 2; ++i) {
        double m = 0.5 * (c[L - 1 - i] - c[i]);
        c[i] = -m;
        c[L - 1 - i] = m;
    }
    for (int i = 0; i + 1 < L; ++i) bnd[i] = 0.5 * (c[i] + c[i + 1]);
    return TQ_OK;
}

extern "C" tq_status tq_build_rotation(int32_t d, uint64_t seed, int8_t *signs, uint16_t *S) {
    if (!signs || !S || !pow2(d) || d < 8 || d > 4096) return TQ_ERR_INVALID_ARG;
    for (int j = 0; j < d; ++j) signs[j] = (splitmix64_word(seed, (uint64_t)j) >> 63) ? int8_t(-1) : int8_t(1);
    const double two_pi = 6.283185307179586476925286766559;
    const int64_t n = (int64_t)d * d;
    const double inv53 = 1.0 / 9007199254740992.0;
    for (int64_t e = 0; e < n; e += 2) {
        double u1 = (double)(splitmix64_word(seed, (uint64_t)(d + e)) >> 11) * inv53;
        double u2 = (double)(splitmix64_word(seed, (uint64_t)(d + e + 1)) >> 11) * inv53;
        double rad = std::sqrt(-2.0 * std::log(1.0 - u1));
        double ang = two_pi * u2;
        S[e] = to_half_bits(rad * std::cos(ang));
        if (e + 1 < n) S[e + 1] = to_half_bits(rad * std::sin(ang));
    }
    return TQ_OK;
}

extern "C" size_t tq_tables_bytes(const tq_config *cfg) {
    if (!cfg || tq::check_config(*cfg) != TQ_OK) return 0;
    return tq::kTableSOffset + 2 * (size_t)cfg->head_dim * cfg->head_dim;
}

extern "C" tq_status tq_build_tables(const tq_config *cfg, uint64_t seed, void *blob, size_t bytes) {
    if (!cfg || !blob) return TQ_ERR_INVALID_ARG;
    tq_status st = tq::check_config(*cfg);
    if (st != TQ_OK) return st;
    if (bytes < tq_tables_bytes(cfg)) return TQ_ERR_INVALID_ARG;
    const int d = cfg->head_dim, L = 1 << cfg->key_bits;
    std::memset(blob, 0, tq_tables_bytes(cfg));
    unsigned char *p = static_cast<unsigned char *>(blob);
    double c[16], b[16];
    st = tq_build_codebook(d, cfg->key_bits, c, b);
    if (st != TQ_OK) return st;
    float *cf = reinterpret_cast<float *>(p + tq::kTableCentroidOffset);
    float *bf = reinterpret_cast<float *>(p + tq::kTableBoundaryOffset);
    // stored table: centroids rounded to binary16, boundaries their exact midpoints
    for (int i = 0; i < L; ++i) cf[i] = (float)(_Float16)c[i];
    for (int i = 0; i + 1 < L; ++i) bf[i] = (float)(0.5 * ((double)cf[i] + (double)cf[i + 1]));
    // the decode's integer score path (head_dim 128) takes c * 2^Sc (Sc: the power of two that
    // keeps every |c * 2^Sc| below 2^14) as exact integers
    if (d == 128 && cfg->key_bits == 3 && !tq::centroids_are_scaled_integers(cf, L)) return TQ_ERR_UNSUPPORTED;
    std::vector<int8_t> sg(d);
    uint16_t *S = reinterpret_cast<uint16_t *>(p + tq::kTableSOffset);
    st = tq_build_rotation(d, seed, sg.data(), S);
    if (st != TQ_OK) return st;
    uint32_t *sb = reinterpret_cast<uint32_t *>(p + tq::kTableSignOffset);
    for (int j = 0; j < d; ++j)
        if (sg[j] < 0) sb[j / 32] |= 1u << (j % 32);
    return TQ_OK;
}

namespace tq {
bool centroids_are_scaled_integers(const float *c, int n) {
    float cmax = 0.f;
    for (int i = 0; i < n; ++i) cmax = std::fmax(cmax, std::fabs(c[i]));
    int ec = 0;
    (void)std::frexp(cmax, &ec);
    for (int i = 0; i < n; ++i) {
        const double v = std::ldexp((double)c[i], 14 - ec);
        if (v != std::nearbyint(v) || std::fabs(v) >= 16384.0) return false;
    }
    return true;
}
}  // namespace tq

extern "C" tq_status tq_tables_view(const tq_config *cfg, const void *blob, tq_tables *out) {
    if (!cfg || !blob || !out) return TQ_ERR_INVALID_ARG;
    tq_status st = tq::check_config(*cfg);
    if (st != TQ_OK) return st;
    if (reinterpret_cast<uintptr_t>(blob) % 256) return TQ_ERR_INVALID_ARG;
    const unsigned char *p = static_cast<const unsigned char *>(blob);
    out->centroids = reinterpret_cast<const float *>(p + tq::kTableCentroidOffset);
    out->boundaries = reinterpret_cast<const float *>(p + tq::kTableBoundaryOffset);
    out->sign_bits = reinterpret_cast<const uint32_t *>(p + tq::kTableSignOffset);
    out->qjl_S = reinterpret_cast<const uint16_t *>(p + tq::kTableSOffset);
    return TQ_OK;
}

extern "C" size_t tq_packed_bytes_per_token(const tq_config *cfg) {
    if (!cfg || tq::check_config(*cfg) != TQ_OK) return 0;
    const size_t d = cfg->head_dim;
    return d * (cfg->key_bits + 1) / 8 + 8 + d * cfg->value_bits / 8 + 2 * (d / cfg->group_size);
}

extern "C" const char *tq_status_string(tq_status s) {
    switch (s) {
        case TQ_OK: return "ok";
        case TQ_ERR_INVALID_ARG: return "invalid argument";
        case TQ_ERR_UNSUPPORTED: return "unsupported configuration";
        case TQ_ERR_RING_FULL: return "ring buffer full";
        case TQ_ERR_WORKSPACE: return "decode workspace too small";
        case TQ_ERR_HIP: return "HIP runtime error";
        case TQ_ERR_SCRATCH_LIMIT: return "call needs more scratch than the library's static decode buffer holds";
    }
    return "unknown status";
}

namespace tq {

int device_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int c = 0;
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
        cus[dev] = c;
    }
    return cus[dev];
}

tq_status check_config(const tq_config &c) {
    if (c.head_dim <= 0 || c.key_bits <= 0 || c.value_bits <= 0 || c.group_size <= 0 || c.buffer_size <= 0)
        return TQ_ERR_INVALID_ARG;
    if (c.head_dim != 64 && c.head_dim != 128 && c.head_dim != 256) return TQ_ERR_UNSUPPORTED;
    if (c.key_bits < 1 || c.key_bits > 4) return TQ_ERR_UNSUPPORTED;
    if (c.head_dim == 256 && c.key_bits != 3) return TQ_ERR_UNSUPPORTED;
    if (c.value_bits != 2 && c.value_bits != 4) return TQ_ERR_UNSUPPORTED;
    if (c.group_size != 32) return TQ_ERR_UNSUPPORTED;
    if (c.buffer_size > 1024) return TQ_ERR_UNSUPPORTED;
    return TQ_OK;
}

}  // namespace tq

// tq_decode.hip -- hybrid decode attention over the packed store plus the exact ring
// (hotelren.com guide "企业官网建设流程全解析", section 5.1 item 2: attention over the
// compressed history together with the exact recent buffer), and the ring append
// (section 5.1 item 1: a decode-time token goes into the ring buffer).
//
// Score of a packed token t for query head g is the unbiased inner-product estimate of
// section 二 evaluated in the rotated domain (q' = Pi q, w = S q', computed once per query
// by k_decode_prep):
//   s_tg = |k_t| ( sum_j q'_gj c[idx_tj] + g_t sqrt(pi/2)/d sum_j w_gj (2 z_tj - 1) ).
//
// k_decode_main, grid (splits, batch * kv heads), 4 waves per workgroup.  Splits 0..P-1
// cover the packed tokens in contiguous ranges; split P (present when the ring holds
// tokens) covers the ring.  Each wave of a packed split streams blocks of 32 tokens:
//   * scores on MFMA (v_mfma_f32_16x16x32_f16, 16 tokens x 16 columns): A holds, per
//     token, the fp16 centroid values of 8 coordinates (a 256-entry LDS table maps one
//     byte = two nibbles to a packed fp16 pair) and the +-1 sign of each QJL bit; B holds
//     q'_g in columns g and -w_g in columns 8+g as fp16 hi + lo pairs (kept in registers);
//   * per-wave online softmax on the accumulator layout;
//   * values on MFMA: A = raw value codes as fp16 (lane row m owns the codes of
//     coordinates m*NT .. m*NT+NT-1, read from LDS-staged records), B = p_t * scale_t,grp
//     (hi + lo) in columns (head, group); the constant code offset is removed with the
//     column sums of B at the end.
// The four waves' (m, l, o) are combined in LDS, every split writes (m, l, o) partials,
// and the last split to finish a (batch, kv head) -- atomic ticket -- merges them and
// re-arms the ticket to zero.
#include <hip/hip_runtime.h>

#include "tq.h"
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kBlock = 32;       // tokens per wave iteration
constexpr int kLutCopies = 32;   // copies of the byte -> centroid-pair table (one per LDS bank)
constexpr int kRingChunk = 256;  // ring tokens per pass of the ring split

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
// raw buffer descriptor word 3 for gfx9-family raw (untyped) buffer loads
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint32_t pack_half2(float lo, float hi) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}

// x = hi + lo with hi = fp16(x), lo = fp16(x - hi)
__device__ __forceinline__ void split_hl(float x, _Float16 &hi, _Float16 &lo) {
    hi = (_Float16)x;
    lo = (_Float16)(x - (float)hi);
}

// ------------------------------------------------------------------ query preparation
template <typename Tag, int D>
__global__ __launch_bounds__(D) void k_decode_prep(DecodeArgs a) {
    __shared__ float y[D];
    __shared__ float red[D / 64];
    const int j = threadIdx.x;
    const int64_t bh = blockIdx.x;  // b * hq + h
    const float qv = load1(a.q, bh * D + j, Tag{});
    y[j] = flip_sign(qv, (a.sign_bits[j >> 5] >> (j & 31)) & 1u);
    __syncthreads();
    for (int len = 1; len < D; len <<= 1) {
        float p = y[j], o = y[j ^ len];
        __syncthreads();
        y[j] = (j & len) ? (o - p) : (p + o);
        __syncthreads();
    }
    const float qr = y[j] * (1.0f / sqrtf((float)D));
    __syncthreads();
    y[j] = qr;
    __syncthreads();
    // w_j = sum_i S[j][i] q'_i
    const uint16_t *srow = a.S + (int64_t)j * D;
    float acc = 0.f;
    for (int i = 0; i < D; i += 8) {
        uint4 pk = *reinterpret_cast<const uint4 *>(srow + i);
        acc = fmaf(f16_lo(pk.x), y[i + 0], acc);
        acc = fmaf(f16_hi(pk.x), y[i + 1], acc);
        acc = fmaf(f16_lo(pk.y), y[i + 2], acc);
        acc = fmaf(f16_hi(pk.y), y[i + 3], acc);
        acc = fmaf(f16_lo(pk.z), y[i + 4], acc);
        acc = fmaf(f16_hi(pk.z), y[i + 5], acc);
        acc = fmaf(f16_lo(pk.w), y[i + 6], acc);
        acc = fmaf(f16_hi(pk.w), y[i + 7], acc);
    }
    float *p = a.prep + bh * (3 * D + 4);
    p[j] = qr;
    p[D + j] = acc;
    p[2 * D + j] = qv;
    float sw = acc;
    for (int o = 32; o > 0; o >>= 1) sw += __shfl_xor(sw, o);
    if ((j & 63) == 0) red[j >> 6] = sw;
    __syncthreads();
    if (j == 0) {
        float tot = 0.f;
        for (int i = 0; i < D / 64; ++i) tot += red[i];
        p[3 * D] = tot;
    }
}

template <int D, int VB, int G>
struct DecodeShape {
    static constexpr int KW = D / 8;          // key words per token
    static constexpr int NKS = D / 32;        // score k-steps per part (one key word per lane group)
    static constexpr int VW = VB * D / 32;    // value words per token
    static constexpr int VWP = VW + 2;        // padded LDS row (row groups of 8 hit distinct banks)
    static constexpr int NG = D / 32;         // value groups
    static constexpr int NT = D / 16;         // value tiles; row m owns coordinates m*NT .. m*NT+NT-1
    static constexpr int H = VB * NT / 16;    // halfwords of codes per row and token (1, 2 or 4)
    static constexpr int NCOL = G * NG;       // value columns (head, group)
    static constexpr int NPASS = (NCOL + 15) / 16;
    static constexpr int HALF = 1 << (VB - 1);
    static constexpr int PARTS = kThreads / D;  // ring split: token partitions per coordinate
};

template <int D, int VB, int G>
struct alignas(16) DecodeSmem {
    using S = DecodeShape<D, VB, G>;
    uint32_t lut[256 * kLutCopies];
    uint32_t val[kWaves][kBlock][S::VWP];
    float scl[kWaves][S::NG][kBlock + 4];
    float pb[kWaves][G][kBlock + 4];
    float corr[kWaves][G];
    float wm[kWaves][G], wl[kWaves][G];
    float wo[kWaves][G][D];
    float ring_q[G][D];
    float ring_p[G][kRingChunk];
    float ring_red[kWaves * G];
    float ml[G];
    float merge_f[G][256];
    unsigned ticket;
};

// block-wide reduction of G values (max or sum); every thread gets the result
template <int G, bool IsMax>
__device__ __forceinline__ void block_reduce(float (&v)[G], float *scratch /* [kWaves][G] */) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float x = v[g];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            float y = __shfl_xor(x, o);
            x = IsMax ? fmaxf(x, y) : x + y;
        }
        if (lane == 0) scratch[wv * G + g] = x;
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float x = scratch[g];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) x = IsMax ? fmaxf(x, scratch[w * G + g]) : x + scratch[w * G + g];
        v[g] = x;
    }
    __syncthreads();
}

// ------------------------------------------------------------------ packed split (one wave)
template <int D, int VB, int G>
__device__ void packed_wave(const DecodeArgs &a, DecodeSmem<D, VB, G> &sm, int bk, int b, int kvh,
                            int64_t t_begin, int64_t t_end) {
    using S = DecodeShape<D, VB, G>;
    constexpr float kQjl = 1.2533141373155003f / D;  // sqrt(pi/2) / d
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n16 = lane & 15, q = lane >> 4;

    // score B fragments, column g < G for head g: q'_g (fp16 hi + lo) for the centroid part,
    // w_g (fp16) for the sign part.  k-step ks of lane group q covers key word
    // w = q*NKS + ks; centroid element e is coordinate 8w+e, sign element e = 2r+h' is
    // coordinate 8w + r + 4h' (nibbles r and r+4 of the word).
    half8_t bm_hi[S::NKS], bm_lo[S::NKS], bq[S::NKS];
    {
        const bool col = n16 < G;
        const float *pq = a.prep + ((int64_t)b * a.hq + kvh * G + (col ? n16 : 0)) * (3 * D + 4);
#pragma unroll
        for (int ks = 0; ks < S::NKS; ++ks) {
            const int w = q * S::NKS + ks;
            const float4 m0 = *reinterpret_cast<const float4 *>(pq + 8 * w);
            const float4 m1 = *reinterpret_cast<const float4 *>(pq + 8 * w + 4);
            const float4 s0 = *reinterpret_cast<const float4 *>(pq + D + 8 * w);
            const float4 s1 = *reinterpret_cast<const float4 *>(pq + D + 8 * w + 4);
            const float vm[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
            const float vq[8] = {s0.x, s1.x, s0.y, s1.y, s0.z, s1.z, s0.w, s1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                _Float16 h, l;
                split_hl(col ? vm[e] : 0.f, h, l);
                bm_hi[ks][e] = h;
                bm_lo[ks][e] = l;
                bq[ks][e] = (_Float16)(col ? vq[e] : 0.f);
            }
        }
    }

    // running reference max per head (lanes n16 == g), per-lane partial sums of p (the
    // lane's rows), value accumulators and column sums of B
    float m_ref = -INFINITY, l_part = 0.f;
    f32x4_t acc_v[S::NPASS][S::NT];
    float sumb[S::NPASS];
#pragma unroll
    for (int p = 0; p < S::NPASS; ++p) {
        sumb[p] = 0.f;
#pragma unroll
        for (int t = 0; t < S::NT; ++t) acc_v[p][t] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    }
    const uint32_t *lut = sm.lut + (lane & (kLutCopies - 1));
    const int64_t rec0 = (int64_t)bk * a.cap;

    // one block's global data, held in registers so that the next block's loads are in
    // flight while the current block is computed
    struct Blk {
        uint32_t kw[2][S::NKS];   // key words of A row token t0 + 16 tt + n16, words q*NKS ..
        float2 an[2];             // (norm, residual norm) of that token
        float dn[2][4];           // norm of accumulator row token t0 + 16 tt + 4 q + i
        uint4 vw[S::VW / 8];      // half hv of the value record of token t0 + (lane & 31)
        uint32_t sc[S::NG / 2];   // fp16 scale pairs of token t0 + (lane & 31)
    };
    const int tl = lane & 31, hv = lane >> 5;
    // buffer descriptors over this slice's records: 32-bit offsets, and loads past the
    // last packed token return zeros (those rows are masked out of the softmax)
    const int np = (int)a.n_packed;
    const __amdgpu_buffer_rsrc_t rs_kw = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.kw + rec0 * S::KW), (short)0, np * S::KW * 4, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rs_kn = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.kn + rec0 * 2), (short)0, np * 8, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rs_vw = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.vw + rec0 * S::VW), (short)0, np * S::VW * 4, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rs_vs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.vs + rec0 * S::NG), (short)0, np * S::NG * 2, kBufferFlags);
    auto load_blk = [&](int t0, Blk &r) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int tok = t0 + 16 * tt + n16;
#pragma unroll
            for (int i = 0; i < S::NKS / 4; ++i) {
                const u32x4_t u = __builtin_amdgcn_raw_buffer_load_b128(
                    rs_kw, (uint32_t)((tok * S::KW + q * S::NKS + 4 * i) * 4), 0, 0);
                r.kw[tt][4 * i + 0] = u[0]; r.kw[tt][4 * i + 1] = u[1];
                r.kw[tt][4 * i + 2] = u[2]; r.kw[tt][4 * i + 3] = u[3];
            }
            const u32x2_t an = __builtin_amdgcn_raw_buffer_load_b64(rs_kn, (uint32_t)(tok * 8), 0, 0);
            r.an[tt] = make_float2(__uint_as_float(an[0]), __uint_as_float(an[1]));
            const int tr = t0 + 16 * tt + 4 * q;  // four consecutive row tokens: 32 bytes
            const u32x4_t d01 = __builtin_amdgcn_raw_buffer_load_b128(rs_kn, (uint32_t)(tr * 8), 0, 0);
            const u32x4_t d23 = __builtin_amdgcn_raw_buffer_load_b128(rs_kn, (uint32_t)(tr * 8 + 16), 0, 0);
            r.dn[tt][0] = __uint_as_float(d01[0]);
            r.dn[tt][1] = __uint_as_float(d01[2]);
            r.dn[tt][2] = __uint_as_float(d23[0]);
            r.dn[tt][3] = __uint_as_float(d23[2]);
        }
        const int tok = t0 + tl;
#pragma unroll
        for (int i = 0; i < S::VW / 8; ++i) {
            const u32x4_t u = __builtin_amdgcn_raw_buffer_load_b128(
                rs_vw, (uint32_t)((tok * S::VW + hv * (S::VW / 2) + 4 * i) * 4), 0, 0);
            r.vw[i] = make_uint4(u[0], u[1], u[2], u[3]);
        }
        if constexpr (S::NG == 4) {
            const u32x2_t u = __builtin_amdgcn_raw_buffer_load_b64(rs_vs, (uint32_t)(tok * 8), 0, 0);
            r.sc[0] = u[0];
            r.sc[1] = u[1];
        } else {
            const u32x4_t u = __builtin_amdgcn_raw_buffer_load_b128(rs_vs, (uint32_t)(tok * S::NG * 2), 0, 0);
#pragma unroll
            for (int i = 0; i < S::NG / 2; ++i) r.sc[i] = u[i];
        }
    };

    // ping-pong register buffers: the loads of the block after next are issued right
    // after a buffer is consumed, and every load is issued unconditionally (clamped to the
    // last token) so that each wait covers exactly the buffer about to be used
    auto process = [&](const Blk &cur, int t0) {
        // ---- stage this block's value records and scales in the wave's LDS slots
#pragma unroll
        for (int i = 0; i < S::VW / 8; ++i) {
            uint32_t *dst = &sm.val[wave][tl][hv * (S::VW / 2) + 4 * i];
            dst[0] = cur.vw[i].x; dst[1] = cur.vw[i].y; dst[2] = cur.vw[i].z; dst[3] = cur.vw[i].w;
        }
        if (hv == 0) {
#pragma unroll
            for (int i = 0; i < S::NG / 2; ++i) {
                sm.scl[wave][2 * i][tl] = f16_lo(cur.sc[i]);
                sm.scl[wave][2 * i + 1][tl] = f16_hi(cur.sc[i]);
            }
        }

        // ---- scores: centroid part and sign part in separate accumulators (4 independent
        //      MFMA chains); the sign part's A carries (2z - 1) g_t sqrt(pi/2)/d, hi + lo
        f32x4_t acc_m[2], acc_q[2];
        uint32_t kg_hi[2], kg_lo[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            acc_m[tt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
            acc_q[tt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
            _Float16 h, l;
            split_hl(-cur.an[tt].y * kQjl, h, l);  // negative: the sign bit is cleared where z = 1
            const uint32_t hb = __builtin_bit_cast(uint16_t, h), lb = __builtin_bit_cast(uint16_t, l);
            kg_hi[tt] = hb | (hb << 16);
            kg_lo[tt] = lb | (lb << 16);
        }
#pragma unroll
        for (int ks = 0; ks < S::NKS; ++ks) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const uint32_t word = cur.kw[tt][ks];
                half8_t am, aqh, aql;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t mr = lut[((word >> (8 * r)) & 0xffu) * kLutCopies];
                    const uint32_t zs = (word << (12 - 4 * r)) & 0x80008000u;
                    const half2_t hm = __builtin_bit_cast(half2_t, mr);
                    const half2_t hh = __builtin_bit_cast(half2_t, kg_hi[tt] ^ zs);
                    const half2_t hl = __builtin_bit_cast(half2_t, kg_lo[tt] ^ zs);
                    am[2 * r] = hm[0]; am[2 * r + 1] = hm[1];
                    aqh[2 * r] = hh[0]; aqh[2 * r + 1] = hh[1];
                    aql[2 * r] = hl[0]; aql[2 * r + 1] = hl[1];
                }
                acc_m[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(am, bm_hi[ks], acc_m[tt], 0, 0, 0);
                acc_q[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aqh, bq[ks], acc_q[tt], 0, 0, 0);
                acc_m[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(am, bm_lo[ks], acc_m[tt], 0, 0, 0);
                acc_q[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aql, bq[ks], acc_q[tt], 0, 0, 0);
            }
        }
        // lane (n16, q) holds head n16 (if < G) for rows 4q..4q+3 of each tile
        float lg[2][4];
        float lmax = -INFINITY;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t tok = t0 + 16 * tt + 4 * q + i;
                const bool ok = (n16 < G) && (tok < t_end);
                lg[tt][i] = ok ? cur.dn[tt][i] * (acc_m[tt][i] + acc_q[tt][i]) * a.scale : -INFINITY;
                lmax = fmaxf(lmax, lg[tt][i]);
            }

        // ---- online softmax with a reference max that only moves when a logit exceeds it
        //      (rare after the first block); p <= 1 always
        if (__ballot(lmax > m_ref)) {
            float mb = lmax;
            mb = fmaxf(mb, __shfl_xor(mb, 16));
            mb = fmaxf(mb, __shfl_xor(mb, 32));
            const float m_new = fmaxf(m_ref, mb);
            const float corr = (m_ref == -INFINITY) ? 0.f : __expf(m_ref - m_new);
            if (n16 < G && q == 0) sm.corr[wave][n16] = corr;
            l_part *= corr;
            m_ref = m_new;
            wave_sync();
#pragma unroll
            for (int p = 0; p < S::NPASS; ++p) {
                const int n = n16 + 16 * p;
                const float c = (n < S::NCOL) ? sm.corr[wave][n / S::NG] : 0.f;
                sumb[p] *= c;
#pragma unroll
                for (int t = 0; t < S::NT; ++t) acc_v[p][t] *= c;
            }
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            f32x4_t pv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pv[i] = (n16 < G) ? __expf(lg[tt][i] - m_ref) : 0.f;
                l_part += pv[i];
            }
            if (n16 < G) *reinterpret_cast<f32x4_t *>(&sm.pb[wave][n16][16 * tt + 4 * q]) = pv;
        }
        wave_sync();

        // ---- values: B = p * scale in columns (head, group), hi + lo; A = codes of row n16
        half8_t bv_hi[S::NPASS], bv_lo[S::NPASS];
#pragma unroll
        for (int p = 0; p < S::NPASS; ++p) {
            const int n = n16 + 16 * p;
            const bool col = n < S::NCOL;
            const int gg = col ? n / S::NG : 0, grp = col ? n % S::NG : 0;
            const f32x4_t p0 = *reinterpret_cast<const f32x4_t *>(&sm.pb[wave][gg][8 * q]);
            const f32x4_t p1 = *reinterpret_cast<const f32x4_t *>(&sm.pb[wave][gg][8 * q + 4]);
            const f32x4_t s0 = *reinterpret_cast<const f32x4_t *>(&sm.scl[wave][grp][8 * q]);
            const f32x4_t s1 = *reinterpret_cast<const f32x4_t *>(&sm.scl[wave][grp][8 * q + 4]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float bvv = col ? (e < 4 ? p0[e] * s0[e] : p1[e - 4] * s1[e - 4]) : 0.f;
                sumb[p] += bvv;
                _Float16 h, l;
                split_hl(bvv, h, l);
                bv_hi[p][e] = h;
                bv_lo[p][e] = l;
            }
        }
        // row n16's code run of each of the lane's 8 tokens (8q .. 8q+7), as halfword pairs
        // z[k][r] = (halfword k of token 8q+2r) | (halfword k of token 8q+2r+1) << 16
        uint32_t z[S::H][4];
#pragma unroll
        for (int k = 0; k < S::H; ++k) {
            const int hw = n16 * S::H + k;       // halfword index inside the record
            const int wi = hw >> 1;
            const uint32_t sel = (hw & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t wa = sm.val[wave][8 * q + 2 * r][wi];
                const uint32_t wb = sm.val[wave][8 * q + 2 * r + 1][wi];
                z[k][r] = __builtin_amdgcn_perm(wb, wa, sel);
            }
        }
        constexpr uint32_t kMask = ((1u << VB) - 1u) * 0x00010001u;
        const half2_t k1024 = {(_Float16)1024.f, (_Float16)1024.f};
#pragma unroll
        for (int t = 0; t < S::NT; ++t) {
            const int k = (VB * t) / 16, sh = (VB * t) % 16;
            half8_t av;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t x = ((z[k][r] >> sh) & kMask) | 0x64006400u;
                const half2_t hv2 = __builtin_bit_cast(half2_t, x) - k1024;
                av[2 * r] = hv2[0];
                av[2 * r + 1] = hv2[1];
            }
#pragma unroll
            for (int p = 0; p < S::NPASS; ++p) {
                acc_v[p][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv_hi[p], acc_v[p][t], 0, 0, 0);
                acc_v[p][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv_lo[p], acc_v[p][t], 0, 0, 0);
            }
        }
        wave_sync();  // this wave's LDS slots are rewritten by its next block
    };
    const int stride = kWaves * kBlock;
    const int t_stop = (int)t_end;
    int t0 = (int)t_begin + wave * kBlock;
    if (t0 < t_stop) {
        Blk bufa, bufb;
        load_blk(t0, bufa);
        load_blk(t0 + stride, bufb);
        while (true) {
            process(bufa, t0);
            load_blk(t0 + 2 * stride, bufa);
            t0 += stride;
            if (t0 >= t_stop) break;
            process(bufb, t0);
            load_blk(t0 + 2 * stride, bufb);
            t0 += stride;
            if (t0 >= t_stop) break;
        }
    }

    // ---- wave results: m, l per head; o[g][c] = acc - (HALF - 1/2) * column sum of B
    l_part += __shfl_xor(l_part, 16);
    l_part += __shfl_xor(l_part, 32);
#pragma unroll
    for (int p = 0; p < S::NPASS; ++p) {
        sumb[p] += __shfl_xor(sumb[p], 16);
        sumb[p] += __shfl_xor(sumb[p], 32);
    }
    if (n16 < G && q == 0) {
        sm.wm[wave][n16] = m_ref;
        sm.wl[wave][n16] = l_part;
    }
#pragma unroll
    for (int p = 0; p < S::NPASS; ++p) {
        const int n = n16 + 16 * p;
        if (n >= S::NCOL) continue;
        const int gg = n / S::NG, grp = n % S::NG;
#pragma unroll
        for (int t = 0; t < S::NT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = (4 * q + i) * S::NT + t;
                if (c / 32 == grp) sm.wo[wave][gg][c] = acc_v[p][t][i] - (float)(S::HALF - 0.5f) * sumb[p];
            }
    }
}

// ------------------------------------------------------------------ ring split (VALU)
template <int D, int VB, int G>
__device__ void ring_split(const DecodeArgs &a, DecodeSmem<D, VB, G> &sm, int bk, int b, int kvh,
                           float (&m_out)[G], float (&l_out)[G], float (&o_out)[G], int jv, int part) {
    using S = DecodeShape<D, VB, G>;
    const int tid = threadIdx.x;
    for (int i = tid; i < G * D; i += kThreads) {
        const int g = i / D, j = i - g * D;
        sm.ring_q[g][j] = a.prep[((int64_t)b * a.hq + kvh * G + g) * (3 * D + 4) + 2 * D + j];
    }
    __syncthreads();
    float m_run[G], l_run[G], o[G];
#pragma unroll
    for (int g = 0; g < G; ++g) { m_run[g] = -INFINITY; l_run[g] = 0.f; o[g] = 0.f; }
    for (int c0 = 0; c0 < a.n_ring; c0 += kRingChunk) {
        const int cnt = min(kRingChunk, a.n_ring - c0);
        float lg[G];
        if (tid < cnt) {
            const uint16_t *kr = a.rk + ((int64_t)bk * a.buffer_size + c0 + tid) * D;
            float acc[G];
#pragma unroll
            for (int g = 0; g < G; ++g) acc[g] = 0.f;
            for (int i = 0; i < D; i += 8) {
                float kv8[8];
                load8(kr, i, kv8, f16_tag{});
#pragma unroll
                for (int e = 0; e < 8; ++e)
#pragma unroll
                    for (int g = 0; g < G; ++g) acc[g] = fmaf(sm.ring_q[g][i + e], kv8[e], acc[g]);
            }
#pragma unroll
            for (int g = 0; g < G; ++g) lg[g] = acc[g] * a.scale;
        } else {
#pragma unroll
            for (int g = 0; g < G; ++g) lg[g] = -INFINITY;
        }
        float mx[G];
#pragma unroll
        for (int g = 0; g < G; ++g) mx[g] = lg[g];
        block_reduce<G, true>(mx, sm.ring_red);
        float pe[G], corr[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float mnew = fmaxf(m_run[g], mx[g]);
            corr[g] = (m_run[g] == -INFINITY) ? 0.f : __expf(m_run[g] - mnew);
            pe[g] = (tid < cnt) ? __expf(lg[g] - mnew) : 0.f;
            sm.ring_p[g][tid] = pe[g];
            m_run[g] = mnew;
        }
        block_reduce<G, false>(pe, sm.ring_red);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            l_run[g] = l_run[g] * corr[g] + pe[g];
            o[g] *= corr[g];
        }
        for (int tt = part; tt < cnt; tt += S::PARTS) {
            const float vh = (float)__builtin_bit_cast(
                _Float16, a.rv[((int64_t)bk * a.buffer_size + c0 + tt) * D + jv]);
#pragma unroll
            for (int g = 0; g < G; ++g) o[g] = fmaf(sm.ring_p[g][tt], vh, o[g]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int g = 0; g < G; ++g) { m_out[g] = m_run[g]; l_out[g] = l_run[g]; o_out[g] = o[g]; }
}

// ------------------------------------------------------------------ main kernel
template <int D, int VB, int G>
__global__ __launch_bounds__(kThreads) void k_decode_main(DecodeArgs a) {
    using S = DecodeShape<D, VB, G>;
    __shared__ DecodeSmem<D, VB, G> sm;
    const int tid = threadIdx.x;
    const int split = blockIdx.x;
    const int bk = blockIdx.y;  // b * hkv + kv head == slice
    const int b = bk / a.hkv, kvh = bk - b * a.hkv;
    const int n_total = a.n_split_total;
    float *pp = a.partial + ((int64_t)bk * n_total + split) * G * (D + 2);

    if (split < a.n_split) {
        // byte -> (c[low nibble & 7], c[high nibble & 7]) as an fp16 pair, one copy per bank
        {
            const float c_lo = a.centroids[tid & 7];
            const float c_hi = a.centroids[(tid >> 4) & 7];
            const uint32_t e = pack_half2(c_lo, c_hi);
#pragma unroll
            for (int cp = 0; cp < kLutCopies; ++cp) sm.lut[tid * kLutCopies + cp] = e;
        }
        __syncthreads();
        const int64_t t_begin = (int64_t)split * a.per_split;
        const int64_t t_end = min(a.n_packed, t_begin + a.per_split);
        packed_wave<D, VB, G>(a, sm, bk, b, kvh, t_begin, t_end);
        __syncthreads();
        // combine the four waves
        for (int i = tid; i < G * D; i += kThreads) {
            const int g = i / D, j = i - g * D;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.wm[w][g]);
            float L = 0.f, O = 0.f;
            if (M != -INFINITY) {
#pragma unroll
                for (int w = 0; w < kWaves; ++w) {
                    if (sm.wm[w][g] == -INFINITY) continue;
                    const float f = __expf(sm.wm[w][g] - M);
                    L = fmaf(sm.wl[w][g], f, L);
                    O = fmaf(sm.wo[w][g][j], f, O);
                }
            }
            pp[g * (D + 2) + j] = O;
            if (j == 0) {
                pp[g * (D + 2) + D] = M;
                pp[g * (D + 2) + D + 1] = L;
            }
        }
    } else {
        float m_r[G], l_r[G], o_r[G];
        const int jv = tid % D, part = tid / D;
        ring_split<D, VB, G>(a, sm, bk, b, kvh, m_r, l_r, o_r, jv, part);
        if constexpr (S::PARTS > 1) {
            if (part > 0)
#pragma unroll
                for (int g = 0; g < G; ++g) sm.wo[part - 1][g][jv] = o_r[g];
            __syncthreads();
            if (part == 0)
#pragma unroll
                for (int pt = 0; pt < S::PARTS - 1; ++pt)
#pragma unroll
                    for (int g = 0; g < G; ++g) o_r[g] += sm.wo[pt][g][jv];
        }
        if (part == 0) {
#pragma unroll
            for (int g = 0; g < G; ++g) pp[g * (D + 2) + jv] = o_r[g];
            if (jv == 0)
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    pp[g * (D + 2) + D] = m_r[g];
                    pp[g * (D + 2) + D + 1] = l_r[g];
                }
        }
    }

    // ---- ticket: the last split of this (batch, kv head) merges all partials
    __threadfence();
    __syncthreads();
    if (tid == 0)
        sm.ticket = __hip_atomic_fetch_add(a.tickets + bk, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (sm.ticket != (unsigned)(n_total - 1)) return;
    __threadfence();
    const float *base = a.partial + (int64_t)bk * n_total * G * (D + 2);
    {
        const int lane = tid & 63, wv = tid >> 6;
        for (int g = wv; g < G; g += kWaves) {
            float mx = -INFINITY;
            for (int sp = lane; sp < n_total; sp += 64) mx = fmaxf(mx, base[(sp * G + g) * (D + 2) + D]);
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
            float ls = 0.f;
            for (int sp = lane; sp < n_total; sp += 64) {
                const float ms = base[(sp * G + g) * (D + 2) + D];
                const float f = (ms == -INFINITY) ? 0.f : __expf(ms - mx);
                sm.merge_f[g][sp] = f;
                ls = fmaf(base[(sp * G + g) * (D + 2) + D + 1], f, ls);
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) ls += __shfl_xor(ls, o);
            if (lane == 0) sm.ml[g] = ls;
        }
    }
    __syncthreads();
    for (int i = tid; i < G * D; i += kThreads) {
        const int g = i / D, j = i - g * D;
        float O = 0.f;
#pragma unroll 8
        for (int sp = 0; sp < n_total; ++sp) O = fmaf(sm.merge_f[g][sp], base[(sp * G + g) * (D + 2) + j], O);
        const float L = sm.ml[g];
        a.out[((int64_t)b * a.hq + kvh * G + g) * D + j] = L > 0.f ? O / L : 0.f;
    }
    if (tid == 0) __hip_atomic_store(a.tickets + bk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ ring append
template <typename Tag, int D>
__global__ __launch_bounds__(256) void k_ring_append(const void *kn, const void *vn, uint16_t *rk, uint16_t *rv,
                                                     int n_slices, int buffer_size, int slot) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // one thread per 8 elements
    const int64_t total = (int64_t)n_slices * D / 8;
    if (i >= total) return;
    const int64_t sl = i / (D / 8);
    const int c = (int)(i - sl * (D / 8)) * 8;
    float kv[8], vv[8];
    load8(kn, sl * D + c, kv, Tag{});
    load8(vn, sl * D + c, vv, Tag{});
    uint32_t kp[4], vp[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        kp[e] = f32_to_f16_bits(kv[2 * e]) | ((uint32_t)f32_to_f16_bits(kv[2 * e + 1]) << 16);
        vp[e] = f32_to_f16_bits(vv[2 * e]) | ((uint32_t)f32_to_f16_bits(vv[2 * e + 1]) << 16);
    }
    const int64_t off = (sl * buffer_size + slot) * D + c;
    *reinterpret_cast<uint4 *>(rk + off) = make_uint4(kp[0], kp[1], kp[2], kp[3]);
    *reinterpret_cast<uint4 *>(rv + off) = make_uint4(vp[0], vp[1], vp[2], vp[3]);
}

// ------------------------------------------------------------------ launchers
template <typename Tag>
static hipError_t launch_prep_t(int d, const DecodeArgs &a, hipStream_t st) {
    const unsigned grid = (unsigned)(a.batch * a.hq);
    if (d == 128)
        hipLaunchKernelGGL((k_decode_prep<Tag, 128>), dim3(grid), dim3(128), 0, st, a);
    else
        hipLaunchKernelGGL((k_decode_prep<Tag, 256>), dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <int D, int VB>
static hipError_t launch_main_dv(int G, const DecodeArgs &a, hipStream_t st) {
    dim3 grid((unsigned)a.n_split_total, (unsigned)(a.batch * a.hkv));
    switch (G) {
        case 1: hipLaunchKernelGGL((k_decode_main<D, VB, 1>), grid, dim3(kThreads), 0, st, a); break;
        case 2: hipLaunchKernelGGL((k_decode_main<D, VB, 2>), grid, dim3(kThreads), 0, st, a); break;
        case 4: hipLaunchKernelGGL((k_decode_main<D, VB, 4>), grid, dim3(kThreads), 0, st, a); break;
        default: hipLaunchKernelGGL((k_decode_main<D, VB, 8>), grid, dim3(kThreads), 0, st, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_decode(int d, int vb, int G, tq_dtype qdt, const DecodeArgs &a, hipStream_t st) {
    hipError_t e;
    switch (qdt) {
        case TQ_F32: e = launch_prep_t<f32_tag>(d, a, st); break;
        case TQ_BF16: e = launch_prep_t<bf16_tag>(d, a, st); break;
        default: e = launch_prep_t<f16_tag>(d, a, st); break;
    }
    if (e != hipSuccess) return e;
    if (d == 128 && vb == 2) return launch_main_dv<128, 2>(G, a, st);
    if (d == 128 && vb == 4) return launch_main_dv<128, 4>(G, a, st);
    if (d == 256 && vb == 2) return launch_main_dv<256, 2>(G, a, st);
    return launch_main_dv<256, 4>(G, a, st);
}

hipError_t launch_ring_append(int d, tq_dtype dt, const void *kn, const void *vn, uint16_t *rk, uint16_t *rv,
                              int n_slices, int buffer_size, int slot, hipStream_t st) {
    const int64_t total = (int64_t)n_slices * d / 8;
    const unsigned grid = (unsigned)((total + 255) / 256);
#define TQ_RING(TAG, DD) hipLaunchKernelGGL((k_ring_append<TAG, DD>), dim3(grid), dim3(256), 0, st, kn, vn, rk, rv, \
                                            n_slices, buffer_size, slot)
    if (d == 128) {
        if (dt == TQ_F32) TQ_RING(f32_tag, 128);
        else if (dt == TQ_BF16) TQ_RING(bf16_tag, 128);
        else TQ_RING(f16_tag, 128);
    } else {
        if (dt == TQ_F32) TQ_RING(f32_tag, 256);
        else if (dt == TQ_BF16) TQ_RING(bf16_tag, 256);
        else TQ_RING(f16_tag, 256);
    }
#undef TQ_RING
    return hipGetLastError();
}

}  // namespace tq

// tq_quantize.hip -- compression of keys and values into the packed store (gfx950).
//
// Method: hotelren.com guide "企业官网建设流程全解析", section 二: (1) random orthogonal
// rotation, (2) Lloyd-Max quantisation of the rotated unit key against the Beta-law
// codebook, (3) one QJL sign bit per coordinate for the residual, (4) symmetric 2/4-bit
// value quantisation in groups of 32 with a per-group scale, (5) bit packing.
//
// k_quant_kv: one wave per tile of R tokens (R = 32 at d = 128 on v_mfma_f32_32x32x16,
// R = 16 at d = 256, and at d = 128 for short inputs, on v_mfma_f32_16x16x32); the
// KG = 64 / R lanes of a token each hold D / KG of its coordinates and values.
//   * values first: the lane's values are whole groups of 32, so group max, fp16 scale and
//     exact floor (see quant_group) are in-lane;
//   * rotation: the Walsh-Hadamard product H (sigma o x) runs on the matrix cores with the
//     raw 16-bit inputs as the B operand (exact: H has entries +-1, sigma is a sign flip
//     applied by XOR on the raw words) and fp32 accumulation.  H factorises over the index
//     bits, so the A operand of every (output tile, k-step) pair is one of two per-lane
//     +-1 fragments, possibly negated;
//   * the accumulator layout leaves lane group g of a token with the coordinates
//     slot_coord(f, g); encode is elementwise on them: the codebook is antisymmetric with
//     b_3 = 0, so |y| is compared with the row's thresholds for the three positive
//     boundaries, and the side decides the sign (the oracle resolves ties as
//     idx = #{i : u > b_i}; here a tie within a few ulp may take either neighbouring cell);
//   * QJL: the projection is computed transposed, D = S R^T with the residual (scaled by
//     2^8, split into fp16 hi + lo) as the B operand, so the accumulator hands every lane
//     the projections of exactly the coordinates it encoded; byte permutes gather their
//     sign bits into the nibbles;
//   * nibble half-words of a key word live in the two lanes g, g ^ 1; one permlane swap
//     and two byte permutes assemble the words.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "tq.h"
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// tile shape: RR tokens per wave, 32 (v_mfma_f32_32x32x16, d = 128 only) or 16
// (v_mfma_f32_16x16x32)
template <int D, int RR, int KB = 3>
struct KeyShape {
    static constexpr int R = RR;                  // tokens per wave (MFMA M = N)
    static constexpr int KG = 64 / R;             // lanes per token
    static constexpr int K = 8 * KG;              // MFMA k per instruction
    static constexpr int NS = D / K;              // rotation k-steps
    static constexpr int NJ = D / R;              // rotation / projection output tiles
    static constexpr int RPT = R * R / 64;        // accumulator registers per tile and lane
    static constexpr int NV = D / KG;             // coordinates per lane (64, or 32 at d = 128, R = 16)
    static constexpr int NQ = NV / 8;             // projection k-steps
    static constexpr int KW = (KB + 1) * D / 32;  // key words per record
    static constexpr int NP = NV / 8;             // u32 registers of nibble half-word pairs (KB = 3)
    static constexpr int NVG = NV / 32;           // value groups per lane
    static constexpr int NCW = KB * D / 32;       // code-plane words (KB = 1, 2, 4)
    static_assert(R == 16 || (R == 32 && D <= 128), "tile shapes");
    static_assert(KB == 3 || R == 32, "two-plane key records are assembled from 32-token tiles");
};

template <int R>
using acc_t = std::conditional_t<R == 32, f32x16_t, f32x4_t>;

// coordinate held in accumulator slot f (tile f / RPT, register f % RPT) by lane group g:
// the MFMA result layout (row 4 g + (r & 3) + 4 KG (r >> 2) of the tile)
template <int D, int RR>
__device__ __host__ constexpr int slot_coord(int f, int g) {
    using S = KeyShape<D, RR>;
    return S::R * (f / S::RPT) + 4 * g + ((f % S::RPT) & 3) + 4 * S::KG * ((f % S::RPT) >> 2);
}

// rotation A operand of (output tile jt, k-step s): fragment variant and global sign, from
// popcount((R jt + i) & (K s + k)) split over the index bits
template <int RR>
__device__ __host__ constexpr int h_variant(int jt, int s) {
    return RR == 32 ? (s & 1) : (jt & 1);
}
template <int RR>
__device__ __host__ constexpr int h_negated(int jt, int s) {
    return __builtin_popcount(RR == 32 ? (jt & (s >> 1)) : ((jt >> 1) & s)) & 1;
}

template <int R, typename Tag>
__device__ __forceinline__ acc_t<R> mfma_in(u32x4_t a, u32x4_t b, acc_t<R> c) {
    if constexpr (R == 32) {
        if constexpr (std::is_same_v<Tag, f16_tag>)
            return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a),
                                                          __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                           __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    } else {
        if constexpr (std::is_same_v<Tag, f16_tag>)
            return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                          __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                           __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
}

template <int R>
__device__ __forceinline__ acc_t<R> mfma_f16(u32x4_t a, u32x4_t b, acc_t<R> c) {
    if constexpr (R == 32)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b),
                                                      c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b),
                                                      c, 0, 0, 0);
}

// exact split of an fp32 value into three bf16 parts (x = hi + mid + lo)
__device__ __forceinline__ void split3_bf16(float x, uint16_t &hi, uint16_t &mid, uint16_t &lo) {
    const __bf16 h = (__bf16)x;
    const float r1 = x - (float)h;
    const __bf16 m = (__bf16)r1;
    const __bf16 l = (__bf16)(r1 - (float)m);
    hi = __builtin_bit_cast(uint16_t, h);
    mid = __builtin_bit_cast(uint16_t, m);
    lo = __builtin_bit_cast(uint16_t, l);
}

// ------------------------------------------------------------------------------ values of one group
// Codes of one group: code = clamp(floor(v / s), -HALF, HALF - 1) + HALF, floor exact.
// Fast form (16-bit inputs, normal fp16 s): v / s is then either an integer or at least
// 2^-11 away from every integer (or inside (-1, 1)), so floor(p + |v| 2^-20 / s), p = v * r
// rounded with r = 1/s from v_rcp_f32 (within 1 ulp), is exact: the nudge (|v / s| 2^-20,
// eight times the rounding error of p) lifts exact integers that rounding pushed below, and
// is far too small to cross a non-integer.  Otherwise the estimate (off by at most one) is
// corrected with exact products (q + 1) s and q s.
__device__ __forceinline__ int floor_to_int(float x) {
    int q;
    asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(q) : "v"(x));
    return q;
}
template <int VB, bool Exact>
__device__ __forceinline__ void quant_group(const float (&v)[32], float sc, uint32_t (&wd)[VB]) {
    constexpr int HALF = 1 << (VB - 1);
    constexpr int PER = 32 / VB;  // codes per word
    const float rinv = __builtin_amdgcn_rcpf(sc);
    const float nudge = rinv * 0x1p-20f;
    // code offset HALF in every field
    constexpr uint32_t kOff = VB == 2 ? 0xAAAAAAAAu : 0x88888888u;
#pragma unroll
    for (int w = 0; w < VB; ++w) {
        uint32_t acc = kOff;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const float x = v[w * PER + e];
            int q;
            if constexpr (Exact) {
                float qf = floorf(x * rinv);
                if ((qf + 1.f) * sc <= x) qf += 1.f;
                else if (qf * sc > x) qf -= 1.f;
                q = (int)fminf(fmaxf(qf, (float)-HALF), (float)(HALF - 1));
            } else {
                q = floor_to_int(fmaf(fabsf(x), nudge, x * rinv));
                q = min(max(q, -HALF), HALF - 1);
            }
            // acc += q << (VB e): one shift-add per code
            asm("v_lshl_add_u32 %0, %1, %2, %0" : "+v"(acc) : "v"(q), "i"(VB * e));
        }
        wd[w] = acc;
    }
}

// ------------------------------------------------------------------------------ keys (and values)
// Launch shape: one persistent 12-wave workgroup per CU (one LDS copy of S: 33 KB at d = 128,
// 130 KB at d = 256), 3 waves per SIMD (<= 168 VGPRs).  Workgroup g owns the wave tiles (R
// rows each) g, g + G, g + 2G, ... and its waves take the next one from an LDS counter, so
// the waves of a CU finish together.  (With several workgroups per CU on a static split, the
// first-dispatched one was measured to finish at about half the time of the last.)
// Measured alternative: 16-token waves at d = 128 (5 per SIMD) are slower -- each S fragment
// read from LDS then serves half as many tokens.
template <int D>
constexpr int kKeyGroupWaves = 12;

// waves per workgroup (at least 4, which the S copy relies on): 12 (one workgroup per CU)
// once the waves have a tile each on average, else 4, so that short inputs spread over more
// CUs (d = 256: its LDS copy of S allows one workgroup per CU, so always 12)
static int quant_waves_per_group(int d, int64_t tiles, int64_t cus) {
    if (d == 256) return 12;
    return tiles >= cus * 12 ? 12 : 4;
}
template <int D>
constexpr int kKeyWavesPerSimd = 3;
// S rows in LDS are padded by 8 bytes (2 banks): the 8-byte A-fragment reads of 32
// consecutive rows at one column then fall into distinct banks
template <int D>
constexpr int kSRow = D + 4;  // halfwords

// row -> (slice, token) without a 64-bit integer division: the quotient from the fp64
// product is off by at most one for rows < 2^52 and is corrected exactly
__device__ __forceinline__ void split_row(int64_t r, int64_t n_tok, double inv, int64_t &sl, int64_t &t) {
    int64_t q = (int64_t)((double)r * inv);
    int64_t rem = r - q * n_tok;
    if (rem < 0) {
        q -= 1;
        rem += n_tok;
    } else if (rem >= n_tok) {
        q += 1;
        rem -= n_tok;
    }
    sl = q;
    t = rem;
}

template <typename Tag, int D, int VB, int RR, int KB>
__global__ __launch_bounds__(64 * kKeyGroupWaves<D>)
__attribute__((amdgpu_waves_per_eu(kKeyWavesPerSimd<D>, kKeyWavesPerSimd<D>)))
void k_quant_kv(QuantArgs a) {
    using S = KeyShape<D, RR, KB>;
    constexpr int L = 1 << KB;         // codebook size
    constexpr int NPOS = L / 2;        // cells on each side of 0 (the codebook is antisymmetric)
    constexpr uint32_t kTag = L - 1;   // tag bits of the tagged centroids
    constexpr int R = S::R;
    constexpr bool kF32 = std::is_same_v<Tag, f32_tag>;
    constexpr bool kF16 = std::is_same_v<Tag, f16_tag>;
    constexpr int RAWW = kF32 ? 8 : 4;

    // sigma as XOR masks on 16-bit pairs: word p has bit 15 = sigma_2p, bit 31 = sigma_2p+1
    __shared__ __attribute__((aligned(16))) uint32_t smask[D / 2];
    __shared__ __attribute__((aligned(16))) uint16_t sS[D * kSRow<D>];
    if (threadIdx.x < D / 2) {
        const int c = 2 * threadIdx.x;
        const uint32_t w = a.sign_bits[c >> 5] >> (c & 31);
        smask[threadIdx.x] = ((w & 1u) << 15) | ((w & 2u) << 30);
    }
    {
        // 16-byte chunks of S: every load of the thread issued before the LDS stores (the
        // block has at least 256 threads at d = 128 and 768 at d = 256)
        constexpr int NCH = D * D / 8, KMAX = D <= 128 ? NCH / 256 : (NCH + 767) / 768;
        uint4 x[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const int i = threadIdx.x + k * blockDim.x;
            if (i < NCH) x[k] = *reinterpret_cast<const uint4 *>(a.S + (int64_t)(i / (D / 8)) * D + (i % (D / 8)) * 8);
        }
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const int i = threadIdx.x + k * blockDim.x;
            if (i < NCH) {
                uint2 *dst = reinterpret_cast<uint2 *>(&sS[(i / (D / 8)) * kSRow<D> + (i % (D / 8)) * 8]);
                dst[0] = make_uint2(x[k].x, x[k].y);
                dst[1] = make_uint2(x[k].z, x[k].w);
            }
        }
    }
    // this workgroup's wave tiles blockIdx.x + c * gridDim.x (c = 0, 1, ...: all workgroups
    // move through the rows together), handed out one at a time
    const int64_t n_tiles = (a.n_rows + R - 1) / R;
    __shared__ unsigned long long next_tile;
    if (threadIdx.x == 0) next_tile = 0ull;
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int n = lane % R, g = lane / R;
    const double inv_tok = 1.0 / (double)a.n_tokens;

    // raw inputs of one row: k-step s holds coordinates K s + 8 g + 0..7 (rows past the end
    // are clamped to the last row, so every lane reads real data)
    uint32_t raw[S::NS][RAWW];
    auto load_raw = [&](int64_t sl, int64_t t) {
        const int64_t in_off = sl * a.in_slice_stride + t * D + 8 * g;
#pragma unroll
        for (int s = 0; s < S::NS; ++s) {
            if constexpr (kF32) {
                const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const float *>(a.k) + in_off + S::K * s);
                const uint4 x0 = p[0], x1 = p[1];
                raw[s][0] = x0.x; raw[s][1] = x0.y; raw[s][2] = x0.z; raw[s][3] = x0.w;
                raw[s][4] = x1.x; raw[s][5] = x1.y; raw[s][6] = x1.z; raw[s][7] = x1.w;
            } else {
                const uint4 x =
                    *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.k) + in_off + S::K * s);
                raw[s][0] = x.x; raw[s][1] = x.y; raw[s][2] = x.z; raw[s][3] = x.w;
            }
        }
    };

    // rotation A fragments: lane (row i = n, group g), element e <-> k = 8 g + e, the two
    // variants v of (-1)^popcount(i & k) (R = 32: times (-1)^(i_4 v); R = 16: (-1)^(k_4 v))
    u32x4_t hf[2];
    {
        const uint32_t one = kF16 ? 0x3C00u : 0x3F80u;
#pragma unroll
        for (int v = 0; v < 2; ++v)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                uint32_t pair = 0;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int k = 8 * g + 2 * w + hh;
                    const int par = __builtin_popcount(n & k & 15) +
                                    (R == 32 ? ((n >> 4) & 1) * v : ((k >> 4) & 1) * v);
                    pair |= (one | ((uint32_t)(par & 1) << 15)) << (16 * hh);
                }
                hf[v][w] = pair;
            }
    }
    // the positive decision boundaries b_{L/2} < ... < b_{L-2} (the codebook is antisymmetric
    // with b_{L/2-1} = 0)
    float BP[NPOS > 1 ? NPOS - 1 : 1];
#pragma unroll
    for (int k = 0; k + 1 < NPOS; ++k) BP[k] = a.boundaries[NPOS + k];
    // tagged positive centroids: the binary16 value 2^8 c[L/2+k] in the upper half-word (exact:
    // the stored centroids are binary16 values well inside its range) and the index L/2 + k in
    // the low bits; negating the word as fp32 negates the binary16 value
    float M[NPOS];
#pragma unroll
    for (int k = 0; k < NPOS; ++k) {
        const _Float16 c16 = (_Float16)(256.f * a.centroids[NPOS + k]);
        M[k] = __uint_as_float(((uint32_t)__builtin_bit_cast(uint16_t, c16) << 16) | (uint32_t)(NPOS + k));
        asm volatile("" : "+v"(M[k]));
    }

    for (;;) {
        int64_t tile = 0;
        if (lane == 0) tile = (int64_t)atomicAdd(&next_tile, 1ull) * gridDim.x + blockIdx.x;
        tile = (int64_t)__builtin_amdgcn_readfirstlane((int)tile) |
               ((int64_t)__builtin_amdgcn_readfirstlane((int)(tile >> 32)) << 32);
        if (tile >= n_tiles) break;
        const int64_t row = tile * R + n;
        int64_t sl, t;
        split_row(row < a.n_rows ? row : a.n_rows - 1, a.n_tokens, inv_tok, sl, t);
        load_raw(sl, t);
        // destination record, -1 past the last row
        const int64_t rec =
            row < a.n_rows ? record_index(a.bt, a.pt, a.pps, a.n_pages, a.cap, a.err, sl, a.dst_offset + t) : -1;

        // ---- the tile's values: this lane's NV coordinates g NV .. g NV + NV - 1 of its token
        //      (NVG groups of 32), loaded with the keys and quantised first (their registers are
        //      free again before the key encode needs its peak)
        constexpr int NVG = S::NVG;
        constexpr int VCH = NVG * (kF32 ? 8 : 4);  // 16-byte chunks of the lane's values
        uint4 vr[VCH];
        {
            const uint4 *vp = reinterpret_cast<const uint4 *>(static_cast<const unsigned char *>(a.v) +
                                                              ((sl * a.in_slice_stride + t * D + S::NV * g) * (kF32 ? 4 : 2)));
#pragma unroll
            for (int i = 0; i < VCH; ++i) vr[i] = vp[i];
        }

        // ---- values: groups NVG g .. NVG g + NVG - 1 of the token, all in this lane
        {
            constexpr int NG = D / 32;
            constexpr int VW = VB * D / 32;
            uint32_t wd[NVG][VB];
            uint16_t scb[NVG];
#pragma unroll
            for (int gi = 0; gi < NVG; ++gi) {
                float vv[32];
#pragma unroll
                for (int c = 0; c < VCH / NVG; ++c) {
                    const uint4 x = vr[gi * (VCH / NVG) + c];
                    if constexpr (kF32) {
                        vv[4 * c + 0] = __uint_as_float(x.x); vv[4 * c + 1] = __uint_as_float(x.y);
                        vv[4 * c + 2] = __uint_as_float(x.z); vv[4 * c + 3] = __uint_as_float(x.w);
                    } else if constexpr (kF16) {
                        vv[8 * c + 0] = f16_lo(x.x); vv[8 * c + 1] = f16_hi(x.x);
                        vv[8 * c + 2] = f16_lo(x.y); vv[8 * c + 3] = f16_hi(x.y);
                        vv[8 * c + 4] = f16_lo(x.z); vv[8 * c + 5] = f16_hi(x.z);
                        vv[8 * c + 6] = f16_lo(x.w); vv[8 * c + 7] = f16_hi(x.w);
                    } else {
                        vv[8 * c + 0] = bf16_lo(x.x); vv[8 * c + 1] = bf16_hi(x.x);
                        vv[8 * c + 2] = bf16_lo(x.y); vv[8 * c + 3] = bf16_hi(x.y);
                        vv[8 * c + 4] = bf16_lo(x.z); vv[8 * c + 5] = bf16_hi(x.z);
                        vv[8 * c + 6] = bf16_lo(x.w); vv[8 * c + 7] = bf16_hi(x.w);
                    }
                }
                float am = 0.f;
#pragma unroll
                for (int e = 0; e < 32; ++e) am = fmaxf(am, fabsf(vv[e]));
                const _Float16 sh = (_Float16)(am * (1.0f / (1 << (VB - 1))));
                const float sc = (float)sh;
                scb[gi] = __builtin_bit_cast(uint16_t, sh);
                if (sc == 0.f) {
#pragma unroll
                    for (int w = 0; w < VB; ++w) wd[gi][w] = VB == 2 ? 0xAAAAAAAAu : 0x88888888u;
                } else if (kF32 || sc < 0x1p-14f) {
                    quant_group<VB, true>(vv, sc, wd[gi]);
                } else {
                    quant_group<VB, false>(vv, sc, wd[gi]);
                }
            }
            if (rec >= 0) {
                uint32_t *dstv = a.vw + rec * VW + NVG * g * VB;
                if constexpr (NVG == 1) {
                    if constexpr (VB == 2) *reinterpret_cast<uint2 *>(dstv) = make_uint2(wd[0][0], wd[0][1]);
                    else *reinterpret_cast<uint4 *>(dstv) = make_uint4(wd[0][0], wd[0][1], wd[0][2], wd[0][3]);
                    a.vs[rec * NG + g] = scb[0];
                } else if constexpr (VB == 2) {
                    *reinterpret_cast<uint4 *>(dstv) = make_uint4(wd[0][0], wd[0][1], wd[1][0], wd[1][1]);
                } else {
                    uint4 *d4 = reinterpret_cast<uint4 *>(dstv);
                    d4[0] = make_uint4(wd[0][0], wd[0][1], wd[0][2], wd[0][3]);
                    d4[1] = make_uint4(wd[1][0], wd[1][1], wd[1][2], wd[1][3]);
                }
                if constexpr (NVG == 2)
                    *reinterpret_cast<uint32_t *>(a.vs + rec * NG + 2 * g) = scb[0] | ((uint32_t)scb[1] << 16);
            }
        }

        // ---- |k|^2 in fp32 (products of 16-bit inputs are exact; several partial sums)
        float ssp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < S::NS; ++s)
#pragma unroll
            for (int w = 0; w < RAWW; ++w) {
                if constexpr (kF32) {
                    const float x = __uint_as_float(raw[s][w]);
                    ssp[w & 3] = fmaf(x, x, ssp[w & 3]);
                } else if constexpr (kF16) {
                    typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
                    const h2_t x = __builtin_bit_cast(h2_t, raw[s][w]);
                    ssp[w] = __builtin_amdgcn_fdot2(x, x, ssp[w], false);
                } else {
                    typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
                    const b2_t x = __builtin_bit_cast(b2_t, raw[s][w]);
                    ssp[w] = __builtin_amdgcn_fdot2_f32_bf16(x, x, ssp[w], false);
                }
            }
        float ss = (ssp[0] + ssp[1]) + (ssp[2] + ssp[3]);
#pragma unroll
        for (int o = R; o < 64; o <<= 1) ss += __shfl_xor(ss, o);

        // ---- rotation on the matrix cores: y = H (sigma o x), fp32
        acc_t<R> y[S::NJ];
#pragma unroll
        for (int jt = 0; jt < S::NJ; ++jt) y[jt] = acc_t<R>{};
#pragma unroll
        for (int s = 0; s < S::NS; ++s) {
            const u32x4_t m4 = *reinterpret_cast<const u32x4_t *>(&smask[(S::K * s + 8 * g) / 2]);
            if constexpr (kF32) {
                u32x4_t bh, bm, bl;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    uint16_t h0, m0, l0, h1, m1, l1;
                    split3_bf16(__uint_as_float(raw[s][2 * w] ^ (m4[w] << 16)), h0, m0, l0);
                    split3_bf16(__uint_as_float(raw[s][2 * w + 1] ^ (m4[w] & 0x80000000u)), h1, m1, l1);
                    bh[w] = h0 | ((uint32_t)h1 << 16);
                    bm[w] = m0 | ((uint32_t)m1 << 16);
                    bl[w] = l0 | ((uint32_t)l1 << 16);
                }
#pragma unroll
                for (int jt = 0; jt < S::NJ; ++jt) {
                    const u32x4_t A0 = hf[h_variant<R>(jt, s)];
                    const u32x4_t A = h_negated<R>(jt, s) ? (A0 ^ 0x80008000u) : A0;
                    y[jt] = mfma_in<R, bf16_tag>(A, bh, y[jt]);
                    y[jt] = mfma_in<R, bf16_tag>(A, bm, y[jt]);
                    y[jt] = mfma_in<R, bf16_tag>(A, bl, y[jt]);
                }
            } else {
                u32x4_t b;
#pragma unroll
                for (int w = 0; w < 4; ++w) b[w] = raw[s][w] ^ m4[w];
#pragma unroll
                for (int jt = 0; jt < S::NJ; ++jt) {
                    const u32x4_t A0 = hf[h_variant<R>(jt, s)];
                    const u32x4_t A = h_negated<R>(jt, s) ? (A0 ^ 0x80008000u) : A0;
                    y[jt] = mfma_in<R, Tag>(A, b, y[jt]);
                }
            }
        }

        // ---- encode.  u' = 2^8 u = y inv256 with inv256 = 2^8 / sqrt(d |k|^2).  The cell of u
        //      follows from |y| against the row's thresholds b_i sqrt(d |k|^2) (i = 4, 5, 6, the
        //      positive boundaries; fp32 products, within a few ulp of the exact ones) and the
        //      side y > 0 or y <= 0 (a zero row gives u = 0, cell 3, as the count of boundaries
        //      strictly below 0).  A tie with a boundary may land in either neighbouring cell.
        const float knorm = sqrtf(ss);
        const float rsd = sqrtf((float)D * ss);
        const float inv256 = ss > 0.f ? 256.f / rsd : 0.f;
        float T[NPOS > 1 ? NPOS - 1 : 1];
#pragma unroll
        for (int k = 0; k + 1 < NPOS; ++k) T[k] = BP[k] * rsd;
        uint32_t P[S::NP];  // KB = 3: nibble half-words: slot f at bit 4 (f & 7) of P[f >> 3]
        // KB = 1, 2, 4: the lane's fields of the code plane and of the sign plane, at the
        // positions of lane group 0 (lane group g is shifted into place at the end)
        uint32_t CW[KB == 3 ? 1 : S::NCW], SW[KB == 3 ? 1 : D / 32];
        if constexpr (KB != 3) {
#pragma unroll
            for (int i = 0; i < S::NCW; ++i) CW[i] = 0;
#pragma unroll
            for (int i = 0; i < D / 32; ++i) SW[i] = 0;
        }
        float ggp[4] = {0.f, 0.f, 0.f, 0.f};
        // negated scaled residual -r' as fp16 hi + lo; projection k-step q = slots 8q .. 8q+7
        u32x4_t rhi[S::NQ], rlo[S::NQ];
        typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
        typedef float f2_t __attribute__((ext_vector_type(2)));
        // indices of slots (x, z) from one byte permute: bytes 0, 1 = the tags of x and z,
        // bytes 2, 3 = their sign bits replicated (selectors 11 and 9); index = tag, or
        // tag ^ 7 = 3 - k on the non-positive side
        auto pair_idx = [](uint32_t x, uint32_t z) {
            const uint32_t w = __builtin_amdgcn_perm(x, z, 0x090B0004u);
            return (w ^ (w >> 16)) & 0x0707u;
        };
#pragma unroll
        for (int f4 = 0; f4 < S::NV; f4 += 4) {
            uint32_t sb[4];
            float nr[4];
#pragma unroll
            for (int o = 0; o < 4; ++o) {
                const float yv = y[(f4 + o) / S::RPT][(f4 + o) % S::RPT];
                const float ay = fabsf(yv);
                // signed tagged centroid: sign = (y <= 0), low bits = L/2 + #{boundaries passed}
                float mt = M[0];
#pragma unroll
                for (int k = 0; k + 1 < NPOS; ++k) mt = ay > T[k] ? M[k + 1] : mt;
                sb[o] = __float_as_uint(yv > 0.f ? mt : -mt);
                // -r' = c[idx] - u', one fused product-add with the binary16 centroid as addend
                asm("v_fma_mix_f32 %0, -%1, %2, %3 op_sel:[0,0,1] op_sel_hi:[0,0,1]"
                    : "=v"(nr[o]) : "v"(yv), "v"(inv256), "v"(sb[o]));
                ggp[o] = fmaf(nr[o], nr[o], ggp[o]);
            }
            if constexpr (KB == 3) {
                // slots (0, 2) and (1, 3) of the four at nibble offsets 0 and 4 (plus 16 for the
                // upper four of a word); materialised here so that the centroids die now
                uint32_t q4 = pair_idx(sb[0], sb[2]) | (pair_idx(sb[1], sb[3]) << 4);
                asm volatile("" : "+v"(q4));
                if (f4 & 4) P[f4 >> 3] |= q4 << 16;
                else P[f4 >> 3] = q4;
            } else {
                // index = tag on the positive side, tag ^ (L - 1) = L/2 - 1 - k otherwise, into
                // the code plane at coordinate slot_coord(f, 0)
#pragma unroll
                for (int o = 0; o < 4; ++o) {
                    const int c = slot_coord<D, R>(f4 + o, 0);
                    const uint32_t ix = (sb[o] ^ (uint32_t)((int32_t)sb[o] >> 31)) & kTag;
                    CW[c / (32 / KB)] |= ix << (KB * (c % (32 / KB)));
                }
            }
#pragma unroll
            for (int o = 0; o < 4; o += 2) {
                const int f2 = f4 + o;
                const h2_t hi = __builtin_convertvector((f2_t){nr[o], nr[o + 1]}, h2_t);
                const uint32_t hb = __builtin_bit_cast(uint32_t, hi);
                // lo = fp16(-r' - hi), one rounding of an exact difference, per half
                uint32_t lb;
                asm("v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=&v"(lb) : "v"(hb), "v"(nr[o]));
                asm("v_fma_mixhi_f16 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
                    : "+v"(lb) : "v"(hb), "v"(nr[o + 1]));
                rhi[f2 >> 3][(f2 & 7) >> 1] = hb;
                rlo[f2 >> 3][(f2 & 7) >> 1] = lb;
            }
        }
        float gg = (ggp[0] + ggp[1]) + (ggp[2] + ggp[3]);
#pragma unroll
        for (int o = R; o < 64; o <<= 1) gg += __shfl_xor(gg, o);

        // (a tile's inputs are loaded at the top of its iteration, not during the previous
        // tile: the kernel is bound by instruction issue, and a copy of the next tile's values
        // into LDS one tile ahead was measured slower)

        // ---- QJL on the matrix cores: D[j][token] = -sum_c S[j][c] r'[c]; lane (n, g)
        //      receives the projections j = slot_coord(f, g) of its own coordinates
        //      The S fragments of output tile jt2 + 1 are read from LDS while the sign bits of
        //      tile jt2 are extracted, so the products wait on one LDS read latency at most.
        uint32_t se = 0, so = 0;  // sign bytes of the first half of the current word
        u32x4_t sf[S::NQ];
        auto load_sfrag = [&](int jt2) {
            const uint16_t *srow = sS + (R * jt2 + n) * kSRow<D>;
#pragma unroll
            for (int q = 0; q < S::NQ; ++q) {
                const uint2 s0 = *reinterpret_cast<const uint2 *>(srow + slot_coord<D, R>(8 * q, g));
                const uint2 s1 = *reinterpret_cast<const uint2 *>(srow + slot_coord<D, R>(8 * q + 4, g));
                sf[q] = u32x4_t{s0.x, s0.y, s1.x, s1.y};
            }
        };
        __builtin_amdgcn_sched_barrier(0);
        load_sfrag(0);
#pragma unroll
        for (int jt2 = 0; jt2 < S::NJ; ++jt2) {
            __builtin_amdgcn_sched_barrier(0);
            acc_t<R> acc = acc_t<R>{};
#pragma unroll
            for (int q = 0; q < S::NQ; ++q) {
                acc = mfma_f16<R>(sf[q], rhi[q], acc);
                acc = mfma_f16<R>(sf[q], rlo[q], acc);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (jt2 + 1 < S::NJ) load_sfrag(jt2 + 1);
            // the accumulator holds -(S r')_j: its sign bit is set exactly when the projection
            // is positive (or a zero came out as -0); it goes to bit 4 (f & 7) + 3 of
            // P[f >> 3].  Byte permutes replicate the sign bits of slots (f, f + 2) into bytes
            // (0, 1) of a word for f & 7 < 4, else bytes (2, 3), and of slots (f + 1, f + 3)
            // likewise into a second word shifted by 4 at the end.
            if constexpr (KB != 3) {
                // sign bit of slot f (set when the projection is positive) to bit
                // slot_coord(f, 0) mod 32 of sign word slot_coord(f, 0) / 32
#pragma unroll
                for (int r = 0; r < S::RPT; ++r) {
                    const int c = slot_coord<D, R>(jt2 * S::RPT + r, 0);
                    SW[c / 32] |= (__float_as_uint(acc[r]) >> 31) << (c % 32);
                }
                continue;
            }
#pragma unroll
            for (int r4 = 0; r4 < S::RPT; r4 += 4) {
                const int f = jt2 * S::RPT + r4;
                const uint32_t sel = (f & 4) ? 0x090B0C0Cu : 0x0C0C090Bu;
                const uint32_t e = __builtin_amdgcn_perm(__float_as_uint(acc[r4]), __float_as_uint(acc[r4 + 2]), sel);
                const uint32_t o = __builtin_amdgcn_perm(__float_as_uint(acc[r4 + 1]), __float_as_uint(acc[r4 + 3]), sel);
                if (f & 4) {
                    P[f >> 3] |= ((se | e) & 0x08080808u) | (((so | o) & 0x08080808u) << 4);
                } else {
                    se = e;
                    so = o;
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);

        if constexpr (KB != 3) {
            // ---- two-plane record: lane group 1 holds the coordinates 4 further of every
            //      field it shares a word with; shift into place, OR the two lanes' words
            //      (lanes n and n + 32) and store from lane group 0
            static_assert(R == 32 && S::KG == 2 && S::KW % 2 == 0, "two lane groups per token");
#pragma unroll
            for (int i = 0; i < S::NCW; ++i) {
                const uint32_t x = CW[i] << (4 * KB * g);
                CW[i] = x | (uint32_t)__shfl_xor((int)x, 32);
            }
#pragma unroll
            for (int i = 0; i < D / 32; ++i) {
                const uint32_t x = SW[i] << (4 * g);
                SW[i] = x | (uint32_t)__shfl_xor((int)x, 32);
            }
            if (rec >= 0 && g == 0) {
                uint32_t outw[S::KW];
#pragma unroll
                for (int i = 0; i < S::NCW; ++i) outw[i] = CW[i];
#pragma unroll
                for (int i = 0; i < D / 32; ++i) outw[S::NCW + i] = SW[i];
                uint2 *d2 = reinterpret_cast<uint2 *>(a.kw + rec * S::KW);
#pragma unroll
                for (int i = 0; i < S::KW / 2; ++i) d2[i] = make_uint2(outw[2 * i], outw[2 * i + 1]);
                *reinterpret_cast<float2 *>(a.kn + rec * 2) = make_float2(knorm, sqrtf(gg) * (1.0f / 256.f));
            }
            continue;
        }
        // ---- assemble key words: half-words of word w live in lanes g (even) and g ^ 1
        uint32_t outw[S::NP];
#pragma unroll
        for (int p = 0; p < S::NP / 2; ++p) {
            const uint32_t x = P[p], z = P[p + S::NP / 2];
            uint32_t xs, zs;
            if constexpr (R == 32) {
                const auto pr = __builtin_amdgcn_permlane32_swap(x, z, false, false);
                xs = pr[0];
                zs = pr[1];
            } else {
                const auto pr = __builtin_amdgcn_permlane16_swap(x, z, false, false);
                xs = pr[0];
                zs = pr[1];
            }
            // even lanes now hold (own, partner) halves of P[p], odd lanes (partner, own) of
            // P[p + NP/2]: low half-words from xs, high half-words from zs
            outw[2 * p] = __builtin_amdgcn_perm(zs, xs, 0x05040100u);
            outw[2 * p + 1] = __builtin_amdgcn_perm(zs, xs, 0x07060302u);
        }
        if (rec >= 0) {
            uint32_t *dst = a.kw + rec * S::KW;
            const int odd = g & 1;
            if constexpr (R == 32) {
                // slots of P[p] cover words 2p, 2p+1; even lanes store words 0..NP-1, odd
                // NP..2NP-1
                uint4 *d4 = reinterpret_cast<uint4 *>(dst + S::NP * odd);
#pragma unroll
                for (int i = 0; i < S::NP / 4; ++i)
                    d4[i] = make_uint4(outw[4 * i], outw[4 * i + 1], outw[4 * i + 2], outw[4 * i + 3]);
            } else {
#pragma unroll
                for (int p = 0; p < S::NP / 2; ++p) {
                    const int pp = p + odd * (S::NP / 2);
                    dst[slot_coord<D, R>(8 * pp, g) >> 3] = outw[2 * p];
                    dst[slot_coord<D, R>(8 * pp + 4, g) >> 3] = outw[2 * p + 1];
                }
            }
            if (g == 0)
                *reinterpret_cast<float2 *>(a.kn + rec * 2) = make_float2(knorm, sqrtf(gg) * (1.0f / 256.f));
        }

    }
}

// ------------------------------------------------------------------------------ values
// ------------------------------------------------------------------------------ launch
template <typename Tag, int D, int VB, int RR, int KB>
static void launch_kv_r(const QuantArgs &a, int64_t cus, hipStream_t st) {
    const int64_t tiles = (a.n_rows + RR - 1) / RR;
    const int nw = quant_waves_per_group(D, tiles, cus);
    const int64_t per_cu = kKeyGroupWaves<D> / nw;  // workgroups of nw waves resident per CU
    int64_t grid = (tiles + nw - 1) / nw;
    if (grid > cus * per_cu) grid = cus * per_cu;
    hipLaunchKernelGGL((k_quant_kv<Tag, D, VB, RR, KB>), dim3((unsigned)grid), dim3(64 * nw), 0, st, a);
}

// d = 128, 3-bit keys: 32-token tiles, or 16-token tiles (half the arithmetic per wave, twice
// the waves) while the 32-token ones would not give every CU one: a short input such as a
// ring flush is bound by the latency of one tile.  d = 64 and the two-plane key widths: 32-token
// tiles (a lane then holds whole value groups and its token's other lane group is lane + 32).
// d = 256: 16-token tiles.
template <typename Tag, int D, int VB, int KB>
static void launch_kv_t(const QuantArgs &a, hipStream_t st) {
    const int64_t cus = (int64_t)device_cus();
    if constexpr (D == 256) {
        launch_kv_r<Tag, D, VB, 16, KB>(a, cus, st);
    } else if constexpr (D == 128 && KB == 3) {
        if ((a.n_rows + 31) / 32 >= cus) launch_kv_r<Tag, D, VB, 32, KB>(a, cus, st);
        else launch_kv_r<Tag, D, VB, 16, KB>(a, cus, st);
    } else {
        launch_kv_r<Tag, D, VB, 32, KB>(a, cus, st);
    }
}

template <typename Tag, int D, int VB>
static void launch_kv_kb(int kb, const QuantArgs &a, hipStream_t st) {
    if constexpr (D == 256) {
        launch_kv_t<Tag, D, VB, 3>(a, st);
    } else {
        switch (kb) {
            case 1: launch_kv_t<Tag, D, VB, 1>(a, st); break;
            case 2: launch_kv_t<Tag, D, VB, 2>(a, st); break;
            case 4: launch_kv_t<Tag, D, VB, 4>(a, st); break;
            default: launch_kv_t<Tag, D, VB, 3>(a, st); break;
        }
    }
}

template <typename Tag>
static hipError_t launch_quantize_d(int d, int kb, int vb, const QuantArgs &a, hipStream_t st) {
    if (d == 64) {
        if (vb == 2) launch_kv_kb<Tag, 64, 2>(kb, a, st);
        else launch_kv_kb<Tag, 64, 4>(kb, a, st);
    } else if (d == 128) {
        if (vb == 2) launch_kv_kb<Tag, 128, 2>(kb, a, st);
        else launch_kv_kb<Tag, 128, 4>(kb, a, st);
    } else {
        if (vb == 2) launch_kv_kb<Tag, 256, 2>(kb, a, st);
        else launch_kv_kb<Tag, 256, 4>(kb, a, st);
    }
    return hipGetLastError();
}

hipError_t launch_quantize(int d, int kb, int vb, tq_dtype dt, const QuantArgs &a, hipStream_t st) {
    if (a.n_rows == 0) return hipSuccess;
    switch (dt) {
        case TQ_F32: return launch_quantize_d<f32_tag>(d, kb, vb, a, st);
        case TQ_BF16: return launch_quantize_d<bf16_tag>(d, kb, vb, a, st);
        default: return launch_quantize_d<f16_tag>(d, kb, vb, a, st);
    }
}

}  // namespace tq

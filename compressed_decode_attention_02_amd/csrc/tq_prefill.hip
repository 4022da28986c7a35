// tq_prefill.hip -- prefill attention over the packed cache by query tiles: the full_tq mode
// of the hotelren.com guide "企业官网建设流程全解析" (section 三: attention for every prompt
// token taken from the compressed records), with the estimate of its section 二,
//   s_t = |k_t| ( <q', c[idx_t]> + gamma_t sqrt(pi/2)/d <w, 2 z_t - 1> ),  q' = Pi q,  w = S q',
// softmax over the packed tokens a query may see (causal: those up to its own position) and
// values dequantised to their bin centres (code - 2^(vb-1) + 1/2) * group scale.
//
// One workgroup of NW waves per (query tile, sequence, kv head, split of the packed range):
// NW = 8 at head_dim 64 and 128, 4 at 256 (its query operands take twice the registers).  A
// tile is 16 NW query rows (token, head) of one kv head, the G heads of a token in consecutive
// rows; wave w takes rows 16 w .. 16 w + 15.  The workgroup walks the packed tokens the tile can
// see in blocks of 64 tokens (32 at head_dim 256), with two LDS buffers of matrix-core operands
// and one barrier per block; while a wave computes on block n it expands block n + 1 (loaded
// into registers one block ahead) into the other buffer, issued between its products so that
// the expansion (VALU) overlaps them:
//   * the key centroids and the signs as +-1 in fp16, [token][coordinate];
//   * the values as fp16 hi + lo pairs (v = hi + lo exactly: v has at most 16 significant
//     bits), [coordinate][token], two tokens per lane from their value words;
//   * each wave forms its scores transposed (tokens as rows: A = the key operand from LDS, B =
//     the query rows held in registers as fp16 hi + lo of q' * scale * log2 e / sqrt d and of
//     -w * scale * log2 e * sqrt(pi/2) / d), v_mfma_f32_16x16x32_f16; a lane then holds one
//     query row and four tokens of each 16-token tile, logit = |k| (c + gamma s) in log2 units;
//   * online softmax per row (running maximum raised only when a block exceeds it; the 4 lanes
//     of a row share it through two lane exchanges), p = 2^(logit - m) with hi + lo parts;
//   * o^T += V^T P^T on the matrix cores (A = the value pairs from LDS, B = the lane's own p:
//     the token order of the value columns is chosen so that the score lanes already hold
//     the operand), three products per pair (hi hi, hi lo, lo hi).
// Rows are divided by their l at the end; a row with no token gets zeros.  When the tiles alone
// would not fill the GPU, each tile's packed range is split over several workgroups, which write
// their unnormalised o and (m, l) per row for the decode's split merge.
#include <hip/hip_runtime.h>

#include "tq.h"
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kPfLog2e = 1.4426950408889634f;

// waves per workgroup (16 query rows each)
template <int D>
constexpr int kPfWaves = D == 256 ? 4 : 8;

template <int D, int KB, int VB>
struct PfShape {
    static constexpr int BLK = D == 256 ? 32 : 64;  // packed tokens per block
    static constexpr int NTT = BLK / 16;            // 16-token tiles of a block (score products)
    static constexpr int NPS = BLK / 32;            // 32-token steps of a block (value products)
    static constexpr int NW = kPfWaves<D>;
    static constexpr int THREADS = 64 * NW;
    static constexpr int ROWS = 16 * NW;          // query rows per tile
    static constexpr int KW = (KB + 1) * D / 32;  // key record words
    static constexpr int NCW = KB * D / 32;       // code-plane words (KB != 3)
    static constexpr int VW = VB * D / 32;        // value record words
    static constexpr int NG = D / 32;             // value groups (fp16 scales)
    static constexpr int NKS = D / 32;            // k-steps of the score products
    static constexpr int NDT = D / 16;            // 16-coordinate tiles of the output
    static constexpr int KRS = D + 8;             // key operand row stride (halfwords)
    static constexpr int VRS = BLK + 8;           // value operand row stride (halfwords)
    static constexpr int ITEMS = BLK * D / 8;     // key items of a block: (token, 8-coordinate chunk)
    static constexpr int NI = (ITEMS + THREADS - 1) / THREADS;
    static constexpr int VITEMS = ITEMS / 2;      // value items: (token pair, 8-coordinate chunk)
    static constexpr int VNI = (VITEMS + THREADS - 1) / THREADS;
    static constexpr int HALF = 1 << (VB - 1);
};

// one block's matrix-core operands
template <int D, int KB, int VB>
struct alignas(16) PfBuf {
    using S = PfShape<D, KB, VB>;
    // key operands: 8-coordinate chunk c of token t at [t][8 c ..]; centroids in the slot order
    // (0 2 4 6 1 3 5 7) of the chunk's coordinates, signs (as 1 - 2 z) in the order (0 4 1 5 2 6 3 7)
    uint16_t kc[S::BLK * S::KRS];
    uint16_t ks[S::BLK * S::KRS];
    // value operands [coordinate][slot]: in each 32-token step, slot 8 b + j holds token 4 b + j
    // (j < 4) or 16 + 4 b + j - 4 (j >= 4) of the step, the tokens the score lanes of group b hold
    uint16_t vh[D * S::VRS];
    uint16_t vl[D * S::VRS];
    float nrm[2 * S::BLK];  // |k| then gamma, per token
};

__device__ __forceinline__ uint32_t pack_h2(_Float16 lo, _Float16 hi) {
    return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

// x0 s0 and x1 s1 (x fp32, s fp16) as fp16 pairs: hi = fp16(x s), lo = fp16(x s - hi), each one
// rounding of an exact value (mixed fma)
__device__ __forceinline__ uint2 mix_split(float x0, _Float16 s0, float x1, _Float16 s1) {
    uint32_t hi, lo;
    asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "=&v"(hi) : "v"(x0), "v"(s0));
    asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "+v"(hi) : "v"(x1), "v"(s1));
    asm("v_fma_mixlo_f16 %0, %1, %2, -%3 op_sel_hi:[0,1,1]" : "=&v"(lo) : "v"(x0), "v"(s0), "v"(hi));
    asm("v_fma_mixhi_f16 %0, %1, %2, -%3 op_sel:[0,0,1] op_sel_hi:[0,1,1]" : "+v"(lo) : "v"(x1), "v"(s1), "v"(hi));
    return make_uint2(hi, lo);
}

// x = hi + lo, hi = fp16(x), lo = fp16(x - hi), for the pairs (x0, x1): (hi pair, lo pair)
__device__ __forceinline__ uint2 split_pair(float x0, float x1) {
    const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
    return make_uint2(pack_h2(h0, h1), pack_h2((_Float16)(x0 - (float)h0), (_Float16)(x1 - (float)h1)));
}

// the 8 codebook indices of chunk c8 of a key record as bytes (coordinates 0 2 4 6 in sel_e,
// 1 3 5 7 in sel_o) and its sign bits at bit 4 j + 3 of zw (the nibble layout's places)
template <int D, int KB>
__device__ __forceinline__ void key_chunk(uint32_t w0, uint32_t w1, int c8, uint32_t &sel_e, uint32_t &sel_o,
                                          uint32_t &zw) {
    if constexpr (KB == 3) {
        sel_e = w0 & 0x07070707u;
        sel_o = (w0 >> 4) & 0x07070707u;
        zw = w0;
    } else {
        const uint32_t f = w0 >> ((8 * c8 * KB) % 32);  // 8 KB bits, coordinate j at KB j
        const uint32_t s8 = w1 >> ((8 * c8) % 32);      // 8 bits, coordinate j at j
        sel_e = sel_o = zw = 0u;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t idx = (f >> (KB * j)) & ((1u << KB) - 1u);
            if (j & 1) sel_o |= idx << (8 * (j >> 1));
            else sel_e |= idx << (8 * (j >> 1));
            zw |= ((s8 >> j) & 1u) << (4 * j + 3);
        }
    }
}

// slot of token t in the value operand rows (see PfBuf)
__device__ __forceinline__ int value_slot(int t) {
    return 32 * (t >> 5) + 8 * ((t & 15) >> 2) + 4 * ((t >> 4) & 1) + (t & 3);
}

template <int D, int KB, int VB>
__global__ __launch_bounds__(64 * kPfWaves<D>) void k_prefill_tile(PrefillArgs a) {
    using S = PfShape<D, KB, VB>;
    __shared__ PfBuf<D, KB, VB> sm[2];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lb = lane >> 4;

    // workgroup -> (slice, tile): consecutive tiles of a slice on one XCD (workgroups are dealt
    // to the 8 XCDs in turn), so that they share its L2; the longest tiles of a slice first
    const int64_t nwg = gridDim.x, id = blockIdx.x;
    const int64_t per = nwg / 8, rem = nwg % 8, xcd = id % 8, kk = id / 8;
    const int64_t lid = xcd < rem ? xcd * (per + 1) + kk : rem * (per + 1) + (xcd - rem) * per + kk;
    const int64_t sps = lid / a.tiles;  // (slice, split)
    const int tile = a.tiles - 1 - (int)(lid - sps * a.tiles);
    const int sl = (int)(sps / a.n_split), split = (int)(sps - (int64_t)sl * a.n_split);
    const int seq = sl / a.hkv, kvh = sl - seq * a.hkv;
    const int G = a.hq / a.hkv;
    const int rows = a.T * G;
    const int64_t sbk = a.slice0 + sl;  // store slice

    // the tile's packed range: what its last row may see
    const int r_last = min(rows, (tile + 1) * S::ROWS) - 1;
    auto row_limit = [&](int r) -> int {
        if (r >= rows) return 0;
        const int64_t lim = a.causal ? min(a.n_packed, a.q_pos0 + r / G + 1) : a.n_packed;
        return (int)max((int64_t)0, lim);
    };
    const int kv_all = row_limit(r_last);
    // this workgroup's part of it: [t_lo, kv_end)
    const int t_lo = split * a.per_split;
    const int kv_end = a.n_split > 1 ? min(kv_all, t_lo + a.per_split) : kv_all;

    // this lane's row
    const int r = tile * S::ROWS + 16 * wave + lr;
    const bool row_ok = r < rows;
    const int rc = row_ok ? r : rows - 1;
    const int qi = rc / G, qg = rc - qi * G;
    const int lim = row_limit(r);
    const int wave_lim = __builtin_amdgcn_readfirstlane(lim);  // lane 0: the wave's first row
    float *const orow = a.out + (((int64_t)seq * a.T + qi) * a.hq + kvh * G + qg) * D;

    f32x4_t o[S::NDT];
#pragma unroll
    for (int i = 0; i < S::NDT; ++i) o[i] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    // split partials of this lane's row: o, then (m, l)
    const int64_t prow = (((int64_t)seq * a.T + qi) * a.hkv + kvh) * a.n_split + split;
    float *const po = a.partial + (prow * G + qg) * D;
    float *const pml = a.partial_ml + (prow * G + qg) * 2;
    if (kv_end <= t_lo) {
        if (row_ok) {
            if (a.n_split == 1) {
#pragma unroll
                for (int dt = 0; dt < S::NDT; ++dt) *reinterpret_cast<f32x4_t *>(orow + 16 * dt + 4 * lb) = o[dt];
            } else {
#pragma unroll
                for (int dt = 0; dt < S::NDT; ++dt) *reinterpret_cast<f32x4_t *>(po + 16 * dt + 4 * lb) = o[dt];
                if (lb == 0) *reinterpret_cast<float2 *>(pml) = make_float2(-INFINITY, 0.f);
            }
        }
        return;
    }

    // ---- query preparation of the tile's rows, in LDS (the operand buffers serve as scratch
    //      before the first block; each wave works on its own 16 rows): q' = H (sigma o q),
    //      unnormalised, by lane exchanges with four rows in flight; w = S q' on the matrix
    //      cores (S fp16 exact; q' 2^-e as fp16 hi + lo, e per row so that its largest entry
    //      lies in [2^13, 2^14): no overflow, no subnormals; the sums scaled back by 2^e)
    constexpr int QRS = D + 4;  // scratch row stride (floats)
    float *const qsc = reinterpret_cast<float *>(&sm[0]);         // q' [ROWS][QRS]
    float *const wsc = qsc + S::ROWS * QRS;                      // w  [ROWS][QRS]
    int *const qex = reinterpret_cast<int *>(wsc + S::ROWS * QRS);  // e [ROWS]
    static_assert((2 * S::ROWS * QRS + S::ROWS) * 4 <= sizeof(sm), "preparation scratch");
    {
        constexpr int E = D / 64, RB = 4;
        for (int i0 = 0; i0 < 16; i0 += RB) {
            float v[RB][E];
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                const int rr = min(tile * S::ROWS + 16 * wave + i0 + i, rows - 1);
                const int ti = rr / G, gi = rr - ti * G;
                const int64_t qrow = (((int64_t)seq * a.T + ti) * a.hq + kvh * G + gi) * D;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int j = lane + 64 * e;
                    float x;
                    if (a.q_dtype == TQ_F32) x = load1(a.q, qrow + j, f32_tag{});
                    else if (a.q_dtype == TQ_BF16) x = load1(a.q, qrow + j, bf16_tag{});
                    else x = load1(a.q, qrow + j, f16_tag{});
                    v[i][e] = flip_sign(x, (a.sign_bits[j >> 5] >> (j & 31)) & 1u);
                }
            }
#pragma unroll
            for (int len = 1; len < 64; len <<= 1)
#pragma unroll
                for (int i = 0; i < RB; ++i)
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const float o2 = __shfl_xor(v[i][e], len);
                        v[i][e] = (lane & len) ? (o2 - v[i][e]) : (v[i][e] + o2);
                    }
            float mx[RB];
#pragma unroll
            for (int i = 0; i < RB; ++i) {
#pragma unroll
                for (int m = 1; m < E; m <<= 1) {
                    float u[E];
#pragma unroll
                    for (int e = 0; e < E; ++e) u[e] = (e & m) ? (v[i][e ^ m] - v[i][e]) : (v[i][e] + v[i][e ^ m]);
#pragma unroll
                    for (int e = 0; e < E; ++e) v[i][e] = u[e];
                }
                const int rl = 16 * wave + i0 + i;
                mx[i] = 0.f;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    qsc[rl * QRS + lane + 64 * e] = v[i][e];
                    mx[i] = fmaxf(mx[i], fabsf(v[i][e]));
                }
            }
#pragma unroll
            for (int o2 = 32; o2 > 0; o2 >>= 1)
#pragma unroll
                for (int i = 0; i < RB; ++i) mx[i] = fmaxf(mx[i], __shfl_xor(mx[i], o2));
            if (lane < RB) {
                float m = mx[0];
#pragma unroll
                for (int i = 1; i < RB; ++i) m = lane == i ? mx[i] : m;
                int ex = 0;
                if (m > 0.f) (void)frexpf(m, &ex);  // m < 2^ex
                qex[16 * wave + i0 + lane] = ex - 14;
            }
        }
    }
    __syncthreads();
    {
        // w^T = S q'^T for the wave's rows: A = 16 rows of S x 32, B = q' 2^-e of the 16 rows
        // as hi + lo; C lane: row lr, coordinates 16 ot + 4 lb + i
        const int rl = 16 * wave + lr, ex = qex[rl];
        half8_t bh[S::NKS], bl[S::NKS];
#pragma unroll
        for (int ks = 0; ks < S::NKS; ++ks) {
            const float4 x0 = *reinterpret_cast<const float4 *>(&qsc[rl * QRS + 32 * ks + 8 * lb]);
            const float4 x1 = *reinterpret_cast<const float4 *>(&qsc[rl * QRS + 32 * ks + 8 * lb + 4]);
            const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float y = ldexpf(x[j], -ex);
                bh[ks][j] = (_Float16)y;
                bl[ks][j] = (_Float16)(y - (float)bh[ks][j]);
            }
        }
#pragma unroll
        for (int ot = 0; ot < S::NDT; ++ot) {
            f32x4_t acc = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < S::NKS; ++ks) {
                const half8_t sa = *reinterpret_cast<const half8_t *>(a.S + (int64_t)(16 * ot + lr) * D + 32 * ks + 8 * lb);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(sa, bh[ks], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(sa, bl[ks], acc, 0, 0, 0);
            }
            f32x4_t wv;
#pragma unroll
            for (int i = 0; i < 4; ++i) wv[i] = ldexpf(acc[i], ex);
            *reinterpret_cast<f32x4_t *>(&wsc[rl * QRS + 16 * ot + 4 * lb]) = wv;
        }
    }
    __syncthreads();

    // query operands of the row: k-step ks covers coordinates 32 ks + 8 lb .. + 7 in the slot
    // orders of the key operands, as fp16 hi + lo
    u32x4_t qch[S::NKS], qcl[S::NKS], qsh[S::NKS], qsl[S::NKS];
    {
        const float cs = a.scale * kPfLog2e * rsqrtf((float)D);
        const float ss = -cs * (1.2533141373155003f / (float)D);  // -sqrt(pi/2) / d
        const float *pq = qsc + (16 * wave + lr) * QRS;
        const float *pw = wsc + (16 * wave + lr) * QRS;
#pragma unroll
        for (int ks = 0; ks < S::NKS; ++ks) {
            const int c0 = 32 * ks + 8 * lb;
            const float4 x0 = *reinterpret_cast<const float4 *>(pq + c0);
            const float4 x1 = *reinterpret_cast<const float4 *>(pq + c0 + 4);
            const float4 y0 = *reinterpret_cast<const float4 *>(pw + c0);
            const float4 y1 = *reinterpret_cast<const float4 *>(pw + c0 + 4);
            const float xc[8] = {x0.x, x0.z, x1.x, x1.z, x0.y, x0.w, x1.y, x1.w};  // 0 2 4 6 1 3 5 7
            const float xs[8] = {y0.x, y1.x, y0.y, y1.y, y0.z, y1.z, y0.w, y1.w};  // 0 4 1 5 2 6 3 7
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint2 c2 = split_pair(cs * xc[2 * p], cs * xc[2 * p + 1]);
                const uint2 s2 = split_pair(ss * xs[2 * p], ss * xs[2 * p + 1]);
                qch[ks][p] = c2.x;
                qcl[ks][p] = c2.y;
                qsh[ks][p] = s2.x;
                qsl[ks][p] = s2.y;
            }
        }
    }
    __syncthreads();  // the scratch is the first block's buffer

    // codebook as fp16 byte tables (entry e: byte e % 4 of word e / 4)
    uint32_t tl[4] = {0u, 0u, 0u, 0u}, th[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < (1 << KB); ++e) {
        const uint32_t h = f32_to_f16_bits(a.centroids[e]);
        tl[e / 4] |= (h & 0xffu) << (8 * (e % 4));
        th[e / 4] |= (h >> 8) << (8 * (e % 4));
    }

    // ---- one block's records into registers.  Key items: (token it / (D / 8), chunk
    // it % (D / 8)); value items: (token it % 32, chunk it / 32).  Tokens past kv_end read the
    // last one (their logits are masked).
    auto rec_of = [&](int tok) -> int64_t {
        return record_index(a.bt, a.pt, a.pps, a.n_pages, a.cap, a.err, sbk, min(tok, kv_end - 1));
    };
    uint32_t kr0[S::NI], kr1[S::NI], vr[S::VNI][2], vsr[S::VNI][2];
    float2 knr = make_float2(0.f, 0.f);
    auto load_block = [&](int t0) {
        const int tmax = kv_end - 1 - t0;  // last valid token of the block, relative
        if (!a.bt) {
            // contiguous store: the block's records from one base (scalar), 32-bit offsets
            const int64_t r0 = sbk * a.cap + t0;
            const uint32_t *kwb = a.kw + r0 * S::KW;
            const uint32_t *vwb = a.vw + r0 * S::VW;
            const uint16_t *vsb = a.vs + r0 * S::NG;
#pragma unroll
            for (int k = 0; k < S::NI; ++k) {
                const int it = tid + S::THREADS * k;
                kr0[k] = kr1[k] = 0u;
                if (S::ITEMS % S::THREADS == 0 || it < S::ITEMS) {
                    const int tk = min(it / (D / 8), tmax), c8 = it % (D / 8);
                    if constexpr (KB == 3) {
                        kr0[k] = kwb[tk * S::KW + c8];
                    } else {
                        kr0[k] = kwb[tk * S::KW + (8 * c8 * KB) / 32];
                        kr1[k] = kwb[tk * S::KW + S::NCW + c8 / 4];
                    }
                }
            }
#pragma unroll
            for (int k = 0; k < S::VNI; ++k) {
                const int it = tid + S::THREADS * k;
                if (S::VITEMS % S::THREADS == 0 || it < S::VITEMS) {
                    const int pr = it % (S::BLK / 2), cv = it / (S::BLK / 2);
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int tv = min(2 * pr + e, tmax);
                        vr[k][e] = vwb[tv * S::VW + (8 * cv * VB) / 32];
                        vsr[k][e] = vsb[tv * S::NG + cv / 4];
                    }
                }
            }
            if (tid < S::BLK) knr = *reinterpret_cast<const float2 *>(a.kn + (r0 + min(tid, tmax)) * 2);
            return;
        }
#pragma unroll
        for (int k = 0; k < S::NI; ++k) {
            const int it = tid + S::THREADS * k;
            kr0[k] = kr1[k] = 0u;
            if (S::ITEMS % S::THREADS == 0 || it < S::ITEMS) {
                const int t = it / (D / 8), c8 = it - t * (D / 8);
                const uint32_t *kp = a.kw + rec_of(t0 + t) * S::KW;
                if constexpr (KB == 3) {
                    kr0[k] = kp[c8];
                } else {
                    kr0[k] = kp[(8 * c8 * KB) / 32];
                    kr1[k] = kp[S::NCW + c8 / 4];
                }
            }
        }
#pragma unroll
        for (int k = 0; k < S::VNI; ++k) {
            const int it = tid + S::THREADS * k;
            if (S::VITEMS % S::THREADS == 0 || it < S::VITEMS) {
                const int pr = it % (S::BLK / 2), cv = it / (S::BLK / 2);
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int64_t rec = rec_of(t0 + 2 * pr + e);
                    vr[k][e] = a.vw[rec * S::VW + (8 * cv * VB) / 32];
                    vsr[k][e] = a.vs[rec * S::NG + cv / 4];
                }
            }
        }
        if (tid < S::BLK) knr = *reinterpret_cast<const float2 *>(a.kn + rec_of(t0 + tid) * 2);
    };

    // ---- expand the registers' block into buffer B
    auto stage = [&](PfBuf<D, KB, VB> &B) {
#pragma unroll
        for (int k = 0; k < S::NI; ++k) {
            const int it = tid + S::THREADS * k;
            if (S::ITEMS % S::THREADS == 0 || it < S::ITEMS) {
                {
                    const int t = it / (D / 8), c8 = it - t * (D / 8);
                    uint32_t sel_e, sel_o, zw;
                    key_chunk<D, KB>(kr0[k], kr1[k], c8, sel_e, sel_o, zw);
                    uint32_t le, he, lo, ho;
                    if constexpr (KB <= 3) {
                        le = __builtin_amdgcn_perm(tl[1], tl[0], sel_e);
                        he = __builtin_amdgcn_perm(th[1], th[0], sel_e);
                        lo = __builtin_amdgcn_perm(tl[1], tl[0], sel_o);
                        ho = __builtin_amdgcn_perm(th[1], th[0], sel_o);
                    } else {
                        // 16 entries: the low three index bits pick within a half of the
                        // table, bit 3 (as a byte mask) picks the half
                        const uint32_t e3 = sel_e & 0x07070707u, o3 = sel_o & 0x07070707u;
                        const uint32_t me = ((sel_e >> 3) & 0x01010101u) * 0xffu;
                        const uint32_t mo = ((sel_o >> 3) & 0x01010101u) * 0xffu;
                        le = (__builtin_amdgcn_perm(tl[3], tl[2], e3) & me) | (__builtin_amdgcn_perm(tl[1], tl[0], e3) & ~me);
                        he = (__builtin_amdgcn_perm(th[3], th[2], e3) & me) | (__builtin_amdgcn_perm(th[1], th[0], e3) & ~me);
                        lo = (__builtin_amdgcn_perm(tl[3], tl[2], o3) & mo) | (__builtin_amdgcn_perm(tl[1], tl[0], o3) & ~mo);
                        ho = (__builtin_amdgcn_perm(th[3], th[2], o3) & mo) | (__builtin_amdgcn_perm(th[1], th[0], o3) & ~mo);
                    }
                    const u32x4_t kc = {__builtin_amdgcn_perm(he, le, 0x05010400u), __builtin_amdgcn_perm(he, le, 0x07030602u),
                                        __builtin_amdgcn_perm(ho, lo, 0x05010400u), __builtin_amdgcn_perm(ho, lo, 0x07030602u)};
                    u32x4_t kz;
#pragma unroll
                    for (int q = 0; q < 4; ++q) kz[q] = ((zw << (12 - 4 * q)) & 0x80008000u) | 0x3c003c00u;
                    *reinterpret_cast<u32x4_t *>(&B.kc[t * S::KRS + 8 * c8]) = kc;
                    *reinterpret_cast<u32x4_t *>(&B.ks[t * S::KRS + 8 * c8]) = kz;
                }
            }
        }
        // values of coordinates 8 c8 .. 8 c8 + 7 of tokens 2 p and 2 p + 1, (code - HALF + 1/2) s,
        // whose slots are adjacent: one 32-bit write per coordinate and part
#pragma unroll
        for (int k = 0; k < S::VNI; ++k) {
            const int it = tid + S::THREADS * k;
            if (S::VITEMS % S::THREADS == 0 || it < S::VITEMS) {
                const int pr = it % (S::BLK / 2), c8 = it / (S::BLK / 2);
                const uint32_t w0 = vr[k][0] >> ((8 * c8 * VB) % 32), w1 = vr[k][1] >> ((8 * c8 * VB) % 32);
                const _Float16 s0 = __builtin_bit_cast(_Float16, (uint16_t)vsr[k][0]);
                const _Float16 s1 = __builtin_bit_cast(_Float16, (uint16_t)vsr[k][1]);
                const int dw = value_slot(2 * pr) / 2;
                uint32_t *const vh = reinterpret_cast<uint32_t *>(B.vh), *const vl = reinterpret_cast<uint32_t *>(B.vl);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float u0 = (float)((w0 >> (VB * j)) & ((1u << VB) - 1u)) + (0.5f - (float)S::HALF);
                    const float u1 = (float)((w1 >> (VB * j)) & ((1u << VB) - 1u)) + (0.5f - (float)S::HALF);
                    const uint2 hl = mix_split(u0, s0, u1, s1);
                    const int row = (8 * c8 + j) * (S::VRS / 2) + dw;
                    vh[row] = hl.x;
                    vl[row] = hl.y;
                }
            }
        }
        if (tid < S::BLK) {
            B.nrm[tid] = knr.x;
            B.nrm[S::BLK + tid] = knr.y;
        }
    };

    float m_run = -INFINITY, l_run = 0.f;
    const int nb = (kv_end - t_lo + S::BLK - 1) / S::BLK;
    load_block(t_lo);
    stage(sm[0]);
    if (nb > 1) load_block(t_lo + S::BLK);
    __syncthreads();
    for (int n = 0; n < nb; ++n) {
        const int t0 = t_lo + n * S::BLK;
        const PfBuf<D, KB, VB> &B = sm[n & 1];
        // ---- scores, transposed: C[token][row], lane (row lr, tokens 16 tt + 4 lb + i).
        //      Issue order: four independent accumulators between dependent products.
        f32x4_t sc[S::NTT], sz[S::NTT];
#pragma unroll
        for (int tt = 0; tt < S::NTT; ++tt) sc[tt] = sz[tt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < S::NKS; ++ks) {
            const half8_t qh = __builtin_bit_cast(half8_t, qch[ks]), ql = __builtin_bit_cast(half8_t, qcl[ks]);
            const half8_t wh = __builtin_bit_cast(half8_t, qsh[ks]), wl = __builtin_bit_cast(half8_t, qsl[ks]);
#pragma unroll
            for (int tp = 0; tp < S::NTT; tp += 2) {
                half8_t kc[2], kz[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int off = (16 * (tp + u) + lr) * S::KRS + 32 * ks + 8 * lb;
                    kc[u] = *reinterpret_cast<const half8_t *>(&B.kc[off]);
                    kz[u] = *reinterpret_cast<const half8_t *>(&B.ks[off]);
                }
                sc[tp] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kc[0], qh, sc[tp], 0, 0, 0);
                sc[tp + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kc[1], qh, sc[tp + 1], 0, 0, 0);
                sz[tp] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kz[0], wh, sz[tp], 0, 0, 0);
                sz[tp + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kz[1], wh, sz[tp + 1], 0, 0, 0);
                sc[tp] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kc[0], ql, sc[tp], 0, 0, 0);
                sc[tp + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kc[1], ql, sc[tp + 1], 0, 0, 0);
                sz[tp] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kz[0], wl, sz[tp], 0, 0, 0);
                sz[tp + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kz[1], wl, sz[tp + 1], 0, 0, 0);
            }
        }
        // ---- the next block into the other buffer (no wave reads it before the barrier; a stage
        //      past the end writes a buffer no wave reads again), issued while this block's
        //      products run: after the score products at head_dim 64 and 128, before the value
        //      products at 256 (measured)
        if constexpr (D != 256) {
            stage(sm[(n + 1) & 1]);
            if (n + 2 < nb) load_block(t0 + 2 * S::BLK);  // the block after next into registers
        }
        constexpr int NL = 4 * S::NTT;  // logits per lane
        float lg[NL];
#pragma unroll
        for (int tt = 0; tt < S::NTT; ++tt) {
            const f32x4_t n1 = *reinterpret_cast<const f32x4_t *>(&B.nrm[16 * tt + 4 * lb]);
            const f32x4_t n2 = *reinterpret_cast<const f32x4_t *>(&B.nrm[S::BLK + 16 * tt + 4 * lb]);
#pragma unroll
            for (int i = 0; i < 4; ++i) lg[4 * tt + i] = n1[i] * fmaf(n2[i], sz[tt][i], sc[tt][i]);
        }
        if (t0 + S::BLK > wave_lim) {
            // tokens at or past the row's limit (its causal end, or the packed end) drop out
#pragma unroll
            for (int j = 0; j < NL; ++j)
                if (t0 + 16 * (j / 4) + 4 * lb + (j % 4) >= lim) lg[j] = -INFINITY;
        }
        // ---- online softmax of the row (its 4 lanes: lb = 0 .. 3)
        float mx = lg[0];
#pragma unroll
        for (int j = 1; j < NL; ++j) mx = fmaxf(mx, lg[j]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool raise = mx > m_run;
        if (__ballot(raise)) {
            const float mn = raise ? mx : m_run;
            const float alpha = raise ? (m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mn)) : 1.f;
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < S::NDT; ++dt) o[dt] *= alpha;
            m_run = mn;
        }
        const float mu = m_run == -INFINITY ? 0.f : m_run;
        float p[NL];
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            p[j] = __builtin_amdgcn_exp2f(lg[j] - mu);
            l_run += p[j];
        }
        // value step s takes the lane's tokens of tiles 2 s and 2 s + 1 as its 8 k-slots
        u32x4_t ph[S::NPS], pl[S::NPS];
#pragma unroll
        for (int st = 0; st < S::NPS; ++st)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                // hi = fp16 pair (round to nearest), lo = fp16(p - hi) by mixed fma
                const float x0 = p[8 * st + 2 * q], x1 = p[8 * st + 2 * q + 1];
                uint32_t hi, lo;
                asm("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(hi) : "v"(x0), "v"(x1));
                asm("v_fma_mixlo_f16 %0, %1, 1.0, -%2 op_sel_hi:[0,0,1]" : "=&v"(lo) : "v"(x0), "v"(hi));
                asm("v_fma_mixhi_f16 %0, %1, 1.0, -%2 op_sel:[0,0,1] op_sel_hi:[0,0,1]" : "+v"(lo) : "v"(x1), "v"(hi));
                ph[st][q] = hi;
                pl[st][q] = lo;
            }
        if constexpr (D == 256) {
            stage(sm[(n + 1) & 1]);
            if (n + 2 < nb) load_block(t0 + 2 * S::BLK);
        }
        // ---- o^T[coordinate][row] += V^T P^T, four output tiles at a time (independent
        //      accumulators between dependent products)
#pragma unroll
        for (int st = 0; st < S::NPS; ++st) {
            const half8_t bph = __builtin_bit_cast(half8_t, ph[st]), bpl = __builtin_bit_cast(half8_t, pl[st]);
#pragma unroll
            for (int d4 = 0; d4 < S::NDT; d4 += 4) {
                half8_t vh[4], vl[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int off = (16 * (d4 + u) + lr) * S::VRS + 32 * st + 8 * lb;
                    vh[u] = *reinterpret_cast<const half8_t *>(&B.vh[off]);
                    vl[u] = *reinterpret_cast<const half8_t *>(&B.vl[off]);
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) o[d4 + u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh[u], bph, o[d4 + u], 0, 0, 0);
#pragma unroll
                for (int u = 0; u < 4; ++u) o[d4 + u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh[u], bpl, o[d4 + u], 0, 0, 0);
#pragma unroll
                for (int u = 0; u < 4; ++u) o[d4 + u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vl[u], bph, o[d4 + u], 0, 0, 0);
            }
        }
        __syncthreads();
    }
    // ---- l of the row over its 4 lanes; lane holds coordinates 16 dt + 4 lb + i
    float l = l_run;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (!row_ok) return;
    if (a.n_split == 1) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
        for (int dt = 0; dt < S::NDT; ++dt) *reinterpret_cast<f32x4_t *>(orow + 16 * dt + 4 * lb) = o[dt] * inv;
    } else {
#pragma unroll
        for (int dt = 0; dt < S::NDT; ++dt) *reinterpret_cast<f32x4_t *>(po + 16 * dt + 4 * lb) = o[dt];
        if (lb == 0) *reinterpret_cast<float2 *>(pml) = make_float2(m_run, l);
    }
}

template <int D, int KB>
hipError_t launch_kb(int vb, dim3 grid, const PrefillArgs &a, hipStream_t st) {
    const dim3 block(64 * kPfWaves<D>);
    if (vb == 2) hipLaunchKernelGGL((k_prefill_tile<D, KB, 2>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_prefill_tile<D, KB, 4>), grid, block, 0, st, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(int kb, int vb, dim3 grid, const PrefillArgs &a, hipStream_t st) {
    switch (kb) {
        case 1: return launch_kb<D, 1>(vb, grid, a, st);
        case 2: return launch_kb<D, 2>(vb, grid, a, st);
        case 3: return launch_kb<D, 3>(vb, grid, a, st);
        default: return launch_kb<D, 4>(vb, grid, a, st);
    }
}

}  // namespace

int prefill_block_tokens(int d) { return d == 256 ? PfShape<256, 3, 2>::BLK : PfShape<128, 3, 2>::BLK; }

int prefill_tile_rows(int d) { return 16 * (d == 256 ? kPfWaves<256> : kPfWaves<128>); }

hipError_t launch_prefill(int d, int kb, int vb, int64_t n_seq, const PrefillArgs &a, hipStream_t st) {
    const dim3 grid((unsigned)(n_seq * a.hkv * a.n_split * a.tiles));
    if (d == 64) return launch_d<64>(kb, vb, grid, a, st);
    if (d == 128) return launch_d<128>(kb, vb, grid, a, st);
    return launch_kb<256, 3>(vb, grid, a, st);
}

}  // namespace tq

// tq_decode.hip -- hybrid decode attention over the packed store plus the exact ring
// (hotelren.com guide "企业官网建设流程全解析", section 5.1 item 2: attention over the
// compressed history together with the exact recent buffer), and the ring append
// (section 5.1 item 1: a decode-time token goes into the ring buffer).
//
// Score of a packed token t for query head g is the unbiased inner-product estimate of
// section 二 evaluated in the rotated domain (q' = Pi q, w = S q'):
//   s_tg = |k_t| ( sum_j q'_gj c[idx_tj] + g_t sqrt(pi/2)/d sum_j w_gj (2 z_tj - 1) ).
//
// Launches per call:
//   * d = 256 only: k_decode_prep, q' and w of every query head into the workspace (bands of
//     S rows per workgroup);
//   * k_decode_main, grid (splits, batch * kv heads): each workgroup attends to its split's
//     share of the ring's exact fp16 tokens against the unrotated queries (the new token of a
//     fused step taken from the input), prepares its slice's queries in LDS (d = 128) or copies
//     them from the workspace (d = 256), then its waves stream blocks of 32 packed tokens
//     through LDS (hand-issued global -> LDS copies):
//     scores on MFMA (query rows x token columns; centroid values from byte tables by
//     v_perm_b32, QJL signs as +-1), a lazily rescaled online softmax, values on MFMA with
//     A = 1 + code / 2^vb and B = p * scale; the waves' and the ring's (m, l, o) are combined
//     in LDS and written as the split's partials;
//   * k_decode_merge, one workgroup per query head: the splits' partials combined (skipped
//     with a single split, whose workgroup writes the output itself).
#include <hip/hip_runtime.h>

#include "tq.h"
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kBlock = 32;       // tokens per wave iteration
// logits and running maxima are kept in log2 units (softmax weights by exp2)
constexpr float kLog2e = 1.4426950408889634f;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

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

// The products x0 = p0 s0, x1 = p1 s1 (p fp32, s fp16) as fp16 pairs: hi = fp16(x) and
// lo = fp16(x - hi), each one rounding of an exact value (mixed fma)
__device__ __forceinline__ void mix_hl2(float p0, _Float16 s0, float p1, _Float16 s1, uint32_t &hi, uint32_t &lo) {
    asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "=&v"(hi) : "v"(p0), "v"(s0));
    asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "+v"(hi) : "v"(p1), "v"(s1));
    asm("v_fma_mixlo_f16 %0, %1, %2, -%3 op_sel_hi:[0,1,1]" : "=&v"(lo) : "v"(p0), "v"(s0), "v"(hi));
    asm("v_fma_mixhi_f16 %0, %1, %2, -%3 op_sel:[0,0,1] op_sel_hi:[0,1,1]" : "+v"(lo) : "v"(p1), "v"(s1), "v"(hi));
}

// ------------------------------------------------------------------ query loads
// element `off` of q in its storage dtype, as fp32
__device__ __forceinline__ float load_q(const DecodeArgs &a, int64_t off) {
    if (a.q_dtype == TQ_F32) return load1(a.q, off, f32_tag{});
    if (a.q_dtype == TQ_BF16) return load1(a.q, off, bf16_tag{});
    return load1(a.q, off, f16_tag{});
}

// ------------------------------------------------------------------ query preparation
// Every workgroup of the packed splits prepares the G query heads of its (batch, kv head)
// in LDS: q'_g = H (sigma o q_g) (unnormalised; the rotation's 1/sqrt(d) is folded into the
// score operands' scale) and w_g = S q'_g as PARTS partial sums over column ranges of S,
// added by the reader.  qw layout (fp32): q' [G][D], then the partial sums [PARTS][G][D].
// Thread (row, part) holds D / PARTS entries of one row of S, loaded first (S is a few
// tens of kilobytes, shared by every workgroup, so after the first ones these are L2 hits).
template <int D, int NW>
struct PrepShape {
    static constexpr int NT = 64 * NW;
    // (12-wave groups form w = S q' whole, one (row, head) per thread, from an LDS copy of S)
    static constexpr int PARTS = NW == 12 ? 1 : (NT / D >= 4 ? 4 : (NT / D >= 2 ? 2 : 1));
    static constexpr int SEG = D / PARTS;  // columns of S per thread
    template <int G>
    static constexpr int floats() { return (1 + PARTS) * G * D; }
};

// The loads of the preparation (this thread's part of S, the query coordinates it
// transforms), issued ahead of other work; prep_query then computes from them.
template <int D, int G, int NW>
struct PrepRegs {
    static constexpr int E = D / 64;                // coordinates per lane in the transform
    static constexpr int HPW = (G + NW - 1) / NW;   // heads per wave
    uint4 spk[PrepShape<D, NW>::SEG / 8];
    float v[HPW][E];
};

template <int D, int G, int NW>
__device__ __forceinline__ void prep_load(const DecodeArgs &a, PrepRegs<D, G, NW> &pr, int b, int kvh) {
    using P = PrepShape<D, NW>;
    using Q = PrepRegs<D, G, NW>;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = tid % D, part = tid / D;
    if (part < P::PARTS) {
        const uint4 *src = reinterpret_cast<const uint4 *>(a.S + (int64_t)row * D + part * P::SEG);
#pragma unroll
        for (int i = 0; i < P::SEG / 8; ++i) pr.spk[i] = src[i];
    }
#pragma unroll
    for (int h = 0; h < Q::HPW; ++h) {
        const int g = wave + h * NW;
        if (g < G) {
            const int64_t qoff = ((int64_t)b * a.hq + kvh * G + g) * D;
#pragma unroll
            for (int e = 0; e < Q::E; ++e) {
                const int j = lane + 64 * e;
                pr.v[h][e] = flip_sign(load_q(a, qoff + j), (a.sign_bits[j >> 5] >> (j & 31)) & 1u);
            }
        }
    }
}

template <int D, int G, int NW>
__device__ __forceinline__ void prep_transform(PrepRegs<D, G, NW> &pr, float *qw) {
    using Q = PrepRegs<D, G, NW>;
    constexpr int E = Q::E;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // Walsh-Hadamard transform of head g by wave g (mod NW): strides below 64 across lanes,
    // the others between a lane's own coordinates
#pragma unroll
    for (int h = 0; h < Q::HPW; ++h) {
        const int g = wave + h * NW;
        if (g >= G) break;
        float *v = pr.v[h];
#pragma unroll
        for (int len = 1; len < 64; len <<= 1)
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float o = __shfl_xor(v[e], len);
                v[e] = (lane & len) ? (o - v[e]) : (v[e] + o);
            }
#pragma unroll
        for (int m = 1; m < E; m <<= 1) {
            float u[E];
#pragma unroll
            for (int e = 0; e < E; ++e) u[e] = (e & m) ? (v[e ^ m] - v[e]) : (v[e] + v[e ^ m]);
#pragma unroll
            for (int e = 0; e < E; ++e) v[e] = u[e];
        }
#pragma unroll
        for (int e = 0; e < E; ++e) qw[g * D + lane + 64 * e] = v[e];
    }
}

// the partial sums of w = S q' (after a barrier that makes q' visible)
template <int D, int G, int NW>
__device__ __forceinline__ void prep_product(PrepRegs<D, G, NW> &pr, float *qw) {
    using P = PrepShape<D, NW>;
    const int tid = threadIdx.x;
    const int row = tid % D, part = tid / D;
    if (part < P::PARTS) {
        float acc[G];
#pragma unroll
        for (int g = 0; g < G; ++g) acc[g] = 0.f;
#pragma unroll
        for (int i = 0; i < P::SEG / 8; ++i) {
            const uint4 pk = pr.spk[i];
            const float s[8] = {f16_lo(pk.x), f16_hi(pk.x), f16_lo(pk.y), f16_hi(pk.y),
                                f16_lo(pk.z), f16_hi(pk.z), f16_lo(pk.w), f16_hi(pk.w)};
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float *qg = qw + g * D + part * P::SEG + 8 * i;
                const float4 q0 = *reinterpret_cast<const float4 *>(qg);
                const float4 q1 = *reinterpret_cast<const float4 *>(qg + 4);
                acc[g] = fmaf(s[0], q0.x, acc[g]);
                acc[g] = fmaf(s[1], q0.y, acc[g]);
                acc[g] = fmaf(s[2], q0.z, acc[g]);
                acc[g] = fmaf(s[3], q0.w, acc[g]);
                acc[g] = fmaf(s[4], q1.x, acc[g]);
                acc[g] = fmaf(s[5], q1.y, acc[g]);
                acc[g] = fmaf(s[6], q1.z, acc[g]);
                acc[g] = fmaf(s[7], q1.w, acc[g]);
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) qw[(G + part * G + g) * D + row] = acc[g];
    }
}

// the preparation in turn: transform, barrier, product, barrier
template <int D, int G, int NW>
__device__ void prep_query(PrepRegs<D, G, NW> &pr, float *qw) {
    prep_transform<D, G, NW>(pr, qw);
    __syncthreads();
    prep_product<D, G, NW>(pr, qw);
    __syncthreads();
}

// 12-wave groups (d = 128): the preparation from LDS copies of S and of the slice's queries,
// made by the waves' first copies ahead of their packed blocks (so that it does not wait for
// those).  S is stored piece-major: 16-byte piece k of row i (columns 8k .. 8k + 7) at slot
// k D + i; the queries in their input dtype, [G][D].
// element j of head g of the copied queries, as fp32
__device__ __forceinline__ float lds_q(const unsigned char *pq, int dtype, int idx) {
    if (dtype == TQ_F32) return reinterpret_cast<const float *>(pq)[idx];
    const uint32_t h = reinterpret_cast<const uint16_t *>(pq)[idx];
    return dtype == TQ_BF16 ? __uint_as_float(h << 16) : f16_lo(h);
}

// q'_g = H (sigma o q_g) by wave g < G, as prep_transform
template <int D, int G, int NW>
__device__ __forceinline__ void prep_transform12(const DecodeArgs &a, const uint32_t (&sg)[4], const unsigned char *pq,
                                                 float *qw) {
    static_assert(D == 128, "two coordinates per lane");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (wave >= G) return;
    const int g = wave;
    // sigma (its words loaded at the start); coordinate lane + 64 e is bit `lane` of the 64-bit
    // pair of words 2 e, 2 e + 1
    const uint64_t sw0 = sg[0] | ((uint64_t)sg[1] << 32), sw1 = sg[2] | ((uint64_t)sg[3] << 32);
    float v[2];
    v[0] = flip_sign(lds_q(pq, a.q_dtype, g * D + lane), (uint32_t)(sw0 >> lane) & 1u);
    v[1] = flip_sign(lds_q(pq, a.q_dtype, g * D + lane + 64), (uint32_t)(sw1 >> lane) & 1u);
#pragma unroll
    for (int len = 1; len < 64; len <<= 1)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const float o = __shfl_xor(v[e], len);
            v[e] = (lane & len) ? (o - v[e]) : (v[e] + o);
        }
    const float u0 = v[0] + v[1], u1 = v[0] - v[1];
    qw[g * D + lane] = u0;
    qw[g * D + lane + 64] = u1;
}

// w_g = S q'_g: thread (row i, head g) of the first G D threads, from the piece-major copy of S
// (a wave reads one piece of 64 consecutive rows: one contiguous kilobyte) and q'_g (the same
// address in every lane); written as the single partial sum
template <int D, int G, int NW>
__device__ __forceinline__ void prep_product12(const unsigned char *ps, float *qw) {
    const int tid = threadIdx.x;
    if (tid >= G * D) return;
    const int i = tid % D, g = tid / D;
    const float *qg = qw + g * D;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};  // four chains (the sum is latency-bound)
#pragma unroll
    for (int k = 0; k < D / 8; ++k) {
        const uint4 pk = *reinterpret_cast<const uint4 *>(ps + (k * D + i) * 16);
        const float4 q0 = *reinterpret_cast<const float4 *>(qg + 8 * k);
        const float4 q1 = *reinterpret_cast<const float4 *>(qg + 8 * k + 4);
        float &c = acc[k & 3];
        c = fmaf(f16_lo(pk.x), q0.x, c);
        c = fmaf(f16_hi(pk.x), q0.y, c);
        c = fmaf(f16_lo(pk.y), q0.z, c);
        c = fmaf(f16_hi(pk.y), q0.w, c);
        c = fmaf(f16_lo(pk.z), q1.x, c);
        c = fmaf(f16_hi(pk.z), q1.y, c);
        c = fmaf(f16_lo(pk.w), q1.z, c);
        c = fmaf(f16_hi(pk.w), q1.w, c);
    }
    qw[(G + g) * D + i] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

template <int D, int VB, int G>
struct DecodeShape {
    static constexpr int KW = D / 8;          // key words per token
    static constexpr int NKS = D / 32;        // score k-steps per tile (one key word per lane group)
    static constexpr int VW = VB * D / 32;    // value words per token
    static constexpr int NG = D / 32;         // value groups
    static constexpr int NT = D / 16;         // value tiles; row m owns coordinates m*NT .. m*NT+NT-1
    static constexpr int H = VB * NT / 16;    // halfwords of codes per row and token (1, 2 or 4)
    static constexpr int NCOL = G * NG;       // value columns (head, group)
    static constexpr int NPASS = (NCOL + 15) / 16;
    static constexpr int HALF = 1 << (VB - 1);
    // per-wave staging buffer of one 32-token block (bytes): key words, norms, value words
    // (records in slot order 4 (t % 8) + t / 8, so that the code reads of four lane groups
    // hit different banks), scales
    static constexpr int KW_B = kBlock * KW * 4;
    static constexpr int KN_B = kBlock * 8;
    static constexpr int VW_B = kBlock * VW * 4;
    static constexpr int VS_B = kBlock * NG * 2;
    static constexpr int OFF_KN = KW_B;
    static constexpr int OFF_VW = OFF_KN + KN_B;
    static constexpr int OFF_VS = OFF_VW + VW_B;
    static constexpr int BUF_B = OFF_VS + VS_B;
    // global -> LDS copies per block: 16-byte (key and value words) and 4-byte (norms, scales)
    static constexpr int N_KW = KW_B / 1024;
    static constexpr int N_VW = VW_B / 1024;
    static constexpr int N_VS = VS_B / 256;
    static constexpr int N_DMA = N_KW + 1 + N_VW + N_VS;
    // d = 128: the score B fragments live in LDS (one copy per workgroup: all four waves
    // serve the same query heads), which frees 32 VGPRs per lane; d = 256 keeps them in
    // registers (its LDS is taken by the staging buffers)
    static constexpr bool BLDS = D == 128;
};

template <int D, int VB, int G, int NW>
struct alignas(16) DecodeSmem {
    using S = DecodeShape<D, VB, G>;
    // score query operands in LDS (d = 128): NSL nonzero rows per operand and lane group
    // are stored; lanes of zero rows read one zero fragment at index FZ
    static constexpr int NSL = G == 8 ? 16 : (G == 4 ? 8 : 4);
    static constexpr int FZ = 4 * NSL;
    union {
        // per-wave double buffer, buffer-major: stage[1] (NW * BUF_B contiguous bytes) also
        // holds the query preparation before the first copy into it
        unsigned char stage[2][NW][S::BUF_B];
        struct {  // wave combine (after the loop)
            float wo[NW][G][D];
        } x;
    };
    u32x4_t bfrag[S::BLDS ? 2 * S::NKS : 1][FZ + 1];  // [centroid, sign k-steps][row slot]
    float pb[NW][G][kBlock + 4];
    float corr[NW][G];
    float i8c[G][4];    // int8 score path: per head alpha, beta / 4, -beta W (see packed_wave)
    float mref[NW][G];  // running reference max per wave and head (packed splits)
    float wm[NW][G], wl[NW][G];
    float rm[G], rl[G];  // the split's ring tokens: maximum and sum of p per head
    int next_blk;       // the split's next block not yet handed to a wave
    // 12-wave groups: the split's ring rows, copied into LDS by the wave that attends to them
    // (4-token chunks: keys 1 KB each padded by 16 bytes, values 1 KB each), its unrotated
    // queries (then its p values) and its result o
    static constexpr bool RW = NW == 12;
    static constexpr int RCH = 16;  // 64 ring tokens per split at most
    alignas(16) unsigned char rk[RW ? RCH * 1040 : 16];
    alignas(16) unsigned char rv[RW ? RCH * 1024 : 16];
    alignas(16) float rq[RW ? G : 1][RW ? D : 1];
    alignas(16) float ro[RW ? G : 1][RW ? D : 1];
};

// ---- global -> LDS copies issued by hand, waited for with explicit counts.  M0 holds the
//      LDS destination of the wave's 64 x 16 (or 64 x 4) bytes: an input operand of the asm
//      bound to that register, so the compiler writes M0 itself and knows it is read.  The
//      global address is a uniform base plus a 32-bit per-lane byte offset; the instruction's
//      immediate offset IMM is added to both the global and the LDS address.  The compiler
//      does not count these loads, so every read of a staged buffer follows an explicit
//      vmcnt wait, and every LDS read of a buffer is complete (lgkmcnt(0)) before the buffer
//      is refilled.  Nor does its hazard recognizer look into the asm: the s_nop 4 in front
//      of each copy gives the wait states the ISA requires between a VALU write of an SGPR
//      (the v_readfirstlane of the base) and a VMEM read of it (5), which also covers an SALU
//      write of M0 before an LDS-DMA load (1).
// (the base is uniform by construction; readfirstlane makes that visible to the compiler
// wherever it would otherwise keep the pointer in vector registers, and folds away elsewhere)
__device__ __forceinline__ const void *uniform_ptr(const void *p) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
    return reinterpret_cast<const void *>(lo | (hi << 32));
}
template <int IMM = 0>
__device__ __forceinline__ void dma16(const void *base, uint32_t off, uint32_t lds) {
    static_assert(IMM >= 0 && IMM < 4096, "global instruction offset range");
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1 offset:%2"
                 :
                 : "v"(off), "s"(uniform_ptr(base)), "n"(IMM), "{m0}"(lds)
                 : "memory");
}
template <int IMM = 0>
__device__ __forceinline__ void dma4(const void *base, uint32_t off, uint32_t lds) {
    static_assert(IMM >= 0 && IMM < 4096, "global instruction offset range");
    asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1 offset:%2"
                 :
                 : "v"(off), "s"(uniform_ptr(base)), "n"(IMM), "{m0}"(lds)
                 : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// lane n16 < G receives the value of lane n16 + G of its 16-lane row (DPP row shift)
template <int G>
__device__ __forceinline__ float from_lane_plus_g(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x100 + G, 0xf,
                                                                  0xf, true));
}

// ------------------------------------------------------------------ ring tokens of a split
// The ring's exact fp16 tokens are spread over the packed splits of their slice (at most
// kRingPerSplit<D> per split: 64 at d = 128, 32 at d = 256, a register budget).  Each
// main-kernel workgroup attends to its share against the unrotated queries while its first
// packed block's copy is in flight and folds the result into the split's (m, l, o) partial.
// The ring words are loaded right after the first block's copies, with the query
// preparation's inputs (one wait for both); scores, softmax statistics and values use the
// second staging buffers as scratch before the query preparation and the second block's
// copies take them.
template <int D>
constexpr int kRingPerSplit = D == 128 ? 64 : 32;

template <int D, int G, int NW>
struct RingShape {
    static constexpr int NT = 64 * NW;
    static constexpr int TPT = 8;                     // scoring threads per token
    static constexpr int SEG = D / TPT;               // key coordinates per scoring thread
    static constexpr int TCH = NT / TPT;              // tokens per scoring pass
    static constexpr int NP = (kRingPerSplit<D> + TCH - 1) / TCH;  // scoring passes
    static constexpr int NCP = D / 2;                 // value coordinate pairs
    static constexpr int NTG = NT / NCP;              // value token classes
    static constexpr int TPV = (kRingPerSplit<D> + NTG - 1) / NTG;  // value tokens per thread
    static constexpr int NE = (G * D + NT - 1) / NT;  // combined output elements per thread
    // LDS scratch (floats): q [G][D], logits then p [G][kRingPerSplit<D>], per-class value sums
    // [NTG][GB][D] for a group of GB heads at a time
    static constexpr int fixed() { return G * D + G * kRingPerSplit<D>; }
    static constexpr int gb(int bytes) {
        return (fixed() + NTG * 4 * D) * 4 <= bytes ? (G < 4 ? G : 4) : ((fixed() + NTG * 2 * D) * 4 <= bytes ? (G < 2 ? G : 2) : 1);
    }
};

template <int D, int G, int NW>
struct RingRegs {
    using R = RingShape<D, G, NW>;
    uint4 k4[R::NP][R::SEG / 8];
    uint32_t v2[R::TPV];
};

// 8 elements of the new token (fused append) from element `off` of its input, rounded to
// fp16 as the ring append rounds them, packed in pairs
__device__ __forceinline__ uint4 new_token8(const void *src, int dtype, int64_t off) {
    float f[8];
    if (dtype == TQ_F32) load8(src, off, f, f32_tag{});
    else if (dtype == TQ_BF16) load8(src, off, f, bf16_tag{});
    else load8(src, off, f, f16_tag{});
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = f32_to_f16_bits(f[2 * e]) | ((uint32_t)f32_to_f16_bits(f[2 * e + 1]) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// loads of the split's ring tokens [r0, r0 + n) (addresses clamped into the ring, unused
// words ignored)
template <int D, int G, int NW>
__device__ __forceinline__ void ring_load(const DecodeArgs &a, RingRegs<D, G, NW> &rr, int bk, int r0, int n) {
    using R = RingShape<D, G, NW>;
    const int tid = threadIdx.x;
    const int part = tid % R::TPT, cp = tid % R::NCP, tg = tid / R::NCP;
    const uint16_t *rk = a.rk + (int64_t)bk * a.buffer_size * D;
    const uint32_t *rv2 = reinterpret_cast<const uint32_t *>(a.rv + (int64_t)bk * a.buffer_size * D);
#pragma unroll
    for (int ps = 0; ps < R::NP; ++ps) {
        const int tt = min(ps * R::TCH + tid / R::TPT, n - 1);
        const uint4 *kr = reinterpret_cast<const uint4 *>(rk + (int64_t)(r0 + tt) * D + part * R::SEG);
#pragma unroll
        for (int i = 0; i < R::SEG / 8; ++i) rr.k4[ps][i] = ps * R::TCH < n ? kr[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < R::TPV; ++u) {
        const int tt = tg + u * R::NTG;
        rr.v2[u] = tt < n ? rv2[(int64_t)(r0 + tt) * R::NCP + cp] : 0u;
    }
    // fused append: the new token replaces what the ring slot held, read from the input and
    // rounded as the append rounds it (ring_attend writes it into the ring from these
    // registers, once every load has landed)
    const int ns = a.new_slot - r0;
    if (a.new_slot >= 0 && ns >= 0 && ns < n) {
        const int64_t in0 = (int64_t)bk * D;
#pragma unroll
        for (int ps = 0; ps < R::NP; ++ps)
            if (ps * R::TCH + tid / R::TPT == ns)
#pragma unroll
                for (int i = 0; i < R::SEG / 8; ++i) rr.k4[ps][i] = new_token8(a.k_new, a.kv_dtype, in0 + part * R::SEG + 8 * i);
#pragma unroll
        for (int u = 0; u < R::TPV; ++u)
            if (tg + u * R::NTG == ns) {
                const uint4 w = new_token8(a.v_new, a.kv_dtype, in0 + (2 * cp & ~7));
                const uint32_t sel = (cp & 3);
                rr.v2[u] = sel == 0 ? w.x : (sel == 1 ? w.y : (sel == 2 ? w.z : w.w));
            }
    }
}

// Attention of the G query heads over the split's n ring tokens, in phases separated by
// workgroup barriers (so that another start-up task can share them): per head the maximum m_r
// (log2 units) and sum l_r into rm / rl (LDS), and the unnormalised o_r of this thread's output
// elements e = tid + k NT ([G][D] order) into orr.  Scratch: qr [G][D], pr [G][RP], os
// [NTG][GB][D] (floats).
// phase 1: the unrotated queries into LDS; a fused step's new token into its ring slot (by
// the threads holding its words)
template <int D, int G, int NW>
__device__ __forceinline__ void ring_p1(const DecodeArgs &a, const RingRegs<D, G, NW> &rr, float *qr, int bk, int b,
                                        int kvh, int r0, int n) {
    using R = RingShape<D, G, NW>;
    const int tid = threadIdx.x;
    const int part = tid % R::TPT, cp = tid % R::NCP, tg = tid / R::NCP;
    for (int i = tid; i < G * D; i += R::NT) qr[i] = load_q(a, ((int64_t)b * a.hq + kvh * G) * D + i);
    const int ns = a.new_slot - r0;
    if (a.new_slot >= 0 && ns >= 0 && ns < n) {
        uint16_t *rkw = a.rk + ((int64_t)bk * a.buffer_size + a.new_slot) * D;
        uint32_t *rvw = reinterpret_cast<uint32_t *>(a.rv + ((int64_t)bk * a.buffer_size + a.new_slot) * D);
#pragma unroll
        for (int ps = 0; ps < R::NP; ++ps)
            if (ps * R::TCH + tid / R::TPT == ns)
#pragma unroll
                for (int i = 0; i < R::SEG / 8; ++i) *reinterpret_cast<uint4 *>(rkw + part * R::SEG + 8 * i) = rr.k4[ps][i];
#pragma unroll
        for (int u = 0; u < R::TPV; ++u)
            if (tg + u * R::NTG == ns) rvw[cp] = rr.v2[u];
    }
}

// phase 2: logits (log2 units) of the token-head pairs into pr
template <int D, int G, int NW>
__device__ __forceinline__ void ring_p2(const DecodeArgs &a, const RingRegs<D, G, NW> &rr, const float *qr, float *pr,
                                        int n) {
    using R = RingShape<D, G, NW>;
    constexpr int RP = kRingPerSplit<D>;
    const int tid = threadIdx.x, part = tid % R::TPT;
    const float lscale = a.scale * kLog2e;
#pragma unroll
    for (int ps = 0; ps < R::NP; ++ps) {
        if (ps * R::TCH >= n) break;
        const int tt = ps * R::TCH + tid / R::TPT;
        float acc[G];
#pragma unroll
        for (int g = 0; g < G; ++g) acc[g] = 0.f;
#pragma unroll
        for (int i = 0; i < R::SEG / 8; ++i) {
            const uint4 k = rr.k4[ps][i];
            const float kv[8] = {f16_lo(k.x), f16_hi(k.x), f16_lo(k.y), f16_hi(k.y),
                                 f16_lo(k.z), f16_hi(k.z), f16_lo(k.w), f16_hi(k.w)};
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float4 q0 = *reinterpret_cast<const float4 *>(qr + g * D + part * R::SEG + 8 * i);
                const float4 q1 = *reinterpret_cast<const float4 *>(qr + g * D + part * R::SEG + 8 * i + 4);
                acc[g] = fmaf(q0.x, kv[0], acc[g]);
                acc[g] = fmaf(q0.y, kv[1], acc[g]);
                acc[g] = fmaf(q0.z, kv[2], acc[g]);
                acc[g] = fmaf(q0.w, kv[3], acc[g]);
                acc[g] = fmaf(q1.x, kv[4], acc[g]);
                acc[g] = fmaf(q1.y, kv[5], acc[g]);
                acc[g] = fmaf(q1.z, kv[6], acc[g]);
                acc[g] = fmaf(q1.w, kv[7], acc[g]);
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
#pragma unroll
            for (int o = 1; o < R::TPT; o <<= 1) acc[g] += __shfl_xor(acc[g], o);
            if (part == 0 && tt < n) pr[g * RP + tt] = acc[g] * lscale;
        }
    }
}

// phase 3: per head (wave g, g + NW, ...) the maximum, then p = 2^(logit - m) in place and
// its sum
template <int D, int G, int NW>
__device__ __forceinline__ void ring_p3(float *pr, float *rm, float *rl, int n) {
    constexpr int RP = kRingPerSplit<D>;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int g = wave; g < G; g += NW) {
        float m = -INFINITY;
        for (int tt = lane; tt < n; tt += 64) m = fmaxf(m, pr[g * RP + tt]);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
        float l = 0.f;
        for (int tt = lane; tt < n; tt += 64) {
            const float pv = exp2f(pr[g * RP + tt] - m);
            pr[g * RP + tt] = pv;
            l += pv;
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o);
        if (lane == 0) {
            rm[g] = m;
            rl[g] = l;
        }
    }
}

// phase 4: values of heads g0 .. g0 + GB - 1 by (coordinate pair, token class) into os
template <int D, int G, int NW, int GB>
__device__ __forceinline__ void ring_p4(const RingRegs<D, G, NW> &rr, const float *pr, float *os, int g0, int n) {
    using R = RingShape<D, G, NW>;
    constexpr int RP = kRingPerSplit<D>;
    const int tid = threadIdx.x, cp = tid % R::NCP, tg = tid / R::NCP;
    float o0[GB], o1[GB];
#pragma unroll
    for (int h = 0; h < GB; ++h) o0[h] = o1[h] = 0.f;
#pragma unroll
    for (int u = 0; u < R::TPV; ++u) {
        const int tt = tg + u * R::NTG;
        const float va = f16_lo(rr.v2[u]), vb = f16_hi(rr.v2[u]);
#pragma unroll
        for (int h = 0; h < GB; ++h) {
            const float pv = tt < n ? pr[(g0 + h) * RP + tt] : 0.f;
            o0[h] = fmaf(pv, va, o0[h]);
            o1[h] = fmaf(pv, vb, o1[h]);
        }
    }
#pragma unroll
    for (int h = 0; h < GB; ++h) *reinterpret_cast<float2 *>(os + (tg * GB + h) * D + 2 * cp) = make_float2(o0[h], o1[h]);
}

// phase 5: this thread's output elements of heads g0 .. g0 + GB - 1, summed over the classes
template <int D, int G, int NW, int GB>
__device__ __forceinline__ void ring_p5(const float *os, int g0, float (&orr)[RingShape<D, G, NW>::NE]) {
    using R = RingShape<D, G, NW>;
    const int tid = threadIdx.x;
#pragma unroll
    for (int k = 0; k < R::NE; ++k) {
        const int e = tid + k * R::NT, g = e / D, j = e - g * D;
        if (e < G * D && g >= g0 && g < g0 + GB) {
            float s = 0.f;
#pragma unroll
            for (int c = 0; c < R::NTG; ++c) s += os[(c * GB + g - g0) * D + j];
            orr[k] = s;
        }
    }
}

// the phases in turn, on SCR bytes of scratch
template <int D, int G, int NW, int SCR>
__device__ void ring_attend(const DecodeArgs &a, const RingRegs<D, G, NW> &rr, float *scr, float *rm, float *rl,
                            int bk, int b, int kvh, int r0, int n, float (&orr)[RingShape<D, G, NW>::NE]) {
    using R = RingShape<D, G, NW>;
    constexpr int RP = kRingPerSplit<D>;
    constexpr int GB = R::gb(SCR);
    static_assert((R::fixed() + R::NTG * GB * D) * 4 <= SCR, "ring scratch in LDS");
    float *qr = scr, *pr = scr + G * D, *os = pr + G * RP;
    ring_p1<D, G, NW>(a, rr, qr, bk, b, kvh, r0, n);
    __syncthreads();
    ring_p2<D, G, NW>(a, rr, qr, pr, n);
    __syncthreads();
    ring_p3<D, G, NW>(pr, rm, rl, n);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < R::NE; ++k) orr[k] = 0.f;
#pragma unroll
    for (int g0 = 0; g0 < G; g0 += GB) {
        ring_p4<D, G, NW, GB>(rr, pr, os, g0, n);
        __syncthreads();
        ring_p5<D, G, NW, GB>(os, g0, orr);
        __syncthreads();  // os is rewritten by the next group, the region by the staging copies
    }
}

// The split's ring tokens in 12-wave groups, attended by one wave from the LDS copies of their
// rows (made by that wave's first copies): logits with lane = token, the softmax of each head
// across the lanes, o with lane = coordinate pair; (m, l) into rm / rl and o into ro.  A fused
// step's new token (ring slot new_slot) is taken from the input rounded to fp16, as the append
// rounds it, and written into the ring and into the LDS rows first.  rq holds the unrotated
// queries on entry and the p values afterwards.
template <int D, int VB, int G, int NW>
__device__ void ring_wave12(const DecodeArgs &a, DecodeSmem<D, VB, G, NW> &sm, int bk, int r0, int n) {
    static_assert(D == 128 && NW == 12, "12-wave groups at head_dim 128");
    const int lane = threadIdx.x & 63;
    wait_vm<0>();  // the wave's own copies of the rows
    const int ns = a.new_slot - r0;
    if (a.new_slot >= 0 && ns >= 0 && ns < n) {
        const int64_t e0 = (int64_t)bk * D + 2 * lane;
        float k0, k1, v0, v1;
        if (a.kv_dtype == TQ_F32) {
            k0 = load1(a.k_new, e0, f32_tag{}); k1 = load1(a.k_new, e0 + 1, f32_tag{});
            v0 = load1(a.v_new, e0, f32_tag{}); v1 = load1(a.v_new, e0 + 1, f32_tag{});
        } else if (a.kv_dtype == TQ_BF16) {
            k0 = load1(a.k_new, e0, bf16_tag{}); k1 = load1(a.k_new, e0 + 1, bf16_tag{});
            v0 = load1(a.v_new, e0, bf16_tag{}); v1 = load1(a.v_new, e0 + 1, bf16_tag{});
        } else {
            k0 = load1(a.k_new, e0, f16_tag{}); k1 = load1(a.k_new, e0 + 1, f16_tag{});
            v0 = load1(a.v_new, e0, f16_tag{}); v1 = load1(a.v_new, e0 + 1, f16_tag{});
        }
        const uint32_t kw = f32_to_f16_bits(k0) | ((uint32_t)f32_to_f16_bits(k1) << 16);
        const uint32_t vw = f32_to_f16_bits(v0) | ((uint32_t)f32_to_f16_bits(v1) << 16);
        *reinterpret_cast<uint32_t *>(sm.rk + (ns >> 2) * 1040 + (ns & 3) * 256 + 4 * lane) = kw;
        *reinterpret_cast<uint32_t *>(sm.rv + (ns >> 2) * 1024 + (ns & 3) * 256 + 4 * lane) = vw;
        const int64_t slot = ((int64_t)bk * a.buffer_size + a.new_slot) * D;
        reinterpret_cast<uint32_t *>(a.rk + slot)[lane] = kw;
        reinterpret_cast<uint32_t *>(a.rv + slot)[lane] = vw;
    }
    wave_sync();
    // logits (log2 units) of token `lane` for every head
    const int tk = min(lane, n - 1);
    const unsigned char *kr = sm.rk + (tk >> 2) * 1040 + (tk & 3) * 256;
    float s[G];
#pragma unroll
    for (int g = 0; g < G; ++g) s[g] = 0.f;
#pragma unroll 4
    for (int k = 0; k < D / 8; ++k) {
        const uint4 kv = *reinterpret_cast<const uint4 *>(kr + 16 * k);
        const float e[8] = {f16_lo(kv.x), f16_hi(kv.x), f16_lo(kv.y), f16_hi(kv.y),
                            f16_lo(kv.z), f16_hi(kv.z), f16_lo(kv.w), f16_hi(kv.w)};
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float4 q0 = *reinterpret_cast<const float4 *>(&sm.rq[g][8 * k]);
            const float4 q1 = *reinterpret_cast<const float4 *>(&sm.rq[g][8 * k + 4]);
            s[g] = fmaf(e[0], q0.x, s[g]);
            s[g] = fmaf(e[1], q0.y, s[g]);
            s[g] = fmaf(e[2], q0.z, s[g]);
            s[g] = fmaf(e[3], q0.w, s[g]);
            s[g] = fmaf(e[4], q1.x, s[g]);
            s[g] = fmaf(e[5], q1.y, s[g]);
            s[g] = fmaf(e[6], q1.z, s[g]);
            s[g] = fmaf(e[7], q1.w, s[g]);
        }
    }
    const float lscale = a.scale * kLog2e;
    float m[G], l[G], pv[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float x = lane < n ? s[g] * lscale : -INFINITY;
        float mx = x;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        pv[g] = lane < n ? exp2f(x - mx) : 0.f;
        float sum = pv[g];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
        m[g] = mx;
        l[g] = sum;
    }
    wave_sync();  // every lane has read the queries
#pragma unroll
    for (int g = 0; g < G; ++g) sm.rq[g][lane] = pv[g];
    wave_sync();
    // o of coordinates 2 lane, 2 lane + 1: sum over the tokens of p v (p = 0 past n)
    float o0[G], o1[G];
#pragma unroll
    for (int g = 0; g < G; ++g) o0[g] = o1[g] = 0.f;
    for (int t4 = 0; t4 < n; t4 += 4) {
        float4 pp[G];
#pragma unroll
        for (int g = 0; g < G; ++g) pp[g] = *reinterpret_cast<const float4 *>(&sm.rq[g][t4]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int tt = t4 + u;
            const uint32_t vv = *reinterpret_cast<const uint32_t *>(sm.rv + (tt >> 2) * 1024 + (tt & 3) * 256 + 4 * lane);
            const float va = f16_lo(vv), vb = f16_hi(vv);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float pg = u == 0 ? pp[g].x : (u == 1 ? pp[g].y : (u == 2 ? pp[g].z : pp[g].w));
                o0[g] = fmaf(pg, va, o0[g]);
                o1[g] = fmaf(pg, vb, o1[g]);
            }
        }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) *reinterpret_cast<float2 *>(&sm.ro[g][2 * lane]) = make_float2(o0[g], o1[g]);
    if (lane == 0)
#pragma unroll
        for (int g = 0; g < G; ++g) {
            sm.rm[g] = m[g];
            sm.rl[g] = l[g];
        }
}

// ------------------------------------------------------------------ packed split (one wave)
template <int D, int VB, int G, int NW>
__device__ void packed_wave(const DecodeArgs &a, DecodeSmem<D, VB, G, NW> &sm, int bk, int sbk, int b, int kvh,
                            int n_packed, int t_begin, int t_end, int r0, int nr,
                            float (&orr)[RingShape<D, G, NW>::NE]) {
    using S = DecodeShape<D, VB, G>;
    constexpr float kQjl = 1.2533141373155003f / D;  // sqrt(pi/2) / d
    const int lane = threadIdx.x & 63;
    // wave index made visibly uniform: block positions, record bases and LDS addresses are
    // then scalar values
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n16 = lane & 15, q = lane >> 4;
    // 12-wave groups: the codebook and sigma, loaded first and waited for here (loads issued
    // after the block copies of every workgroup come back late, and the LDS waits of the
    // preparation would wait for them too when they are scalar loads: lgkmcnt counts both)
    float cent[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    uint32_t sgw[4] = {0u, 0u, 0u, 0u};
    if constexpr (NW == 12) {
#pragma unroll
        for (int i = 0; i < 8; ++i) cent[i] = a.centroids[i];
#pragma unroll
        for (int i = 0; i < 4; ++i) sgw[i] = a.sign_bits[i];
        asm volatile("" : "+v"(cent[0]), "+v"(cent[1]), "+v"(cent[2]), "+v"(cent[3]), "+v"(cent[4]), "+v"(cent[5]),
                     "+v"(cent[6]), "+v"(cent[7]), "+v"(sgw[0]), "+v"(sgw[1]), "+v"(sgw[2]), "+v"(sgw[3]));
    }
    auto centroid = [&](int i) -> float {
        if constexpr (NW == 12) return cent[i];
        else return a.centroids[i];
    };

    // score products.  The query is the A operand (16 rows of query parts), the key block
    // the B operand (16 token columns per tile), so a tile's result holds every part of
    // every head for each of its tokens.  k-step ks of lane group q covers key word
    // w = q*NKS + ks.  Centroid part: element e is coordinate 8w + {0,2,4,6,1,3,5,7}[e] (even
    // nibbles, then odd), rows hold q'_g as fp16 hi and lo.  Sign part: element e is
    // coordinate 8w + {0,4,1,5,2,6,3,7}[e], rows hold -w_g hi and lo.  Row roles: G <= 4
    // places centroid hi, centroid lo, sign hi and sign lo of every head in disjoint rows of
    // one accumulator (G = 1: rows 0..3 and a copy in rows 8..11; G = 2: rows 0..7; G = 4:
    // all 16); G = 8 has one accumulator for the centroid rows (hi 0..7, lo 8..15) and one
    // for the sign rows.
    // ---- staging setup
    // record of token t0 of this slice (a block of 32 tokens from t0, a multiple of 32, lies in
    // one page of a paged store, since pages hold a multiple of 32 tokens)
    // (the same for every lane: made visibly uniform, so the copy bases are scalar values)
    auto block_rec = [&](int t0) -> int64_t {
        const int64_t r = record_index(a.bt, a.pt, a.pps, a.n_pages, a.cap, a.err, sbk, t0);
        return (int64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)r) |
               ((int64_t)__builtin_amdgcn_readfirstlane((int)(r >> 32)) << 32);
    };
    const int last = n_packed - 1;
    const uint32_t lds_wave = (uint32_t)(uintptr_t)&sm.stage[0][wave][0];
    // ---- staging: block at token t0 into buffer bi (token indices clamped to the last
    //      packed token, so every copy reads records of this slice)
    // per-lane parts of the copies of a block (offsets from the block's first record);
    // value records go to LDS slot 4 (t % 8) + t / 8
    // (copy i of a kind: record r of the block, byte column inside the record; the clamped
    // path recomputes them, the offsets of the whole-block path stay in registers)
    // key words: LDS chunk (copy i = tile tt * NC + j, lane L) holds the 16 bytes that lane L
    // reads for tile tt, part j: token 16 tt + L % 16, words (L / 16) NKS + 4 j .. + 3, so the
    // reads of a tile are one contiguous kilobyte (no bank conflicts)
    constexpr int NC = S::NKS / 4;
    static_assert(S::N_KW == 2 * NC, "two tiles of key chunks per block");
    auto vw_rc = [&](int ln, int i, uint32_t &r, uint32_t &col) {
        const int c = ln + 64 * i;
        const int slot = c / (S::VW / 4);
        r = 8 * (slot & 3) + (slot >> 2);
        col = (c % (S::VW / 4)) * 16;
    };
    auto vs_rc = [&](int ln, int i, uint32_t &r, uint32_t &col) {
        const int c = ln + 64 * i;  // 4-byte piece of the block's scales
        r = c / (S::NG / 2);
        col = (c % (S::NG / 2)) * 4;
    };
    // whole-block path: norms and scales of a block are contiguous bytes (copy i of a lane at
    // 4 (lane + 64 i), the 64 i part as an immediate); key chunks at the lane's offset plus a
    // uniform part per copy; the value records are permuted into LDS slot order
    const uint32_t ok0 = (uint32_t)n16 * (S::KW * 4) + (uint32_t)q * (S::NKS * 4), o4 = 4u * lane;
    uint32_t o_vw[S::N_VW];
#pragma unroll
    for (int i = 0; i < S::N_VW; ++i) {
        uint32_t r, col;
        vw_rc(lane, i, r, col);
        o_vw[i] = r * (S::VW * 4) + col;
    }
    auto issue = [&](int t0, int bi, bool first = false) {
        const uint32_t base = lds_wave + (uint32_t)(bi * NW * S::BUF_B);
        // (a wave's first copies overwrite no buffer it has read)
        if (!first) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int64_t rb = block_rec(t0);
        const uint32_t *kw_b = a.kw + rb * S::KW;
        const float *kn_b = a.kn + rb * 2;
        const uint32_t *vw_b = a.vw + rb * S::VW;
        const uint16_t *vs_b = a.vs + rb * S::NG;
        if (t0 + kBlock - 1 <= last) {
            // whole block in range: uniform record base, loop-invariant lane offsets
            static_assert(S::N_KW <= 4 && S::N_VS <= 16, "immediate offsets");
            // (the immediate offset IMM moves the LDS destination too: copy i of the keys reads
            // the block at ok0 + IMM, IMM = 16 tt KW 4 + 16 j, and lands at base + 1024 i)
            dma16<0>(kw_b, ok0, base);
            if constexpr (NC == 1) {
                dma16<1024>(kw_b, ok0, base);  // tile 1: 16 records of 64 bytes further
            } else {
                static_assert(NC == 1 || (NC == 2 && S::KW * 4 * 16 == 2048), "key chunk layout");
                dma16<16>(kw_b, ok0, base + 1024 - 16);
                dma16<2048>(kw_b, ok0, base + 2048 - 2048);
                dma16<2064>(kw_b, ok0, base + 3072 - 2064);
            }
            dma4<0>(kn_b, o4, base + S::OFF_KN);
#pragma unroll
            for (int i = 0; i < S::N_VW; ++i) dma16(vw_b, o_vw[i], base + S::OFF_VW + 1024 * i);
            dma4<0>(vs_b, o4, base + S::OFF_VS);
            if constexpr (S::N_VS > 1) dma4<256>(vs_b, o4, base + S::OFF_VS);
            static_assert(S::N_VS <= 2, "scale copies");
        } else {
            // the last block(s): token indices clamped to the last packed token, as offsets
            // from the block's first record (the lane's rows and columns are recomputed here
            // rather than held across the loop)
            int lane_c = lane;
            asm volatile("" : "+v"(lane_c));
#pragma unroll
            for (int i = 0; i < S::N_KW; ++i) {
                const int tt = i / NC, j = i % NC;
                const uint32_t tok = (uint32_t)(min(t0 + 16 * tt + (lane_c & 15), last) - t0);
                dma16(kw_b, tok * (S::KW * 4) + (uint32_t)(lane_c >> 4) * (S::NKS * 4) + 16 * j, base + 1024 * i);
            }
            {
                const uint32_t tok = (uint32_t)(min(t0 + (lane_c >> 1), last) - t0);
                dma4(kn_b, tok * 8 + (lane_c & 1) * 4, base + S::OFF_KN);
            }
#pragma unroll
            for (int i = 0; i < S::N_VW; ++i) {
                uint32_t r, col;
                vw_rc(lane_c, i, r, col);
                const uint32_t tok = (uint32_t)(min(t0 + (int)r, last) - t0);
                dma16(vw_b, tok * (S::VW * 4) + col, base + S::OFF_VW + 1024 * i);
            }
#pragma unroll
            for (int i = 0; i < S::N_VS; ++i) {
                uint32_t r, col;
                vs_rc(lane_c, i, r, col);
                const uint32_t tok = (uint32_t)(min(t0 + (int)r, last) - t0);
                dma4(vs_b, tok * (S::NG * 2) + col, base + S::OFF_VS + 256 * i);
            }
        }
    };

    // The split's blocks (32 tokens from t_begin): wave w starts with blocks w and w + NW.
    // 4-wave groups: then every NW-th block (a fixed order, so results repeat bit for bit).
    // 12-wave groups: each further block from an LDS counter, so the waves of the CU finish
    // together (which wave sums which block then varies between calls).  The first block's
    // copies go out before the query preparation (which uses the second staging buffers),
    // the second block's after it.  The compiler's own waits for the preparation's loads
    // then also cover the older copies.
    const int nb = (t_end - t_begin + kBlock - 1) / kBlock;
    // 12-wave groups: wave NW - 1 attends to the split's ring tokens and takes no first blocks
    constexpr bool RW = NW == 12;
    const bool ringw = RW && nr > 0;
    const int nws = ringw ? NW - 1 : NW;
    int b0 = wave, b1 = wave + nws;
    if (wave >= nws) b0 = b1 = nb;
    if (threadIdx.x == 0) sm.next_blk = 2 * nws;  // read after the barriers below
    // 12-wave groups: S (piece-major) and the slice's queries into the second staging buffers,
    // copied ahead of the first blocks (the preparation then waits for these alone); the ring
    // wave copies its tokens' rows instead
    unsigned char *const prepb = &sm.stage[1][0][0];
    constexpr int PS_B = D * D * 2;
    constexpr int PQ_B = G * D * 4 > 1024 ? G * D * 4 : 1024;
    if constexpr (RW) {
        static_assert(D == 128 && PS_B + PQ_B + 2 * G * D * 4 <= NW * S::BUF_B, "12-wave preparation in LDS");
        if (wave < nws) {
            const int qbytes = a.q_dtype == TQ_F32 ? 4 : 2;
            const int qsz = G * D * qbytes;
            const int nch = PS_B / 1024 + (qsz + 1023) / 1024;
            const unsigned char *qsrc =
                static_cast<const unsigned char *>(a.q) + ((int64_t)b * a.hq + kvh * G) * D * qbytes;
            const uint32_t pl = (uint32_t)(uintptr_t)prepb;
            for (int c = wave; c < nch; c += nws) {
                if (c < PS_B / 1024) {
                    const int s = 64 * c + lane, k = s / D, i = s % D;
                    dma16(a.S, (uint32_t)((i * D + 8 * k) * 2), pl + 1024 * c);
                } else {
                    const int cq = c - PS_B / 1024;
                    dma16(qsrc, (uint32_t)min(1024 * cq + 16 * lane, qsz - 16), pl + PS_B + 1024 * cq);
                }
            }
        } else {
            const int64_t r0e = ((int64_t)bk * a.buffer_size + r0) * D;
            const uint32_t lk = (uint32_t)(uintptr_t)&sm.rk[0], lv = (uint32_t)(uintptr_t)&sm.rv[0];
            for (int c = 0; 4 * c < nr; ++c) {
                const uint32_t off = (uint32_t)(min(4 * c + (lane >> 4), nr - 1) * D * 2 + (lane & 15) * 16);
                dma16(a.rk + r0e, off, lk + 1040 * c);
                dma16(a.rv + r0e, off, lv + 1024 * c);
            }
        }
        // S and the queries come back before the block copies of every workgroup crowd the
        // memory system, and the preparation then runs while those are in flight
        if (wave < nws) wait_vm<0>();
    }
    if (b0 < nb) issue(t_begin + kBlock * b0, 0, true);
    // centroid byte tables (built after the first copies are out): v_perm with selector byte idx picks byte idx of (t*1 : t*0), so
    // tl/th hold the low/high bytes of the eight fp16 centroids
    uint32_t tl0 = 0, tl1 = 0, th0 = 0, th1 = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t h = f32_to_f16_bits(centroid(i));
        const int sh = 8 * (i & 3);
        if (i < 4) {
            tl0 |= (h & 0xffu) << sh;
            th0 |= (h >> 8) << sh;
        } else {
            tl1 |= (h & 0xffu) << sh;
            th1 |= (h >> 8) << sh;
        }
    }

    // all loads of the start at once: the ring tokens' words, then the query preparation's
    // inputs (at d = 256 the prepared queries from the workspace)
    RingRegs<D, G, NW> rr;
    if constexpr (!RW) {
        if (nr > 0) ring_load<D, G, NW>(a, rr, bk, r0, nr);
    }
    float *qw = reinterpret_cast<float *>(RW ? prepb + PS_B + PQ_B : &sm.stage[1][0][0]);
    static_assert(PrepShape<D, NW>::template floats<G>() * 4 <= NW * S::BUF_B, "query preparation in LDS");
    constexpr int NQ4 = 2 * G * D / 4;                        // float4 of the prepared queries (d = 256)
    constexpr int NPW = (NQ4 + 64 * NW - 1) / (64 * NW);      // per thread
    float4 pw4[D == 256 ? NPW : 1];
    PrepRegs<D, G, NW> prg;
    if constexpr (D == 256) {
        // prepared once per slice by k_decode_prep (at d = 256, reading the 128 KB S matrix
        // in every workgroup costs more than a launch)
        static_assert(D != 256 || PrepShape<D, NW>::PARTS == 1, "prepared-query layout");
        const float4 *src = reinterpret_cast<const float4 *>(a.prep + (int64_t)bk * 2 * G * D);
#pragma unroll
        for (int i = 0; i < NPW; ++i)
            if (threadIdx.x + i * 64 * NW < NQ4) pw4[i] = src[threadIdx.x + i * 64 * NW];
    } else if constexpr (!RW) {
        prep_load<D, G, NW>(a, prg, b, kvh);
    }
    // The split's ring tokens use the second staging buffers as scratch too.  Where the ring
    // scratch fits after the query preparation's (with the same head grouping as on its own),
    // the phases of the two share their barriers (MERGED); otherwise the ring goes first.
    using RS = RingShape<D, G, NW>;
    constexpr int QWB = PrepShape<D, NW>::template floats<G>() * 4;
    constexpr int RSB = NW * S::BUF_B - QWB;
    constexpr int GBM = RS::gb(NW * S::BUF_B);
    constexpr bool MERGED = !RW && (RS::fixed() + RS::NTG * GBM * D) * 4 <= RSB;
    float *rqr = qw + QWB / 4, *rpr = rqr + G * D, *ros = rpr + G * kRingPerSplit<D>;
    if constexpr (!MERGED && !RW) {
        if (nr > 0) ring_attend<D, G, NW, NW * S::BUF_B>(a, rr, qw, sm.rm, sm.rl, bk, b, kvh, r0, nr, orr);
    }
    if constexpr (RW) {
        __syncthreads();  // every wave's copies of S and of the queries
        prep_transform12<D, G, NW>(a, sgw, prepb + PS_B, qw);
        if (ringw && wave == NW - 1) {
            // the ring wave's unrotated queries (fp32)
#pragma unroll
            for (int e = 0; e < G * D / 64; ++e) {
                const int idx = lane + 64 * e;
                sm.rq[idx / D][idx % D] = lds_q(prepb + PS_B, a.q_dtype, idx);
            }
        }
    } else if constexpr (D == 256) {
#pragma unroll
        for (int i = 0; i < NPW; ++i)
            if (threadIdx.x + i * 64 * NW < NQ4) reinterpret_cast<float4 *>(qw)[threadIdx.x + i * 64 * NW] = pw4[i];
    } else {
        prep_transform<D, G, NW>(prg, qw);
    }
    if constexpr (MERGED) {
        if (nr > 0) ring_p1<D, G, NW>(a, rr, rqr, bk, b, kvh, r0, nr);
    }
    __syncthreads();
    if constexpr (RW) prep_product12<D, G, NW>(prepb, qw);
    else if constexpr (D != 256) prep_product<D, G, NW>(prg, qw);
    if constexpr (MERGED) {
        if (nr > 0) ring_p2<D, G, NW>(a, rr, rqr, rpr, nr);
    }
    __syncthreads();

    // Both parts are pre-scaled by scale * log2(e) / sqrt(d) (the sign part also by
    // sqrt(pi/2)/d), so that the logit in log2 units is |k| (centroid part + gamma * sign part).
    // This lane's row n16: role in the centroid and in the sign operand (0: zero row, 1: hi,
    // 2: lo), its head, and its slot among the nonzero rows (compact LDS copy).
    using SM = DecodeSmem<D, VB, G, NW>;
    int rc, rs, rg, ri;
    if constexpr (G == 8) {
        rg = n16 & 7;
        rc = rs = 1 + (n16 >> 3);
        ri = n16;
    } else {
        int part;  // 0: centroid hi, 1: centroid lo, 2: sign hi, 3: sign lo, -1: none
        if constexpr (G == 1) {
            part = (n16 & 4) ? -1 : (n16 & 3);
            rg = 0;
            ri = (n16 & 1) + 2 * (n16 >> 3);
        } else if constexpr (G == 2) {
            part = n16 < 8 ? (n16 >> 1) : -1;
            rg = n16 & 1;
            ri = n16 & 3;
        } else {
            part = n16 >> 2;
            rg = n16 & 3;
            ri = n16 & 7;
        }
        rc = part == 0 ? 1 : (part == 1 ? 2 : 0);
        rs = part == 2 ? 1 : (part == 3 ? 2 : 0);
    }
    u32x4_t bc[S::BLDS ? 1 : S::NKS], bs[S::BLDS ? 1 : S::NKS];
    // ---- int8 score path (head_dim 128, four query heads per kv head).  The stored centroids
    // are binary16 values, so c * 2^Sc is an integer for a power of two 2^Sc that keeps every
    // |c * 2^Sc| < 2^14 (checked when the tables are built); each such integer is two signed
    // bytes (hi * 256 + lo), looked up by index with byte permutes.  q' and w = S q' of each head
    // are taken to 24-bit fixed point (x * 2^s rounded, |x * 2^s| < 2^22 for the head's largest
    // coordinate) and split into three signed byte digits (x = 2^16 d0 + 2^8 d1 + d2): A rows
    // 4 g + k hold digit k of head g (row 4 g + 3 is zero), so the products on
    // v_mfma_i32_16x16x64_i8 are exact integer sums, and lane group q of the result holds head q.
    // (Measured against the oracle at every workload's full size: the same decode errors as the
    // fp16 hi + lo query operands this replaces, and as a fourth digit.)
    // Coordinates: lane group q covers key words 4q .. 4q + 3; k-step ks uses words 4q + 2ks and
    // 4q + 2ks + 1; dword r of an operand holds the even (r even) or odd coordinates of word
    // 4q + 2ks + r / 2, byte b being coordinate 8 w + 2 b + r % 2.
    constexpr bool I8 = D == 128 && G == 4;
    i32x4_t qa[2], wa[2];
    float i8_alpha = 0.f, i8_beta4 = 0.f, i8_mbw = 0.f;
    uint32_t ch0 = 0, ch1 = 0, cl0 = 0, cl1 = 0;  // int8 path: hi / lo bytes of c * 2^Sc by index
    u32x4_t *const afrag = reinterpret_cast<u32x4_t *>(&sm.bfrag[0][0]);  // the digit bytes
    static_assert(!I8 || sizeof(sm.bfrag) >= 2 * G * 3 * 128, "int8 digits in the fragment area");
    int i8_sc = 0;
    if constexpr (I8) {
        float cmax = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) cmax = fmaxf(cmax, fabsf(centroid(i)));
        int ec;
        (void)frexpf(cmax, &ec);  // cmax < 2^ec
        i8_sc = 14 - ec;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int ci = (int)ldexpf(centroid(i), i8_sc);
            const int lo = ((ci + 128) & 255) - 128, hi = (ci - lo) >> 8;
            const int sh = 8 * (i & 3);
            if (i < 4) {
                cl0 |= (uint32_t)(lo & 255) << sh;
                ch0 |= (uint32_t)(hi & 255) << sh;
            } else {
                cl1 |= (uint32_t)(lo & 255) << sh;
                ch1 |= (uint32_t)(hi & 255) << sh;
            }
        }
    }
    if constexpr (I8) {
        const float cs = a.scale * kLog2e * (1.0f / sqrtf((float)D)), ss = cs * kQjl;
        // wave g takes head g to fixed point and writes the digit bytes straight into the
        // operand layout: region (which = q' or w, head g, digit k) holds 128 bytes, coordinate
        // c at byte 8 (c / 8) + 4 (c % 2) + (c % 8) / 2, so that the operand of lane (row
        // 4 g + k, lane group qq) at k-step ks is the 16 bytes at 32 qq + 16 ks; and stores the
        // head's constants
        unsigned char *const dig = reinterpret_cast<unsigned char *>(afrag);  // [which][g][k][128]
        if (wave < G) {
            constexpr int PARTS = PrepShape<D, NW>::PARTS;
            const int g = wave;
            float xq[2], xw[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int j = lane + 64 * e;
                xq[e] = qw[g * D + j];
                float sw = 0.f;
#pragma unroll
                for (int pt = 0; pt < PARTS; ++pt) sw += qw[(G + pt * G + g) * D + j];
                xw[e] = sw;
            }
            float mq = fmaxf(fabsf(xq[0]), fabsf(xq[1])), mw = fmaxf(fabsf(xw[0]), fabsf(xw[1]));
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                mq = fmaxf(mq, __shfl_xor(mq, o));
                mw = fmaxf(mw, __shfl_xor(mw, o));
            }
            int eq, ew;
            (void)frexpf(mq, &eq);
            (void)frexpf(mw, &ew);
            const int sq = 22 - eq, sw = 22 - ew;
            int wsum = 0;  // |sum| < 128 * 2^22: exact in 32 bits
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int c = lane + 64 * e;
                const int pos = 8 * (c >> 3) + 4 * (c & 1) + ((c & 7) >> 1);
                const int iq = (int)rintf(ldexpf(xq[e], sq)), iw = (int)rintf(ldexpf(xw[e], sw));
                wsum += iw;
#pragma unroll
                for (int wh = 0; wh < 2; ++wh) {
                    const int v = wh ? iw : iq;
                    const int d2 = ((v + 128) & 255) - 128, v1 = (v - d2) >> 8;
                    const int d1 = ((v1 + 128) & 255) - 128, d0 = (v1 - d1) >> 8;
                    unsigned char *r = dig + ((wh * G + g) * 3) * 128 + pos;
                    r[0] = (unsigned char)d0;
                    r[128] = (unsigned char)d1;
                    r[256] = (unsigned char)d2;
                }
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) wsum += __shfl_xor(wsum, o);
            if (lane == 0) {
                // logit = |k| (alpha S + gamma (beta / 4 Z - beta W)), S and Z the integer sums
                const float beta = ldexpf(ss, -sw);
                sm.i8c[g][0] = ldexpf(cs, -(sq + i8_sc));
                sm.i8c[g][1] = 0.25f * beta;
                sm.i8c[g][2] = -beta * (float)wsum;
            }
        }
        if constexpr (MERGED) {
            if (nr > 0) ring_p3<D, G, NW>(rpr, sm.rm, sm.rl, nr);
        }
        __syncthreads();
    } else {
        const float cs = a.scale * kLog2e * (1.0f / sqrtf((float)D)), ss = cs * kQjl;
        // q' of head rg, and the partial sums of w = S q' (summed here)
        constexpr int PARTS = PrepShape<D, NW>::PARTS;
        const float *pq = qw + rg * D;
        const float *pw = qw + (G + rg) * D;
        constexpr int ce[8] = {0, 2, 4, 6, 1, 3, 5, 7};
        constexpr int se[8] = {0, 4, 1, 5, 2, 6, 3, 7};
        auto frag = [&](int ks, u32x4_t &fc, u32x4_t &fs) {
            const int w = q * S::NKS + ks;
            const float4 m0 = *reinterpret_cast<const float4 *>(pq + 8 * w);
            const float4 m1 = *reinterpret_cast<const float4 *>(pq + 8 * w + 4);
            float4 s0 = *reinterpret_cast<const float4 *>(pw + 8 * w);
            float4 s1 = *reinterpret_cast<const float4 *>(pw + 8 * w + 4);
#pragma unroll
            for (int pt = 1; pt < PARTS; ++pt) {
                const float4 u0 = *reinterpret_cast<const float4 *>(pw + pt * G * D + 8 * w);
                const float4 u1 = *reinterpret_cast<const float4 *>(pw + pt * G * D + 8 * w + 4);
                s0.x += u0.x; s0.y += u0.y; s0.z += u0.z; s0.w += u0.w;
                s1.x += u1.x; s1.y += u1.y; s1.z += u1.z; s1.w += u1.w;
            }
            const float vm[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
            const float vs[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
            uint16_t hc[8], hs[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                _Float16 h, l;
                split_hl(cs * vm[ce[e]], h, l);
                hc[e] = rc == 1 ? __builtin_bit_cast(uint16_t, h) : (rc == 2 ? __builtin_bit_cast(uint16_t, l) : 0);
                split_hl(-ss * vs[se[e]], h, l);
                hs[e] = rs == 1 ? __builtin_bit_cast(uint16_t, h) : (rs == 2 ? __builtin_bit_cast(uint16_t, l) : 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                fc[i] = hc[2 * i] | ((uint32_t)hc[2 * i + 1] << 16);
                fs[i] = hs[2 * i] | ((uint32_t)hs[2 * i + 1] << 16);
            }
        };
        if constexpr (S::BLDS) {
            // wave w < NKS builds k-step w (NKS == 4 at d = 128)
            static_assert(!S::BLDS || (S::NKS == 4 && NW >= 4), "one k-step per wave");
            if (wave < S::NKS) {
                u32x4_t fc, fs;
                frag(wave, fc, fs);
                if (rc) sm.bfrag[wave][q * SM::NSL + ri] = fc;
                if (rs) sm.bfrag[S::NKS + wave][q * SM::NSL + ri] = fs;
                if (lane == 0) {
                    sm.bfrag[wave][SM::FZ] = (u32x4_t){0u, 0u, 0u, 0u};
                    sm.bfrag[S::NKS + wave][SM::FZ] = (u32x4_t){0u, 0u, 0u, 0u};
                }
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < S::NKS; ++ks) frag(ks, bc[ks], bs[ks]);
        }
        if constexpr (MERGED) {
            if (nr > 0) ring_p3<D, G, NW>(rpr, sm.rm, sm.rl, nr);
        }
        __syncthreads();  // fragments visible (d = 128)
    }
    if constexpr (MERGED) {
        if (nr > 0) {
#pragma unroll
            for (int k = 0; k < RS::NE; ++k) orr[k] = 0.f;
#pragma unroll
            for (int g0 = 0; g0 < G; g0 += GBM) {
                ring_p4<D, G, NW, GBM>(rr, rpr, ros, g0, nr);
                __syncthreads();
                ring_p5<D, G, NW, GBM>(ros, g0, orr);
                __syncthreads();  // os is rewritten by the next group, the region by the staging copies
            }
        }
    }
    if constexpr (I8) {
        // row n16 = 4 g + k: digit k of head g (row 4 g + 3 is zero)
        const int fg = n16 >> 2, fk = n16 & 3;
        const unsigned char *dig = reinterpret_cast<const unsigned char *>(afrag);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int off = 32 * q + 16 * ks;
            qa[ks] = fk < 3 ? *reinterpret_cast<const i32x4_t *>(dig + (fg * 3 + fk) * 128 + off) : (i32x4_t){0, 0, 0, 0};
            wa[ks] = fk < 3 ? *reinterpret_cast<const i32x4_t *>(dig + ((G + fg) * 3 + fk) * 128 + off)
                            : (i32x4_t){0, 0, 0, 0};
        }
        i8_alpha = sm.i8c[q][0];
        i8_beta4 = sm.i8c[q][1];
        i8_mbw = sm.i8c[q][2];
    }
    // (the second staging buffers are free)
    if constexpr (RW) {
        if (ringw && wave == NW - 1) {
            ring_wave12<D, VB, G, NW>(a, sm, bk, r0, nr);
            // then two blocks from the counter
            int nx = 0;
            if (lane == 0) nx = atomicAdd(&sm.next_blk, 2);
            nx = __builtin_amdgcn_readfirstlane(nx);
            b0 = nx;
            b1 = nx + 1;
            if (b0 < nb) issue(t_begin + kBlock * b0, 0);
        }
    }
    if (b1 < nb) issue(t_begin + kBlock * b1, 1);
    const int cslot = rc ? q * SM::NSL + ri : SM::FZ, sslot = rs ? q * SM::NSL + ri : SM::FZ;
    // The lane's logits after the score products: token row trow of the block, heads
    // hbase .. hbase + NLR - 1.  The running reference max per head is kept in LDS (read
    // once per block); value accumulators; per value column (head, group): sums of B and of
    // p over the lane's tokens.
    constexpr int NLR = G < 4 ? G : 4;
    const int trow = (G == 2 || G == 8) ? 16 * (q >> 1) + n16 : 16 * (q & 1) + n16;
    const int hbase = G == 8 ? 4 * (q & 1) : 0;
    if (lane < G) sm.mref[wave][lane] = -INFINITY;
    wave_sync();
    f32x4_t acc_v[S::NPASS][S::NT];
    float sumb[S::NPASS], lsum[S::NPASS];
#pragma unroll
    for (int p = 0; p < S::NPASS; ++p) {
        sumb[p] = 0.f;
        lsum[p] = 0.f;
#pragma unroll
        for (int t = 0; t < S::NT; ++t) acc_v[p][t] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    }

    // constants kept in registers so that and-or forms take them as operands
    uint32_t kSel = 0x07070707u, kSgn = 0x80008000u, kOne = 0x3C003C00u;
    uint32_t kCode = (((1u << VB) - 1u) << (10 - VB)) * 0x00010001u;
    asm volatile("" : "+v"(kSel), "+v"(kSgn), "+v"(kOne), "+v"(kCode));

    auto process = [&](const unsigned char *buf, int t0) {
        // ---- scores: query rows x token columns, centroid and sign parts on MFMA
        uint32_t wds[2][S::NKS];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
            for (int i = 0; i < S::NKS / 4; ++i) {
                const u32x4_t u = *reinterpret_cast<const u32x4_t *>(buf + (tt * (S::NKS / 4) + i) * 1024 + 16 * lane);
                wds[tt][4 * i] = u[0]; wds[tt][4 * i + 1] = u[1]; wds[tt][4 * i + 2] = u[2]; wds[tt][4 * i + 3] = u[3];
            }
        }
        if constexpr (I8) {
            // ---- scores on int8 matrix cores: S (centroid part, c hi and lo bytes against the
            //      digits of q') and Z (8 x the sign bits against the digits of w) per tile
            const uint32_t m7 = 0x07070707u, m8 = 0x08080808u;
            float lgv[2];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                i32x4_t ah = {0, 0, 0, 0}, al = {0, 0, 0, 0}, az = {0, 0, 0, 0};
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const uint32_t w0 = wds[tt][2 * ks], w1 = wds[tt][2 * ks + 1];
                    const uint32_t s0 = w0 >> 4, s1 = w1 >> 4;
                    const uint32_t e0 = w0 & m7, o0 = s0 & m7, e1 = w1 & m7, o1 = s1 & m7;
                    const i32x4_t bh = {(int)__builtin_amdgcn_perm(ch1, ch0, e0), (int)__builtin_amdgcn_perm(ch1, ch0, o0),
                                        (int)__builtin_amdgcn_perm(ch1, ch0, e1), (int)__builtin_amdgcn_perm(ch1, ch0, o1)};
                    const i32x4_t bl = {(int)__builtin_amdgcn_perm(cl1, cl0, e0), (int)__builtin_amdgcn_perm(cl1, cl0, o0),
                                        (int)__builtin_amdgcn_perm(cl1, cl0, e1), (int)__builtin_amdgcn_perm(cl1, cl0, o1)};
                    const i32x4_t bz = {(int)(w0 & m8), (int)(s0 & m8), (int)(w1 & m8), (int)(s1 & m8)};
                    ah = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[ks], bh, ah, 0, 0, 0);
                    al = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[ks], bl, al, 0, 0, 0);
                    az = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa[ks], bz, az, 0, 0, 0);
                }
                // lane (n16, q): head q, token 16 tt + n16; registers 0, 1, 2 = digits 0, 1, 2
                const int c0 = (ah[0] << 8) + al[0], c1 = (ah[1] << 8) + al[1], c2 = (ah[2] << 8) + al[2];
                const float sf = fmaf((float)c0, 65536.f, fmaf((float)c1, 256.f, (float)c2));
                const float zf = fmaf((float)az[0], 65536.f, fmaf((float)az[1], 256.f, (float)az[2]));
                const float2 kn = *reinterpret_cast<const float2 *>(buf + S::OFF_KN + (16 * tt + n16) * 8);
                float lv = kn.x * fmaf(kn.y, fmaf(i8_beta4, zf, i8_mbw), i8_alpha * sf);
                if (t0 + 16 * tt + n16 >= t_end) lv = -INFINITY;
                lgv[tt] = lv;
            }
            // ---- online softmax of head q with a reference max that only moves when a logit
            //      exceeds it (rare after the first block); p <= 1 always
            float m_ref = sm.mref[wave][q];
            if (__ballot(lgv[0] > m_ref || lgv[1] > m_ref)) {
                float mb = fmaxf(lgv[0], lgv[1]);
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) mb = fmaxf(mb, __shfl_xor(mb, o));
                const float m_new = fmaxf(m_ref, mb);
                const float corr = (m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
                m_ref = m_new;
                if (n16 == 0) {
                    sm.corr[wave][q] = corr;
                    sm.mref[wave][q] = m_new;
                }
                wave_sync();
#pragma unroll
                for (int p = 0; p < S::NPASS; ++p) {
                    const int n = n16 + 16 * p;
                    const float c = (n < S::NCOL) ? sm.corr[wave][n / S::NG] : 0.f;
                    sumb[p] *= c;
                    lsum[p] *= c;
#pragma unroll
                    for (int t = 0; t < S::NT; ++t)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            float e = acc_v[p][t][i];
                            asm volatile("v_mul_f32 %0, %0, %1" : "+v"(e) : "v"(c));
                            acc_v[p][t][i] = e;
                        }
                }
            }
            sm.pb[wave][q][n16] = __builtin_amdgcn_exp2f(lgv[0] - m_ref);
            sm.pb[wave][q][16 + n16] = __builtin_amdgcn_exp2f(lgv[1] - m_ref);
        } else {
        constexpr int NACC = G == 8 ? 2 : 1;  // [centroid, sign] for G = 8, one stacked otherwise
        f32x4_t acc[NACC][2];
#pragma unroll
        for (int j = 0; j < NACC; ++j)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) acc[j][tt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < S::NKS; ++ks) {
            u32x4_t qc, qs;
            if constexpr (S::BLDS) {
                qc = sm.bfrag[ks][cslot];
                qs = sm.bfrag[S::NKS + ks][sslot];
            } else {
                qc = bc[ks];
                qs = bs[ks];
            }
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const uint32_t word = wds[tt][ks];
                const uint32_t sel_e = word & kSel, sel_o = (word >> 4) & kSel;
                const uint32_t le = __builtin_amdgcn_perm(tl1, tl0, sel_e);
                const uint32_t he = __builtin_amdgcn_perm(th1, th0, sel_e);
                const uint32_t lo = __builtin_amdgcn_perm(tl1, tl0, sel_o);
                const uint32_t ho = __builtin_amdgcn_perm(th1, th0, sel_o);
                const u32x4_t Kc = {__builtin_amdgcn_perm(he, le, 0x05010400u), __builtin_amdgcn_perm(he, le, 0x07030602u),
                                    __builtin_amdgcn_perm(ho, lo, 0x05010400u), __builtin_amdgcn_perm(ho, lo, 0x07030602u)};
                u32x4_t Ks;
#pragma unroll
                for (int r = 0; r < 4; ++r) Ks[r] = ((word << (12 - 4 * r)) & kSgn) | kOne;
                acc[0][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, qc),
                                                                    __builtin_bit_cast(half8_t, Kc), acc[0][tt], 0, 0, 0);
                acc[NACC - 1][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    __builtin_bit_cast(half8_t, qs), __builtin_bit_cast(half8_t, Ks), acc[NACC - 1][tt], 0, 0, 0);
            }
        }
        // ---- logits: hi + lo of each part and centroid + gamma * sign, gathered by row swaps
        //      (lane rows q: 16-lane swaps exchange rows 1 <-> 0 and 3 <-> 2 of two registers,
        //      32-lane swaps the halves)
        float lg[NLR];
        {
            const float2 kn = *reinterpret_cast<const float2 *>(buf + S::OFF_KN + trow * 8);
            const float dn = kn.x, gm = kn.y;
            auto f2u = [](float x) { return __builtin_bit_cast(uint32_t, x); };
            auto u2f = [](uint32_t x) { return __builtin_bit_cast(float, x); };
            if constexpr (G == 4) {
                // rows (tile 0, 1): [c hi | c lo | s hi | s lo] -> [c0 c1 s0 s1] -> c and s
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const auto x = __builtin_amdgcn_permlane16_swap(f2u(acc[0][0][i]), f2u(acc[0][1][i]), false, false);
                    const float y = u2f(x[0]) + u2f(x[1]);
                    const auto z = __builtin_amdgcn_permlane32_swap(f2u(y), f2u(y), false, false);
                    lg[i] = dn * fmaf(gm, u2f(z[1]), u2f(z[0]));
                }
            } else if constexpr (G == 2) {
                // row 0: [c hi g0 g1, c lo g0 g1], row 1: the sign part; tile 1 into rows 2, 3
                float f[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    f[i] = u2f(__builtin_amdgcn_permlane32_swap(f2u(acc[0][0][i]), f2u(acc[0][1][i]), false, false)[0]);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const float u = f[h] + f[h + 2];  // rows [c t0, s t0, c t1, s t1]
                    const auto z = __builtin_amdgcn_permlane16_swap(f2u(u), f2u(u), false, false);
                    lg[h] = dn * fmaf(gm, u2f(z[1]), u2f(z[0]));
                }
            } else if constexpr (G == 1) {
                // rows 0 and 2: [c hi, c lo, s hi, s lo]; tile 1 into rows 1 and 3
                float f[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    f[i] = u2f(__builtin_amdgcn_permlane16_swap(f2u(acc[0][0][i]), f2u(acc[0][1][i]), false, false)[0]);
                lg[0] = dn * fmaf(gm, f[2] + f[3], f[0] + f[1]);
            } else {
                // rows: hi g0..3, hi g4..7, lo g0..3, lo g4..7 -> tile 0 in rows 0, 1, tile 1 in 2, 3
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const auto c = __builtin_amdgcn_permlane32_swap(f2u(acc[0][0][i]), f2u(acc[0][1][i]), false, false);
                    const auto sg = __builtin_amdgcn_permlane32_swap(f2u(acc[1][0][i]), f2u(acc[1][1][i]), false, false);
                    lg[i] = dn * fmaf(gm, u2f(sg[0]) + u2f(sg[1]), u2f(c[0]) + u2f(c[1]));
                }
            }
            if (t0 + kBlock > t_end && t0 + trow >= t_end)
#pragma unroll
                for (int i = 0; i < NLR; ++i) lg[i] = -INFINITY;
        }

        // ---- online softmax with a reference max that only moves when a logit exceeds it
        //      (rare after the first block); p <= 1 always
        float m_ref[NLR];
#pragma unroll
        for (int i = 0; i < NLR; ++i) m_ref[i] = sm.mref[wave][hbase + i];
        uint64_t gt = 0;
#pragma unroll
        for (int i = 0; i < NLR; ++i) gt |= __ballot(lg[i] > m_ref[i]);
        if (gt) {
#pragma unroll
            for (int i = 0; i < NLR; ++i) {
                float mb = lg[i];
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) mb = fmaxf(mb, __shfl_xor(mb, o));
                if constexpr (G != 8) mb = fmaxf(mb, __shfl_xor(mb, 16));
                mb = fmaxf(mb, __shfl_xor(mb, 32));
                float m_new = fmaxf(m_ref[i], mb);
                // G <= 4: every lane holds the same heads, so the max is wave-uniform (scalar)
                if constexpr (G != 8)
                    m_new = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, m_new)));
                // 2^(m_old - m_new) <= 1 (flushes to 0 far below); nothing to rescale at the start
                const float corr = (m_ref[i] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_ref[i] - m_new);
                m_ref[i] = m_new;
                if (n16 == 0) {
                    sm.corr[wave][hbase + i] = corr;
                    sm.mref[wave][hbase + i] = m_new;
                }
            }
            wave_sync();
#pragma unroll
            for (int p = 0; p < S::NPASS; ++p) {
                const int n = n16 + 16 * p;
                const float c = (n < S::NCOL) ? sm.corr[wave][n / S::NG] : 0.f;
                sumb[p] *= c;
                lsum[p] *= c;
#pragma unroll
                for (int t = 0; t < S::NT; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        // in place, so the accumulators keep their registers across the branch
                        float e = acc_v[p][t][i];
                        asm volatile("v_mul_f32 %0, %0, %1" : "+v"(e) : "v"(c));
                        acc_v[p][t][i] = e;
                    }
            }
        }
        // p = 2^(logit - m): the argument is <= 0 (or -inf for masked tokens, giving 0)
#pragma unroll
        for (int i = 0; i < NLR; ++i) {
            sm.pb[wave][hbase + i][trow] = __builtin_amdgcn_exp2f(lg[i] - m_ref[i]);
        }
        }
        wave_sync();

        // ---- values: B = p * scale in columns (head, group), hi + lo; A = codes of row n16
        u32x4_t bv_hi[S::NPASS], bv_lo[S::NPASS];
#pragma unroll
        for (int p = 0; p < S::NPASS; ++p) {
            const int n = n16 + 16 * p;
            const bool col = n < S::NCOL;
            const int gg = col ? n / S::NG : 0, grp = col ? n % S::NG : 0;
            const f32x4_t p0 = *reinterpret_cast<const f32x4_t *>(&sm.pb[wave][gg][8 * q]);
            const f32x4_t p1 = *reinterpret_cast<const f32x4_t *>(&sm.pb[wave][gg][8 * q + 4]);
            float pe[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
            lsum[p] += ((pe[0] + pe[1]) + (pe[2] + pe[3])) + ((pe[4] + pe[5]) + (pe[6] + pe[7]));
            if constexpr (S::NCOL % 16 != 0)
#pragma unroll
                for (int e = 0; e < 8; ++e) pe[e] = col ? pe[e] : 0.f;
            const _Float16 *scl = reinterpret_cast<const _Float16 *>(buf + S::OFF_VS) + 8 * q * S::NG + grp;
            typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
            const h2_t ones = __builtin_bit_cast(h2_t, kOne);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t h, l;
                mix_hl2(pe[2 * i], scl[2 * i * S::NG], pe[2 * i + 1], scl[(2 * i + 1) * S::NG], h, l);
                bv_hi[p][i] = h;
                bv_lo[p][i] = l;
                // column sums of B as the products see them (hi + lo)
                sumb[p] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, h), ones, sumb[p], false);
                sumb[p] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, l), ones, sumb[p], false);
            }
        }
        // row n16's code run of each of the lane's 8 tokens (8q .. 8q+7, LDS slot 4e + q), as
        // halfword pairs z[k][r] = (halfword k of token 8q+2r) | (halfword k of token 8q+2r+1) << 16
        uint32_t z[S::H][4];
        {
            const unsigned char *vb = buf + S::OFF_VW + q * S::VW * 4 + n16 * S::H * 2;
            constexpr int SLOT = S::VW * 4 * 4;  // bytes between tokens e and e + 1 (slots 4 apart)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if constexpr (S::H == 1) {
                    const uint32_t ha = *reinterpret_cast<const uint16_t *>(vb + (2 * r) * SLOT);
                    const uint32_t hb = *reinterpret_cast<const uint16_t *>(vb + (2 * r + 1) * SLOT);
                    z[0][r] = ha | (hb << 16);
                } else if constexpr (S::H == 2) {
                    const uint32_t wa = *reinterpret_cast<const uint32_t *>(vb + (2 * r) * SLOT);
                    const uint32_t wb = *reinterpret_cast<const uint32_t *>(vb + (2 * r + 1) * SLOT);
                    z[0][r] = __builtin_amdgcn_perm(wb, wa, 0x05040100u);
                    z[1][r] = __builtin_amdgcn_perm(wb, wa, 0x07060302u);
                } else {
                    const u32x2_t wa = *reinterpret_cast<const u32x2_t *>(vb + (2 * r) * SLOT);
                    const u32x2_t wb = *reinterpret_cast<const u32x2_t *>(vb + (2 * r + 1) * SLOT);
#pragma unroll
                    for (int hw = 0; hw < 2; ++hw) {
                        z[2 * hw][r] = __builtin_amdgcn_perm(wb[hw], wa[hw], 0x05040100u);
                        z[2 * hw + 1][r] = __builtin_amdgcn_perm(wb[hw], wa[hw], 0x07060302u);
                    }
                }
            }
        }
        // A = 1 + code / 2^VB (exact fp16: the code in the top VB mantissa bits of each half; the
        // codes kept in place as fp16 denormals would need no shift, but sums of the smallest
        // products were measured to lose precision on the matrix cores: decode error 2.8e-5
        // against 5.6e-6 this way)
#pragma unroll
        for (int t = 0; t < S::NT; ++t) {
            const int k = (VB * t) / 16, sh = (VB * t) % 16;
            u32x4_t avu;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t zz = sh >= 10 - VB ? (z[k][r] >> (sh - (10 - VB))) : (z[k][r] << ((10 - VB) - sh));
                avu[r] = (zz & kCode) | kOne;
            }
            const half8_t av = __builtin_bit_cast(half8_t, avu);
#pragma unroll
            for (int p = 0; p < S::NPASS; ++p) {
                acc_v[p][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(half8_t, bv_hi[p]), acc_v[p][t], 0, 0, 0);
                acc_v[p][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(half8_t, bv_lo[p]), acc_v[p][t], 0, 0, 0);
            }
        }
        wave_sync();  // this wave's p slots are rewritten by its next block
    };

    // ---- the wave's blocks b0 (being computed) and b1 (copies in flight), two staging
    //      buffers.  Only blocks of the split are copied: before the last one every copy is
    //      waited for.
    for (int k = 0; b0 < nb; ++k) {
        if (b1 < nb) wait_vm<S::N_DMA>(); else wait_vm<0>();
        process(&sm.stage[k & 1][wave][0], t_begin + kBlock * b0);
        b0 = b1;
        if (b1 < nb) {
            if constexpr (NW == 12) {
                int nx = 0;
                if (lane == 0) nx = atomicAdd(&sm.next_blk, 1);
                b1 = __builtin_amdgcn_readfirstlane(nx);
            } else {
                b1 += NW;
            }
            if (b1 < nb) issue(t_begin + kBlock * b1, k & 1);
        }
    }
    __syncthreads();  // every wave is done with its staging buffers (aliased by wo below)

    // ---- wave results: m, l per head; o[g][c] from the accumulators and the column sums of B
    if (lane < G) sm.wm[wave][lane] = sm.mref[wave][lane];
#pragma unroll
    for (int p = 0; p < S::NPASS; ++p) {
        sumb[p] += __shfl_xor(sumb[p], 16);
        sumb[p] += __shfl_xor(sumb[p], 32);
        lsum[p] += __shfl_xor(lsum[p], 16);
        lsum[p] += __shfl_xor(lsum[p], 32);
        // column (head, group 0) holds the head's sum of p
        const int n = n16 + 16 * p;
        if (q == 0 && n < S::NCOL && n % S::NG == 0) sm.wl[wave][n / S::NG] = lsum[p];
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
                // acc = sum B (1 + code / 2^VB): o = 2^VB acc - (2^VB + HALF - 1/2) sum B
                if (c / 32 == grp)
                    sm.x.wo[wave][gg][c] = (float)(1 << VB) * acc_v[p][t][i] - (float)((1 << VB) + S::HALF - 0.5f) * sumb[p];
            }
    }
}

// ------------------------------------------------------------------ prep kernel (d = 256)
// Workgroup (slice, band): rows band*RB .. band*RB + RB - 1 of w = S q' for the G query heads
// of one (batch, kv head); band 0 also stores q'.  prep[slice] = (q' [G][D], w [G][D]).
// The band of S is copied into LDS with coalesced loads (consecutive 16-byte chunks per
// wave), rows padded by 16 bytes; TPR threads per row (adjacent lanes) split its columns and
// are summed by lane shuffles.  Every workgroup transforms the G queries itself.
template <int D>
struct PrepBand {
    static constexpr int RB = 64;                   // rows of S per workgroup
    static constexpr int NB = D / RB;               // bands per slice
    static constexpr int RS = D + 8;                // padded LDS row stride (halfwords)
    static constexpr int TPR = kThreads / RB;       // threads per row
    static constexpr int CPT = D / TPR;             // columns per thread
    static constexpr int NCH = RB * D / 8 / kThreads;  // 16-byte chunks of the band per thread
};

template <int D, int G>
__global__ __launch_bounds__(kThreads) void k_decode_prep(DecodeArgs a) {
    using P = PrepBand<D>;
    static_assert(P::CPT % 8 == 0 && (P::TPR & (P::TPR - 1)) == 0 && P::NCH * kThreads * 8 == P::RB * D, "band shape");
    __shared__ __align__(16) uint16_t s_lds[P::RB * P::RS];
    __shared__ __align__(16) float qs[G * D];  // q' [G][D]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bk = blockIdx.x / P::NB, band = blockIdx.x % P::NB;
    const int b = bk / a.hkv, kvh = bk - b * a.hkv;
    uint4 ch[P::NCH];
    const uint4 *src = reinterpret_cast<const uint4 *>(a.S + (int64_t)band * P::RB * D);
#pragma unroll
    for (int k = 0; k < P::NCH; ++k) ch[k] = src[k * kThreads + tid];
    // q' of head g by wave g (mod 4), as in prep_query
    constexpr int E = D / 64;
    float *dst = a.prep + (int64_t)bk * 2 * G * D;
    for (int g = wave; g < G; g += kWaves) {
        const int64_t qoff = ((int64_t)b * a.hq + kvh * G + g) * D;
        float v[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int j = lane + 64 * e;
            v[e] = flip_sign(load_q(a, qoff + j), (a.sign_bits[j >> 5] >> (j & 31)) & 1u);
        }
#pragma unroll
        for (int len = 1; len < 64; len <<= 1)
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float o = __shfl_xor(v[e], len);
                v[e] = (lane & len) ? (o - v[e]) : (v[e] + o);
            }
#pragma unroll
        for (int m = 1; m < E; m <<= 1) {
            float u[E];
#pragma unroll
            for (int e = 0; e < E; ++e) u[e] = (e & m) ? (v[e ^ m] - v[e]) : (v[e] + v[e ^ m]);
#pragma unroll
            for (int e = 0; e < E; ++e) v[e] = u[e];
        }
#pragma unroll
        for (int e = 0; e < E; ++e) {
            qs[g * D + lane + 64 * e] = v[e];
            if (band == 0) dst[g * D + lane + 64 * e] = v[e];
        }
    }
#pragma unroll
    for (int k = 0; k < P::NCH; ++k) {
        const int f = k * kThreads + tid;  // chunk f: band row f / (D / 8), columns 8 (f % (D / 8)) ..
        *reinterpret_cast<uint4 *>(s_lds + (f / (D / 8)) * P::RS + 8 * (f % (D / 8))) = ch[k];
    }
    __syncthreads();
    const int row = tid / P::TPR, part = tid % P::TPR;
    float acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = 0.f;
    const uint16_t *srow = s_lds + row * P::RS + part * P::CPT;
#pragma unroll
    for (int i = 0; i < P::CPT / 8; ++i) {
        const uint4 pk = *reinterpret_cast<const uint4 *>(srow + 8 * i);
        const float s[8] = {f16_lo(pk.x), f16_hi(pk.x), f16_lo(pk.y), f16_hi(pk.y),
                            f16_lo(pk.z), f16_hi(pk.z), f16_lo(pk.w), f16_hi(pk.w)};
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float4 q0 = *reinterpret_cast<const float4 *>(qs + g * D + part * P::CPT + 8 * i);
            const float4 q1 = *reinterpret_cast<const float4 *>(qs + g * D + part * P::CPT + 8 * i + 4);
            acc[g] = fmaf(s[0], q0.x, acc[g]);
            acc[g] = fmaf(s[1], q0.y, acc[g]);
            acc[g] = fmaf(s[2], q0.z, acc[g]);
            acc[g] = fmaf(s[3], q0.w, acc[g]);
            acc[g] = fmaf(s[4], q1.x, acc[g]);
            acc[g] = fmaf(s[5], q1.y, acc[g]);
            acc[g] = fmaf(s[6], q1.z, acc[g]);
            acc[g] = fmaf(s[7], q1.w, acc[g]);
        }
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int o = 1; o < P::TPR; o <<= 1) acc[g] += __shfl_xor(acc[g], o);
    if (part == 0)
#pragma unroll
        for (int g = 0; g < G; ++g) dst[(G + g) * D + band * P::RB + row] = acc[g];
}

// ------------------------------------------------------------------ main kernel
// Workgroups of NW waves: 4 (several workgroups per CU) or 12 (one per CU, d = 128 with up
// to 4 query heads per kv head, for long splits: its waves share the split's blocks, so a
// CU's waves finish together).  Register budget (waves per SIMD): 12-wave groups 3; 4-wave
// groups 4 (<= 128 VGPRs) for d = 128 / 2-bit values with up to 4 query heads per kv head
// (LDS allows four workgroups per CU), 3 for 4-bit values (LDS allows three), 2 otherwise.
template <int D, int VB, int G, int NW>
constexpr int kDecodeWavesPerSimd = NW == 12 ? 3 : ((D == 128 && G <= 4) ? (VB == 2 ? 4 : 3) : 2);

template <int D, int VB, int G, int NW>
__global__ __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(kDecodeWavesPerSimd<D, VB, G, NW>, kDecodeWavesPerSimd<D, VB, G, NW>)))
void k_decode_main(DecodeArgs a) {
    static_assert(sizeof(DecodeSmem<D, VB, G, NW>) <= 160 * 1024, "LDS of one workgroup");
    __shared__ DecodeSmem<D, VB, G, NW> sm;
    // the arguments the start of every workgroup reads, loaded in one batch (arguments read
    // only under branches would otherwise be loaded and waited for one after another before
    // the first copies go out)
    asm volatile("" ::"s"(a.n_packed), "s"(a.per_split), "s"(a.seq_packed), "s"(a.seq_ring), "s"(a.n_ring),
                 "s"(a.ring_per_split), "s"(a.q_tokens), "s"(a.causal), "s"(a.hkv), "s"(a.n_split), "s"(a.kw),
                 "s"(a.kn), "s"(a.vw), "s"(a.vs), "s"(a.bt), "s"(a.cap));
    const int tid = threadIdx.x;
    const int split = blockIdx.x;  // split: a range of packed tokens and of ring tokens
    const int bk = blockIdx.y;     // b * hkv + kv head == slice
    const int b = bk / a.hkv, kvh = bk - b * a.hkv;
    const int n_total = a.n_split;
    float *pp = a.partial + ((int64_t)bk * n_total + split) * G * D;
    float *pml = a.partial_ml + ((int64_t)bk * n_total + split) * G * 2;

    {
        using R = RingShape<D, G, NW>;
        // this sequence's lengths: the call's, or (ragged batches) its own, clamped to them;
        // prefill: batch element b is query token b % q_tokens of sequence b / q_tokens, whose
        // packed records it reads (store slice sbk), causally up to its own position
        int n_packed = (int)a.n_packed, n_ring = a.n_ring;
        int sbk = bk;
        if (a.seq_packed) n_packed = (int)min(max(a.seq_packed[b], (int64_t)0), a.n_packed);
        if (a.seq_ring) n_ring = min(max(a.seq_ring[b], 0), a.n_ring);
        if (a.q_tokens) {
            const int seq = b / a.q_tokens, qi = b - seq * a.q_tokens;
            sbk = (int)(a.q_slice0 + seq * a.hkv + kvh);
            if (a.causal) n_packed = (int)max((int64_t)0, min((int64_t)n_packed, a.q_pos0 + qi + 1));
        }
        // ragged batches (and causal prefill): this sequence's own lengths divided evenly over
        // the splits (whole 32-token blocks; at most the call's split sizes, since the lengths
        // are clamped)
        int per_split = (int)a.per_split, ring_per_split = a.ring_per_split;
        if (a.seq_packed || (a.q_tokens && a.causal))
            per_split = ((n_packed + a.n_split - 1) / a.n_split + kBlock - 1) / kBlock * kBlock;
        if (a.seq_ring) ring_per_split = (n_ring + a.n_split - 1) / a.n_split;
        const int t_begin = split * per_split;
        const int t_end = max(t_begin, min(n_packed, t_begin + per_split));
        const int r0 = split * ring_per_split, nr = max(0, min(n_ring - r0, ring_per_split));
        float orr[R::NE];
        packed_wave<D, VB, G, NW>(a, sm, bk, sbk, b, kvh, n_packed, t_begin, t_end, r0, nr, orr);
        __syncthreads();
        // combine the waves and the split's ring tokens
#pragma unroll
        for (int k = 0; k < R::NE; ++k) {
            const int i = tid + k * 64 * NW;
            if (i >= G * D) break;
            const int g = i / D, j = i - g * D;
            const float mr = nr > 0 ? sm.rm[g] : -INFINITY;
            float M = mr;
#pragma unroll
            for (int w = 0; w < NW; ++w) M = fmaxf(M, sm.wm[w][g]);
            float L = 0.f, O = 0.f;
            if (M != -INFINITY) {
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    if (sm.wm[w][g] == -INFINITY) continue;
                    const float f = exp2f(sm.wm[w][g] - M);
                    L = fmaf(sm.wl[w][g], f, L);
                    O = fmaf(sm.x.wo[w][g][j], f, O);
                }
                if (mr != -INFINITY) {
                    const float f = exp2f(mr - M);
                    L = fmaf(sm.rl[g], f, L);
                    if constexpr (NW == 12) O = fmaf(sm.ro[g][j], f, O);
                    else O = fmaf(orr[k], f, O);
                }
            }
            if (a.n_split == 1) {
                // the only split: its result is the output (no merge launch)
                a.out[((int64_t)b * a.hq + kvh * G + g) * D + j] = L > 0.f ? O / L : 0.f;
            } else {
                pp[g * D + j] = O;
                if (j == 0) {
                    pml[g * 2] = M;
                    pml[g * 2 + 1] = L;
                }
            }
        }
    }
}

// ------------------------------------------------------------------ split merge
// One workgroup per (batch * kv head, query head of the group): combines the (m, l, o)
// partials of every split, the ring included (a separate launch, so the partials of all
// workgroups are visible without device-wide fences).  The thread's first PF partial columns and its
// (m, l) pair are loaded together up front, so the merge waits on memory once.
template <int D, int G>
__global__ __launch_bounds__(kThreads) void k_decode_merge(DecodeArgs a) {
    constexpr int NJ4 = D / 4;             // float4 columns of one head
    constexpr int NSG = kThreads / NJ4;    // split groups summed in parallel
    constexpr int PF = 96 / NSG;           // partials per thread loaded up front
    __shared__ float f[256];
    __shared__ float red[kWaves];
    __shared__ float4 acc_s[NSG][NJ4];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int bk = blockIdx.x / G, g = blockIdx.x % G;
    const int b = bk / a.hkv, kvh = bk - b * a.hkv;
    const int n_total = a.n_split;  // <= 256
    const float *ml = a.partial_ml + (int64_t)bk * n_total * G * 2;
    const float *po = a.partial + (int64_t)bk * n_total * G * D;
    const int j4 = tid % NJ4, sg = tid / NJ4;

    float4 pre[PF];
#pragma unroll
    for (int k = 0; k < PF; ++k) {
        const int sp = sg + k * NSG;
        pre[k] = sp < n_total ? *reinterpret_cast<const float4 *>(po + (int64_t)(sp * G + g) * D + 4 * j4)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float2 mlv = make_float2(-INFINITY, 0.f);
    if (tid < n_total) mlv = *reinterpret_cast<const float2 *>(ml + (tid * G + g) * 2);

    float m = mlv.x;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if (lane == 0) red[wv] = m;
    __syncthreads();
    float M = red[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, red[w]);
    __syncthreads();
    const float fw = (mlv.x == -INFINITY) ? 0.f : exp2f(mlv.x - M);
    if (tid < n_total) f[tid] = fw;
    float l = fw * mlv.y;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o);
    if (lane == 0) red[wv] = l;
    __syncthreads();
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) L += red[w];

    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < PF; ++k) {
        const int sp = sg + k * NSG;
        const float w = sp < n_total ? f[sp] : 0.f;
        acc.x = fmaf(w, pre[k].x, acc.x);
        acc.y = fmaf(w, pre[k].y, acc.y);
        acc.z = fmaf(w, pre[k].z, acc.z);
        acc.w = fmaf(w, pre[k].w, acc.w);
    }
    for (int sp = sg + PF * NSG; sp < n_total; sp += NSG) {
        const float4 v = *reinterpret_cast<const float4 *>(po + (int64_t)(sp * G + g) * D + 4 * j4);
        const float w = f[sp];
        acc.x = fmaf(w, v.x, acc.x);
        acc.y = fmaf(w, v.y, acc.y);
        acc.z = fmaf(w, v.z, acc.z);
        acc.w = fmaf(w, v.w, acc.w);
    }
    acc_s[sg][j4] = acc;
    __syncthreads();
    if (sg == 0) {
#pragma unroll
        for (int k = 1; k < NSG; ++k) {
            const float4 v = acc_s[k][j4];
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
        }
        const float inv = L > 0.f ? 1.f / L : 0.f;
        *reinterpret_cast<float4 *>(a.out + ((int64_t)b * a.hq + kvh * G + g) * D + 4 * j4) =
            make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    }
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
template <int D, int VB, int G>
static void launch_g(const DecodeArgs &a, hipStream_t st) {
    {
        if constexpr (D == 256)
            hipLaunchKernelGGL((k_decode_prep<D, G>), dim3((unsigned)(a.batch * a.hkv * PrepBand<D>::NB)),
                               dim3(kThreads), 0, st, a);
        const dim3 grid((unsigned)a.n_split, (unsigned)(a.batch * a.hkv));
        if constexpr (D == 128 && G <= 4) {
            if (a.waves == 12) hipLaunchKernelGGL((k_decode_main<D, VB, G, 12>), grid, dim3(64 * 12), 0, st, a);
            else hipLaunchKernelGGL((k_decode_main<D, VB, G, 4>), grid, dim3(64 * 4), 0, st, a);
        } else {
            hipLaunchKernelGGL((k_decode_main<D, VB, G, 4>), grid, dim3(64 * 4), 0, st, a);
        }
    }
    if (a.n_split > 1)
        hipLaunchKernelGGL((k_decode_merge<D, G>), dim3((unsigned)(a.batch * a.hkv * G)), dim3(kThreads), 0, st, a);
}

template <int D, int VB>
static hipError_t launch_main_dv(int G, const DecodeArgs &a, hipStream_t st) {
    switch (G) {
        case 1: launch_g<D, VB, 1>(a, st); break;
        case 2: launch_g<D, VB, 2>(a, st); break;
        case 4: launch_g<D, VB, 4>(a, st); break;
        default: launch_g<D, VB, 8>(a, st); break;
    }
    return hipGetLastError();
}

// the other key widths and head_dim 64: k_decode_prep for the queries, k_decode_any
// (tq_decode_any.hip) for the splits, the same merge; a fused step's new token is appended to
// the ring first
template <int D>
static hipError_t launch_any_d(int kb, int vb, int G, const DecodeArgs &a, hipStream_t st) {
    if (a.k_new && a.new_slot >= 0) {
        const hipError_t e = launch_ring_append(D, (tq_dtype)a.kv_dtype, a.k_new, a.v_new, a.rk, a.rv,
                                                a.batch * a.hkv, a.buffer_size, a.new_slot, st);
        if (e != hipSuccess) return e;
    }
    const dim3 pgrid((unsigned)(a.batch * a.hkv * PrepBand<D>::NB));
    switch (G) {
        case 1: hipLaunchKernelGGL((k_decode_prep<D, 1>), pgrid, dim3(kThreads), 0, st, a); break;
        case 2: hipLaunchKernelGGL((k_decode_prep<D, 2>), pgrid, dim3(kThreads), 0, st, a); break;
        case 4: hipLaunchKernelGGL((k_decode_prep<D, 4>), pgrid, dim3(kThreads), 0, st, a); break;
        default: hipLaunchKernelGGL((k_decode_prep<D, 8>), pgrid, dim3(kThreads), 0, st, a); break;
    }
    launch_decode_any_main(D, kb, vb, G, a, st);
    if (a.n_split > 1) {
        const dim3 mgrid((unsigned)(a.batch * a.hkv * G));
        switch (G) {
            case 1: hipLaunchKernelGGL((k_decode_merge<D, 1>), mgrid, dim3(kThreads), 0, st, a); break;
            case 2: hipLaunchKernelGGL((k_decode_merge<D, 2>), mgrid, dim3(kThreads), 0, st, a); break;
            case 4: hipLaunchKernelGGL((k_decode_merge<D, 4>), mgrid, dim3(kThreads), 0, st, a); break;
            default: hipLaunchKernelGGL((k_decode_merge<D, 8>), mgrid, dim3(kThreads), 0, st, a); break;
        }
    }
    return hipGetLastError();
}

bool decode_uses_any(int d, int kb) { return kb != 3 || d == 64; }

hipError_t launch_decode(int d, int kb, int vb, int G, const DecodeArgs &a, hipStream_t st) {
    if (decode_uses_any(d, kb)) return d == 64 ? launch_any_d<64>(kb, vb, G, a, st) : launch_any_d<128>(kb, vb, G, a, st);
    if (d == 128 && vb == 2) return launch_main_dv<128, 2>(G, a, st);
    if (d == 128 && vb == 4) return launch_main_dv<128, 4>(G, a, st);
    if (d == 256 && vb == 2) return launch_main_dv<256, 2>(G, a, st);
    return launch_main_dv<256, 4>(G, a, st);
}

template <int D>
hipError_t launch_merge_d(int G, const DecodeArgs &a, hipStream_t st) {
    const dim3 mgrid((unsigned)(a.batch * a.hkv * G));
    switch (G) {
        case 1: hipLaunchKernelGGL((k_decode_merge<D, 1>), mgrid, dim3(kThreads), 0, st, a); break;
        case 2: hipLaunchKernelGGL((k_decode_merge<D, 2>), mgrid, dim3(kThreads), 0, st, a); break;
        case 4: hipLaunchKernelGGL((k_decode_merge<D, 4>), mgrid, dim3(kThreads), 0, st, a); break;
        default: hipLaunchKernelGGL((k_decode_merge<D, 8>), mgrid, dim3(kThreads), 0, st, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_decode_merge(int d, int G, const DecodeArgs &a, hipStream_t st) {
    if (d == 64) return launch_merge_d<64>(G, a, st);
    if (d == 128) return launch_merge_d<128>(G, a, st);
    return launch_merge_d<256>(G, a, st);
}

hipError_t launch_ring_append(int d, tq_dtype dt, const void *kn, const void *vn, uint16_t *rk, uint16_t *rv,
                              int n_slices, int buffer_size, int slot, hipStream_t st) {
    const int64_t total = (int64_t)n_slices * d / 8;
    const unsigned grid = (unsigned)((total + 255) / 256);
#define TQ_RING(TAG, DD) hipLaunchKernelGGL((k_ring_append<TAG, DD>), dim3(grid), dim3(256), 0, st, kn, vn, rk, rv, \
                                            n_slices, buffer_size, slot)
    if (d == 64) {
        if (dt == TQ_F32) TQ_RING(f32_tag, 64);
        else if (dt == TQ_BF16) TQ_RING(bf16_tag, 64);
        else TQ_RING(f16_tag, 64);
    } else if (d == 128) {
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

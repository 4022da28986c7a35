// tq_decode_any.hip -- decode attention over packed records of every key width (1 to 4
// codebook bits, two-plane or nibble records) at head_dim 64 and 128: the path of the
// configurations the matrix-core decode (tq_decode.hip, 3-bit nibble records at head_dim
// 128 and 256) does not cover.
//
// Method: hotelren.com guide "企业官网建设流程全解析", section 二 (the estimate
//   s_t = |k_t| ( <q', c[idx_t]> + gamma_t sqrt(pi/2)/d <w, 2 z_t - 1> ),  q' = Pi q,
//   w = S q') and section 5.1 item 2 (the ring's exact fp16 tokens), softmax over both, values
// dequantised to the bin centres.  Same split-K scheme and partial layout as the matrix-core
// decode, so k_decode_merge combines the splits of either.
//
// k_decode_any: one 4-wave workgroup per (split, slice).  The split's tokens go in 64-token
// chunks to the waves in turn (packed chunks, then the ring chunk).  Per chunk:
//   * scores, one lane per token: the lane reads its token's key record and norms and sums
//     G heads over the d coordinates in fp32 (the codebook value from an LDS table, q' and w
//     as scalar operands; sum_j w_j (2 z_j - 1) taken as 2 sum_{z_j = 1} w_j - sum_j w_j);
//   * online softmax per head across the wave's chunks (chunk maximum by lane shuffles);
//   * values, one lane per coordinate (d / 64 each): p of every token of the chunk and its
//     value record come from LDS (the lane of the token wrote them), fp32 accumulation.
// The waves' (m, l, o) are combined through LDS at the end.  The query preparation (q' and
// w = S q' for the G heads of the slice) is k_decode_prep's, read from the workspace.
#include <hip/hip_runtime.h>

#include "tq.h"
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kAnyThreads = 256;
constexpr int kAnyWaves = kAnyThreads / 64;
constexpr int kChunk = 64;  // tokens per wave chunk
constexpr float kAnyLog2e = 1.4426950408889634f;

template <int D, int KB, int VB, int G>
struct AnyShape {
    static constexpr int KW = (KB + 1) * D / 32;  // key record words
    static constexpr int NCW = KB * D / 32;       // code-plane words (KB != 3)
    static constexpr int VW = VB * D / 32;        // value record words
    static constexpr int NG = D / 32;             // value groups (fp16 scales)
    static constexpr int EPL = D / 64;            // value coordinates per lane
    static constexpr int HALF = 1 << (VB - 1);
    static_assert(KW % 2 == 0 && (D == 64 || D == 128), "record shapes");
};

template <int D, int KB, int VB, int G>
struct alignas(16) AnySmem {
    using S = AnyShape<D, KB, VB, G>;
    float qr[G][D];  // scale log2(e) * q (the ring's exact scores)
    float ctab[16];  // stored centroids
    float wsum[G];   // sum_j w[g][j]
    float pb[kAnyWaves][kChunk][G];  // p of the chunk's tokens (ring chunks)
    union alignas(16) {
        struct {
            // the chunk's value records, word-major (rows padded by 4 words: the rows one
            // 16-byte read reaches fall in different banks), and p times the token's group
            // scale per head and group
            uint32_t vrec[kAnyWaves][S::VW][kChunk + 4];
            float psc[kAnyWaves][G][S::NG][kChunk];
        } c;
        float wo[kAnyWaves][G][D];  // wave combine
    };
    float wm[kAnyWaves][G], wl[kAnyWaves][G];
};

// codebook index and sign bit of coordinate j of a key record (layouts of include/tq.h)
template <int D, int KB>
__device__ __forceinline__ void key_field(const uint32_t (&kw)[(KB + 1) * D / 32], int j, uint32_t &idx,
                                          uint32_t &z) {
    if constexpr (KB == 3) {
        const uint32_t nib = (kw[j / 8] >> (4 * (j % 8))) & 15u;
        idx = nib & 7u;
        z = nib >> 3;
    } else {
        constexpr int PER = 32 / KB;
        idx = (kw[j / PER] >> (KB * (j % PER))) & ((1u << KB) - 1u);
        z = (kw[KB * D / 32 + j / 32] >> (j % 32)) & 1u;
    }
}

// element `off` of q in its storage dtype, as fp32
__device__ __forceinline__ float load_q_elem(const DecodeArgs &a, int64_t off) {
    if (a.q_dtype == TQ_F32) return load1(a.q, off, f32_tag{});
    if (a.q_dtype == TQ_BF16) return load1(a.q, off, bf16_tag{});
    return load1(a.q, off, f16_tag{});
}

template <int D, int KB, int VB, int G>
__global__ __launch_bounds__(kAnyThreads)
__attribute__((amdgpu_waves_per_eu(G <= 4 ? 4 : 2, G <= 4 ? 4 : 2)))
void k_decode_any(DecodeArgs a) {
    using S = AnyShape<D, KB, VB, G>;
    __shared__ AnySmem<D, KB, VB, G> sm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int split = blockIdx.x, bk = blockIdx.y;
    const int b = bk / a.hkv, kvh = bk - b * a.hkv;

    // this sequence's lengths and the split's token ranges (as in the matrix-core decode)
    int n_packed = (int)a.n_packed, n_ring = a.n_ring;
    int sbk = bk;  // store slice (prefill: the sequence's, shared by its query tokens)
    if (a.seq_packed) n_packed = (int)min(max(a.seq_packed[b], (int64_t)0), a.n_packed);
    if (a.seq_ring) n_ring = min(max(a.seq_ring[b], 0), a.n_ring);
    if (a.q_tokens) {
        const int seq = b / a.q_tokens, qi = b - seq * a.q_tokens;
        sbk = (int)(a.q_slice0 + seq * a.hkv + kvh);
        if (a.causal) n_packed = (int)max((int64_t)0, min((int64_t)n_packed, a.q_pos0 + qi + 1));
    }
    int per_split = (int)a.per_split, ring_per_split = a.ring_per_split;
    if (a.seq_packed || (a.q_tokens && a.causal)) per_split = ((n_packed + a.n_split - 1) / a.n_split + 31) / 32 * 32;
    if (a.seq_ring) ring_per_split = (n_ring + a.n_split - 1) / a.n_split;
    const int t_begin = split * per_split;
    const int t_end = max(t_begin, min(n_packed, t_begin + per_split));
    const int r0 = split * ring_per_split, nr = max(0, min(n_ring - r0, ring_per_split));

    // prepared queries of the slice (q' [G][D], then w [G][D]): the same values in every lane,
    // read through the scalar unit (constant address space: the kernel never writes them);
    // the log2-domain scales are applied to the sums
    const float cs = a.scale * kAnyLog2e * rsqrtf((float)D);
    const float ss = cs * (1.2533141373155003f / (float)D);  // sqrt(pi/2) / d
    typedef const __attribute__((address_space(4))) float cfloat;
    cfloat *prep = (cfloat *)(a.prep + (int64_t)bk * 2 * G * D);
    const float lscale = a.scale * kAnyLog2e;
    const int64_t qoff = ((int64_t)b * a.hq + kvh * G) * D;
    for (int i = tid; i < G * D; i += kAnyThreads) (&sm.qr[0][0])[i] = lscale * load_q_elem(a, qoff + i);
    if (tid < (1 << KB)) sm.ctab[tid] = a.centroids[tid];
    if (tid < G) {
        float sw = 0.f;
        for (int j = 0; j < D; ++j) sw += prep[G * D + tid * D + j];
        sm.wsum[tid] = sw;
    }
    __syncthreads();

    float M[G], Lw[G], o[G][S::EPL];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        M[h] = -INFINITY;
        Lw[h] = 0.f;
#pragma unroll
        for (int e = 0; e < S::EPL; ++e) o[h][e] = 0.f;
    }

    const int n_pc = (t_end - t_begin + kChunk - 1) / kChunk;  // packed chunks
    const int n_rc = (nr + kChunk - 1) / kChunk;               // ring chunks
    for (int ch = wave; ch < n_pc + n_rc; ch += kAnyWaves) {
        const bool ring = ch >= n_pc;
        const int c0 = ring ? r0 + (ch - n_pc) * kChunk : t_begin + ch * kChunk;
        const int cn = ring ? min(kChunk, r0 + nr - c0) : min(kChunk, t_end - c0);
        const bool valid = lane < cn;
        const int tt = c0 + (valid ? lane : cn - 1);  // clamped: every lane reads a real token
        float s[G];
#pragma unroll
        for (int h = 0; h < G; ++h) s[h] = 0.f;
        float vsc[S::NG] = {};  // packed chunks: the lane's token's value group scales
        if (!ring) {
            // ---- scores of a packed token (one per lane)
            const int64_t rec = record_index(a.bt, a.pt, a.pps, a.n_pages, a.cap, a.err, sbk, tt);
            uint32_t kw[S::KW];
            const uint2 *kp = reinterpret_cast<const uint2 *>(a.kw + rec * S::KW);
#pragma unroll
            for (int i = 0; i < S::KW / 2; ++i) {
                const uint2 x = kp[i];
                kw[2 * i] = x.x;
                kw[2 * i + 1] = x.y;
            }
            const float2 kn = *reinterpret_cast<const float2 *>(a.kn + rec * 2);
            float mse[G], sgn[G];
#pragma unroll
            for (int h = 0; h < G; ++h) mse[h] = sgn[h] = 0.f;
#pragma unroll
            for (int j = 0; j < D; ++j) {
                uint32_t idx, z;
                key_field<D, KB>(kw, j, idx, z);
                const float c = sm.ctab[idx];
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    mse[h] = fmaf(prep[h * D + j], c, mse[h]);
                    sgn[h] = fmaf((float)z, prep[G * D + h * D + j], sgn[h]);  // sum of w over the set sign bits
                }
            }
#pragma unroll
            for (int h = 0; h < G; ++h)
                s[h] = kn.x * fmaf(ss * kn.y, fmaf(2.f, sgn[h], -sm.wsum[h]), cs * mse[h]);
            // the token's value record for the value phase; its group scales for the p products
            const uint32_t *vp = a.vw + rec * S::VW;
#pragma unroll
            for (int i = 0; i < S::VW; ++i) sm.c.vrec[wave][i][lane] = vp[i];
#pragma unroll
            for (int i = 0; i < S::NG; ++i) vsc[i] = f16_lo(a.vs[rec * S::NG + i]);
        } else {
            // ---- scores of a ring token: q . k over its exact fp16 key
            const uint16_t *kr = a.rk + ((int64_t)bk * a.buffer_size + tt) * D;
#pragma unroll 4
            for (int j = 0; j < D; j += 8) {
                const uint4 x = *reinterpret_cast<const uint4 *>(kr + j);
                const float k8[8] = {f16_lo(x.x), f16_hi(x.x), f16_lo(x.y), f16_hi(x.y),
                                     f16_lo(x.z), f16_hi(x.z), f16_lo(x.w), f16_hi(x.w)};
#pragma unroll
                for (int h = 0; h < G; ++h)
#pragma unroll
                    for (int e = 0; e < 8; ++e) s[h] = fmaf(sm.qr[h][j + e], k8[e], s[h]);
            }
        }
        // ---- online softmax over the wave's chunks
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float cm = valid ? s[h] : -INFINITY;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) cm = fmaxf(cm, __shfl_xor(cm, off));
            const float mn = fmaxf(M[h], cm);
            const float alpha = M[h] == -INFINITY ? 0.f : exp2f(M[h] - mn);
            M[h] = mn;
            const float p = valid ? exp2f(s[h] - mn) : 0.f;
            float ps = p;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) ps += __shfl_xor(ps, off);
            Lw[h] = fmaf(Lw[h], alpha, ps);
#pragma unroll
            for (int e = 0; e < S::EPL; ++e) o[h][e] *= alpha;
            if (ring) {
                sm.pb[wave][lane][h] = p;
            } else {
                // v = (code - HALF + 1/2) s: sum_t p_t s_t code_t over the chunk below, and the
                // offset -(HALF - 1/2) sum_t p_t s_t of each group, the same for its coordinates
#pragma unroll
                for (int i = 0; i < S::NG; ++i) {
                    const float q = p * vsc[i];
                    sm.c.psc[wave][h][i][lane] = q;
                    float r = q;
#pragma unroll
                    for (int off = 32; off > 0; off >>= 1) r += __shfl_xor(r, off);
#pragma unroll
                    for (int e = 0; e < S::EPL; ++e)
                        if ((lane + 64 * e) / 32 == i) o[h][e] = fmaf(-((float)S::HALF - 0.5f), r, o[h][e]);
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        // ---- values: lane holds coordinates lane + 64 e
        if (!ring) {
            // four tokens per pass (tokens past cn have p = 0): their code words of the lane's
            // coordinates and their p s of every head as 16-byte reads
            for (int t4 = 0; t4 < cn; t4 += 4) {
#pragma unroll
                for (int e = 0; e < S::EPL; ++e) {
                    const int j = lane + 64 * e;
                    const uint4 wd = *reinterpret_cast<const uint4 *>(&sm.c.vrec[wave][j / (32 / VB)][t4]);
                    const uint32_t sh = VB * (j % (32 / VB)), msk = (1u << VB) - 1u;
                    const float c0f = (float)((wd.x >> sh) & msk), c1f = (float)((wd.y >> sh) & msk);
                    const float c2f = (float)((wd.z >> sh) & msk), c3f = (float)((wd.w >> sh) & msk);
#pragma unroll
                    for (int h = 0; h < G; ++h) {
                        const float4 q = *reinterpret_cast<const float4 *>(&sm.c.psc[wave][h][j / 32][t4]);
                        float x = o[h][e];
                        x = fmaf(q.x, c0f, x);
                        x = fmaf(q.y, c1f, x);
                        x = fmaf(q.z, c2f, x);
                        x = fmaf(q.w, c3f, x);
                        o[h][e] = x;
                    }
                }
            }
        } else {
            for (int t = 0; t < cn; ++t) {
                float p[G];
#pragma unroll
                for (int h = 0; h < G; ++h) p[h] = sm.pb[wave][t][h];
#pragma unroll
                for (int e = 0; e < S::EPL; ++e) {
                    const float v = f16_lo(a.rv[((int64_t)bk * a.buffer_size + c0 + t) * D + lane + 64 * e]);
#pragma unroll
                    for (int h = 0; h < G; ++h) o[h][e] = fmaf(p[h], v, o[h][e]);
                }
            }
        }
        // the chunk's LDS rows are rewritten by the wave's next chunk only after every lane
        // has read them
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }

    // ---- combine the waves: (m, l) per head, o per head and coordinate
    __syncthreads();  // every wave is done with the chunk buffers (aliased by wo)
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int e = 0; e < S::EPL; ++e) sm.wo[wave][h][lane + 64 * e] = o[h][e];
        if (lane == 0) {
            sm.wm[wave][h] = M[h];
            sm.wl[wave][h] = Lw[h];
        }
    }
    __syncthreads();
    float *pp = a.partial + ((int64_t)bk * a.n_split + split) * G * D;
    float *pml = a.partial_ml + ((int64_t)bk * a.n_split + split) * G * 2;
    for (int i = tid; i < G * D; i += kAnyThreads) {
        const int h = i / D, j = i - h * D;
        float Mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < kAnyWaves; ++w) Mx = fmaxf(Mx, sm.wm[w][h]);
        float Lt = 0.f, Ot = 0.f;
        if (Mx != -INFINITY) {
#pragma unroll
            for (int w = 0; w < kAnyWaves; ++w) {
                if (sm.wm[w][h] == -INFINITY) continue;
                const float f = exp2f(sm.wm[w][h] - Mx);
                Lt = fmaf(sm.wl[w][h], f, Lt);
                Ot = fmaf(sm.wo[w][h][j], f, Ot);
            }
        }
        if (a.n_split == 1) {
            a.out[((int64_t)b * a.hq + kvh * G + h) * D + j] = Lt > 0.f ? Ot / Lt : 0.f;
        } else {
            pp[h * D + j] = Ot;
            if (j == 0) {
                pml[h * 2] = Mx;
                pml[h * 2 + 1] = Lt;
            }
        }
    }
}

template <int D, int KB, int VB>
void launch_any_g(int G, const DecodeArgs &a, hipStream_t st) {
    const dim3 grid((unsigned)a.n_split, (unsigned)(a.batch * a.hkv));
    switch (G) {
        case 1: hipLaunchKernelGGL((k_decode_any<D, KB, VB, 1>), grid, dim3(kAnyThreads), 0, st, a); break;
        case 2: hipLaunchKernelGGL((k_decode_any<D, KB, VB, 2>), grid, dim3(kAnyThreads), 0, st, a); break;
        case 4: hipLaunchKernelGGL((k_decode_any<D, KB, VB, 4>), grid, dim3(kAnyThreads), 0, st, a); break;
        default: hipLaunchKernelGGL((k_decode_any<D, KB, VB, 8>), grid, dim3(kAnyThreads), 0, st, a); break;
    }
}

template <int D, int VB>
void launch_any_kb(int kb, int G, const DecodeArgs &a, hipStream_t st) {
    switch (kb) {
        case 1: launch_any_g<D, 1, VB>(G, a, st); break;
        case 2: launch_any_g<D, 2, VB>(G, a, st); break;
        case 3: launch_any_g<D, 3, VB>(G, a, st); break;
        default: launch_any_g<D, 4, VB>(G, a, st); break;
    }
}

}  // namespace

void launch_decode_any_main(int d, int kb, int vb, int G, const DecodeArgs &a, hipStream_t st) {
    if (d == 64) {
        if (vb == 2) launch_any_kb<64, 2>(kb, G, a, st);
        else launch_any_kb<64, 4>(kb, G, a, st);
    } else {
        if (vb == 2) launch_any_kb<128, 2>(kb, G, a, st);
        else launch_any_kb<128, 4>(kb, G, a, st);
    }
}

}  // namespace tq

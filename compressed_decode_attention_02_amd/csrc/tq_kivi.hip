// tq_kivi.hip -- the KIVI 2-bit asymmetric variant (forum page zingnex.cn "TurboQuant-vLLM：
// 大模型推理的KV缓存量化实战方案", section "KIVI非对称量化"): keys quantised per channel, values
// per token, each set with a scale and a zero point, at 2 bits; and decode attention over such
// a store.
//
// Format (per slice): key and value codes 2 bits each, channel c at bits 2 (c % 16) of word
// c / 16 of the token's record; key scale and zero (binary16) per 32-token group and channel;
// value scale and zero (binary16) per token.  scale = binary16(fp32(fp32(max - min) / 3)),
// zero = binary16(min), code = clamp(rint(fp32(x - zero) / scale), 0, 3) (IEEE binary32
// division), 0 where the scale is 0.
//
// Launches:
//   * k_kivi_quant, one workgroup per (slice, 32-token group): keys per channel (a channel's
//     tokens split over 256 / D threads), values per token (8 threads per token);
//   * k_kivi_decode, grid (splits, slices), 4 waves, each wave in turn a chunk of 64 tokens
//     (two key groups): the scaled query a = scale log2e q * s per group and channel and the
//     group's constant b = scale log2e q . z into LDS, logits with lane = token from the
//     token's code words, a lazily rescaled online softmax per head, values with lane =
//     channel pair from the chunk's value code words in LDS; the waves' (m, l, o) combined
//     into the split's partials, then the decode merge launch (or the output with one split).
#include <hip/hip_runtime.h>

#include "tq.h"
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

namespace {

constexpr int kKThreads = 256;
constexpr int kGroup = 32;
constexpr float kLog2eK = 1.4426950408889634f;

__device__ __forceinline__ void kwave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename Tag> struct TagBytes { typedef float type; };
template <> struct TagBytes<bf16_tag> { typedef uint16_t type; };
template <> struct TagBytes<f16_tag> { typedef uint16_t type; };

template <typename Tag>
__device__ __forceinline__ float in_elem(const void *p, int64_t off) {
    return load1(p, off, Tag{});
}

// scale and zero of a set with minimum mn and maximum mx (binary16 bits)
__device__ __forceinline__ void kivi_params(float mn, float mx, uint16_t &sb, uint16_t &zb) {
    const float span = mx - mn;
    const float s = span / 3.0f;  // IEEE division (correctly rounded)
    sb = f32_to_f16_bits(s);
    zb = f32_to_f16_bits(mn);
}
__device__ __forceinline__ uint32_t kivi_code(float x, float s, float z) {
    if (s == 0.f) return 0u;
    const float qv = rintf((x - z) / s);
    return (uint32_t)fminf(fmaxf(qv, 0.f), 3.f);
}

template <typename Tag, int D>
__global__ __launch_bounds__(kKThreads) void k_kivi_quant(const void *k, const void *v, int64_t n_tokens,
                                                           int64_t n_groups, tq_kivi_store dst, int64_t dst_token0) {
    constexpr int TPC = kKThreads / D;      // threads per key channel
    constexpr int TPT = kGroup / TPC;       // tokens per thread (keys)
    constexpr int W = D / 16;               // code words per token
    constexpr int VPT = kKThreads / kGroup;  // threads per value token (8)
    constexpr int VE = D / VPT;             // value entries per thread
    static_assert(VE == 8 || VE == 16 || VE == 32, "value entries per thread");
    constexpr int IB = sizeof(typename TagBytes<Tag>::type);  // input bytes per element
    __shared__ float red[2][kKThreads];
    __shared__ __align__(16) uint8_t kc[kGroup][D];
    __shared__ __align__(16) uint4 kt[kGroup * D * IB / 16];  // the group's keys (16-byte loads)
    const int tid = threadIdx.x;
    const int64_t sl = blockIdx.x / n_groups, grp = blockIdx.x % n_groups;
    const int64_t t0 = grp * kGroup;                        // first token of the group (input)
    const int64_t r0 = dst_token0 + t0;                     // its record index in the slice
    const int64_t in0 = (sl * n_tokens + t0) * D;           // element offset of the group's first token

    // ---- keys: the group's tile into LDS with 16-byte loads, then channel c = tid % D,
    //      tokens h TPT .. h TPT + TPT - 1 (h = tid / D)
    {
        const uint4 *ksrc = reinterpret_cast<const uint4 *>(static_cast<const unsigned char *>(k) + in0 * IB);
#pragma unroll
        for (int i = tid; i < kGroup * D * IB / 16; i += kKThreads) kt[i] = ksrc[i];
        __syncthreads();
        const int c = tid % D, h = tid / D;
        float x[TPT];
        float mn = INFINITY, mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
            x[i] = in_elem<Tag>(kt, (int64_t)(h * TPT + i) * D + c);
            mn = fminf(mn, x[i]);
            mx = fmaxf(mx, x[i]);
        }
        red[0][tid] = mn;
        red[1][tid] = mx;
        __syncthreads();
#pragma unroll
        for (int o = 1; o < TPC; ++o) {
            mn = fminf(mn, red[0][(h ^ o) * D + c]);
            mx = fmaxf(mx, red[1][(h ^ o) * D + c]);
        }
        uint16_t sb, zb;
        kivi_params(mn, mx, sb, zb);
        const float s = (float)__builtin_bit_cast(_Float16, sb), z = (float)__builtin_bit_cast(_Float16, zb);
        if (h == 0) {
            const int64_t pg = (sl * (dst.capacity / kGroup) + r0 / kGroup) * D + c;
            dst.key_scale[pg] = sb;
            dst.key_zero[pg] = zb;
        }
#pragma unroll
        for (int i = 0; i < TPT; ++i) kc[h * TPT + i][c] = (uint8_t)kivi_code(x[i], s, z);
        __syncthreads();
        // pack: thread (token t, word w) for t < 32, w < W
        for (int e = tid; e < kGroup * W; e += kKThreads) {
            const int t = e / W, w = e % W;
            const uint4 b = *reinterpret_cast<const uint4 *>(&kc[t][16 * w]);  // 16 codes, one per byte
            const uint32_t bb[4] = {b.x, b.y, b.z, b.w};
            uint32_t word = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // bytes (c0, c1, c2, c3) of bb[j] -> 8 bits c0 | c1 << 2 | c2 << 4 | c3 << 6
                const uint32_t y = bb[j];
                const uint32_t packed = (y & 3u) | ((y >> 6) & 0xCu) | ((y >> 12) & 0x30u) | ((y >> 18) & 0xC0u);
                word |= packed << (8 * j);
            }
            dst.key_codes[(sl * dst.capacity + r0 + t) * W + w] = word;
        }
    }

    // ---- values: token t = tid / VPT, entries part VE .. part VE + VE - 1 (part = tid % VPT)
    {
        const int t = tid / VPT, part = tid % VPT;
        float x[VE];
        float mn = INFINITY, mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < VE; i += 8) {
            float f[8];
            load8(v, in0 + (int64_t)t * D + part * VE + i, f, Tag{});
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                x[i + e] = f[e];
                mn = fminf(mn, f[e]);
                mx = fmaxf(mx, f[e]);
            }
        }
#pragma unroll
        for (int o = 1; o < VPT; o <<= 1) {
            mn = fminf(mn, __shfl_xor(mn, o));
            mx = fmaxf(mx, __shfl_xor(mx, o));
        }
        uint16_t sb, zb;
        kivi_params(mn, mx, sb, zb);
        const float s = (float)__builtin_bit_cast(_Float16, sb), z = (float)__builtin_bit_cast(_Float16, zb);
        const int64_t rec = sl * dst.capacity + r0 + t;
        if (part == 0) *reinterpret_cast<uint32_t *>(dst.val_params + rec * 2) = (uint32_t)sb | ((uint32_t)zb << 16);
        // VE codes -> VE / 16 words (VE = 8: half a word, merged with the neighbour lane)
        if constexpr (VE >= 16) {
#pragma unroll
            for (int w = 0; w < VE / 16; ++w) {
                uint32_t word = 0;
#pragma unroll
                for (int e = 0; e < 16; ++e) word |= kivi_code(x[16 * w + e], s, z) << (2 * e);
                dst.val_codes[rec * W + part * (VE / 16) + w] = word;
            }
        } else {
            uint32_t half = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) half |= kivi_code(x[e], s, z) << (2 * e + 16 * (part & 1));
            const uint32_t word = half | (uint32_t)__shfl_xor((int)half, 1);
            if ((part & 1) == 0) dst.val_codes[rec * W + part / 2] = word;
        }
    }
}

// ------------------------------------------------------------------ decode
constexpr int kChunk = 64;  // tokens per wave iteration (one per lane; two key groups)

template <int D, int G>
struct alignas(16) KivDecodeSmem {
    float a[4][2][G][D];          // per wave: scaled query per (group of the chunk, head, channel)
    float bq[4][2][G];            // per wave: group constants
    // per wave: the chunk's value code words, word-major (rows padded by 4 words: the four
    // rows one read reaches fall in different banks)
    uint32_t vcw[4][D / 16][kChunk + 4];
    float pv[4][G][kChunk];       // per wave: p scale per head and token
    float wm[4][G], wl[4][G];
    float wo[4][G][D];
};

// waves per SIMD the decode is compiled for: four (<= 128 VGPRs) where a lane's heads and
// channels allow it, so that the chunks' loads of more waves overlap; fewer as they grow (d = 256
// with eight heads: one, as its LDS allows one workgroup per CU)
template <int D, int G>
constexpr int kKivDecWaves = D * G <= 256 || (D * G <= 512 && D <= 128) ? 4 : (D * G <= 512 ? 3 : (D * G < 2048 ? 2 : 1));

template <int D, int G>
__global__ __launch_bounds__(kKThreads)
__attribute__((amdgpu_waves_per_eu(kKivDecWaves<D, G>, kKivDecWaves<D, G>)))
void k_kivi_decode(DecodeArgs a, tq_kivi_store src) {
    constexpr int W = D / 16;
    constexpr int CPL = D / 64;  // value channels per lane
    __shared__ KivDecodeSmem<D, G> sm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int split = blockIdx.x, bk = blockIdx.y;
    const int b = bk / a.hkv, kvh = bk - b * a.hkv;
    const int n_packed = (int)a.n_packed;
    const int t_begin = split * (int)a.per_split;
    const int t_end = max(t_begin, min(n_packed, t_begin + (int)a.per_split));
    const float lscale = a.scale * kLog2eK;
    // the lane's query coordinates (channels lane + 64 e) of every head
    float qv[G][CPL];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
            const int64_t off = ((int64_t)b * a.hq + kvh * G + g) * D + lane + 64 * e;
            qv[g][e] = a.q_dtype == TQ_F32 ? load1(a.q, off, f32_tag{})
                     : (a.q_dtype == TQ_BF16 ? load1(a.q, off, bf16_tag{}) : load1(a.q, off, f16_tag{}));
        }
    float m[G], l[G];
    float oacc[G][CPL];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < CPL; ++e) oacc[g][e] = 0.f;
    }
    const int64_t ngp = src.capacity / 32;
    for (int c0 = t_begin + wave * kChunk; c0 < t_end; c0 += 4 * kChunk) {
        // ---- a and b of the chunk's two groups (lane = channels lane + 64 e)
#pragma unroll
        for (int gi = 0; gi < 2; ++gi) {
            const int64_t grp = min((int64_t)(c0 / 32 + gi), ngp - 1);
            const int64_t pg = ((int64_t)bk * ngp + grp) * D;
            float bs[G];
#pragma unroll
            for (int g = 0; g < G; ++g) bs[g] = 0.f;
#pragma unroll
            for (int e = 0; e < CPL; ++e) {
                const int c = lane + 64 * e;
                const float s = (float)__builtin_bit_cast(_Float16, src.key_scale[pg + c]);
                const float z = (float)__builtin_bit_cast(_Float16, src.key_zero[pg + c]);
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    sm.a[wave][gi][g][c] = lscale * qv[g][e] * s;
                    bs[g] = fmaf(qv[g][e], z, bs[g]);
                }
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float x = bs[g];
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
                if (lane == 0) sm.bq[wave][gi][g] = lscale * x;
            }
        }
        // ---- the lane's token: its key code words; its value code words into LDS
        const int t = c0 + lane;
        const bool live = t < t_end;
        const int tc = min(t, n_packed - 1);
        const int64_t rec = (int64_t)bk * src.capacity + tc;
        uint32_t kw[W];
#pragma unroll
        for (int w = 0; w < W; w += 4) {
            const uint4 u = *reinterpret_cast<const uint4 *>(src.key_codes + rec * W + w);
            kw[w] = u.x; kw[w + 1] = u.y; kw[w + 2] = u.z; kw[w + 3] = u.w;
        }
#pragma unroll
        for (int w = 0; w < W; w += 4) {
            const uint4 u = *reinterpret_cast<const uint4 *>(src.val_codes + rec * W + w);
            sm.vcw[wave][w][lane] = u.x;
            sm.vcw[wave][w + 1][lane] = u.y;
            sm.vcw[wave][w + 2][lane] = u.z;
            sm.vcw[wave][w + 3][lane] = u.w;
        }
        const uint32_t vp = *reinterpret_cast<const uint32_t *>(src.val_params + rec * 2);
        const float vs = f16_lo(vp), vz = f16_hi(vp);
        kwave_sync();  // a, b and the value code words visible to the wave
        // ---- logits (log2 units) of the lane's token for every head
        const int gi = lane >> 5;  // the token's group within the chunk (c0 is a multiple of 64)
        float s[G];
#pragma unroll
        for (int g = 0; g < G; ++g) s[g] = sm.bq[wave][gi][g];
#pragma unroll
        for (int w = 0; w < W; ++w) {
#pragma unroll
            for (int j = 0; j < 16; j += 4) {
                float cf[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) cf[u] = (float)((kw[w] >> (2 * (j + u))) & 3u);
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const float4 av = *reinterpret_cast<const float4 *>(&sm.a[wave][gi][g][16 * w + j]);
                    s[g] = fmaf(av.x, cf[0], s[g]);
                    s[g] = fmaf(av.y, cf[1], s[g]);
                    s[g] = fmaf(av.z, cf[2], s[g]);
                    s[g] = fmaf(av.w, cf[3], s[g]);
                }
            }
        }
        // ---- online softmax per head (reference max raised when a logit exceeds it)
        float zsum[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float x = live ? s[g] : -INFINITY;
            float mx = x;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
            const float mnew = fmaxf(m[g], mx);
            const float corr = m[g] == -INFINITY ? 0.f : exp2f(m[g] - mnew);
            m[g] = mnew;
            const float p = live ? exp2f(x - mnew) : 0.f;
            float ps = p;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) ps += __shfl_xor(ps, off);
            l[g] = l[g] * corr + ps;
#pragma unroll
            for (int e = 0; e < CPL; ++e) oacc[g][e] *= corr;
            sm.pv[wave][g][lane] = p * vs;
            // the zero points' share, sum over the chunk of p zero: the same for every channel
            float pz = p * vz;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) pz += __shfl_xor(pz, off);
            zsum[g] = pz;
        }
        kwave_sync();
        // ---- values: lane = channels lane + 64 e; sum over the chunk's tokens
        // (four tokens per pass: their code words of the lane's channels and their p scale of
        // every head as 16-byte reads)
        for (int t4 = 0; t4 < kChunk; t4 += 4) {
            float4 pw[G];
#pragma unroll
            for (int g = 0; g < G; ++g) pw[g] = *reinterpret_cast<const float4 *>(&sm.pv[wave][g][t4]);
#pragma unroll
            for (int e = 0; e < CPL; ++e) {
                const int c = lane + 64 * e;
                const uint4 cw = *reinterpret_cast<const uint4 *>(&sm.vcw[wave][c >> 4][t4]);
                const uint32_t sh = 2 * (c & 15);
                const float c0 = (float)((cw.x >> sh) & 3u), c1 = (float)((cw.y >> sh) & 3u);
                const float c2 = (float)((cw.z >> sh) & 3u), c3 = (float)((cw.w >> sh) & 3u);
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    float o = oacc[g][e];
                    o = fmaf(pw[g].x, c0, o);
                    o = fmaf(pw[g].y, c1, o);
                    o = fmaf(pw[g].z, c2, o);
                    o = fmaf(pw[g].w, c3, o);
                    oacc[g][e] = o;
                }
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < CPL; ++e) oacc[g][e] += zsum[g];
        kwave_sync();  // every lane is done with the chunk's LDS before the next chunk
    }
    // ---- the waves' (m, l, o) combined
#pragma unroll
    for (int g = 0; g < G; ++g) {
        if (lane == 0) {
            sm.wm[wave][g] = m[g];
            sm.wl[wave][g] = l[g];
        }
#pragma unroll
        for (int e = 0; e < CPL; ++e) sm.wo[wave][g][lane + 64 * e] = oacc[g][e];
    }
    __syncthreads();
    float *pp = a.partial + ((int64_t)bk * a.n_split + split) * G * D;
    float *pml = a.partial_ml + ((int64_t)bk * a.n_split + split) * G * 2;
    for (int i = tid; i < G * D; i += kKThreads) {
        const int g = i / D, j = i % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, sm.wm[w][g]);
        float L = 0.f, O = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                if (sm.wm[w][g] == -INFINITY) continue;
                const float f = exp2f(sm.wm[w][g] - M);
                L = fmaf(sm.wl[w][g], f, L);
                O = fmaf(sm.wo[w][g][j], f, O);
            }
        }
        if (a.n_split == 1) {
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

template <typename Tag>
hipError_t launch_quant_t(int d, const void *k, const void *v, int64_t n_slices, int64_t n_tokens,
                          const tq_kivi_store &dst, int64_t dst_token0, hipStream_t st) {
    const int64_t ng = n_tokens / kGroup;
    const dim3 grid((unsigned)(n_slices * ng));
    switch (d) {
        case 64: hipLaunchKernelGGL((k_kivi_quant<Tag, 64>), grid, dim3(kKThreads), 0, st, k, v, n_tokens, ng, dst, dst_token0); break;
        case 128: hipLaunchKernelGGL((k_kivi_quant<Tag, 128>), grid, dim3(kKThreads), 0, st, k, v, n_tokens, ng, dst, dst_token0); break;
        default: hipLaunchKernelGGL((k_kivi_quant<Tag, 256>), grid, dim3(kKThreads), 0, st, k, v, n_tokens, ng, dst, dst_token0); break;
    }
    return hipGetLastError();
}

template <int D>
void launch_kdec_d(int G, const DecodeArgs &a, const tq_kivi_store &src, hipStream_t st) {
    const dim3 grid((unsigned)a.n_split, (unsigned)(a.batch * a.hkv));
    switch (G) {
        case 1: hipLaunchKernelGGL((k_kivi_decode<D, 1>), grid, dim3(kKThreads), 0, st, a, src); break;
        case 2: hipLaunchKernelGGL((k_kivi_decode<D, 2>), grid, dim3(kKThreads), 0, st, a, src); break;
        case 4: hipLaunchKernelGGL((k_kivi_decode<D, 4>), grid, dim3(kKThreads), 0, st, a, src); break;
        default: hipLaunchKernelGGL((k_kivi_decode<D, 8>), grid, dim3(kKThreads), 0, st, a, src); break;
    }
}

}  // namespace

hipError_t launch_kivi_quantize(int d, tq_dtype dt, const void *k, const void *v, int64_t n_slices, int64_t n_tokens,
                                const tq_kivi_store &dst, int64_t dst_token0, hipStream_t st) {
    if (dt == TQ_F32) return launch_quant_t<f32_tag>(d, k, v, n_slices, n_tokens, dst, dst_token0, st);
    if (dt == TQ_BF16) return launch_quant_t<bf16_tag>(d, k, v, n_slices, n_tokens, dst, dst_token0, st);
    return launch_quant_t<f16_tag>(d, k, v, n_slices, n_tokens, dst, dst_token0, st);
}

hipError_t launch_kivi_decode(int d, int G, const DecodeArgs &a, const tq_kivi_store &src, hipStream_t st) {
    if (d == 64) launch_kdec_d<64>(G, a, src, st);
    else if (d == 128) launch_kdec_d<128>(G, a, src, st);
    else launch_kdec_d<256>(G, a, src, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.n_split > 1) return launch_decode_merge(d, G, a, st);
    return hipSuccess;
}

}  // namespace tq

// tq_decode.hip -- hybrid decode attention over the packed store plus the exact ring
// (hotelren.com guide "企业官网建设流程全解析", section 5.1 item 2: attention over the
// compressed history together with the exact recent buffer), and the ring append
// (section 5.1 item 1: a decode-time token goes into the ring buffer).
//
// Scores of packed tokens are the unbiased inner-product estimate of section 二:
//   s_t = |k_t| ( <q', c[idx_t]> + g_t sqrt(pi/2)/d <w, 2 z_t - 1> ),  q' = Pi q,  w = S q',
// computed in the rotated domain: the query is rotated once (k_decode_prep) and each
// packed token costs one table lookup per coordinate instead of an inverse rotation.
//
// k_decode_main: grid (n_split, batch * n_kv_heads), 256 threads.  One workgroup owns all
// G = n_q_heads / n_kv_heads query heads of one kv head and a contiguous token range
// (split-K over the context).  Chunks of 256 tokens: one thread scores one token for all
// G heads; the chunk's value codes are staged in LDS and each thread then accumulates
// one coordinate (online softmax across chunks).  The last split also covers the ring.
// Each workgroup writes (m, l, o) partials; the last workgroup to finish a (batch, kv
// head) -- found with an atomic ticket -- merges them into the output and re-arms the
// ticket to zero.
#include <hip/hip_runtime.h>

#include "tq.h"
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

constexpr int kChunk = 256;
constexpr int kThreads = 256;

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
    // sum of w over coordinates
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

// block-wide reduction of G values (max or sum); every thread gets the result
template <int G, bool IsMax>
__device__ __forceinline__ void block_reduce(float (&v)[G], float *scratch /* [4][G] */) {
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
        for (int w = 1; w < kThreads / 64; ++w) x = IsMax ? fmaxf(x, scratch[w * G + g]) : x + scratch[w * G + g];
        v[g] = x;
    }
    __syncthreads();
}

template <int D, int VB, int G>
__global__ __launch_bounds__(kThreads) void k_decode_main(DecodeArgs a) {
    constexpr int VW = VB * D / 32;   // value words per record
    constexpr int NG = D / 32;        // value groups
    constexpr int HALF = 1 << (VB - 1);
    constexpr int PARTS = kThreads / D;  // token partitions in the value phase
    constexpr float kQjl = 1.2533141373155003f / D;  // sqrt(pi/2) / d

    __shared__ float s_qp[G][D];
    __shared__ float s_w[G][D];
    __shared__ float s_qr[G][D];
    __shared__ float s_wsum[G];
    __shared__ float s_c[8];
    __shared__ float s_p[G][kChunk];
    __shared__ uint32_t s_vw[kChunk][VW];
    __shared__ float s_vs[kChunk][NG];
    __shared__ float s_red[4 * G];
    __shared__ float s_corr[G];
    __shared__ float s_o[PARTS > 1 ? PARTS - 1 : 1][G][D];
    __shared__ unsigned s_ticket;

    const int tid = threadIdx.x;
    const int split = blockIdx.x;
    const int bk = blockIdx.y;  // b * hkv + kv head == slice
    const int b = bk / a.hkv, kvh = bk - b * a.hkv;

    for (int i = tid; i < G * D; i += kThreads) {
        const int g = i / D, j = i - g * D;
        const float *p = a.prep + ((int64_t)b * a.hq + kvh * G + g) * (3 * D + 4);
        s_qp[g][j] = p[j];
        s_w[g][j] = p[D + j];
        s_qr[g][j] = p[2 * D + j];
        if (j == 0) s_wsum[g] = p[3 * D];
    }
    if (tid < 8) s_c[tid] = a.centroids[tid];
    __syncthreads();

    const int64_t t_begin = (int64_t)split * a.per_split;
    const int64_t t_end = min(a.n_packed, t_begin + a.per_split);
    const bool do_ring = (split == a.n_split - 1) && a.n_ring > 0;

    float m_run[G], l_run[G], o[G];
#pragma unroll
    for (int g = 0; g < G; ++g) { m_run[g] = -INFINITY; l_run[g] = 0.f; o[g] = 0.f; }
    const int jv = tid % D, part = tid / D;

    const int64_t n_pk_chunks = t_end > t_begin ? (t_end - t_begin + kChunk - 1) / kChunk : 0;
    const int64_t n_chunks = n_pk_chunks + (do_ring ? (a.n_ring + kChunk - 1) / kChunk : 0);

    for (int64_t ch = 0; ch < n_chunks; ++ch) {
        const bool ring = ch >= n_pk_chunks;
        int64_t c0;
        int cnt;
        if (!ring) {
            c0 = t_begin + ch * kChunk;
            cnt = (int)min<int64_t>(kChunk, t_end - c0);
        } else {
            c0 = (ch - n_pk_chunks) * kChunk;
            cnt = (int)min<int64_t>(kChunk, a.n_ring - c0);
        }
        // ---- scores: thread tid scores token c0 + tid for all G heads
        float lg[G];
        if (tid < cnt) {
            if (!ring) {
                const int64_t rec = (int64_t)bk * a.cap + c0 + tid;
                float mse[G], sg[G];
#pragma unroll
                for (int g = 0; g < G; ++g) { mse[g] = 0.f; sg[g] = 0.f; }
                const uint4 *kp = reinterpret_cast<const uint4 *>(a.kw + rec * (D / 8));
#pragma unroll 1
                for (int q4 = 0; q4 < D / 32; ++q4) {
                    const uint4 wq = kp[q4];
                    const uint32_t ws[4] = {wq.x, wq.y, wq.z, wq.w};
#pragma unroll
                    for (int wi = 0; wi < 4; ++wi) {
                        const uint32_t word = ws[wi];
#pragma unroll
                        for (int k = 0; k < 8; ++k) {
                            const int j = 32 * q4 + 8 * wi + k;
                            const float c = s_c[(word >> (3 * k)) & 7u];
                            const float zf = (float)((word >> (24 + k)) & 1u);
#pragma unroll
                            for (int g = 0; g < G; ++g) {
                                mse[g] = fmaf(s_qp[g][j], c, mse[g]);
                                sg[g] = fmaf(s_w[g][j], zf, sg[g]);
                            }
                        }
                    }
                }
                const float2 nr = *reinterpret_cast<const float2 *>(a.kn + rec * 2);
#pragma unroll
                for (int g = 0; g < G; ++g)
                    lg[g] = nr.x * (mse[g] + nr.y * kQjl * (2.f * sg[g] - s_wsum[g])) * a.scale;
                // stage this token's value record
                const uint4 *vp = reinterpret_cast<const uint4 *>(a.vw + rec * VW);
#pragma unroll
                for (int i = 0; i < VW / 4; ++i) {
                    const uint4 u = vp[i];
                    s_vw[tid][4 * i + 0] = u.x; s_vw[tid][4 * i + 1] = u.y;
                    s_vw[tid][4 * i + 2] = u.z; s_vw[tid][4 * i + 3] = u.w;
                }
#pragma unroll
                for (int gi = 0; gi < NG; ++gi)
                    s_vs[tid][gi] = (float)__builtin_bit_cast(_Float16, a.vs[rec * NG + gi]);
            } else {
                const uint16_t *kr = a.rk + ((int64_t)bk * a.buffer_size + c0 + tid) * D;
                float acc[G];
#pragma unroll
                for (int g = 0; g < G; ++g) acc[g] = 0.f;
#pragma unroll 1
                for (int i = 0; i < D; i += 8) {
                    float kv8[8];
                    load8(kr, i, kv8, f16_tag{});
#pragma unroll
                    for (int e = 0; e < 8; ++e)
#pragma unroll
                        for (int g = 0; g < G; ++g) acc[g] = fmaf(s_qr[g][i + e], kv8[e], acc[g]);
                }
#pragma unroll
                for (int g = 0; g < G; ++g) lg[g] = acc[g] * a.scale;
            }
        } else {
#pragma unroll
            for (int g = 0; g < G; ++g) lg[g] = -INFINITY;
        }
        // ---- online softmax update
        float mx[G];
#pragma unroll
        for (int g = 0; g < G; ++g) mx[g] = lg[g];
        block_reduce<G, true>(mx, s_red);
        float pe[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float mnew = fmaxf(m_run[g], mx[g]);
            const float corr = (m_run[g] == -INFINITY) ? 0.f : __expf(m_run[g] - mnew);
            pe[g] = (tid < cnt) ? __expf(lg[g] - mnew) : 0.f;
            s_p[g][tid] = pe[g];
            if (tid == 0) s_corr[g] = corr;
            m_run[g] = mnew;
            l_run[g] *= corr;
        }
        block_reduce<G, false>(pe, s_red);  // also orders the s_p / s_vw writes
#pragma unroll
        for (int g = 0; g < G; ++g) {
            l_run[g] += pe[g];
            o[g] *= s_corr[g];
        }
        // ---- values: thread (jv, part) accumulates coordinate jv over tokens part, part+PARTS, ...
        if (!ring) {
            const int wsel = jv * VB / 32;
            const int shift = VB * (jv % (32 / VB));
            const int gsel = jv / 32;
            for (int tt = part; tt < cnt; tt += PARTS) {
                const uint32_t code = (s_vw[tt][wsel] >> shift) & ((1u << VB) - 1u);
                const float vh = ((float)code - (float)HALF + 0.5f) * s_vs[tt][gsel];
#pragma unroll
                for (int g = 0; g < G; ++g) o[g] = fmaf(s_p[g][tt], vh, o[g]);
            }
        } else {
            for (int tt = part; tt < cnt; tt += PARTS) {
                const uint16_t vb16 = a.rv[((int64_t)bk * a.buffer_size + c0 + tt) * D + jv];
                const float vh = (float)__builtin_bit_cast(_Float16, vb16);
#pragma unroll
                for (int g = 0; g < G; ++g) o[g] = fmaf(s_p[g][tt], vh, o[g]);
            }
        }
        __syncthreads();  // s_p / s_vw are rewritten by the next chunk
    }

    // ---- combine the token partitions of the value phase
    if constexpr (PARTS > 1) {
        if (part > 0)
#pragma unroll
            for (int g = 0; g < G; ++g) s_o[part - 1][g][jv] = o[g];
        __syncthreads();
        if (part == 0)
#pragma unroll
            for (int pp = 0; pp < PARTS - 1; ++pp)
#pragma unroll
                for (int g = 0; g < G; ++g) o[g] += s_o[pp][g][jv];
    }
    // ---- partials: [G][D + 2] = o (unnormalised), m, l
    float *pp = a.partial + ((int64_t)bk * a.n_split + split) * G * (D + 2);
    if (part == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) pp[g * (D + 2) + jv] = o[g];
        if (jv == 0)
#pragma unroll
            for (int g = 0; g < G; ++g) {
                pp[g * (D + 2) + D] = m_run[g];
                pp[g * (D + 2) + D + 1] = l_run[g];
            }
    }
    __threadfence();
    __syncthreads();
    if (tid == 0)
        s_ticket = __hip_atomic_fetch_add(a.tickets + bk, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_ticket != (unsigned)(a.n_split - 1)) return;
    __threadfence();
    // ---- last workgroup of this (batch, kv head): merge the n_split partials.
    // Split weights f_s = exp(m_s - M) and the sum L per head are computed by one wave per
    // head with all splits' loads in flight; then every thread sums o over the splits for
    // its (head, coordinate) outputs, with the loads of many splits issued back to back.
    const float *base = a.partial + (int64_t)bk * a.n_split * G * (D + 2);
    {
        const int lane = tid & 63, wv = tid >> 6;
        for (int g = wv; g < G; g += kThreads / 64) {
            float mx = -INFINITY;
            for (int sp = lane; sp < a.n_split; sp += 64) mx = fmaxf(mx, base[(sp * G + g) * (D + 2) + D]);
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
            float ls = 0.f;
            for (int sp = lane; sp < a.n_split; sp += 64) {
                const float ms = base[(sp * G + g) * (D + 2) + D];
                const float f = (ms == -INFINITY) ? 0.f : __expf(ms - mx);
                s_p[g][sp] = f;
                ls = fmaf(base[(sp * G + g) * (D + 2) + D + 1], f, ls);
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) ls += __shfl_xor(ls, o);
            if (lane == 0) s_corr[g] = ls;
        }
    }
    __syncthreads();
    for (int i = tid; i < G * D; i += kThreads) {
        const int g = i / D, j = i - g * D;
        float O = 0.f;
#pragma unroll 8
        for (int sp = 0; sp < a.n_split; ++sp) O = fmaf(s_p[g][sp], base[(sp * G + g) * (D + 2) + j], O);
        const float L = s_corr[g];
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
    dim3 grid((unsigned)a.n_split, (unsigned)(a.batch * a.hkv));
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

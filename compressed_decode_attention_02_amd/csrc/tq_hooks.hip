// tq_hooks.hip -- test hooks of the library, off the hot path: the rotation Pi applied to
// rows (hotelren.com guide "企业官网建设流程全解析", section 二 step 1: Pi = H diag(sigma)
// / sqrt(d)), and the raw attention scores of a decode call before the softmax (section 二:
// the unbiased inner-product estimate over packed records; the exact product over the ring
// of section 5.1 item 2).  Plain kernels written to be checked by eye, not for speed:
//   * k_rotate: one wave per row; lane l holds coordinates l + 64 e, the Sylvester
//     butterflies run over the lane bits by shuffles, then over e in registers;
//   * k_scores: one workgroup per (query head, 256 tokens) derives q' = Pi q and
//     w = S q' in LDS itself, then one thread scores one token in fp32.
#include <hip/hip_runtime.h>

#include "tq.h"
#include "tq_device.h"
#include "tq_internal.h"
#include "tq_hooks.h"

namespace tq {
namespace {

constexpr int kHookThreads = 256;

__device__ __forceinline__ float load_elem(const void *p, int dtype, int64_t i) {
    if (dtype == TQ_F32) return load1(p, i, f32_tag{});
    if (dtype == TQ_BF16) return load1(p, i, bf16_tag{});
    return load1(p, i, f16_tag{});
}

// v (lane l, register e: coordinate l + 64 e) <- Pi v given sigma o v: the natural-order
// Sylvester transform, pairs (i, i + len) -> (a + b, a - b), then the 1/sqrt(D) scale
template <int D>
__device__ void hadamard_row(float (&v)[D / 64], int lane) {
    constexpr int E = D / 64;
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
    const float inv_sqrt_d = D == 64 ? 0.125f : (D == 128 ? 0.08838834764831845f : 0.0625f);
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] *= inv_sqrt_d;
}

template <int D>
__global__ __launch_bounds__(kHookThreads) void k_rotate(const uint32_t *sign_bits, const void *x, int dtype,
                                                         int64_t n_rows, float *out) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * (kHookThreads / 64) + (threadIdx.x >> 6);
    if (row >= n_rows) return;  // whole waves leave; the kernel has no barrier
    float v[D / 64];
#pragma unroll
    for (int e = 0; e < D / 64; ++e) {
        const int j = lane + 64 * e;
        v[e] = flip_sign(load_elem(x, dtype, row * D + j), (sign_bits[j >> 5] >> (j & 31)) & 1u);
    }
    hadamard_row<D>(v, lane);
#pragma unroll
    for (int e = 0; e < D / 64; ++e) out[row * D + lane + 64 * e] = v[e];
}

template <int D>
__global__ __launch_bounds__(kHookThreads) void k_scores(ScoreArgs a) {
    __shared__ float qs[D], qr[D], ws[D];
    const int tid = threadIdx.x, lane = tid & 63;
    const int bh = blockIdx.y;  // b * hq + query head
    const int b = bh / a.hq, h = bh - b * a.hq;
    const int64_t sl = (int64_t)b * a.hkv + h / (a.hq / a.hkv);
    for (int j = tid; j < D; j += kHookThreads) qs[j] = load_elem(a.q, a.q_dtype, (int64_t)bh * D + j);
    __syncthreads();
    if (tid < 64) {
        float v[D / 64];
#pragma unroll
        for (int e = 0; e < D / 64; ++e) {
            const int j = lane + 64 * e;
            v[e] = flip_sign(qs[j], (a.sign_bits[j >> 5] >> (j & 31)) & 1u);
        }
        hadamard_row<D>(v, lane);
#pragma unroll
        for (int e = 0; e < D / 64; ++e) qr[lane + 64 * e] = v[e];
    }
    __syncthreads();
    for (int i = tid; i < D; i += kHookThreads) {
        float acc = 0.f;
        for (int j = 0; j < D; ++j) acc = fmaf(f16_lo(a.S[(int64_t)i * D + j]), qr[j], acc);
        ws[i] = acc;
    }
    __syncthreads();
    const int64_t T = a.n_packed + a.n_ring;
    const int64_t t = (int64_t)blockIdx.x * kHookThreads + tid;
    if (t >= T) return;  // after the last barrier
    float s;
    if (t < a.n_packed) {
        // s = |k| (sum_j q'_j c[idx_j] + gamma sqrt(pi/2)/d sum_j w_j (2 z_j - 1))
        // key record: (kb + 1) d / 32 words; kb = 3: nibbles (index, sign bit on top), else a
        // code plane of kb-bit fields and a sign plane
        const int64_t rec = record_index(a.bt, a.pt, a.pps, a.n_pages, a.cap, a.err, sl, t);
        const int kb = a.kb, per = 32 / kb;
        const uint32_t *kw = a.kw + rec * ((kb + 1) * D / 32);
        float mse = 0.f, sgn = 0.f;
        for (int j = 0; j < D; ++j) {
            uint32_t idx, z;
            if (kb == 3) {
                const uint32_t nib = (kw[j / 8] >> (4 * (j % 8))) & 15u;
                idx = nib & 7u;
                z = nib >> 3;
            } else {
                idx = (kw[j / per] >> (kb * (j % per))) & ((1u << kb) - 1u);
                z = (kw[kb * D / 32 + j / 32] >> (j % 32)) & 1u;
            }
            mse = fmaf(qr[j], a.centroids[idx], mse);
            sgn += z ? ws[j] : -ws[j];
        }
        const float kqjl = 1.2533141373155003f / (float)D;  // sqrt(pi / 2) / d
        s = a.kn[rec * 2] * fmaf(a.kn[rec * 2 + 1] * kqjl, sgn, mse);
    } else {
        // ring token: q . k over the exact fp16 key
        const uint16_t *kr = a.rk + (sl * a.buffer_size + (t - a.n_packed)) * D;
        float acc = 0.f;
        for (int j = 0; j < D; ++j) acc = fmaf(qs[j], f16_lo(kr[j]), acc);
        s = acc;
    }
    a.scores[(int64_t)bh * T + t] = s;
}

}  // namespace

hipError_t launch_rotate(int d, const uint32_t *sign_bits, const void *x, int dtype, int64_t n_rows, float *out,
                         hipStream_t st) {
    if (n_rows == 0) return hipSuccess;
    const dim3 grid((unsigned)((n_rows + kHookThreads / 64 - 1) / (kHookThreads / 64)));
    if (d == 64) hipLaunchKernelGGL((k_rotate<64>), grid, dim3(kHookThreads), 0, st, sign_bits, x, dtype, n_rows, out);
    else if (d == 128) hipLaunchKernelGGL((k_rotate<128>), grid, dim3(kHookThreads), 0, st, sign_bits, x, dtype, n_rows, out);
    else hipLaunchKernelGGL((k_rotate<256>), grid, dim3(kHookThreads), 0, st, sign_bits, x, dtype, n_rows, out);
    return hipGetLastError();
}

hipError_t launch_scores(int d, const ScoreArgs &a, hipStream_t st) {
    const int64_t T = a.n_packed + a.n_ring;
    if (T == 0) return hipSuccess;
    const dim3 grid((unsigned)((T + kHookThreads - 1) / kHookThreads), (unsigned)(a.batch * a.hq));
    if (d == 64) hipLaunchKernelGGL((k_scores<64>), grid, dim3(kHookThreads), 0, st, a);
    else if (d == 128) hipLaunchKernelGGL((k_scores<128>), grid, dim3(kHookThreads), 0, st, a);
    else hipLaunchKernelGGL((k_scores<256>), grid, dim3(kHookThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace tq

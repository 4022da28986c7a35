// tq_hooks.h -- launchers of the library's test hooks (tq_hooks.hip), called by the C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace tq {

// test hooks (tq_hooks.hip): raw scores of a decode call, [batch][hq][n_packed + n_ring]
struct ScoreArgs {
    const void *q;
    int q_dtype;
    int batch, hq, hkv;
    const uint32_t *kw;
    const float *kn;
    int64_t cap;
    const int32_t *bt;
    int pt, pps;
    int64_t n_pages;
    int32_t *err;
    int64_t n_packed;
    const uint16_t *rk;
    int buffer_size;
    int n_ring;
    int kb;  // codebook bits of the key records
    const float *centroids;
    const uint32_t *sign_bits;
    const uint16_t *S;
    float *scores;
};
hipError_t launch_rotate(int d, const uint32_t *sign_bits, const void *x, int dtype, int64_t n_rows, float *out,
                         hipStream_t st);
hipError_t launch_scores(int d, const ScoreArgs &a, hipStream_t st);

}  // namespace tq

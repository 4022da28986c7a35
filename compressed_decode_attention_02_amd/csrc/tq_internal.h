// tq_internal.h -- declarations shared by the host and device translation units of the
// library (not installed; the public interface is include/tq.h).
#pragma once
#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime.h>

#include "tq.h"

namespace tq {

// byte offsets inside the device table blob (see tq_tables_bytes in tq.h)
constexpr size_t kTableCentroidOffset = 0;
constexpr size_t kTableBoundaryOffset = 64;
constexpr size_t kTableSignOffset = 128;
constexpr size_t kTableSOffset = 256;

tq_status check_config(const tq_config &c);

// true when every c[i] * 2^(14 - e) is an integer below 2^14 in magnitude, 2^e the power of two
// just above max |c[i]| (the decode's integer score path relies on it)
bool centroids_are_scaled_integers(const float *c, int n);

// compute units of the current device (cached per device; 256 if the query fails)
int device_cus();

struct QuantArgs {
    const void *k;
    const void *v;
    int64_t in_slice_stride;  // elements between consecutive slices of the input
    int64_t n_tokens;         // tokens per slice
    int64_t n_rows;           // n_slices * n_tokens
    const float *centroids;
    const float *boundaries;
    const uint32_t *sign_bits;
    const uint16_t *S;
    uint32_t *kw;
    float *kn;
    uint32_t *vw;
    uint16_t *vs;
    int64_t cap;
    int64_t dst_offset;
    // paged store (bt != nullptr): record of token t of slice s = pt * bt[s * pps + t / pt] + t % pt
    const int32_t *bt;
    int pt, pps;
    int64_t n_pages;
    int32_t *err;  // set to 1 when a table entry lies outside the pool (may be null)
};

struct DecodeArgs {
    const void *q;
    int q_dtype;  // tq_dtype of q
    const float *centroids;
    const uint32_t *sign_bits;
    const uint16_t *S;
    const uint32_t *kw;
    const float *kn;
    const uint32_t *vw;
    const uint16_t *vs;
    int64_t cap;
    const int32_t *bt;  // paged store, as in QuantArgs
    int pt, pps;
    int64_t n_pages;
    int32_t *err;
    int64_t n_packed;
    uint16_t *rk;  // ring (written only by a fused step's append)
    uint16_t *rv;
    int buffer_size;
    int n_ring;
    int batch, hq, hkv;
    int n_split;        // splits of the packed and the ring tokens (>= 1), <= 256
    int ring_per_split; // ring tokens per split (<= 64 at d = 128, <= 32 at d = 256)
    int waves;          // waves per workgroup of the packed splits (4 or 12)
    int64_t per_split;  // packed tokens per split
    float scale;
    float *out;
    float *prep;         // d = 256 and k_decode_any: [batch*hkv][2][G][D], q' then w of the slice's query heads
    // ragged batches: per-sequence lengths [batch] on the device (n_packed / n_ring are then
    // their maxima, each length clamped to [0, maximum]); null: every sequence n_packed / n_ring
    const int64_t *seq_packed;
    const int32_t *seq_ring;
    // fused append (tq_decode_step): the new token of every slice, [batch*hkv][D] in kv_dtype,
    // goes to ring slot new_slot (< n_ring) by the split that attends to that slot; -1: none
    const void *k_new;
    const void *v_new;
    int kv_dtype;
    int new_slot;
    // prefill (tq_prefill_attention): q_tokens > 0 makes batch element b query token
    // b % q_tokens of sequence b / q_tokens, which reads that sequence's packed records; with
    // causal set, query token i attends to packed tokens [0, q_pos0 + i] only
    int q_tokens;
    int64_t q_pos0;
    int causal;
    int64_t q_slice0;  // prefill: store slice of the launch's first sequence
    float *partial;      // [batch*hkv][n_split][G][D]: o of each split
    float *partial_ml;   // [batch*hkv][n_split][G][2]: (m, l) of each split
};

// record index of token t of slice s (paged or contiguous store).  A table entry outside
// [0, n_pages) is clamped to the pool, so no access leaves it, and reported through *err
// (set to 1; every writer stores the same value) when err is not null.
__device__ inline int64_t record_index(const int32_t *bt, int pt, int pps, int64_t n_pages, int64_t cap,
                                       int32_t *err, int64_t s, int64_t t) {
    if (!bt) return s * cap + t;
    int64_t p = bt[s * pps + t / pt];
    if (p < 0 || p >= n_pages) {
        if (err) __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        p = p < 0 ? 0 : n_pages - 1;
    }
    return p * pt + t % pt;
}

// prefill attention by query tiles (tq_prefill.hip): the launch's query rows are (sequence,
// query token, head) with the G heads of a kv head consecutive; each workgroup prepares its
// rows' q' and w itself
struct PrefillArgs {
    const void *q;      // [n_seq][T][hq][D] in q_dtype
    int q_dtype;
    const uint32_t *sign_bits;
    const uint16_t *S;
    const float *centroids;
    const uint32_t *kw;
    const float *kn;
    const uint32_t *vw;
    const uint16_t *vs;
    int64_t cap;
    const int32_t *bt;  // paged store, as in QuantArgs
    int pt, pps;
    int64_t n_pages;
    int32_t *err;
    int64_t n_packed;
    int64_t q_pos0;     // position of the launch's first query token
    int causal;
    int T;              // query tokens per sequence in this launch
    int hq, hkv;
    int64_t slice0;     // store slice of the launch's first sequence (times hkv)
    int tiles;          // query tiles per (sequence, kv head)
    float scale;
    float *out;         // [n_seq][T][hq][D] fp32 (n_split == 1)
    // split of each tile's packed tokens over n_split workgroups (per_split tokens each, a
    // multiple of the block size): each writes its unnormalised o and (m, l) per row in the decode's split
    // layout, [n_seq * T * hkv][n_split][G][D] and [..][n_split][G][2], for k_decode_merge
    int n_split;
    int per_split;
    float *partial;
    float *partial_ml;
};

hipError_t launch_quantize(int d, int kb, int vb, tq_dtype dt, const QuantArgs &a, hipStream_t st);
hipError_t launch_decode(int d, int kb, int vb, int G, const DecodeArgs &a, hipStream_t st);
// decode through k_decode_any (the key widths other than 3 bits, and head_dim 64), whose
// workspace holds the prepared queries
bool decode_uses_any(int d, int kb);
void launch_decode_any_main(int d, int kb, int vb, int G, const DecodeArgs &a, hipStream_t st);
// query rows per prefill tile, and the tiled prefill itself
int prefill_tile_rows(int d);
int prefill_block_tokens(int d);
hipError_t launch_prefill(int d, int kb, int vb, int64_t n_seq, const PrefillArgs &a, hipStream_t st);
// the split merge alone (a.n_split > 1), for decode kernels that write the same partials
hipError_t launch_decode_merge(int d, int G, const DecodeArgs &a, hipStream_t st);
// KIVI 2-bit variant (tq_kivi.hip)
hipError_t launch_kivi_quantize(int d, tq_dtype dt, const void *k, const void *v, int64_t n_slices, int64_t n_tokens,
                                const tq_kivi_store &dst, int64_t dst_token0, hipStream_t st);
hipError_t launch_kivi_decode(int d, int G, const DecodeArgs &a, const tq_kivi_store &src, hipStream_t st);
hipError_t launch_ring_append(int d, tq_dtype dt, const void *kn, const void *vn, uint16_t *rk, uint16_t *rv,
                              int n_slices, int buffer_size, int slot, hipStream_t st);

}  // namespace tq

/*
 * tq.h -- C ABI of the MI355X (gfx950) TurboQuant KV-cache library.
 *
 * The library compresses attention keys and values into a packed cache and runs
 * decode attention directly on that cache plus an exact ring buffer of recent tokens.
 * The method (rotation, Lloyd-Max codebook for a Beta law, one QJL residual sign bit per
 * coordinate, 2/4-bit symmetric value groups of 32, bit packing, exact recent buffer,
 * hybrid attention) is the one described in the hotelren.com guide
 * "企业官网建设流程全解析", sections 二 (five-step pipeline) and 5.1 (KV-write and
 * forward hooks: prefill batch capture, single-token ring buffer, hybrid attention).
 *
 * Conventions for every entry point:
 *   - Pointers named host_* are host memory; every other buffer pointer is device memory
 *     owned by the caller.  The library never allocates device memory.  Its only state is a
 *     per-device cache of the compute-unit count and of the address of the static scratch
 *     array of tq_decode_attention_noalloc (a fixed-size device array per GPU, held until the
 *     process ends).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Device work is enqueued
 *     asynchronously on it; the call returns once the work is enqueued.
 *   - All argument checks run synchronously on the host before anything is enqueued; on
 *     any error nothing is launched and a negative tq_status is returned.
 *   - Device pointers must be 16-byte aligned, except tq_packed.key_norms and
 *     tq_packed.val_scales, which need 8 bytes (TQ_ERR_INVALID_ARG otherwise).
 *   - Supported: head_dim in {64, 128, 256}; key_bits in {1, 2, 3, 4} (head_dim 256: 3 only);
 *     value_bits in {2, 4}; group_size = 32; 1 <= buffer_size <= 1024.  Other values give
 *     TQ_ERR_UNSUPPORTED.  The guide (section 二) ships codebooks for dimensions 64 and 128
 *     at 1 to 4 bits; 3-bit keys at head_dim 128 and 256 decode on the matrix cores, the
 *     other configurations through a plain fp32 decode kernel.
 *   - Decode calls address tokens with 32-bit indices: a context (packed + ring tokens) of
 *     2^31 - 256 tokens or more gives TQ_ERR_UNSUPPORTED.
 *   - Reproducibility: quantisation is deterministic.  A decode call repeats bit for bit
 *     when its workgroups have 4 waves; for long contexts at head_dim 128 with up to four
 *     query heads per kv head it uses one 12-wave workgroup per compute unit whose waves
 *     take token blocks in arrival order, so the fp32 summation order, and with it the last
 *     bits of the output, may differ between identical calls (well inside the accuracy of
 *     the method; the tests bound the spread at 1e-5 relative).
 *   - Non-finite inputs give unspecified output (no device-side scan).
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TQ_OK = 0,
    TQ_ERR_INVALID_ARG = -1,  /* null/misaligned pointer, negative size, inconsistent shape */
    TQ_ERR_UNSUPPORTED = -2,  /* head_dim / bit width / group size not implemented          */
    TQ_ERR_RING_FULL = -3,    /* append to a ring that already holds buffer_size tokens     */
    TQ_ERR_WORKSPACE = -4,    /* decode workspace smaller than tq_decode_workspace_bytes()  */
    TQ_ERR_HIP = -5,          /* a HIP launch or runtime call failed                        */
    TQ_ERR_SCRATCH_LIMIT = -6 /* tq_decode_attention_noalloc: the call needs more scratch     */
                              /* than TQ_NOALLOC_SCRATCH_BYTES                              */
} tq_status;

typedef enum { TQ_F32 = 0, TQ_BF16 = 1, TQ_F16 = 2 } tq_dtype;

/* Compression parameters, named after the pages' hook arguments (key_bits, value_bits,
 * buffer_size; guide section 5.1) and the value grouping (32 per group; section 二).
 * key_bits counts the codebook bits only; every key coordinate also stores one QJL sign
 * bit (so key_bits = 3 costs 4 bits per coordinate). */
typedef struct {
    int32_t head_dim;     /* d: 64, 128 or 256                              */
    int32_t key_bits;     /* codebook bits per key coordinate: 1 to 4       */
    int32_t value_bits;   /* 2 or 4                                         */
    int32_t group_size;   /* values per quantisation group: 32              */
    int32_t buffer_size;  /* ring capacity in tokens (the pages use 128)    */
} tq_config;

/* ------------------------------------------------------------------ host-side tables */

/* Lloyd-Max codebook for one coordinate of a uniform unit vector in R^head_dim, i.e. the
 * law (t+1)/2 ~ Beta((d-1)/2, (d-1)/2) (guide section 二, step 2 and the pre-generated
 * codebooks per dimension and bit width).  Writes 2^key_bits centroids (ascending,
 * antisymmetric) and 2^key_bits - 1 decision boundaries (midpoints), in double precision.
 * head_dim: power of two in [8, 4096]; key_bits in [1, 4].  Host buffers, caller-owned. */
tq_status tq_build_codebook(int32_t head_dim, int32_t key_bits, double *host_centroids,
                            double *host_boundaries);

/* Seeded random tables of the method (guide section 二, steps 1 and 3): the sign vector
 * sigma of the rotation Pi = H diag(sigma) / sqrt(d) (H: natural-order Sylvester Hadamard
 * matrix) and the d x d QJL projection S with N(0,1) entries rounded to fp16, row-major.
 * Drawn from the splitmix64 stream seed + (i+1) * 0x9E3779B97F4A7C15: sigma_j from the
 * top bit of word j, S pairs by Box-Muller from words d + 2m, d + 2m + 1.
 * host_signs: d int8 (+1/-1); host_qjl_S: d*d fp16 bit patterns. */
tq_status tq_build_rotation(int32_t head_dim, uint64_t seed, int8_t *host_signs, uint16_t *host_qjl_S);

/* The device-side table blob: centroids at byte 0 (fp32 holding the binary16 rounding of
 * the Lloyd-Max values: the table precision of the fp16 KV path), decision boundaries at
 * byte 64 (fp32, exact midpoints of adjacent stored centroids),
 * sign bits at byte 128 (bit j%32 of word j/32 set when sigma_j = -1), fp16 S at byte 256.
 * tq_tables_bytes: blob size.  tq_build_tables: fills a host blob of that size (the caller
 * copies it to device memory once).  tq_tables_view: fills `out` with pointers into a
 * device copy of the blob. */
size_t tq_tables_bytes(const tq_config *cfg);
tq_status tq_build_tables(const tq_config *cfg, uint64_t seed, void *host_blob, size_t blob_bytes);

typedef struct {
    const float *centroids;     /* 2^key_bits fp32                    */
    const float *boundaries;    /* 2^key_bits - 1 fp32                */
    const uint32_t *sign_bits;  /* d/32 words                         */
    const uint16_t *qjl_S;      /* d*d fp16, row-major                */
} tq_tables;

tq_status tq_tables_view(const tq_config *cfg, const void *device_blob, tq_tables *out);

/* ------------------------------------------------------------------ packed store */

/* One packed record per (slice, token), slice = flattened (layer, batch, kv head);
 * every array is [n_slices][capacity][...] with the record of token t at t:
 *   key_words  [(kb+1)*d/32] u32, kb = key_bits:
 *                          kb = 3: word w covers coordinates 8w..8w+7 as nibbles: bits
 *                          4k..4k+2 hold the codebook index of coordinate 8w+k, bit 4k+3
 *                          its QJL sign bit (1 when the projected residual is >= 0);
 *                          kb = 1, 2, 4: a code plane, words 0..kb*d/32-1, index of
 *                          coordinate j at bit kb*(j mod 32/kb) of word j*kb/32, then a
 *                          sign plane, sign bit of coordinate j at bit j mod 32 of word
 *                          kb*d/32 + j/32;
 *   key_norms  [2]   f32 : |k| and the residual norm |u - c[idx]| of the unit key u;
 *   val_words  [vb*d/32] u32 : vb-bit codes, code j at bit vb*(j mod 32/vb) of word
 *                          j*vb/32 (least significant first: four 2-bit codes per byte);
 *   val_scales [d/32] fp16 : per-group scale s; value = (code - 2^(vb-1) + 1/2) * s.
 * Bytes per record: (kb+1)*d/8 + 8 + vb*d/8 + d/16, e.g. 112 (d 128, kb 3, vb 2), 144
 * (d 128, kb 3, vb 4), 280 (d 256, kb 3, vb 4), 44 (d 64, kb 1, vb 2). */
typedef struct {
    uint32_t *key_words;
    float *key_norms;
    uint32_t *val_words;
    uint16_t *val_scales;
    int64_t capacity;           /* tokens per slice */
    /* Paged store (block_table != NULL; NULL/0 fields give the contiguous layout above): the
     * four arrays are a pool of n_pages pages of page_tokens records ([n_pages][page_tokens]
     * [...]), and token t of slice s is record page_tokens * p + t % page_tokens of page
     * p = block_table[s * pages_per_slice + t / page_tokens] (device int32 table, 4-byte
     * aligned).  page_tokens must be a multiple of 32 and capacity == pages_per_slice *
     * page_tokens.  Table entries outside [0, n_pages) are clamped on the device, so no entry
     * addresses outside the pool; pages shared by two slices receive both writes (the
     * caller's table decides which tokens land where).
     * error_flag (paged stores only; may be NULL): a device int32 (4-byte aligned) that a
     * kernel sets to 1 when it meets a table entry outside [0, n_pages).  The library never
     * clears it: the caller zeroes it, and reads it after the calls it covers have finished
     * (a clamped entry reads or writes another page of the pool, so results of those calls
     * are then unspecified). */
    const int32_t *block_table;
    int32_t page_tokens;
    int32_t pages_per_slice;
    int64_t n_pages;
    int32_t *error_flag;
} tq_packed;

/* Exact recent tokens: fp16 [n_slices][buffer_size][d] keys and values (guide 5.1). */
typedef struct {
    uint16_t *k;
    uint16_t *v;
} tq_ring;

/* Bytes of one packed record (one token of one kv head) in device memory: the compressed
 * size that replaces 4 * head_dim bytes of a bf16/fp16 K+V cache (the guide's section 5.2
 * reports the bytes its free_kv_cache releases; this is the per-token figure behind such a
 * report).  0 for an unsupported configuration. */
size_t tq_packed_bytes_per_token(const tq_config *cfg);

/* ------------------------------------------------------------------ device entry points */

/* Prefill batch capture (guide 5.1 item 1; pipeline of section 二): compress n_tokens
 * tokens of each of n_slices slices.  k, v: [n_slices][n_tokens][d] in in_dtype.
 * Writes records dst_offset .. dst_offset + n_tokens - 1 of every slice.
 * Requires dst_offset + n_tokens <= dst->capacity.  n_tokens == 0 is a no-op. */
tq_status tq_quantize_kv(const tq_config *cfg, const tq_tables *tables, const void *k, const void *v,
                         tq_dtype in_dtype, int32_t n_slices, int64_t n_tokens,
                         const tq_packed *dst, int64_t dst_offset, void *stream);

/* Decode single-token capture into the ring (guide 5.1 item 1): k_new, v_new
 * [n_slices][d] in in_dtype are rounded to fp16 into ring slot n_ring of each slice.
 * n_ring is the caller's current fill count; n_ring == buffer_size -> TQ_ERR_RING_FULL. */
tq_status tq_append_ring(const tq_config *cfg, const tq_ring *ring, const void *k_new, const void *v_new,
                         tq_dtype in_dtype, int32_t n_slices, int32_t n_ring, void *stream);

/* Periodic flush of the ring into the compressed store (zingnex.cn page, Bonsai section:
 * the recent exact window is flushed into the main cache): compresses ring slots
 * 0 .. n_ring-1 of every slice into records n_packed .. n_packed + n_ring - 1.  The caller
 * then sets n_packed += n_ring and n_ring = 0. */
tq_status tq_flush(const tq_config *cfg, const tq_tables *tables, const tq_ring *ring, int32_t n_slices,
                   int32_t n_ring, const tq_packed *dst, int64_t n_packed, void *stream);

/* Workspace (device bytes) needed by tq_decode_attention for up to max_context tokens
 * (packed + ring): per-split partial results (the split-K decode of long contexts across
 * compute units), and at head_dim 256 and for the configurations decoded in fp32 (key_bits
 * other than 3, head_dim 64) the prepared queries; scratch only (no initialisation
 * needed).  Calls that share a workspace must be ordered (same stream), as they use it in
 * turn.  0 for invalid arguments. */
size_t tq_decode_workspace_bytes(const tq_config *cfg, int32_t batch, int32_t n_q_heads,
                                 int32_t n_kv_heads, int64_t max_context);

/* Hybrid decode attention (guide 5.1 item 2): for each batch b and query head h (GQA:
 * kv head h / (n_q_heads / n_kv_heads)), softmax(scale * s) over the n_packed compressed
 * tokens (s = unbiased inner-product estimate from codes, signs and norms) and the n_ring
 * exact ring tokens, applied to the dequantised / exact values.
 * q: [batch][n_q_heads][d] in q_dtype; packed / ring slices are b * n_kv_heads + kv head;
 * out: [batch][n_q_heads][d] fp32.  n_packed + n_ring == 0 writes zeros. */
tq_status tq_decode_attention(const tq_config *cfg, const tq_tables *tables, const void *q, tq_dtype q_dtype,
                              int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                              const tq_packed *packed, int64_t n_packed, const tq_ring *ring, int32_t n_ring,
                              float softmax_scale, float *out, void *workspace, size_t workspace_bytes,
                              void *stream);

/* Hybrid decode attention over a ragged batch (sequences of unequal length; a serving batch
 * holds requests at different positions): as tq_decode_attention, but batch element b
 * attends to its own seq_packed[b] records and seq_ring[b] ring tokens.  seq_packed (int64,
 * 8-byte aligned) and seq_ring (int32, 4-byte aligned) are device arrays of `batch` entries,
 * read by the kernel; n_packed_max / n_ring_max bound them (each length is clamped to
 * [0, its maximum] on the device) and size the work split; the workspace must cover
 * n_packed_max + n_ring_max tokens.  A sequence with no tokens gets zeros. */
tq_status tq_decode_attention_ragged(const tq_config *cfg, const tq_tables *tables, const void *q, tq_dtype q_dtype,
                                     int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, const tq_packed *packed,
                                     const int64_t *seq_packed, int64_t n_packed_max, const tq_ring *ring,
                                     const int32_t *seq_ring, int32_t n_ring_max, float softmax_scale, float *out,
                                     void *workspace, size_t workspace_bytes, void *stream);

/* One decode step (guide 5.1 items 1 and 2 in one call, with the forum's flush of a full
 * recent window): the new token k_new / v_new ([batch * n_kv_heads][d] in kv_dtype) of every
 * slice enters the ring and the hybrid attention runs over packed + ring, as
 * tq_append_ring followed by tq_decode_attention would, without the append's launch: the
 * decode kernel takes the new token from k_new / v_new (rounded to fp16 as the append rounds
 * it) and writes it into ring slot *n_ring.  When the ring is full (*n_ring == buffer_size)
 * it is first flushed into records *n_packed .. *n_packed + buffer_size - 1, as tq_flush.
 * *n_packed and *n_ring (host memory) are updated in place only on success; every argument
 * is checked before anything is launched.  Other arguments as tq_decode_attention; the
 * workspace must cover *n_packed + *n_ring + 1 tokens. */
tq_status tq_decode_step(const tq_config *cfg, const tq_tables *tables, const void *q, tq_dtype q_dtype,
                         int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, const tq_packed *packed,
                         int64_t *n_packed, const tq_ring *ring, int32_t *n_ring, const void *k_new,
                         const void *v_new, tq_dtype kv_dtype, float softmax_scale, float *out, void *workspace,
                         size_t workspace_bytes, void *stream);

/* Prefill attention over the packed cache (guide section 三, the full_tq mode: attention taken
 * entirely from the compressed cache, prefill included).  For sequence b (packed slices
 * b * n_kv_heads + kv head, as in tq_decode_attention) and query token i of q_tokens, query
 * head h attends, with the same estimator and value reconstruction as the decode, to packed
 * tokens [0, min(n_packed, q_pos0 + i + 1)) when causal == 1 (the query token at position
 * q_pos0 + i of a prompt whose tokens are already in the store), else to [0, n_packed).
 *   q   : [batch][q_tokens][n_q_heads][head_dim] in q_dtype (device);
 *   out : [batch][q_tokens][n_q_heads][head_dim] fp32 (device); a token with no packed token
 *         to attend to gets zeros.
 * Calls whose query rows per kv head (q_tokens * G, G = n_q_heads / n_kv_heads) fill at least
 * half a query tile (64 rows; 32 at head_dim 256) run the tiled kernel: one launch over (query
 * tile of 128 rows (64 at head_dim 256), sequence, kv head, split of the packed range) and, when
 * the packed range is split, the decode's merge; launches of at most 65536 / n_kv_heads query
 * tokens.  Fewer rows run the decode kernels with one batch element per query token reading its
 * sequence's records (launches of at most 65535 / n_kv_heads query tokens).  Every launch is
 * checked before the first; no ring.  workspace: tq_prefill_workspace_bytes(cfg, batch,
 * q_tokens, n_q_heads, n_kv_heads, n_packed) bytes (scratch; never needs clearing).  Errors as
 * tq_decode_attention; q_pos0 < 0 or causal not 0/1: TQ_ERR_INVALID_ARG. */
size_t tq_prefill_workspace_bytes(const tq_config *cfg, int32_t batch, int32_t q_tokens, int32_t n_q_heads,
                                  int32_t n_kv_heads, int64_t n_packed);
tq_status tq_prefill_attention(const tq_config *cfg, const tq_tables *tables, const void *q, tq_dtype q_dtype,
                               int32_t batch, int32_t q_tokens, int32_t n_q_heads, int32_t n_kv_heads,
                               const tq_packed *packed, int64_t n_packed, int64_t q_pos0, int32_t causal,
                               float softmax_scale, float *out, void *workspace, size_t workspace_bytes,
                               void *stream);

/* Decode without a workspace, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): tq_decode_attention
 * with the workspace taken from a static device array of TQ_NOALLOC_SCRATCH_BYTES (8 MiB) per
 * GPU instead of the caller's buffer.  The call allocates nothing (no hipMalloc, no library
 * allocation); its first call on a device looks the array's address up once.  A call whose
 * scratch (tq_decode_workspace_bytes for its shape) exceeds the array returns
 * TQ_ERR_SCRATCH_LIMIT before anything is launched.  Every call on one GPU uses that GPU's one
 * array: calls that may overlap on a GPU (different streams, or several host threads) race on
 * it and must be ordered by the caller.  The scratch needs no clearing (each call writes every
 * byte it reads).  Arguments and results as tq_decode_attention. */
#define TQ_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
tq_status tq_decode_attention_noalloc(const tq_config *cfg, const tq_tables *tables, const void *q,
                                      tq_dtype q_dtype, int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                      const tq_packed *packed, int64_t n_packed, const tq_ring *ring, int32_t n_ring,
                                      float softmax_scale, float *out, void *stream);

/* ------------------------------------------------------------------ KIVI 2-bit variant
 * The forum page's asymmetric quantiser (zingnex.cn "TurboQuant-vLLM：大模型推理的KV缓存量化
 * 实战方案", section "KIVI非对称量化"): keys per channel, values per token, each set with a scale
 * and a zero point, 2 bits; a second workload beside the TurboQuant records, with no rotation,
 * codebook or QJL bit.  A key channel's scale and zero cover 32 consecutive tokens, a value
 * token's pair its head_dim entries.  scale = binary16(fp32(fp32(max - min) / 3)), zero =
 * binary16(min) of the set; code = clamp(round-to-nearest-even(fp32(x - zero) / scale), 0, 3)
 * (IEEE binary32 division; 0 where the scale is 0); x^ = code scale + zero.  Inputs are taken
 * to lie within the binary16 range.  head_dim in {64, 128, 256}.
 *
 * Store (device arrays per slice, [n_slices][capacity][...], capacity a multiple of 32):
 *   key_codes  uint32 [capacity][head_dim / 16]: 2-bit codes, channel c at bits 2 (c % 16)
 *              of word c / 16;
 *   key_scale, key_zero  binary16 [capacity / 32][head_dim]: per 32-token group and channel;
 *   val_codes  uint32 [capacity][head_dim / 16] as key_codes;
 *   val_params binary16 [capacity][2]: (scale, zero) per token.
 * Arrays 16-byte aligned (TQ_ERR_INVALID_ARG otherwise); owned by the caller. */
typedef struct tq_kivi_store {
    uint32_t *key_codes;
    uint16_t *key_scale;
    uint16_t *key_zero;
    uint32_t *val_codes;
    uint16_t *val_params;
    int64_t capacity;
} tq_kivi_store;

/* Store bytes per token: head_dim / 4 (key codes) + head_dim / 8 (key scale and zero, a
 * 32-token group's share) + head_dim / 4 (value codes) + 4 (value scale and zero); 84 at
 * head_dim 128.  0 for an unsupported head_dim. */
size_t tq_kivi_bytes_per_token(int32_t head_dim);

/* Quantise k and v [n_slices][n_tokens][head_dim] (in_dtype) into records dst_token0 ..
 * dst_token0 + n_tokens - 1 of every slice.  n_tokens and dst_token0 multiples of 32 (whole
 * key groups; TQ_ERR_INVALID_ARG otherwise), dst_token0 + n_tokens <= capacity. */
tq_status tq_kivi_quantize(int32_t head_dim, const void *k, const void *v, tq_dtype in_dtype, int32_t n_slices,
                           int64_t n_tokens, const tq_kivi_store *dst, int64_t dst_token0, void *stream);

/* Decode attention over the first n_packed records of every slice of a KIVI store: out[b][h]
 * = softmax(softmax_scale q[b][h] . k^) v^ over the dequantised keys and values of kv head
 * h / (n_q_heads / n_kv_heads); q [batch][n_q_heads][head_dim] (q_dtype), out fp32, slices
 * b * n_kv_heads + kv head.  n_q_heads / n_kv_heads in {1, 2, 4, 8}; n_packed <= capacity; a
 * zero context writes zeros.  The workspace (tq_kivi_decode_workspace_bytes for the largest
 * context the caller will pass) holds the splits' partial results; it needs no clearing. */
size_t tq_kivi_decode_workspace_bytes(int32_t head_dim, int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                      int64_t max_context);
tq_status tq_kivi_decode_attention(int32_t head_dim, const void *q, tq_dtype q_dtype, int32_t batch,
                                   int32_t n_q_heads, int32_t n_kv_heads, const tq_kivi_store *src,
                                   int64_t n_packed, float softmax_scale, float *out, void *workspace,
                                   size_t workspace_bytes, void *stream);

const char *tq_status_string(tq_status s);

/* ------------------------------------------------------------------ test hooks
 * Unstable entry points for checking the method's steps one at a time; plain kernels, off
 * the decode path.  Device pointers, 16-byte aligned; same errors as the calls above. */

/* out = Pi x for n_rows rows of head_dim values (guide section 二 step 1: Pi = H diag(sigma)
 * / sqrt(d)); x [n_rows][d] in in_dtype, out [n_rows][d] fp32. */
tq_status tq_rotate(const tq_config *cfg, const tq_tables *tables, const void *x, tq_dtype in_dtype,
                    int64_t n_rows, float *out, void *stream);

/* The raw scores of a decode call before the softmax and its scale, scores [batch]
 * [n_q_heads][n_packed + n_ring] fp32: packed tokens first, by the estimate of guide section
 * 二 (|k| (q'.c[idx] + gamma sqrt(pi/2)/d w.(2z - 1)), q' = Pi q, w = S q'), then the ring's
 * tokens by q.k over the exact fp16 keys (guide 5.1 item 2).  Arguments as
 * tq_decode_attention; no workspace. */
tq_status tq_decode_scores(const tq_config *cfg, const tq_tables *tables, const void *q, tq_dtype q_dtype,
                           int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, const tq_packed *packed,
                           int64_t n_packed, const tq_ring *ring, int32_t n_ring, float *scores, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* TQ_H */

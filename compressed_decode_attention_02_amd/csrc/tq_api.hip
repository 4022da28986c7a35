// tq_api.hip -- C-ABI entry points: argument validation on the host, then kernel
// launches on the caller's stream.  Declarations and contracts: include/tq.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>

#include "tq.h"
#include "tq_internal.h"
#include "tq_hooks.h"

namespace {

constexpr int64_t kSplitQuantum = 128;     // split sizes are multiples of four 32-token blocks
constexpr int64_t kMinSplitTokens = 512;   // at least four blocks per wave
constexpr int64_t kMaxSplits = 256;        // the merge keeps one weight per split in LDS
constexpr int64_t kMaxContext = (int64_t(1) << 31) - 256;  // decode token indices are 32-bit
// ring tokens attended to per split, at most (the main kernel's register budget)
int64_t ring_per_split_max(int d) { return d == 128 ? 64 : 32; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned8(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

bool packed_ok(const tq_packed *p) {
    if (!(p && p->key_words && p->key_norms && p->val_words && p->val_scales && p->capacity >= 0 &&
          aligned16(p->key_words) && aligned8(p->key_norms) && aligned16(p->val_words) && aligned8(p->val_scales)))
        return false;
    if (!p->block_table) return true;
    // paged: whole 32-token blocks per page, the capacity the table covers, a non-empty pool
    return (reinterpret_cast<uintptr_t>(p->block_table) & 3u) == 0 &&
           (reinterpret_cast<uintptr_t>(p->error_flag) & 3u) == 0 && p->page_tokens > 0 &&
           p->page_tokens % 32 == 0 && p->pages_per_slice > 0 && p->n_pages > 0 &&
           p->capacity == (int64_t)p->pages_per_slice * p->page_tokens;
}

template <typename Args>
void set_pages(Args &a, const tq_packed *p) {
    a.bt = p->block_table;
    a.pt = p->block_table ? p->page_tokens : 1;
    a.pps = p->block_table ? p->pages_per_slice : 0;
    a.n_pages = p->block_table ? p->n_pages : 0;
    a.err = p->block_table ? p->error_flag : nullptr;
}

bool tables_ok(const tq_tables *t) {
    return t && t->centroids && t->boundaries && t->sign_bits && t->qjl_S && aligned16(t->qjl_S);
}

// waves per decode workgroup: 12 (one workgroup per CU; d = 128 with up to 4 query heads per
// kv head) when every wave then has at least 2 blocks of 32 tokens, else 4
int decode_waves(int d, int64_t G, int64_t slices, int64_t n_packed) {
    if (d != 128 || G > 4) return 4;
    const int64_t blocks_per_wave = slices * n_packed / ((int64_t)tq::device_cus() * 12 * 32);
    return blocks_per_wave >= 2 ? 12 : 4;
}

// decode workgroups resident per CU (LDS and registers; see the decode kernel's budget): the
// split count fills one such wave of workgroups on the current device
int64_t decode_target_wgs(int d, int vb, int64_t G, int waves, bool any) {
    const int64_t cus = tq::device_cus();
    if (any) return cus * 4;  // k_decode_any: 4-wave workgroups of at most 41 KB LDS, 4 per CU
    if (waves == 12) return cus;
    return cus * ((d == 128 && G <= 4) ? (vb == 2 ? 4 : 3) : 2);
}

// (4-wave workgroups give the most splits: the workspace is sized with them)
int64_t decode_splits(int d, int vb, int64_t G, int64_t slices, int64_t n_packed, int waves, bool any) {
    const int64_t by_tokens = std::max<int64_t>(1, (n_packed + kMinSplitTokens - 1) / kMinSplitTokens);
    const int64_t want = std::max<int64_t>(1, (decode_target_wgs(d, vb, G, waves, any) + slices - 1) / slices);
    return std::min({by_tokens, want, kMaxSplits});
}

// tokens per split: a whole number of 128-token passes; then as few splits as cover n_packed
void split_shape(int d, int vb, int64_t G, int64_t slices, int64_t n_packed, int waves, bool any, int64_t &n_split,
                 int64_t &per_split) {
    const int64_t s0 = decode_splits(d, vb, G, slices, n_packed, waves, any);
    per_split = (n_packed + s0 - 1) / s0;
    per_split = (per_split + kSplitQuantum - 1) / kSplitQuantum * kSplitQuantum;
    n_split = (n_packed + per_split - 1) / per_split;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// decode workspace: at d = 256 and on the k_decode_any path the prepared queries (q', w)
// [slices][2][G][d]; the packed
// splits' partials o [slices][n_split][G][d] and (m, l) pairs [slices][n_split][G][2]
// (slices * G = batch * hq)
struct DecodeLayout {
    size_t prep, partial, partial_ml, total;
};

DecodeLayout decode_layout(int d, int kb, int64_t batch, int64_t hq, int64_t n_split) {
    DecodeLayout L;
    L.prep = 0;
    const bool prep = d == 256 || tq::decode_uses_any(d, kb);
    L.partial = prep ? align256(sizeof(float) * (size_t)(batch * hq) * 2 * d) : 0;
    L.partial_ml = L.partial + align256(sizeof(float) * (size_t)(batch * hq) * n_split * d);
    L.total = std::max<size_t>(256, L.partial_ml + align256(sizeof(float) * (size_t)(batch * hq) * n_split * 2));
    return L;
}

tq_status hip_status(hipError_t e) { return e == hipSuccess ? TQ_OK : TQ_ERR_HIP; }

}  // namespace

extern "C" tq_status tq_quantize_kv(const tq_config *cfg, const tq_tables *tables, const void *k, const void *v,
                                    tq_dtype in_dtype, int32_t n_slices, int64_t n_tokens, const tq_packed *dst,
                                    int64_t dst_offset, void *stream) {
    if (!cfg) return TQ_ERR_INVALID_ARG;
    tq_status st = tq::check_config(*cfg);
    if (st != TQ_OK) return st;
    if (n_slices < 0 || n_tokens < 0 || dst_offset < 0) return TQ_ERR_INVALID_ARG;
    if (in_dtype != TQ_F32 && in_dtype != TQ_BF16 && in_dtype != TQ_F16) return TQ_ERR_INVALID_ARG;
    if (n_slices == 0 || n_tokens == 0) return TQ_OK;
    if (!tables_ok(tables) || !packed_ok(dst) || !k || !v || !aligned16(k) || !aligned16(v))
        return TQ_ERR_INVALID_ARG;
    if (dst_offset + n_tokens > dst->capacity) return TQ_ERR_INVALID_ARG;
    tq::QuantArgs a{};
    a.k = k;
    a.v = v;
    a.in_slice_stride = n_tokens * cfg->head_dim;
    a.n_tokens = n_tokens;
    a.n_rows = (int64_t)n_slices * n_tokens;
    a.centroids = tables->centroids;
    a.boundaries = tables->boundaries;
    a.sign_bits = tables->sign_bits;
    a.S = tables->qjl_S;
    a.kw = dst->key_words;
    a.kn = dst->key_norms;
    a.vw = dst->val_words;
    a.vs = dst->val_scales;
    a.cap = dst->capacity;
    a.dst_offset = dst_offset;
    set_pages(a, dst);
    return hip_status(tq::launch_quantize(cfg->head_dim, cfg->key_bits, cfg->value_bits, in_dtype, a, (hipStream_t)stream));
}

extern "C" tq_status tq_append_ring(const tq_config *cfg, const tq_ring *ring, const void *k_new, const void *v_new,
                                    tq_dtype in_dtype, int32_t n_slices, int32_t n_ring, void *stream) {
    if (!cfg) return TQ_ERR_INVALID_ARG;
    tq_status st = tq::check_config(*cfg);
    if (st != TQ_OK) return st;
    if (n_slices < 0 || n_ring < 0 || n_ring > cfg->buffer_size) return TQ_ERR_INVALID_ARG;
    if (in_dtype != TQ_F32 && in_dtype != TQ_BF16 && in_dtype != TQ_F16) return TQ_ERR_INVALID_ARG;
    if (n_ring == cfg->buffer_size) return TQ_ERR_RING_FULL;
    if (n_slices == 0) return TQ_OK;
    if (!ring || !ring->k || !ring->v || !aligned16(ring->k) || !aligned16(ring->v) || !k_new || !v_new ||
        !aligned16(k_new) || !aligned16(v_new))
        return TQ_ERR_INVALID_ARG;
    return hip_status(tq::launch_ring_append(cfg->head_dim, in_dtype, k_new, v_new, ring->k, ring->v, n_slices,
                                             cfg->buffer_size, n_ring, (hipStream_t)stream));
}

extern "C" tq_status tq_flush(const tq_config *cfg, const tq_tables *tables, const tq_ring *ring, int32_t n_slices,
                              int32_t n_ring, const tq_packed *dst, int64_t n_packed, void *stream) {
    if (!cfg) return TQ_ERR_INVALID_ARG;
    tq_status st = tq::check_config(*cfg);
    if (st != TQ_OK) return st;
    if (n_slices < 0 || n_ring < 0 || n_ring > cfg->buffer_size || n_packed < 0) return TQ_ERR_INVALID_ARG;
    if (n_slices == 0 || n_ring == 0) return TQ_OK;
    if (!ring || !ring->k || !ring->v || !aligned16(ring->k) || !aligned16(ring->v) || !tables_ok(tables) ||
        !packed_ok(dst))
        return TQ_ERR_INVALID_ARG;
    if (n_packed + n_ring > dst->capacity) return TQ_ERR_INVALID_ARG;
    tq::QuantArgs a{};
    a.k = ring->k;
    a.v = ring->v;
    a.in_slice_stride = (int64_t)cfg->buffer_size * cfg->head_dim;
    a.n_tokens = n_ring;
    a.n_rows = (int64_t)n_slices * n_ring;
    a.centroids = tables->centroids;
    a.boundaries = tables->boundaries;
    a.sign_bits = tables->sign_bits;
    a.S = tables->qjl_S;
    a.kw = dst->key_words;
    a.kn = dst->key_norms;
    a.vw = dst->val_words;
    a.vs = dst->val_scales;
    a.cap = dst->capacity;
    a.dst_offset = n_packed;
    set_pages(a, dst);
    return hip_status(tq::launch_quantize(cfg->head_dim, cfg->key_bits, cfg->value_bits, TQ_F16, a, (hipStream_t)stream));
}

extern "C" size_t tq_decode_workspace_bytes(const tq_config *cfg, int32_t batch, int32_t n_q_heads,
                                            int32_t n_kv_heads, int64_t max_context) {
    if (!cfg || tq::check_config(*cfg) != TQ_OK || batch <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 ||
        max_context < 0)
        return 0;
    if (n_q_heads % n_kv_heads != 0) return 0;
    const int64_t n_split =
        std::max(decode_splits(cfg->head_dim, cfg->value_bits, n_q_heads / n_kv_heads, (int64_t)batch * n_kv_heads,
                               max_context, 4, tq::decode_uses_any(cfg->head_dim, cfg->key_bits)),
                 ((int64_t)cfg->buffer_size + ring_per_split_max(cfg->head_dim) - 1) / ring_per_split_max(cfg->head_dim));
    return decode_layout(cfg->head_dim, cfg->key_bits, batch, n_q_heads, n_split).total;
}

namespace {
// decode over n_packed records and n_ring ring tokens; with k_new / v_new, ring slot
// n_ring - 1 is the new token, taken from them (and written into the ring) by the kernel
tq_status decode_impl(const tq_config *cfg, const tq_tables *tables, const void *q, tq_dtype q_dtype, int32_t batch,
                      int32_t n_q_heads, int32_t n_kv_heads, const tq_packed *packed, int64_t n_packed,
                      const tq_ring *ring, int32_t n_ring, float softmax_scale, float *out, void *workspace,
                      size_t workspace_bytes, void *stream, const void *k_new, const void *v_new, tq_dtype kv_dtype,
                      bool check_only = false, const int64_t *seq_packed = nullptr,
                      const int32_t *seq_ring = nullptr, int32_t q_tokens = 0, int64_t q_pos0 = 0,
                      int32_t causal = 0, int64_t q_slice0 = 0) {
    if (!cfg) return TQ_ERR_INVALID_ARG;
    tq_status st = tq::check_config(*cfg);
    if (st != TQ_OK) return st;
    if (batch <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads != 0 || n_packed < 0 ||
        n_ring < 0 || n_ring > cfg->buffer_size)
        return TQ_ERR_INVALID_ARG;
    if (q_dtype != TQ_F32 && q_dtype != TQ_BF16 && q_dtype != TQ_F16) return TQ_ERR_INVALID_ARG;
    const int G = n_q_heads / n_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8) return TQ_ERR_UNSUPPORTED;
    if ((int64_t)batch * n_kv_heads > 65535) return TQ_ERR_UNSUPPORTED;
    if (!tables_ok(tables) || !q || !out || !aligned16(q) || !aligned16(out) || !workspace || !aligned16(workspace))
        return TQ_ERR_INVALID_ARG;
    if (n_packed > 0 && (!packed_ok(packed) || n_packed > packed->capacity)) return TQ_ERR_INVALID_ARG;
    if (n_ring > 0 && (!ring || !ring->k || !ring->v || !aligned16(ring->k) || !aligned16(ring->v)))
        return TQ_ERR_INVALID_ARG;
    if (n_packed + n_ring >= kMaxContext) return TQ_ERR_UNSUPPORTED;  // 32-bit token indices in the kernels
    const int64_t slices = (int64_t)batch * n_kv_heads;
    // splits of the packed tokens, at least one (an empty context still writes its zeros), and
    // enough for the ring tokens at ring_per_split_max per split; the ring is spread evenly
    int64_t n_split = 1, per_split = 0;
    // (k_decode_any has 4-wave workgroups: its splits are planned for those)
    const bool any = tq::decode_uses_any(cfg->head_dim, cfg->key_bits);
    const int waves = n_packed > 0 && !any ? decode_waves(cfg->head_dim, G, slices, n_packed) : 4;
    if (n_packed > 0)
        split_shape(cfg->head_dim, cfg->value_bits, G, slices, n_packed, waves, any, n_split, per_split);
    const int64_t ring_splits = (n_ring + ring_per_split_max(cfg->head_dim) - 1) / ring_per_split_max(cfg->head_dim);
    if (ring_splits > n_split) {
        // more splits for the ring than for the packed tokens: spread the packed tokens too
        n_split = ring_splits;
        if (n_packed > 0) {
            per_split = (n_packed + n_split - 1) / n_split;
            per_split = (per_split + kSplitQuantum - 1) / kSplitQuantum * kSplitQuantum;
        }
    }
    const int64_t ring_per_split = (n_ring + n_split - 1) / n_split;
    const DecodeLayout L = decode_layout(cfg->head_dim, cfg->key_bits, batch, n_q_heads, n_split);
    if (workspace_bytes < L.total) return TQ_ERR_WORKSPACE;
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    if (check_only) return TQ_OK;
    tq::DecodeArgs a{};
    a.q = q;
    a.q_dtype = (int)q_dtype;
    a.centroids = tables->centroids;
    a.sign_bits = tables->sign_bits;
    a.S = tables->qjl_S;
    if (n_packed > 0) {
        a.kw = packed->key_words;
        a.kn = packed->key_norms;
        a.vw = packed->val_words;
        a.vs = packed->val_scales;
        a.cap = packed->capacity;
        set_pages(a, packed);
    }
    a.n_packed = n_packed;
    if (n_ring > 0) {
        a.rk = ring->k;
        a.rv = ring->v;
    }
    a.buffer_size = cfg->buffer_size;
    a.n_ring = n_ring;
    a.batch = batch;
    a.hq = n_q_heads;
    a.hkv = n_kv_heads;
    a.n_split = (int)n_split;
    a.ring_per_split = (int)ring_per_split;
    a.waves = waves;
    a.per_split = per_split;
    a.scale = softmax_scale;
    a.out = out;
    a.prep = reinterpret_cast<float *>(ws + L.prep);
    a.seq_packed = seq_packed;
    a.seq_ring = seq_ring;
    a.k_new = k_new;
    a.v_new = v_new;
    a.kv_dtype = (int)kv_dtype;
    a.new_slot = k_new ? n_ring - 1 : -1;
    a.q_tokens = q_tokens;
    a.q_pos0 = q_pos0;
    a.causal = causal;
    a.q_slice0 = q_slice0;
    a.partial = reinterpret_cast<float *>(ws + L.partial);
    a.partial_ml = reinterpret_cast<float *>(ws + L.partial_ml);
    return hip_status(tq::launch_decode(cfg->head_dim, cfg->key_bits, cfg->value_bits, G, a, (hipStream_t)stream));
}
}  // namespace

extern "C" tq_status tq_decode_attention(const tq_config *cfg, const tq_tables *tables, const void *q,
                                         tq_dtype q_dtype, int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                         const tq_packed *packed, int64_t n_packed, const tq_ring *ring,
                                         int32_t n_ring, float softmax_scale, float *out, void *workspace,
                                         size_t workspace_bytes, void *stream) {
    return decode_impl(cfg, tables, q, q_dtype, batch, n_q_heads, n_kv_heads, packed, n_packed, ring, n_ring,
                       softmax_scale, out, workspace, workspace_bytes, stream, nullptr, nullptr, TQ_F32);
}

extern "C" tq_status tq_decode_attention_ragged(const tq_config *cfg, const tq_tables *tables, const void *q,
                                                tq_dtype q_dtype, int32_t batch, int32_t n_q_heads,
                                                int32_t n_kv_heads, const tq_packed *packed,
                                                const int64_t *seq_packed, int64_t n_packed_max, const tq_ring *ring,
                                                const int32_t *seq_ring, int32_t n_ring_max, float softmax_scale,
                                                float *out, void *workspace, size_t workspace_bytes, void *stream) {
    if (!seq_packed || !seq_ring || !aligned8(seq_packed) || (reinterpret_cast<uintptr_t>(seq_ring) & 3u))
        return TQ_ERR_INVALID_ARG;
    return decode_impl(cfg, tables, q, q_dtype, batch, n_q_heads, n_kv_heads, packed, n_packed_max, ring, n_ring_max,
                       softmax_scale, out, workspace, workspace_bytes, stream, nullptr, nullptr, TQ_F32, false,
                       seq_packed, seq_ring);
}

// ------------------------------------------------------------------ prefill (full_tq)
namespace {
// query tokens per launch of a prefill call: batch * kv heads of a decode launch stays within
// the grid's 65535 rows, and it bounds the workspace of either path
int64_t prefill_launch_tokens(int32_t n_kv_heads) { return std::max<int64_t>(1, 65535 / n_kv_heads); }

// a launch of T query tokens per sequence goes to the tiled kernel when its rows (T G per kv
// head) fill at least half a tile; shorter ones (a few query tokens over a long history) to the
// decode kernels, whose splits spread one row's tokens over many workgroups
bool prefill_tiled(int d, int64_t T, int64_t G) { return T * G * 2 >= tq::prefill_tile_rows(d); }

// query tokens per launch of the tiled path (bounds its split partials)
int64_t prefill_tiled_launch_tokens(int32_t n_kv_heads) { return std::max<int64_t>(1, 65536 / n_kv_heads); }

// the tiled path's plan for n_seq sequences of T query tokens: tiles per (sequence, kv head)
// and the split of each tile's packed range (so that the workgroups cover the CUs; splits of
// whole blocks, at least 256 tokens each, at most 16 splits)
struct PrefillPlan {
    int tiles, n_split, per_split;
    size_t partial, partial_ml, total;  // workspace layout (bytes): split partials only
};
PrefillPlan prefill_plan(int d, int64_t n_seq, int64_t T, int64_t hq, int64_t hkv, int64_t n_packed) {
    PrefillPlan p{};
    const int64_t G = hq / hkv, tr = tq::prefill_tile_rows(d);
    p.tiles = (int)((T * G + tr - 1) / tr);
    const int64_t wg = n_seq * hkv * p.tiles, cus = tq::device_cus();
    const int64_t bt = tq::prefill_block_tokens(d), blocks = (n_packed + bt - 1) / bt;
    int64_t ns = wg < cus ? (cus + wg - 1) / wg : 1;
    ns = std::max<int64_t>(1, std::min<int64_t>({ns, 16, blocks * bt / 256}));
    p.n_split = (int)ns;
    p.per_split = (int)(((blocks + ns - 1) / ns) * bt);
    const int64_t rows = n_seq * T * hq;
    p.partial = 0;
    const size_t part = ns > 1 ? align256(sizeof(float) * (size_t)(rows * ns) * d) : 0;
    p.partial_ml = p.partial + part;
    p.total = std::max<size_t>(256, p.partial_ml + (ns > 1 ? align256(sizeof(float) * (size_t)(rows * ns) * 2) : 0));
    return p;
}

// prefill by query tiles: n_seq sequences of T query tokens at positions q_pos0 .., store
// slices slice0 ..; every argument checked before anything is launched
tq_status prefill_tiled_impl(const tq_config *cfg, const tq_tables *tables, const void *q, tq_dtype q_dtype,
                             int64_t n_seq, int32_t T, int32_t n_q_heads, int32_t n_kv_heads, const tq_packed *packed,
                             int64_t n_packed, int64_t q_pos0, int32_t causal, float softmax_scale, float *out,
                             void *workspace, size_t workspace_bytes, void *stream, bool check_only, int64_t slice0) {
    const int G = n_q_heads / n_kv_heads;
    if (n_q_heads % n_kv_heads != 0 || (G != 1 && G != 2 && G != 4 && G != 8)) return TQ_ERR_UNSUPPORTED;
    if (!tables_ok(tables) || !q || !out || !aligned16(q) || !aligned16(out) || !workspace || !aligned16(workspace))
        return TQ_ERR_INVALID_ARG;
    if (n_packed > 0 && (!packed_ok(packed) || n_packed > packed->capacity)) return TQ_ERR_INVALID_ARG;
    if (n_packed >= kMaxContext) return TQ_ERR_UNSUPPORTED;  // 32-bit token indices in the kernels
    const PrefillPlan plan = prefill_plan(cfg->head_dim, n_seq, T, n_q_heads, n_kv_heads, n_packed);
    if (workspace_bytes < plan.total) return TQ_ERR_WORKSPACE;
    if (check_only) return TQ_OK;
    const hipStream_t st = (hipStream_t)stream;
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    tq::PrefillArgs a{};
    a.q = q;
    a.q_dtype = (int)q_dtype;
    a.sign_bits = tables->sign_bits;
    a.S = tables->qjl_S;
    a.centroids = tables->centroids;
    if (n_packed > 0) {
        a.kw = packed->key_words;
        a.kn = packed->key_norms;
        a.vw = packed->val_words;
        a.vs = packed->val_scales;
        a.cap = packed->capacity;
        set_pages(a, packed);
    }
    a.n_packed = n_packed;
    a.q_pos0 = q_pos0;
    a.causal = causal;
    a.T = T;
    a.hq = n_q_heads;
    a.hkv = n_kv_heads;
    a.slice0 = slice0;
    a.tiles = plan.tiles;
    a.scale = softmax_scale;
    a.out = out;
    a.n_split = plan.n_split;
    a.per_split = plan.per_split;
    a.partial = reinterpret_cast<float *>(ws + plan.partial);
    a.partial_ml = reinterpret_cast<float *>(ws + plan.partial_ml);
    hipError_t e = tq::launch_prefill(cfg->head_dim, cfg->key_bits, cfg->value_bits, n_seq, a, st);
    if (e != hipSuccess || plan.n_split == 1) return hip_status(e);
    // the splits' partials of every row combined by the decode's merge (query token = batch
    // element of the decode's layout)
    tq::DecodeArgs m{};
    m.batch = (int)(n_seq * T);
    m.hq = n_q_heads;
    m.hkv = n_kv_heads;
    m.n_split = plan.n_split;
    m.out = out;
    m.partial = a.partial;
    m.partial_ml = a.partial_ml;
    return hip_status(tq::launch_decode_merge(cfg->head_dim, G, m, st));
}
}  // namespace

extern "C" size_t tq_prefill_workspace_bytes(const tq_config *cfg, int32_t batch, int32_t q_tokens,
                                             int32_t n_q_heads, int32_t n_kv_heads, int64_t n_packed) {
    if (!cfg || tq::check_config(*cfg) != TQ_OK || batch <= 0 || q_tokens <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 ||
        n_q_heads % n_kv_heads != 0 || n_packed < 0)
        return 0;
    if (prefill_tiled(cfg->head_dim, q_tokens, n_q_heads / n_kv_heads)) {
        // the launches' plans: whole sequences per launch, or chunks of one sequence
        const int64_t per = prefill_tiled_launch_tokens(n_kv_heads);
        const int64_t ns = q_tokens <= per ? std::min<int64_t>(batch, per / q_tokens) : 1;
        const int64_t T = std::min<int64_t>(q_tokens, per);
        size_t need = prefill_plan(cfg->head_dim, ns, T, n_q_heads, n_kv_heads, n_packed).total;
        if (q_tokens > per && q_tokens % per)  // the last chunk of a sequence
            need = std::max(need, prefill_plan(cfg->head_dim, 1, q_tokens % per, n_q_heads, n_kv_heads, n_packed).total);
        if (q_tokens <= per && batch % ns)     // the last launch's sequences
            need = std::max(need, prefill_plan(cfg->head_dim, batch % ns, q_tokens, n_q_heads, n_kv_heads, n_packed).total);
        return need;
    }
    const int64_t vb = std::min<int64_t>((int64_t)batch * q_tokens, prefill_launch_tokens(n_kv_heads));
    return tq_decode_workspace_bytes(cfg, (int32_t)vb, n_q_heads, n_kv_heads, n_packed);
}

extern "C" tq_status tq_prefill_attention(const tq_config *cfg, const tq_tables *tables, const void *q,
                                          tq_dtype q_dtype, int32_t batch, int32_t q_tokens, int32_t n_q_heads,
                                          int32_t n_kv_heads, const tq_packed *packed, int64_t n_packed,
                                          int64_t q_pos0, int32_t causal, float softmax_scale, float *out,
                                          void *workspace, size_t workspace_bytes, void *stream) {
    if (!cfg) return TQ_ERR_INVALID_ARG;
    tq_status st = tq::check_config(*cfg);
    if (st != TQ_OK) return st;
    if (batch <= 0 || q_tokens <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || n_packed < 0 || q_pos0 < 0 ||
        (causal != 0 && causal != 1) || !packed)
        return TQ_ERR_INVALID_ARG;
    if (q_dtype != TQ_F32 && q_dtype != TQ_BF16 && q_dtype != TQ_F16) return TQ_ERR_INVALID_ARG;
    if (n_q_heads % n_kv_heads != 0) return TQ_ERR_INVALID_ARG;
    const bool tiled = prefill_tiled(cfg->head_dim, q_tokens, n_q_heads / n_kv_heads);
    const int64_t per = tiled ? prefill_tiled_launch_tokens(n_kv_heads) : prefill_launch_tokens(n_kv_heads);
    const int64_t esz = q_dtype == TQ_F32 ? 4 : 2;
    const int64_t row = (int64_t)n_q_heads * cfg->head_dim;  // elements of one query token
    // the launches: whole sequences per launch while a sequence's tokens fit one launch,
    // else chunks of one sequence's tokens; every launch is checked before the first one
    for (int pass = 0; pass < 2; ++pass) {
        const bool check = pass == 0;
        if (q_tokens <= per) {
            const int64_t seqs = std::max<int64_t>(1, per / q_tokens);
            for (int64_t s0 = 0; s0 < batch; s0 += seqs) {
                const int64_t ns = std::min<int64_t>(seqs, batch - s0);
                const void *qs = static_cast<const char *>(q) + s0 * q_tokens * row * esz;
                if (tiled)
                    st = prefill_tiled_impl(cfg, tables, qs, q_dtype, ns, q_tokens, n_q_heads, n_kv_heads, packed,
                                            n_packed, q_pos0, causal, softmax_scale, out + s0 * q_tokens * row,
                                            workspace, workspace_bytes, stream, check, s0 * n_kv_heads);
                else
                    st = decode_impl(cfg, tables, qs, q_dtype, (int32_t)(ns * q_tokens), n_q_heads, n_kv_heads, packed,
                                     n_packed, nullptr, 0, softmax_scale, out + s0 * q_tokens * row, workspace,
                                     workspace_bytes, stream, nullptr, nullptr, TQ_F32, check, nullptr, nullptr,
                                     q_tokens, q_pos0, causal, s0 * n_kv_heads);
                if (st != TQ_OK) return st;
            }
        } else {
            for (int64_t s = 0; s < batch; ++s)
                for (int64_t i0 = 0; i0 < q_tokens; i0 += per) {
                    const int64_t c = std::min<int64_t>(per, q_tokens - i0);
                    const int64_t off = (s * q_tokens + i0) * row;
                    const void *qs = static_cast<const char *>(q) + off * esz;
                    if (tiled)
                        st = prefill_tiled_impl(cfg, tables, qs, q_dtype, 1, (int32_t)c, n_q_heads, n_kv_heads, packed,
                                                n_packed, q_pos0 + i0, causal, softmax_scale, out + off, workspace,
                                                workspace_bytes, stream, check, s * n_kv_heads);
                    else
                        st = decode_impl(cfg, tables, qs, q_dtype, (int32_t)c, n_q_heads, n_kv_heads, packed, n_packed,
                                         nullptr, 0, softmax_scale, out + off, workspace, workspace_bytes, stream,
                                         nullptr, nullptr, TQ_F32, check, nullptr, nullptr, (int32_t)c, q_pos0 + i0,
                                         causal, s * n_kv_heads);
                    if (st != TQ_OK) return st;
                }
        }
    }
    return TQ_OK;
}

extern "C" tq_status tq_decode_step(const tq_config *cfg, const tq_tables *tables, const void *q, tq_dtype q_dtype,
                                    int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, const tq_packed *packed,
                                    int64_t *n_packed, const tq_ring *ring, int32_t *n_ring, const void *k_new,
                                    const void *v_new, tq_dtype kv_dtype, float softmax_scale, float *out,
                                    void *workspace, size_t workspace_bytes, void *stream) {
    if (!cfg || !n_packed || !n_ring) return TQ_ERR_INVALID_ARG;
    tq_status st = tq::check_config(*cfg);
    if (st != TQ_OK) return st;
    if (kv_dtype != TQ_F32 && kv_dtype != TQ_BF16 && kv_dtype != TQ_F16) return TQ_ERR_INVALID_ARG;
    if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new) || !ring || !ring->k || !ring->v)
        return TQ_ERR_INVALID_ARG;
    if (batch <= 0 || n_kv_heads <= 0) return TQ_ERR_INVALID_ARG;
    int64_t np = *n_packed;
    int32_t nr = *n_ring;
    if (np < 0 || nr < 0 || nr > cfg->buffer_size) return TQ_ERR_INVALID_ARG;
    const int32_t slices = batch * n_kv_heads;
    const bool flush = nr == cfg->buffer_size;
    // every argument is checked before anything is launched
    st = decode_impl(cfg, tables, q, q_dtype, batch, n_q_heads, n_kv_heads, packed, flush ? np + nr : np, ring,
                     flush ? 1 : nr + 1, softmax_scale, out, workspace, workspace_bytes, stream, k_new, v_new,
                     kv_dtype, true);
    if (st != TQ_OK) return st;
    if (flush) {
        // a full ring is flushed into the packed store first (tq_flush checks its arguments
        // before it launches)
        st = tq_flush(cfg, tables, ring, slices, nr, packed, np, stream);
        if (st != TQ_OK) return st;
        np += nr;
        nr = 0;
    }
    st = decode_impl(cfg, tables, q, q_dtype, batch, n_q_heads, n_kv_heads, packed, np, ring, nr + 1, softmax_scale,
                     out, workspace, workspace_bytes, stream, k_new, v_new, kv_dtype);
    if (st != TQ_OK) return st;
    *n_packed = np;
    *n_ring = nr + 1;
    return TQ_OK;
}

// ------------------------------------------------------------------ decode without allocation
// The scratch of tq_decode_attention_noalloc: a file-scope device array (one copy per GPU, held
// until the process ends).  Host code never passes the array's name to a kernel (in host code it
// is only a stand-in for the symbol): the device address comes from hipGetSymbolAddress, taken
// once per device on the entry point's first call there, with that device current.
static __device__ __align__(256) unsigned char scratch[TQ_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
void *g_scratch_ptr[64];  // per device: device address of `scratch`

tq_status scratch_address(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TQ_ERR_HIP;
    if (dev < 0 || dev >= 64) return TQ_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TQ_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return TQ_OK;
}
}  // namespace

extern "C" tq_status tq_decode_attention_noalloc(const tq_config *cfg, const tq_tables *tables, const void *q,
                                                 tq_dtype q_dtype, int32_t batch, int32_t n_q_heads,
                                                 int32_t n_kv_heads, const tq_packed *packed, int64_t n_packed,
                                                 const tq_ring *ring, int32_t n_ring, float softmax_scale,
                                                 float *out, void *stream) {
    // every argument checked, and the scratch the call needs against the array's size, before
    // anything else (the check reads no scratch; a placeholder stands for its address).  The
    // decode's scratch needs no clearing: every byte it reads was written earlier in the call.
    void *const placeholder = reinterpret_cast<void *>(uintptr_t(256));
    tq_status st = decode_impl(cfg, tables, q, q_dtype, batch, n_q_heads, n_kv_heads, packed, n_packed, ring,
                               n_ring, softmax_scale, out, placeholder, TQ_NOALLOC_SCRATCH_BYTES, stream, nullptr,
                               nullptr, TQ_F32, true);
    if (st == TQ_ERR_WORKSPACE) return TQ_ERR_SCRATCH_LIMIT;
    if (st != TQ_OK) return st;
    void *ws = nullptr;
    st = scratch_address(&ws);
    if (st != TQ_OK) return st;
    return decode_impl(cfg, tables, q, q_dtype, batch, n_q_heads, n_kv_heads, packed, n_packed, ring, n_ring,
                       softmax_scale, out, ws, TQ_NOALLOC_SCRATCH_BYTES, stream, nullptr, nullptr, TQ_F32);
}

// ------------------------------------------------------------------ test hooks
extern "C" tq_status tq_rotate(const tq_config *cfg, const tq_tables *tables, const void *x, tq_dtype in_dtype,
                               int64_t n_rows, float *out, void *stream) {
    if (!cfg) return TQ_ERR_INVALID_ARG;
    tq_status st = tq::check_config(*cfg);
    if (st != TQ_OK) return st;
    if (!tables_ok(tables) || n_rows < 0 || (in_dtype != TQ_F32 && in_dtype != TQ_BF16 && in_dtype != TQ_F16))
        return TQ_ERR_INVALID_ARG;
    if (n_rows > 0 && (!x || !out || !aligned16(x) || !aligned16(out))) return TQ_ERR_INVALID_ARG;
    if ((n_rows + 3) / 4 > 0x7fffffff) return TQ_ERR_UNSUPPORTED;
    return hip_status(tq::launch_rotate(cfg->head_dim, tables->sign_bits, x, (int)in_dtype, n_rows, out,
                                        (hipStream_t)stream));
}

extern "C" tq_status tq_decode_scores(const tq_config *cfg, const tq_tables *tables, const void *q, tq_dtype q_dtype,
                                      int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, const tq_packed *packed,
                                      int64_t n_packed, const tq_ring *ring, int32_t n_ring, float *scores,
                                      void *stream) {
    if (!cfg) return TQ_ERR_INVALID_ARG;
    tq_status st = tq::check_config(*cfg);
    if (st != TQ_OK) return st;
    if (batch <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads != 0 || n_packed < 0 ||
        n_ring < 0 || n_ring > cfg->buffer_size)
        return TQ_ERR_INVALID_ARG;
    if (q_dtype != TQ_F32 && q_dtype != TQ_BF16 && q_dtype != TQ_F16) return TQ_ERR_INVALID_ARG;
    if ((int64_t)batch * n_q_heads > 65535) return TQ_ERR_UNSUPPORTED;
    if (!tables_ok(tables) || !q || !scores || !aligned16(q) || !aligned16(scores)) return TQ_ERR_INVALID_ARG;
    if (n_packed > 0 && (!packed_ok(packed) || n_packed > packed->capacity)) return TQ_ERR_INVALID_ARG;
    if (n_ring > 0 && (!ring || !ring->k || !aligned16(ring->k))) return TQ_ERR_INVALID_ARG;
    if (n_packed + n_ring >= kMaxContext) return TQ_ERR_UNSUPPORTED;
    tq::ScoreArgs a{};
    a.q = q;
    a.q_dtype = (int)q_dtype;
    a.batch = batch;
    a.hq = n_q_heads;
    a.hkv = n_kv_heads;
    if (n_packed > 0) {
        a.kw = packed->key_words;
        a.kn = packed->key_norms;
        a.cap = packed->capacity;
        a.bt = packed->block_table;
        a.pt = packed->block_table ? packed->page_tokens : 1;
        a.pps = packed->block_table ? packed->pages_per_slice : 0;
        a.n_pages = packed->block_table ? packed->n_pages : 0;
        a.err = packed->block_table ? packed->error_flag : nullptr;
    }
    a.n_packed = n_packed;
    a.rk = n_ring > 0 ? ring->k : nullptr;
    a.buffer_size = cfg->buffer_size;
    a.n_ring = n_ring;
    a.kb = cfg->key_bits;
    a.centroids = tables->centroids;
    a.sign_bits = tables->sign_bits;
    a.S = tables->qjl_S;
    a.scores = scores;
    return hip_status(tq::launch_scores(cfg->head_dim, a, (hipStream_t)stream));
}

// ------------------------------------------------------------------ KIVI 2-bit variant
namespace {

bool kivi_dim_ok(int32_t d) { return d == 64 || d == 128 || d == 256; }

bool kivi_store_ok(const tq_kivi_store *s) {
    return s && s->key_codes && s->key_scale && s->key_zero && s->val_codes && s->val_params && s->capacity >= 0 &&
           s->capacity % 32 == 0 && aligned16(s->key_codes) && aligned16(s->key_scale) && aligned16(s->key_zero) &&
           aligned16(s->val_codes) && aligned16(s->val_params);
}

// splits of a KIVI decode: four 4-wave workgroups per CU, 64-token chunks per wave, whole
// chunks per split
void kivi_split_shape(int64_t slices, int64_t n_packed, int64_t &n_split, int64_t &per_split) {
    const int64_t want = std::max<int64_t>(1, ((int64_t)tq::device_cus() * 4 + slices - 1) / slices);
    const int64_t by_tokens = std::max<int64_t>(1, (n_packed + 255) / 256);  // a chunk for each wave
    n_split = std::min({want, by_tokens, kMaxSplits});
    per_split = (n_packed + n_split - 1) / n_split;
    per_split = std::max<int64_t>(64, (per_split + 63) / 64 * 64);
    n_split = std::max<int64_t>(1, (n_packed + per_split - 1) / per_split);
}

size_t kivi_ws_bytes(int64_t slices, int64_t G, int64_t d, int64_t n_split) {
    const size_t po = align256(sizeof(float) * (size_t)(slices * n_split * G * d));
    return std::max<size_t>(256, po + align256(sizeof(float) * (size_t)(slices * n_split * G * 2)));
}

}  // namespace

extern "C" size_t tq_kivi_bytes_per_token(int32_t head_dim) {
    if (!kivi_dim_ok(head_dim)) return 0;
    return (size_t)head_dim / 4 + (size_t)head_dim / 8 + (size_t)head_dim / 4 + 4;
}

extern "C" tq_status tq_kivi_quantize(int32_t head_dim, const void *k, const void *v, tq_dtype in_dtype,
                                      int32_t n_slices, int64_t n_tokens, const tq_kivi_store *dst, int64_t dst_token0,
                                      void *stream) {
    if (!kivi_dim_ok(head_dim)) return TQ_ERR_UNSUPPORTED;
    if (in_dtype != TQ_F32 && in_dtype != TQ_BF16 && in_dtype != TQ_F16) return TQ_ERR_INVALID_ARG;
    if (n_slices <= 0 || n_tokens < 0 || n_tokens % 32 != 0 || dst_token0 < 0 || dst_token0 % 32 != 0)
        return TQ_ERR_INVALID_ARG;
    if (!kivi_store_ok(dst) || dst_token0 + n_tokens > dst->capacity) return TQ_ERR_INVALID_ARG;
    if (n_tokens == 0) return TQ_OK;
    if (!k || !v || !aligned16(k) || !aligned16(v)) return TQ_ERR_INVALID_ARG;
    if ((int64_t)n_slices * (n_tokens / 32) > 0x7fffffff) return TQ_ERR_UNSUPPORTED;
    return hip_status(tq::launch_kivi_quantize(head_dim, in_dtype, k, v, n_slices, n_tokens, *dst, dst_token0,
                                               (hipStream_t)stream));
}

extern "C" size_t tq_kivi_decode_workspace_bytes(int32_t head_dim, int32_t batch, int32_t n_q_heads,
                                                 int32_t n_kv_heads, int64_t max_context) {
    if (!kivi_dim_ok(head_dim) || batch <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads != 0 ||
        max_context < 0)
        return 0;
    const int64_t slices = (int64_t)batch * n_kv_heads, G = n_q_heads / n_kv_heads;
    int64_t n_split, per_split;
    kivi_split_shape(slices, max_context, n_split, per_split);
    return kivi_ws_bytes(slices, G, head_dim, n_split);
}

extern "C" tq_status tq_kivi_decode_attention(int32_t head_dim, const void *q, tq_dtype q_dtype, int32_t batch,
                                              int32_t n_q_heads, int32_t n_kv_heads, const tq_kivi_store *src,
                                              int64_t n_packed, float softmax_scale, float *out, void *workspace,
                                              size_t workspace_bytes, void *stream) {
    if (!kivi_dim_ok(head_dim)) return TQ_ERR_UNSUPPORTED;
    if (batch <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads != 0 || n_packed < 0)
        return TQ_ERR_INVALID_ARG;
    if (q_dtype != TQ_F32 && q_dtype != TQ_BF16 && q_dtype != TQ_F16) return TQ_ERR_INVALID_ARG;
    const int G = n_q_heads / n_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8) return TQ_ERR_UNSUPPORTED;
    if ((int64_t)batch * n_kv_heads > 65535) return TQ_ERR_UNSUPPORTED;
    if (!q || !out || !aligned16(q) || !aligned16(out) || !workspace || !aligned16(workspace))
        return TQ_ERR_INVALID_ARG;
    if (!kivi_store_ok(src) || n_packed > src->capacity) return TQ_ERR_INVALID_ARG;
    if (n_packed >= kMaxContext) return TQ_ERR_UNSUPPORTED;
    const int64_t slices = (int64_t)batch * n_kv_heads;
    int64_t n_split, per_split;
    kivi_split_shape(slices, n_packed, n_split, per_split);
    const size_t need = kivi_ws_bytes(slices, G, head_dim, n_split);
    if (workspace_bytes < need) return TQ_ERR_WORKSPACE;
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    tq::DecodeArgs a{};
    a.q = q;
    a.q_dtype = (int)q_dtype;
    a.batch = batch;
    a.hq = n_q_heads;
    a.hkv = n_kv_heads;
    a.n_packed = n_packed;
    a.n_split = (int)n_split;
    a.per_split = per_split;
    a.scale = softmax_scale;
    a.out = out;
    a.partial = reinterpret_cast<float *>(ws);
    a.partial_ml = reinterpret_cast<float *>(ws + align256(sizeof(float) * (size_t)(slices * n_split * G * head_dim)));
    return hip_status(tq::launch_kivi_decode(head_dim, G, a, *src, (hipStream_t)stream));
}

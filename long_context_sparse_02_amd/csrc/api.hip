// C ABI of libgsa (declared in include/gsa.h): host-side argument checks,
// then launches on the caller's stream. Nothing here allocates, frees or
// synchronises; no C++ exception crosses the boundary.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "../../include/gsa.h"
#include "launch.h"

namespace {

thread_local char g_err[512] = "";

gsa_status fail(gsa_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

gsa_status hip_result(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(GSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    g_err[0] = 0;
    return GSA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define REQUIRE(cond, ...) \
    do { if (!(cond)) return fail(GSA_ERR_INVALID_ARG, __VA_ARGS__); } while (0)
#define REQUIRE_PTR(p) \
    do { if ((p) == nullptr) return fail(GSA_ERR_INVALID_ARG, "%s is NULL", #p); \
         if (!aligned16(p)) return fail(GSA_ERR_INVALID_ARG, "%s is not 16-byte aligned", #p); } while (0)

constexpr int kMaxGridY = 65535;

// with_scores = false: the indexer inputs only (the path without a score buffer)
gsa_status check_score(gsa_dtype dt, const void* q, const float* qs, const float* w, const void* k,
                       const float* ks, const int32_t* q_seq, const int32_t* q_pos, int n_q,
                       int batch, int64_t n_cap, const float* scores, int64_t ld, bool with_scores = true) {
    if (dt != GSA_BF16 && dt != GSA_FP8_E4M3) return fail(GSA_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
    REQUIRE_PTR(q); REQUIRE_PTR(w); REQUIRE_PTR(k); REQUIRE_PTR(q_seq); REQUIRE_PTR(q_pos);
    if (with_scores) REQUIRE_PTR(scores);
    if (dt == GSA_FP8_E4M3) { REQUIRE_PTR(qs); REQUIRE_PTR(ks); }
    REQUIRE(n_q >= 1, "n_q must be >= 1 (got %d)", n_q);
    REQUIRE(batch >= 1, "batch must be >= 1 (got %d)", batch);
    REQUIRE(n_cap >= 1 && n_cap <= 0x7fffffff, "n_cap must be in [1, 2^31-1] (got %lld)", (long long)n_cap);
    if (with_scores) {
        REQUIRE(ld >= n_cap, "ld_scores (%lld) must be >= n_cap (%lld)", (long long)ld, (long long)n_cap);
        REQUIRE(ld % 4 == 0, "ld_scores must be a multiple of 4 (got %lld)", (long long)ld);
    }
    if (n_q > kMaxGridY) return fail(GSA_ERR_UNSUPPORTED, "n_q must be <= %d (got %d)", kMaxGridY, n_q);
    return GSA_OK;
}

gsa_status check_topk(const float* scores, int64_t ld, const int32_t* q_pos, int n_q, int k,
                      const int32_t* idx, const void* ws, size_t ws_bytes) {
    REQUIRE_PTR(scores); REQUIRE_PTR(q_pos); REQUIRE_PTR(idx);
    REQUIRE(n_q >= 1, "n_q must be >= 1 (got %d)", n_q);
    if (n_q > kMaxGridY) return fail(GSA_ERR_UNSUPPORTED, "n_q must be <= %d (got %d)", kMaxGridY, n_q);
    if (k != GSA_TOPK) return fail(GSA_ERR_UNSUPPORTED, "k must be %d (got %d)", GSA_TOPK, k);
    REQUIRE(ld >= 1 && ld % 4 == 0, "ld_scores must be a positive multiple of 4 (got %lld)", (long long)ld);
    if (ld > ((int64_t)1 << 23))
        return fail(GSA_ERR_UNSUPPORTED, "ld_scores must be <= 2^23 (got %lld)", (long long)ld);
    const size_t need = gsa::topk_workspace_bytes(n_q, ld, k);
    if (ws == nullptr || ws_bytes < need)
        return fail(GSA_ERR_WORKSPACE, "top-k workspace needs %zu bytes (got %zu%s)", need, ws_bytes,
                    ws == nullptr ? ", NULL" : "");
    REQUIRE(aligned16(ws), "workspace is not 16-byte aligned");
    return GSA_OK;
}

// The selection without a score buffer (after check_score without scores).
gsa_status check_indexer_topk(int n_q, int64_t n_cap, int k, const int32_t* idx, const void* ws,
                              size_t ws_bytes) {
    REQUIRE_PTR(idx);
    if (k != GSA_TOPK) return fail(GSA_ERR_UNSUPPORTED, "k must be %d (got %d)", GSA_TOPK, k);
    const int64_t ld = gsa::indexer_topk_ld(n_cap);
    if (ld > ((int64_t)1 << 23))
        return fail(GSA_ERR_UNSUPPORTED, "n_cap must be <= 2^23 (got %lld)", (long long)n_cap);
    const size_t need = gsa::topk_workspace_bytes(n_q, ld, k);
    if (ws == nullptr || ws_bytes < need)
        return fail(GSA_ERR_WORKSPACE, "indexer top-k workspace needs %zu bytes (got %zu%s)", need, ws_bytes,
                    ws == nullptr ? ", NULL" : "");
    REQUIRE(aligned16(ws), "workspace is not 16-byte aligned");
    return GSA_OK;
}

// One attention layer's checks; the workspace must serve n_layers layers launched together.
gsa_status check_mla(const void* q_lat, const void* q_rope, const void* kv, const int32_t* q_seq,
                     const int32_t* idx, int k, int n_q, int n_heads, int batch, int64_t n_cap,
                     float scale, const float* out, const float* lse, const void* ws, size_t ws_bytes,
                     int n_layers) {
    REQUIRE_PTR(q_lat); REQUIRE_PTR(q_rope); REQUIRE_PTR(kv); REQUIRE_PTR(q_seq); REQUIRE_PTR(idx);
    REQUIRE_PTR(out);
    if (lse != nullptr) REQUIRE(aligned16(lse), "lse is not 16-byte aligned");
    REQUIRE(n_q >= 1, "n_q must be >= 1 (got %d)", n_q);
    if (n_q > kMaxGridY) return fail(GSA_ERR_UNSUPPORTED, "n_q must be <= %d (got %d)", kMaxGridY, n_q);
    REQUIRE(batch >= 1, "batch must be >= 1 (got %d)", batch);
    REQUIRE(n_cap >= 1 && n_cap <= 0x7fffffff, "n_cap must be in [1, 2^31-1] (got %lld)", (long long)n_cap);
    if (n_heads != 64) return fail(GSA_ERR_UNSUPPORTED, "n_heads must be 64 (got %d)", n_heads);
    if (k != GSA_TOPK) return fail(GSA_ERR_UNSUPPORTED, "k must be %d (got %d)", GSA_TOPK, k);
    REQUIRE(scale > 0.f && scale < 1e30f, "scale must be positive and finite");
    const size_t need = gsa::mla_workspace_bytes(n_q, n_heads, k, n_layers);
    if (need > 0 && (ws == nullptr || ws_bytes < need))
        return fail(GSA_ERR_WORKSPACE, "attention workspace needs %zu bytes (got %zu)", need, ws_bytes);
    if (need > 0) REQUIRE(aligned16(ws), "workspace is not 16-byte aligned");
    return GSA_OK;
}

// Host checks of a paged-cache description; *n_cap = positions a sequence can hold.
gsa_status check_paged(const gsa_paged_kv* pg, int64_t* n_cap) {
    REQUIRE(pg != nullptr, "paged_kv is NULL");
    REQUIRE_PTR(pg->block_table_dev);
    REQUIRE(pg->page_size >= 1, "page_size must be >= 1 (got %d)", pg->page_size);
    REQUIRE(pg->max_pages >= 1, "max_pages must be >= 1 (got %d)", pg->max_pages);
    REQUIRE(pg->n_pages >= 1, "n_pages must be >= 1");
    REQUIRE(pg->n_pages * (int64_t)pg->page_size <= 0x7fffffff, "a pool must hold < 2^31 rows");
    REQUIRE((int64_t)pg->max_pages * pg->page_size <= 0x7fffffff, "a sequence must hold < 2^31 positions");
    *n_cap = (int64_t)pg->max_pages * pg->page_size;
    return GSA_OK;
}

// Attention for layers that share one index buffer, in one launch per 8 layers.
gsa_status enqueue_attention(const gsa_mla_layer* layers, int n_layers, const int32_t* q_seq,
                             const int32_t* idx, int k, int n_q, int n_heads, int64_t n_cap,
                             const gsa_paged_kv* paged, bool fp8_kv, float scale, void* ws,
                             hipStream_t s) {
    gsa::MlaLayerPtrs ptrs[8];
    for (int l0 = 0; l0 < n_layers; l0 += 8) {
        const int nl = n_layers - l0 < 8 ? n_layers - l0 : 8;
        for (int i = 0; i < nl; ++i)
            ptrs[i] = {layers[l0 + i].q_lat_dev, layers[l0 + i].q_rope_dev, layers[l0 + i].kv_dev,
                       layers[l0 + i].out_dev, layers[l0 + i].lse_dev};
        // the workspace was sized for n_layers; a later launch of fewer layers needs no more
        const hipError_t e = gsa::launch_sparse_mla_layers(
            ptrs, nl, q_seq, idx, k, n_q, n_heads, n_cap, paged ? paged->block_table_dev : nullptr,
            paged ? paged->page_size : 0, paged ? paged->max_pages : 0, fp8_kv, scale, ws, s);
        if (e != hipSuccess) return hip_result(e, "sparse_mla_attn");
    }
    g_err[0] = 0;
    return GSA_OK;
}

}  // namespace

extern "C" {

const char* gsa_status_string(gsa_status s) {
    switch (s) {
        case GSA_OK: return "GSA_OK";
        case GSA_ERR_INVALID_ARG: return "GSA_ERR_INVALID_ARG";
        case GSA_ERR_UNSUPPORTED: return "GSA_ERR_UNSUPPORTED";
        case GSA_ERR_WORKSPACE: return "GSA_ERR_WORKSPACE";
        case GSA_ERR_HIP: return "GSA_ERR_HIP";
        case GSA_ERR_STALE_INDEX: return "GSA_ERR_STALE_INDEX";
    }
    return "GSA_ERR_UNKNOWN";
}

const char* gsa_last_error(void) { return g_err; }

const char* gsa_version(void) { return "gsa 0.2 gfx950"; }

gsa_status gsa_quantize_e4m3(const void* x, int64_t n_blocks, uint8_t* codes, float* scales,
                             void* stream) {
    REQUIRE_PTR(x); REQUIRE_PTR(codes); REQUIRE_PTR(scales);
    REQUIRE(n_blocks >= 0, "n_blocks must be >= 0");
    return hip_result(gsa::launch_quantize_e4m3(x, n_blocks, codes, scales, false, (hipStream_t)stream),
                      "quantize_e4m3");
}

gsa_status gsa_quantize_e4m3_hadamard(const void* x, int64_t n_blocks, uint8_t* codes, float* scales,
                                      void* stream) {
    REQUIRE_PTR(x); REQUIRE_PTR(codes); REQUIRE_PTR(scales);
    REQUIRE(n_blocks >= 0, "n_blocks must be >= 0");
    return hip_result(gsa::launch_quantize_e4m3(x, n_blocks, codes, scales, true, (hipStream_t)stream),
                      "quantize_e4m3_hadamard");
}

gsa_status gsa_indexer_score(gsa_dtype dt, const void* q, const float* q_scale, const float* w,
                             const void* k, const float* k_scale, const int32_t* q_seq,
                             const int32_t* q_pos, int n_q, int batch, int64_t n_cap,
                             float* scores, int64_t ld, float* group_max, void* stream) {
    gsa_status st = check_score(dt, q, q_scale, w, k, k_scale, q_seq, q_pos, n_q, batch, n_cap, scores, ld);
    if (st != GSA_OK) return st;
    return hip_result(gsa::launch_indexer_score(dt == GSA_FP8_E4M3, q, q_scale, w, k, k_scale, q_seq,
                                                q_pos, n_q, batch, n_cap, scores, ld, group_max,
                                                (hipStream_t)stream),
                      "indexer_score");
}

size_t gsa_indexer_topk_workspace_bytes(int n_q, int64_t n_cap, int k) {
    if (n_q < 1 || n_cap < 1) return 0;
    return gsa::topk_workspace_bytes(n_q, gsa::indexer_topk_ld(n_cap), k);
}

gsa_status gsa_indexer_topk(gsa_dtype dt, const void* q, const float* q_scale, const float* w,
                            const void* k, const float* k_scale, const int32_t* q_seq,
                            const int32_t* q_pos, int n_q, int batch, int64_t n_cap, int k_sel,
                            int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
    gsa_status st = check_score(dt, q, q_scale, w, k, k_scale, q_seq, q_pos, n_q, batch, n_cap, nullptr, 0,
                                false);
    if (st != GSA_OK) return st;
    st = check_indexer_topk(n_q, n_cap, k_sel, idx, ws, ws_bytes);
    if (st != GSA_OK) return st;
    return hip_result(gsa::launch_indexer_topk(dt == GSA_FP8_E4M3, q, q_scale, w, k, k_scale, q_seq, q_pos,
                                               n_q, batch, n_cap, k_sel, idx, ws, (hipStream_t)stream),
                      "indexer_topk");
}

int64_t gsa_group_max_ld(int64_t ld) { return ld < 1 ? 0 : gsa::group_max_ld(ld); }

size_t gsa_topk_workspace_bytes(int n_q, int64_t ld, int k) {
    if (n_q < 1 || ld < 1) return 0;
    return gsa::topk_workspace_bytes(n_q, ld, k);
}

gsa_status gsa_topk(const float* scores, int64_t ld, const int32_t* q_pos, int n_q, int k,
                    const float* group_max, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
    gsa_status st = check_topk(scores, ld, q_pos, n_q, k, idx, ws, ws_bytes);
    if (st != GSA_OK) return st;
    return hip_result(gsa::launch_topk(scores, ld, q_pos, n_q, k, group_max, idx, ws, (hipStream_t)stream),
                      "topk");
}

size_t gsa_mla_workspace_bytes(int n_q, int n_heads, int k) {
    return gsa_mla_layers_workspace_bytes(n_q, n_heads, k, 1);
}

size_t gsa_mla_layers_workspace_bytes(int n_q, int n_heads, int k, int n_layers) {
    if (n_q < 1 || n_heads != 64 || k != GSA_TOPK || n_layers < 1) return 0;
    return gsa::mla_workspace_bytes(n_q, n_heads, k, n_layers);
}

gsa_status gsa_sparse_mla_attn(const void* q_lat, const void* q_rope, const void* kv,
                               const int32_t* q_seq, const int32_t* idx, int k, int n_q, int n_heads,
                               int batch, int64_t n_cap, float scale, float* out, float* lse,
                               void* ws, size_t ws_bytes, void* stream) {
    const gsa_mla_layer layer = {q_lat, q_rope, kv, out, lse};
    return gsa_sparse_mla_attn_layers(&layer, 1, q_seq, idx, k, n_q, n_heads, batch, n_cap, scale, ws,
                                      ws_bytes, stream);
}

gsa_status gsa_sparse_mla_attn_layers(const gsa_mla_layer* layers, int n_layers, const int32_t* q_seq,
                                      const int32_t* idx, int k, int n_q, int n_heads, int batch,
                                      int64_t n_cap, float scale, void* ws, size_t ws_bytes,
                                      void* stream) {
    REQUIRE(n_layers >= 1, "n_layers must be >= 1 (got %d)", n_layers);
    REQUIRE(layers != nullptr, "layers is NULL");
    for (int l = 0; l < n_layers; ++l) {
        const gsa_status st = check_mla(layers[l].q_lat_dev, layers[l].q_rope_dev, layers[l].kv_dev, q_seq,
                                        idx, k, n_q, n_heads, batch, n_cap, scale, layers[l].out_dev,
                                        layers[l].lse_dev, ws, ws_bytes, n_layers);
        if (st != GSA_OK) {
            if (n_layers > 1) {
                char tmp[512];
                snprintf(tmp, sizeof(tmp), "layer %d: %s", l, g_err);
                snprintf(g_err, sizeof(g_err), "%s", tmp);
            }
            return st;
        }
    }
    return enqueue_attention(layers, n_layers, q_seq, idx, k, n_q, n_heads, n_cap, nullptr, false, scale, ws,
                             (hipStream_t)stream);
}

}  // extern "C"

namespace {

// Checks and enqueues attention over paged (paged_kv) or contiguous (n_cap)
// caches of bf16 or FP8 latent rows.
gsa_status attention_call(const gsa_mla_layer* layers, int n_layers, const gsa_paged_kv* paged_kv,
                          bool fp8_kv, const int32_t* q_seq, const int32_t* idx, int k, int n_q,
                          int n_heads, int batch, int64_t n_cap, float scale, void* ws, size_t ws_bytes,
                          void* stream) {
    gsa_status st;
    if (paged_kv != nullptr) {
        st = check_paged(paged_kv, &n_cap);
        if (st != GSA_OK) return st;
    }
    REQUIRE(n_layers >= 1, "n_layers must be >= 1 (got %d)", n_layers);
    REQUIRE(layers != nullptr, "layers is NULL");
    for (int l = 0; l < n_layers; ++l) {
        st = check_mla(layers[l].q_lat_dev, layers[l].q_rope_dev, layers[l].kv_dev, q_seq, idx, k, n_q,
                       n_heads, batch, n_cap, scale, layers[l].out_dev, layers[l].lse_dev, ws, ws_bytes,
                       n_layers);
        if (st != GSA_OK) return st;
    }
    return enqueue_attention(layers, n_layers, q_seq, idx, k, n_q, n_heads, n_cap, paged_kv, fp8_kv, scale, ws,
                             (hipStream_t)stream);
}

}  // namespace

extern "C" {

gsa_status gsa_sparse_mla_attn_paged(const gsa_mla_layer* layers, int n_layers, const gsa_paged_kv* paged_kv,
                                     const int32_t* q_seq, const int32_t* idx, int k, int n_q, int n_heads,
                                     int batch, float scale, void* ws, size_t ws_bytes, void* stream) {
    if (paged_kv == nullptr) return fail(GSA_ERR_INVALID_ARG, "paged_kv is NULL");
    return attention_call(layers, n_layers, paged_kv, false, q_seq, idx, k, n_q, n_heads, batch, 0, scale, ws,
                          ws_bytes, stream);
}

gsa_status gsa_sparse_mla_attn_fp8kv(const gsa_mla_layer* layers, int n_layers, const gsa_paged_kv* paged_kv,
                                     const int32_t* q_seq, const int32_t* idx, int k, int n_q, int n_heads,
                                     int batch, int64_t n_cap, float scale, void* ws, size_t ws_bytes,
                                     void* stream) {
    return attention_call(layers, n_layers, paged_kv, true, q_seq, idx, k, n_q, n_heads, batch,
                          paged_kv != nullptr ? 0 : n_cap, scale, ws, ws_bytes, stream);
}

gsa_status gsa_quantize_latent_fp8(const void* rows, int64_t n_rows, uint8_t* out, void* stream) {
    REQUIRE_PTR(rows); REQUIRE_PTR(out);
    REQUIRE(n_rows >= 0, "n_rows must be >= 0");
    return hip_result(gsa::launch_quantize_latent(rows, n_rows, out, (hipStream_t)stream), "quantize_latent_fp8");
}

size_t gsa_group_workspace_bytes(int n_q, int64_t ld, int k, int n_heads, int n_layers) {
    const size_t a = gsa_topk_workspace_bytes(n_q, ld, k);
    const size_t b = gsa_mla_layers_workspace_bytes(n_q, n_heads, k, n_layers);
    return a > b ? a : b;     // top-k finishes (stream order) before attention reuses the space
}

size_t gsa_stack_workspace_bytes(int n_q, int64_t ld, int k, int n_heads, int n_layers) {
    size_t need = 0;
    for (int i = 0; i < n_layers; ++i) {                   // every group: a full layer + the shared after it
        if (!(i < 3 || i % 4 == 2)) continue;
        int len = 1;
        while (i + len < n_layers && !(i + len < 3 || (i + len) % 4 == 2)) ++len;
        const size_t g = gsa_group_workspace_bytes(n_q, ld, k, n_heads, len);
        need = g > need ? g : need;
    }
    return need;
}

}  // extern "C"

namespace {

// ---- The group call without a workspace argument ------------------------------
// Its workspace is this file-scope device array: every GPU the library runs on
// holds its own copy (at its own address) until the process ends. Host code must
// not pass the array's name to a kernel (on the host it is a stand-in, not a
// device address): the address of the current device's copy is taken once per
// device with hipGetSymbolAddress and used instead.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up on the first call on that device).
gsa_status scratch_for_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(GSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(GSA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(GSA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return GSA_OK;
}

// Host-side checks of one group; enqueues nothing.
gsa_status validate_group(const gsa_group_desc* d) {
    if (d == nullptr) return fail(GSA_ERR_INVALID_ARG, "desc is NULL");
    REQUIRE_PTR(d->index_buf_dev); REQUIRE_PTR(d->q_seq_dev);
    REQUIRE(d->n_layers >= 0, "n_layers must be >= 0");
    REQUIRE(d->n_layers == 0 || d->layers != nullptr, "layers is NULL");
    REQUIRE(d->compute_index == 0 || d->compute_index == 1, "compute_index must be 0 or 1");
    REQUIRE(d->kv_dt == GSA_BF16 || d->kv_dt == GSA_FP8_E4M3, "kv_dt must be GSA_BF16 or GSA_FP8_E4M3");
    if (d->paged_kv != nullptr) {
        int64_t n_cap_pg = 0;
        const gsa_status st = check_paged(d->paged_kv, &n_cap_pg);
        if (st != GSA_OK) return st;
        REQUIRE(n_cap_pg >= d->n_cap, "paged_kv holds %lld positions per sequence, fewer than n_cap %lld",
                (long long)n_cap_pg, (long long)d->n_cap);
    }
    REQUIRE(d->index_epoch == 0 || d->index_tag != nullptr, "index_epoch is set but index_tag is NULL");
    if (!d->compute_index && d->index_epoch != 0) {
        // the buffer must hold what this call names (Serving §10: a reused index
        // cache is valid only for the prefix, positions and revision it was made for)
        const gsa_index_tag& t = *d->index_tag;
        if (t.epoch != d->index_epoch || t.index_buf_dev != d->index_buf_dev || t.full_layer != d->index_layer ||
            t.n_q != d->n_q || t.k != d->k || t.n_cap > d->n_cap)
            return fail(GSA_ERR_STALE_INDEX,
                        "index buffer %p holds epoch %llu, full layer %d, n_q %d, k %d, n_cap %lld; the call "
                        "names buffer %p, epoch %llu, full layer %d, n_q %d, k %d, n_cap %lld",
                        (const void*)t.index_buf_dev, (unsigned long long)t.epoch, t.full_layer, t.n_q, t.k,
                        (long long)t.n_cap, (const void*)d->index_buf_dev, (unsigned long long)d->index_epoch,
                        d->index_layer, d->n_q, d->k, (long long)d->n_cap);
    }
    if (d->compute_index) {
        const bool buffered = d->scores_dev != nullptr;        // else: selection without a score buffer
        gsa_status st = check_score(d->dt, d->q_idx_dev, d->q_scale_dev, d->w_dev, d->k_idx_dev,
                                    d->k_scale_dev, d->q_seq_dev, d->q_pos_dev, d->n_q, d->batch,
                                    d->n_cap, d->scores_dev, d->ld_scores, buffered);
        if (st != GSA_OK) return st;
        st = buffered ? check_topk(d->scores_dev, d->ld_scores, d->q_pos_dev, d->n_q, d->k, d->index_buf_dev,
                                   d->workspace_dev, d->workspace_bytes)
                      : check_indexer_topk(d->n_q, d->n_cap, d->k, d->index_buf_dev, d->workspace_dev,
                                           d->workspace_bytes);
        if (st != GSA_OK) return st;
    }
    for (int l = 0; l < d->n_layers; ++l) {
        const gsa_mla_layer& L = d->layers[l];
        gsa_status st = check_mla(L.q_lat_dev, L.q_rope_dev, L.kv_dev, d->q_seq_dev, d->index_buf_dev,
                                  d->k, d->n_q, d->n_heads, d->batch, d->n_cap, d->scale, L.out_dev,
                                  L.lse_dev, d->workspace_dev, d->workspace_bytes, d->n_layers);
        if (st != GSA_OK) {
            char tmp[512];
            snprintf(tmp, sizeof(tmp), "layer %d: %s", l, g_err);
            snprintf(g_err, sizeof(g_err), "%s", tmp);
            return st;
        }
    }
    return GSA_OK;
}

// Enqueues a validated group: score -> top-k (F layer) -> attention per layer.
gsa_status enqueue_group(const gsa_group_desc* d, hipStream_t s) {
    if (d->compute_index && d->scores_dev == nullptr) {
        const hipError_t e = gsa::launch_indexer_topk(d->dt == GSA_FP8_E4M3, d->q_idx_dev, d->q_scale_dev,
                                                      d->w_dev, d->k_idx_dev, d->k_scale_dev, d->q_seq_dev,
                                                      d->q_pos_dev, d->n_q, d->batch, d->n_cap, d->k,
                                                      d->index_buf_dev, d->workspace_dev, s);
        if (e != hipSuccess) return hip_result(e, "group: indexer_topk");
    } else if (d->compute_index) {
        // the score kernel writes the group maxima where the top-k keeps them
        float* gm = gsa::topk_group_max_area(d->workspace_dev, d->n_q, d->ld_scores);
        hipError_t e = gsa::launch_indexer_score(d->dt == GSA_FP8_E4M3, d->q_idx_dev, d->q_scale_dev,
                                                 d->w_dev, d->k_idx_dev, d->k_scale_dev, d->q_seq_dev,
                                                 d->q_pos_dev, d->n_q, d->batch, d->n_cap,
                                                 d->scores_dev, d->ld_scores, gm, s);
        if (e != hipSuccess) return hip_result(e, "group: indexer_score");
        e = gsa::launch_topk(d->scores_dev, d->ld_scores, d->q_pos_dev, d->n_q, d->k, gm, d->index_buf_dev,
                             d->workspace_dev, s);
        if (e != hipSuccess) return hip_result(e, "group: topk");
    }
    if (d->n_layers > 0)
        return enqueue_attention(d->layers, d->n_layers, d->q_seq_dev, d->index_buf_dev, d->k, d->n_q,
                                 d->n_heads, d->n_cap, d->paged_kv, d->kv_dt == GSA_FP8_E4M3, d->scale,
                                 d->workspace_dev, s);
    return GSA_OK;
}

// Layer i is full when i < 3 or i = 2 (mod 4); a shared layer uses the latest
// full layer before it.
bool layer_is_full(int i) { return i < 3 || i % 4 == 2; }

// After a group that computed its indices was enqueued: the host record of its buffer.
void write_tag(const gsa_group_desc* d) {
    if (!d->compute_index || d->index_tag == nullptr) return;
    gsa_index_tag& t = *d->index_tag;
    t.index_buf_dev = d->index_buf_dev;
    t.epoch = d->index_epoch;
    t.full_layer = d->index_layer;
    t.n_q = d->n_q;
    t.k = d->k;
    t.n_cap = d->n_cap;
}

}  // namespace

extern "C" {

gsa_status gsa_indexshare_group(const gsa_group_desc* d, void* stream) {
    gsa_status st = validate_group(d);
    if (st != GSA_OK) return st;
    st = enqueue_group(d, (hipStream_t)stream);
    if (st == GSA_OK) {
        write_tag(d);
        g_err[0] = 0;
    }
    return st;
}

size_t gsa_noalloc_scratch_bytes(void) { return kScratchBytes; }

gsa_status gsa_indexshare_group_noalloc(const gsa_group_desc* d, void* stream) {
    if (d == nullptr) return fail(GSA_ERR_INVALID_ARG, "desc is NULL");
    // the workspace this group needs (the same rule as gsa_group_workspace_bytes;
    // without a score buffer the top-k rows span n_cap rounded up to 4)
    size_t need = 0;
    if (d->n_layers >= 1) need = gsa_mla_layers_workspace_bytes(d->n_q, d->n_heads, d->k, d->n_layers);
    if (d->compute_index) {
        const int64_t ld = d->scores_dev != nullptr ? d->ld_scores : gsa::indexer_topk_ld(d->n_cap);
        const size_t t = (d->n_q >= 1 && ld >= 1 && d->k == GSA_TOPK) ? gsa::topk_workspace_bytes(d->n_q, ld, d->k) : 0;
        need = t > need ? t : need;
    }
    if (need > kScratchBytes)
        return fail(GSA_ERR_WORKSPACE,
                    "the group call without a workspace argument has a %zu-byte static scratch; this group needs %zu",
                    kScratchBytes, need);
    void* ws = nullptr;
    gsa_status st = scratch_for_current_device(&ws);
    if (st != GSA_OK) return st;
    gsa_group_desc g = *d;
    g.workspace_dev = ws;
    g.workspace_bytes = kScratchBytes;
    st = validate_group(&g);
    if (st != GSA_OK) return st;
    st = enqueue_group(&g, (hipStream_t)stream);
    if (st == GSA_OK) {
        write_tag(&g);
        g_err[0] = 0;
    }
    return st;
}

int gsa_layer_pattern(int n_layers, int32_t* src) {
    if (n_layers < 1) return -1;
    int n_full = 0, last = 0;
    for (int i = 0; i < n_layers; ++i) {
        if (layer_is_full(i)) { last = i; ++n_full; }
        if (src) src[i] = last;
    }
    return n_full;
}

gsa_status gsa_layer_stack(const gsa_stack_desc* d, void* stream) {
    if (d == nullptr) return fail(GSA_ERR_INVALID_ARG, "desc is NULL");
    REQUIRE(d->n_layers >= 1, "n_layers must be >= 1");
    REQUIRE(d->layers != nullptr && d->indexers != nullptr, "layers / indexers is NULL");
    REQUIRE(d->index_stride == 0 || d->index_stride >= (int64_t)d->n_q * d->k,
            "index_stride must be 0 or >= n_q * k");
    REQUIRE(d->index_stride % 4 == 0, "index_stride must be a multiple of 4 (16-byte rows)");
    // one group per full layer: the full layer and the shared layers after it
    auto group_at = [&](int i, int f) {                   // i: a full layer, f: its ordinal
        const gsa_indexer_layer& X = d->indexers[f];
        gsa_group_desc g{};
        g.compute_index = 1;
        g.dt = d->dt;
        g.q_idx_dev = X.q_idx_dev; g.q_scale_dev = X.q_scale_dev; g.w_dev = X.w_dev;
        g.k_idx_dev = X.k_idx_dev; g.k_scale_dev = X.k_scale_dev;
        g.scores_dev = d->scores_dev; g.ld_scores = d->ld_scores;
        g.q_seq_dev = d->q_seq_dev; g.q_pos_dev = d->q_pos_dev;
        g.n_q = d->n_q; g.batch = d->batch; g.n_cap = d->n_cap; g.k = d->k;
        g.index_buf_dev = d->index_buf_dev + (int64_t)f * d->index_stride;
        g.n_layers = 1;
        while (i + g.n_layers < d->n_layers && !layer_is_full(i + g.n_layers)) ++g.n_layers;
        g.layers = d->layers + i;
        g.n_heads = d->n_heads; g.scale = d->scale;
        g.workspace_dev = d->workspace_dev; g.workspace_bytes = d->workspace_bytes;
        g.paged_kv = d->paged_kv;
        g.kv_dt = d->kv_dt;
        g.index_epoch = d->index_epoch;
        g.index_layer = i;
        g.index_tag = d->index_tags != nullptr ? &d->index_tags[f] : nullptr;
        return g;
    };
    for (int i = 0, f = 0; i < d->n_layers; ++i) {      // validate all before enqueuing any
        if (!layer_is_full(i)) continue;
        const gsa_group_desc g = group_at(i, f++);
        const gsa_status st = validate_group(&g);
        if (st != GSA_OK) {
            char tmp[512];
            snprintf(tmp, sizeof(tmp), "group of full layer %d: %s", i, g_err);
            snprintf(g_err, sizeof(g_err), "%s", tmp);
            return st;
        }
    }
    for (int i = 0, f = 0; i < d->n_layers; ++i) {
        if (!layer_is_full(i)) continue;
        const gsa_group_desc g = group_at(i, f);
        const gsa_status st = enqueue_group(&g, (hipStream_t)stream);
        if (st != GSA_OK) return st;
        if (d->index_tags != nullptr) {
            // a record of an earlier full layer whose buffer this group overwrote describes nothing now
            for (int e = 0; e < f; ++e)
                if (d->index_tags[e].index_buf_dev == g.index_buf_dev) d->index_tags[e].epoch = 0;
            write_tag(&g);
        }
        ++f;
    }
    g_err[0] = 0;
    return GSA_OK;
}

}  // extern "C"

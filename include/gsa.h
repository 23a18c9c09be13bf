/*
 * gsa.h — C ABI of libgsa: GLM-5.2's DSA lightning indexer, IndexShare and
 * absorbed sparse MLA on one AMD Instinct MI355X (gfx950).
 *
 * Sources (page titles as published):
 *   [Overview]  "GLM-5.2 总览" (t6page), table tbl-glm52-config and glossary.
 *   [Arch]      "GLM-5.2 架构深度拆解" (pillumina), CH2 §2.1-§2.4, §7.3.
 *   [Q&A]       "GLM-5.2架构与基准" (lzwjava), §2 IndexShare / IndexCache.
 *   [Serving]   "GLM-5→5.1→5.2：稀疏索引、Agent 后训练与 1M 上下文服务"
 *               (papers-3lj), §10 operator-level changes.
 *
 * Conventions for every call:
 *   - Pointers named *_dev are device pointers (HBM); everything else is host.
 *     All device buffers are owned and allocated by the caller; the library
 *     never allocates, frees or synchronises.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and the call returns without waiting for it.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     failed check returns GSA_ERR_INVALID_ARG / GSA_ERR_UNSUPPORTED /
 *     GSA_ERR_WORKSPACE and enqueues nothing. A launch failure returns
 *     GSA_ERR_HIP. gsa_last_error() gives the calling thread's last message.
 *   - Device pointers must be 16-byte aligned. Tensors are dense row-major
 *     unless a leading dimension is given.
 *   - Values the library cannot check without reading device memory (indices,
 *     positions, sequence ids) must lie in the documented ranges; violating
 *     them is undefined behaviour.
 *   - Calls are re-entrant; calls that share a workspace must not overlap.
 */
#ifndef GSA_H
#define GSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gsa_status {
    GSA_OK = 0,
    GSA_ERR_INVALID_ARG = 1,   /* null pointer, bad size, misalignment, ... */
    GSA_ERR_UNSUPPORTED = 2,   /* valid but not implemented (e.g. k != 2048) */
    GSA_ERR_WORKSPACE = 3,     /* workspace missing or too small */
    GSA_ERR_HIP = 4,           /* a HIP launch failed */
    GSA_ERR_STALE_INDEX = 5    /* a shared-only group call's index buffer was not written for the
                                  epoch, full layer and shape the call names (gsa_index_tag) */
} gsa_status;

typedef enum gsa_dtype {
    GSA_BF16 = 0,              /* bfloat16 */
    GSA_FP8_E4M3 = 1           /* OCP E4M3FN bytes with fp32 per-128-block scales */
} gsa_dtype;

/* Fixed shapes of the GLM-5.2 indexer and MLA ([Overview] tbl-glm52-config;
 * [Arch] §1.1: index_n_heads 32, index_head_dim 128, index_topk 2048; 64 heads;
 * kv_lora_rank 512; qk_rope_head_dim 64). */
#define GSA_INDEX_HEADS 32
#define GSA_INDEX_DIM 128
#define GSA_TOPK 2048
#define GSA_LATENT_DIM 512
#define GSA_ROPE_DIM 64
#define GSA_KV_ROW 576          /* 512 latent + 64 RoPE bf16 = 1152 B per token */

const char* gsa_status_string(gsa_status s);
const char* gsa_last_error(void);
const char* gsa_version(void);

/*
 * gsa_quantize_e4m3 — per-block FP8 quantisation of indexer q or k
 * ([Overview] sub-document index row 02: FP8 per-block; glossary: E4M3).
 *
 * x_dev      bf16 [n_blocks, 128]: each 128-element row is one block (one
 *            indexer key row, or one (query, head) vector).
 * codes_dev  uint8 [n_blocks, 128] out: E4M3FN, round to nearest even,
 *            saturating at +-448.
 * scales_dev fp32 [n_blocks] out: 2^e with e the smallest integer such that
 *            max|x| <= 448 * 2^e, clamped to [-126, 127]; 1 for a zero block.
 * Errors: null pointers, n_blocks < 0 (0 is a no-op).
 */
gsa_status gsa_quantize_e4m3(const void* x_dev, int64_t n_blocks,
                             uint8_t* codes_dev, float* scales_dev, void* stream);

/*
 * gsa_quantize_e4m3_hadamard — the same after a Hadamard rotation of each block
 * ([Overview] sub-document index row 02 names FP8 per-block quantisation with a
 * Hadamard rotation for the indexer):
 *   y = H x / sqrt(128), H the Sylvester-ordered 128 x 128 Hadamard matrix
 *   (H[i][j] = (-1)^popcount(i & j)), computed as the exact +-1 sums in fp32
 *   times the fp32 value of 1/sqrt(128); then codes and scale of y as above.
 * Rotating both q and k leaves q . k unchanged in exact arithmetic (H is
 * orthogonal up to the factor 128), so gsa_indexer_score takes the rotated
 * codes as they are. Same arguments and errors as gsa_quantize_e4m3.
 */
gsa_status gsa_quantize_e4m3_hadamard(const void* x_dev, int64_t n_blocks,
                                      uint8_t* codes_dev, float* scales_dev, void* stream);

/*
 * gsa_indexer_score — the full (F) layer's lightning-indexer score
 * ([Arch] §2.2: an F layer scores each query against every history token
 * with 32 heads x 128 dims; [Overview] sub-document index: ReLU).
 *
 *   scores[i, s] = sum_h w[i,h] * max(0, q[i,h,:] . k[q_seq[i], s, :])  s <= q_pos[i]
 *   scores[i, s] = -inf                                                q_pos[i] < s < n_cap
 *   columns n_cap .. ld_scores-1 are not written.
 *
 * dt         GSA_BF16 or GSA_FP8_E4M3.
 * q_dev      [n_q, 32, 128] bf16, or E4M3 bytes when dt is FP8.
 * q_scale_dev fp32 [n_q, 32] per-(query, head) block scales (FP8 only, else NULL).
 * w_dev      fp32 [n_q, 32] per-(query, head) weights.
 * k_dev      [batch, n_cap, 128] bf16 or E4M3 bytes: one key per position,
 *            shared by all heads.
 * k_scale_dev fp32 [batch, n_cap] per-key-row block scales (FP8 only, else NULL).
 *            FP8 scales must be powers of two (as gsa_quantize_e4m3 makes them);
 *            only their exponent is used.
 * q_seq_dev  int32 [n_q], each in [0, batch). q_pos_dev int32 [n_q], each in
 *            [0, n_cap). Queries of one sequence should be adjacent (any order
 *            is correct; adjacency lets them share key reads).
 * scores_dev fp32 [n_q, ld_scores], ld_scores >= n_cap, ld_scores % 4 == 0.
 * group_max_dev fp32 [n_q, gsa_group_max_ld(ld_scores)] out, or NULL (not
 *            written): group_max[i, g] = the largest of scores[i, 32g .. 32g+31]
 *            over columns < n_cap, -0.0 given as +0.0. gsa_topk uses them to
 *            pass over scores that cannot be selected.
 * Errors: null pointers, n_q < 1, batch < 1, n_cap < 1, bad ld, bad dtype,
 *         missing scales for FP8, n_cap > 2^31 - 1.
 * Concurrency: FP8 calls with one query per sequence, a query count dividing
 * 256, n_cap a multiple of 1024 and n_q * n_cap >= 2^23 hand out key chunks
 * through per-query counters in a static device array of 64 slots (no
 * allocation; every launch leaves its slot at zero). Such a launch takes a
 * new slot each call: at most 63 other such launches may start on the same
 * device while one runs.
 */
gsa_status gsa_indexer_score(gsa_dtype dt,
                             const void* q_dev, const float* q_scale_dev, const float* w_dev,
                             const void* k_dev, const float* k_scale_dev,
                             const int32_t* q_seq_dev, const int32_t* q_pos_dev,
                             int n_q, int batch, int64_t n_cap,
                             float* scores_dev, int64_t ld_scores, float* group_max_dev,
                             void* stream);

/* Row stride of the group maxima of score rows of stride ld_scores: ceil(ld / 32). */
int64_t gsa_group_max_ld(int64_t ld_scores);

/*
 * gsa_topk — causal top-k over each score row ([Arch] §2.2 and §1.1:
 * index_topk 2048, the selected tokens are the layer's sparse attention set).
 *
 * For row i, among positions s = 0..q_pos[i], keeps the min(k, q_pos[i]+1)
 * largest scores; ties go to the lower position; -0.0 ties with +0.0.
 * idx_dev int32 [n_q, k] out: the kept positions in ascending order, then -1.
 * NaN scores are not supported.
 * scores_dev fp32 [n_q, ld_scores] (ld_scores % 4 == 0, >= max q_pos + 1,
 *            <= 2^23).
 * group_max_dev the group maxima of these scores as gsa_indexer_score writes
 *            them, or NULL (then computed in the workspace, at the cost of one
 *            more read of the rows). Rows of at least 2048 full groups
 *            (q_pos + 1 >= 65536) select only among scores >= the 2048th
 *            largest group maximum, which holds the selection exactly when the
 *            maxima are those of the scores (the caller's duty when passing them).
 * workspace_dev: at least gsa_topk_workspace_bytes(n_q, ld_scores, k) bytes,
 *            16-byte aligned; its contents on entry do not matter.
 * Errors: k != 2048 or ld_scores > 2^23 (GSA_ERR_UNSUPPORTED), null pointers,
 *         small workspace.
 */
size_t gsa_topk_workspace_bytes(int n_q, int64_t ld_scores, int k);
gsa_status gsa_topk(const float* scores_dev, int64_t ld_scores, const int32_t* q_pos_dev,
                    int n_q, int k, const float* group_max_dev, int32_t* idx_dev,
                    void* workspace_dev, size_t workspace_bytes, void* stream);

/*
 * gsa_indexer_topk — the full layer's score and top-k without a score buffer
 * ([Serving] §10: the candidate scoring and top-k a sparse layer adds perform
 * according to how far they are fused; here no [n_q, n_cap] score matrix
 * reaches memory).
 *
 * Selects exactly what gsa_indexer_score followed by gsa_topk selects (same
 * positions, same order, -1 padded), from the same inputs (arguments as in
 * gsa_indexer_score, without scores_dev / ld_scores / group_max_dev). Rows of at
 * least 2048 full 32-position groups run the score kernel writing only group
 * maxima, take the 2048th largest of them as a lower bound of every selected
 * score, and recompute the scores of the groups whose maximum reaches it with
 * the score kernel's own arithmetic (bit-identical scores); shorter rows
 * recompute every group. It saves the score buffer's memory (4 * n_q * n_cap
 * bytes: 2 GiB for 4096 queries over 2^17 positions) and its traffic; on
 * MI355X it is not faster than the buffered pair at 2^17 to 2^20 positions
 * (the key rows of the ~6% of groups that reach the bound at 2^20 are re-read
 * one row per lane, and the score pass without a buffer measured no faster).
 * k must be 2048; n_cap <= 2^23.
 * workspace_dev: at least gsa_indexer_topk_workspace_bytes(n_q, n_cap, k)
 *            bytes, 16-byte aligned; its contents on entry do not matter.
 * Errors: as gsa_indexer_score and gsa_topk.
 */
size_t gsa_indexer_topk_workspace_bytes(int n_q, int64_t n_cap, int k);
gsa_status gsa_indexer_topk(gsa_dtype dt,
                            const void* q_dev, const float* q_scale_dev, const float* w_dev,
                            const void* k_dev, const float* k_scale_dev,
                            const int32_t* q_seq_dev, const int32_t* q_pos_dev,
                            int n_q, int batch, int64_t n_cap, int k, int32_t* idx_dev,
                            void* workspace_dev, size_t workspace_bytes, void* stream);

/*
 * gsa_sparse_mla_attn — absorbed MLA over the selected positions of one layer
 * ([Overview] tbl-glm52-config: 64 heads, QK dim 256 = 192 + 64, latent 512,
 * cache row 512 + 64 in BF16 = 1152 B; sub-document index: decode in latent
 * space; [Serving] §10: each layer gathers the selected entries of its own
 * K/V cache, then sparse attention).
 *
 * For query i, head h, selected rows s_j = idx[i, j] (entries outside [0, n_cap)
 * skipped, -1 in particular):
 *   z_j = scale * (q_lat[i,h,:] . c[s_j] + q_rope[i,h,:] . kr[s_j])
 *   out[i,h,:] = sum_j softmax(z)_j * c[s_j];  lse[i,h] = log sum_j exp(z_j)
 * (c = kv[..., :512], kr = kv[..., 512:]). A row with no valid index gives
 * out = 0 and lse = -inf.
 *
 * q_lat_dev  bf16 [n_q, n_heads, 512]; q_rope_dev bf16 [n_q, n_heads, 64].
 * kv_dev     bf16 [batch, n_cap, 576] (packed 1152-byte rows).
 * q_seq_dev  int32 [n_q] in [0, batch). idx_dev int32 [n_q, k]: positions in
 *            [0, n_cap); -1 pads, and any entry outside that range is skipped the
 *            same way (an unsigned compare in the gather), so a stale or foreign
 *            buffer cannot make the gather read outside the sequence's rows.
 * n_heads    must be 64. k must be 2048.
 * out_dev    fp32 [n_q, n_heads, 512]; lse_dev fp32 [n_q, n_heads] or NULL.
 * workspace_dev: at least gsa_mla_workspace_bytes(n_q, n_heads, k) bytes.
 */
size_t gsa_mla_workspace_bytes(int n_q, int n_heads, int k);
gsa_status gsa_sparse_mla_attn(const void* q_lat_dev, const void* q_rope_dev, const void* kv_dev,
                               const int32_t* q_seq_dev, const int32_t* idx_dev, int k,
                               int n_q, int n_heads, int batch, int64_t n_cap, float scale,
                               float* out_dev, float* lse_dev,
                               void* workspace_dev, size_t workspace_bytes, void* stream);

/*
 * gsa_indexshare_group — one IndexShare group: a full layer and the shared
 * layers that reuse its indices ([Arch] §2.2 and §2.4: the F layer runs the
 * indexer and writes the shared top-k buffer, S layers skip the indexer and
 * read it; [Serving] §10: indexer once per group, buffer written once, every
 * layer gathers from its own cache; [Arch] §7.3: with no shared layers this is
 * per-layer DSA; [Arch] §2.4: MTP steps may reuse the buffer).
 *
 * compute_index = 1: score + top-k run and write index_buf_dev, then every
 *                    layer in `layers` attends over it (layers[0] is the F layer).
 * compute_index = 0: the caller supplies index_buf_dev (e.g. an earlier F
 *                    layer's, or for MTP draft steps); only attention runs, and
 *                    the indexer fields are ignored.
 * index_buf_dev int32 [n_q, k], owned by the caller, who keeps it consistent
 *                    with the prefix and positions it was computed for.
 * scores_dev   fp32 [n_q, ld_scores] scratch for the F layer's scores, or NULL:
 *              then the F layer selects as gsa_indexer_topk does (no score
 *              buffer; ld_scores is ignored) and the workspace is sized with
 *              ld_scores = n_cap rounded up to a multiple of 4.
 * workspace    at least gsa_group_workspace_bytes(n_q, ld_scores, k, n_heads, n_layers).
 * Attention for all n_layers layers runs as gsa_sparse_mla_attn_layers.
 */
typedef struct gsa_mla_layer {
    const void* q_lat_dev;     /* bf16 [n_q, n_heads, 512] */
    const void* q_rope_dev;    /* bf16 [n_q, n_heads, 64] */
    const void* kv_dev;        /* bf16 [batch, n_cap, 576] */
    float* out_dev;            /* fp32 [n_q, n_heads, 512] */
    float* lse_dev;            /* fp32 [n_q, n_heads] or NULL */
} gsa_mla_layer;

/*
 * gsa_paged_kv — a latent cache kept in pages ([Arch] §4.4 names PagedAttention
 * as the paging used with the 512-d latent cache), for the gather of [Serving]
 * §10 (each layer gathers its own cache rows at the selected positions). Each layer's kv_dev is then a
 * pool of n_pages pages of page_size rows ([n_pages * page_size, 576] bf16),
 * and position s of sequence b is pool row
 *     block_table_dev[b * max_pages + s / page_size] * page_size + s % page_size.
 * The table (int32 [batch, max_pages], device) is shared by the layers; the
 * caller keeps it consistent with the indices, and its entries must be page
 * numbers < n_pages for every page a selected position falls in (not checked
 * on the device). A sequence holds max_pages * page_size positions.
 */
typedef struct gsa_paged_kv {
    const int32_t* block_table_dev;
    int page_size;
    int max_pages;
    int64_t n_pages;
} gsa_paged_kv;

/*
 * gsa_quantize_latent_fp8 — the FP8 latent cache row ([Overview]
 * tbl-glm52-config: about 656 bytes per token and layer with per-group scales;
 * glossary: KV FP8 is E4M3 on the 512-dim latent):
 *   out[r] = [512 E4M3 codes | 4 fp32 scales | 64 bf16 RoPE dims] (656 bytes)
 * The latent is quantised in four 128-dim groups with the rule of
 * gsa_quantize_e4m3 (power-of-two scale, nearest even, saturating at 448); the
 * RoPE dims are copied. rows_dev bf16 [n_rows, 576]; out_dev uint8 [n_rows,
 * 656]; both 16-byte aligned. Errors: null or misaligned pointers, n_rows < 0.
 */
gsa_status gsa_quantize_latent_fp8(const void* rows_dev, int64_t n_rows, uint8_t* out_dev, void* stream);

/*
 * gsa_sparse_mla_attn_fp8kv — gsa_sparse_mla_attn_layers over FP8 latent
 * caches: each layers[l].kv_dev holds 656-byte rows (gsa_quantize_latent_fp8),
 * [batch, n_cap, 656] contiguous, or page pools [n_pages * page_size, 656] when
 * paged_kv is not NULL (n_cap is then ignored). Attention is computed on the
 * dequantised rows (code x group scale, exact in bf16) with the same
 * arithmetic as the bf16 cache. Same workspace and errors as
 * gsa_sparse_mla_attn_layers / gsa_sparse_mla_attn_paged.
 */
gsa_status gsa_sparse_mla_attn_fp8kv(const gsa_mla_layer* layers, int n_layers,
                                     const gsa_paged_kv* paged_kv, const int32_t* q_seq_dev,
                                     const int32_t* idx_dev, int k, int n_q, int n_heads, int batch,
                                     int64_t n_cap, float scale, void* workspace_dev,
                                     size_t workspace_bytes, void* stream);

/*
 * gsa_index_tag — what an index buffer holds, kept by the caller on the host next
 * to the buffer ([Serving] §10: a reused index cache is valid only for the prefix,
 * positions and model revision it was computed for; [Arch] §2.4: shared layers and
 * MTP steps read the buffer a full layer wrote). The library cannot read device
 * memory to check a buffer, so the check is on this host record:
 *   - a group call with compute_index = 1 and index_tag != NULL fills the record
 *     in once its launches are enqueued (the buffer holds those indices when the
 *     stream reaches them);
 *   - a group call with compute_index = 0 and index_epoch != 0 compares the
 *     record with its own description and returns GSA_ERR_STALE_INDEX, enqueuing
 *     nothing, unless the buffer, epoch, full layer, n_q and k are equal and the
 *     record's n_cap is at most the call's (every stored position is then inside
 *     the call's caches).
 * epoch is the caller's name for the prefix, positions and revision (any value
 * but 0; 0 marks a record that describes nothing).
 */
typedef struct gsa_index_tag {
    const int32_t* index_buf_dev;  /* the buffer the record describes */
    uint64_t epoch;                /* the epoch of the call that wrote it; 0: nothing written */
    int full_layer;                /* the full layer whose indexer wrote it */
    int n_q;                       /* rows written */
    int k;                         /* indices per row */
    int64_t n_cap;                 /* positions of the writing call's caches */
} gsa_index_tag;

typedef struct gsa_group_desc {
    int compute_index;
    gsa_dtype dt;
    const void* q_idx_dev; const float* q_scale_dev; const float* w_dev;
    const void* k_idx_dev; const float* k_scale_dev;
    float* scores_dev; int64_t ld_scores;
    const int32_t* q_seq_dev; const int32_t* q_pos_dev;
    int n_q; int batch; int64_t n_cap; int k;
    int32_t* index_buf_dev;
    int n_layers; const gsa_mla_layer* layers;   /* host array of n_layers */
    int n_heads; float scale;
    void* workspace_dev; size_t workspace_bytes;
    const gsa_paged_kv* paged_kv;   /* NULL: contiguous caches [batch, n_cap, row]; else each
                                       layer's kv_dev is a page pool and n_cap still sizes the
                                       indexer keys and scores (max_pages * page_size >= n_cap) */
    gsa_dtype kv_dt;                 /* GSA_BF16 (0): 1152-byte bf16 rows; GSA_FP8_E4M3: 656-byte
                                       FP8 latent rows (gsa_sparse_mla_attn_fp8kv) */
    uint64_t index_epoch;            /* the caller's epoch of this call (gsa_index_tag); 0: the
                                       buffer is not checked and a written record gets epoch 0 */
    int index_layer;                 /* the full layer whose indices index_buf_dev holds: the
                                       one this call's indexer is (compute_index = 1), or the
                                       one whose buffer it reuses (compute_index = 0) */
    gsa_index_tag* index_tag;        /* host record of index_buf_dev, or NULL: written when
                                       compute_index = 1, checked when 0 (NULL with a non-zero
                                       index_epoch is GSA_ERR_INVALID_ARG) */
} gsa_group_desc;

/* workspace of a group with n_layers attention layers (the full layer included) */
size_t gsa_group_workspace_bytes(int n_q, int64_t ld_scores, int k, int n_heads, int n_layers);
gsa_status gsa_indexshare_group(const gsa_group_desc* desc, void* stream);

/*
 * gsa_indexshare_group_noalloc — gsa_indexshare_group for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid allocation. It takes no workspace: desc->workspace_dev
 * and workspace_bytes are ignored, and the group runs on a static device scratch
 * of gsa_noalloc_scratch_bytes() bytes (64 MiB) that the library holds on every
 * GPU it runs on until the process ends. It calls no allocating routine. On the
 * first call on a device it looks up that device's scratch address (once).
 * Results are those of gsa_indexshare_group on the same descriptor (same kernels;
 * the kernels need no scratch contents on entry).
 * All calls on one GPU share its scratch: calls that overlap on one GPU (other
 * streams, other threads) race and must not be issued.
 * Errors: as gsa_indexshare_group; GSA_ERR_WORKSPACE when the group needs more
 * than the scratch holds (e.g. thousands of queries over 128K positions).
 */
size_t gsa_noalloc_scratch_bytes(void);
gsa_status gsa_indexshare_group_noalloc(const gsa_group_desc* desc, void* stream);

/*
 * gsa_sparse_mla_attn_layers — gsa_sparse_mla_attn for n_layers layers that
 * attend over the same index buffer, the layers of one IndexShare group
 * ([Serving] §10: the indexer runs once per group, then every layer gathers
 * from its own cache and attends; [Arch] §2.2: the same index set serves the
 * full layer and its shared layers). The layers are independent given the
 * indices, so they run in one launch (per 8 layers), which lets a small batch
 * fill the chip with fewer row splits per query.
 *
 * layers        host array of n_layers gsa_mla_layer (each layer's own q, cache, out, lse).
 * The other arguments mean what they mean in gsa_sparse_mla_attn.
 * workspace_dev at least gsa_mla_layers_workspace_bytes(n_q, n_heads, k, n_layers) bytes.
 * Errors as gsa_sparse_mla_attn, checked for every layer before anything is enqueued.
 */
size_t gsa_mla_layers_workspace_bytes(int n_q, int n_heads, int k, int n_layers);

/*
 * gsa_sparse_mla_attn_paged — gsa_sparse_mla_attn_layers over paged caches
 * (gsa_paged_kv above): each layers[l].kv_dev is that layer's page pool.
 * Indices are sequence positions; entries outside [0, max_pages * page_size) are
 * skipped as -1 is. Same workspace as
 * gsa_sparse_mla_attn_layers; errors as there, plus GSA_ERR_INVALID_ARG for a
 * NULL or malformed paged_kv.
 */
gsa_status gsa_sparse_mla_attn_paged(const gsa_mla_layer* layers, int n_layers,
                                     const gsa_paged_kv* paged_kv, const int32_t* q_seq_dev,
                                     const int32_t* idx_dev, int k, int n_q, int n_heads, int batch,
                                     float scale, void* workspace_dev, size_t workspace_bytes,
                                     void* stream);
gsa_status gsa_sparse_mla_attn_layers(const gsa_mla_layer* layers, int n_layers,
                                      const int32_t* q_seq_dev, const int32_t* idx_dev, int k,
                                      int n_q, int n_heads, int batch, int64_t n_cap, float scale,
                                      void* workspace_dev, size_t workspace_bytes, void* stream);

/*
 * gsa_layer_pattern — which layers run the indexer in GLM-5.2's layer stack
 * ([Arch] §2.1 table: layers 0, 1, 2 are full, then every fourth layer from 6
 * (6, 10, ..., 74) is full and the three after it are shared; 21 full and 57
 * shared of 78; §1.2: index_topk_freq = 4). A shared layer uses the indices of
 * the latest full layer before it; the §2.1 table makes layer 76 shared, so
 * layer 77 uses layer 74 (not "L76" as the §1.3 diagram labels it).
 *
 * src (host, n_layers int32, or NULL): src[i] = the full layer whose indices
 * layer i attends over (i itself when layer i is full).
 * Returns the number of full layers, or -1 when n_layers < 1.
 */
int gsa_layer_pattern(int n_layers, int32_t* src);

/*
 * gsa_layer_stack — the attention stack of n_layers layers under that pattern:
 * one IndexShare group per full layer (score + top-k into its index buffer,
 * then attention for it and the shared layers after it), in layer order on
 * `stream` ([Arch] §2.1-§2.4; [Serving] §10). Every group is validated before
 * the first is enqueued; the groups then run as gsa_indexshare_group would.
 *
 * indexers      host array, one gsa_indexer_layer per full layer, in layer
 *               order (gsa_layer_pattern(n_layers, NULL) entries).
 * layers        host array of n_layers gsa_mla_layer (each layer's own cache).
 * scores_dev    fp32 [n_q, ld_scores], scratch reused by every full layer.
 * index_buf_dev int32: full layer number f (its ordinal among full layers)
 *               writes [n_q, k] at index_buf_dev + f * index_stride.
 *               index_stride = 0 reuses one buffer (enough for the stack
 *               itself, since each group reads only its own full layer's
 *               indices); otherwise index_stride >= n_q * k, a multiple of 4.
 * workspace     at least gsa_stack_workspace_bytes(n_q, ld_scores, k, n_heads, n_layers)
 *               (the largest need of its groups).
 * The other fields mean what they mean in gsa_group_desc.
 */
typedef struct gsa_indexer_layer {
    const void* q_idx_dev; const float* q_scale_dev; const float* w_dev;
    const void* k_idx_dev; const float* k_scale_dev;
} gsa_indexer_layer;

typedef struct gsa_stack_desc {
    int n_layers;
    gsa_dtype dt;
    const gsa_indexer_layer* indexers;
    const gsa_mla_layer* layers;
    float* scores_dev; int64_t ld_scores;
    const int32_t* q_seq_dev; const int32_t* q_pos_dev;
    int n_q; int batch; int64_t n_cap; int k;
    int32_t* index_buf_dev; int64_t index_stride;
    int n_heads; float scale;
    void* workspace_dev; size_t workspace_bytes;
    const gsa_paged_kv* paged_kv;   /* as in gsa_group_desc */
    gsa_dtype kv_dt;                 /* as in gsa_group_desc */
    uint64_t index_epoch;            /* as in gsa_group_desc */
    gsa_index_tag* index_tags;       /* NULL, or one host record per full layer (ordinal f):
                                       record f describes full layer f's buffer once its group
                                       is enqueued; a record whose buffer a later group of the
                                       same call overwrites (index_stride = 0) is reset to
                                       epoch 0 */
} gsa_stack_desc;

size_t gsa_stack_workspace_bytes(int n_q, int64_t ld_scores, int k, int n_heads, int n_layers);
gsa_status gsa_layer_stack(const gsa_stack_desc* desc, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* GSA_H */

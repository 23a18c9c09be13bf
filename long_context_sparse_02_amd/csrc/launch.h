// Host-side launchers of the gfx950 kernels (internal to libgsa; the C ABI in
// include/gsa.h validates arguments and then calls these).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gsa {

// A new tag per call: a per-process 64-bit sequence from a start that differs
// between processes, never 0. Kernels that hand work over through device
// memory mark it with the tag of their launch.
unsigned long long launch_tag();

// rotate: multiply each 128-element block by the orthonormal Hadamard matrix first.
hipError_t launch_quantize_e4m3(const void* x, int64_t n_blocks, uint8_t* codes, float* scales,
                                bool rotate, hipStream_t stream);

hipError_t launch_indexer_score(bool fp8, const void* q, const float* q_scale, const float* w,
                                const void* k, const float* k_scale, const int32_t* q_seq,
                                const int32_t* q_pos, int n_q, int batch, int64_t n_cap,
                                float* scores, int64_t ld, float* group_max, hipStream_t stream);

// Group maxima: group_max[q * ((ld + 31) / 32) + g] = the largest score of
// positions [32g, 32g + 32) of row q (by the order-preserving key).
constexpr int kGroup = 32;
inline int64_t group_max_ld(int64_t ld) { return (ld + kGroup - 1) / kGroup; }

size_t topk_workspace_bytes(int n_q, int64_t ld, int k);
// Where, inside a top-k workspace, the group maxima of these scores are kept
// (NULL when rows this short need none): a score launch that writes them there
// saves the top-k their computation.
float* topk_group_max_area(void* ws, int n_q, int64_t ld);
// group_max: the score kernel's group maxima of these scores, or NULL (the
// top-k then computes them in its workspace).
hipError_t launch_topk(const float* scores, int64_t ld, const int32_t* q_pos, int n_q, int k,
                       const float* group_max, int32_t* idx, void* ws, hipStream_t stream);

// Score and top-k without a score buffer: group maxima from the score kernel,
// their bound, then a rescoring of the 32-position groups that reach it. The
// workspace is topk_workspace_bytes(n_q, indexer_topk_ld(n_cap), k) bytes.
inline int64_t indexer_topk_ld(int64_t n_cap) { return (n_cap + 3) / 4 * 4; }
hipError_t launch_indexer_topk(bool fp8, const void* q, const float* q_scale, const float* w, const void* k,
                               const float* k_scale, const int32_t* q_seq, const int32_t* q_pos, int n_q,
                               int batch, int64_t n_cap, int k_sel, int32_t* idx, void* ws, hipStream_t stream);

// One attention layer's operands (a layer of an IndexShare group).
struct MlaLayerPtrs {
    const void* q_lat;
    const void* q_rope;
    const void* kv;
    float* out;
    float* lse;
};

// Workspace for attention over n_layers layers that share one index buffer.
size_t mla_workspace_bytes(int n_q, int n_heads, int k, int n_layers);
// block_table NULL: each layer's cache is [batch, n_cap, row]; otherwise a pool
// of page_size-row pages addressed through block_table [batch, max_pages].
// Rows are 576 bf16 (1152 bytes) or, with fp8_kv, 656-byte FP8 latent rows.
hipError_t launch_sparse_mla_layers(const MlaLayerPtrs* layers, int n_layers, const int32_t* q_seq,
                                    const int32_t* idx, int k, int n_q, int n_heads, int64_t n_cap,
                                    const int32_t* block_table, int page_size, int max_pages,
                                    bool fp8_kv, float scale, void* ws, hipStream_t stream);

// FP8 latent cache rows [512 E4M3 | 4 fp32 scales | 64 bf16 RoPE] from bf16 rows [n, 576].
hipError_t launch_quantize_latent(const void* rows, int64_t n_rows, uint8_t* out, hipStream_t stream);

}  // namespace gsa

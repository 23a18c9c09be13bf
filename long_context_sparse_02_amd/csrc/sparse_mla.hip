// Absorbed sparse MLA over the selected rows of one layer, on gfx950.
//
// "GLM-5.2 总览" tbl-glm52-config: 64 heads, QK dim 256 (192 NoPE + 64 RoPE),
// KV latent 512; a cache row is the 512-dim latent plus the 64-dim RoPE key,
// 1152 bytes in BF16; its sub-document index: decode attends in latent space
// (absorb). "GLM-5→5.1→5.2…" §10: every layer gathers the selected entries
// of its own cache, then runs sparse attention; "GLM-5.2 架构深度拆解" §2.2:
// attention covers only the selected tokens, in F and S layers alike.
//
//   z_j = scale * (q_lat . c[s_j] + q_rope . kr[s_j]);  out = sum_j softmax(z)_j c[s_j]
//
// One work-group (4 waves, 16 heads each) takes one query and a contiguous
// slice of its selected rows ("split"); slices are merged with their
// log-sum-exp when a query is split. Per 32-row block:
//   gather  each thread pulls 16-byte pieces of two adjacent rows (wave loads
//           cover whole 128-byte lines) into LDS twice: row-major for Q.K,
//           and as bf16 pairs (row 2p, row 2p+1) per latent dim for P.V, the
//           pairing done in registers with v_perm. The next block's loads are
//           in flight while the current block is multiplied.
//   Q.K     S^T (rows x heads) on v_mfma_f32_16x16x32_bf16 with Q resident in
//           registers; in that layout a lane holds 8 rows of one head, so the
//           softmax max/sum need only two cross-lane steps.
//   softmax online, base 2; the running max moves only when a block max
//           exceeds it by more than 2^8, so the O rescale is rare.
//   P.V     P (bf16) is the MFMA A operand straight from registers; the V
//           operand comes from the pair-transposed copy; O (16 heads x 512)
//           stays in accumulators for the whole slice.
#include "device_common.h"
#include "launch.h"

namespace gsa {
namespace {

constexpr int kHeads = 64;
constexpr int kLat = 512;
constexpr int kRowElems = 576;
constexpr int kRowBytes = kRowElems * 2;      // 1152
constexpr int kBlk = 32;                      // rows per block
constexpr int kThreads = 256;
constexpr int kRowStride = kRowBytes + 16;    // LDS row pitch (bank spread)
constexpr int kCtStride = 72;                 // bytes per latent dim: 16 pairs x 4 B + 8 pad
constexpr int kRowBuf = kBlk * kRowStride;
constexpr int kCtBuf = kLat * kCtStride;
constexpr int kBuf = kRowBuf + kCtBuf;
constexpr int kMaxRows = 2048;
constexpr float kRescale = 8.0f;              // lazy-rescale threshold (log2 units)

__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }

__global__ __launch_bounds__(kThreads) void sparse_mla_kernel(
    const uint8_t* __restrict__ q_lat, const uint8_t* __restrict__ q_rope,
    const uint8_t* __restrict__ kv, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ idx, int k, int64_t n_cap, float scale_log2, int rows_per_split,
    float* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    int32_t* rows_s = (int32_t*)(smem + 2 * kBuf);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    const int q = blockIdx.y, split = blockIdx.x, n_split = gridDim.x;
    const int r0 = split * rows_per_split;
    const int nrows = rows_per_split;
    const int seq = q_seq[q];
    const uint8_t* kvs = kv + (int64_t)seq * n_cap * kRowBytes;

    for (int i = tid; i < nrows; i += kThreads) rows_s[i] = idx[(int64_t)q * k + r0 + i];

    // Q of this wave's 16 heads as the B operand: head = 16*wave + l16, dims 32t + 8g
    const int head = 16 * wave + l16;
    bf16x8 qr[18];
    {
        const uint8_t* ql = q_lat + ((int64_t)q * kHeads + head) * (kLat * 2);
        const uint8_t* qp = q_rope + ((int64_t)q * kHeads + head) * (64 * 2);
#pragma unroll
        for (int t = 0; t < 16; ++t) qr[t] = *(const bf16x8*)(ql + 2 * (32 * t + 8 * g));
#pragma unroll
        for (int t = 0; t < 2; ++t) qr[16 + t] = *(const bf16x8*)(qp + 2 * (32 * t + 8 * g));
    }
    __syncthreads();

    // gather registers: 4 latent units (2 rows x 16 B each) + 1 RoPE unit
    i32x4 gl[4][2], gr;
    auto gather = [&](int b) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int u = i * kThreads + tid;
            const int p = u & 15, c = u >> 4;          // row pair, 16-byte latent chunk
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int s = rows_s[b * kBlk + 2 * p + h];
                gl[i][h] = s >= 0 ? *(const i32x4*)(kvs + (int64_t)s * kRowBytes + 16 * c)
                                  : i32x4{0, 0, 0, 0};
            }
        }
        const int r = tid >> 3, c = tid & 7;
        const int s = rows_s[b * kBlk + r];
        gr = s >= 0 ? *(const i32x4*)(kvs + (int64_t)s * kRowBytes + 1024 + 16 * c)
                    : i32x4{0, 0, 0, 0};
    };
    auto stash = [&](uint8_t* buf) {
        uint8_t* rowb = buf;
        uint8_t* ctb = buf + kRowBuf;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int u = i * kThreads + tid;
            const int p = u & 15, c = u >> 4;
            *(i32x4*)(rowb + (2 * p) * kRowStride + 16 * c) = gl[i][0];
            *(i32x4*)(rowb + (2 * p + 1) * kRowStride + 16 * c) = gl[i][1];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t x = (uint32_t)gl[i][0][e], y = (uint32_t)gl[i][1][e];
                const uint32_t lo = __builtin_amdgcn_perm(y, x, 0x05040100u);   // dim 8c+2e
                const uint32_t hi = __builtin_amdgcn_perm(y, x, 0x07060302u);   // dim 8c+2e+1
                *(uint32_t*)(ctb + (8 * c + 2 * e) * kCtStride + 4 * p) = lo;
                *(uint32_t*)(ctb + (8 * c + 2 * e + 1) * kCtStride + 4 * p) = hi;
            }
        }
        const int r = tid >> 3, c = tid & 7;
        *(i32x4*)(rowb + r * kRowStride + 1024 + 16 * c) = gr;
    };

    f32x4 o[32];
#pragma unroll
    for (int d = 0; d < 32; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = neg_inf();      // running max (log2 units) of head `head`
    float l_part = 0.f;           // this lane's share of the running sum

    const int nblk = nrows / kBlk;
    if (nblk > 0) gather(0);
    for (int b = 0; b < nblk; ++b) {
        uint8_t* buf = smem + (b & 1) * kBuf;
        stash(buf);
        __syncthreads();
        if (b + 1 < nblk) gather(b + 1);

        // S^T tiles: rows 16tt + 4g + i, head l16 of this wave
        const uint8_t* rowb = buf;
        f32x4 sacc[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            const uint8_t* arow = rowb + (16 * tt + l16) * kRowStride + 16 * g;
#pragma unroll
            for (int t = 0; t < 18; ++t) {
                const bf16x8 a = *(const bf16x8*)(arow + 64 * t);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qr[t], acc, 0, 0, 0);
            }
            sacc[tt] = acc;
        }
        float z[8];
        float mb = neg_inf();
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * tt + 4 * g + i;
                const bool ok = rows_s[b * kBlk + r] >= 0;
                const float v = ok ? sacc[tt][i] * scale_log2 : neg_inf();
                z[tt * 4 + i] = v;
                mb = fmaxf(mb, v);
            }
        mb = fmaxf(mb, shfl_xor(mb, 16));
        mb = fmaxf(mb, shfl_xor(mb, 32));
        const bool move = mb > m_run + kRescale || (m_run == neg_inf() && mb != neg_inf());
        if (__builtin_amdgcn_ballot_w64(move) != 0) {   // wave-uniform branch
            const float m_new = move ? mb : m_run;
            const float alpha = move ? exp2_(m_run - m_new) : 1.f;   // exp2(-inf) = 0
            l_part *= alpha;
            m_run = m_new;
            float al[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g + i, 64);
#pragma unroll
            for (int d = 0; d < 32; ++d)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[d][i] *= al[i];
        }
        const float m_use = m_run == neg_inf() ? 0.f : m_run;
        bf16x8 pa;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float p = exp2_(z[e] - m_use);
            l_part += p;
            pa[e] = (__bf16)p;
        }
        // P.V: O[heads][16 dims] += P[heads][32 rows] * V[32 rows][16 dims]
        const uint8_t* ctb = buf + kRowBuf + l16 * kCtStride + 8 * g;
#pragma unroll
        for (int d = 0; d < 32; ++d) {
            const uint8_t* cp = ctb + 16 * d * kCtStride;
            const uint2 lo = *(const uint2*)(cp);        // rows 4g..4g+3
            const uint2 hi = *(const uint2*)(cp + 32);   // rows 16+4g..16+4g+3
            const i32x4 bi = {(int)lo.x, (int)lo.y, (int)hi.x, (int)hi.y};
            o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, __builtin_bit_cast(bf16x8, bi), o[d], 0, 0, 0);
        }
    }

    float l_tot = l_part + shfl_xor(l_part, 16);
    l_tot += shfl_xor(l_tot, 32);
    if (n_split == 1) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        float iv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) iv[i] = __shfl(inv, 4 * g + i, 64);
        float* oq = out + (int64_t)q * kHeads * kLat;
#pragma unroll
        for (int d = 0; d < 32; ++d)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                oq[(16 * wave + 4 * g + i) * kLat + 16 * d + l16] = o[d][i] * iv[i];
        if (lse != nullptr && g == 0)
            lse[(int64_t)q * kHeads + head] =
                l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : neg_inf();
    } else {
        float* po = part_o + ((int64_t)q * n_split + split) * kHeads * kLat;
#pragma unroll
        for (int d = 0; d < 32; ++d)
#pragma unroll
            for (int i = 0; i < 4; ++i) po[(16 * wave + 4 * g + i) * kLat + 16 * d + l16] = o[d][i];
        if (g == 0) {
            float* pm = part_ml + ((int64_t)q * n_split + split) * kHeads * 2;
            pm[2 * head] = m_run;
            pm[2 * head + 1] = l_tot;
        }
    }
}

// Combine the per-split partial results of each query with their log-sum-exp.
__global__ __launch_bounds__(kThreads) void sparse_mla_merge(const float* __restrict__ part_o,
                                                             const float* __restrict__ part_ml,
                                                             int n_split, float* __restrict__ out,
                                                             float* __restrict__ lse) {
    const int q = blockIdx.x;
    const int dim4 = threadIdx.x & 127;        // float4 column
    for (int h = threadIdx.x >> 7; h < kHeads; h += 2) {
        float mx = neg_inf();
        for (int s = 0; s < n_split; ++s)
            mx = fmaxf(mx, part_ml[(((int64_t)q * n_split + s) * kHeads + h) * 2]);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        float lsum = 0.f;
        if (mx != neg_inf()) {
            for (int s = 0; s < n_split; ++s) {
                const float* pm = part_ml + (((int64_t)q * n_split + s) * kHeads + h) * 2;
                const float wgt = exp2_(pm[0] - mx);
                lsum += wgt * pm[1];
                const f32x4 v = *(const f32x4*)(part_o + (((int64_t)q * n_split + s) * kHeads + h) * kLat + 4 * dim4);
                acc += wgt * v;
            }
        }
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        *(f32x4*)(out + ((int64_t)q * kHeads + h) * kLat + 4 * dim4) = acc * inv;
        if (lse != nullptr && dim4 == 0)
            lse[(int64_t)q * kHeads + h] = lsum > 0.f ? (mx + log2f(lsum)) * 0.69314718055994531f : neg_inf();
    }
}

int choose_split(int n_q, int k) {
    int s = 1;
    while (s < 32 && n_q * s < 256 && (k / (2 * s)) % kBlk == 0 && k / (2 * s) >= kBlk) s *= 2;
    return s;
}

}  // namespace

size_t mla_workspace_bytes(int n_q, int n_heads, int k) {
    const int s = choose_split(n_q, k);
    if (s == 1) return 0;
    return (size_t)n_q * s * n_heads * (kLat + 2) * sizeof(float);
}

hipError_t launch_sparse_mla(const void* q_lat, const void* q_rope, const void* kv,
                             const int32_t* q_seq, const int32_t* idx, int k, int n_q, int n_heads,
                             int64_t n_cap, float scale, float* out, float* lse, void* ws,
                             hipStream_t st) {
    (void)n_heads;
    const int s = choose_split(n_q, k);
    const int rows = k / s;
    const size_t lds = 2 * kBuf + kMaxRows * sizeof(int32_t);
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)sparse_mla_kernel,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    float* part_o = (float*)ws;
    float* part_ml = s > 1 ? part_o + (size_t)n_q * s * kHeads * kLat : nullptr;
    const float scale_log2 = scale * 1.4426950408889634f;
    hipLaunchKernelGGL(sparse_mla_kernel, dim3(s, n_q), dim3(kThreads), lds, st,
                       (const uint8_t*)q_lat, (const uint8_t*)q_rope, (const uint8_t*)kv, q_seq, idx,
                       k, n_cap, scale_log2, rows, out, lse, part_o, part_ml);
    if (s > 1)
        hipLaunchKernelGGL(sparse_mla_merge, dim3(n_q), dim3(kThreads), 0, st, part_o, part_ml, s,
                           out, lse);
    return hipGetLastError();
}

}  // namespace gsa

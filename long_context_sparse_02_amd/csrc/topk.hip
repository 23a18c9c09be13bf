// Causal top-k (k = 2048) with ties toward the lower position, on gfx950.
//
// "GLM-5.2 架构深度拆解" §1.1 and CH2 §2.2: an F layer keeps the 2048
// highest-scoring history positions of each query as its sparse attention set.
//
// Method: exact radix select on order-preserving uint32 keys of the fp32
// scores (-0 folded onto +0), then an ordered compaction.
//   pass 1  histogram of key bits 31..21 (2048 bins) over positions 0..pos
//   pass 2  histogram of bits 20..10 among keys in the pass-1 threshold bin
//   pass 3  histogram of bits 9..0 among keys in the pass-2 threshold bin
//           -> T, the k-th largest key, n_gt keys above it, need = k - n_gt
//   count   per chunk: keys > T and keys == T
//   compact per chunk, in position order: keys > T, and keys == T whose rank
//           among equal keys (in position order) is below `need`
// Every row is split into 16K-score chunks, one work-group each, so a single
// 1M-long row spreads over 64 CUs. Cross-chunk state is integer histograms
// built with atomic adds (order-free, hence deterministic) and per-chunk
// counts combined in chunk order, so the output is the same on every run.
// Output positions are ascending; rows with <= k valid positions select all
// of them and pad with -1.
#include "device_common.h"
#include "launch.h"

namespace gsa {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 16384;       // scores per work-group
constexpr int kB1 = 2048, kB2 = 2048, kB3 = 1024;
constexpr int kHistWords = kB1 + kB2 + kB3;

struct Ws {
    uint32_t* hist;     // [n_q][kHistWords]
    uint32_t* counts;   // [n_q][n_chunks][2]  (gt, eq)
    uint32_t* state;    // [n_q][4]  (T, n_gt, need, valid)
};

__device__ __forceinline__ Ws ws_of(void* base, int n_q, int n_chunks) {
    Ws w;
    w.hist = (uint32_t*)base;
    w.counts = w.hist + (size_t)n_q * kHistWords;
    w.state = w.counts + (size_t)n_q * n_chunks * 2;
    return w;
}

// Exclusive prefix sum over the 256 threads of the block (in thread order);
// also returns the block total. `scratch` holds >= 4 words.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* scratch, uint32_t& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) scratch[wave] = x;
    __syncthreads();
    uint32_t before = 0;
    total = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t t = scratch[i];
        if (i < wave) before += t;
        total += t;
    }
    __syncthreads();
    return before + x - v;
}

// In a histogram `h` (LDS, nb bins), find the bin b where the count of keys in
// bins >= b first reaches `need`, scanning from the top. Returns b and the
// count strictly above it (through LDS, visible to all threads).
__device__ void find_bin(const uint32_t* h, int nb, uint32_t need, uint32_t* scratch,
                         int* out_bin, uint32_t* out_above) {
    const int per = nb / kThreads;          // 8 or 4 consecutive bins per thread
    const int t = threadIdx.x;
    if (t == 0) { *out_bin = 0; *out_above = 0; }
    // thread t owns bins [nb - per*(t+1), nb - per*t): thread order = descending bins
    const int hi = nb - per * t;
    uint32_t s = 0;
    for (int b = hi - 1; b >= hi - per; --b) s += h[b];
    uint32_t total;
    uint32_t run = block_excl_scan(s, scratch, total);   // count in bins above this thread's range
    for (int b = hi - 1; b >= hi - per; --b) {
        const uint32_t c = h[b];
        if (run < need && run + c >= need) {
            *out_bin = b;
            *out_above = run;
        }
        run += c;
    }
    __syncthreads();
}

// A thread's share of one chunk: kPer float4 loads issued together before any
// is used (each thread owns float4 slots tid, tid + 256, ...), so a pass costs
// one memory round trip instead of kPer. Slots past the valid range read as
// -inf and are skipped by the callers' bounds test.
constexpr int kPer = kChunk / (4 * kThreads);   // 16 float4 per thread
__device__ __forceinline__ void load_chunk(const float* row, int64_t s0, int64_t s1, f32x4 (&v)[kPer]) {
    const f32x4* r4 = (const f32x4*)(row + s0);
    const int64_t n4 = (s1 - s0 + 3) >> 2;           // float4 slots touching [s0, s1)
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int64_t j = (int64_t)i * kThreads + threadIdx.x;
        if (j < n4) {
            if (s0 + 4 * j + 4 <= s1) v[i] = r4[j];
            else {                                      // ragged tail of the row
                f32x4 t = {neg_inf(), neg_inf(), neg_inf(), neg_inf()};
                for (int e = 0; e < 4; ++e)
                    if (s0 + 4 * j + e < s1) t[e] = row[s0 + 4 * j + e];
                v[i] = t;
            }
        } else {
            v[i] = f32x4{neg_inf(), neg_inf(), neg_inf(), neg_inf()};
        }
    }
}

__global__ __launch_bounds__(kThreads) void topk_zero(uint32_t* hist, int n_q) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t n = (int64_t)n_q * kB1;
    if (i < n) hist[(i / kB1) * kHistWords + (i % kB1)] = 0u;
}

// pass 1..3: histogram of one radix digit over the chunk's valid positions.
template <int PASS>
__global__ __launch_bounds__(kThreads) void topk_hist(const float* __restrict__ scores, int64_t ld,
                                                      const int32_t* __restrict__ q_pos, int n_q,
                                                      int k, int n_chunks, void* ws_base) {
    __shared__ uint32_t h[2048];
    __shared__ uint32_t hprev[2048];
    __shared__ uint32_t scratch[8];
    __shared__ int sbin[2];
    __shared__ uint32_t sabove[2];
    const int q = blockIdx.y, c = blockIdx.x;
    Ws w = ws_of(ws_base, n_q, n_chunks);
    const int64_t len = (int64_t)q_pos[q] + 1;
    if (len <= k) return;                             // selects everything; nothing to rank
    const int64_t s0 = (int64_t)c * kChunk;
    const int64_t s1 = min(s0 + kChunk, len);
    uint32_t* hq = w.hist + (size_t)q * kHistWords;
    // the pass that follows accumulates into the next histogram: clear it now
    if (c == 0 && PASS < 3) {
        uint32_t* nxt = hq + (PASS == 1 ? kB1 : kB1 + kB2);
        const int nb = PASS == 1 ? kB2 : kB3;
        for (int i = threadIdx.x; i < nb; i += kThreads) nxt[i] = 0u;
    }
    if (s0 >= s1) return;
    constexpr int NB = PASS == 3 ? kB3 : 2048;
    for (int i = threadIdx.x; i < NB; i += kThreads) h[i] = 0u;

    // threshold prefix from the earlier passes
    uint32_t prefix = 0;
    if (PASS >= 2) {
        for (int i = threadIdx.x; i < kB1; i += kThreads) hprev[i] = hq[i];
        __syncthreads();
        find_bin(hprev, kB1, (uint32_t)k, scratch, &sbin[0], &sabove[0]);
        prefix = (uint32_t)sbin[0];
        if (PASS == 3) {
            for (int i = threadIdx.x; i < kB2; i += kThreads) hprev[i] = hq[kB1 + i];
            __syncthreads();
            find_bin(hprev, kB2, (uint32_t)k - sabove[0], scratch, &sbin[1], &sabove[1]);
            prefix = (prefix << 11) | (uint32_t)sbin[1];
        }
    }
    __syncthreads();

    const float* row = scores + (int64_t)q * ld;
    f32x4 v[kPer];
    load_chunk(row, s0, s1, v);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int64_t p0 = s0 + 4 * ((int64_t)i * kThreads + threadIdx.x);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (p0 + e >= s1) continue;
            const uint32_t key = score_key(v[i][e]);
            if (PASS == 1) atomicAdd(&h[key >> 21], 1u);
            else if (PASS == 2) { if ((key >> 21) == prefix) atomicAdd(&h[(key >> 10) & 2047u], 1u); }
            else { if ((key >> 10) == prefix) atomicAdd(&h[key & 1023u], 1u); }
        }
    }
    __syncthreads();
    uint32_t* dst = hq + (PASS == 1 ? 0 : PASS == 2 ? kB1 : kB1 + kB2);
    for (int i = threadIdx.x; i < NB; i += kThreads)
        if (h[i]) atomicAdd(&dst[i], h[i]);
}

// Resolve T from the three histograms; count keys > T and == T per chunk.
__global__ __launch_bounds__(kThreads) void topk_count(const float* __restrict__ scores, int64_t ld,
                                                       const int32_t* __restrict__ q_pos, int n_q,
                                                       int k, int n_chunks, void* ws_base) {
    __shared__ uint32_t hprev[2048];
    __shared__ uint32_t scratch[8];
    __shared__ int sbin[3];
    __shared__ uint32_t sabove[3];
    const int q = blockIdx.y, c = blockIdx.x;
    Ws w = ws_of(ws_base, n_q, n_chunks);
    const int64_t len = (int64_t)q_pos[q] + 1;
    const int64_t s0 = (int64_t)c * kChunk;
    if (len <= k || s0 >= len) return;
    const int64_t s1 = min(s0 + kChunk, len);
    const uint32_t* hq = w.hist + (size_t)q * kHistWords;
    for (int i = threadIdx.x; i < kB1; i += kThreads) hprev[i] = hq[i];
    __syncthreads();
    find_bin(hprev, kB1, (uint32_t)k, scratch, &sbin[0], &sabove[0]);
    for (int i = threadIdx.x; i < kB2; i += kThreads) hprev[i] = hq[kB1 + i];
    __syncthreads();
    find_bin(hprev, kB2, (uint32_t)k - sabove[0], scratch, &sbin[1], &sabove[1]);
    for (int i = threadIdx.x; i < kB3; i += kThreads) hprev[i] = hq[kB1 + kB2 + i];
    __syncthreads();
    find_bin(hprev, kB3, (uint32_t)k - sabove[0] - sabove[1], scratch, &sbin[2], &sabove[2]);
    const uint32_t T = ((uint32_t)sbin[0] << 21) | ((uint32_t)sbin[1] << 10) | (uint32_t)sbin[2];
    const uint32_t n_gt = sabove[0] + sabove[1] + sabove[2];

    const float* row = scores + (int64_t)q * ld;
    uint32_t gt = 0, eq = 0;
    f32x4 v[kPer];
    load_chunk(row, s0, s1, v);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int64_t p0 = s0 + 4 * ((int64_t)i * kThreads + threadIdx.x);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (p0 + e >= s1) continue;
            const uint32_t key = score_key(v[i][e]);
            gt += key > T;
            eq += key == T;
        }
    }
    uint32_t tg, te;
    block_excl_scan(gt, scratch, tg);
    block_excl_scan(eq, scratch + 4, te);
    if (threadIdx.x == 0) {
        w.counts[((size_t)q * n_chunks + c) * 2 + 0] = tg;
        w.counts[((size_t)q * n_chunks + c) * 2 + 1] = te;
        if (c == 0) {
            w.state[q * 4 + 0] = T;
            w.state[q * 4 + 1] = n_gt;
            w.state[q * 4 + 2] = (uint32_t)k - n_gt;
        }
    }
}

// Ordered compaction: every selected position, ascending, into idx[q][...].
__global__ __launch_bounds__(kThreads) void topk_compact(const float* __restrict__ scores, int64_t ld,
                                                         const int32_t* __restrict__ q_pos, int n_q,
                                                         int k, int n_chunks, void* ws_base,
                                                         int32_t* __restrict__ idx) {
    __shared__ uint32_t scratch[8];
    __shared__ uint32_t sbase[2];
    const int q = blockIdx.y, c = blockIdx.x;
    Ws w = ws_of(ws_base, n_q, n_chunks);
    const int64_t len = (int64_t)q_pos[q] + 1;
    int32_t* out = idx + (int64_t)q * k;
    const int64_t s0 = (int64_t)c * kChunk;
    if (len <= k) {
        // every valid position is selected; pad with -1
        if (c == 0)
            for (int j = threadIdx.x; j < k; j += kThreads) out[j] = j < len ? j : -1;
        return;
    }
    if (s0 >= len) return;
    const int64_t s1 = min(s0 + kChunk, len);
    const uint32_t T = w.state[q * 4 + 0];
    const uint32_t need = w.state[q * 4 + 2];
    // counts of the chunks before this one (in chunk order)
    if (threadIdx.x == 0) {
        uint32_t gb = 0, eb = 0;
        for (int cc = 0; cc < c; ++cc) {
            gb += w.counts[((size_t)q * n_chunks + cc) * 2 + 0];
            eb += w.counts[((size_t)q * n_chunks + cc) * 2 + 1];
        }
        sbase[0] = gb;
        sbase[1] = eb;
    }
    __syncthreads();
    const uint32_t eq_before = sbase[1];
    uint32_t out_run = sbase[0] + min(eq_before, need);   // output slot of the next selected key
    uint32_t eq_run = eq_before;                          // equal keys seen before the sub-block

    const float* row = scores + (int64_t)q * ld;
    f32x4 v[kPer];
    load_chunk(row, s0, s1, v);
    // sub-block i holds 4 consecutive scores per thread, so thread order is
    // position order inside it and sub-blocks follow each other
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int64_t b0 = s0 + (int64_t)i * 4 * kThreads;
        if (b0 >= s1) break;                                 // uniform over the block
        const int64_t p0 = b0 + 4 * threadIdx.x;
        uint32_t key[4];
        bool valid[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            valid[e] = p0 + e < s1;
            key[e] = valid[e] ? score_key(v[i][e]) : 0u;
        }
        uint32_t n_eq = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) n_eq += valid[e] && key[e] == T;
        uint32_t eq_tot;
        uint32_t eq_rank = eq_run + block_excl_scan(n_eq, scratch, eq_tot);
        bool sel[4];
        uint32_t n_sel = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            bool s = false;
            if (valid[e]) {
                if (key[e] > T) s = true;
                else if (key[e] == T) { s = eq_rank < need; ++eq_rank; }
            }
            sel[e] = s;
            n_sel += s;
        }
        uint32_t sel_tot;
        uint32_t o = out_run + block_excl_scan(n_sel, scratch + 4, sel_tot);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (sel[e]) {
                if (o < (uint32_t)k) out[o] = (int32_t)(p0 + e);   // guard: never past the row
                ++o;
            }
        out_run += sel_tot;
        eq_run += eq_tot;
    }
}

}  // namespace

size_t topk_workspace_bytes(int n_q, int64_t ld, int k) {
    (void)k;
    const int64_t n_chunks = (ld + kChunk - 1) / kChunk;
    return ((size_t)n_q * kHistWords + (size_t)n_q * n_chunks * 2 + (size_t)n_q * 4) * 4;
}

hipError_t launch_topk(const float* scores, int64_t ld, const int32_t* q_pos, int n_q, int k,
                       int32_t* idx, void* ws, hipStream_t st) {
    const int n_chunks = (int)((ld + kChunk - 1) / kChunk);
    const dim3 grid(n_chunks, n_q), block(kThreads);
    const int64_t nz = (int64_t)n_q * kB1;
    hipLaunchKernelGGL(topk_zero, dim3((unsigned)((nz + kThreads - 1) / kThreads)), block, 0, st,
                       (uint32_t*)ws, n_q);
    hipLaunchKernelGGL(topk_hist<1>, grid, block, 0, st, scores, ld, q_pos, n_q, k, n_chunks, ws);
    hipLaunchKernelGGL(topk_hist<2>, grid, block, 0, st, scores, ld, q_pos, n_q, k, n_chunks, ws);
    hipLaunchKernelGGL(topk_hist<3>, grid, block, 0, st, scores, ld, q_pos, n_q, k, n_chunks, ws);
    hipLaunchKernelGGL(topk_count, grid, block, 0, st, scores, ld, q_pos, n_q, k, n_chunks, ws);
    hipLaunchKernelGGL(topk_compact, grid, block, 0, st, scores, ld, q_pos, n_q, k, n_chunks, ws, idx);
    return hipGetLastError();
}

}  // namespace gsa

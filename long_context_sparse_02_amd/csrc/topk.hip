// Causal top-k (k = 2048) with ties toward the lower position, on gfx950.
//
// "GLM-5.2 架构深度拆解" §1.1 and CH2 §2.2: an F layer keeps the 2048
// highest-scoring history positions of each query as its sparse attention set.
//
// Order: (score descending, position ascending) is a strict total order on the
// positions 0..pos of a row, so the top-k set is unique, and it is contained in
// the union of the top-k sets of any partition of the row. The selection runs
// as a tree over that fact:
//   level 1  one work-group per 16K-score chunk: each wave holds 2048
//            consecutive scores in registers (32 per lane) as order-preserving
//            uint32 keys (-0 folded onto +0). The k-th largest key T is found
//            by bisection over [min, max]: every step counts keys >= mid with
//            one ballot and popcount per 64 keys plus an 8-wave sum, so no
//            histogram or atomic is involved; ties at T keep the lowest
//            positions. An ordered compaction (ballot ranks) writes the
//            chunk's top-k as (key, position) pairs in position order;
//   level 2+ one work-group merges up to 8 lists of a row (concatenated in
//            chunk order, hence in position order) with the same selection,
//            until one list remains.
// The last level writes the positions (ascending) and pads with -1. The row is
// read from HBM once; no counter or histogram is shared between work-groups,
// so the result is the same on every run.
#include "device_common.h"
#include "launch.h"

namespace gsa {
namespace {

constexpr int kK = 2048;
constexpr int kChunk = 16384;                  // scores per level-1 work-group
constexpr int kFan = 8;                        // lists per merge work-group
constexpr int kMaxItems = kFan * kK;           // = kChunk
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr size_t kListBytes = 16 + (size_t)kK * 8; // count (16-byte slot) + (key, position) pairs

constexpr int kPer = kMaxItems / kThreads;      // items per lane (32)
constexpr int kSeg = 64 * kPer;                 // items per wave (2048)

constexpr int kBins = 256;                     // 8-bit radix digit

struct Scratch {
    uint32_t hist[2][kWaves][kBins];            // per-wave digit histograms, double-buffered
    uint32_t wsum[kWaves];
    uint32_t weq[kWaves];
    uint32_t wmin[kWaves];
    uint32_t wmax[kWaves];
    uint32_t wtot[4];
    uint32_t pick[3];                           // chosen bin, count above it, count in it
};

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
    return v;
}
__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, 64));
    return v;
}
// The fp32 value of an order-preserving key (inverse of score_key).
__device__ __forceinline__ float key_value(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}
// A value every lane of the wave holds (read from LDS after a barrier, or a
// wave reduction), moved to a scalar register so that branches on it are
// scalar branches.
__device__ __forceinline__ uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v += (uint32_t)__shfl_xor((int)v, o, 64);
    return v;
}
// number of set bits of `mask` in lanes below this one
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Sum over the block of a per-wave value (uniform inside each wave).
__device__ __forceinline__ uint32_t block_sum(uint32_t wave_val, Scratch& sc, uint32_t* before = nullptr) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) sc.wsum[wave] = wave_val;
    __syncthreads();
    uint32_t tot = 0, bef = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const uint32_t t = sc.wsum[w];
        bef += w < wave ? t : 0u;
        tot += t;
    }
    __syncthreads();
    if (before) *before = bef;
    return tot;
}

__device__ __forceinline__ void clear_hist(Scratch& sc, int b) {
    uint4* h = (uint4*)&sc.hist[b][0][0];                       // kWaves*kBins/4 = kThreads
    h[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
}

// Item i = kSeg*wave + 64*r + lane of the block is v[r] of that lane (valid for
// i < n; kFull: n = kMaxItems). The items are in position order. Selects the
// min(k, n) largest by (key desc, position asc) and emits them in position
// order through emit(slot, i, r). Returns the number emitted.
//
// Threshold: the k-th largest key T is found by radix selection on keys
// relative to the block minimum: each pass histograms the next 8 bits of the
// candidates (the keys inside the bin chosen by the previous pass), then keeps
// the bin where the count of larger keys first reaches k. A pass ends the
// search early when its bin is taken whole; otherwise the last pass leaves a
// single key value T and the number `need` of its copies to keep, which are
// the lowest positions among them.
template <bool kFull, typename Emit>
__device__ __forceinline__ int select_regs(const uint32_t (&v)[kPer], int n, Scratch& sc, Emit emit) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int seg0 = kSeg * wave;
    auto valid = [&](int r) { return kFull || seg0 + 64 * r + lane < n; };
    if (!kFull && n <= kK) {                                  // everything is kept
        uint32_t c = 0;
#pragma unroll
        for (int r = 0; r < kPer; ++r) c += __builtin_popcountll(__builtin_amdgcn_ballot_w64(valid(r)));
        uint32_t slot;
        block_sum(c, sc, &slot);
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            const uint64_t m = __builtin_amdgcn_ballot_w64(valid(r));
            if (valid(r)) emit(slot + lanes_below(m), seg0 + 64 * r + lane, r);
            slot += __builtin_popcountll(m);
        }
        return n < 0 ? 0 : n;
    }
    // ---- min / max of the valid keys
    uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
    for (int r = 0; r < kPer; ++r)
        if (valid(r)) { mn = min(mn, v[r]); mx = max(mx, v[r]); }
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (lane == 0) { sc.wmin[wave] = mn; sc.wmax[wave] = mx; }
    clear_hist(sc, 0);
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) { mn = min(mn, sc.wmin[w]); mx = max(mx, sc.wmax[w]); }
    mn = uni(mn);
    mx = uni(mx);

    // ---- Search for the k-th key. Candidates are the keys in [lo, hi], the exact
    // key range of the bin chosen last (at first: all keys). Each pass
    // histograms the candidates into 256 bins and keeps the bin where the count
    // of candidates in it and above first reaches `need`. Bins are linear in the
    // score value while the range is wide (keys crowd into a few exponents, so
    // bins of key bits would put most lanes of a wave on two or three
    // counters); once the range is narrow they are the top bits of key - lo.
    // Both are monotone in the key, lo lands in bin 0 and hi in the last used
    // bin, so each pass shrinks the range.
    uint32_t lo = mn, hi = mx, need = kK, in_bin = 0;
    uint32_t sel_w = 0, in_bin_w = 0;      // this wave: keys above the current bin, keys in it
    bool whole = false;                    // the last bin was taken whole: keys >= lo are the set
    int buf = 0;
    auto pick_bin = [&](uint32_t& b, uint32_t& above, uint32_t& tot_b) {
        // after the histogram of sc.hist[buf] is complete (uniform over the block)
        __syncthreads();
        clear_hist(sc, buf ^ 1);
        uint32_t tot = 0, sfx = 0;
        if (threadIdx.x < kBins) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) tot += sc.hist[buf][w][threadIdx.x];
            sfx = tot;                                         // suffix sum within the wave
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t t = (uint32_t)__shfl_down((int)sfx, o, 64);
                if (lane + o < 64) sfx += t;
            }
            if (lane == 0) sc.wtot[wave] = sfx;
        }
        __syncthreads();
        if (threadIdx.x < kBins) {
#pragma unroll
            for (int w = 0; w < 4; ++w) sfx += w > wave ? sc.wtot[w] : 0u;
            if (sfx >= need && sfx - tot < need) {
                sc.pick[0] = threadIdx.x;
                sc.pick[1] = sfx - tot;
                sc.pick[2] = tot;
            }
        }
        __syncthreads();
        b = uni(sc.pick[0]);
        above = uni(sc.pick[1]);
        tot_b = uni(sc.pick[2]);
        // this wave's share: its keys in bins above b (selected for good) and in b
        const uint4 hv = ((const uint4*)sc.hist[buf][wave])[lane];
        const uint32_t d0 = 4 * lane;
        uint32_t mine = (d0 > b ? hv.x : 0u) + (d0 + 1 > b ? hv.y : 0u) + (d0 + 2 > b ? hv.z : 0u) +
                        (d0 + 3 > b ? hv.w : 0u);
        sel_w += uni(wave_sum(mine));
        in_bin_w = uni(sc.hist[buf][wave][b]);
        buf ^= 1;
    };
    while (lo != hi) {                                         // uniform over the block
        const float flo = key_value(lo), fspan = key_value(hi) - flo;
        const bool by_value = hi - lo > 4096u && fspan > 1e-30f && fspan < 3.0e38f;
        const float inv = by_value ? 256.f / fspan : 0.f;
        const int nb = 32 - __builtin_clz(hi - lo);
        const int sh = nb > 8 ? nb - 8 : 0;
        auto bin_of = [&](uint32_t key) {
            return by_value ? min((int)((key_value(key) - flo) * inv), kBins - 1) : (int)((key - lo) >> sh);
        };
        uint32_t* h = sc.hist[buf][wave];
        // the empty asm keeps the compiler from hoisting 32 converted keys out of
        // the loop (registers that would cost a work-group of occupancy)
        if (by_value) {
#pragma unroll
            for (int r = 0; r < kPer; ++r) {
                uint32_t key = v[r];
                asm volatile("" : "+v"(key));
                if (valid(r) && key >= lo && key <= hi)
                    atomicAdd(&h[min((int)((key_value(key) - flo) * inv), kBins - 1)], 1u);
            }
        } else {
#pragma unroll
            for (int r = 0; r < kPer; ++r) {
                const uint32_t d = v[r] - lo;
                if (valid(r) && v[r] >= lo && d <= hi - lo) atomicAdd(&h[d >> sh], 1u);
            }
        }
        uint32_t b, above, tot_b;
        pick_bin(b, above, tot_b);
        need -= above;
        in_bin = tot_b;
        // exact key range of the chosen bin
        uint32_t nlo = 0xffffffffu, nhi = 0u;
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            uint32_t key = v[r];
            asm volatile("" : "+v"(key));     // recompute the bin: keeping 32 values live costs occupancy
            if (valid(r) && key >= lo && key <= hi && bin_of(key) == (int)b) {
                nlo = min(nlo, key);
                nhi = max(nhi, key);
            }
        }
        nlo = wave_min(nlo);
        nhi = wave_max(nhi);
        if (lane == 0) { sc.wmin[wave] = nlo; sc.wmax[wave] = nhi; }
        __syncthreads();
#pragma unroll
        for (int w = 0; w < kWaves; ++w) { nlo = min(nlo, sc.wmin[w]); nhi = max(nhi, sc.wmax[w]); }
        __syncthreads();
        lo = uni(nlo);
        hi = uni(nhi);
        if (in_bin == need) { whole = true; break; }
    }
    const uint32_t base = lo;
    // Selection. whole: every key >= lo (exactly k of them). Otherwise the
    // search ended on one key value T = lo with `in_bin` copies: keys > T,
    // plus the first `need` copies of T by position (all of them if need = in_bin).
    const uint32_t T = base;
    if (mx == mn) {                                            // no pass ran: every key is T
        in_bin = kFull ? (uint32_t)kMaxItems : (uint32_t)n;
        uint32_t c = 0;
#pragma unroll
        for (int r = 0; r < kPer; ++r) c += __builtin_popcountll(__builtin_amdgcn_ballot_w64(valid(r)));
        in_bin_w = c;
    }
    const bool partial = !whole && need != in_bin;
    if (!partial) { sel_w += in_bin_w; in_bin_w = 0; }
    // every wave's count of keys above T and of copies of T, from the histograms
    if (lane == 0) { sc.wsum[wave] = sel_w; sc.weq[wave] = in_bin_w; }
    __syncthreads();
    uint32_t slot = 0, eq_before = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        if (w < wave) {
            const uint32_t eq = sc.weq[w];
            const uint32_t taken = partial ? min(eq, need > eq_before ? need - eq_before : 0u) : 0u;
            slot += sc.wsum[w] + taken;
            eq_before += eq;
        }
    }
    auto take = [&](int r, uint32_t& eq_run) {                 // wave-uniform call
        if (!partial) return valid(r) && v[r] >= T;
        const bool in = valid(r);
        const uint64_t eqm = __builtin_amdgcn_ballot_w64(in && v[r] == T);
        const bool s = in && (v[r] > T || (v[r] == T && eq_run + lanes_below(eqm) < need));
        eq_run += __builtin_popcountll(eqm);
        return s;
    };
    {
        uint32_t eq_run = eq_before;
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            const bool s = take(r, eq_run);
            const uint64_t sm = __builtin_amdgcn_ballot_w64(s);
            const uint32_t my = slot + lanes_below(sm);
            if (s && my < (uint32_t)kK) emit(my, seg0 + 64 * r + lane, r);   // guard: never past k slots
            slot += __builtin_popcountll(sm);
        }
    }
    return kK;
}

__device__ __forceinline__ void write_final_pad(int32_t* out, int count) {
    for (int j = count + threadIdx.x; j < kK; j += kThreads) out[j] = -1;
}

// Level 1: chunk c of row q.
__global__ __launch_bounds__(kThreads) void topk_chunk(const float* __restrict__ scores, int64_t ld,
                                                       const int32_t* __restrict__ q_pos, int n_chunks,
                                                       uint8_t* __restrict__ lists, int32_t* __restrict__ idx) {
    __shared__ Scratch sc;
    const int q = blockIdx.y, c = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t len = (int64_t)q_pos[q] + 1;
    const int64_t s0 = (int64_t)c * kChunk;
    const int n = (int)max((int64_t)0, min(s0 + kChunk, len) - s0);
    const float* row = scores + (int64_t)q * ld + s0;
    // lane holds items kSeg*wave + 64r + lane: each wave load reads 256 contiguous bytes.
    // Loads are unconditional (clamped address) so all 32 are in flight together; a
    // branch around each would make the compiler wait for each one at the join.
    uint32_t v[kPer];
    if (n > 0) {
        float x[kPer];
#pragma unroll
        for (int r = 0; r < kPer; ++r) x[r] = row[min(kSeg * wave + 64 * r + lane, n - 1)];
#pragma unroll
        for (int r = 0; r < kPer; ++r) v[r] = kSeg * wave + 64 * r + lane < n ? score_key(x[r]) : 0u;
    } else {
#pragma unroll
        for (int r = 0; r < kPer; ++r) v[r] = 0u;
    }
    if (n_chunks == 1) {
        int32_t* out = idx + (int64_t)q * kK;
        auto em = [&](uint32_t slot, int i, int) { out[slot] = (int32_t)(s0 + i); };
        const int cnt = n == kMaxItems ? select_regs<true>(v, n, sc, em) : select_regs<false>(v, n, sc, em);
        write_final_pad(out, cnt);
    } else {
        uint8_t* L = lists + ((size_t)q * n_chunks + c) * kListBytes;
        uint2* items = (uint2*)(L + 16);
        auto em = [&](uint32_t slot, int i, int r) { items[slot] = make_uint2(v[r], (uint32_t)(s0 + i)); };
        const int cnt = n == kMaxItems ? select_regs<true>(v, n, sc, em) : select_regs<false>(v, n, sc, em);
        if (threadIdx.x == 0) *(uint32_t*)L = (uint32_t)cnt;
    }
}

// Level 2+: lists [kFan*g, kFan*g + kFan) of row q (n_in lists per row) into one.
__global__ __launch_bounds__(kThreads) void topk_merge(const uint8_t* __restrict__ in, int n_in,
                                                       uint8_t* __restrict__ out_lists, int n_out,
                                                       int32_t* __restrict__ idx) {
    __shared__ Scratch sc;
    __shared__ uint32_t base[kFan + 1];
    const int q = blockIdx.y, g = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l0 = g * kFan;
    const int nl = min(kFan, n_in - l0);
    if (threadIdx.x == 0) {
        uint32_t b = 0;
        for (int l = 0; l < nl; ++l) {
            base[l] = b;
            b += min(*(const uint32_t*)(in + ((size_t)q * n_in + l0 + l) * kListBytes), (uint32_t)kK);
        }
        base[nl] = b;
    }
    __syncthreads();
    const int n = (int)base[nl];
    // item i of the concatenation (lists in order) is item i - base[l] of list l
    uint32_t v[kPer], p[kPer];
    uint32_t bl[kFan];
#pragma unroll
    for (int j = 0; j < kFan; ++j) bl[j] = j < nl ? base[j] : 0xffffffffu;
    {
        uint2 it[kPer];
#pragma unroll
        for (int r = 0; r < kPer; ++r) {        // unconditional loads: all in flight together
            const int i = min(kSeg * wave + 64 * r + lane, max(n - 1, 0));
            int l = 0;
#pragma unroll
            for (int j = 1; j < kFan; ++j) l += (uint32_t)i >= bl[j] ? 1 : 0;
            it[r] = ((const uint2*)(in + ((size_t)q * n_in + l0 + l) * kListBytes + 16))[i - bl[l]];
        }
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            const bool ok = kSeg * wave + 64 * r + lane < n;
            v[r] = ok ? it[r].x : 0u;
            p[r] = ok ? it[r].y : 0u;
        }
    }
    if (n_out == 1) {
        int32_t* out = idx + (int64_t)q * kK;
        auto em = [&](uint32_t slot, int, int r) { out[slot] = (int32_t)p[r]; };
        const int cnt = n == kMaxItems ? select_regs<true>(v, n, sc, em) : select_regs<false>(v, n, sc, em);
        write_final_pad(out, cnt);
    } else {
        uint8_t* L = out_lists + ((size_t)q * n_out + g) * kListBytes;
        uint2* items = (uint2*)(L + 16);
        auto em = [&](uint32_t slot, int, int r) { items[slot] = make_uint2(v[r], p[r]); };
        const int cnt = n == kMaxItems ? select_regs<true>(v, n, sc, em) : select_regs<false>(v, n, sc, em);
        if (threadIdx.x == 0) *(uint32_t*)L = (uint32_t)cnt;
    }
}

int n_chunks_of(int64_t ld) { return (int)((ld + kChunk - 1) / kChunk); }

}  // namespace

size_t topk_workspace_bytes(int n_q, int64_t ld, int k) {
    (void)k;
    const int nc = n_chunks_of(ld);
    if (nc <= 1) return 16;
    const int n2 = (nc + kFan - 1) / kFan;
    return (size_t)n_q * (nc + n2) * kListBytes;
}

hipError_t launch_topk(const float* scores, int64_t ld, const int32_t* q_pos, int n_q, int k,
                       int32_t* idx, void* ws, hipStream_t st) {
    (void)k;
    const int nc = n_chunks_of(ld);
    uint8_t* a = (uint8_t*)ws;                                  // level-1 lists (n_q x nc)
    uint8_t* b = a + (size_t)n_q * nc * kListBytes;            // level-2 lists (n_q x nc/8)
    hipLaunchKernelGGL(topk_chunk, dim3(nc, n_q), dim3(kThreads), 0, st, scores, ld, q_pos, nc, a, idx);
    int n = nc;
    uint8_t* in = a;
    uint8_t* out = b;
    while (n > 1) {
        const int ng = (n + kFan - 1) / kFan;
        hipLaunchKernelGGL(topk_merge, dim3(ng, n_q), dim3(kThreads), 0, st, in, n, out, ng, idx);
        n = ng;
        uint8_t* t = in;
        in = out;
        out = t;
    }
    return hipGetLastError();
}

}  // namespace gsa

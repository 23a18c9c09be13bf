// Causal top-k (k = 2048) with ties toward the lower position, on gfx950.
//
// "GLM-5.2 架构深度拆解" §1.1 and CH2 §2.2: an F layer keeps the 2048
// highest-scoring history positions of each query as its sparse attention set.
//
// Order: (score descending, position ascending) is a strict total order on the
// positions 0..pos of a row, so the top-k set is unique. Scores compare as
// order-preserving uint32 keys (-0 folded onto +0).
//
// Selection core. select_regs holds the items of one 512-thread work-group in
// registers and finds the k-th key by radix-histogram passes: each pass counts
// the candidate keys (those in the exact key range of the bin chosen last)
// into 256 bins per wave in LDS, linear in the score value while the range is
// wide and then the top bits of key - lo, and keeps the bin where the count of
// keys in it and above first reaches the number still needed. select_wide is
// the same selection with one 2048-bin work-group histogram per pass (fewer
// passes and barriers). Emission is an ordered ballot compaction, ties at the
// threshold keeping the lowest positions.
//
// Bound. The largest score of every 32 positions (the score kernel writes these
// group maxima) bounds the selection: with L the k-th largest group maximum, at
// least k positions score >= L, so every selected score is >= L and lies in a
// group whose maximum reaches L (about k groups, whatever the row length).
//
// Final selection. The candidates that pass the bound have keys in [L, largest
// maximum], both known: select_final finds the 2048th key with one histogram
// pass over 2048 equal key ranges and one wave's rank of the range holding it
// (more than 64 items there, heavy ties: select_wide), then keeps every key
// above that item and the equal ones not after it.
//
// Kernels:
//   topk_row    rows of 64K to 1M positions: one work-group per row takes the
//               row's maxima, L, the list of groups that reach it, those groups'
//               scores only (each wave a contiguous share, compacted without
//               work-group barriers) and the final selection, in one launch.
//   topk_row_split
//               the same for launches of at most 128 rows, each row split over
//               2, 4 or 8 work-groups: every share bounds the whole row, lists
//               and streams its own part of the groups, and hands its
//               candidates over through the workspace (write-through stores,
//               then a flag set to the launch's tag); the share that finds every
//               flag of its row set runs the final selection and clears them.
//   topk_small  rows of at most 4096 positions: one work-group per row, the
//               row's smallest and largest key bounding select_final.
//   topk_chunk + topk_merge
//               other widths: one work-group per 16K-score chunk keeps its top
//               k as a (key, position) list in position order (with a bound
//               from topk_bound when the row has one), and one work-group per
//               row merges the lists (their union holds the row's top k).
//   topk_rescore
//               the selection without a score buffer: the groups that reach the
//               bound are rescored with the score kernel's arithmetic.
#include <atomic>
#include <chrono>
#include <type_traits>

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
// count (16-byte slot) + (key, position) pairs, rounded to whole 128-byte lines
constexpr size_t kListBytes = (16 + (size_t)kK * 8 + 127) / 128 * 128;

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

// Reductions over the 64 lanes of a wave, every lane active, without LDS: the
// two quad permutations and the half-row and row mirrors (DPP) combine the 16
// lanes of a row, then the gfx950 permlane16 / permlane32 swaps combine rows
// and halves (each step pairs disjoint lane sets, so the result is exact for a
// sum as well as for min and max).
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v, Op op) {
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xb1, 0xf, 0xf, false));   // lane ^ 1
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4e, 0xf, 0xf, false));   // lane ^ 2
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false));  // 7 - lane in 8
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false));  // 15 - lane in 16
    auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);                         // other row
    v = op((uint32_t)r[0], (uint32_t)r[1]);
    r = __builtin_amdgcn_permlane32_swap(v, v, false, false);                              // other half
    return op((uint32_t)r[0], (uint32_t)r[1]);
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
    return wave_reduce(v, [](uint32_t a, uint32_t b) { return max(a, b); });
}
__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
    return wave_reduce(v, [](uint32_t a, uint32_t b) { return min(a, b); });
}
// A value every lane of the wave holds (read from LDS after a barrier, or a
// wave reduction), moved to a scalar register so that branches on it are
// scalar branches.
__device__ __forceinline__ uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
    return wave_reduce(v, [](uint32_t a, uint32_t b) { return a + b; });
}
// number of set bits of `mask` in lanes below this one
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Work-group barrier for LDS traffic: this wave's LDS operations are complete
// (lgkmcnt 0), then s_barrier. Unlike __syncthreads it does not wait for the
// wave's global loads, so loads issued before a selection stay in flight
// through its barriers. Global stores are not ordered by it: no wave reads
// another wave's global stores inside a selection.
__device__ __forceinline__ void sync_lds() {
    __builtin_amdgcn_s_waitcnt(0xC07F);                         // lgkmcnt(0) only
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Sum over the block of a per-wave value (uniform inside each wave).
__device__ __forceinline__ uint32_t block_sum(uint32_t wave_val, Scratch& sc, uint32_t* before = nullptr) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) sc.wsum[wave] = wave_val;
    sync_lds();
    uint32_t tot = 0, bef = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const uint32_t t = sc.wsum[w];
        bef += w < wave ? t : 0u;
        tot += t;
    }
    sync_lds();
    if (before) *before = bef;
    return tot;
}

__device__ __forceinline__ void clear_hist(Scratch& sc, int b) {
    uint4* h = (uint4*)&sc.hist[b][0][0];                       // kWaves*kBins/4 = kThreads
    h[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
}

// Item i = 64*PER*wave + 64*r + lane of the block is v[r] of that lane; key 0 (the
// key of no score but a NaN with every bit set) marks an item that is not there
// (kFull: every item is). The items are in position order. Selects the min(k, #valid) largest valid items by (key desc,
// position asc) and emits them in position order through emit(slot, i, r).
// Returns the number emitted. With t_out (and at least k valid items) only the
// k-th largest key is found, stored to *t_out by every thread, and nothing is
// emitted.
//
// Threshold: the k-th largest key T is found by radix selection on keys
// relative to the block minimum: each pass histograms the next 8 bits of the
// candidates (the keys inside the bin chosen by the previous pass), then keeps
// the bin where the count of larger keys first reaches k. A pass ends the
// search early when its bin is taken whole; otherwise the last pass leaves a
// single key value T and the number `need` of its copies to keep, which are
// the lowest positions among them.
template <int PER, bool kFull, typename Emit>
__device__ __forceinline__ int select_regs(const uint32_t (&v)[PER], Scratch& sc, Emit emit,
                                           uint32_t* t_out = nullptr) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    constexpr int SEG = 64 * PER;                          // items per wave
    const int seg0 = SEG * wave;
    auto valid = [&](int r) { return kFull || v[r] != 0u; };
    uint32_t n_valid = kThreads * PER;
    if (!kFull) {
        uint32_t c = 0;
#pragma unroll
        for (int r = 0; r < PER; ++r) c += __builtin_popcountll(__builtin_amdgcn_ballot_w64(valid(r)));
        uint32_t slot;
        n_valid = uni(block_sum(uni(c), sc, &slot));
        if (n_valid <= (uint32_t)kK && t_out == nullptr) {    // everything is kept
#pragma unroll
            for (int r = 0; r < PER; ++r) {
                const uint64_t m = __builtin_amdgcn_ballot_w64(valid(r));
                if (valid(r)) emit(slot + lanes_below(m), seg0 + 64 * r + lane, r);
                slot += __builtin_popcountll(m);
            }
            return (int)n_valid;
        }
    }
    // ---- min / max of the valid keys
    uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
    for (int r = 0; r < PER; ++r)
        if (valid(r)) { mn = min(mn, v[r]); mx = max(mx, v[r]); }
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (lane == 0) { sc.wmin[wave] = mn; sc.wmax[wave] = mx; }
    clear_hist(sc, 0);
    sync_lds();
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
        sync_lds();
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
        sync_lds();
        if (threadIdx.x < kBins) {
#pragma unroll
            for (int w = 0; w < 4; ++w) sfx += w > wave ? sc.wtot[w] : 0u;
            if (sfx >= need && sfx - tot < need) {
                sc.pick[0] = threadIdx.x;
                sc.pick[1] = sfx - tot;
                sc.pick[2] = tot;
            }
        }
        sync_lds();
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
            for (int r = 0; r < PER; ++r) {
                uint32_t key = v[r];
                asm volatile("" : "+v"(key));
                if (valid(r) && key >= lo && key <= hi)
                    atomicAdd(&h[min((int)((key_value(key) - flo) * inv), kBins - 1)], 1u);
            }
        } else {
#pragma unroll
            for (int r = 0; r < PER; ++r) {
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
        for (int r = 0; r < PER; ++r) {
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
        sync_lds();
#pragma unroll
        for (int w = 0; w < kWaves; ++w) { nlo = min(nlo, sc.wmin[w]); nhi = max(nhi, sc.wmax[w]); }
        sync_lds();
        lo = uni(nlo);
        hi = uni(nhi);
        if (in_bin == need) { whole = true; break; }
    }
    const uint32_t base = lo;
    // Selection. whole: every key >= lo (exactly k of them). Otherwise the
    // search ended on one key value T = lo with `in_bin` copies: keys > T,
    // plus the first `need` copies of T by position (all of them if need = in_bin).
    const uint32_t T = base;
    if (t_out != nullptr) {                                    // the k-th largest key only
        *t_out = T;
        return 0;
    }
    if (mx == mn) {                                            // no pass ran: every key is T
        in_bin = n_valid;
        uint32_t c = 0;
#pragma unroll
        for (int r = 0; r < PER; ++r) c += __builtin_popcountll(__builtin_amdgcn_ballot_w64(valid(r)));
        in_bin_w = c;
    }
    const bool partial = !whole && need != in_bin;
    if (!partial) { sel_w += in_bin_w; in_bin_w = 0; }
    // every wave's count of keys above T and of copies of T, from the histograms
    if (lane == 0) { sc.wsum[wave] = sel_w; sc.weq[wave] = in_bin_w; }
    sync_lds();
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
        for (int r = 0; r < PER; ++r) {
            const bool s = take(r, eq_run);
            const uint64_t sm = __builtin_amdgcn_ballot_w64(s);
            const uint32_t my = slot + lanes_below(sm);
            if (s && my < (uint32_t)kK) emit(my, seg0 + 64 * r + lane, r);   // guard: never past k slots
            slot += __builtin_popcountll(sm);
        }
    }
    return kK;
}

// Inclusive prefix sum over the 64 lanes of a wave, every lane active, without
// LDS: shifts by 1, 2, 4 and 8 inside each row of 16 (lanes shifted in from
// outside the row add 0), then row 15's sum into rows 1 and 3 and lane 31's
// into rows 2 and 3 (DPP row broadcasts).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true);   // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true);   // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true);   // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true);   // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}

// The selection of select_regs (same items, same order, same result) with one
// work-group histogram of 2048 bins per pass instead of a 256-bin histogram
// per wave (the two views share Scratch::hist): each pass takes four
// barriers, and integer-valued scores, whose candidates span a few thousand
// units, usually resolve in one pass. Bins are linear in the score value while
// the key range is wide, then the top 11 bits of key - lo; thread t owns bins
// 4t .. 4t+3, and the bin holding the k-th key is found from a prefix sum over
// the threads (a DPP scan inside each wave, the wave totals through LDS).
constexpr int kWBins = kWaves * kBins;          // 2048

template <int PER, typename Emit>
__device__ __forceinline__ int select_wide(const uint32_t (&v)[PER], Scratch& sc, Emit emit,
                                           uint32_t* t_out = nullptr) {
    static_assert(kWBins == 4 * kThreads, "four bins per thread");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    constexpr int SEG = 64 * PER;
    const int seg0 = SEG * wave;
    uint32_t* const H[2] = {&sc.hist[0][0][0], &sc.hist[1][0][0]};
    // ---- count, min and max of the valid keys, one exchange
    uint32_t c = 0, mn = 0xffffffffu, mx = 0u;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
        c += __builtin_popcountll(__builtin_amdgcn_ballot_w64(v[r] != 0u));
        if (v[r] != 0u) { mn = min(mn, v[r]); mx = max(mx, v[r]); }
    }
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (lane == 0) { sc.wsum[wave] = c; sc.wmin[wave] = mn; sc.wmax[wave] = mx; }
    ((uint4*)H[0])[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
    sync_lds();
    uint32_t n_valid = 0, before = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const uint32_t x = sc.wsum[w];
        n_valid += x;
        before += w < wave ? x : 0u;
        mn = min(mn, sc.wmin[w]);
        mx = max(mx, sc.wmax[w]);
    }
    n_valid = uni(n_valid);
    mn = uni(mn);
    mx = uni(mx);
    if (n_valid <= (uint32_t)kK && t_out == nullptr) {          // everything is kept
        uint32_t slot = before;
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            const uint64_t m = __builtin_amdgcn_ballot_w64(v[r] != 0u);
            if (v[r] != 0u) emit(slot + lanes_below(m), seg0 + 64 * r + lane, r);
            slot += __builtin_popcountll(m);
        }
        return (int)n_valid;
    }
    // ---- the k-th largest key: candidates are the keys in [lo, hi] (the exact
    // key range of the bin chosen last); a pass keeps the bin where the count of
    // candidates in it and above first reaches `need`
    uint32_t lo = mn, hi = mx, need = kK, in_bin = n_valid;
    bool whole = false;                                         // the last bin was taken whole
    int buf = 0;
    while (lo != hi) {                                          // uniform
        uint32_t* h = H[buf];
        const float flo = key_value(lo), fspan = key_value(hi) - flo;
        const bool by_value = hi - lo > 4u * kWBins && fspan > 1e-30f && fspan < 3.0e38f;
        const float inv = by_value ? (float)kWBins / fspan : 0.f;
        const int nb = 32 - __builtin_clz(hi - lo);
        const int sh = nb > 11 ? nb - 11 : 0;
        auto bin_of = [&](uint32_t key) __attribute__((always_inline)) {
            return by_value ? min((int)((key_value(key) - flo) * inv), kWBins - 1) : (int)((key - lo) >> sh);
        };
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            uint32_t key = v[r];
            asm volatile("" : "+v"(key));                      // keep the bin math inside the loop
            if (key != 0u && key >= lo && key <= hi) atomicAdd(&h[bin_of(key)], 1u);
        }
        ((uint4*)H[buf ^ 1])[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);   // for the next pass
        sync_lds();
        const uint4 hb = ((const uint4*)h)[threadIdx.x];
        const uint32_t s4 = hb.x + hb.y + hb.z + hb.w;
        const uint32_t incl = wave_incl_scan(s4);
        if (lane == 63) sc.weq[wave] = incl;
        sync_lds();
        uint32_t above = 0;                                     // candidates in bins past this thread's 4
#pragma unroll
        for (int w = 0; w < kWaves; ++w) above += w > wave ? sc.weq[w] : 0u;
        above += (uint32_t)__builtin_amdgcn_readlane((int)incl, 63) - incl;
        const uint32_t cnt4[4] = {hb.w, hb.z, hb.y, hb.x};      // bins 4t+3 .. 4t
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (above < need && above + cnt4[q] >= need) {
                sc.pick[0] = 4 * threadIdx.x + 3 - q;
                sc.pick[1] = above;
                sc.pick[2] = cnt4[q];
            }
            above += cnt4[q];
        }
        sync_lds();
        const int b = (int)uni(sc.pick[0]);
        need -= uni(sc.pick[1]);
        in_bin = uni(sc.pick[2]);
        uint32_t nlo = 0xffffffffu, nhi = 0u;
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            uint32_t key = v[r];
            asm volatile("" : "+v"(key));
            if (key != 0u && key >= lo && key <= hi && bin_of(key) == b) {
                nlo = min(nlo, key);
                nhi = max(nhi, key);
            }
        }
        nlo = wave_min(nlo);
        nhi = wave_max(nhi);
        if (lane == 0) { sc.wmin[wave] = nlo; sc.wmax[wave] = nhi; }
        sync_lds();
#pragma unroll
        for (int w = 0; w < kWaves; ++w) { nlo = min(nlo, sc.wmin[w]); nhi = max(nhi, sc.wmax[w]); }
        lo = uni(nlo);
        hi = uni(nhi);
        buf ^= 1;
        if (in_bin == need) { whole = true; break; }
    }
    const uint32_t T = lo;
    if (t_out != nullptr) {
        *t_out = T;
        return 0;
    }
    // ---- emission: keys above T, then the first `need` copies of T (all of them
    // when the bin was taken whole or need = in_bin), in item order
    const bool partial = !whole && need != in_bin;
    uint32_t sel_w = 0, eq_w = 0;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
        sel_w += __builtin_popcountll(__builtin_amdgcn_ballot_w64(v[r] != 0u && (partial ? v[r] > T : v[r] >= T)));
        eq_w += partial ? __builtin_popcountll(__builtin_amdgcn_ballot_w64(v[r] == T)) : 0;
    }
    if (lane == 0) { sc.wsum[wave] = sel_w; sc.weq[wave] = eq_w; }
    sync_lds();
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
    uint32_t eq_run = eq_before;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
        bool sl;
        if (!partial) {
            sl = v[r] != 0u && v[r] >= T;
        } else {
            const bool in = v[r] != 0u;
            const uint64_t eqm = __builtin_amdgcn_ballot_w64(in && v[r] == T);
            sl = in && (v[r] > T || (v[r] == T && eq_run + lanes_below(eqm) < need));
            eq_run += __builtin_popcountll(eqm);
        }
        const uint64_t sm = __builtin_amdgcn_ballot_w64(sl);
        const uint32_t my = slot + lanes_below(sm);
        if (sl && my < (uint32_t)kK) emit(my, seg0 + 64 * r + lane, r);   // never past k slots
        slot += __builtin_popcountll(sm);
    }
    return kK;
}

// Bound of the row kernels: a key L such that at least kK valid items are >= L,
// in one histogram pass: the exact lower edge (in key space) of the one of 2048
// equal key ranges between the smallest and largest item that holds the kK-th
// largest item. Looser than the kK-th largest item by less than one range; 0
// (no bound) with fewer than kK valid items (key 0: no item). `largest` is
// the largest item (0 without one).
template <int PER>
__device__ __forceinline__ uint32_t bound_one_pass(const uint32_t (&v)[PER], Scratch& sc, uint32_t& largest) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t* const h = &sc.hist[0][0][0];
    uint32_t c = 0, mn = 0xffffffffu, mx = 0u;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
        c += __builtin_popcountll(__builtin_amdgcn_ballot_w64(v[r] != 0u));
        if (v[r] != 0u) { mn = min(mn, v[r]); mx = max(mx, v[r]); }
    }
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (lane == 0) { sc.wsum[wave] = c; sc.wmin[wave] = mn; sc.wmax[wave] = mx; }
    ((uint4*)h)[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
    sync_lds();
    uint32_t n = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        n += sc.wsum[w];
        mn = min(mn, sc.wmin[w]);
        mx = max(mx, sc.wmax[w]);
    }
    n = uni(n);
    mn = uni(mn);
    mx = uni(mx);
    largest = mx;
    if (n < (uint32_t)kK) return 0u;                            // uniform
    if (mn == mx) return mn;
    const int nb = 32 - __builtin_clz(mx - mn);
    const int sh = nb > 11 ? nb - 11 : 0;                       // (key - mn) >> sh < 2048
#pragma unroll
    for (int r = 0; r < PER; ++r) {
        uint32_t key = v[r];
        asm volatile("" : "+v"(key));
        if (key != 0u) atomicAdd(&h[(key - mn) >> sh], 1u);
    }
    sync_lds();
    const uint4 hb = ((const uint4*)h)[threadIdx.x];
    const uint32_t incl = wave_incl_scan(hb.x + hb.y + hb.z + hb.w);
    if (lane == 63) sc.weq[wave] = incl;
    sync_lds();
    uint32_t above = 0;                                         // items in bins past this thread's 4
#pragma unroll
    for (int w = 0; w < kWaves; ++w) above += w > wave ? sc.weq[w] : 0u;
    above += (uint32_t)__builtin_amdgcn_readlane((int)incl, 63) - incl;
    const uint32_t cnt4[4] = {hb.w, hb.z, hb.y, hb.x};          // bins 4t+3 .. 4t
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (above < (uint32_t)kK && above + cnt4[q] >= (uint32_t)kK) sc.pick[0] = 4 * threadIdx.x + 3 - q;
        above += cnt4[q];
    }
    sync_lds();
    return mn + (uni(sc.pick[0]) << sh);
}

// The top kK of the candidates v (keys, 0: none; item i = 64 PER wave + 64 r +
// lane in position order, positions p), n of them valid and every key in [lo,
// hi], written to out[] as ascending positions. One histogram pass over 2048
// equal key ranges of [lo, hi] finds the range that holds the kK-th largest
// key; one wave ranks that range's items by (key descending, item ascending),
// which names the last selected item (T, iT): an item is selected iff its key
// exceeds T, or equals T and the item is not after iT. A range of more than 64
// items (heavy ties) goes to select_wide. The caller zeroes sc.hist[0] before
// a barrier that precedes the call. Returns the number written.
template <int PER>
__device__ __forceinline__ int select_final(const uint32_t (&v)[PER], const uint32_t (&p)[PER], uint32_t lo,
                                            uint32_t hi, uint32_t n, int32_t* out, Scratch& sc) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int seg0 = 64 * PER * wave;
    uint32_t T = 1u, iT = 0xffffffffu;                          // n <= kK: every valid item
    if (n > (uint32_t)kK) {                                     // uniform
        uint32_t* const h = &sc.hist[0][0][0];
        const int nb = hi > lo ? 32 - __builtin_clz(hi - lo) : 0;
        const int sh = nb > 11 ? nb - 11 : 0;                   // (key - lo) >> sh < 2048
        // (clamped, so keys outside [lo, hi], which valid inputs never hold, stay in bounds)
        auto range = [&](uint32_t key) { return min((key - lo) >> sh, (uint32_t)(kWBins - 1)); };
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            uint32_t key = v[r];
            asm volatile("" : "+v"(key));
            if (key != 0u) atomicAdd(&h[range(key)], 1u);
        }
        if (threadIdx.x == 0) sc.wtot[0] = 0u;                  // the range's item count, below
        sync_lds();
        const uint4 hb = ((const uint4*)h)[threadIdx.x];
        const uint32_t incl = wave_incl_scan(hb.x + hb.y + hb.z + hb.w);
        if (lane == 63) sc.weq[wave] = incl;
        sync_lds();
        uint32_t above = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) above += w > wave ? sc.weq[w] : 0u;
        above += (uint32_t)__builtin_amdgcn_readlane((int)incl, 63) - incl;
        const uint32_t cnt4[4] = {hb.w, hb.z, hb.y, hb.x};      // ranges 4t+3 .. 4t
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (above < (uint32_t)kK && above + cnt4[q] >= (uint32_t)kK) {
                sc.pick[0] = 4 * threadIdx.x + 3 - q;
                sc.pick[1] = above;
                sc.pick[2] = cnt4[q];
            }
            above += cnt4[q];
        }
        sync_lds();
        const uint32_t b = uni(sc.pick[0]), need = (uint32_t)kK - uni(sc.pick[1]), nin = uni(sc.pick[2]);
        if (nin > 64u)                                          // uniform: heavy ties at the threshold
            return select_wide<PER>(v, sc, [&](uint32_t slot, int, int r) { out[slot] = (int32_t)p[r]; });
        uint32_t* const lst = &sc.hist[1][0][0];                // (key, item) of the range's items
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            if (v[r] != 0u && range(v[r]) == b) {
                const uint32_t at = atomicAdd(&sc.wtot[0], 1u);
                lst[2 * at] = v[r];
                lst[2 * at + 1] = (uint32_t)(seg0 + 64 * r + lane);
            }
        }
        sync_lds();
        if (wave == 0) {
            const uint32_t kl = lane < (int)nin ? lst[2 * lane] : 0u;
            const uint32_t il = lane < (int)nin ? lst[2 * lane + 1] : 0xffffffffu;
            uint32_t rank = 0;                                  // items of the range before this one
            for (uint32_t m = 0; m < nin; ++m) {                // uniform
                const uint32_t km = (uint32_t)__builtin_amdgcn_readlane((int)kl, (int)m);
                const uint32_t im = (uint32_t)__builtin_amdgcn_readlane((int)il, (int)m);
                rank += (km > kl || (km == kl && im < il)) ? 1u : 0u;
            }
            if (lane < (int)nin && rank == need - 1u) {
                sc.pick[0] = kl;
                sc.pick[1] = il;
            }
        }
        sync_lds();
        T = uni(sc.pick[0]);
        iT = uni(sc.pick[1]);
    }
    // ---- emission in item order
    bool sl[PER];
    uint32_t c = 0;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
        const uint32_t i = (uint32_t)(seg0 + 64 * r + lane);
        sl[r] = v[r] != 0u && (v[r] > T || (v[r] == T && i <= iT));
        c += __builtin_popcountll(__builtin_amdgcn_ballot_w64(sl[r]));
    }
    if (lane == 0) sc.wsum[wave] = c;
    sync_lds();
    uint32_t slot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) slot += w < wave ? sc.wsum[w] : 0u;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
        const uint64_t m = __builtin_amdgcn_ballot_w64(sl[r]);
        if (sl[r]) out[slot + lanes_below(m)] = (int32_t)p[r];
        slot += __builtin_popcountll(m);
    }
    return (int)min(n, (uint32_t)kK);
}

__device__ __forceinline__ void write_final_pad(int32_t* out, int count) {
    for (int j = count + threadIdx.x; j < kK; j += kThreads) out[j] = -1;
}

// Row q's causal length (never past the row: positions must be < ld).
__device__ __forceinline__ int64_t row_len(const int32_t* q_pos, int q, int64_t ld) {
    return min((int64_t)q_pos[q] + 1, ld);
}

// Group maxima of rows whose scores came without them: work-group (c, q) covers
// positions [16K c, 16K c + 16K) of row q; positions past q's own are -inf.
__global__ __launch_bounds__(kThreads) void topk_group_max(const float* __restrict__ scores, int64_t ld,
                                                           const int32_t* __restrict__ q_pos,
                                                           float* __restrict__ gmax, int64_t ldg) {
    const int q = blockIdx.y, c = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t len = row_len(q_pos, q, ld);
    const int64_t s0 = (int64_t)c * kChunk + kSeg * wave;
    const float* row = scores + (int64_t)q * ld;
    float x[kPer];
#pragma unroll
    for (int r = 0; r < kPer; ++r) x[r] = row[min(s0 + 64 * r + lane, ld - 1)];
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
        const int64_t s = s0 + 64 * r + lane;               // groups: lanes 0-31 and 32-63
        const uint32_t m = max_x32(score_key(s < len && s < ld ? x[r] : neg_inf()));
        const int64_t grp = (s0 + 64 * r) / kGroup + (lane >> 5);
        if ((lane & 31) == 0 && grp < ldg) gmax[(int64_t)q * ldg + grp] = key_value(m);
    }
}

// Bound: L(q) = the k-th largest maximum over the full 32-position groups of row
// q, or 0 (no bound) with fewer than k full groups. At most kSmall items take
// part: beyond that, runs of rg adjacent groups count as one (the maximum of
// the run), which keeps the bound valid and only loosens it.
constexpr int kPerSmall = 8;                   // items per lane of the small selections
constexpr int kSmall = kThreads * kPerSmall;   // 4096 items

__global__ __launch_bounds__(kThreads) void topk_bound(const float* __restrict__ gmax, int64_t ldg,
                                                       const int32_t* __restrict__ q_pos,
                                                       uint32_t* __restrict__ bound) {
    __shared__ Scratch sc;
    const int q = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t n_full = row_len(q_pos, q, ldg * kGroup) / kGroup;
    if (n_full < kK) {
        if (threadIdx.x == 0) bound[q] = 0u;
        return;
    }
    const int64_t rg = (n_full + kSmall - 1) / kSmall;       // groups per item
    const int n_items = (int)((n_full + rg - 1) / rg);
    const float* gm = gmax + (int64_t)q * ldg;
    uint32_t v[kPerSmall];                                    // 0: no item
#pragma unroll
    for (int r = 0; r < kPerSmall; ++r) v[r] = 0u;
    // item i is the maximum of groups i, i + n_items, i + 2 n_items, ... (< n_full):
    // consecutive lanes read consecutive groups; 4 group runs per load batch
    auto take = [&](int64_t j, const float (&x)[kPerSmall]) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < kPerSmall; ++r) {
            const int i = 64 * kPerSmall * wave + 64 * r + lane;
            if (i < n_items && j * n_items + i < n_full) v[r] = max(v[r], score_key(x[r]));
        }
    };
    auto load = [&](int64_t j, float (&x)[kPerSmall]) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < kPerSmall; ++r)
            x[r] = __builtin_nontemporal_load(gm + min(j * n_items + 64 * kPerSmall * wave + 64 * r + lane, n_full - 1));
    };
    int64_t j = 0;
    for (; j + 4 <= rg; j += 4) {                            // uniform
        float x0[kPerSmall], x1[kPerSmall], x2[kPerSmall], x3[kPerSmall];
        load(j, x0); load(j + 1, x1); load(j + 2, x2); load(j + 3, x3);
        take(j, x0); take(j + 1, x1); take(j + 2, x2); take(j + 3, x3);
    }
    for (; j + 2 <= rg; j += 2) {                            // 2-round rows: one latency
        float x0[kPerSmall], x1[kPerSmall];
        load(j, x0); load(j + 1, x1);
        take(j, x0); take(j + 1, x1);
    }
    for (; j < rg; ++j) {
        float x0[kPerSmall];
        load(j, x0);
        take(j, x0);
    }
    uint32_t T = 0;
    select_regs<kPerSmall, false>(v, sc, [](uint32_t, int, int) {}, &T);
    if (threadIdx.x == 0) bound[q] = T;
}

// Chunk c of row q: its keys >= the row's bound (all keys without one), cut to
// their top k. One list per chunk, or the final indices when the row has one chunk.
__global__ __launch_bounds__(kThreads) void topk_chunk(const float* __restrict__ scores, int64_t ld,
                                                       const int32_t* __restrict__ q_pos, int n_chunks,
                                                       const uint32_t* __restrict__ bound,
                                                       uint8_t* __restrict__ lists, int32_t* __restrict__ idx) {
    __shared__ Scratch sc;
    const int q = blockIdx.y, c = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t s0 = (int64_t)c * kChunk;
    const float* row = scores + (int64_t)q * ld + s0;
    // lane holds items kSeg*wave + 64r + lane: each wave load reads 256 contiguous bytes.
    // Loads are unconditional (clamped address) so all 32 are in flight together; a
    // branch around each would make the compiler wait for each one at the join.
    // Each score is read once: non-temporal loads (prefill top-k 1.7-3.4% faster).
    // The clamp keeps the loads inside the row (ld), not inside the causal length,
    // and no branch depends on it, so they do not wait for q_pos: positions past
    // the length (a whole chunk, for short rows) are masked below.
    uint32_t v[kPer];                                         // 0: not a candidate
    int n;
    uint32_t L;
    {
        const int lim = (int)min((int64_t)kChunk, ld - s0) - 1;
        float x[kPer];
#pragma unroll
        for (int r = 0; r < kPer; ++r) x[r] = __builtin_nontemporal_load(row + min(kSeg * wave + 64 * r + lane, lim));
        asm volatile("" ::: "memory");                        // the row's length and bound are read after
        const int64_t len = row_len(q_pos, q, ld);
        n = (int)max((int64_t)0, min(s0 + kChunk, len) - s0);
        L = bound != nullptr ? uni(bound[q]) : 0u;
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            const uint32_t key = score_key(x[r]);
            v[r] = (kSeg * wave + 64 * r + lane < n && key >= L) ? key : 0u;
        }
    }
    const bool full = n == kMaxItems && L == 0u;                // uniform
    if (n_chunks == 1) {
        int32_t* out = idx + (int64_t)q * kK;
        auto em = [&](uint32_t slot, int i, int) { out[slot] = (int32_t)(s0 + i); };
        const int cnt = full ? select_regs<kPer, true>(v, sc, em) : select_regs<kPer, false>(v, sc, em);
        write_final_pad(out, cnt);
    } else {
        uint8_t* Lst = lists + ((size_t)q * n_chunks + c) * kListBytes;
        uint2* items = (uint2*)(Lst + 16);
        auto em = [&](uint32_t slot, int i, int r) { items[slot] = make_uint2(v[r], (uint32_t)(s0 + i)); };
        const int cnt = full ? select_regs<kPer, true>(v, sc, em) : select_regs<kPer, false>(v, sc, em);
        if (threadIdx.x == 0) *(uint32_t*)Lst = (uint32_t)cnt;
    }
}

// Rows of at most 4096 positions (kPerSmall = 8 per lane): the smallest and
// largest valid keys of the row bound select_final's one histogram pass, so the
// row needs one reduction and one selection instead of select_regs' passes
// (4 rows of 4096 positions: 10.9 against 19.7 us per call).
__global__ __launch_bounds__(kThreads) void topk_small(const float* __restrict__ scores, int64_t ld,
                                                       const int32_t* __restrict__ q_pos,
                                                       int32_t* __restrict__ idx) {
    __shared__ Scratch sc;
    const int q = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float* row = scores + (int64_t)q * ld;
    const int lim = (int)ld - 1;
    float x[kPerSmall];
#pragma unroll
    for (int r = 0; r < kPerSmall; ++r)                         // clamped, unconditional: all in flight
        x[r] = __builtin_nontemporal_load(row + min(64 * kPerSmall * wave + 64 * r + lane, lim));
    asm volatile("" ::: "memory");
    const int n = (int)row_len(q_pos, q, ld);
    uint32_t v[kPerSmall], pos[kPerSmall];
    uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
    for (int r = 0; r < kPerSmall; ++r) {
        const int i = 64 * kPerSmall * wave + 64 * r + lane;    // item i = position i
        const uint32_t key = score_key(x[r]);
        const bool ok = i < n;
        v[r] = ok ? key : 0u;
        pos[r] = (uint32_t)i;
        mn = ok ? min(mn, key) : mn;
        mx = ok ? max(mx, key) : mx;
    }
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (lane == 0) {
        sc.wmin[wave] = mn;
        sc.wmax[wave] = mx;
    }
    ((uint4*)&sc.hist[0][0][0])[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);   // for select_final
    sync_lds();
    uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        lo = min(lo, sc.wmin[w]);
        hi = max(hi, sc.wmax[w]);
    }
    int32_t* out = idx + (int64_t)q * kK;
    const int cnt = select_final<kPerSmall>(v, pos, lo, hi, (uint32_t)n, out, sc);
    write_final_pad(out, cnt);
}

// ---- One work-group per row, or a few per row -------------------------------
// For rows of up to 512 * GPL groups whose group maxima are known. The top-k
// set lies in the groups whose maximum reaches the bound L, and with L the
// kK-th largest maximum those are about kK groups whatever the row length
// (kK x 128 bytes of scores), so a row is selected from its maxima and those
// groups' scores alone:
//   1. every group maximum of the row into registers (group 512 i + t in
//      thread t, round i); L = the kK-th largest of 4096 items, each the
//      largest of GPL / 8 of a thread's maxima: at least kK positions score
//      >= L, so every selected score is >= L. Fewer than kK items (a row of
//      fewer groups): no bound.
//   2. the groups whose maximum reaches L, in position order, into an LDS list.
//   3. the scores of a contiguous share of the list, each wave its own part of
//      the share, compacted into per-wave candidate parts in position order.
//   4. the top kK of the candidates, written as ascending positions, -1 padded.
// Split rows (few rows per launch): work-groups (q, p), p < pn, all find the
// same L and list, each streams share p of the list (step 3) and writes its
// candidates to its region of the workspace, then sets its flag to the
// launch's tag; a work-group that then finds every flag of the row set runs
// step 4 over all regions (two may, with identical results) and clears the
// flags, so a replay of the same launch starts clean and a workspace of any
// prior contents works. The hand-over uses device-scope stores and loads
// (written through to, and read from, the device's coherence point), and each
// wave waits for its stores to complete before the flag is set, so no L2
// write-back (a release fence: microseconds per wave) is needed. A part that
// overflows (ties at the bound, rows without one), or more than 2 kK
// candidates in all, sends the row to a batched fallback over the whole list
// in the work-group that runs step 4; a share with more than its window of
// 2 kK / pn candidates costs one more round trip to load them compacted.
struct SplitArgs {
    unsigned long long* flags;   // [row][share]: the tag of the launch that filled the share
    uint8_t* regions;            // [row][share]: candidate count, then (score bits, position) pairs
    unsigned long long tag;      // this launch's tag (never 0)
    int pn;                      // shares per row: 2, 4 or 8
};
constexpr int kMaxShares = 8;
constexpr size_t kRegionHead = 128;
constexpr size_t kRegionBytes = kRegionHead + (size_t)2 * kK * sizeof(uint2);

__device__ __forceinline__ void store_dev(unsigned long long* p, unsigned long long v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long load_dev(const unsigned long long* p) {
    return __hip_atomic_load(const_cast<unsigned long long*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// this wave's stores and loads are complete (also a compiler barrier)
__device__ __forceinline__ void drain_vm() {
    asm volatile("" ::: "memory");
    wait_vmcnt<0>();
    asm volatile("" ::: "memory");
}

template <int GPL, int kEnt, bool kSplit>
__device__ __forceinline__ void topk_row_body(const float* __restrict__ scores, int64_t ld,
                                              const int32_t* __restrict__ q_pos,
                                              const float* __restrict__ gmax, int64_t ldg, bool al16,
                                              int32_t* __restrict__ idx, const SplitArgs& sa) {
    constexpr int kMaxGroups = kThreads * GPL;
    constexpr int IPL = kPerSmall;                 // bound items per thread: 4096 in all
    constexpr int GPI = GPL / IPL;                 // maxima per item
    static_assert(GPL % IPL == 0 && kMaxGroups <= 65536, "GPL");
    constexpr int kWaveCap = 2 * kK / kWaves;      // candidates a wave's part holds (512)
    constexpr int R4 = GPL / 4;                    // rounds of 4 groups per thread
    struct Lds {
        Scratch sc;
        uint2 pend[2 * kK];                        // candidates (key, position), in position order
        uint2 ptrash[kThreads];                    // where a lane writes what it does not keep
        alignas(16) uint8_t nib[kMaxGroups / 4];   // passing groups: 4 per byte, bit g % 4
        f32x4 ent_x[kWaves][kEnt];                 // per wave: loads that hold a candidate (scores,
        int ent_p[kWaves][kEnt];                   // first position)
        uint32_t wtot[kWaves];
        uint32_t wmin[kWaves];
        uint32_t wcnt[kWaves];                     // candidates per wave part (all ones: overflow)
        uint16_t glist[kMaxGroups];                // passing groups, in position order
    };
    __shared__ __attribute__((aligned(16))) Lds s;
    const int q = blockIdx.x;
    const int share = kSplit ? (int)blockIdx.y : 0, pn = kSplit ? sa.pn : 1;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t len = row_len(q_pos, q, ld);
    const int ng = (int)((len + kGroup - 1) / kGroup);          // groups with a causal position
    const float* grow = gmax + (int64_t)q * ldg;
    const float* srow = scores + (int64_t)q * ld;
    int32_t* out = idx + (int64_t)q * kK;

    // ---- 1. the maxima and the bound. Round i of thread t holds groups
    // 2048 i + 4 t .. + 3: one 16-byte load when the maxima rows are 16-byte
    // aligned (al16), else four 4-byte loads; gk[4 i + c] is group 2048 i + 4 t + c.
    // The work-groups of a split row all read the row's maxima, so they are
    // cached loads there, and non-temporal ones otherwise.
    auto load_maxima = [&](uint32_t (&g)[GPL]) __attribute__((always_inline)) {
        if (al16) {                                             // uniform
#pragma unroll
            for (int i = 0; i < R4; ++i) {
                const f32x4* a = (const f32x4*)(grow + min(2048 * i + 4 * t, (int)ldg - 4));
                const f32x4 x = kSplit ? *a : __builtin_nontemporal_load(a);
#pragma unroll
                for (int c = 0; c < 4; ++c) g[4 * i + c] = score_key(x[c]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < R4; ++i)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float* a = grow + min(2048 * i + 4 * t + c, max(ng - 1, 0));
                    g[4 * i + c] = score_key(kSplit ? *a : __builtin_nontemporal_load(a));
                }
        }
#pragma unroll
        for (int i = 0; i < R4; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c) g[4 * i + c] = 2048 * i + 4 * t + c < ng ? g[4 * i + c] : 0u;   // 0: no causal group
    };
    uint32_t gk[GPL];
    load_maxima(gk);
    uint32_t L, Mx;                                             // the bound, the largest maximum
    {
        uint32_t it[IPL];
#pragma unroll
        for (int k = 0; k < IPL; ++k) {
            uint32_t m = 0u;
#pragma unroll
            for (int j = 0; j < GPI; ++j) m = max(m, gk[GPI * k + j]);
            it[k] = m;
        }
        L = bound_one_pass<IPL>(it, s.sc, Mx);
    }
    // ---- 2. the groups of words w0 .. w1 - 1 (64 groups each) that reach L, in
    // position order: every thread writes a 4-bit mask per round (a byte in
    // LDS), then lists the groups of a few consecutive masks after those of the
    // lower threads (a scan of the counts). Returns their number.
    auto build_list = [&](const uint32_t (&g)[GPL], int w0, int w1) __attribute__((always_inline)) {
        const int g0 = 64 * w0, g1 = 64 * w1;
#pragma unroll
        for (int i = 0; i < R4; ++i) {
            if (2048 * (i + 1) <= g0 || 2048 * i >= g1) continue;   // uniform: round outside the words
            const int b = 2048 * i + 4 * t;
            uint32_t m = 0u;
#pragma unroll
            for (int c = 0; c < 4; ++c) m |= (g[4 * i + c] != 0u && g[4 * i + c] >= L) ? 1u << c : 0u;
            if (b >= g0 && b < g1) s.nib[(b - g0) >> 2] = (uint8_t)m;
        }
        sync_lds();
        // thread t takes mask bytes t B .. t B + B - 1 (groups g0 + 4 t B ..): few
        // per thread, so that dense lists (half the groups of a 128K row) are
        // written by many threads at once
        const int nbytes = (g1 - g0) >> 2;
        int B = 1;
        while (B * kThreads < nbytes) B <<= 1;                  // <= 16
        uint64_t word = 0ull;
        for (int k = 0; k < B; ++k) {
            const int j = t * B + k;
            if (j < nbytes) word |= (uint64_t)s.nib[j] << (4 * k);
        }
        const uint32_t cw = (uint32_t)__builtin_popcountll(word);
        const uint32_t incl = wave_incl_scan(cw);
        if (lane == 63) s.wtot[wave] = incl;
        sync_lds();
        uint32_t before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const uint32_t x = s.wtot[w];
            before += w < wave ? x : 0u;
            total += x;
        }
        uint32_t o = before + incl - cw;
        while (word != 0ull) {                                  // about 5 groups per word at the bound
            s.glist[o++] = (uint16_t)(g0 + 4 * B * t + __builtin_ctzll(word));
            word &= word - 1;
        }
        sync_lds();
        return (int)uni(total);
    };
    // this work-group's words: the row's, or (split rows) its share of them
    const int nwr = (ng + 63) / 64;
    int P = build_list(gk, kSplit ? (int)((int64_t)nwr * share / pn) : 0,
                       kSplit ? (int)((int64_t)nwr * (share + 1) / pn) : nwr);   // >= kK with a bound, else ng

    // ---- 3. candidates of the passing groups. Usual case: wave w streams its own
    // contiguous part of the list, 64 groups (2048 scores, 32 per lane) at a
    // time with the next 64 in flight, and appends its keys >= L in position
    // order to its own part of the LDS candidate list, without work-group
    // barriers. The parts (and the shares of a split row) are contiguous and in
    // order, so the parts, concatenated, are in position order.
    auto gpos = [&](int gi, int e) __attribute__((always_inline)) {
        return (int64_t)s.glist[min(gi, max(P, 1) - 1)] * kGroup + e;
    };
    {
        const int gs = (int)(((int64_t)P * wave) / kWaves), ge = (int)(((int64_t)P * (wave + 1)) / kWaves);
        uint2* part = s.pend + kWaveCap * wave;
        uint32_t cnt = 0;
        bool over = false;
        const int nsb = (ge - gs + 63) / 64;
        // sub-batch j, load r: lane l reads scores 4 (l % 8) .. + 3 of group
        // gs + 64 j + 8 r + l / 8 (16 bytes; a start past the row's last full
        // 4 is moved back to ld - 4, and its positions are masked by len).
        // Scores are compared as floats against the bound's value (the order of
        // the keys; -0 equals +0 as floats), so only the kept ones are turned
        // into keys, at the end; the part holds (score bits, position).
        constexpr int NL = 8;                                   // 16-byte loads per lane per sub-batch
        const float Lf = L == 0u ? neg_inf() : key_value(L);
        auto sb_groups = [&](int j, int (&g)[NL]) __attribute__((always_inline)) {
#pragma unroll
            for (int r = 0; r < NL; ++r) g[r] = s.glist[min(gs + 64 * j + 8 * r + (lane >> 3), ge - 1)];
        };
        auto sb_load = [&](const int (&g)[NL], f32x4 (&x)[NL]) __attribute__((always_inline)) {
#pragma unroll
            for (int r = 0; r < NL; ++r) {
                const int64_t p = min((int64_t)g[r] * kGroup + 4 * (lane & 7), ld - 4);
                x[r] = __builtin_nontemporal_load((const f32x4*)(srow + p));
            }
        };
        const int len32 = (int)len;
        f32x4 x[NL];
        int g[NL];
        if (nsb > 0) {
            sb_groups(0, g);
            sb_load(g, x);
        }
        for (int j = 0; j < nsb; ++j) {                        // uniform in the wave
            f32x4 xc[NL];
            int lim[NL], p0[NL];                                // positions p0 .. p0 + lim - 1 count
#pragma unroll
            for (int r = 0; r < NL; ++r) {
                xc[r] = x[r];
                p0[r] = g[r] * kGroup + 4 * (lane & 7);
                lim[r] = gs + 64 * j + 8 * r + (lane >> 3) < ge ? len32 - p0[r] : 0;
            }
            if (j + 1 < nsb) {                                  // in flight while this one is compacted
                sb_groups(j + 1, g);
                sb_load(g, x);
            }
            // two levels, per half sub-batch: (a) the loads whose largest score
            // reaches the bound (about 1 in 6) go, in order, to this wave's entry
            // list; (b) lane e of a round of 64 entries keeps that entry's scores
            // >= the bound after those of the lower lanes (a wave scan of the
            // counts), in position order
#pragma unroll
            for (int h = 0; h < NL / 4; ++h) {
                uint32_t ecnt = 0;
#pragma unroll
                for (int r = 4 * h; r < 4 * h + 4; ++r) {
                    const bool b = (xc[r][0] >= Lf) | (xc[r][1] >= Lf) | (xc[r][2] >= Lf) | (xc[r][3] >= Lf);
                    const bool bl = b & (lim[r] > 0);
                    const uint64_t m = __builtin_amdgcn_ballot_w64(bl);
                    const uint32_t slot = ecnt + lanes_below(m);
                    if (bl & (slot < (uint32_t)kEnt)) {
                        s.ent_x[wave][slot] = xc[r];
                        s.ent_p[wave][slot] = p0[r];
                    }
                    ecnt += (uint32_t)__builtin_popcountll(m);
                }
                over = over || ecnt > (uint32_t)kEnt;
                for (uint32_t k = 0; k < ecnt && !over; k += 64) {      // uniform
                    const uint32_t ei = min(k + lane, (uint32_t)kEnt - 1);
                    const f32x4 xe = s.ent_x[wave][ei];
                    const int pe = s.ent_p[wave][ei];
                    const int le = k + lane < ecnt ? len32 - pe : 0;
                    uint32_t f[4], c = 0;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        f[e] = ((xe[e] >= Lf) & (e < le)) ? 1u : 0u;
                        c += f[e];
                    }
                    const uint32_t incl = wave_incl_scan(c);
                    const uint32_t n = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
                    over = over || cnt + n > (uint32_t)kWaveCap;
                    uint32_t at = cnt + incl - c;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        uint2* dst = (f[e] != 0u && !over) ? part + at : s.ptrash + t;
                        *dst = make_uint2(__float_as_uint(xe[e]), (uint32_t)(pe + e));
                        at += f[e];
                    }
                    cnt += n;
                }
            }
        }
        if (lane == 0) s.wcnt[wave] = over ? 0xffffffffu : cnt;
    }
    ((uint4*)&s.sc.hist[0][0][0])[t] = make_uint4(0u, 0u, 0u, 0u);   // for step 4
    sync_lds();
    uint32_t off[kWaves + 1];
    bool any_over = false;
    off[0] = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const uint32_t c = s.wcnt[w];
        any_over = any_over || c == 0xffffffffu;
        off[w + 1] = off[w] + (c == 0xffffffffu ? 0u : c);
    }
    if constexpr (kSplit) {
        // ---- hand-over: this share's candidates (compacted, in position order)
        // and their count (all ones: a part overflowed) to its region, then its flag
        uint8_t* reg = sa.regions + ((size_t)q * pn + share) * kRegionBytes;
        unsigned long long* ent = (unsigned long long*)(reg + kRegionHead);
        unsigned long long* flag = sa.flags + (size_t)q * pn;
        const uint32_t total = off[kWaves];
        if (!any_over) {
            for (uint32_t i = t; i < total; i += kThreads) {
                int w = 0;
#pragma unroll
                for (int u = 1; u < kWaves; ++u) w += i >= off[u] ? 1 : 0;
                const uint2 e = s.pend[kWaveCap * w + (i - off[w])];
                store_dev(ent + i, ((unsigned long long)e.y << 32) | e.x);
            }
        }
        if (t == 0) store_dev((unsigned long long*)reg, any_over ? 0xffffffffull : (unsigned long long)total);
        drain_vm();                                             // every store of this wave is complete
        sync_lds();                                             // ... and of every wave
        ((uint4*)&s.sc.hist[0][0][0])[t] = make_uint4(0u, 0u, 0u, 0u);   // for step 4
        if (wave == 0) {                                        // lane u reads share u's flag
            if (lane == 0) store_dev(flag + share, sa.tag);
            drain_vm();
            const unsigned long long f = load_dev(flag + (lane < pn ? lane : 0));
            const uint64_t set = __builtin_amdgcn_ballot_w64(lane >= pn || f == sa.tag);
            if (lane == 0) s.wtot[0] = set == ~0ull ? 1u : 0u;
        }
        sync_lds();
        if (uni(s.wtot[0]) == 0u) return;                       // uniform: a later share finishes the row
        // ---- 4. the top kK of every share's candidates: share u's first W
        // entries are items u W .. u W + W - 1, in position order across shares
        static_assert(2 * kK == 1 << 12, "two selections' worth of items is 2^12");
        const int wsh = 12 - __builtin_ctz((unsigned)pn);       // W = 2 kK / pn = 2^wsh
        const int W = 1 << wsh;
        const uint8_t* rrow = sa.regions + (size_t)q * pn * kRegionBytes;
        unsigned long long x[kPerSmall];
#pragma unroll
        for (int r = 0; r < kPerSmall; ++r) {
            const int i = 64 * kPerSmall * wave + 64 * r + lane;     // < 2 kK = pn W
            x[r] = load_dev((const unsigned long long*)(rrow + (size_t)(i >> wsh) * kRegionBytes + kRegionHead) +
                            (i & (W - 1)));
        }
        uint32_t cnt_u[kMaxShares];                             // 0 past the row's shares
#pragma unroll
        for (int u = 0; u < kMaxShares; ++u) {
            const uint32_t c = (uint32_t)load_dev((const unsigned long long*)(rrow + (size_t)(u < pn ? u : 0) * kRegionBytes));
            cnt_u[u] = u < pn ? c : 0u;
        }
        bool fits = true, over = false;                         // every share in its window; a part overflowed
        uint32_t n = 0;
#pragma unroll
        for (int u = 0; u < kMaxShares; ++u) {
            over = over || cnt_u[u] == 0xffffffffu;
            fits = fits && cnt_u[u] <= (uint32_t)W;
            n += cnt_u[u] == 0xffffffffu ? 0u : cnt_u[u];
        }
        if (t < pn) store_dev(flag + t, 0ull);                  // every share has arrived: clear for the next launch
        if (!over && n <= (uint32_t)(2 * kK)) {                 // uniform
            if (!fits) {
                // a share holds more than its window (candidates clustered in
                // part of the row): load again, compacted, item i being entry i -
                // roff[u] of share u
                uint32_t roff[kMaxShares + 1];
                roff[0] = 0;
#pragma unroll
                for (int u = 0; u < kMaxShares; ++u) roff[u + 1] = roff[u] + cnt_u[u];
#pragma unroll
                for (int r = 0; r < kPerSmall; ++r) {
                    const uint32_t i = 64 * kPerSmall * wave + 64 * r + lane;
                    int u = 0;
#pragma unroll
                    for (int j = 1; j < kMaxShares; ++j) u += (j < pn && i >= roff[j]) ? 1 : 0;
                    x[r] = load_dev((const unsigned long long*)(rrow + (size_t)u * kRegionBytes + kRegionHead) +
                                    min(i - roff[u], (uint32_t)(2 * kK - 1)));
                }
            }
            uint32_t pv[kPerSmall], pp[kPerSmall];
#pragma unroll
            for (int r = 0; r < kPerSmall; ++r) {
                const int i = 64 * kPerSmall * wave + 64 * r + lane;
                uint32_t c = cnt_u[0];
#pragma unroll
                for (int u = 1; u < kMaxShares; ++u) c = (i >> wsh) == u ? cnt_u[u] : c;
                const bool valid = fits ? (uint32_t)(i & (W - 1)) < c : (uint32_t)i < n;
                pv[r] = valid ? score_key(__uint_as_float((uint32_t)x[r])) : 0u;
                pp[r] = (uint32_t)(x[r] >> 32);
            }
            const int cnt = select_final<kPerSmall>(pv, pp, L == 0u ? 1u : L, Mx, n, out, s.sc);
            write_final_pad(out, cnt);
            return;
        }
    } else if (!any_over) {                                     // uniform
        // ---- 4. the top kK of the concatenated parts (at most kWaves * kWaveCap = 4096)
        uint32_t pv[kPerSmall], pp[kPerSmall];
#pragma unroll
        for (int r = 0; r < kPerSmall; ++r) {
            const uint32_t i = 64 * kPerSmall * wave + 64 * r + lane;
            int w = 0;
#pragma unroll
            for (int u = 1; u < kWaves; ++u) w += i >= off[u] ? 1 : 0;
            const uint2 e = s.pend[kWaveCap * w + min(i - off[w], (uint32_t)kWaveCap - 1)];
            pv[r] = i < off[kWaves] ? score_key(__uint_as_float(e.x)) : 0u;
            pp[r] = e.y;
        }
        const int cnt = select_final<kPerSmall>(pv, pp, L == 0u ? 1u : L, Mx, off[kWaves], out, s.sc);
        write_final_pad(out, cnt);
        return;
    }

    // ---- Fallback (a part overflowed: ties at the bound, or a row too short for
    // one; split rows: also more than 2 kK candidates in all): the whole list's
    // groups again, 256 per batch (a smaller batch keeps this rare path's
    // registers below the usual path's): item (r, lane) of wave w is position
    // lane % 32 of group glist[256 b + 32 w + 2 r + lane / 32]; a batch's keys
    // >= thr are cut to their top kK and appended to the candidate list in
    // position order; a list of more than kK is first cut to its top kK and thr
    // becomes one above the kK-th key (a later position with that key loses the
    // tie).
    constexpr int kFb = 16;                                     // items per lane
    constexpr int kGb = kThreads * kFb / kGroup;                // groups per batch
    auto load = [&](int b, float (&x)[kFb]) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < kFb; ++r)
            x[r] = __builtin_nontemporal_load(
                srow + min(gpos(kGb * b + 2 * kFb * wave + 2 * r + (lane >> 5), lane & 31), len - 1));
    };
    sync_lds();                                                 // every wave is done with the parts
    if constexpr (kSplit) {                                     // the list holds this share's groups: the row's
        uint32_t g[GPL];
        load_maxima(g);
        P = build_list(g, 0, nwr);
    }
    const int nb = (P + kGb - 1) / kGb;
    uint32_t thr = L, npend = 0;
    float x[kFb];
    if (nb > 0) load(0, x);
    for (int b = 0; b < nb; ++b) {                              // uniform
        uint32_t v[kFb];
#pragma unroll
        for (int r = 0; r < kFb; ++r) {
            const int gi = kGb * b + 2 * kFb * wave + 2 * r + (lane >> 5);
            const uint32_t key = score_key(x[r]);
            v[r] = (gi < P && gpos(gi, lane & 31) < len && key >= thr) ? key : 0u;
        }
        if (b + 1 < nb) load(b + 1, x);                         // in flight during this batch's selection
        if (npend > (uint32_t)kK) {                             // uniform: cut the list to its top kK
            sync_lds();                                         // the list is complete
            uint32_t pv[kPerSmall], pp[kPerSmall];
#pragma unroll
            for (int r = 0; r < kPerSmall; ++r) {
                const uint32_t i = 64 * kPerSmall * wave + 64 * r + lane;
                const uint2 e = s.pend[min(i, npend - 1)];
                pv[r] = i < npend ? e.x : 0u;
                pp[r] = e.y;
            }
            uint32_t mn = 0xffffffffu;
            // every thread read its items before the selection's first barrier, and
            // nothing is emitted before it, so the list is rewritten in place
            select_wide<kPerSmall>(pv, s.sc, [&](uint32_t slot, int, int r) {
                s.pend[slot] = make_uint2(pv[r], pp[r]);
                mn = min(mn, pv[r]);
            });
            mn = wave_min(mn);
            if (lane == 0) s.wmin[wave] = mn;
            sync_lds();
#pragma unroll
            for (int w = 0; w < kWaves; ++w) mn = min(mn, s.wmin[w]);
            thr = uni(mn) + 1u;                                 // the kK-th key, plus one
            npend = kK;
        }
        const uint32_t at = npend;
        sync_lds();                                             // the last selection's readers of sc are done
        npend += (uint32_t)select_wide<kFb>(v, s.sc, [&](uint32_t slot, int i, int r) {
            s.pend[at + slot] = make_uint2(v[r], (uint32_t)gpos(kGb * b + (i >> 5), i & 31));
        });
        npend = uni(npend);
    }
    // the list's top kK
    sync_lds();
    uint32_t pv[kPerSmall], pp[kPerSmall];
#pragma unroll
    for (int r = 0; r < kPerSmall; ++r) {
        const uint32_t i = 64 * kPerSmall * wave + 64 * r + lane;
        const uint2 e = s.pend[min(i, max(npend, 1u) - 1)];
        pv[r] = i < npend ? e.x : 0u;
        pp[r] = e.y;
    }
    const int cnt = select_wide<kPerSmall>(pv, s.sc, [&](uint32_t slot, int, int r) {
        out[slot] = (int32_t)pp[r];
    });
    write_final_pad(out, cnt);
}

// kEnt: candidate-holding loads a wave's entry list holds per half sub-batch.
// The default build keeps one work-group per CU (about 215 registers); the
// capped build (128 registers, spills in the rare paths, 72 KiB of LDS) runs two
// per CU, for launches of many rows (prefill).
template <int GPL>
__global__ __launch_bounds__(kThreads) void topk_row(const float* __restrict__ scores, int64_t ld,
                                                     const int32_t* __restrict__ q_pos,
                                                     const float* __restrict__ gmax, int64_t ldg, int al16,
                                                     int32_t* __restrict__ idx) {
    topk_row_body<GPL, 128, false>(scores, ld, q_pos, gmax, ldg, al16 != 0, idx, SplitArgs{});
}
template <int GPL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void topk_row_wide(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ q_pos,
    const float* __restrict__ gmax, int64_t ldg, int al16, int32_t* __restrict__ idx) {
    topk_row_body<GPL, 64, false>(scores, ld, q_pos, gmax, ldg, al16 != 0, idx, SplitArgs{});
}
// grid (rows, shares)
template <int GPL>
__global__ __launch_bounds__(kThreads) void topk_row_split(const float* __restrict__ scores, int64_t ld,
                                                           const int32_t* __restrict__ q_pos,
                                                           const float* __restrict__ gmax, int64_t ldg, int al16,
                                                           int32_t* __restrict__ idx, SplitArgs sa) {
    topk_row_body<GPL, 128, true>(scores, ld, q_pos, gmax, ldg, al16 != 0, idx, sa);
}

// ---- Selection without a score buffer ----------------------------------------
// The score kernel wrote only the group maxima (the largest score of every 32
// positions) and topk_bound turned them into the bound L of each row. A
// selected position scores >= L, so it lies in a group whose maximum reaches L;
// this kernel recomputes the scores of exactly those groups and selects among
// them as topk_chunk does among stored scores (same lists, same merge). The
// recomputation is the score kernels' own arithmetic: the same MFMA, the same
// split of the 128 dims (lane group g owns dims [64g, 64g + 64) of query and
// key) and the same ReLU, weight and head-sum order, so every score, and with
// it the selection, is bit-identical to the path through a score buffer.
// Rows without a bound (too short) recompute every group.
template <bool FP8>
__global__ __launch_bounds__(kThreads) void topk_rescore(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const uint8_t* __restrict__ k, const float* __restrict__ k_scale, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int64_t n_cap, const float* __restrict__ gmax, int64_t ldg,
    const uint32_t* __restrict__ bound, int n_chunks, uint8_t* __restrict__ lists, int32_t* __restrict__ idx) {
    constexpr int kHeadsIx = 32, kDimIx = 128;
    constexpr int kRowBytes = FP8 ? kDimIx : 2 * kDimIx;
    constexpr int KSTEPS = FP8 ? 2 : 8;              // MFMA steps over the 128 dims
    constexpr int NLD = FP8 ? 4 : 8;                 // 16-byte key loads per lane per group
    using AVec = std::conditional_t<FP8, i32x8, bf16x8>;
    // the chunk's candidate keys, each written and read back by the wave that
    // owns it; the selection scratch reuses the space once they are in registers
    __shared__ union { uint32_t keys[kChunk]; Scratch sc; } lds;
    const int qi = blockIdx.y, c = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 31, g = lane >> 5;
    const int64_t len = min((int64_t)q_pos[qi] + 1, n_cap);          // positions 0..len-1 are causal
    const int64_t s0 = (int64_t)c * kChunk;
    const int nvalid = (int)max((int64_t)0, min(s0 + kChunk, len) - s0);
    const uint32_t L = bound != nullptr ? uni(bound[qi]) : 0u;
    // this wave: positions w0 + [0, kSeg), 64 groups of 32; group j passes when
    // it holds a causal position and (with a bound) its maximum reaches L
    const int64_t w0 = s0 + (int64_t)kSeg * wave;
    const int nw = max(0, min(kSeg, nvalid - kSeg * wave));
    bool ok = 32 * lane < nw;
    if (ok && bound != nullptr) ok = score_key(gmax[(int64_t)qi * ldg + (w0 >> 5) + lane]) >= L;
    const uint64_t pass = __builtin_amdgcn_ballot_w64(ok);

    if (pass != 0) {                                                  // uniform
        // A operand: row = head n, this lane group's 64 dims; weights in accumulator order
        AVec a[KSTEPS];
        float wr[16];
        const uint8_t* qh = q + ((int64_t)qi * kHeadsIx + n) * kRowBytes;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
            if constexpr (FP8) {
                const i32x4* pq = (const i32x4*)(qh + 64 * g + 32 * t);
                const i32x4 lo = pq[0], hi = pq[1];
                a[t] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            } else {
                a[t] = *(const bf16x8*)(qh + 2 * (64 * g + 8 * t));
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) wr[i] = w[(int64_t)qi * kHeadsIx + 8 * (i >> 2) + 4 * g + (i & 3)];
        const int a_e8 = FP8 ? e8m0_of(q_scale[(int64_t)qi * kHeadsIx + n]) : 127;
        const int seq = q_seq[qi];
        const uint8_t* kb = k + (int64_t)seq * n_cap * kRowBytes;
        const float* ksb = FP8 ? k_scale + (int64_t)seq * n_cap : nullptr;
        uint32_t* kw = lds.keys + kSeg * wave;
        // lane (n, g) of group j: key w0 + 32j + n, its dims [64g, 64g + 64)
        // (a row past n_cap in a ragged last group reads row n_cap - 1: not a candidate)
        auto load = [&](int j, i32x4 (&kr)[NLD], float& ks) __attribute__((always_inline)) {
            const int64_t p = min(w0 + 32 * j + n, n_cap - 1);
            const i32x4* src = (const i32x4*)(kb + p * kRowBytes + (kRowBytes / 2) * g);
#pragma unroll
            for (int i = 0; i < NLD; ++i) kr[i] = src[i];
            ks = FP8 ? ksb[p] : 1.f;
        };
        // the passing groups in batches whose key loads are all in flight together
        constexpr int NB = FP8 ? 4 : 2;
        uint64_t todo = pass;
        while (todo != 0) {                                           // uniform: todo is a ballot
            int js[NB];
            i32x4 kr[NB][NLD];
            float ks[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                js[b] = todo != 0 ? (int)__builtin_ctzll(todo) : -1;
                todo &= todo - 1;
                if (js[b] >= 0) load(js[b], kr[b], ks[b]);
            }
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                if (js[b] < 0) break;
                f32x16 acc = {};
#pragma unroll
                for (int t = 0; t < KSTEPS; ++t) {
                    if constexpr (FP8) {
                        const i32x4 lo = kr[b][2 * t], hi = kr[b][2 * t + 1];
                        const i32x8 bv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[t], bv, acc, 0, 0, 0, a_e8, 0,
                                                                              e8m0_of(ks[b]));
                    } else {
                        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[t], __builtin_bit_cast(bf16x8, kr[b][t]),
                                                                      acc, 0, 0, 0);
                    }
                }
                float part = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i)               // relu on the bit pattern, as the score kernels
                    part = fmaf(wr[i], __int_as_float(max(__float_as_int(acc[i]), 0)), part);
                part = sum_x32(part);
                const int64_t s = w0 + 32 * js[b] + n;
                const uint32_t key = score_key(part);
                if (g == 0) kw[32 * js[b] + n] = (s < len && key >= L) ? key : 0u;
            }
        }
    }
    // items as topk_chunk holds them: lane item r = position kSeg*wave + 64r + lane,
    // group 2r + g of the wave; groups that did not pass hold no candidate
    uint32_t v[kPer];
#pragma unroll
    for (int r = 0; r < kPer; ++r)
        v[r] = ((pass >> (2 * r + g)) & 1u) ? lds.keys[kSeg * wave + 64 * r + lane] : 0u;
    __syncthreads();                                                  // keys read: the scratch may reuse them
    if (n_chunks == 1) {
        int32_t* out = idx + (int64_t)qi * kK;
        auto em = [&](uint32_t slot, int i, int) { out[slot] = (int32_t)(s0 + i); };
        write_final_pad(out, select_regs<kPer, false>(v, lds.sc, em));
    } else {
        uint8_t* Lst = lists + ((size_t)qi * n_chunks + c) * kListBytes;
        uint2* items = (uint2*)(Lst + 16);
        auto em = [&](uint32_t slot, int i, int r) { items[slot] = make_uint2(v[r], (uint32_t)(s0 + i)); };
        const int cnt = select_regs<kPer, false>(v, lds.sc, em);
        if (threadIdx.x == 0) *(uint32_t*)Lst = (uint32_t)cnt;
    }
}

// Number of list levels the merge may write: rounds of 8 until one list is left.
__host__ __device__ inline int64_t level_lists(int64_t n_lists) { return (n_lists + kFan - 1) / kFan; }

struct MergeLds {
    Scratch sc;
    uint32_t base[kThreads + 1];                // item offset of each list in the concatenation
};

// Lists [l0, l0 + nl) of a row (each at most k items, in position order), at
// most kMaxItems items in all, concatenated into registers: item i of the
// concatenation sits in list l with base[l] <= i < base[l + 1] (a binary search
// over the offsets in LDS) and is read from HBM / L2 directly. Returns the
// number of items.
template <int PER>
__device__ __forceinline__ int gather_lists(const uint8_t* lists0, int l0, int nl, MergeLds& m,
                                            uint32_t (&v)[PER], uint32_t (&p)[PER]) {
    constexpr int SEG = 64 * PER;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();                                          // earlier readers of sc and base are done
    uint32_t cnt = 0;
    if (threadIdx.x < nl)
        cnt = min(*(const uint32_t*)(lists0 + (size_t)(l0 + threadIdx.x) * kListBytes), (uint32_t)kK);
    // exclusive prefix over the lists (nl <= kThreads)
    uint32_t incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = (uint32_t)__shfl_up((int)incl, o, 64);
        if (lane >= o) incl += t;
    }
    if (lane == 63) m.sc.wsum[wave] = incl;
    __syncthreads();
    uint32_t before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const uint32_t t = m.sc.wsum[w];
        before += w < wave ? t : 0u;
        total += t;
    }
    total = uni(total);
    if (threadIdx.x < nl) m.base[threadIdx.x] = before + incl - cnt;
    if (threadIdx.x == 0) m.base[nl] = total;
    __syncthreads();
    const int steps = 32 - __builtin_clz((uint32_t)nl);         // ceil(log2(nl + 1))
#pragma unroll
    for (int r = 0; r < PER; ++r) { v[r] = 0u; p[r] = 0u; }
    if ((uint32_t)(SEG * wave) < total) {                    // uniform: this wave holds items
        // li[r]: the largest l with base[l] <= item r's index; the PER searches
        // advance together, so each step issues PER independent LDS reads
        uint32_t li[PER];
#pragma unroll
        for (int r = 0; r < PER; ++r) li[r] = 0;
        uint32_t span = 1u << steps;
        for (int t = 0; t < steps; ++t) {
            span >>= 1;
#pragma unroll
            for (int r = 0; r < PER; ++r) {
                const uint32_t i = min((uint32_t)(SEG * wave + 64 * r + lane), total - 1);
                const uint32_t mid = li[r] + span;
                if (mid < (uint32_t)nl && m.base[min(mid, (uint32_t)nl)] <= i) li[r] = mid;
            }
        }
        uint2 it[PER];
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            const uint32_t i = min((uint32_t)(SEG * wave + 64 * r + lane), total - 1);
            it[r] = ((const uint2*)(lists0 + (size_t)(l0 + li[r]) * kListBytes + 16))[i - m.base[li[r]]];
        }
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            const bool ok = (uint32_t)(SEG * wave + 64 * r + lane) < total;
            v[r] = ok ? it[r].x : 0u;
            p[r] = ok ? it[r].y : 0u;
        }
    }
    return (int)total;
}

// Row q: its n_lists chunk lists into the final indices. levels: workspace for
// the rounds of the fallback (level_lists(n_lists) lists per row, then
// level_lists of that, ...), used only when the lists hold more than 16K items.
__device__ __forceinline__ void merge_row(const uint8_t* __restrict__ lists, int n_lists,
                                          uint8_t* __restrict__ levels, int32_t* __restrict__ idx, MergeLds& m) {
    const int q = blockIdx.x;
    int32_t* out = idx + (int64_t)q * kK;
    const uint8_t* in = lists + (size_t)q * n_lists * kListBytes;
    int nl = n_lists;
    // The usual case, at most kSmall items in all: one gather (which sums the
    // counts itself) and one selection, without a separate pass over the counts.
    if (nl <= kThreads) {                                     // uniform
        uint32_t v[kPerSmall], p[kPerSmall];
        const int total = gather_lists<kPerSmall>(in, 0, nl, m, v, p);
        if (total <= kSmall) {                                // uniform
            auto em = [&](uint32_t slot, int, int r) { out[slot] = (int32_t)p[r]; };
            write_final_pad(out, select_regs<kPerSmall, false>(v, m.sc, em));
            return;
        }
    }
    // items of this row's lists (each count read once per list)
    uint32_t tot_local = 0;
    for (int l = threadIdx.x; l < nl; l += kThreads)
        tot_local += min(*(const uint32_t*)(in + (size_t)l * kListBytes), (uint32_t)kK);
    uint32_t total = uni(block_sum(uni(wave_sum(tot_local)), m.sc));
    // fallback: rounds of 8 lists until the rest fits in one selection
    uint8_t* lvl = levels;
    int64_t lvl_rows = level_lists(n_lists);
    while (total > (uint32_t)kMaxItems) {                     // uniform
        const int ng = (nl + kFan - 1) / kFan;
        uint8_t* outl = lvl + (size_t)q * lvl_rows * kListBytes;
        uint32_t new_total = 0;
        for (int gi = 0; gi < ng; ++gi) {
            uint32_t v[kPer], p[kPer];
            gather_lists<kPer>(in, gi * kFan, min(kFan, nl - gi * kFan), m, v, p);
            uint8_t* Lst = outl + (size_t)gi * kListBytes;
            uint2* items = (uint2*)(Lst + 16);
            auto em = [&](uint32_t slot, int, int r) { items[slot] = make_uint2(v[r], p[r]); };
            const int cnt = select_regs<kPer, false>(v, m.sc, em);
            if (threadIdx.x == 0) *(uint32_t*)Lst = (uint32_t)cnt;
            new_total += (uint32_t)cnt;
            __threadfence();
            __syncthreads();
        }
        in = outl;
        nl = ng;
        total = new_total;
        lvl += (size_t)gridDim.x * lvl_rows * kListBytes;
        lvl_rows = level_lists(lvl_rows);
    }
    int cnt;
    if (total <= (uint32_t)kSmall) {                          // the usual case with a bound
        uint32_t v[kPerSmall], p[kPerSmall];
        gather_lists<kPerSmall>(in, 0, nl, m, v, p);
        auto em = [&](uint32_t slot, int, int r) { out[slot] = (int32_t)p[r]; };
        cnt = select_regs<kPerSmall, false>(v, m.sc, em);
    } else {
        uint32_t v[kPer], p[kPer];
        gather_lists<kPer>(in, 0, nl, m, v, p);
        auto em = [&](uint32_t slot, int, int r) { out[slot] = (int32_t)p[r]; };
        cnt = select_regs<kPer, false>(v, m.sc, em);
    }
    write_final_pad(out, cnt);
}

// Two builds of the merge: few rows want each work-group's latency low (no cap
// on registers); many rows (prefill) want two work-groups per CU, i.e. at most
// 128 registers, at the cost of spills in the rare paths (measured: 4096 rows
// 746 -> 665 us; 8 to 64 rows about 1.5 us slower).
__global__ __launch_bounds__(kThreads) void topk_merge(const uint8_t* __restrict__ lists, int n_lists,
                                                       uint8_t* __restrict__ levels, int32_t* __restrict__ idx) {
    __shared__ MergeLds m;
    merge_row(lists, n_lists, levels, idx, m);
}
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void topk_merge_wide(
    const uint8_t* __restrict__ lists, int n_lists, uint8_t* __restrict__ levels, int32_t* __restrict__ idx) {
    __shared__ MergeLds m;
    merge_row(lists, n_lists, levels, idx, m);
}
constexpr int kWideRows = 512;                  // rows from which the capped build is used

int n_chunks_of(int64_t ld) { return (int)((ld + kChunk - 1) / kChunk); }

// Rows of at least kK full groups exist only when ld >= kK * kGroup.
bool bounded(int64_t ld) { return ld >= (int64_t)kK * kGroup; }

constexpr int kRowMaxGpl = 64;                  // topk_row: rows of up to 512 * 64 groups (2^20 positions)

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

bool row_path(int64_t ld) { return bounded(ld) && group_max_ld(ld) <= (int64_t)kThreads * kRowMaxGpl; }

// Shares per row for the row kernels: launches of at most 128 rows split each
// row in 2, 4 or 8 so that at most 256 work-groups (one per CU) run.
int row_shares(int n_q) {
    int p = 1;
    while (2 * p <= kMaxShares && n_q * 2 * p <= 256) p *= 2;
    return p;
}

// Split-row area of the workspace, after the bounds and the group maxima: the
// flags, then the regions.
size_t split_offset(int n_q, int64_t ld) {
    return align256((size_t)n_q * 4) + align256((size_t)n_q * group_max_ld(ld) * 4);
}

// Launch tags: a new one per launch, from a per-process start that differs
// between processes; never 0 (a cleared flag).
unsigned long long next_tag() {
    static std::atomic<unsigned long long> counter{
        (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count() * 0x9E3779B97F4A7C15ull};
    const unsigned long long t = counter.fetch_add(1ull);
    return t != 0ull ? t : counter.fetch_add(1ull);
}

}  // namespace

unsigned long long launch_tag() { return next_tag(); }

size_t topk_workspace_bytes(int n_q, int64_t ld, int k) {
    (void)k;
    const int nc = n_chunks_of(ld);
    if (nc <= 1) return 16;
    size_t b = 0;
    if (bounded(ld)) {
        b += align256((size_t)n_q * 4);                              // bounds
        b += align256((size_t)n_q * group_max_ld(ld) * 4);           // group maxima (when not given)
    }
    b += (size_t)n_q * nc * kListBytes;                             // chunk lists
    for (int64_t n = level_lists(nc); ; n = level_lists(n)) {       // merge fallback rounds
        b += (size_t)n_q * n * kListBytes;
        if (n <= 1) break;
    }
    const int pn = row_shares(n_q);
    if (row_path(ld) && pn > 1) {                                   // split rows: counters and regions
        const size_t sp = split_offset(n_q, ld) + align256((size_t)n_q * pn * 8) + (size_t)n_q * pn * kRegionBytes;
        b = b > sp ? b : sp;
    }
    return b;
}

float* topk_group_max_area(void* ws, int n_q, int64_t ld) {
    if (n_chunks_of(ld) <= 1 || !bounded(ld)) return nullptr;
    return (float*)((uint8_t*)ws + align256((size_t)n_q * 4));
}

hipError_t launch_topk(const float* scores, int64_t ld, const int32_t* q_pos, int n_q, int k,
                       const float* group_max, int32_t* idx, void* ws, hipStream_t st) {
    (void)k;
    const int nc = n_chunks_of(ld);
    if (nc == 1) {
        if (ld <= (int64_t)kPerSmall * kThreads)                // rows of at most 4096 positions
            hipLaunchKernelGGL(topk_small, dim3(n_q), dim3(kThreads), 0, st, scores, ld, q_pos, idx);
        else
            hipLaunchKernelGGL(topk_chunk, dim3(1, n_q), dim3(kThreads), 0, st, scores, ld, q_pos, 1,
                               (const uint32_t*)nullptr, (uint8_t*)nullptr, idx);
        return hipGetLastError();
    }
    const int64_t ldg = group_max_ld(ld);
    if (row_path(ld)) {
        // rows of 64K to 1M positions: one work-group per row (or per share of a
        // row), over the group maxima
        if (group_max == nullptr) {
            float* gm = topk_group_max_area(ws, n_q, ld);
            hipLaunchKernelGGL(topk_group_max, dim3(nc, n_q), dim3(kThreads), 0, st, scores, ld, q_pos, gm, ldg);
            group_max = gm;
        }
        const int gpl = ldg <= kThreads * 8 ? 8 : ldg <= kThreads * 16 ? 16 : ldg <= kThreads * 32 ? 32 : 64;
        const int al16 = ldg % 4 == 0 && ((uintptr_t)group_max & 15u) == 0 ? 1 : 0;   // 16-byte maxima loads
        const int pn = row_shares(n_q);
        if (pn > 1) {
            uint8_t* sp = (uint8_t*)ws + split_offset(n_q, ld);
            const SplitArgs sa{(unsigned long long*)sp, sp + align256((size_t)n_q * pn * 8), next_tag(), pn};
            auto* kern = gpl == 8 ? topk_row_split<8> : gpl == 16 ? topk_row_split<16>
                       : gpl == 32 ? topk_row_split<32> : topk_row_split<64>;
            hipLaunchKernelGGL(kern, dim3(n_q, pn), dim3(kThreads), 0, st, scores, ld, q_pos, group_max, ldg, al16, idx,
                               sa);
            return hipGetLastError();
        }
        auto* kern = gpl == 8 ? (n_q >= kWideRows ? topk_row_wide<8> : topk_row<8>)
                   : gpl == 16 ? topk_row<16> : gpl == 32 ? topk_row<32> : topk_row<64>;
        hipLaunchKernelGGL(kern, dim3(n_q), dim3(kThreads), 0, st, scores, ld, q_pos, group_max, ldg, al16, idx);
        return hipGetLastError();
    }
    uint8_t* p = (uint8_t*)ws;
    const uint32_t* bound = nullptr;
    if (bounded(ld)) {
        uint32_t* b = (uint32_t*)p;
        p += align256((size_t)n_q * 4);
        float* gm = (float*)p;
        p += align256((size_t)n_q * group_max_ld(ld) * 4);
        const int64_t ldg = group_max_ld(ld);
        if (group_max == nullptr) {
            hipLaunchKernelGGL(topk_group_max, dim3(nc, n_q), dim3(kThreads), 0, st, scores, ld, q_pos, gm, ldg);
            group_max = gm;
        }
        hipLaunchKernelGGL(topk_bound, dim3(n_q), dim3(kThreads), 0, st, group_max, ldg, q_pos, b);
        bound = b;
    }
    uint8_t* lists = p;
    uint8_t* levels = lists + (size_t)n_q * nc * kListBytes;
    hipLaunchKernelGGL(topk_chunk, dim3(nc, n_q), dim3(kThreads), 0, st, scores, ld, q_pos, nc, bound, lists, idx);
    if (n_q >= kWideRows)
        hipLaunchKernelGGL(topk_merge_wide, dim3(n_q), dim3(kThreads), 0, st, (const uint8_t*)lists, nc, levels, idx);
    else
        hipLaunchKernelGGL(topk_merge, dim3(n_q), dim3(kThreads), 0, st, (const uint8_t*)lists, nc, levels, idx);
    return hipGetLastError();
}


hipError_t launch_indexer_topk(bool fp8, const void* q, const float* q_scale, const float* w, const void* k,
                               const float* k_scale, const int32_t* q_seq, const int32_t* q_pos, int n_q,
                               int batch, int64_t n_cap, int k_sel, int32_t* idx, void* ws, hipStream_t st) {
    (void)k_sel;
    const int64_t ld = indexer_topk_ld(n_cap);
    const int nc = n_chunks_of(ld);
    const int64_t ldg = group_max_ld(ld);
    uint8_t* p = (uint8_t*)ws;
    const uint32_t* bound = nullptr;
    const float* gm = nullptr;
    if (nc > 1 && bounded(ld)) {
        // the workspace layout of launch_topk: bounds, group maxima, lists, merge levels
        uint32_t* b = (uint32_t*)p;
        p += align256((size_t)n_q * 4);
        float* g = (float*)p;
        p += align256((size_t)n_q * ldg * 4);
        hipError_t e = launch_indexer_score(fp8, q, q_scale, w, k, k_scale, q_seq, q_pos, n_q, batch, n_cap,
                                            nullptr, ld, g, st);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(topk_bound, dim3(n_q), dim3(kThreads), 0, st, (const float*)g, ldg, q_pos, b);
        bound = b;
        gm = g;
    }
    uint8_t* lists = nc > 1 ? p : nullptr;
    uint8_t* levels = nc > 1 ? lists + (size_t)n_q * nc * kListBytes : nullptr;
    if (fp8)
        hipLaunchKernelGGL(topk_rescore<true>, dim3(nc, n_q), dim3(kThreads), 0, st, (const uint8_t*)q, q_scale,
                           w, (const uint8_t*)k, k_scale, q_seq, q_pos, n_cap, gm, ldg, bound, nc, lists, idx);
    else
        hipLaunchKernelGGL(topk_rescore<false>, dim3(nc, n_q), dim3(kThreads), 0, st, (const uint8_t*)q, q_scale,
                           w, (const uint8_t*)k, k_scale, q_seq, q_pos, n_cap, gm, ldg, bound, nc, lists, idx);
    if (nc > 1) {
        if (n_q >= kWideRows)
            hipLaunchKernelGGL(topk_merge_wide, dim3(n_q), dim3(kThreads), 0, st, (const uint8_t*)lists, nc, levels, idx);
        else
            hipLaunchKernelGGL(topk_merge, dim3(n_q), dim3(kThreads), 0, st, (const uint8_t*)lists, nc, levels, idx);
    }
    return hipGetLastError();
}

}  // namespace gsa

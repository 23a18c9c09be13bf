// Lightning-indexer score of a full (F) layer on gfx950 MFMA.
//
// "GLM-5.2 架构深度拆解" CH2 §2.2: an F layer scores each query against every
// history token with 32 heads x 128 dims; "GLM-5.2 总览" sub-document index:
// the indexer applies a ReLU (and FP8 per-block q/k as one variant).
//
//   score[i, s] = sum_h w[i,h] * max(0, q[i,h,:] . k[seq(i), s, :])   (s <= pos(i))
//
// Mapping to CDNA4. The 32 heads of one query are the 32 rows (M) of a
// 32x32 MFMA tile and 32 consecutive keys its columns (N); the 128 dims are the
// contraction. bf16 uses v_mfma_f32_32x32x16_bf16 (8 k-steps); fp8 uses
// v_mfma_scale_f32_32x32x64_f8f6f4 (2 k-steps) with the per-block power-of-two
// scales fed as E8M0 operand scales, so no dequantisation pass exists.
// Because the contraction order is free, lane group g of a tile owns dims
// [64g, 64g+64) in both operands. The epilogue (ReLU, head weight, sum over
// heads) stays in registers: each lane holds 16 heads of one key and one
// cross-lane add finishes the sum, so only the final fp32 score reaches HBM.
//
// Keys stream through LDS in 32 KiB tiles (128 bf16 or 256 fp8 keys) with LDS-DMA (global_load_lds:
// whole 1 KiB key blocks per wave instruction, no staging registers) into a
// ring of kRing slots, so kRing - 1 tiles are in flight per work-group (with
// the non-temporal hint when each key is read by one work-group only). The
// DMA source chunk of each lane is chosen so that 16-byte chunks land XOR-
// swizzled inside their key row, which makes the MFMA-layout ds_read_b128
// conflict-free. Queries of one sequence that share a work-group (QB of them)
// reuse each key tile from LDS.
//
// Kernels: indexer_score_kernel (one or two queries per work-group, a 2D grid
// of equal key chunks); indexer_score_dyn (fp8 decode with one query per
// sequence on a persistent grid that hands out 1024-key chunks through
// self-resetting counters); indexer_score_mq (4, 8 or 16 queries of one
// sequence per work-group, MTP verify and chunked prefill).
#include <mutex>
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace gsa {
namespace {

constexpr int kHeads = 32;
constexpr int kDim = 128;
constexpr int kTile = 128;      // keys per LDS tile
constexpr int kThreads = 256;   // 4 waves
constexpr int kRing = 4;        // LDS tile slots
constexpr int kStageKeys = 4096;  // longest chunk whose scores a one-query bf16 work-group keeps in LDS

// Score stores of the streaming loops. The fp8 kernels write twice the score
// bytes per key byte of the bf16 ones, and there the non-temporal hint measured
// faster (prefill 2,368 -> 2,270 us, 1M-key decode 200 -> 195 us); for bf16 it
// measured 1-3% slower, so bf16 scores keep plain stores.
template <bool NT>
__device__ __forceinline__ void store_score(float* p, float v) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

template <bool FP8, int KEYS = kTile>
struct KeyTile {
    static constexpr int kKeys = KEYS;                          // keys per tile
    static constexpr int kRowBytes = FP8 ? kDim : kDim * 2;
    static constexpr int kChunks = kRowBytes / 16;              // 16-byte chunks per key row
    static constexpr int kBytes = KEYS * kRowBytes;
    static constexpr int kRowsPerDma = 1024 / kRowBytes;        // key rows per 1 KiB DMA
    static constexpr int kDma = kBytes / 1024;
    static constexpr int kDmaPerWave = kDma / 4;
    static constexpr int kScaleDma = FP8 ? KEYS / 64 : 0;       // 256-byte DMAs of fp32 scales
    static constexpr int kScaleBytes = 256 * kScaleDma;
    static constexpr int kSlot = kBytes + kScaleBytes;
    // Chunk c of tile row r is stored at chunk c ^ swz(r) of the row. A 16-byte
    // read of 16 consecutive rows (16 lanes) then touches 16 distinct chunks
    // of the 64 banks: a bf16 row spans all 64 (256 bytes), so r mod 16 spreads
    // them; an fp8 row spans 32, and rows r and r + 1 sit in the two halves, so
    // (r / 2) mod 8 spreads the 8 rows of each half (r mod 8 put rows r and
    // r + 8 on the same banks: 3 conflict cycles per LDS read in the FP8 decode
    // kernel).
    __device__ static __forceinline__ int swz(int r) { return FP8 ? (r >> 1) & 7 : r & (kChunks - 1); }
    // byte offset of logical chunk c of tile row r
    __device__ static __forceinline__ int off(int r, int c) {
        return r * kRowBytes + ((c ^ swz(r)) << 4);
    }
};

// NTK: the keys are read by this work-group only (one query block per
// sequence), so they stream with the non-temporal hint.
template <int QB, bool FP8, bool NTK, bool STAGE = false>
__global__ __launch_bounds__(kThreads) void indexer_score_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ k,
    const float* __restrict__ k_scale, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int n_q, int64_t n_cap,
    float* __restrict__ scores, int64_t ld, float* __restrict__ gmax, int64_t ldg, int chunk) {
    // fp8 tiles hold 256 keys, so every tile moves 32 KiB like a bf16 tile and the
    // per-tile barrier and waits are paid per 32 KiB either way
    using T = KeyTile<FP8, FP8 ? 256 : 128>;
    static_assert(QB <= 2, "one or two queries per work-group");
    constexpr int NSUBT = T::kKeys / 32;         // 32-key subtiles per tile
    constexpr int PPW = QB * NSUBT / 4;          // (query, subtile) pairs per wave
    constexpr int QPW = 1;                       // queries per wave
    constexpr int KSTEPS = FP8 ? 2 : 8;         // MFMA steps over 128 dims
    using AVec = std::conditional_t<FP8, i32x8, bf16x8>;
    typedef __attribute__((address_space(3))) uint8_t lds_u8;

    __shared__ __attribute__((aligned(16))) uint8_t ring[kRing * T::kSlot];
    // STAGE: the chunk's scores and group maxima collect in LDS (16.5 KiB beside
    // the 128 KiB ring) and leave in one burst when the chunk ends, so that no
    // global store is issued between the ring's DMAs (64 x 128K bf16 keys:
    // 361-363 against 370 us)
    static_assert(!STAGE || (QB == 1 && !FP8), "staged scores: one bf16 query per work-group");
    __shared__ __attribute__((aligned(16))) float stage_sc[STAGE ? kStageKeys : 1];
    __shared__ float stage_gm[STAGE ? kStageKeys / 32 : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave: uniform (SGPR)
    const int n = lane & 31, g = lane >> 5;
    const int qb0 = blockIdx.y * QB;
    const int64_t c0 = (int64_t)blockIdx.x * chunk;
    if (c0 >= n_cap) return;
    const int64_t c1 = min(c0 + (int64_t)chunk, n_cap);

    // This wave owns the (query, 32-key subtile) pairs [wave*QB, wave*QB + QB):
    // pair p -> query p/4 of the block, subtile p%4 of the 128-key tile.
    const int jw0 = (wave * QB) / 4;

    AVec a[QPW][KSTEPS];
    float wr[QPW][16];
    int apos[QPW], a_e8[QPW];
#pragma unroll
    for (int jj = 0; jj < QPW; ++jj) {
        const int qi = qb0 + jw0 + jj;
        const bool ok = qi < n_q;
        const int qr = ok ? qi : 0;
        apos[jj] = ok ? q_pos[qi] : -1;
        // A operand: row = head n, this lane group's 64 dims [64g, 64g+64)
        const uint8_t* qh = q + ((int64_t)qr * kHeads + n) * T::kRowBytes;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
            if constexpr (FP8) {
                const i32x4* p = (const i32x4*)(qh + 64 * g + 32 * t);
                const i32x4 lo = p[0], hi = p[1];
                a[jj][t] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            } else {
                a[jj][t] = *(const bf16x8*)(qh + 2 * (64 * g + 8 * t));
            }
        }
        // accumulator register i of a 32x32 tile holds row 8*(i/4) + 4*g + i%4
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int h = 8 * (i >> 2) + 4 * g + (i & 3);
            wr[jj][i] = ok ? w[(int64_t)qr * kHeads + h] : 0.f;
        }
        if constexpr (FP8) a_e8[jj] = e8m0_of(q_scale[(int64_t)qr * kHeads + n]);
        else a_e8[jj] = 127;
    }
    wait_vmcnt<0>();   // operands are in registers before any ring load is counted

    // DMA instructions per tile issued by this wave (wave 0 also moves the fp8 scales)
    const int per = T::kDmaPerWave + ((FP8 && wave == 0) ? T::kScaleDma : 0);
    const uint32_t ring_base = (uint32_t)(uintptr_t)(lds_u8*)ring;
    // lane offsets (bytes from a tile's first key row) of this wave's DMAs:
    // DMA i moves rows 8i .. (fp8) or 4i .. (bf16), and lane l's 16-byte chunk
    // lands at the XOR-swizzled place of its row
    uint32_t doff[T::kDmaPerWave];
#pragma unroll
    for (int jd = 0; jd < T::kDmaPerWave; ++jd) {
        const int i = wave * T::kDmaPerWave + jd;
        const int r = i * T::kRowsPerDma + lane / T::kChunks;
        const int c = (lane % T::kChunks) ^ T::swz(r);
        doff[jd] = (uint32_t)(r * T::kRowBytes + 16 * c);
    }

    // Queries of the block are processed in runs that share a sequence.
    int j0 = 0;
    while (j0 < QB && qb0 + j0 < n_q) {
        const int seq = q_seq[qb0 + j0];
        int j1 = j0 + 1;
        int maxpos = q_pos[qb0 + j0];
        while (j1 < QB && qb0 + j1 < n_q && q_seq[qb0 + j1] == seq) {
            maxpos = max(maxpos, (int)q_pos[qb0 + j1]);
            ++j1;
        }
        const uint8_t* kb = k + (int64_t)seq * n_cap * T::kRowBytes;
        const float* ksb = FP8 ? k_scale + (int64_t)seq * n_cap : nullptr;
        // tiles [0, na) hold keys at or before the run's last position; later ones are masked
        const int64_t t_end = min(c1, (int64_t)maxpos + 1);
        const int na = t_end > c0 ? (int)((t_end - c0 + T::kKeys - 1) / T::kKeys) : 0;
        const int nt_all = (int)((c1 - c0 + T::kKeys - 1) / T::kKeys);
        // score stores this wave issues per tile in this run (one per owned pair in the run)
        // (none without a score buffer: the group-maximum stores then go uncounted,
        // which only makes the waits stricter)
        int stores = 0;
#pragma unroll
        for (int p = 0; p < PPW; ++p) {
            const int j = (wave * PPW + p) / NSUBT;
            stores += (j >= j0 && j < j1 && scores != nullptr && !STAGE) ? 1 : 0;
        }

        auto issue = [&](int ti, int slot) __attribute__((always_inline)) {
            const int64_t t0 = c0 + (int64_t)ti * T::kKeys;
            const uint32_t dst = ring_base + slot * T::kSlot;
            if (t0 + T::kKeys <= c1) {                   // uniform: a whole tile, scalar base + lane offsets
                const uint8_t* base = kb + t0 * T::kRowBytes;
#pragma unroll
                for (int jd = 0; jd < T::kDmaPerWave; ++jd)
                    lds_dma16_so<NTK>(base, doff[jd], dst + 1024 * (wave * T::kDmaPerWave + jd));
                if constexpr (FP8) {
                    if (wave == 0) {
#pragma unroll
                        for (int h = 0; h < T::kScaleDma; ++h)
                            lds_dma4_so<NTK>(ksb + t0, 4 * (64 * h + lane), dst + T::kBytes + 256 * h);
                    }
                }
                return;
            }
#pragma unroll
            for (int jd = 0; jd < T::kDmaPerWave; ++jd) {
                const int i = wave * T::kDmaPerWave + jd;
                const int r = i * T::kRowsPerDma + lane / T::kChunks;
                const int p = lane % T::kChunks;                     // physical chunk in the row
                const int c = p ^ T::swz(r);            // logical chunk stored there
                const int64_t krow = min(t0 + r, c1 - 1);            // rows past the chunk: any valid row
                lds_dma16_t<NTK>(kb + krow * T::kRowBytes + 16 * c, dst + 1024 * i);
            }
            if constexpr (FP8) {
                if (wave == 0) {
#pragma unroll
                    for (int h = 0; h < T::kScaleDma; ++h) {
                        const int64_t krow = min(t0 + 64 * h + lane, c1 - 1);
                        lds_dma4_t<NTK>(ksb + krow, dst + T::kBytes + 256 * h);
                    }
                }
            }
        };

        for (int p = 0; p < kRing - 1; ++p)
            if (p < na) issue(p, p);
        for (int ti = 0; ti < nt_all; ++ti) {
            const int64_t t0 = c0 + (int64_t)ti * T::kKeys;
            const bool active = ti < na;                 // uniform over the work-group
            const lds_u8* tile = (const lds_u8*)ring + (ti % kRing) * T::kSlot;
            if (active) {
                // wait for this wave's DMAs of tile ti: the later issued ones are the
                // DMAs of tiles ti+1 .. min(na, ti+kRing-1)-1 and the score stores of
                // the iterations since tile ti was issued
                const int later = min(na, ti + kRing - 1) - ti - 1;
                wait_vmcnt_le(__builtin_amdgcn_readfirstlane(later * per + stores * min(ti, kRing - 1)));
                ring_barrier();   // every wave's part of tile ti landed; tile ti-1's readers are done
                if (ti + kRing - 1 < na) issue(ti + kRing - 1, (ti + kRing - 1) % kRing);
            }
            // this wave's pairs: the MFMAs of every pair first, then every pair's head
            // sums, so that one pair's sums run while the next pair's MFMAs occupy
            // the matrix core (no branch between them); a pair outside the run or
            // the causal range is computed anyway, from whatever the slot holds,
            // and discarded (the last tiles of a query only)
            f32x16 acc[PPW];
#pragma unroll
            for (int p = 0; p < PPW; ++p) {
                const int pp = wave * PPW + p;
                const int nt = pp % NSUBT;
                const int jj = pp / NSUBT - jw0;         // 0: one query per wave
                const int row = nt * 32 + n;
                acc[p] = f32x16{};
#pragma unroll
                for (int t = 0; t < KSTEPS; ++t) {
                    if constexpr (FP8) {
                        const i32x4 lo = *(const __attribute__((address_space(3))) i32x4*)(tile + T::off(row, 4 * g + 2 * t));
                        const i32x4 hi = *(const __attribute__((address_space(3))) i32x4*)(tile + T::off(row, 4 * g + 2 * t + 1));
                        const i32x8 b = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                        const float ks = *(const __attribute__((address_space(3))) float*)(tile + T::kBytes + 4 * row);
                        acc[p] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            a[jj][t], b, acc[p], 0, 0, 0, a_e8[jj], 0, e8m0_of(ks));
                    } else {
                        const bf16x8 b = *(const __attribute__((address_space(3))) bf16x8*)(tile + T::off(row, 8 * g + t));
                        acc[p] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[jj][t], b, acc[p], 0, 0, 0);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);          // keep every MFMA ahead of the head sums
            float res[PPW];                              // every pair's sums before any branch
#pragma unroll
            for (int p = 0; p < PPW; ++p) {
                const int pp = wave * PPW + p;
                const int jj = pp / NSUBT - jw0;
                const int64_t s = t0 + (pp % NSUBT) * 32 + n;
                float part = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i)             // relu on the bit pattern: exact, one instruction
                    part = fmaf(wr[jj][i], __int_as_float(max(__float_as_int(acc[p][i]), 0)), part);
                part = sum_x32(part);
                res[p] = (active && s <= apos[jj]) ? part : neg_inf();
            }
#pragma unroll
            for (int p = 0; p < PPW; ++p) {
                const int pp = wave * PPW + p;
                const int j = pp / NSUBT, nt = pp % NSUBT;
                if (j < j0 || j >= j1) continue;         // other run (wave-uniform)
                const int64_t s0 = t0 + nt * 32;
                const int64_t s = s0 + n;
                if (scores != nullptr && g == 0 && s < c1)   // uniform pointer test
                {
                    if constexpr (STAGE) stage_sc[s - c0] = res[p];
                    else store_score<FP8>(scores + (int64_t)(qb0 + j) * ld + s, res[p]);
                }
                if (gmax != nullptr && s0 < c1) {                       // uniform
                    const uint32_t m = max_x32(score_key(s < c1 ? res[p] : neg_inf()));
                    if (lane == 0) {
                        if constexpr (STAGE) stage_gm[(s0 - c0) >> 5] = key_value(m);
                        else gmax[(int64_t)(qb0 + j) * ldg + (s0 >> 5)] = key_value(m);
                    }
                }
            }
        }
        ring_barrier();     // the next run refills slots this run's last tiles were read from
        if constexpr (STAGE) {
            // every position of [c0, c1) and every group there was written above
            // (the masked ones as -inf); the launcher keeps c1 - c0 <= kStageKeys
            __syncthreads();                             // the LDS writes of all waves are visible
            const int len = (int)(c1 - c0);
            if (scores != nullptr) {
                float* dst = scores + (int64_t)qb0 * ld + c0;
                if ((((uintptr_t)dst) & 15) == 0 && (len & 3) == 0) {
                    // non-temporal: 346-349 against 352-363 us for the launch; the
                    // top-k that reads these scores next loses under 1 us
                    for (int i = 4 * tid; i < len; i += 4 * kThreads)
                        __builtin_nontemporal_store(*(const f32x4*)(stage_sc + i), (f32x4*)(dst + i));
                } else {
                    for (int i = tid; i < len; i += kThreads) dst[i] = stage_sc[i];
                }
            }
            if (gmax != nullptr) {
                float* gd = gmax + (int64_t)qb0 * ldg + (c0 >> 5);
                for (int i = tid; i < (len + 31) / 32; i += kThreads) gd[i] = stage_gm[i];
            }
        }
        j0 = j1;
    }
}

// ---- fp8 decode rows on a persistent grid --------------------------------------
// One query per sequence, fp8 keys, rows of whole 1024-key chunks: 256
// work-groups, one per CU; work-group b serves query (b/8 + 32 (b%8)) mod n_q
// (so a query's work-groups sit on every XCD) and takes its query's chunks one
// by one from a per-query counter until the counter passes the row's chunk
// count. With equal chunks handed out in launch order (two rounds of 16K-key
// work-groups) the CUs stop at different times: the second round's last
// work-groups run alone for about 7% of the launch; here every CU keeps taking
// 1024-key chunks until none are left, and the ring runs on across chunks.
//
// The counters are a static array of kDynSlots slots of 256, zero when the
// library loads; a launch uses the slot its tag selects, and the work-group
// whose grab comes last (each work-group fails exactly once, so the last grab
// returns chunks + work-groups - 1) sets the counter back to zero, so every
// launch finds its counters at zero. Launches running at the same time must use
// different slots: at most kDynSlots - 1 other launches may start while one runs.
//
// Waves 0-3 move, score and store the keys as in the one-query kernel. A fifth
// wave only takes the grabs: a grab is an atomic add whose result the compiler
// waits for with the wave's whole memory counter, which in a wave with DMAs or
// score stores in flight would wait for those too. It grabs the chunk of slot
// s + 2 when slot s starts and posts it to LDS one slot later; the other waves
// read it there.
constexpr int kDynChunk = 1024;                 // keys per grab (4 tiles)
constexpr int kDynWGs = 256;
constexpr int kDynSlots = 64;
constexpr int kDynMaxQ = 256;
constexpr int kDynThreads = kThreads + 64;      // four streaming waves and the grabbing wave
__device__ int g_dyn_ctr[kDynSlots * kDynMaxQ];

__global__ __launch_bounds__(kDynThreads) void indexer_score_dyn(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ k,
    const float* __restrict__ k_scale, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int n_q, int64_t n_cap,
    float* __restrict__ scores, int64_t ld, float* __restrict__ gmax, int64_t ldg, int* __restrict__ ctr) {
    using T = KeyTile<true, 256>;
    constexpr int TPC = kDynChunk / T::kKeys;   // tiles per chunk
    static_assert(TPC >= kRing - 1, "a tile issued kRing - 1 ahead is at most one chunk ahead");
    constexpr int NSUBT = T::kKeys / 32;        // 32-key subtiles per tile
    constexpr int PPW = NSUBT / 4;              // subtiles per streaming wave
    constexpr int KSTEPS = 2;
    constexpr int kGrab = 4;                    // the grabbing wave
    typedef __attribute__((address_space(3))) uint8_t lds_u8;
    typedef __attribute__((address_space(1))) int gint;
    __shared__ __attribute__((aligned(16))) uint8_t ring[kRing * T::kSlot];
    __shared__ int chq[4];                      // chunk of slot s at chq[s % 4], -1: none

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, g = lane >> 5;
    const int b = blockIdx.x;
    const int qi = ((b >> 3) + 32 * (b & 7)) % n_q;
    const int wgs = (int)gridDim.x / n_q;       // work-groups of this query
    const int nch = (int)(n_cap / kDynChunk);
    // the counter's address in a vector register: the compiler's atomic
    // optimizer, which rewrites an add at a uniform address into one lane's add
    // plus a broadcast of its result (a wait for the result right after the
    // add), leaves it alone; a global (not generic) pointer, so the add counts
    // in vmcnt only
    uint64_t cnt_addr = (uint64_t)(uintptr_t)(ctr + qi);
    asm volatile("" : "+v"(cnt_addr));
    gint* const cnt = (gint*)cnt_addr;

    int pend = 0;                               // grabbing wave, lane 0: the grab in flight
    bool more = true;                           // no grab of this work-group has failed yet
    if (wave == kGrab && lane == 0) pend = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // grabbing wave: post the grab in flight as the chunk of slot `sl`, and grab
    // again while chunks remain
    auto post = [&](int sl) __attribute__((always_inline)) {
        if (wave == kGrab) {
            if (lane == 0) {
                const int v = more ? pend : nch;
                const bool ok = v >= 0 && v < nch;              // (any other value: no chunk)
                if (more && !ok && v == nch + wgs - 1)          // the last grab of this launch
                    __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                chq[sl & 3] = ok ? v : -1;
                if (ok) pend = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                more = ok;
            }
            more = __builtin_amdgcn_readfirstlane(more ? 1 : 0) != 0;
            __builtin_amdgcn_s_waitcnt(0xC07F);          // lgkmcnt(0): the posted chunk is in LDS
        }
    };

    i32x8 a[KSTEPS];
    float wr[16];
    int apos = 0, a_e8 = 127, seq = 0;
    if (wave < kGrab) {
        apos = q_pos[qi];
        seq = q_seq[qi];
        const uint8_t* qh = q + ((int64_t)qi * kHeads + n) * T::kRowBytes;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
            const i32x4* p = (const i32x4*)(qh + 64 * g + 32 * t);
            const i32x4 lo = p[0], hi = p[1];
            a[t] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) wr[i] = w[(int64_t)qi * kHeads + 8 * (i >> 2) + 4 * g + (i & 3)];
        a_e8 = e8m0_of(q_scale[(int64_t)qi * kHeads + n]);
        wait_vmcnt<0>();   // operands are in registers before any ring load is counted
    }
    post(0);
    __syncthreads();

    const uint8_t* kb = k + (int64_t)seq * n_cap * T::kRowBytes;
    const float* ksb = k_scale + (int64_t)seq * n_cap;
    // DMA instructions per tile issued by this wave (wave 0 also moves the scales)
    const int per = wave < kGrab ? T::kDmaPerWave + (wave == 0 ? T::kScaleDma : 0) : 0;
    const uint32_t ring_base = (uint32_t)(uintptr_t)(lds_u8*)ring;
    uint32_t doff[T::kDmaPerWave];
#pragma unroll
    for (int jd = 0; jd < T::kDmaPerWave; ++jd) {
        const int i = wave * T::kDmaPerWave + jd;
        const int r = i * T::kRowsPerDma + lane / T::kChunks;
        const int c = (lane % T::kChunks) ^ T::swz(r);
        doff[jd] = (uint32_t)(r * T::kRowBytes + 16 * c);
    }
    auto issue = [&](int64_t t0, int slot) __attribute__((always_inline)) {   // a whole tile inside the row
        if (wave >= kGrab) return;
        const uint32_t dst = ring_base + slot * T::kSlot;
        const uint8_t* base = kb + t0 * T::kRowBytes;
#pragma unroll
        for (int jd = 0; jd < T::kDmaPerWave; ++jd)
            lds_dma16_so<true>(base, doff[jd], dst + 1024 * (wave * T::kDmaPerWave + jd));
        if (wave == 0) {
#pragma unroll
            for (int h = 0; h < T::kScaleDma; ++h)
                lds_dma4_so<true>(ksb + t0, 4 * (64 * h + lane), dst + T::kBytes + 256 * h);
        }
    };

    // tiles are numbered u = 0, 1, ... over this work-group's chunks: tile u is
    // tile u % TPC of the chunk of slot u / TPC
    int cc = __builtin_amdgcn_readfirstlane(chq[0]);   // chunk being computed
    int ic = cc;                                        // chunk being issued
    int issued = 0;
    if (cc >= 0) {
#pragma unroll
        for (int p = 0; p < kRing - 1; ++p) issue((int64_t)cc * kDynChunk + (int64_t)p * T::kKeys, p);
        issued = kRing - 1;
    }
    const int stores = (scores != nullptr) ? PPW : 0;     // score stores per tile and streaming wave
    for (int u = 0; cc >= 0; ++u) {
        const int ut = u % TPC;
        if (wave < kGrab) {
            // later issued: the DMAs of tiles u+1 .. issued-1 and the score stores
            // of the iterations since tile u was issued
            wait_vmcnt_le(__builtin_amdgcn_readfirstlane((issued - u - 1) * per + stores * min(u, kRing - 1)));
        }
        ring_barrier();   // every wave's part of tile u landed; tile u-1's readers are done
        if (ut == 0) post(u / TPC + 1);
        {
            const int un = u + kRing - 1;        // the tile to issue now
            if (un % TPC == 0) ic = ic >= 0 ? __builtin_amdgcn_readfirstlane(chq[(un / TPC) & 3]) : -1;
            if (ic >= 0) {
                issue((int64_t)ic * kDynChunk + (int64_t)(un % TPC) * T::kKeys, un % kRing);
                ++issued;
            }
        }
        if (wave < kGrab) {
            const int64_t t0 = (int64_t)cc * kDynChunk + (int64_t)ut * T::kKeys;
            const lds_u8* tile = (const lds_u8*)ring + (u % kRing) * T::kSlot;
            f32x16 acc[PPW];
#pragma unroll
            for (int p = 0; p < PPW; ++p) {
                const int row = (wave * PPW + p) * 32 + n;
                acc[p] = f32x16{};
#pragma unroll
                for (int t = 0; t < KSTEPS; ++t) {
                    const i32x4 lo = *(const __attribute__((address_space(3))) i32x4*)(tile + T::off(row, 4 * g + 2 * t));
                    const i32x4 hi = *(const __attribute__((address_space(3))) i32x4*)(tile + T::off(row, 4 * g + 2 * t + 1));
                    const i32x8 bb = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    const float ks = *(const __attribute__((address_space(3))) float*)(tile + T::kBytes + 4 * row);
                    acc[p] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[t], bb, acc[p], 0, 0, 0, a_e8, 0, e8m0_of(ks));
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            float res[PPW];
#pragma unroll
            for (int p = 0; p < PPW; ++p) {
                const int64_t sk = t0 + (wave * PPW + p) * 32 + n;
                float part = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    part = fmaf(wr[i], __int_as_float(max(__float_as_int(acc[p][i]), 0)), part);
                part = sum_x32(part);
                res[p] = sk <= apos ? part : neg_inf();
            }
#pragma unroll
            for (int p = 0; p < PPW; ++p) {
                const int64_t s0 = t0 + (wave * PPW + p) * 32;
                if (scores != nullptr && g == 0) store_score<true>(scores + (int64_t)qi * ld + s0 + n, res[p]);
                if (gmax != nullptr) {
                    const uint32_t m = max_x32(score_key(res[p]));
                    if (lane == 0) gmax[(int64_t)qi * ldg + (s0 >> 5)] = key_value(m);
                }
            }
        }
        if ((u + 1) % TPC == 0) cc = __builtin_amdgcn_readfirstlane(chq[((u + 1) / TPC) & 3]);
    }
}

// Several queries of one sequence per work-group (MTP verify, chunked prefill).
// Here the MFMA rate, not HBM, bounds the kernel, so the key tile in LDS must
// feed as many MFMAs per LDS read as registers allow, and each SIMD needs a
// second wave to issue MFMAs while the first waits on LDS or runs the epilogue.
// 8 waves (2 per SIMD). Wave w holds the A operands of 2 queries (pair qp =
// w mod QB/2) and takes NSUB of the 4 32-key subtiles of every tile; each key
// fragment read from LDS feeds the MFMAs of both queries.
constexpr int kMqWaves = 8;
constexpr int kMqThreads = 64 * kMqWaves;

template <int QB, bool FP8>
__global__ __launch_bounds__(kMqThreads) void indexer_score_mq(
    const uint8_t* __restrict__ q, const float* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ k,
    const float* __restrict__ k_scale, const int32_t* __restrict__ q_seq,
    const int32_t* __restrict__ q_pos, int n_q, int64_t n_cap,
    float* __restrict__ scores, int64_t ld, float* __restrict__ gmax, int64_t ldg, int chunk) {
    // 64 KiB tiles (256 bf16 / 512 fp8 keys) in a 2-slot ring: the keys come from
    // L2 (every work-group of a chunk reads the same ones), so one tile in flight
    // covers the latency, and the barrier and DMA issue are paid per 64 KiB
    using T = KeyTile<FP8, FP8 ? 512 : 256>;
    constexpr int kRingMq = 2;
    constexpr int QPW = 2;                       // queries per wave
    constexpr int NQP = QB / QPW;                // query pairs per work-group
    constexpr int NT = T::kKeys / 32;            // 32-key subtiles per tile
    constexpr int NSUB = NT * NQP / kMqWaves;    // subtiles per wave per tile
    static_assert(QB == 4 || QB == 8 || QB == 16, "QB");
    static_assert(NSUB >= 2 && NSUB % 2 == 0, "the fast path pairs subtiles");
    constexpr int KSTEPS = FP8 ? 2 : 8;
    constexpr int kDmaPerWave = T::kDma / kMqWaves;
    using AVec = std::conditional_t<FP8, i32x8, bf16x8>;
    typedef __attribute__((address_space(3))) uint8_t lds_u8;

    __shared__ __attribute__((aligned(16))) uint8_t ring[kRingMq * T::kSlot];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar: wave-uniform values stay in SGPRs
    const int n = lane & 31, g = lane >> 5;
    const int qb0 = blockIdx.y * QB;
    const int64_t c0 = (int64_t)blockIdx.x * chunk;
    if (c0 >= n_cap) return;
    const int64_t c1 = min(c0 + (int64_t)chunk, n_cap);
    const int jw0 = (wave % NQP) * QPW;          // this wave's first query in the block
    const int sub0 = (wave / NQP) * NSUB;        // and first subtile
    // LDS byte offset, inside a 32-key subtile, of the 16-byte chunks this lane
    // reads (row n; the row's swizzle depends on n only, as subtiles are 32 rows)
    constexpr int kReads = FP8 ? 2 * KSTEPS : KSTEPS;
    uint32_t lds_off[kReads];
#pragma unroll
    for (int t = 0; t < kReads; ++t) lds_off[t] = T::off(n, FP8 ? 4 * g + t : 8 * g + t);

    AVec a[QPW][KSTEPS];
    float wr[QPW][16];
    int apos[QPW], a_e8[QPW];
#pragma unroll
    for (int jj = 0; jj < QPW; ++jj) {
        const int qi = qb0 + jw0 + jj;
        const bool ok = qi < n_q;
        const int qr = ok ? qi : 0;
        apos[jj] = ok ? q_pos[qi] : -1;
        const uint8_t* qh = q + ((int64_t)qr * kHeads + n) * T::kRowBytes;
#pragma unroll
        for (int t = 0; t < KSTEPS; ++t) {
            if constexpr (FP8) {
                const i32x4* p = (const i32x4*)(qh + 64 * g + 32 * t);
                const i32x4 lo = p[0], hi = p[1];
                a[jj][t] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            } else {
                a[jj][t] = *(const bf16x8*)(qh + 2 * (64 * g + 8 * t));
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int h = 8 * (i >> 2) + 4 * g + (i & 3);
            wr[jj][i] = ok ? w[(int64_t)qr * kHeads + h] : 0.f;
        }
        if constexpr (FP8) a_e8[jj] = e8m0_of(q_scale[(int64_t)qr * kHeads + n]);
        else a_e8[jj] = 127;
    }
    wait_vmcnt<0>();

    const int per = kDmaPerWave + ((FP8 && wave == 0) ? T::kScaleDma : 0);
    const uint32_t ring_base = (uint32_t)(uintptr_t)(lds_u8*)ring;

    int j0 = 0;
    while (j0 < QB && qb0 + j0 < n_q) {
        const int seq = q_seq[qb0 + j0];
        int j1 = j0 + 1;
        int maxpos = q_pos[qb0 + j0];
        while (j1 < QB && qb0 + j1 < n_q && q_seq[qb0 + j1] == seq) {
            maxpos = max(maxpos, (int)q_pos[qb0 + j1]);
            ++j1;
        }
        const uint8_t* kb = k + (int64_t)seq * n_cap * T::kRowBytes;
        const float* ksb = FP8 ? k_scale + (int64_t)seq * n_cap : nullptr;
        const int64_t t_end = min(c1, (int64_t)maxpos + 1);
        const int na = t_end > c0 ? (int)((t_end - c0 + T::kKeys - 1) / T::kKeys) : 0;
        const int nt_all = (int)((c1 - c0 + T::kKeys - 1) / T::kKeys);
        bool inrun[QPW];
        int nin = 0;
#pragma unroll
        for (int jj = 0; jj < QPW; ++jj) {
            inrun[jj] = jw0 + jj >= j0 && jw0 + jj < j1;
            nin += inrun[jj] ? 1 : 0;
        }
        // vector-memory stores this wave issues per tile, as a lower bound (the wait
        // below lets that many stores stay outstanding besides the later tiles'
        // DMAs; counting more than are issued would let it pass before this tile's
        // DMAs land). The fast path issues one store per subtile for both queries
        // (two with group maxima); the general path one per run query and subtile
        // (two with group maxima) below the chunk end.
        // Without a score buffer only group maxima are stored; they go uncounted.
        const int stores = nin > 0 && scores != nullptr ? NSUB : 0;

        auto issue = [&](int ti, int slot) __attribute__((always_inline)) {
            const int64_t t0 = c0 + (int64_t)ti * T::kKeys;
            const uint32_t dst = ring_base + slot * T::kSlot;
#pragma unroll
            for (int jd = 0; jd < kDmaPerWave; ++jd) {
                const int i = wave * kDmaPerWave + jd;
                const int r = i * T::kRowsPerDma + lane / T::kChunks;
                const int p = lane % T::kChunks;
                const int c = p ^ T::swz(r);
                const int64_t krow = min(t0 + r, c1 - 1);
                lds_dma16(kb + krow * T::kRowBytes + 16 * c, dst + 1024 * i);
            }
            if constexpr (FP8) {
                if (wave == 0) {
#pragma unroll
                    for (int h = 0; h < T::kScaleDma; ++h) {
                        const int64_t krow = min(t0 + 64 * h + lane, c1 - 1);
                        lds_dma4(ksb + krow, dst + T::kBytes + 256 * h);
                    }
                }
            }
        };

        for (int p = 0; p < kRingMq - 1; ++p)
            if (p < na) issue(p, p);
        for (int ti = 0; ti < nt_all; ++ti) {
            const int64_t t0 = c0 + (int64_t)ti * T::kKeys;
            const bool active = ti < na;
            if (active) {
                const int later = min(na, ti + kRingMq - 1) - ti - 1;
                wait_vmcnt_le(__builtin_amdgcn_readfirstlane(later * per + stores * min(ti, kRingMq - 1)));
                ring_barrier();
                if (ti + kRingMq - 1 < na) issue(ti + kRingMq - 1, (ti + kRingMq - 1) % kRingMq);
            }
            if (nin == 0) continue;                       // wave-uniform
            const uint32_t tile_addr = ring_base + (ti % kRingMq) * T::kSlot;
            // Fast path: both queries in the run and every key of this wave's
            // subtiles causal for both. Straight-line code in which the epilogue of
            // subtile ns - 1 is interleaved with the MFMAs of subtile ns, so the VALU
            // work runs while the matrix core is busy.
            const int64_t s_first = t0 + sub0 * 32, s_last = s_first + NSUB * 32 - 1;
            bool fast = active && nin == QPW && s_last < c1;
#pragma unroll
            for (int jj = 0; jj < QPW; ++jj) fast = fast && s_last <= apos[jj];
            if (fast) {
                f32x16 acc[2][QPW];
                // epilogue in two parts: the per-lane head sums (VALU only, scheduled
                // between the MFMAs of the next subtile) and the cross-half add + store
                auto head_sums = [&](const f32x16 (&c)[QPW], float (&part)[QPW]) __attribute__((always_inline)) {
#pragma unroll
                    for (int jj = 0; jj < QPW; ++jj) {
                        float acc_s = 0.f;
#pragma unroll
                        for (int i = 0; i < 16; ++i)
                            acc_s = fmaf(wr[jj][i], __int_as_float(max(__float_as_int(c[jj][i]), 0)), acc_s);
                        part[jj] = acc_s;
                    }
                };
                // One permlane32 swap of the two queries' partial sums leaves query
                // jw0 + g's score of key s0 + n in lane 32g + n: one add and one store
                // serve both queries, and one 32-lane max gives both group maxima. The
                // max runs on order-preserving integer keys (-0.0 folded into +0.0), one
                // DPP max instruction per step, as in the other score kernels: a float
                // max with a DPP operand costs a move and two canonicalisations more.
                // Split in four parts that the fp8 step places between its (64-cycle)
                // MFMAs.
                static_assert(QPW == 2, "the finish pairs two queries");
                struct Fin { float sc; uint32_t m; int64_t s0; };
                auto fin_a = [&](int ns, const float (&part)[QPW], Fin& f) __attribute__((always_inline)) {
                    f.s0 = t0 + (sub0 + ns) * 32;
                    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]),
                                                                    __float_as_uint(part[1]), false, false);
                    f.sc = __uint_as_float(r[0]) + __uint_as_float(r[1]);
                    if (scores != nullptr)                     // uniform
                        store_score<FP8>(scores + (int64_t)(qb0 + jw0 + g) * ld + f.s0 + n, f.sc);
                };
                auto fin_b = [&](Fin& f) __attribute__((always_inline)) {
                    if (gmax == nullptr) return;               // uniform
                    uint32_t v = score_key(f.sc);
                    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xb1, 0xf, 0xf, false));   // lane ^ 1
                    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4e, 0xf, 0xf, false));   // lane ^ 2
                    f.m = v;
                };
                auto fin_c = [&](Fin& f) __attribute__((always_inline)) {
                    if (gmax == nullptr) return;
                    uint32_t v = f.m;
                    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false));  // 7 - lane in 8
                    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false));  // 15 - lane in 16
                    f.m = v;
                };
                auto fin_d = [&](Fin& f) __attribute__((always_inline)) {
                    if (gmax == nullptr) return;
                    const auto r = __builtin_amdgcn_permlane16_swap(f.m, f.m, false, false);        // other row
                    const float m = key_value(max((uint32_t)r[0], (uint32_t)r[1]));
                    if (n == 0) gmax[(int64_t)(qb0 + jw0 + g) * ldg + (f.s0 >> 5)] = m;
                };
                auto finish = [&](int ns, const float (&part)[QPW]) __attribute__((always_inline)) {
                    Fin f;
                    fin_a(ns, part, f);
                    fin_b(f);
                    fin_c(f);
                    fin_d(f);
                };
                // One step of the software pipeline: the LDS reads and MFMAs of subtile
                // ns into cm and, when EPI, the head sums of the previous subtile (ce) cut
                // into pieces that sit between those MFMAs, so that the VALU work issues
                // while the matrix core is busy. The order is fixed in the source:
                // scheduling fences between the pieces keep the compiler from regrouping
                // them (it otherwise clusters all MFMAs and all VALU work).
                auto fence = []() __attribute__((always_inline)) { __builtin_amdgcn_sched_barrier(0); };
                auto piece = [&](const f32x16 (&ce)[QPW], float (&part)[QPW], int jj, int i0, int cnt)
                    __attribute__((always_inline)) {
#pragma unroll
                    for (int i = i0; i < i0 + cnt; ++i)
                        part[jj] = fmaf(wr[jj][i], __int_as_float(max(__float_as_int(ce[jj][i]), 0)),
                                        i == 0 ? 0.f : part[jj]);
                };
                auto step = [&](auto epi_c, auto fin_c_, int ns, f32x16 (&cm)[QPW], const f32x16 (&ce)[QPW],
                                float (&part)[QPW], int ns_fin, const float (&pf)[QPW]) __attribute__((always_inline)) {
                    constexpr bool EPI = decltype(epi_c)::value;
                    constexpr bool FIN = decltype(fin_c_)::value;   // finish subtile ns_fin (sums in pf)
                    Fin f;
                    const int nt = sub0 + ns;
                    const uint32_t sub_addr = tile_addr + nt * 32 * T::kRowBytes;
                    fence();
                    if constexpr (FP8) {
                        // 4 x 16 bytes of key codes and the key scale, then 4 MFMAs with a
                        // quarter of the head sums after the reads and after each MFMA
                        i32x4 ch[4];
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            ch[t] = *(const __attribute__((address_space(3))) i32x4*)(
                                (const lds_u8*)(uintptr_t)(sub_addr + lds_off[t]));
                        const float ksf = *(const __attribute__((address_space(3))) float*)(
                            (const lds_u8*)(uintptr_t)(tile_addr + T::kBytes + nt * 128) + 4 * n);
                        fence();
                        if constexpr (EPI) piece(ce, part, 0, 0, 8);
                        fence();
                        const int ke = e8m0_of(ksf);
                        const i32x8 b0 = {ch[0][0], ch[0][1], ch[0][2], ch[0][3], ch[1][0], ch[1][1], ch[1][2], ch[1][3]};
                        const i32x8 b1 = {ch[2][0], ch[2][1], ch[2][2], ch[2][3], ch[3][0], ch[3][1], ch[3][2], ch[3][3]};
                        cm[0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[0][0], b0, f32x16{}, 0, 0, 0, a_e8[0], 0, ke);
                        fence();
                        if constexpr (EPI) piece(ce, part, 0, 8, 8);
                        fence();
                        if constexpr (FIN) fin_a(ns_fin, pf, f);
                        fence();
                        cm[1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[1][0], b0, f32x16{}, 0, 0, 0, a_e8[1], 0, ke);
                        fence();
                        if constexpr (EPI) piece(ce, part, 1, 0, 8);
                        if constexpr (FIN) fin_b(f);
                        fence();
                        cm[0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[0][1], b1, cm[0], 0, 0, 0, a_e8[0], 0, ke);
                        fence();
                        if constexpr (EPI) piece(ce, part, 1, 8, 8);
                        if constexpr (FIN) fin_c(f);
                        fence();
                        cm[1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[1][1], b1, cm[1], 0, 0, 0, a_e8[1], 0, ke);
                        fence();
                        if constexpr (FIN) fin_d(f);
                    } else {
                        // the B operand of k-step t is read two k-steps ahead; one eighth
                        // of a query's head sums (2 values) after each MFMA
                        bf16x8 b[KSTEPS];
                        auto rd = [&](int t) __attribute__((always_inline)) {
                            b[t] = *(const __attribute__((address_space(3))) bf16x8*)(
                                (const lds_u8*)(uintptr_t)(sub_addr + lds_off[t]));
                        };
                        rd(0);
                        rd(1);
#pragma unroll
                        for (int t = 0; t < KSTEPS; ++t) {
                            if (t + 2 < KSTEPS) rd(t + 2);
                            fence();
#pragma unroll
                            for (int jj = 0; jj < QPW; ++jj) {
                                cm[jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                    a[jj][t], b[t], t == 0 ? f32x16{} : cm[jj], 0, 0, 0);
                                fence();
                                if constexpr (EPI) piece(ce, part, jj, 2 * t, 2);
                                fence();
                            }
                        }
                        static_assert(!FIN || FP8, "bf16 steps finish outside");
                    }
                    fence();
                };
                using Yes = std::integral_constant<bool, true>;
                using No = std::integral_constant<bool, false>;
                // Subtiles in pairs (acc[0]: even, acc[1]: odd). Step ns runs the MFMAs
                // of subtile ns, the head sums of subtile ns - 1 and the finish of
                // subtile ns - 2 (head sums alternate between pa and pb); the first
                // two steps and the last two finishes are peeled, so that no branch
                // splits a step.
                float pa[QPW], pb[QPW];
                if constexpr (FP8) {
                    step(No{}, No{}, 0, acc[0], acc[1], pa, 0, pb);
                    step(Yes{}, No{}, 1, acc[1], acc[0], pa, 0, pb);             // pa: subtile 0
#pragma unroll 1
                    for (int ns = 2; ns + 1 < NSUB; ns += 2) {
                        step(Yes{}, Yes{}, ns, acc[0], acc[1], pb, ns - 2, pa);  // pb: ns - 1
                        step(Yes{}, Yes{}, ns + 1, acc[1], acc[0], pa, ns - 1, pb);  // pa: ns
                    }
                    head_sums(acc[1], pb);                                       // subtile NSUB - 1
                    finish(NSUB - 2, pa);
                    finish(NSUB - 1, pb);
                } else {
                    // bf16 MFMAs are short (32 cycles): each subtile's finish runs as
                    // one block right after the next step (measured faster than
                    // spreading it over the MFMAs)
                    step(No{}, No{}, 0, acc[0], acc[1], pa, 0, pb);
#pragma unroll 1
                    for (int ns = 0; ns + 2 < NSUB; ns += 2) {
                        step(Yes{}, No{}, ns + 1, acc[1], acc[0], pa, 0, pb);
                        finish(ns, pa);
                        step(Yes{}, No{}, ns + 2, acc[0], acc[1], pa, 0, pb);
                        finish(ns + 1, pa);
                    }
                    step(Yes{}, No{}, NSUB - 1, acc[1], acc[0], pa, 0, pb);
                    finish(NSUB - 2, pa);
                    head_sums(acc[1], pa);
                    finish(NSUB - 1, pa);
                }
                continue;
            }
#pragma unroll 1
            for (int ns = 0; ns < NSUB; ++ns) {
                const int nt = sub0 + ns;
                const int64_t s0 = t0 + nt * 32;
                bool any = false;
#pragma unroll
                for (int jj = 0; jj < QPW; ++jj) any = any || (active && inrun[jj] && s0 <= apos[jj]);
                if (any) {                                        // wave-uniform
                    f32x16 acc[QPW];
#pragma unroll
                    for (int t = 0; t < KSTEPS; ++t) {
                        if constexpr (FP8) {
                            const lds_u8* base = (const lds_u8*)(uintptr_t)(tile_addr + nt * 32 * T::kRowBytes);
                            const i32x4 lo = *(const __attribute__((address_space(3))) i32x4*)(base + lds_off[2 * t]);
                            const i32x4 hi = *(const __attribute__((address_space(3))) i32x4*)(base + lds_off[2 * t + 1]);
                            const i32x8 b = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                            const int ke = e8m0_of(*(const __attribute__((address_space(3))) float*)(
                                (const lds_u8*)(uintptr_t)(tile_addr + T::kBytes + nt * 128) + 4 * n));
#pragma unroll
                            for (int jj = 0; jj < QPW; ++jj)
                                acc[jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                    a[jj][t], b, t == 0 ? f32x16{} : acc[jj], 0, 0, 0, a_e8[jj], 0, ke);
                        } else {
                            const lds_u8* base = (const lds_u8*)(uintptr_t)(tile_addr + nt * 32 * T::kRowBytes);
                            const bf16x8 b = *(const __attribute__((address_space(3))) bf16x8*)(base + lds_off[t]);
#pragma unroll
                            for (int jj = 0; jj < QPW; ++jj)
                                acc[jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                    a[jj][t], b, t == 0 ? f32x16{} : acc[jj], 0, 0, 0);
                        }
                    }
#pragma unroll
                    for (int jj = 0; jj < QPW; ++jj) {
                        if (!inrun[jj]) continue;                 // wave-uniform
                        // keys s0 + n with n <= lim are causal for this query
                        const int lim = (int)min((int64_t)apos[jj] - s0, (int64_t)64);
                        float part = 0.f;
#pragma unroll
                        for (int i = 0; i < 16; ++i)              // relu on the bit pattern: exact
                            part = fmaf(wr[jj][i], __int_as_float(max(__float_as_int(acc[jj][i]), 0)), part);
                        part = sum_x32(part);
                        const float res = (active && n <= lim) ? part : neg_inf();
                        if (scores != nullptr && g == 0 && s0 + n < c1)
                            scores[(int64_t)(qb0 + jw0 + jj) * ld + s0 + n] = res;
                        if (gmax != nullptr && s0 < c1) {              // uniform
                            const uint32_t m = max_x32(score_key(s0 + n < c1 ? res : neg_inf()));
                            if (lane == 0) gmax[(int64_t)(qb0 + jw0 + jj) * ldg + (s0 >> 5)] = key_value(m);
                        }
                    }
                } else {
#pragma unroll
                    for (int jj = 0; jj < QPW; ++jj) {
                        if (!inrun[jj]) continue;
                        if (scores != nullptr && g == 0 && s0 + n < c1)
                            scores[(int64_t)(qb0 + jw0 + jj) * ld + s0 + n] = neg_inf();
                        if (gmax != nullptr && s0 < c1 && lane == 0)
                            gmax[(int64_t)(qb0 + jw0 + jj) * ldg + (s0 >> 5)] = neg_inf();
                    }
                }
            }
        }
        ring_barrier();
        j0 = j1;
    }
}

template <int QB>
hipError_t launch_mq(bool fp8, dim3 grid, hipStream_t st, const void* q, const float* qs,
                     const float* w, const void* k, const float* ks, const int32_t* q_seq,
                     const int32_t* q_pos, int n_q, int64_t n_cap, float* scores, int64_t ld,
                     float* gmax, int chunk) {
    const int64_t ldg = (ld + 31) / 32;
    if (fp8)
        hipLaunchKernelGGL((indexer_score_mq<QB, true>), grid, dim3(kMqThreads), 0, st,
                           (const uint8_t*)q, qs, w, (const uint8_t*)k, ks, q_seq, q_pos, n_q,
                           n_cap, scores, ld, gmax, ldg, chunk);
    else
        hipLaunchKernelGGL((indexer_score_mq<QB, false>), grid, dim3(kMqThreads), 0, st,
                           (const uint8_t*)q, qs, w, (const uint8_t*)k, ks, q_seq, q_pos, n_q,
                           n_cap, scores, ld, gmax, ldg, chunk);
    return hipGetLastError();
}

template <int QB, bool FP8, bool NT, bool STAGE = false>
void launch_qb_t(dim3 grid, hipStream_t st, const void* q, const float* qs, const float* w,
                 const void* k, const float* ks, const int32_t* q_seq, const int32_t* q_pos,
                 int n_q, int64_t n_cap, float* scores, int64_t ld, float* gmax, int chunk) {
    hipLaunchKernelGGL((indexer_score_kernel<QB, FP8, NT, STAGE>), grid, dim3(kThreads), 0, st, (const uint8_t*)q, qs, w,
                       (const uint8_t*)k, ks, q_seq, q_pos, n_q, n_cap, scores, ld, gmax,
                       (ld + 31) / 32, chunk);
}

template <int QB>
hipError_t launch_qb(bool fp8, bool nt, dim3 grid, hipStream_t st, const void* q, const float* qs,
                     const float* w, const void* k, const float* ks, const int32_t* q_seq,
                     const int32_t* q_pos, int n_q, int64_t n_cap, float* scores, int64_t ld,
                     float* gmax, int chunk) {
    if constexpr (QB == 1) {
        if (!fp8 && chunk <= kStageKeys) {                  // the chunk's scores fit in LDS
            auto* g = nt ? launch_qb_t<1, false, true, true> : launch_qb_t<1, false, false, true>;
            g(grid, st, q, qs, w, k, ks, q_seq, q_pos, n_q, n_cap, scores, ld, gmax, chunk);
            return hipGetLastError();
        }
    }
    auto* f = fp8 ? (nt ? launch_qb_t<QB, true, true> : launch_qb_t<QB, true, false>)
                  : (nt ? launch_qb_t<QB, false, true> : launch_qb_t<QB, false, false>);
    f(grid, st, q, qs, w, k, ks, q_seq, q_pos, n_q, n_cap, scores, ld, gmax, chunk);
    return hipGetLastError();
}

// The current device's copy of g_dyn_ctr (host code must not use the array's
// name as a device address; its address is looked up once per device).
constexpr int kMaxDevices = 64;
std::mutex g_dyn_mu;
int* g_dyn_ptr[kMaxDevices] = {};
hipError_t dyn_counters(int** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_dyn_mu);
    if (g_dyn_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_dyn_ctr));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_dyn_ptr[dev] = (int*)p;
    }
    *out = g_dyn_ptr[dev];
    return hipSuccess;
}

}  // namespace

hipError_t launch_indexer_score(bool fp8, const void* q, const float* q_scale, const float* w,
                                const void* k, const float* k_scale, const int32_t* q_seq,
                                const int32_t* q_pos, int n_q, int batch, int64_t n_cap,
                                float* scores, int64_t ld, float* gmax, hipStream_t stream) {
    // Queries per work-group: the typical number of queries per sequence.
    const int per_seq = n_q / (batch > 0 ? batch : 1);
    const int qb = per_seq >= 16 ? 16 : per_seq >= 8 ? 8 : per_seq >= 4 ? 4 : per_seq >= 2 ? 2 : 1;
    const int64_t n_qblk = (n_q + qb - 1) / qb;
    // Key chunk per work-group, 1K..16K keys (64K with several queries per
    // work-group). One query per work-group streams
    // from HBM: bf16 rows run best with >= 2048 work-groups (~1 MiB each), fp8
    // rows with >= 512 (~2 MiB each: half the bytes per key, so the ring fill
    // each work-group start costs is spread over more keys). Several queries
    // per work-group are compute bound, and fewer, longer chunks save that
    // refill too: >= 256 work-groups, one per CU (8 x 256K keys with 8 queries
    // per sequence: 142 us against 149 / 171 / 208 us at 512 / 1024 / 2048;
    // prefill has 256 query blocks, so its chunks stay at the cap). The
    // multi-query cap is 64K keys: each work-group first loads the A operands
    // of its 16 queries (128 KiB), and 4096 x 128K-key prefill measured 1.3-2.1%
    // faster than with 16K (32K: 1%; 128K: mixed).
    // Launches too small to give every CU a 1024-key chunk (a few short rows)
    // go down to one LDS tile per work-group: their time is one work-group's
    // start-up and ring fill, so more and shorter chunks finish sooner.
    const int64_t min_wg = qb >= 4 ? 256 : fp8 ? 512 : 2048;
    const int64_t min_chunk = qb >= 4 ? (fp8 ? 512 : 256) : (fp8 ? 256 : 128);
    int64_t chunk = qb >= 4 ? 65536 : 16384;
    while (chunk > 1024 && n_qblk * ((n_cap + chunk - 1) / chunk) < min_wg) chunk >>= 1;
    if (n_qblk * ((n_cap + chunk - 1) / chunk) < 256)
        while (chunk > min_chunk && n_qblk * ((n_cap + chunk - 1) / chunk) < 256) chunk >>= 1;
    const dim3 grid((unsigned)((n_cap + chunk - 1) / chunk), (unsigned)n_qblk);
    // One query block per sequence (decode): every key is read by one
    // work-group only, so the one-query kernel streams its keys with the
    // non-temporal hint (measured: 399 -> 370 us at 64 x 128K bf16 keys,
    // 230 -> 201 us at 8 x 1M fp8 keys). With more blocks per sequence the
    // blocks of a chunk share its keys through L2; the multi-query kernel keeps
    // plain loads (compute bound; the hint measured 1% slower there).
    const bool nt = (per_seq + qb - 1) / qb <= 1;
    // fp8 decode whose rows are whole 1024-key chunks, with at least 32K keys
    // per CU and a query count dividing 256: the persistent grid
    if (qb == 1 && fp8 && nt && n_q <= kDynMaxQ && kDynWGs % n_q == 0 && n_cap % kDynChunk == 0 &&
        (int64_t)n_q * n_cap >= (int64_t)kDynWGs * 32768 && n_cap / kDynChunk < (1 << 30) - kDynWGs) {
        int* ctr = nullptr;
        const hipError_t e = dyn_counters(&ctr);
        if (e != hipSuccess) return e;
        ctr += (launch_tag() % kDynSlots) * kDynMaxQ;
        hipLaunchKernelGGL(indexer_score_dyn, dim3(kDynWGs), dim3(kDynThreads), 0, stream, (const uint8_t*)q, q_scale, w,
                           (const uint8_t*)k, k_scale, q_seq, q_pos, n_q, n_cap, scores, ld, gmax, (ld + 31) / 32, ctr);
        return hipGetLastError();
    }
    switch (qb) {
        case 16: return launch_mq<16>(fp8, grid, stream, q, q_scale, w, k, k_scale, q_seq, q_pos, n_q, n_cap, scores, ld, gmax, (int)chunk);
        case 8: return launch_mq<8>(fp8, grid, stream, q, q_scale, w, k, k_scale, q_seq, q_pos, n_q, n_cap, scores, ld, gmax, (int)chunk);
        case 4: return launch_mq<4>(fp8, grid, stream, q, q_scale, w, k, k_scale, q_seq, q_pos, n_q, n_cap, scores, ld, gmax, (int)chunk);
        case 2: return launch_qb<2>(fp8, nt, grid, stream, q, q_scale, w, k, k_scale, q_seq, q_pos, n_q, n_cap, scores, ld, gmax, (int)chunk);
        default: return launch_qb<1>(fp8, nt, grid, stream, q, q_scale, w, k, k_scale, q_seq, q_pos, n_q, n_cap, scores, ld, gmax, (int)chunk);
    }
}

}  // namespace gsa

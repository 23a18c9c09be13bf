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
// One work-group (8 waves) takes one query and a contiguous slice of its
// selected rows ("split"); slices are merged with their log-sum-exp when a
// query is split. Wave w serves heads 16*(w%4) .. +15 and latent half w/4 of
// P.V; the two waves of a head group (w, w^4) split Q.K in one of two ways and
// swap through LDS, waiting on the partner's flag only, not on the whole
// work-group:
//   dim pair  each takes Q.K over half of the 576 dims for all 32 rows of a
//             block and they swap their fp32 partial scores (a + b == b + a, so
//             both hold the identical S and run the identical softmax); 36
//             registers of Q per wave.
//   row pair  each takes Q.K over all 576 dims for 16 of the 32 rows, runs the
//             softmax of its own rows only, and they swap their bf16 P with the
//             running max each proposes (the larger one is the pair's: where it
//             moved, which is rare, both recompute P and swap again); half the softmax work
//             and half the swapped bytes, for 72 registers of Q, whose loads
//             double: the layout of slices of 1024 rows or more.
// Either way 64 registers of O per wave, which leaves room for two waves per
// SIMD; the LDS reads per 32-row block (each head group reads the block once
// for Q.K and once for P.V) are what bounds this kernel.
// FP8 latent cache ("GLM-5.2 总览" tbl-glm52-config: ~656 bytes per token and
// layer with per-group scales; glossary: E4M3 on the 512-dim latent): rows of
// [512 E4M3 | 4 fp32 scales | 64 bf16 RoPE] are gathered into a ring as they
// are. The row-pair layout computes on them there: Q.K's K operand converts 8
// codes with the row's group scale (exact), and P.V reads V with the 8-bit
// transpose read, converts it unscaled and takes the rows' scales into P
// instead (a power of two, so P.V forms the products of the dequantised rows),
// with half the LDS bytes of a bf16 block. The dim-pair layout (short slices,
// where those conversions per wave cost more than they save) widens each
// block to the bf16 layout first (one scaled conversion per two codes, a
// barrier) and runs the bf16 compute. Both give the outputs of the
// dequantised rows bit for bit.
// Per 32-row block:
//   gather  global_load_lds_dwordx4 copies the block's 32 x 1152 bytes straight
//           into LDS (no staging registers); each wave instruction moves 1 KiB
//           of whole 128-byte lines. A ring of kRing LDS blocks keeps
//           kRing - 1 blocks in flight per CU. Rows sit at a 1184-byte pitch
//           (32 bytes of padding), at which the SQ_LDS_BANK_CONFLICT counter
//           reads zero for Q.K's 16-row reads and P.V's transpose reads alike
//           (with 16 bytes of padding both conflicted, 17.8M cycles per
//           128K launch), and every LDS address is one base register plus an
//           immediate. Indices of -1 load a static zero row.
//   Q.K     S^T (rows x heads) on v_mfma_f32_16x16x32_bf16 with Q resident in
//           registers; in that layout a lane holds 8 rows of one head, so the
//           softmax max/sum need only two cross-lane steps.
//   softmax online, base 2; the running max moves only when a block max
//           exceeds it by more than 2^8, so the O rescale is rare.
//   P.V     P (bf16) is the MFMA A operand straight from registers; the V
//           operand is read from the same block with the gfx950 LDS transpose
//           read (ds_read_b64_tr_b16: 16 lanes' 4x16 block comes back as
//           16x4), so no transposed copy is stored.
#include "device_common.h"
#include "launch.h"

namespace gsa {

// A 1152-byte all-zero cache row: gather source for index -1 (never written).
__device__ __attribute__((aligned(16))) uint8_t g_zero_row[1152];

namespace {

constexpr int kHeads = 64;
constexpr int kLat = 512;
constexpr int kRowBytes = 1152;                 // 576 bf16
constexpr int kChunksPerRow = kRowBytes / 16;   // 72
constexpr int kBlk = 32;                        // rows per block
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kPitch = kRowBytes + 32;          // LDS row pitch
constexpr int kChunksPerPitch = kPitch / 16;    // 74 (the last two are padding)
constexpr int kDmaPerBlock = (kBlk * kPitch + 1023) / 1024;   // 37 one-KiB LDS-DMA instructions
constexpr int kBuf = kDmaPerBlock * 1024;       // 37 KiB per ring slot
constexpr int kDmaBig = kDmaPerBlock - kWaves * (kDmaPerBlock / kWaves);   // waves issuing one more (5)
constexpr int kDmaLo = kDmaPerBlock / kWaves;   // 4
constexpr int kDmaHi = kDmaLo + 1;              // 5
constexpr int kRing = 3;                        // LDS blocks in the ring
constexpr int kMaxRows = 2048;
constexpr float kRescale = 8.0f;                // lazy-rescale threshold (log2 units)
constexpr int kMaxLayersPerLaunch = 8;
constexpr int kRowPairRows = 1024;              // shortest slice for the row-pair layout

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// FP8 latent rows ([512 E4M3 | 4 fp32 scales | 64 bf16 RoPE], 656 bytes): the
// gather lands them unpadded in their own ring.
constexpr int kRowBytesF8 = 656;
constexpr int kChunksF8 = kRowBytesF8 / 16;     // 41
constexpr int kPitchF8 = 656;                   // staging row pitch
constexpr int kDmaF8 = (kBlk * kPitchF8 + 1023) / 1024;   // 21
constexpr int kStageBuf = kDmaF8 * 1024;
constexpr int kDmaLoF8 = kDmaF8 / kWaves;       // 2
constexpr int kDmaHiF8 = kDmaLoF8 + 1;          // 3
constexpr int kDmaBigF8 = kDmaF8 - kWaves * kDmaLoF8;       // 5

__shared__ __attribute__((aligned(16))) uint8_t g_ring[kRing * kBuf];
__shared__ __attribute__((aligned(16))) uint8_t g_stage[kRing * kStageBuf];
__shared__ __attribute__((aligned(16))) uint8_t g_blk[kBuf];
__shared__ int32_t g_rows[kMaxRows];
__shared__ f32x4 g_xs[kWaves][2][64];           // partial S^T of each wave (2 KiB per wave)
__shared__ int g_xflag[kWaves];                  // the block (+1) whose swap post each wave has made
// row-pair layout: each wave's bf16 P of its 16 rows, the running max it was
// computed with, and (at the end) its row sums, per head
__shared__ bf16x4 g_xp[kWaves][64];
__shared__ float g_xm[kWaves][16];
__shared__ float g_xl[kWaves][16];

__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }


typedef int v2i __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i lds_v2i;

// 8 E4M3 codes (bytes 0..7 of c) times the power-of-two scale s, as 8 bf16
// (exact: 4 significand bits and a power of two fit bf16), in byte order.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(v2i c, float s) {
    const auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)c[0], s, false);
    const auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)c[0], s, true);
    const auto d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)c[1], s, false);
    const auto e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)c[1], s, true);
    return bf16x8{a[0], a[1], b[0], b[1], d[0], d[1], e[0], e[1]};
}

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// Largest value over the 16 lanes of a row (DPP: two quad permutations, the
// half-row and row mirrors), in every lane of the row.
__device__ __forceinline__ float max_row16(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xb1, 0xf, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4e, 0xf, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xf, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xf, 0xf, false)));
    return v;
}

// Per-layer operands of one launch (kernel argument, indexed by blockIdx.z):
// the layers of an IndexShare group share the index buffer and are independent
// otherwise, so one launch covers all of them.
struct LayerArgs {
    const uint8_t* q_lat[kMaxLayersPerLaunch];
    const uint8_t* q_rope[kMaxLayersPerLaunch];
    const uint8_t* kv[kMaxLayersPerLaunch];
    float* out[kMaxLayersPerLaunch];
    float* lse[kMaxLayersPerLaunch];
};

// s_waitcnt lgkmcnt(0) alone: this wave's LDS writes have landed
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Cross-lane max / sum over lanes l and l^16 (l^32): the gfx950 permlane swaps
// return, for every lane, its own value and its partner's, in some order.
__device__ __forceinline__ float max_x16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_x32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_x16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int PER>
__device__ __forceinline__ void wait_block(int later) {
    if (later >= 2) wait_vmcnt<2 * PER>();
    else if (later == 1) wait_vmcnt<PER>();
    else wait_vmcnt<0>();
}

template <bool FP8KV, bool RP>
__global__ __launch_bounds__(kThreads) void sparse_mla_kernel(
    LayerArgs L, const int32_t* __restrict__ q_seq, const int32_t* __restrict__ idx, int k,
    int n_q, int64_t n_cap, const int32_t* __restrict__ block_table, int page_size, int max_pages,
    float scale_log2, int rows_per_split, _Float16* __restrict__ part_o_all,
    float* __restrict__ part_ml_all) {
    // this work-group's layer (uniform): its operands and its part of the workspace
    const int layer = blockIdx.z;
    const uint8_t* __restrict__ q_lat = L.q_lat[layer];
    const uint8_t* __restrict__ q_rope = L.q_rope[layer];
    const uint8_t* __restrict__ kv = L.kv[layer];
    float* __restrict__ out = L.out[layer];
    float* __restrict__ lse = L.lse[layer];
    _Float16* __restrict__ part_o = part_o_all + (size_t)layer * n_q * gridDim.x * kHeads * kLat;
    float* __restrict__ part_ml = part_ml_all + (size_t)layer * n_q * gridDim.x * kHeads * 4;
    int32_t* rows_s = g_rows;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    const int hg = wave & 3, hf = wave >> 2;           // head group, latent half
    const int q = blockIdx.y, split = blockIdx.x, n_split = gridDim.x;
    const int r0 = split * rows_per_split;
    const int nrows = rows_per_split;
    const int seq = q_seq[q];
    // Q as the B operand: head 16*hg + l16, K-steps t = 9*hf .. 9*hf+8 of the
    // 576 dims (row-pair layout: all 18), dims 32t + 8g .. +8; steps 16 and 17
    // are the RoPE dims. Issued before the index loads, so that the two
    // latencies overlap (the index stores to LDS wait for every earlier load);
    // the fence keeps that order.
    const int head = 16 * hg + l16;
    constexpr int QS = RP ? 18 : 9;
    bf16x8 qr[QS];
    {
        const uint8_t* ql = q_lat + ((int64_t)q * kHeads + head) * (kLat * 2);
        const uint8_t* qp = q_rope + ((int64_t)q * kHeads + head) * (64 * 2);
#pragma unroll
        for (int j = 0; j < QS; ++j) {
            const int t = RP ? j : 9 * hf + j;
            qr[j] = t < 16 ? *(const bf16x8*)(ql + 2 * (32 * t + 8 * g))
                           : *(const bf16x8*)(qp + 2 * (32 * (t - 16) + 8 * g));
        }
    }
    asm volatile("" ::: "memory");
    // Contiguous cache: the sequence's rows start at seq * n_cap. Paged cache
    // (block_table != NULL): the layer's cache is a pool of page_size-row pages
    // and position s of the sequence is row table[seq][s / page_size] *
    // page_size + s % page_size of the pool; indices become pool rows here, once.
    constexpr int RB = FP8KV ? kRowBytesF8 : kRowBytes;   // bytes per cache row
    const uint8_t* kvs;
    // (all of a thread's index loads, and then its block-table loads, are in
    // flight together: a loop that stores each to LDS before the next load
    // waits out one memory latency per row batch)
    constexpr int kIdxPer = kMaxRows / kThreads;          // rows per thread at most
    int32_t iv[kIdxPer];
#pragma unroll
    for (int u = 0; u < kIdxPer; ++u) {
        const int i = tid + u * kThreads;
        iv[u] = i < nrows ? idx[(int64_t)q * k + r0 + i] : -1;
    }
    // positions outside [0, n_cap) (with a paged cache, outside the sequence's
    // pages) are skipped as -1 is: one unsigned compare, so no index from a stale
    // or foreign buffer makes the gather leave the sequence's rows
#pragma unroll
    for (int u = 0; u < kIdxPer; ++u) iv[u] = (uint32_t)iv[u] < (uint32_t)n_cap ? iv[u] : -1;
    if (block_table == nullptr) {
        kvs = kv + (int64_t)seq * n_cap * RB;
    } else {
        kvs = kv;
        const int32_t* bt = block_table + (int64_t)seq * max_pages;
        int32_t pg[kIdxPer];
#pragma unroll
        for (int u = 0; u < kIdxPer; ++u) pg[u] = iv[u] < 0 ? 0 : bt[iv[u] / page_size];
#pragma unroll
        for (int u = 0; u < kIdxPer; ++u) iv[u] = iv[u] < 0 ? -1 : pg[u] * page_size + iv[u] % page_size;
    }
#pragma unroll
    for (int u = 0; u < kIdxPer; ++u)
        if (tid + u * kThreads < nrows) rows_s[tid + u * kThreads] = iv[u];

    if (lane == 0) g_xflag[wave] = 0;
    wait_vmcnt<0>();     // Q and the indices are in before any ring load is counted
    __syncthreads();

    // bf16: 16-byte LDS position s = 64*i + lane of a block holds row s / 73,
    // chunk s % 73 (chunk 72 and positions past row 31 are padding, filled from
    // the zero row). FP8: row s / 41, chunk s % 41 of the staging slot, unpadded.
    constexpr int DMA_BIG = FP8KV ? kDmaBigF8 : kDmaBig;
    constexpr int DMA_HI = FP8KV ? kDmaHiF8 : kDmaHi;
    constexpr int DMA_LO = FP8KV ? kDmaLoF8 : kDmaLo;
    constexpr int UNIT = FP8KV ? kPitchF8 / 16 : kChunksPerPitch;    // 16-byte units per LDS row
    constexpr int ROW_CHUNKS = FP8KV ? kChunksF8 : kChunksPerRow;
    constexpr int SLOT = FP8KV ? kStageBuf : kBuf;
    uint8_t* const ring = FP8KV ? g_stage : g_ring;
    const bool big = wave < DMA_BIG;
    const int i0 = big ? DMA_HI * wave : DMA_HI * DMA_BIG + DMA_LO * (wave - DMA_BIG);
    auto issue = [&](int b, int slot) __attribute__((always_inline)) {
        const uint32_t dst = (uint32_t)(uintptr_t)(lds_u8*)ring + slot * SLOT;
        const int nload = big ? DMA_HI : DMA_LO;
        int srow[DMA_HI];
#pragma unroll
        for (int j = 0; j < DMA_HI; ++j) {              // every index read first, one wait
            const int pos = 64 * (i0 + j) + lane;
            const int row = pos / UNIT;
            const int c = pos - row * UNIT;
            srow[j] = (j < nload && row < kBlk && c < ROW_CHUNKS) ? rows_s[b * kBlk + row] : -1;
        }
#pragma unroll
        for (int j = 0; j < DMA_HI; ++j) {
            if (j == DMA_HI - 1 && !big) break;
            const int pos = 64 * (i0 + j) + lane;
            const int row = pos / UNIT;
            const int c = pos - row * UNIT;
            const uint8_t* src = srow[j] >= 0 ? kvs + (int64_t)srow[j] * RB + 16 * c : g_zero_row;
            lds_dma16(src, dst + 1024 * (i0 + j));
        }
    };
    // FP8, dim-pair layout: widen staging slot `slot` into g_blk in the bf16 row
    // layout, for the bf16 compute. Thread t
    // converts codes 32*(t%16) .. +31 of row t/16 with that group's scale (the
    // scaled conversion is exact for a power-of-two scale); threads 0-255 move
    // the RoPE dims (16 bytes each).
    auto widen = [&](int slot) __attribute__((always_inline)) {
        const lds_u8* st = (const lds_u8*)g_stage + slot * kStageBuf;
        const int r = tid >> 4, j = tid & 15;
        const lds_u8* sr = st + r * kPitchF8;
        const i32x4 c0 = *(const __attribute__((address_space(3))) i32x4*)(sr + 32 * j);
        const i32x4 c1 = *(const __attribute__((address_space(3))) i32x4*)(sr + 32 * j + 16);
        const float sc = *(const __attribute__((address_space(3))) float*)(sr + 512 + 4 * (j >> 2));
        i32x4 w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const auto lo0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)c0[e], sc, false);
            const auto hi0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)c0[e], sc, true);
            const auto lo1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)c1[e], sc, false);
            const auto hi1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((uint32_t)c1[e], sc, true);
            w[e >> 1][2 * (e & 1)] = __builtin_bit_cast(int, lo0);
            w[e >> 1][2 * (e & 1) + 1] = __builtin_bit_cast(int, hi0);
            w[2 + (e >> 1)][2 * (e & 1)] = __builtin_bit_cast(int, lo1);
            w[2 + (e >> 1)][2 * (e & 1) + 1] = __builtin_bit_cast(int, hi1);
        }
        lds_u8* dr = (lds_u8*)g_blk + r * kPitch + 64 * j;
#pragma unroll
        for (int e = 0; e < 4; ++e) *(__attribute__((address_space(3))) i32x4*)(dr + 16 * e) = w[e];
        if (tid < 256) {
            const int r2 = tid >> 3, c = tid & 7;
            *(__attribute__((address_space(3))) i32x4*)((lds_u8*)g_blk + r2 * kPitch + 1024 + 16 * c) =
                *(const __attribute__((address_space(3))) i32x4*)(st + r2 * kPitchF8 + 528 + 16 * c);
        }
    };

    f32x4 o[16];
#pragma unroll
    for (int d = 0; d < 16; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = neg_inf();      // running max (log2 units) of head `head`
    float l_part = 0.f;           // this lane's share of the running sum

    const int nblk = nrows / kBlk;
    // FP8 rows read in place (row-pair layout); the dim-pair layout widens them first
    constexpr bool F8IN = FP8KV && RP;
    // The A operand of K-step t for the row at `rp` (this lane's dims 32t + 8g ..
    // +7): bf16 rows are read as they are; FP8 rows hold 8 codes there (steps of
    // the latent dims, converted with the row's group scale by kval) or, past the
    // latent, the bf16 RoPE key.
    auto kraw = [&](const lds_u8* rp, int t) __attribute__((always_inline)) -> i32x4 {
        if constexpr (F8IN) {
            if (t < 16) {
                const v2i c = *(const lds_v2i*)(rp + 32 * t + 8 * g);
                return i32x4{c[0], c[1], 0, 0};
            }
            return *(const __attribute__((address_space(3))) i32x4*)(rp + 528 + 64 * (t - 16) + 16 * g);
        } else {
            return *(const __attribute__((address_space(3))) i32x4*)(rp + 64 * t);
        }
    };
    auto kval = [&](const i32x4& raw, int t, const f32x4& srow) __attribute__((always_inline)) -> bf16x8 {
        if constexpr (F8IN) {
            if (t < 16) return fp8x8_to_bf16(v2i{raw[0], raw[1]}, srow[t >> 2]);
        }
        return __builtin_bit_cast(bf16x8, raw);
    };
    auto compute = [&](int b, const lds_u8* buf) __attribute__((always_inline)) {
        // rows of this block with a valid index (bit r), one LDS read per lane
        const uint64_t valid = __builtin_amdgcn_ballot_w64(rows_s[b * kBlk + (lane & 31)] >= 0);
        bf16x8 pa;
        // row-pair layout, bf16 rows: P.V's first kVPre V fragments, read between
        // Q.K and the softmax so that they load while the softmax and the swap run
        constexpr int kVPre = 8;
        bf16x8 vpre[kVPre];
        const lds_u8* const vb = buf + (4 * g + (l16 >> 2)) * kPitch + 8 * (l16 & 3) + 512 * hf;
        auto vfrag = [&](int d) __attribute__((always_inline)) {
            // two 16-bit transpose reads in which lane j of the group supplies row
            // 4g + j/4 (+16), dims 16d + 4(j%4) .. +3
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vb + 32 * d));
            const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vb + 16 * kPitch + 32 * d));
            return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        };
        if constexpr (RP) {
            // S^T of this wave's 16 rows (16hf + 4g + i) and head l16 over all 576 dims,
            // as two accumulation chains (K-steps 0-8 and 9-17) added at the end
            f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
            const lds_u8* arow = F8IN ? buf + (16 * hf + l16) * kPitchF8
                                       : buf + (16 * hf + l16) * kPitch + 16 * g;
            // FP8 rows: the row's four group scales, for the conversion of its codes
            f32x4 srw{};
            if constexpr (F8IN) srw = *(const __attribute__((address_space(3))) f32x4*)(arow + 512);
            // fragment e: chain e & 1, its K-step e >> 1; the first 8 are read before
            // any MFMA and each later one 8 MFMAs ahead of its use
            i32x4 af[18];
            auto frag = [&](int e) __attribute__((always_inline)) {
                const int t = 9 * (e & 1) + (e >> 1);
                af[e] = kraw(arow, t);
            };
#pragma unroll
            for (int e = 0; e < 8; ++e) frag(e);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int e = 0; e < 18; ++e) {
                if (e + 8 < 18) frag(e + 8);
                const int t = 9 * (e & 1) + (e >> 1);
                sacc[e & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kval(af[e], t, srw), qr[t], sacc[e & 1], 0, 0, 0);
            }
            if constexpr (!F8IN) {
#pragma unroll
                for (int d = 0; d < kVPre; ++d) vpre[d] = vfrag(d);
                __builtin_amdgcn_sched_barrier(0);
            }
            const f32x4 sc = sacc[0] + sacc[1];
            // this wave's rows: scores, the block max of the head, the max this wave
            // proposes (moved only past the lazy-rescale margin) and P against it
            float z[4], p[4];
            float mb = neg_inf();
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * hf + 4 * g + i;
                const bool ok = (valid >> r) & 1u;
                z[i] = ok ? sc[i] * scale_log2 : neg_inf();
                mb = fmaxf(mb, z[i]);
            }
            mb = max_x32(max_x16(mb));
            const float mo = mb > m_run + kRescale ? mb : m_run;
            {
                const float mu = mo == neg_inf() ? 0.f : mo;
#pragma unroll
                for (int i = 0; i < 4; ++i) p[i] = exp2_(z[i] - mu);
            }
            // hand the partner (same heads, other 16 rows) this wave's P and proposal
            // (flag f1; a second post in the rare case below sets f1 + 1). The
            // barrier of the next block keeps a wave from overwriting its post before
            // the partner has read it; the polls are bounded, so a post that never
            // came would leave wrong results, never a hang.
            const int f1 = 2 * (b + 1);
            g_xp[wave][lane] = bf16x4{(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3]};
            if (g == 0) g_xm[wave][l16] = mo;
            __hip_atomic_store(&g_xflag[wave], f1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            // the gathers of block b + kRing - 1 into the slot the barrier freed, issued
            // here so that their issue (which stalls while the memory system drains
            // earlier requests) overlaps the partner's post
            if (b + kRing - 1 < nblk) issue(b + kRing - 1, (b + kRing - 1) % kRing);
            for (int spin = 0; spin < (1 << 22); ++spin) {
                const int f = __builtin_amdgcn_readfirstlane(
                    __hip_atomic_load(&g_xflag[wave ^ 4], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
                if (f >= f1) break;
                __builtin_amdgcn_s_sleep(1);
            }
            bf16x4 px = g_xp[wave ^ 4][lane];
            const float mx = g_xm[wave ^ 4][l16];
            // the pair's max is the larger proposal (both waves see the same two, so
            // both take the branch below or neither). Where it moved (rare): O and
            // the sums are rescaled, and both waves compute P against it again and
            // swap once more, so that P is rounded once, as in the dim-pair layout.
            const float mf = fmaxf(mo, mx);
            if (__builtin_amdgcn_ballot_w64(mf != m_run) != 0) {     // wave-uniform branch, rare
                const float alpha = mf != m_run ? exp2_(m_run - mf) : 1.f;   // exp2(-inf) = 0
                l_part *= alpha;
                m_run = mf;
                float al[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g + i, 64);
#pragma unroll
                for (int d = 0; d < 16; ++d)
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[d][i] *= al[i];
                const float mu = mf == neg_inf() ? 0.f : mf;
#pragma unroll
                for (int i = 0; i < 4; ++i) p[i] = exp2_(z[i] - mu);
                // (the partner discards what it read of the first post)
                g_xp[wave][lane] = bf16x4{(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3]};
                __hip_atomic_store(&g_xflag[wave], f1 + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
                for (int spin = 0; spin < (1 << 22); ++spin) {
                    const int f = __builtin_amdgcn_readfirstlane(
                        __hip_atomic_load(&g_xflag[wave ^ 4], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
                    if (f == f1 + 1) break;
                    __builtin_amdgcn_s_sleep(1);
                }
                px = g_xp[wave ^ 4][lane];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) l_part += p[i];
            // P as the A operand: K index e < 4 is row 4g + e (rows 0-15), e >= 4 row
            // 16 + 4g + e - 4 (rows 16-31)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const __bf16 own = (__bf16)p[i];
                pa[i] = hf == 0 ? own : px[i];
                pa[4 + i] = hf == 0 ? px[i] : own;
            }
        } else {
            // partial S^T over this wave's 9 K-steps: rows 16tt + 4g + i, head l16
            f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
            const lds_u8* arow = buf + l16 * kPitch + 16 * g;
            // fragment e = 2j + tt (K-step j, rows 16tt..): the first 8 are read before
            // any MFMA and each later one 8 MFMAs ahead of its use; the scheduling
            // fence keeps the compiler from pulling those reads back next to their
            // MFMAs, which left the LDS latency exposed every second MFMA
            i32x4 af[18];
            auto frag = [&](int e) __attribute__((always_inline)) {
                af[e] = kraw(arow + 16 * (e & 1) * kPitch, 9 * hf + (e >> 1));
            };
#pragma unroll
            for (int e = 0; e < 8; ++e) frag(e);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int e = 0; e < 18; ++e) {
                if (e + 8 < 18) frag(e + 8);
                sacc[e & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kval(af[e], 9 * hf + (e >> 1), f32x4{}), qr[e >> 1],
                                                                      sacc[e & 1], 0, 0, 0);
            }
            // swap partial scores with the partner wave (same heads, other half)
            // (a flag per wave instead of a work-group barrier: only the two waves of
            // a head group wait for each other; the barrier of the next block keeps
            // a wave from overwriting its scores before the partner has read them)
            g_xs[wave][0][lane] = sacc[0];
            g_xs[wave][1][lane] = sacc[1];
            __hip_atomic_store(&g_xflag[wave], b + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            // the gathers of block b + kRing - 1 into the slot the barrier freed, issued
            // here so that their issue (which stalls while the memory system drains
            // earlier requests) overlaps the partner's post rather than delaying Q.K
            if (b + kRing - 1 < nblk) issue(b + kRing - 1, (b + kRing - 1) % kRing);
            // bounded: a post that never came would leave wrong scores, never a hang
            for (int spin = 0; spin < (1 << 22); ++spin) {
                const int f = __builtin_amdgcn_readfirstlane(
                    __hip_atomic_load(&g_xflag[wave ^ 4], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
                if (f == b + 1) break;
                __builtin_amdgcn_s_sleep(1);
            }
            sacc[0] += g_xs[wave ^ 4][0][lane];
            sacc[1] += g_xs[wave ^ 4][1][lane];
            float z[8];
            float mb = neg_inf();
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * tt + 4 * g + i;
                    const bool ok = (valid >> r) & 1u;
                    const float v = ok ? sacc[tt][i] * scale_log2 : neg_inf();
                    z[tt * 4 + i] = v;
                    mb = fmaxf(mb, v);
                }
            mb = max_x16(mb);
            mb = max_x32(mb);
            const bool move = mb > m_run + kRescale;
            if (__builtin_amdgcn_ballot_w64(move) != 0) {   // wave-uniform branch, rare
                const float m_new = move ? mb : m_run;
                const float alpha = move ? exp2_(m_run - m_new) : 1.f;   // exp2(-inf) = 0
                l_part *= alpha;
                m_run = m_new;
                float al[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g + i, 64);
#pragma unroll
                for (int d = 0; d < 16; ++d)
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[d][i] *= al[i];
            }
            const float m_use = m_run == neg_inf() ? 0.f : m_run;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float p = exp2_(z[e] - m_use);
                l_part += p;
                pa[e] = (__bf16)p;
            }
        }
        // P.V over this wave's 256 latent dims: O[heads][16 dims] += P[heads][32 rows] *
        // V[32 rows][16 dims]. The V operand of lane (dim l16, group g) is rows
        // {4g..4g+3, 16+4g..16+4g+3} (K index e of P is row R(e): 4g + e, then
        // 16 + 4g + e - 4).
        if constexpr (!F8IN) {
#pragma unroll
            for (int d = 0; d < 16; ++d) {
                const bf16x8 bv = RP && d < kVPre ? vpre[d < kVPre ? d : 0] : vfrag(d);
                o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, bv, o[d], 0, 0, 0);
            }
        } else {
            // one 8-bit transpose read: lane j of the group supplies row R(j/2), codes
            // of dims 16d + 8(j%2) .. +7, and gets back the 8 codes of dim 16d + j,
            // byte e from row R(e); they convert unscaled. The rows' group scales
            // multiply P instead (a power of two: exact, and P.V's products are those
            // of the dequantised rows): pa for the half's first 128 dims, pb for the
            // second.
            const int k = l16 >> 1;
            const int rsrc = k < 4 ? 4 * g + k : 12 + 4 * g + k;
            const lds_u8* vb8 = buf + rsrc * kPitchF8 + 256 * hf + 8 * (l16 & 1);
            bf16x8 pb;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int r = e < 4 ? 4 * g + e : 12 + 4 * g + e;
                const f32x2 sc = *(const __attribute__((address_space(3))) f32x2*)(buf + r * kPitchF8 + 512 + 8 * hf);
                const float pv = (float)pa[e];
                pb[e] = (__bf16)(pv * sc[1]);
                pa[e] = (__bf16)(pv * sc[0]);
            }
#pragma unroll
            for (int d = 0; d < 16; ++d) {
                const v2i c = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(vb8 + 16 * d));
                o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(d < 8 ? pa : pb, fp8x8_to_bf16(c, 1.0f), o[d], 0, 0, 0);
            }
        }
    };

#pragma unroll
    for (int p = 0; p < kRing - 1; ++p)
        if (p < nblk) issue(p, p);
    for (int b = 0; b < nblk; ++b) {
        // this wave's loads of block b are done once at most the later issued
        // blocks (b+1 .. min(nblk, b+kRing-1) - 1) remain outstanding
        const int later = min(nblk, b + kRing - 1) - b - 1;
        if (big) wait_block<DMA_HI>(later);
        else wait_block<DMA_LO>(later);
        ring_barrier();    // every wave's part of block b is in; block b-1's readers are done
        if constexpr (FP8KV && !RP) {
            widen(b % kRing);
            wait_lgkm0();
            ring_barrier();    // the widened block is complete
            compute(b, (const lds_u8*)g_blk);
        } else {
            compute(b, (const lds_u8*)ring + (b % kRing) * SLOT);
        }
    }

    // the head's sum over the slice (row-pair layout: this wave's rows plus the
    // partner's, added in row-half order so that both hold the same value)
    float l_tot = sum_x32(sum_x16(l_part));
    if constexpr (RP) {
        if (g == 0) g_xl[wave][l16] = l_tot;
        __syncthreads();
        const float lx = g_xl[wave ^ 4][l16];
        l_tot = hf == 0 ? l_tot + lx : lx + l_tot;
    }
    const int dim0 = 256 * hf;
    if (n_split == 1) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        float iv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) iv[i] = __shfl(inv, 4 * g + i, 64);
        float* oq = out + (int64_t)q * kHeads * kLat;
#pragma unroll
        for (int d = 0; d < 16; ++d)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                oq[(16 * hg + 4 * g + i) * kLat + dim0 + 16 * d + l16] = o[d][i] * iv[i];
        if (lse != nullptr && g == 0 && hf == 0)
            lse[(int64_t)q * kHeads + head] =
                l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : neg_inf();
    } else {
        // the split's unnormalised O in fp16 with a power-of-two scale per (head,
        // latent half): 2^-e puts the largest |O| of the half in [2^14, 2^15), so
        // every value keeps 11 significant bits relative to that largest one
        // whatever the cache's magnitudes (half the bytes of fp32 partials,
        // written here and read by the merge)
        int ex[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float mx = 0.f;
#pragma unroll
            for (int d = 0; d < 16; ++d) mx = fmaxf(mx, fabsf(o[d][i]));
            mx = max_row16(mx);                          // the 16 lanes of the row hold the half's dims
            ex[i] = __builtin_amdgcn_frexp_expf(mx) - 15;
        }
        _Float16* po = part_o + ((int64_t)q * n_split + split) * kHeads * kLat;
#pragma unroll
        for (int d = 0; d < 16; ++d)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                po[(16 * hg + 4 * g + i) * kLat + dim0 + 16 * d + l16] = (_Float16)__builtin_amdgcn_ldexpf(o[d][i], -ex[i]);
        float* pm = part_ml + ((int64_t)q * n_split + split) * kHeads * 4;
        if (l16 == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) pm[4 * (16 * hg + 4 * g + i) + 2 + hf] = (float)ex[i];
        }
        if (g == 0 && hf == 0) {
            pm[4 * head] = m_run;
            pm[4 * head + 1] = l_tot;
        }
    }
}

// Combine the per-split partial results with their log-sum-exp. Grid
// (n_q, 16): a work-group merges 4 heads x 512 dims of one query.
template <int SB>
__global__ __launch_bounds__(256) void sparse_mla_merge(LayerArgs L, int n_q,
                                                             const _Float16* __restrict__ part_o_all,
                                                             const float* __restrict__ part_ml_all,
                                                             int n_split) {
    const int layer = blockIdx.z;
    float* __restrict__ out = L.out[layer];
    float* __restrict__ lse = L.lse[layer];
    const _Float16* __restrict__ part_o = part_o_all + (size_t)layer * n_q * n_split * kHeads * kLat;
    const float* __restrict__ part_ml = part_ml_all + (size_t)layer * n_q * n_split * kHeads * 4;
    const int q = blockIdx.x;
    const int h = 4 * blockIdx.y + (threadIdx.x >> 6);
    const int c = threadIdx.x & 63;              // dims 4c .. 4c + 3 of each latent half
    const float* pm = part_ml + ((int64_t)q * n_split * kHeads + h) * 4;
    // Splits in batches of SB (8, or 16 when there are 16 or more) whose loads
    // are all in flight together (a loop that uses each load before issuing the
    // next waits out one memory latency per split); sums in split order.
    float mx = neg_inf();
    for (int s0 = 0; s0 < n_split; s0 += SB) {
        float m[SB];
#pragma unroll
        for (int b = 0; b < SB; ++b) m[b] = s0 + b < n_split ? pm[(int64_t)(s0 + b) * kHeads * 4] : neg_inf();
#pragma unroll
        for (int b = 0; b < SB; ++b) mx = fmaxf(mx, m[b]);
    }
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
    float lsum = 0.f;
    if (mx != neg_inf()) {
        for (int s0 = 0; s0 < n_split; s0 += SB) {
            f32x4 ml[SB];                                      // m, l, exponents of the two halves
            f16x4 x0[SB], x1[SB];
#pragma unroll
            for (int b = 0; b < SB; ++b) {
                const int s = min(s0 + b, n_split - 1);          // past the last split: not summed
                ml[b] = *(const f32x4*)(pm + (int64_t)s * kHeads * 4);
                const f16x4* po = (const f16x4*)(part_o + (((int64_t)q * n_split + s) * kHeads + h) * kLat);
                x0[b] = po[c];
                x1[b] = po[c + 64];
            }
#pragma unroll
            for (int b = 0; b < SB; ++b) {                    // branch-free, so the loads stay batched
                const bool ok = s0 + b < n_split;
                const float wgt = exp2_(ml[b][0] - mx);
                const float w0 = __builtin_amdgcn_ldexpf(wgt, (int)ml[b][2]);
                const float w1 = __builtin_amdgcn_ldexpf(wgt, (int)ml[b][3]);
                const f32x4 y0 = {(float)x0[b][0], (float)x0[b][1], (float)x0[b][2], (float)x0[b][3]};
                const f32x4 y1 = {(float)x1[b][0], (float)x1[b][1], (float)x1[b][2], (float)x1[b][3]};
                lsum = ok ? lsum + wgt * ml[b][1] : lsum;
                a0 = ok ? a0 + w0 * y0 : a0;
                a1 = ok ? a1 + w1 * y1 : a1;
            }
        }
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    f32x4* oo = (f32x4*)(out + ((int64_t)q * kHeads + h) * kLat);
    oo[c] = a0 * inv;
    oo[c + 64] = a1 * inv;
    if (lse != nullptr && c == 0)
        lse[(int64_t)q * kHeads + h] = lsum > 0.f ? (mx + log2f(lsum)) * 0.69314718055994531f : neg_inf();
}

// Splits per (layer, query) so that about 256 work-groups run.
int choose_split(int units, int k) {
    int s = 1;
    while (s < 32 && units * s < 256 && (k / (2 * s)) % kBlk == 0 && k / (2 * s) >= kBlk) s *= 2;
    return s;
}

}  // namespace

size_t mla_workspace_bytes(int n_q, int n_heads, int k, int n_layers) {
    (void)n_heads;
    if (n_layers < 1) return 0;
    const int per = n_layers < kMaxLayersPerLaunch ? n_layers : kMaxLayersPerLaunch;
    const int s = choose_split(n_q * per, k);
    if (s == 1) return 0;
    return (size_t)per * n_q * s * kHeads * (kLat * sizeof(_Float16) + 4 * sizeof(float));
}

hipError_t launch_sparse_mla_layers(const MlaLayerPtrs* layers, int n_layers, const int32_t* q_seq,
                                    const int32_t* idx, int k, int n_q, int n_heads, int64_t n_cap,
                                    const int32_t* block_table, int page_size, int max_pages,
                                    bool fp8_kv, float scale, void* ws, hipStream_t st) {
    (void)n_heads;
    const float scale_log2 = scale * 1.4426950408889634f;
    for (int l0 = 0; l0 < n_layers; l0 += kMaxLayersPerLaunch) {
        const int nl = n_layers - l0 < kMaxLayersPerLaunch ? n_layers - l0 : kMaxLayersPerLaunch;
        LayerArgs L{};
        for (int i = 0; i < nl; ++i) {
            L.q_lat[i] = (const uint8_t*)layers[l0 + i].q_lat;
            L.q_rope[i] = (const uint8_t*)layers[l0 + i].q_rope;
            L.kv[i] = (const uint8_t*)layers[l0 + i].kv;
            L.out[i] = layers[l0 + i].out;
            L.lse[i] = layers[l0 + i].lse;
        }
        // the split is chosen for a full launch, so every launch fits the workspace
        const int per = n_layers < kMaxLayersPerLaunch ? n_layers : kMaxLayersPerLaunch;
        const int s = choose_split(n_q * per, k);
        const int rows = k / s;
        _Float16* part_o = (_Float16*)ws;
        float* part_ml = s > 1 ? (float*)(part_o + (size_t)per * n_q * s * kHeads * kLat) : nullptr;
        // slices of at least kRowPairRows rows take the row-pair layout; shorter ones
        // the dim-pair layout, whose work-groups load half as many Q bytes
        const bool rp = rows >= kRowPairRows;
        auto* kern = fp8_kv ? (rp ? sparse_mla_kernel<true, true> : sparse_mla_kernel<true, false>)
                            : (rp ? sparse_mla_kernel<false, true> : sparse_mla_kernel<false, false>);
        hipLaunchKernelGGL(kern, dim3(s, n_q, nl), dim3(kThreads), 0, st, L, q_seq, idx, k, n_q, n_cap,
                           block_table, page_size, max_pages, scale_log2, rows, part_o, part_ml);
        if (s > 1)
            hipLaunchKernelGGL(s >= 16 ? sparse_mla_merge<16> : sparse_mla_merge<8>, dim3(n_q, kHeads / 4, nl),
                               dim3(256), 0, st, L, n_q,
                               part_o, part_ml, s);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gsa

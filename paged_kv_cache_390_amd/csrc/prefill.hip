// Paged prefill / chunked prefill on the CDNA4 matrix cores (gfx950).
//
// What is computed: sequence s has n cached tokens, the last m of which are
// new (their K/V already written into the blocks by pa_reshape_and_cache);
// new token i sits at position n - m + i and attends causally to positions
// 0 .. n - m + i of its sequence, read through the block table.  This is the
// prompt path of a request (lpnh.cn/news/1824136, 3.2 second step) on a
// paged cache -- which a contiguous-memory attention kernel cannot read
// (explore.n1n.ai, section on trade-offs) -- with the same textbook softmax
// attention as decode; m = 1 is decode.
//
// Design.  Unlike decode, prefill is a dense contraction with reuse: every
// K/V tile meets every later query of its sequence, so the products run on
// the matrix cores (v_mfma_f32_16x16x32_f16, fp32 accumulation).
//  * Query rows: the m new tokens x g query heads of one KV head, token
//    major (row r = token r / g, head r % g).  A wave owns 32 rows as two
//    groups of 16 -- the N side of its MFMA tiles -- so that every K or V
//    operand read from LDS feeds two products.  A 256-thread workgroup is 4
//    such waves (128 rows) of one (KV head, sequence); 2 workgroups share a
//    CU.  The grid is one-dimensional and XCD-grouped: all row tiles of a
//    (KV head, sequence) pair run together on one XCD, last row tile first
//    (the longest causal range starts earliest), so that the K/V tiles they
//    all walk are read from HBM once and then served by that XCD's L2.
//  * K/V tiles of 64 tokens are staged through LDS once per workgroup and
//    read by all 4 waves.  The loads go from HBM straight into LDS
//    (global_load_lds_dwordx4: a wave instruction writes 1 KiB, 4 token rows
//    of 256 bytes, 16 bytes per lane), one tile ahead, into the other of two
//    buffers (32 KiB each) -- no registers hold a tile in flight and no LDS
//    store instructions run.  Each thread issues 8 such loads per tile (4
//    rows of K, 4 of V), waited for explicitly before the step's barrier;
//    one barrier per tile.  A wave's 4 rows of one load share a table entry
//    (blocks of 4 or more tokens), read a tile ahead with a scalar load, so
//    that (outside append mode) such a load is addressed as a scalar base
//    (block, first row) plus a per-lane offset that is the same for every
//    tile: no vector instruction computes a load address.  The DMA writes
//    lane i's 16 bytes at byte 16i, so
//    bank conflicts are avoided by choosing what each lane loads: position
//    p of K row r holds the row's 16-byte chunk p ^ (r & 15), of V row r
//    chunk p ^ 2(r & 3).  Rows past the context or with an id outside the
//    pool are zeroed in LDS by the thread that loaded them, after its loads
//    landed and before the barrier.
//  * QK as S^T = K Q^T: MFMA c takes head_dim 32c + 8*(l/16) + 0..7 in lane
//    l, one 16-byte LDS read of K per two MFMAs; Q^T operands stay in
//    registers.  S^T lands with each lane holding 8 scores of one row
//    (tokens 4j..4j+3 and 16+4j..16+4j+3 of the tile) -- exactly that lane's
//    A operand of P for a 32-token PV product, so the online softmax (base
//    2) runs in place and P goes to the matrix core as fp16.  The row max
//    crosses the 4 lanes of a row with v_permlane32_swap /
//    v_permlane16_swap; the row sum is one more product per 32-token slab,
//    an all-ones operand times P, so it adds exactly the rounded weights
//    the value products see, and no vector instruction sums them.  Tiles
//    wholly before a wave's first row and wholly valid skip the masks;
//    tiles with every token valid take the causal mask only (a compare and
//    a select per score); the running maximum moves lazily (only when a
//    tile's exceeds it by a factor above 2^8), so O is rarely rescaled, and
//    the rescale factor is computed only then.
//  * PV as O^T = V^T P^T: the V operand (8 tokens of one V column per lane)
//    comes straight from the row-major V tile through two LDS transpose
//    reads (ds_read_b64_tr_b16) per d-tile, P is the other operand as the
//    softmax left it, and a lane's O holds 4 consecutive columns of its own
//    row per d-tile: the rescale takes the lane's own factor, and the
//    output goes out in 8-byte stores.
//  * Each wave walks the tiles up to its own last row's position and writes
//    its rows itself, normalised by the row sums it holds for them.
#include <hip/hip_runtime.h>

#include <cmath>
#include <map>
#include <mutex>
#include <utility>
#include <cstdint>

#include "pa.h"
#include "pa_internal.h"

namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr double kLog2e = 1.4426950408889634073599246810019;

// Geometry per head_dim D (64, 128 or 256).
//  * A K/V tile in LDS: kKvTile token rows of K and of V, 2D bytes each with
//    their 16-byte chunks permuted per row (see fetch_tile), plus a flag per
//    token (inside the context and the pool) in an array of its own; two such
//    buffers per workgroup (32 KiB each at D <= 128 with 64-token tiles; at
//    D = 256, 32-token tiles keep a buffer at 32 KiB).
//  * kNT 16-row groups per wave -- the N side of its MFMA tiles, each K or V
//    operand read from LDS feeding kNT products; one at D = 256, whose O
//    and Q^T alone would fill the registers of two.
//  * One thread's share of a K/V tile in flight: kStageRows token rows whose
//    16 bytes at LDS position l % kChunks it loads.  Thread (wave w, lane l)
//    stages rows kRowsPerLoad*w + l/kChunks + 4*kRowsPerLoad*i, i <
//    kStageRows: a wave's rows for one i are kRowsPerLoad consecutive
//    tokens starting at a multiple of kRowsPerLoad, so with blocks of at
//    least kRowsPerLoad tokens they share one table entry, read with a
//    scalar load.
template <int D>
struct PGeo {
    static constexpr int kChunks = D / 8;                      // 16-byte chunks per row
    static constexpr int kKvTile = D >= 256 ? 32 : 64;         // tokens per LDS tile
    static constexpr int kNT = D >= 256 ? 1 : 2;
    static constexpr int kRowsPerWave = 16 * kNT;
    static constexpr int kRowsPerGroup = kWaves * kRowsPerWave;
    static constexpr int kPitch = D * 2;                       // K rows (chunks XOR-swizzled by row & kSwzK)
    static constexpr int kPitchV = D * 2;                      // V rows (chunks swizzled by 2 * (row & 3))
    static constexpr int kTileBytes = kKvTile * kPitch;
    static constexpr int kTileBytesV = kKvTile * kPitchV;
    static constexpr int kBufBytes = kTileBytes + kTileBytesV;
    static constexpr int kRowsPerLoad = 64 / kChunks;          // rows one wave load stages
    static constexpr int kStageRows = kKvTile * kChunks / kThreads;
    static constexpr int kSwzK = kChunks < 16 ? kChunks - 1 : 15;
    static constexpr int kQk = D / 32;                         // QK MFMAs (k = 32) per 16 tokens
    static constexpr int kDTiles = D / 16;                     // PV d-tiles (16 output columns each)
    static_assert(kStageRows >= 1 && kKvTile * kChunks == kStageRows * kThreads, "tile rows must split evenly");
    static_assert(kKvTile % 32 == 0 && kDTiles % 4 == 0, "whole PV slabs and d-tile groups");
    static_assert(kWaves * kRowsPerWave * D * 2 <= kBufBytes, "the output rows of all waves fit one buffer");
};

// The geometry of PGeo<D> under short names inside a kernel or helper.
#define PF_GEO(D)                                                   \
    using PG_ = PGeo<D>;                                            \
    constexpr int kD = D;                                           \
    constexpr int kChunks = PG_::kChunks;                           \
    constexpr int kKvTile = PG_::kKvTile;                           \
    constexpr int kNT = PG_::kNT;                                   \
    constexpr int kRowsPerWave = PG_::kRowsPerWave;                 \
    constexpr int kRowsPerGroup = PG_::kRowsPerGroup;               \
    constexpr int kPitch = PG_::kPitch;                             \
    constexpr int kPitchV = PG_::kPitchV;                           \
    constexpr int kTileBytes = PG_::kTileBytes;                     \
    constexpr int kBufBytes = PG_::kBufBytes;                       \
    constexpr int kRowsPerLoad = PG_::kRowsPerLoad;                 \
    constexpr int kStageRows = PG_::kStageRows;                     \
    constexpr int kSwzK = PG_::kSwzK;                               \
    constexpr int kQk = PG_::kQk;                                   \
    constexpr int kDTiles = PG_::kDTiles;                           \
    (void)kD; (void)kChunks; (void)kKvTile; (void)kNT; (void)kRowsPerWave; (void)kRowsPerGroup; (void)kPitch; \
    (void)kPitchV; (void)kTileBytes; (void)kBufBytes; (void)kRowsPerLoad; (void)kStageRows; (void)kSwzK; \
    (void)kQk; (void)kDTiles

typedef _Float16 half8_t_ __attribute__((ext_vector_type(8)));

// The online-softmax state of a lane for one 16-row group: the running max
// and sum of its row and its share of the unnormalised output rows.
template <int D>
struct Softmax {
    float m;                               // running max (base 2) of row l % 16
    float4_t l;                            // running sum of row l % 16 (in every element)
    float4_t o[D / 16];                    // O[row l % 16][d = 16c + 4*(l/16) + i] in o[c][i]
};

template <int D>
struct Staged {
    bool ok[PGeo<D>::kStageRows];
    int32_t wphys[PGeo<D>::kStageRows];   // append mode: the block this thread writes the row into, or -1
};

// Append mode: the m new tokens of the sequence (positions base_pos ..
// n - 1) are read from the step's key / value tensors, not from the cache,
// and the workgroup holding a token's first query row writes it into the
// cache.  `k` / `v` point at the sequence's first new token, KV head kvh.
struct AppendSrc {
    const _Float16* k;
    const _Float16* v;
    int64_t stride;      // elements between consecutive tokens
    int base_pos;        // position of the first new token
    int w_lo, w_hi;      // positions this workgroup writes: [w_lo, w_hi)
};

// s_waitcnt immediates (GFX9 encoding: vmcnt bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8): wait until at most N vector memory operations are
// outstanding; wait for every LDS / scalar memory operation.
#define PA_WAIT_VM(N) __builtin_amdgcn_s_waitcnt(((N) & 15) | (((N) >> 4) << 14) | (7 << 4) | (15 << 8))
#define PA_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8))

// First token of the wave's stage row i of tile k.
template <int D>
__device__ __forceinline__ int stage_token0(int k, int wave, int i) {
    constexpr int R = PGeo<D>::kRowsPerLoad;
    return k * PGeo<D>::kKvTile + R * wave + (kWaves * R) * i;
}

// Table entries of the wave's stage rows of tile k (B >= kRowsPerLoad: one
// per row, uniform over the wave); tokens past the context read the last
// token's entry and are masked.
template <int D, int B>
__device__ __forceinline__ void table_entries(int32_t (&e)[PGeo<D>::kStageRows], int k, int wave, int n,
                                              const int32_t* __restrict__ trow) {
#pragma unroll
    for (int i = 0; i < PGeo<D>::kStageRows; ++i) {
        const int t = stage_token0<D>(k, wave, i);
        e[i] = trow[(t < n ? t : n - 1) / B];
    }
}

// One wave load of 16 bytes per lane from global memory straight into LDS
// (lane i's bytes land at lds + 16 i), addressed as a uniform 64-bit base
// plus a 32-bit per-lane offset, so that no vector instruction computes an
// address.  Issued in inline asm (M0 holds the LDS address; no other code
// of the kernel uses M0): the compiler does not track these loads, and the
// kernel's explicit waits order them against the LDS reads.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <bool kStream>
__device__ __forceinline__ void load_lds_saddr(const void* base_in, uint32_t lane_off, uint32_t lds_in) {
    // uniform by construction (a table entry read with a scalar load, a
    // buffer address): read from the first lane so that the compiler holds
    // them in scalar registers whatever it concludes about their divergence
    const uint64_t b = (uint64_t)(uintptr_t)base_in;
    const void* base = (const void*)(uintptr_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(b >> 32)) << 32) |
                                                (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b));
    const uint32_t lds_addr = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_in);
    if constexpr (kStream)
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" : : "v"(lane_off), "s"(base),
                     "s"(lds_addr) : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(lane_off), "s"(base),
                     "s"(lds_addr) : "memory", "m0");
}
#pragma clang diagnostic pop

// Fetch tile k (tokens kKvTile*k ..) from HBM into the LDS buffer `buf`;
// `e` holds its table entries when B >= kRowsPerLoad (read a step earlier),
// else every thread looks up its own row.  Rows past the context or with an id outside
// the pool read a row of some valid block (a fixed number of loads per
// tile) and are zeroed by finish_tile.
template <int D, int B, bool kStream, bool kAppend>
__device__ __forceinline__ void fetch_tile(Staged<D>& st, unsigned char* buf, int k,
                                           const int32_t (&e)[PGeo<D>::kStageRows], int wave, int lane,
                                           int n, const int32_t* __restrict__ trow,
                                           const _Float16* __restrict__ kbase, const _Float16* __restrict__ vbase,
                                           int64_t blk_stride, int32_t num_blocks, const AppendSrc& ap) {
    // kStream: every K/V byte is read by one workgroup only (all query rows
    // of a sequence fit one row tile), so the loads are nontemporal (the nt
    // bit of the cache policy); otherwise later row tiles of the sequence
    // re-read the tile and the default policy keeps it for them
    constexpr int kLoadPolicy = kStream ? 2 : 0;
    PF_GEO(D);
    const int col = lane % kChunks;
    if constexpr (!kAppend && B >= kRowsPerLoad) {
        // the wave's rows of load i lie in one block: a uniform base and a
        // per-lane offset (row within the load, swizzled chunk) that is the
        // same for every tile
#pragma unroll
        for (int i = 0; i < kStageRows; ++i) {
            const int t0 = stage_token0<D>(k, wave, i);
            const int32_t phys = e[i];
            const bool in_pool = (uint32_t)phys < (uint32_t)num_blocks;
            const int r = stage_token0<D>(0, wave, i) + lane / kChunks;
            const uint32_t rowb = (uint32_t)((lane / kChunks) * kD * 2);
            const uint32_t lk = rowb + 16u * (uint32_t)(col ^ (r & kSwzK));
            const uint32_t lv = rowb + 16u * (uint32_t)(col ^ (2 * (r & 3)));
            // bytes from the head's first block: the block, then the load's first row in it
            const uint64_t boff = (uint64_t)(uint32_t)(in_pool ? phys : 0) * (uint64_t)(blk_stride * 2) +
                                  (uint32_t)((t0 % B) * kD * 2);
            // a generic address of LDS carries the LDS offset in its low 32 bits
            const uint32_t lds = (uint32_t)(uintptr_t)buf;
            load_lds_saddr<kStream>(reinterpret_cast<const char*>(kbase) + boff, lk,
                                    lds + (uint32_t)(stage_token0<D>(0, wave, i) * kPitch));
            load_lds_saddr<kStream>(reinterpret_cast<const char*>(vbase) + boff, lv,
                                    lds + (uint32_t)(kTileBytes + stage_token0<D>(0, wave, i) * kPitchV));
            st.ok[i] = t0 + lane / kChunks < n && in_pool;
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < kStageRows; ++i) {
        const int t0 = stage_token0<D>(k, wave, i);        // uniform, a multiple of kRowsPerLoad
        const int t = t0 + lane / kChunks;
        int32_t phys;
        int row;                                           // row inside the block
        if constexpr (B >= kRowsPerLoad) {
            // the wave's rows share entry e[i] (of token min(t0, n-1)) and
            // lie at t0 % B + 0.. of a block -- inside it also past the context
            phys = e[i];
            row = t0 % B + lane / kChunks;
        } else {
            const int tc = t < n ? t : n - 1;
            phys = trow[tc / B];
            row = tc % B;
        }
        const bool in_pool = (uint32_t)phys < (uint32_t)num_blocks;
        const bool ok = t < n && in_pool;
        // LDS row r = stage row, position col holds chunk col ^ (r & kSwzK) of
        // K and chunk col ^ 2(r & 3) of V
        const int r = stage_token0<D>(0, wave, i) + lane / kChunks;
        const int64_t off = (int64_t)(in_pool ? phys : 0) * blk_stride + row * kD;
        const int ck = col ^ (r & kSwzK);
        const int cv = col ^ (2 * (r & 3));
        unsigned char* kdst = buf + stage_token0<D>(0, wave, i) * kPitch;
        unsigned char* vdst = buf + kTileBytes + stage_token0<D>(0, wave, i) * kPitchV;
        const _Float16* ksrc = kbase + off + ck * 8;
        const _Float16* vsrc = vbase + off + cv * 8;
        if constexpr (kAppend) {
            const bool fresh = t >= ap.base_pos && t < n;   // a new token: from key / value
            if (fresh) {
                const int64_t tok = (int64_t)(t - ap.base_pos) * ap.stride;
                ksrc = ap.k + tok + ck * 8;
                vsrc = ap.v + tok + cv * 8;
            }
            st.wphys[i] = fresh && in_pool && t >= ap.w_lo && t < ap.w_hi ? phys : -1;
        }
        __builtin_amdgcn_global_load_lds((const void*)ksrc, (__attribute__((address_space(3))) void*)kdst, 16, 0,
                                         kLoadPolicy);
        __builtin_amdgcn_global_load_lds((const void*)vsrc, (__attribute__((address_space(3))) void*)vdst, 16, 0,
                                         kLoadPolicy);
        st.ok[i] = ok;
    }
}

// After this thread's loads of the tile landed: zero its rows that are not
// valid (past the context or outside the pool) and write the flags.
template <int D>
__device__ __forceinline__ void finish_tile(const Staged<D>& st, unsigned char* buf, unsigned char* flags, int wave,
                                            int lane) {
    PF_GEO(D);
    const int col = lane % kChunks;
    bool all_ok = true;
#pragma unroll
    for (int i = 0; i < kStageRows; ++i) all_ok = all_ok && st.ok[i];
    if (!__all(all_ok)) {
#pragma unroll
        for (int i = 0; i < kStageRows; ++i) {
            const int row = stage_token0<D>(0, wave, i) + lane / kChunks;
            const u32x4 z = {0u, 0u, 0u, 0u};
            if (!st.ok[i]) {
                *reinterpret_cast<u32x4*>(buf + row * kPitch + col * 16) = z;
                *reinterpret_cast<u32x4*>(buf + kTileBytes + row * kPitchV + col * 16) = z;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kStageRows; ++i)
        if (col == 0) flags[stage_token0<D>(0, wave, i) + lane / kChunks] = st.ok[i];
}

// Append mode, while tile k is in LDS: the rows this thread loaded that are
// new tokens owned by the workgroup go from LDS into the cache, 16 bytes of
// K and of V each (LDS position col of row r holds chunk col ^ (r & kSwzK)
// of K and col ^ 2(r & 3) of V).  No workgroup reads these rows from the
// cache.
template <int D, int B>
__device__ __forceinline__ void write_own_rows(const Staged<D>& st, const unsigned char* buf, int k, int wave,
                                               int lane, _Float16* __restrict__ kw, _Float16* __restrict__ vw,
                                               int64_t blk_stride) {
    PF_GEO(D);
    const int col = lane % kChunks;
#pragma unroll
    for (int i = 0; i < kStageRows; ++i) {
        if (st.wphys[i] < 0) continue;
        const int r = stage_token0<D>(0, wave, i) + lane / kChunks;
        const int t = k * kKvTile + r;
        const int64_t dst = (int64_t)st.wphys[i] * blk_stride + (int64_t)(t % B) * kD;
        const u32x4 kv = *reinterpret_cast<const u32x4*>(buf + r * kPitch + col * 16);
        const u32x4 vv = *reinterpret_cast<const u32x4*>(buf + kTileBytes + r * kPitchV + col * 16);
        *reinterpret_cast<u32x4*>(kw + dst + (col ^ (r & kSwzK)) * 8) = kv;
        *reinterpret_cast<u32x4*>(vw + dst + (col ^ (2 * (r & 3))) * 8) = vv;
    }
}

// Runtime flags of one of the wave's 16-row groups, for this lane's row.
struct Rows {
    bool live;       // the row (l % 16 of its group) exists
    int pos;         // its position
    int rel;         // pos - 4 * (l / 16)
};


constexpr float kLazyMax = 8.f;           // log2 slack of the running maximum

// Cross-lane maximum over the four lanes l % 16 + 16 j (j = 0..3) that
// hold one row's scores: v_permlane32_swap pairs lanes l and l ^ 32,
// v_permlane16_swap lanes l and l ^ 16; each returns the two values of the
// pair in its two results, so the maximum of them is the pair's.

__device__ __forceinline__ float max2(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ float max3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

__device__ __forceinline__ float row_max4(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = max2(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return max2(__uint_as_float(b[0]), __uint_as_float(b[1]));
}


typedef short v4s_ __attribute__((ext_vector_type(4)));

// LDS transpose reads of kG (1 or 2) groups of 4 PV d-tiles: for group gg,
// r[8gg + 2c] = the 8 bytes at a[c] + base + gg * kGroup and r[8gg + 2c +
// 1] at the same + kHalf (the second half of the 32-token slab), base = u *
// kSlab + grp * kGroup.  Issued in inline asm with their wait inside the
// same block: the builtin carries no memory operand, so the compiler would
// wait for every load into LDS still in flight before it.  The offsets are
// immediates, hence one asm block per (slab, group) pair.
template <int kG, int kSlab, int kHalf, int kGroup>
__device__ __forceinline__ void tr_reads(v4s_ (&r)[8 * kG], const uint32_t (&a)[4], int u, int grp) {
    static_assert(kSlab + 3 * kGroup + kHalf < 65536, "transpose-read offsets fit the 16-bit field");
#define PF_TR8(BASE)                                                                                   \
    asm volatile(                                                                                      \
        "ds_read_b64_tr_b16 %0, %8 offset:%12\n\t"                                                     \
        "ds_read_b64_tr_b16 %1, %8 offset:%13\n\t"                                                     \
        "ds_read_b64_tr_b16 %2, %9 offset:%12\n\t"                                                     \
        "ds_read_b64_tr_b16 %3, %9 offset:%13\n\t"                                                     \
        "ds_read_b64_tr_b16 %4, %10 offset:%12\n\t"                                                    \
        "ds_read_b64_tr_b16 %5, %10 offset:%13\n\t"                                                    \
        "ds_read_b64_tr_b16 %6, %11 offset:%12\n\t"                                                    \
        "ds_read_b64_tr_b16 %7, %11 offset:%13\n\t"                                                    \
        "s_waitcnt lgkmcnt(0)"                                                                         \
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),  \
          "=&v"(r[7])                                                                                  \
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(BASE), "i"((BASE) + kHalf)                 \
        : "memory")
#define PF_TR16(BASE)                                                                                  \
    asm volatile(                                                                                      \
        "ds_read_b64_tr_b16 %0, %16 offset:%20\n\t"                                                    \
        "ds_read_b64_tr_b16 %1, %16 offset:%21\n\t"                                                    \
        "ds_read_b64_tr_b16 %2, %17 offset:%20\n\t"                                                    \
        "ds_read_b64_tr_b16 %3, %17 offset:%21\n\t"                                                    \
        "ds_read_b64_tr_b16 %4, %18 offset:%20\n\t"                                                    \
        "ds_read_b64_tr_b16 %5, %18 offset:%21\n\t"                                                    \
        "ds_read_b64_tr_b16 %6, %19 offset:%20\n\t"                                                    \
        "ds_read_b64_tr_b16 %7, %19 offset:%21\n\t"                                                    \
        "ds_read_b64_tr_b16 %8, %16 offset:%22\n\t"                                                    \
        "ds_read_b64_tr_b16 %9, %16 offset:%23\n\t"                                                    \
        "ds_read_b64_tr_b16 %10, %17 offset:%22\n\t"                                                   \
        "ds_read_b64_tr_b16 %11, %17 offset:%23\n\t"                                                   \
        "ds_read_b64_tr_b16 %12, %18 offset:%22\n\t"                                                   \
        "ds_read_b64_tr_b16 %13, %18 offset:%23\n\t"                                                   \
        "ds_read_b64_tr_b16 %14, %19 offset:%22\n\t"                                                   \
        "ds_read_b64_tr_b16 %15, %19 offset:%23\n\t"                                                   \
        "s_waitcnt lgkmcnt(0)"                                                                         \
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),  \
          "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]),             \
          "=&v"(r[13]), "=&v"(r[14]), "=&v"(r[15])                                                     \
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(BASE), "i"((BASE) + kHalf),                 \
          "i"((BASE) + kGroup), "i"((BASE) + kGroup + kHalf)                                           \
        : "memory")
    if constexpr (kG == 1) {
        switch (u * 8 + grp) {
            case 0: PF_TR8(0); break;
            case 1: PF_TR8(kGroup); break;
            case 2: PF_TR8(2 * kGroup); break;
            case 3: PF_TR8(3 * kGroup); break;
            case 8: PF_TR8(kSlab); break;
            case 9: PF_TR8(kSlab + kGroup); break;
            case 10: PF_TR8(kSlab + 2 * kGroup); break;
            case 11: PF_TR8(kSlab + 3 * kGroup); break;
            default: break;
        }
    } else {
        switch (u * 8 + grp) {
            case 0: PF_TR16(0); break;
            case 2: PF_TR16(2 * kGroup); break;
            case 8: PF_TR16(kSlab); break;
            case 10: PF_TR16(kSlab + 2 * kGroup); break;
            default: break;
        }
    }
#undef PF_TR8
#undef PF_TR16
}

// Causal and flag masks of the scores of tokens 16h + 4j + 0..3 of a tile
// (lane group j), in place: a token is kept when 16h + e <= lim, and in mode
// 2 only when its flag is set too.  One asm block per 16-token half with
// the mode tested inside it: the compiler sees no branch, so every mode
// leaves the scores in the registers they came in (a branch here made it
// copy all 16 scores of a group on every tile).  Mode 2 reads the flag word
// from LDS and waits for it in the same block.  The scores come from
// matrix-core products, whose results a vector instruction may read only some
// cycles after the product issued; the compiler pads its own instructions for
// this but not those inside inline asm, so the causal path opens with 22 wait
// states (the most any product here needs) and the flag path's LDS wait
// covers it.
#define PF_MASK_H(H)                                                                                  \
    asm volatile(                                                                                    \
        "s_cmp_eq_u32 %[mode], 0\n\t"                                                                \
        "s_cbranch_scc1 3f\n\t"                                                                      \
        "s_cmp_eq_u32 %[mode], 1\n\t"                                                                \
        "s_cbranch_scc1 2f\n\t"                                                                      \
        "ds_read_b32 %[fl], %[fa] offset:%[fo]\n\t"                                                  \
        "s_waitcnt lgkmcnt(0)\n\t"                                                                   \
        "v_bfe_u32 %[t], %[fl], 0, 8\n\t"                                                           \
        "v_cmp_ne_u32 vcc, 0, %[t]\n\t"                                                             \
        "v_cndmask_b32 %[t], -1, %[lim], vcc\n\t"                                                   \
        "v_cmp_le_i32 vcc, %[i0], %[t]\n\t"                                                         \
        "v_cndmask_b32 %0, %[ninf], %0, vcc\n\t"                                                    \
        "v_bfe_u32 %[t], %[fl], 8, 8\n\t"                                                           \
        "v_cmp_ne_u32 vcc, 0, %[t]\n\t"                                                             \
        "v_cndmask_b32 %[t], -1, %[lim], vcc\n\t"                                                   \
        "v_cmp_le_i32 vcc, %[i1], %[t]\n\t"                                                         \
        "v_cndmask_b32 %1, %[ninf], %1, vcc\n\t"                                                    \
        "v_bfe_u32 %[t], %[fl], 16, 8\n\t"                                                          \
        "v_cmp_ne_u32 vcc, 0, %[t]\n\t"                                                             \
        "v_cndmask_b32 %[t], -1, %[lim], vcc\n\t"                                                   \
        "v_cmp_le_i32 vcc, %[i2], %[t]\n\t"                                                         \
        "v_cndmask_b32 %2, %[ninf], %2, vcc\n\t"                                                    \
        "v_bfe_u32 %[t], %[fl], 24, 8\n\t"                                                          \
        "v_cmp_ne_u32 vcc, 0, %[t]\n\t"                                                             \
        "v_cndmask_b32 %[t], -1, %[lim], vcc\n\t"                                                   \
        "v_cmp_le_i32 vcc, %[i3], %[t]\n\t"                                                         \
        "v_cndmask_b32 %3, %[ninf], %3, vcc\n\t"                                                    \
        "s_branch 3f\n"                                                                              \
        "2:\n\t"                                                                                    \
        "s_nop 7\n\t"                                                                               \
        "s_nop 7\n\t"                                                                               \
        "s_nop 5\n\t"                                                                               \
        "v_cmp_le_i32 vcc, %[i0], %[lim]\n\t"                                                       \
        "v_cndmask_b32 %0, %[ninf], %0, vcc\n\t"                                                    \
        "v_cmp_le_i32 vcc, %[i1], %[lim]\n\t"                                                       \
        "v_cndmask_b32 %1, %[ninf], %1, vcc\n\t"                                                    \
        "v_cmp_le_i32 vcc, %[i2], %[lim]\n\t"                                                       \
        "v_cndmask_b32 %2, %[ninf], %2, vcc\n\t"                                                    \
        "v_cmp_le_i32 vcc, %[i3], %[lim]\n\t"                                                       \
        "v_cndmask_b32 %3, %[ninf], %3, vcc\n"                                                       \
        "3:"                                                                                         \
        : "+v"(s2[H][0]), "+v"(s2[H][1]), "+v"(s2[H][2]), "+v"(s2[H][3]), [fl] "=&v"(fl_), [t] "=&v"(t_) \
        : [mode] "s"(mode), [lim] "v"(lim), [ninf] "v"(ninf), [fa] "v"(fa), [fo] "i"(16 * (H)),       \
          [i0] "i"(16 * (H)), [i1] "i"(16 * (H) + 1), [i2] "i"(16 * (H) + 2), [i3] "i"(16 * (H) + 3)   \
        : "vcc", "scc", "memory")

template <int NH>
__device__ __forceinline__ void mask_scores(float (&s2)[NH][4], int mode, int lim, uint32_t fa) {
    static_assert(NH == 2 || NH == 4, "16-token halves per tile");
    const float ninf = -INFINITY;
    uint32_t fl_, t_;
    PF_MASK_H(0);
    PF_MASK_H(1);
    if constexpr (NH == 4) {
        PF_MASK_H(2);
        PF_MASK_H(3);
    }
}
#undef PF_MASK_H

// Online softmax of one 16-row group's scores of a tile (mode as for
// consume_lds_tile): masks, running maximum, the rescale of O and l when the
// maximum moved, and the fp16 weights P.
template <int D>
__device__ __forceinline__ void row_softmax(Softmax<D>& st, half8_t_ (&p)[PGeo<D>::kKvTile / 32],
                                            float (&s2)[PGeo<D>::kKvTile / 16][4], const unsigned char* flags,
                                            int t0, int mode, float c_log2, int j, const Rows& rw) {
    PF_GEO(D);
    constexpr int NS = kKvTile / 32;
    // raw scores, -inf where masked; token 16h + 4j + e of the tile is kept
    // when at or before the row's position: 16h + e <= lim = pos - t0 - 4j
    // (-1 for a row that does not exist)
    const uint32_t fa = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)(flags + 4 * j);
    mask_scores<2 * NS>(s2, __builtin_amdgcn_readfirstlane(mode), rw.live ? rw.rel - t0 : -1, fa);  // mode: uniform
    // the maximum as v_max3 chains (IEEE-mode fmaxf would first quiet every
    // operand with a v_max of itself)
    float mt = max3(s2[0][0], s2[0][1], s2[0][2]);
    mt = max2(mt, s2[0][3]);
#pragma unroll
    for (int h = 1; h < 2 * NS; ++h) {
        mt = max3(mt, s2[h][0], s2[h][1]);
        mt = max3(mt, s2[h][2], s2[h][3]);
    }
    mt = row_max4(mt) * c_log2;                 // c > 0: the maximum of the scaled scores
    // The running maximum moves only when the tile's exceeds it by more than
    // kLazyMax: the weights stay below 2^kLazyMax (fine in fp16, summed in
    // fp32) and the rescale of O and l is rare after the first tiles.
    const float m_new = max2(st.m, mt);
    const bool bump = m_new > st.m + kLazyMax;  // also the first finite maximum
    const float m_run = bump ? m_new : st.m;
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    if (__any(bump)) {
        // the lane's O and l belong to its own row: no exchange between lanes
        const float alpha = bump ? fast_exp2(st.m - m_use) : 1.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) st.l[e] *= alpha;
#pragma unroll
        for (int c = 0; c < kDTiles; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) st.o[c][e] *= alpha;
    }
    st.m = m_run;
#pragma unroll
    for (int h = 0; h < 2 * NS; ++h)
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
            // sub-tile u = h / 2 takes halves 2u (k 0..3 of each lane group) and 2u+1 (k 4..7)
            const float w0 = fast_exp2(__builtin_fmaf(s2[h][e], c_log2, -m_use));
            const float w1 = fast_exp2(__builtin_fmaf(s2[h][e + 1], c_log2, -m_use));
            p[h / 2][4 * (h % 2) + e] = (_Float16)w0;
            p[h / 2][4 * (h % 2) + e + 1] = (_Float16)w1;
        }
}

// Consume one LDS tile for the wave's kNT groups of 16 rows on
// v_mfma_f32_16x16x32_f16.  Every operand read from LDS feeds kNT products.
//   QK, per 16-token half h: S^T[token][row] = sum_d K[token][d] Q[row][d];
//     MFMA c takes d = 32c + 8*(l/16) + 0..7 in lane l (one 16-byte LDS read).
//   PV, per 32-token slab u, as O^T += V^T P^T: k = 32 tokens; lane (n, j)
//     supplies P[row n][tokens 32u + 4j..4j+3 and 32u + 16+4j..16+4j+3] --
//     exactly the scores it holds -- as the B operand, and V of the same
//     tokens at column 16c + n for d-tile c (LDS transpose reads) as the A
//     operand; lane (n, j) then holds O[row n][16c + 4j .. +3].  One more
//     product per slab with an all-ones A operand adds each row's weights
//     into the running sum l (every element the row's sum), so that no
//     vector instruction sums them.
// kMask: 0 = the tile lies wholly at or before the wave's first row and
// every token is valid, no score is masked; 1 = every token is valid, only
// the causal mask (and rows past the wave's last) applies; 2 = some token
// is past the context or behind an id outside the pool: the flags too.
// (Each case runs its own copy of the softmax, so that differently masked
// scores are never merged into one set of registers.)
// The exponent of a weight is one FMA of the raw score: c = scale *
// log2(e) > 0, so the raw maximum times c is the maximum of the scaled
// scores, and -inf stays -inf.
template <int D>
__device__ __forceinline__ void consume_lds_tile(Softmax<D> (&st)[PGeo<D>::kNT], const unsigned char* buf,
                                                 const unsigned char* flags, int t0, int mask,
                                                 const half8_t_ (&qb)[PGeo<D>::kNT][PGeo<D>::kQk], float c_log2,
                                                 int lane, const Rows (&rw)[PGeo<D>::kNT]) {
    PF_GEO(D);
    constexpr int NS = kKvTile / 32;            // 32-token sub-tiles (one PV MFMA k-slab each)
    const int n = lane & 15;
    const int j = lane >> 4;
    const unsigned char* kb = buf;
    const unsigned char* vb = buf + kTileBytes;
    float s2[kNT][2 * NS][4];                 // scores as single floats: masked in place, register by register
#pragma unroll
    for (int h = 0; h < 2 * NS; ++h) {
        float4_t acc[kNT];
#pragma unroll
        for (int t = 0; t < kNT; ++t) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < kQk; ++c) {
            const half8_t_ a = __builtin_bit_cast(half8_t_, *reinterpret_cast<const u32x4*>(
                kb + (16 * h + n) * kPitch + 16 * ((4 * c + j) ^ ((16 * h + n) & kSwzK))));
#pragma unroll
            for (int t = 0; t < kNT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qb[t][c], acc[t], 0, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < kNT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) s2[t][h][e] = acc[t][e];
    }
    half8_t_ p[kNT][NS];
#pragma unroll
    for (int t = 0; t < kNT; ++t) row_softmax<D>(st[t], p[t], s2[t], flags, t0, mask, c_log2, j, rw[t]);
    // the row sums: P times an all-ones operand, for every slab
    const half8_t_ ones = {(_Float16)1.f, (_Float16)1.f, (_Float16)1.f, (_Float16)1.f,
                           (_Float16)1.f, (_Float16)1.f, (_Float16)1.f, (_Float16)1.f};
#pragma unroll
    for (int u = 0; u < NS; ++u)
#pragma unroll
        for (int t = 0; t < kNT; ++t) st[t].l = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, p[t][u], st[t].l, 0, 0, 0);
    // PV with the V operand read by ds_read_b64_tr_b16: within each 16 lanes
    // it hands lane i element i%4 of the 8-byte pieces of lanes i/4 + 4e,
    // e = 0..3.  Lane 4e + q of lane group j points at V[token tb + e][16c +
    // 4q] (tb = 4j for k 0..3 of the B operand, 16 + 4j for k 4..7: the
    // tokens whose weights the lane holds in P), so lane (n, j) receives
    // V[tb + e][16c + n]: the A operand of d-tile c (row m = n of V^T being
    // d = 16c + n).  The 32-byte unit c of V row r sits at unit c ^ (r
    // & 3) (the chunk swizzle of fetch_tile), so the 4 rows x 4 pieces of one
    // lane group fall in distinct banks.  d-tiles come in groups of 4 (128
    // bytes of a row); one asm block reads two token halves of one group.
    const int e4 = (lane & 15) >> 2;
    const int q4 = lane & 3;
    const unsigned char* lo = vb + (4 * j + e4) * kPitchV + 8 * q4;
    uint32_t a[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
        a[c] = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)(lo + 32 * (c ^ e4));
    constexpr int kG = kDTiles >= 8 ? 2 : 1;   // d-tile groups per asm block
#pragma unroll
    for (int u = 0; u < NS; ++u) {
#pragma unroll
        for (int grp = 0; grp < kDTiles / 4; grp += kG) {
            v4s_ r[8 * kG];
            tr_reads<kG, 32 * kPitchV, 16 * kPitchV, 128>(r, a, u, grp);
#pragma unroll
            for (int c = 0; c < 4 * kG; ++c) {
                const half4_t h0 = __builtin_bit_cast(half4_t, r[2 * c]);
                const half4_t h1 = __builtin_bit_cast(half4_t, r[2 * c + 1]);
                const half8_t_ b = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
#pragma unroll
                for (int t = 0; t < kNT; ++t)
                    st[t].o[4 * grp + c] =
                        __builtin_amdgcn_mfma_f32_16x16x32_f16(b, p[t][u], st[t].o[4 * grp + c], 0, 0, 0);
            }
        }
    }
}

template <int D, int B, bool kStream, bool kAppend, bool kPersistent = false>
__global__ void __launch_bounds__(kThreads)
prefill_mfma_kernel(_Float16* __restrict__ out, const _Float16* __restrict__ q, int32_t num_tokens,
                    const _Float16* __restrict__ k_cache, const _Float16* __restrict__ v_cache,
                    const int32_t* __restrict__ tables, int32_t max_blocks, const int32_t* __restrict__ lens,
                    const int32_t* __restrict__ query_start, int32_t num_heads, int32_t num_kv_heads,
                    int32_t num_blocks, float scale_log2, int32_t max_query_len, int64_t len_cap,
                    float* __restrict__ ws_ml, float* __restrict__ ws_acc, int32_t tiles_per_part,
                    int32_t num_parts, int32_t num_seqs, int32_t row_tiles, int32_t xcd_grouped,
                    const _Float16* __restrict__ new_k, const _Float16* __restrict__ new_v, int64_t new_stride,
                    _Float16* __restrict__ k_write, _Float16* __restrict__ v_write, unsigned* __restrict__ claim,
                    const int32_t* __restrict__ seq_order) {
    PF_GEO(D);
    // two stage buffers as distinct objects, so that the compiler can tell
    // the buffer a step reads from the one whose loads are in flight
    __shared__ __attribute__((aligned(16))) unsigned char ldsA[kBufBytes];
    __shared__ __attribute__((aligned(16))) unsigned char ldsB[kBufBytes];
    __shared__ __attribute__((aligned(4))) unsigned char flA[kKvTile];
    __shared__ __attribute__((aligned(4))) unsigned char flB[kKvTile];
    // One-dimensional grid over (KV head, sequence) pairs x row tiles x
    // context parts.  Workgroups are dealt to the 8 XCDs round-robin in
    // linear order; with xcd_grouped (pairs a multiple of 8) workgroup L
    // runs item L / 8 of XCD L % 8, whose items are the row tiles and parts
    // of its pairs (pair q on XCD q % 8), pair by pair: the row tiles of a
    // pair, which all walk the same K/V tiles, run together on one XCD and
    // share its L2.  Otherwise the pair is fastest (KV head first).  Either
    // way the last row tile of a pair comes first (the longest causal range
    // starts earliest) and parts are fastest within a row tile.  With
    // seq_order the pairs' sequences are taken in that order (longest first,
    // so that no long prompt's row tiles start last and run alone at the
    // end).
    //
    // Persistent form (claim non-null): the grid is one round of resident
    // workgroups, a multiple of 8, and workgroup b takes items of XCD b % 8
    // (all items when not XCD-grouped) in list order from the counter
    // claim[b % 8], which starts at zero.  A workgroup claims its next item
    // two tile steps before its walk ends and leaves when the list is
    // exhausted.  One
    // workgroup per slot instead of one per item: the hardware deals a new
    // workgroup to the XCDs in strict rotation, so one whose XCD has no free
    // slot holds back those behind it, and slots stood empty for 3-11 us
    // between workgroups (1.4-1.7 of 2 workgroups resident per CU on
    // prompts up to 1024 tokens).
    __shared__ int s_claim[2];
    if constexpr (!kPersistent) claim = nullptr;           // one item per workgroup: the loop below runs once
    const int64_t pairs = (int64_t)num_kv_heads * num_seqs;
    const int64_t rp_n = (int64_t)row_tiles * num_parts;
    const int64_t total = pairs * rp_n;
    const int cx = (xcd_grouped && claim) ? (int)(blockIdx.x & 7) : 0;     // this workgroup's list
    const int cstride = xcd_grouped ? 8 : 1;
    const int items_cx = (int)((total - cx + cstride - 1) / cstride);
    // the counter's index in a vector register (the atomics take their
    // address there; the tile walk's scalar registers are all in use)
    int cxv = cx;
    if constexpr (kPersistent) asm volatile("" : "+v"(cxv));
    int w_cur = 0;
    int cpar = 0;
    if constexpr (kPersistent) {
        if (threadIdx.x == 0) s_claim[0] = (int)atomicAdd(claim + cxv, 1u);
        __syncthreads();
        w_cur = s_claim[0];
    }
    for (;;) {
    int64_t item;
    unsigned nxt = ~0u;         // the next item's ticket (lane 0), once claimed during the walk
    if (claim) {
        if (w_cur >= items_cx) break;
        item = (int64_t)w_cur * cstride + cx;
    } else {
        item = blockIdx.x;
    }
    do {
    // (32-bit arithmetic: the host keeps the item count below 2^31)
    uint32_t pair, rp;
    if (xcd_grouped) {
        const uint32_t w = (uint32_t)item >> 3;
        pair = ((uint32_t)item & 7u) + 8u * (w / (uint32_t)rp_n);
        rp = w % (uint32_t)rp_n;
    } else {
        pair = (uint32_t)item % (uint32_t)pairs;
        rp = (uint32_t)item / (uint32_t)pairs;
    }
    const int kvh = (int)(pair % (uint32_t)num_kv_heads);
    const int s = seq_order ? seq_order[pair / (uint32_t)num_kv_heads] : (int)(pair / (uint32_t)num_kv_heads);
    if ((uint32_t)s >= (uint32_t)num_seqs) break;           // an order entry outside the batch: skipped
    const int rtile = row_tiles - 1 - (int)(rp / (uint32_t)num_parts);
    const int part = (int)(rp % (uint32_t)num_parts);
    // the thread index passed through an opaque instruction on every item,
    // so that no per-lane value is computed once before the item loop and
    // held in registers across every tile walk
    int tid = (int)threadIdx.x;
    if constexpr (kPersistent) asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = num_heads / num_kv_heads;

    const int32_t q0 = query_start[s];
    const int32_t q1 = query_start[s + 1];
    // rows outside [0, num_tokens) are never touched: a sequence whose range
    // is not inside it is skipped
    if (q0 < 0 || q1 < q0 || q1 > num_tokens) break;
    const int32_t m_raw = q1 - q0;
    const int32_t n_raw = lens[s];
    const int rows_all = (m_raw < max_query_len ? m_raw : max_query_len) * g;
    const int grow0 = rtile * kRowsPerGroup;               // first row of the workgroup
    if (grow0 >= rows_all) {                               // uniform over the workgroup
        // a row tile past the sequence's rows: so are the pair's next items
        // in the list (its higher row tiles come first), so the counter
        // skips to the pair's first row tile that has rows
        if (claim && xcd_grouped && threadIdx.x == 0) {
            const int r_s = (rows_all + kRowsPerGroup - 1) / kRowsPerGroup;
            const uint32_t first = (uint32_t)(w_cur / rp_n * rp_n + (int64_t)(row_tiles - r_s) * num_parts);
            atomicMax(claim + cxv, first);
        }
        break;
    }
    const bool bad = m_raw > max_query_len || n_raw < m_raw || (int64_t)n_raw > len_cap;
    const int row0 = grow0 + wave * kRowsPerWave;          // first row of this wave
    const int rows = max(0, min(rows_all - row0, kRowsPerWave));
    const int nrow = lane & 15;
    const int jg = lane >> 4;
    if (bad) {                                             // the sequence's rows come out as NaN
        if (jg == 0 && part == 0)
            for (int t = 0; t < kNT; ++t) {
                if (16 * t + nrow >= rows) continue;
                const int r = row0 + 16 * t + nrow;
                const int64_t orow = ((int64_t)q0 + r / g) * num_heads + (int64_t)kvh * g + r % g;
                for (int d = 0; d < kD; ++d) out[orow * kD + d] = (_Float16)NAN;
            }
        break;                                             // uniform: bad depends on the sequence only
    }
    const int n = n_raw, m = m_raw;
    const int base_pos = n - m;

    // A negative scale is carried by Q's sign (exact in fp16), so that the
    // scale applied to the scores is positive; scale 0 becomes the least
    // normal float, whose products with fp16 dot products (below 2^40) leave
    // every weight exactly 1, as at 0.
    const bool neg = scale_log2 < 0.f;
    const float c_log2 = fmaxf(neg ? -scale_log2 : scale_log2, 1.17549435e-38f);
    Rows rw[kNT];
    half8_t_ qb[kNT][kQk];
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
        rw[t].live = 16 * t + nrow < rows;
        const int r = row0 + 16 * t + (rw[t].live ? nrow : 0);
        rw[t].pos = base_pos + r / g;
        rw[t].rel = rw[t].pos - 4 * jg;
        const _Float16* qrow = q + (((int64_t)q0 + r / g) * num_heads + (int64_t)kvh * g + r % g) * kD;
#pragma unroll
        for (int c = 0; c < kQk; ++c) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            const uint32_t flip = neg ? 0x80008000u : 0u;
            u32x4 v = rw[t].live ? *reinterpret_cast<const u32x4*>(qrow + 32 * c + 8 * jg) : z;
            v ^= u32x4{flip, flip, flip, flip};
            qb[t][c] = __builtin_bit_cast(half8_t_, v);
        }
    }
    // the workgroup walks the tiles up to its last row's position; a wave
    // computes only up to its own last row's; tiles wholly at or before its
    // first row's position need no causal mask
    const int wg_rows = min(rows_all - grow0, kRowsPerGroup);
    const int ntiles = (base_pos + (grow0 + wg_rows - 1) / g) / kKvTile + 1;
    const int my_tiles = rows > 0 ? (base_pos + (row0 + rows - 1) / g) / kKvTile + 1 : 0;
    // this workgroup's share of the context: tiles [k_begin, k_end)
    const int k_begin = part * tiles_per_part;
    if (k_begin >= ntiles) break;                          // uniform: nothing of this part is visible
    const int k_end = min(ntiles, k_begin + tiles_per_part);
    const int my_end = min(k_end, my_tiles);
    const int first_pos = base_pos + row0 / g;

    const int32_t* trow = tables + (int64_t)s * max_blocks;
    const int64_t slab = (int64_t)B * kD;
    const _Float16* kbase = k_cache + (int64_t)kvh * slab;
    const _Float16* vbase = v_cache + (int64_t)kvh * slab;
    const int64_t blk_stride = (int64_t)num_kv_heads * slab;

    Softmax<D> st[kNT];
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
        st[t].m = -INFINITY;
        st[t].l = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < kDTiles; ++c) st[t].o[c] = float4_t{0.f, 0.f, 0.f, 0.f};
    }

    // Pipeline: tile k is consumed from its LDS buffer while tile k+1 is
    // being fetched into the other -- each fetch has one tile period (64
    // tokens of products) to land; the table entries of tile k+2 are read
    // meanwhile.  Tiles kb, kb+1, ... use buffers A, B, A, ... (the loop is
    // unrolled by two, so every step names its buffers at compile time).
    // The waits are explicit and the barriers bare: the compiler, left to
    // itself, would wait for the loads in flight before every LDS read it
    // cannot tell apart from the buffer being filled.  Three 32-token
    // buffers (tile k+2 in flight while waiting for k+1) were slower on
    // every prompt workload (8192-token prompts 641 against 721 TFLOP/s)
    // and faster only on short chunks over long caches (4 x 8192 cached +
    // 32 new: 106 against 110 us).
    AppendSrc ap{};
    _Float16* kw = nullptr;
    _Float16* vw = nullptr;
    if constexpr (kAppend) {
        // the sequence's new tokens (rows q0 .. of key / value); this
        // workgroup writes those whose first query row r = i * g is one of
        // its rows [grow0, grow0 + kRowsPerGroup)
        ap.k = new_k + (int64_t)q0 * new_stride + (int64_t)kvh * kD;
        ap.v = new_v + (int64_t)q0 * new_stride + (int64_t)kvh * kD;
        ap.stride = new_stride;
        ap.base_pos = base_pos;
        ap.w_lo = base_pos + (grow0 + g - 1) / g;
        ap.w_hi = base_pos + (grow0 + kRowsPerGroup + g - 1) / g;
        kw = k_write + (int64_t)kvh * slab;
        vw = v_write + (int64_t)kvh * slab;
    }
    Staged<D> SA, SB;
    int32_t e[kStageRows] = {};
    const int kb = k_begin;
    if constexpr (B >= kRowsPerLoad) table_entries<D, B>(e, kb, wave, n, trow);
    fetch_tile<D, B, kStream, kAppend>(SA, ldsA, kb, e, wave, lane, n, trow, kbase, vbase, blk_stride, num_blocks,
                                       ap);
    if constexpr (B >= kRowsPerLoad) table_entries<D, B>(e, kb + 1, wave, n, trow);
    PA_WAIT_VM(0);
    finish_tile<D>(SA, ldsA, flA, wave, lane);
    PA_WAIT_LGKM0();
    __builtin_amdgcn_s_barrier();
    auto step = [&](int k, unsigned char* cb, unsigned char* cf, const Staged<D>& cs, unsigned char* nb,
                    unsigned char* nf, Staged<D>& ns) {
        // the last step of the walk fetches nothing: no step consumes tile k_end
        const bool more = k + 1 < k_end;
        // the next item is claimed two steps before the walk ends: late
        // enough that the workgroup takes it as it comes free (the items of
        // a list in order, as slots free up), early enough that the claim
        // has returned by the last step's wait
        if (claim && k == max(k_begin, k_end - 2) && wave == 0) {
            // one atomic, from lane 0 (an atomic from every lane of the
            // wave, even adding zero, is 64 operations on one address, which
            // the memory side serialises)
            if (lane == 0) nxt = atomicAdd(claim + cxv, 1u);
        }
        if (more)
            fetch_tile<D, B, kStream, kAppend>(ns, nb, k + 1, e, wave, lane, n, trow, kbase, vbase, blk_stride,
                                               num_blocks, ap);
        if constexpr (B >= kRowsPerLoad)
            if (k + 2 < k_end) table_entries<D, B>(e, k + 2, wave, n, trow);
        if (k < my_end) {
            // uniform: every token of the tile valid; the tile wholly at or
            // before the wave's first row
            bool all_ok = true;              // the flags of tokens 16h + 4*jg .. +3, for every h
#pragma unroll
            for (int h = 0; h < kKvTile / 16; ++h)
                all_ok = all_ok && *reinterpret_cast<const uint32_t*>(cf + 16 * h + 4 * jg) == 0x01010101u;
            const bool tile_ok = __all(all_ok);
            const bool below = k * kKvTile + kKvTile - 1 <= first_pos;
            consume_lds_tile<D>(st, cb, cf, k * kKvTile, tile_ok ? (below ? 0 : 1) : 2, qb, c_log2, lane, rw);
        }
        PA_WAIT_VM(0);
        // append mode: the new tokens of tile k this workgroup owns go to the
        // cache now, after the wait, so that the stores complete under the
        // next step's products instead of stalling this step's wait; the LDS
        // reads finish before the barrier, ahead of the next fetch into `cb`
        if constexpr (kAppend) write_own_rows<D, B>(cs, cb, k, wave, lane, kw, vw, blk_stride);
        if (more) finish_tile<D>(ns, nb, nf, wave, lane);
        // the claim of this step has returned (the wait above): lane 0
        // publishes it in the other slot before the step's barrier
        if (claim && k == max(k_begin, k_end - 2) && threadIdx.x == 0) s_claim[cpar ^ 1] = (int)nxt;
        PA_WAIT_LGKM0();
        __builtin_amdgcn_s_barrier();
    };
    for (int k = kb;;) {
        step(k, ldsA, flA, SA, ldsB, flB, SB);
        if (++k >= k_end) break;
        step(k, ldsB, flB, SB, ldsA, flA, SA);
        if (++k >= k_end) break;
    }
    PA_WAIT_VM(0);                          // no load into LDS outstanding at exit

    if (num_parts > 1) {
        // unnormalised partial state of every row for the merge kernel:
        // (m, l) and O at [output row][part]; a lane holds 4 consecutive
        // columns of its row per d-tile (one 16-byte store each)
#pragma unroll
        for (int t = 0; t < kNT; ++t) {
            if (16 * t + nrow >= rows) continue;
            const int rwi = row0 + 16 * t + nrow;
            const int64_t orow = ((int64_t)q0 + rwi / g) * num_heads + (int64_t)kvh * g + rwi % g;
            const int64_t slot = orow * num_parts + part;
            float* acc = ws_acc + slot * kD + 4 * jg;
#pragma unroll
            for (int c = 0; c < kDTiles; ++c) *reinterpret_cast<float4_t*>(acc + 16 * c) = st[t].o[c];
            if (jg == 0) {
                ws_ml[2 * slot] = st[t].m;
                ws_ml[2 * slot + 1] = st[t].l[0];
            }
        }
        break;
    }

    // Row 16t + nrow of the wave lives in this lane's st[t].o[c] at columns
    // 16c + 4*jg .. +3, its sum in st[t].l.  The normalised rows go out
    // through the wave's own slice of buffer A (free after the walk's last
    // barrier): written there 8 bytes per lane, read back 16 contiguous
    // bytes per lane with kChunks lanes per row, so that each store
    // instruction writes whole rows.  Stored straight from the registers,
    // every 8-byte piece of a wave instruction fell on a different row: a
    // write request per lane.  Chunk q of staged row r sits at position
    // q ^ (r % kChunks), so that the 16 rows of one write and the chunks of
    // one read fall in distinct banks.
    {
        unsigned char* ost = ldsA + wave * (kRowsPerWave * kD * 2);
#pragma unroll
        for (int t = 0; t < kNT; ++t) {
            const int r = 16 * t + nrow;
            const float L = st[t].l[0];
            const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
            for (int c = 0; c < kDTiles; ++c) {
                const half4_t h = {(_Float16)(st[t].o[c][0] * inv), (_Float16)(st[t].o[c][1] * inv),
                                   (_Float16)(st[t].o[c][2] * inv), (_Float16)(st[t].o[c][3] * inv)};
                const int q = 2 * c + (jg >> 1);
                *reinterpret_cast<half4_t*>(ost + r * (kD * 2) + ((q ^ (r & (kChunks - 1))) << 4) + ((jg & 1) << 3)) =
                    h;
            }
        }
        constexpr int kRowsPerStore = 64 / kChunks;
        const int q = lane % kChunks;
        // row row0 + r is query head kvh*g + hd of token tk; r steps by
        // kRowsPerStore, so (tk, hd) step by (kRowsPerStore / g, kRowsPerStore
        // % g) with a carry (one division per lane, not one per row)
        const int rr0 = row0 + lane / kChunks;
        int tk = rr0 / g, hd = rr0 - (rr0 / g) * g;
        const int dt = kRowsPerStore / g, dh = kRowsPerStore - dt * g;
#pragma unroll
        for (int k = 0; k < kRowsPerWave / kRowsPerStore; ++k) {
            const int r = k * kRowsPerStore + lane / kChunks;
            if (r < rows) {
                const int64_t orow = ((int64_t)q0 + tk) * num_heads + (int64_t)kvh * g + hd;
                *reinterpret_cast<u32x4*>(out + orow * kD + 8 * q) =
                    *reinterpret_cast<const u32x4*>(ost + r * (kD * 2) + ((q ^ (r & (kChunks - 1))) << 4));
            }
            tk += dt;
            hd += dh;
            if (hd >= g) {
                hd -= g;
                ++tk;
            }
        }
    }
    } while (false);
    if (!claim) break;
    // the next item: published in the other slot during the walk; an item
    // that ended before walking claims now.  A bare barrier: __syncthreads()
    // would also wait for this item's output stores to be acknowledged (~2
    // us between items).  Two slots, so that a write never meets a read of
    // the previous claim.
    cpar ^= 1;
    if (threadIdx.x == 0 && nxt == ~0u) s_claim[cpar] = (int)atomicAdd(claim + cxv, 1u);
    asm volatile("" ::: "memory");
    PA_WAIT_LGKM0();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    w_cur = s_claim[cpar];
    }
}

// Zeroes the claim counters of the persistent prefill grid (one per XCD)
// before its launch, on the same stream.
__global__ void prefill_claim_reset(unsigned* __restrict__ claim) {
    if (threadIdx.x < 8) claim[threadIdx.x] = 0u;
}

// Merge of the context parts: output row (token i of sequence s, head h)
// combines the (m, l, O) its row tile's parts left, weighted by exp2(m_p -
// max m).  One thread per (token, column): a 256-thread workgroup covers
// 256 / D tokens of one (head, sequence), and the z dimension of the grid
// strides over the tokens.  (With a thread walking 16 tokens in turn, each
// waiting on the previous one's loads, the merge took ~28 us of a ~110 us
// chunked-prefill call.)
constexpr int kMergeThreads = 256;
constexpr int kMergeGridZ = 65535;

template <int D>
__global__ void __launch_bounds__(256)
prefill_merge_kernel(_Float16* __restrict__ out, const float* __restrict__ ws_ml, const float* __restrict__ ws_acc,
                     int32_t num_tokens, const int32_t* __restrict__ lens, const int32_t* __restrict__ query_start,
                     int32_t num_heads, int32_t num_kv_heads, int32_t max_query_len, int64_t len_cap,
                     int32_t tiles_per_part, int32_t num_parts, const int32_t* __restrict__ seq_order) {
    PF_GEO(D);
    constexpr int kTok = kMergeThreads / D;      // tokens per workgroup
    const int h = blockIdx.x;
    // the sequences the first kernel did (an order entry outside the batch
    // was skipped there too)
    const int s = seq_order ? seq_order[blockIdx.y] : (int)blockIdx.y;
    if ((uint32_t)s >= gridDim.y) return;
    const int d = threadIdx.x % D;
    const int g = num_heads / num_kv_heads;
    const int32_t q0 = query_start[s];
    const int32_t q1 = query_start[s + 1];
    if (q0 < 0 || q1 < q0 || q1 > num_tokens) return;     // skipped by the first kernel too
    const int32_t m = q1 - q0;
    const int32_t n = lens[s];
    if (m > max_query_len || n < m || (int64_t)n > len_cap) return;   // NaN rows, written by the first kernel
    const int base_pos = n - m;
    const int rows_all = m * g;
    for (int i = (int)blockIdx.z * kTok + (int)threadIdx.x / D; i < m; i += (int)gridDim.z * kTok) {
        // the row tile of this row, and how many parts its workgroups covered
        const int r = i * g + h % g;
        const int grow0 = (r / kRowsPerGroup) * kRowsPerGroup;
        const int wg_rows = min(rows_all - grow0, kRowsPerGroup);
        const int ntiles = (base_pos + (grow0 + wg_rows - 1) / g) / kKvTile + 1;
        const int np = min(num_parts, (ntiles + tiles_per_part - 1) / tiles_per_part);
        const int64_t orow = ((int64_t)q0 + i) * num_heads + h;
        const int64_t base = orow * num_parts;
        float M = -INFINITY;
        for (int p = 0; p < np; ++p) M = fmaxf(M, ws_ml[2 * (base + p)]);
        float L = 0.f, o = 0.f;
        for (int p = 0; p < np; ++p) {
            const float mp = ws_ml[2 * (base + p)];
            const float w = mp == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mp - M);
            L = fmaf(w, ws_ml[2 * (base + p) + 1], L);
            o = fmaf(w, ws_acc[(base + p) * kD + d], o);
        }
        out[orow * kD + d] = (_Float16)(L > 0.f ? o / L : 0.f);
    }
}

using PrefillFn = void (*)(_Float16*, const _Float16*, int32_t, const _Float16*, const _Float16*, const int32_t*,
                           int32_t, const int32_t*, const int32_t*, int32_t, int32_t, int32_t, float, int32_t,
                           int64_t, float*, float*, int32_t, int32_t, int32_t, int32_t, int32_t, const _Float16*,
                           const _Float16*, int64_t, _Float16*, _Float16*, unsigned*, const int32_t*);

template <int D, bool kStream, bool kAppend>
PrefillFn pick(int32_t b) {
    switch (b) {
        case 1: return prefill_mfma_kernel<D, 1, kStream, kAppend>;
        case 2: return prefill_mfma_kernel<D, 2, kStream, kAppend>;
        case 4: return prefill_mfma_kernel<D, 4, kStream, kAppend>;
        case 8: return prefill_mfma_kernel<D, 8, kStream, kAppend>;
        case 16: return prefill_mfma_kernel<D, 16, kStream, kAppend>;
        case 32: return prefill_mfma_kernel<D, 32, kStream, kAppend>;
        case 64: return prefill_mfma_kernel<D, 64, kStream, kAppend>;
        case 128: return prefill_mfma_kernel<D, 128, kStream, kAppend>;
        default: return nullptr;
    }
}

template <bool kStream, bool kAppend>
PrefillFn pick(int32_t d, int32_t b) {
    switch (d) {
        case 64: return pick<64, kStream, kAppend>(b);
        case 128: return pick<128, kStream, kAppend>(b);
        case 256: return pick<256, kStream, kAppend>(b);
        default: return nullptr;
    }
}

// The persistent-grid kernels (several row tiles per pair: never streaming).
template <int D, bool kAppend>
PrefillFn pick_persistent(int32_t b) {
    switch (b) {
        case 1: return prefill_mfma_kernel<D, 1, false, kAppend, true>;
        case 2: return prefill_mfma_kernel<D, 2, false, kAppend, true>;
        case 4: return prefill_mfma_kernel<D, 4, false, kAppend, true>;
        case 8: return prefill_mfma_kernel<D, 8, false, kAppend, true>;
        case 16: return prefill_mfma_kernel<D, 16, false, kAppend, true>;
        case 32: return prefill_mfma_kernel<D, 32, false, kAppend, true>;
        case 64: return prefill_mfma_kernel<D, 64, false, kAppend, true>;
        case 128: return prefill_mfma_kernel<D, 128, false, kAppend, true>;
        default: return nullptr;
    }
}

template <bool kAppend>
PrefillFn pick_persistent(int32_t d, int32_t b) {
    switch (d) {
        case 64: return pick_persistent<64, kAppend>(b);
        case 128: return pick_persistent<128, kAppend>(b);
        case 256: return pick_persistent<256, kAppend>(b);
        default: return nullptr;
    }
}

using MergeFn = void (*)(_Float16*, const float*, const float*, int32_t, const int32_t*, const int32_t*, int32_t,
                         int32_t, int32_t, int64_t, int32_t, int32_t, const int32_t*);

MergeFn pick_merge(int32_t d) {
    switch (d) {
        case 64: return prefill_merge_kernel<64>;
        case 128: return prefill_merge_kernel<128>;
        case 256: return prefill_merge_kernel<256>;
        default: return nullptr;
    }
}

// Row tile and K/V tile of the kernel serving head_dim d.
struct HostGeo {
    int32_t rows_per_group;
    int32_t kv_tile;
};

HostGeo host_geo(int32_t d) {
    switch (d) {
        case 64: return {PGeo<64>::kRowsPerGroup, PGeo<64>::kKvTile};
        case 256: return {PGeo<256>::kRowsPerGroup, PGeo<256>::kKvTile};
        default: return {PGeo<128>::kRowsPerGroup, PGeo<128>::kKvTile};
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// z dimension of the merge kernel's grid: one step per 256 / head_dim
// tokens, capped (the kernel strides over the rest)
int64_t merge_grid_z(int32_t max_query_len, int32_t head_dim) {
    const int64_t tok = kMergeThreads / head_dim;
    const int64_t z = ((int64_t)max_query_len + tok - 1) / tok;
    return z < 1 ? 1 : z > kMergeGridZ ? kMergeGridZ : z;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Context split.  Workgroups per part: one per (KV head, sequence, row
// tile).  When they fill at most half the resident slots (2 per CU, 512),
// the context is cut into floor(512 / workgroups) parts of at least 4 tiles
// (256 tokens): one full round of workgroups, each leaving the partial
// (m, l, O) of its rows for a merge kernel.  (A second, partial round costs
// more than it brings: on 4 x 8192 cached + 32 new, with 32-token tiles,
// 512 workgroups ran in 113 us, 768 in 149, 1024 in 147, 2048 in 203.)  The
// bound on the context is max_blocks_per_seq * block_size (host-known).
// Only a context long against the new tokens is split: at least 8 times
// max_query_len, or 2 times when the row tiles give at most 128 workgroups.
// The partial states cost (2 + D) x 4 bytes per (token, head, part),
// written and read back, against 4 x D bytes of K/V per (position, KV head)
// read once.  Measured per call (32 / 32 heads, head_dim 128, split against
// unsplit): a whole 774 / 1024-token prompt 45.0 / 55.1 against 29.9 / 37.9
// us (29.9 against 45.1 at 32 / 8 heads), 2 x (2048 positions, 512 new) at
// 32 / 8 heads 76.9 against 68.2; 512 new over 1536 / 2048 / 4096
// positions 45.8 / 53.3 / 76.2 against 52.2 / 68.4 / 131.3, 256 over 2048
// 39.5 against 68.2, 1024 over 8192 198.2 against 255.7.
// Workspace bytes of the persistent grid's claim counters (8 used).
constexpr size_t kClaimBytes = 256;

// Workgroups of a prefill kernel resident at once on the current device:
// its occupancy per CU (2 at head_dim 128 and 256, 3 at 64: registers and
// LDS) times the CU count, both read once per (kernel, device).
int64_t prefill_slots(const void* kernel) {
    static std::mutex mu;
    static std::map<std::pair<const void*, int>, int64_t> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lock(mu);
    const auto key = std::make_pair(kernel, dev);
    const auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    int cus = 0, occ = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, kThreads, 0) != hipSuccess || occ <= 0) return 0;
    return cache[key] = (int64_t)cus * occ;
}

struct SplitPlan {
    int32_t row_tiles;
    int32_t num_parts;
    int32_t tiles_per_part;
    size_t ml_bytes;
    size_t total;
};

SplitPlan split_plan(int32_t num_tokens, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                     int32_t head_dim, int64_t len_cap, int32_t max_query_len) {
    SplitPlan P{};
    const HostGeo hg = host_geo(head_dim);
    const int64_t g = num_heads / num_kv_heads;
    P.row_tiles = (int32_t)(((int64_t)max_query_len * g + hg.rows_per_group - 1) / hg.rows_per_group);
    // contexts shorter than a few tiles are not worth splitting (parts of at
    // least 256 tokens)
    const int64_t max_tiles = len_cap / hg.kv_tile + 1;
    const int64_t min_tiles_per_part = 256 / hg.kv_tile;
    const int64_t wgs = (int64_t)num_kv_heads * num_seqs * P.row_tiles;
    int64_t parts = 1;
    const int64_t mq = max_query_len > 0 ? max_query_len : 1;
    const bool long_context = len_cap >= 8 * mq || (len_cap >= 2 * mq && 4 * wgs <= 512);
    if (wgs > 0 && 2 * wgs <= 512 && max_tiles >= 2 * min_tiles_per_part && long_context) {
        parts = 512 / wgs;
        if (parts > max_tiles / min_tiles_per_part) parts = max_tiles / min_tiles_per_part;
        if (parts * P.row_tiles > 65535) parts = 65535 / P.row_tiles;
        if (parts < 1) parts = 1;
    }
    P.tiles_per_part = (int32_t)((max_tiles + parts - 1) / parts);
    P.num_parts = (int32_t)((max_tiles + P.tiles_per_part - 1) / P.tiles_per_part);
    if (P.num_parts <= 1) {
        P.num_parts = 1;
        // more workgroups than half a round: the claim counters of the
        // persistent grid
        if (wgs > 256) P.total = kClaimBytes;
        return P;
    }
    const size_t rows = (size_t)num_tokens * num_heads * P.num_parts;
    P.ml_bytes = align_up(rows * 2 * sizeof(float), 256);
    P.total = P.ml_bytes + align_up(rows * head_dim * sizeof(float), 256);
    return P;
}

}  // namespace

extern "C" size_t pa_prefill_workspace_size(int32_t num_tokens, int32_t num_seqs, int32_t num_heads,
                                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                            int32_t max_blocks_per_seq, int32_t max_query_len) {
    if (!pick<false, false>(head_dim, block_size) || num_tokens < 0 || num_seqs < 0 || num_heads <= 0 ||
        num_kv_heads <= 0 || num_heads % num_kv_heads != 0 || max_blocks_per_seq < 0 || max_query_len < 0)
        return (size_t)-1;
    return split_plan(num_tokens, num_seqs, num_heads, num_kv_heads, head_dim,
                      (int64_t)max_blocks_per_seq * block_size, max_query_len)
        .total;
}

namespace {

// The new tokens' K/V when pa_prefill_append folds their write into the
// call (null otherwise).
struct PrefillAppend {
    const _Float16* key;
    const _Float16* value;
    int64_t stride;
};

int prefill_impl(const char* fn, void* out, const void* q, int32_t num_tokens, const void* k_cache,
                 const void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                 const int32_t* context_lens, const int32_t* query_start, int32_t num_seqs, int32_t num_heads,
                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                 int32_t max_query_len, void* workspace, size_t workspace_bytes, const int32_t* seq_order,
                 int32_t dtype, void* stream, const PrefillAppend* app) {
    if (dtype != PA_DTYPE_F16) return pa::fail(PA_ERR_UNSUPPORTED, "%s: dtype %d", fn, dtype);
    if (head_dim != 64 && head_dim != 128 && head_dim != 256)
        return pa::fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d (64, 128 or 256)", fn, head_dim);
    if (!pick<false, false>(head_dim, block_size))
        return pa::fail(PA_ERR_UNSUPPORTED, "%s: block_size %d", fn, block_size);
    if (num_seqs < 0 || num_tokens < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 ||
        num_blocks <= 0 || max_blocks_per_seq < 0 || max_query_len < 0)
        return pa::fail(PA_ERR_INVALID, "%s: bad sizes (S=%d H=%d Hkv=%d NB=%d W=%d max_q=%d)", fn, num_seqs,
                        num_heads, num_kv_heads, num_blocks, max_blocks_per_seq, max_query_len);
    if (num_seqs > 65535 || num_kv_heads > 65535 || num_heads > 65535)
        return pa::fail(PA_ERR_INVALID, "%s: num_seqs and the head counts must be <= 65535", fn);
    if (!std::isfinite(scale)) return pa::fail(PA_ERR_INVALID, "%s: scale is not finite", fn);
    if (num_seqs == 0 || max_query_len == 0 || num_tokens == 0) return PA_OK;
    if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
        return pa::fail(PA_ERR_INVALID, "%s: null pointer", fn);
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
        return pa::fail(PA_ERR_INVALID, "%s: out, q and caches must be 16-byte aligned", fn);
    if (workspace && !aligned16(workspace))
        return pa::fail(PA_ERR_INVALID, "%s: workspace must be 16-byte aligned", fn);
    if (app) {
        if (!app->key || !app->value) return pa::fail(PA_ERR_INVALID, "%s: null key or value", fn);
        if (!aligned16(app->key) || !aligned16(app->value) || app->stride % 8 != 0)
            return pa::fail(PA_ERR_INVALID, "%s: key, value and kv_token_stride must be 16-byte aligned", fn);
        if (app->stride < (int64_t)num_kv_heads * head_dim)
            return pa::fail(PA_ERR_INVALID, "%s: kv_token_stride %lld < num_kv_heads * head_dim", fn,
                            (long long)app->stride);
    }
    const int64_t g = num_heads / num_kv_heads;
    const HostGeo hg = host_geo(head_dim);
    const int64_t row_tiles = ((int64_t)max_query_len * g + hg.rows_per_group - 1) / hg.rows_per_group;
    if (row_tiles > 65535)
        return pa::fail(PA_ERR_INVALID, "%s: max_query_len %d x %lld heads needs %lld row tiles (limit 65535)",
                        fn, max_query_len, (long long)g, (long long)row_tiles);
    const int64_t len_cap = (int64_t)max_blocks_per_seq * block_size;
    if (pa::validate_enabled()) {
        if (int rc = pa::validate_queries(fn, query_start, num_seqs, num_tokens, context_lens, max_query_len, stream))
            return rc;
        if (int rc = pa::validate_tables(fn, block_tables, max_blocks_per_seq, context_lens, num_seqs, block_size,
                                         num_blocks, len_cap, stream))
            return rc;
    }
    SplitPlan P = split_plan(num_tokens, num_seqs, num_heads, num_kv_heads, head_dim, len_cap, max_query_len);
    if (P.num_parts > 1 && (!workspace || workspace_bytes < P.total)) {
        // no room for the partial states: one part per row tile
        P.num_parts = 1;
        P.tiles_per_part = (int32_t)(len_cap / hg.kv_tile + 1);
    }
    float* ws_ml = P.num_parts > 1 ? static_cast<float*>(workspace) : nullptr;
    float* ws_acc = P.num_parts > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + P.ml_bytes) : nullptr;
    const float scale_log2 = (float)((double)scale * kLog2e);
    auto st = static_cast<hipStream_t>(stream);
    // one row tile per (KV head, sequence): each K/V tile is read once, so
    // stream it past the caches (measured on 4 x 8192 cached + 32 new: 106
    // against 125 us); several row tiles re-read it (prompts: 233 against 245
    // us with nontemporal loads)
    const bool stream_kv = row_tiles == 1;
    const int64_t pairs = (int64_t)num_kv_heads * num_seqs;
    const int64_t items = pairs * row_tiles * P.num_parts;
    if (items > 0x7fffffff) return pa::fail(PA_ERR_INVALID, "%s: %lld workgroups (limit 2^31 - 1)", fn,
                                               (long long)items);
    PrefillFn fn_main =
        app ? (stream_kv ? pick<true, true>(head_dim, block_size) : pick<false, true>(head_dim, block_size))
            : (stream_kv ? pick<true, false>(head_dim, block_size) : pick<false, false>(head_dim, block_size));
    // persistent grid: more items than one round of resident workgroups, one
    // query head per KV head, at least 1024 query rows per (KV head,
    // sequence) -- 8 row tiles up to head_dim 128, 16 at 256 -- and room for
    // the claim counters (an unsplit call's workspace).  Measured against one
    // workgroup per item (pa_prefill, Llama-2-7B heads): 32 x 1024-token
    // prompts +13%, 16 x 2048 +8%, 8 x 4096 +3.5%, 4 x 8192 +1% (+7% / +10%
    // at 1024 tokens and head_dim 256 / 64); on the short-prompt mix (at
    // most 774 tokens, many row tiles past a prompt's end) -2 to -4% at
    // head_dim 128, -1.5% at 256, -37% at 64, so fewer rows keep one
    // workgroup per item.  With several query heads per KV head it never
    // gained: 32 / 8 heads 0 to -1% on 1024-8192-token prompts, -3 to -7% on
    // 256-774-token ones, 64 / 8 heads -1.4% on 32 x 1024.
    unsigned* claim = nullptr;
    int64_t grid = items;
    if (P.num_parts == 1 && g == 1 && row_tiles * hg.rows_per_group >= 1024 && workspace &&
        workspace_bytes >= kClaimBytes) {
        const PrefillFn fn_p = app ? pick_persistent<true>(head_dim, block_size) : pick_persistent<false>(head_dim, block_size);
        const int64_t slots = prefill_slots(reinterpret_cast<const void*>(fn_p)) / 8 * 8;
        if (slots >= 8 && items > slots) {
            claim = static_cast<unsigned*>(workspace);
            grid = slots;
            fn_main = fn_p;
        }
    }
    // the cache pointers double as write pointers in append mode: the kernel
    // writes only the new tokens' rows, which no workgroup reads from the
    // cache
    if (claim) {
        hipLaunchKernelGGL(prefill_claim_reset, dim3(1), dim3(64), 0, st, claim);
        const hipError_t e0 = hipGetLastError();
        if (e0 != hipSuccess) return pa::fail(PA_ERR_HIP, "%s: %s", fn, hipGetErrorString(e0));
    }
    hipLaunchKernelGGL(fn_main, dim3((unsigned)grid),
                       dim3(kThreads), 0, st, static_cast<_Float16*>(out), static_cast<const _Float16*>(q), num_tokens,
                       static_cast<const _Float16*>(k_cache), static_cast<const _Float16*>(v_cache), block_tables,
                       max_blocks_per_seq, context_lens, query_start, num_heads, num_kv_heads, num_blocks, scale_log2,
                       max_query_len, len_cap, ws_ml, ws_acc, P.tiles_per_part, P.num_parts, num_seqs,
                       (int32_t)row_tiles, (int32_t)(pairs % 8 == 0), app ? app->key : nullptr,
                       app ? app->value : nullptr, app ? app->stride : (int64_t)0,
                       app ? static_cast<_Float16*>(const_cast<void*>(k_cache)) : nullptr,
                       app ? static_cast<_Float16*>(const_cast<void*>(v_cache)) : nullptr, claim, seq_order);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return pa::fail(PA_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
    if (P.num_parts > 1) {
        hipLaunchKernelGGL(pick_merge(head_dim),
                           dim3((unsigned)num_heads, (unsigned)num_seqs,
                                (unsigned)merge_grid_z(max_query_len, head_dim)),
                           dim3((unsigned)kMergeThreads), 0, st, static_cast<_Float16*>(out), (const float*)ws_ml,
                           (const float*)ws_acc,
                           num_tokens, context_lens, query_start, num_heads, num_kv_heads, max_query_len, len_cap,
                           P.tiles_per_part, P.num_parts, seq_order);
        e = hipGetLastError();
        if (e != hipSuccess) return pa::fail(PA_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
    }
    return PA_OK;
}

}  // namespace

extern "C" int pa_prefill(void* out, const void* q, int32_t num_tokens, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                          const int32_t* query_start, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                          int32_t max_query_len, void* workspace, size_t workspace_bytes,
                          const int32_t* seq_order, int32_t dtype, void* stream) {
    return prefill_impl("pa_prefill", out, q, num_tokens, k_cache, v_cache, block_tables, max_blocks_per_seq,
                        context_lens, query_start, num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                        scale, max_query_len, workspace, workspace_bytes, seq_order, dtype, stream, nullptr);
}

extern "C" int pa_prefill_append(void* out, const void* q, int32_t num_tokens, const void* key, const void* value,
                                 int64_t kv_token_stride, void* k_cache, void* v_cache, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens, const int32_t* query_start,
                                 int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t num_blocks, float scale, int32_t max_query_len,
                                 void* workspace, size_t workspace_bytes, const int32_t* seq_order, int32_t dtype,
                                 void* stream) {
    const PrefillAppend app{static_cast<const _Float16*>(key), static_cast<const _Float16*>(value), kv_token_stride};
    return prefill_impl("pa_prefill_append", out, q, num_tokens, k_cache, v_cache, block_tables, max_blocks_per_seq,
                        context_lens, query_start, num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                        scale, max_query_len, workspace, workspace_bytes, seq_order, dtype, stream, &app);
}

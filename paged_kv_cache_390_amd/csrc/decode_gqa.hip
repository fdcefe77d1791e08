// Grouped-query paged decode attention on the CDNA4 matrix cores (gfx950).
//
// What is computed is the same as for every other pa_decode shape: each
// query head attends to its sequence's n cached keys/values through the
// block table, textbook softmax attention over the logically contiguous K/V
// (lpnh.cn/news/1824136, 2.2 and 3.2 step 4; lpnh.cn/news/2758356, 2.1 for
// the KV-head dimension of a block).  This kernel serves the case where g =
// num_heads / num_kv_heads query heads share one KV head (2 <= g <= 16,
// head_dim 64, 128 or 256): then every K/V element read from HBM meets g
// queries, and the two products are small dense contractions,
//     S^T[t, q] = sum_d K[t, d] Q[q, d]        (16 tokens x 16 queries x D)
//     O[q, d]  += sum_t P[q, t] V[t, d]         (16 queries x D x 16 tokens)
// which run on the matrix cores (fp16 inputs, fp32 accumulation): QK on
// v_mfma_f32_16x16x32_f16 (D / 32 per tile), PV on v_mfma_f32_16x16x16_f16
// (D / 16 per tile, one per 16 output columns).  The kernel is still
// HBM-bound: about 4g flops per 2 bytes of K/V, far below the matrix cores'
// ridge, so the design serves the loads.
//
// Layout (one 256-thread workgroup = 4 wave64s per (KV head, sequence,
// context partition); KV head fastest in the grid so every XCD streams the
// same bytes; a wave step is one 16-token tile, steps dealt round-robin to
// the waves, kFlight tiles in flight per wave when a tile lies in one
// block).  Lane l = n + 16j (n = l % 16, j = l / 16):
//  * MFMA lane layouts (checked on the GPU against a host product):
//    16x16x32: A[m][k] in lane m + 16*(k/8) (8 halves), B[k][n] in lane
//    n + 16*(k/8); 16x16x16: A[m][k] in lane m + 16*(k/4), B[k][n] in lane
//    n + 16*(k/4); both: C[m][n] in lane n + 16*(m/4).
//  * QK: A = K tile (m = token), B = Q^T (n = query head of the group,
//    zero-padded past g).  The contraction index of MFMA c is mapped onto
//    head_dim 32c + 8j .. +7 in lane (m, j): one 16-byte load of token m's
//    row per MFMA operand, no register shuffles (at head_dim 64 the tile is
//    read as whole rows instead and moved into this layout through LDS).
//  * S^T lands with lane (n, j) holding tokens 4j..4j+3 of query n: exactly
//    the A-operand layout of P for the 16x16x16 PV product, so the online
//    softmax (running max / sum per query, base 2, log2(e) folded into the
//    scale) runs in place and P goes to the matrix core as fp16.
//  * PV: B = V tile.  Output column n of d-tile c is d = (D/16)*n + c up to
//    head_dim 128, so lane (n, j) loads the D/16 contiguous values d =
//    (D/16)*n .. of tokens 4j..4j+3 (8 or 16 bytes per token: one load of
//    the 16 lanes reads the V row whole), and element c of the four tokens
//    is the B operand of d-tile c.  At head_dim 256 the lane's 16 values are
//    two runs of 8, d = 128*(c/8) + 8n + c%8 (vcol), so that each of its two
//    16-byte loads per token reads one contiguous half of the row across the
//    16 lanes; with one run of 16 values each load read 16-byte pieces 32
//    bytes apart and the call took 189-193 us instead of 175-177 (128
//    sequences at g = 8).
//  * Masking by select: a token past the context, or behind a table entry
//    outside the pool, gets S = -inf and V = 0, so NaN in unused rows cannot
//    reach the sums (0 * NaN would).
//  * Normalisation uses the same fp16-rounded weights the matrix core saw,
//    so each output is an exact convex combination of V rows up to fp32
//    rounding.
//  * The 4 waves' (m, l, O) are merged through LDS (in one round up to
//    head_dim 128, as a tree at 256); rows split over several partitions
//    leave (m, l, O) in the workspace for the shared reduce kernel, in the
//    same layout as the one-query-per-KV-head kernel.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "decode_internal.h"

namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kTile = 16;              // tokens per wave step

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ half8_t as_h8(u32x4 u) { return __builtin_bit_cast(half8_t, u); }

// Per head_dim: QK MFMAs (= K loads of 16 bytes per lane) per tile, V values
// per lane and token (= PV d-tiles), and tiles in flight per wave beside the
// one being consumed (a tile is D/4 VGPRs, O D/4, Q^T D/8: at head_dim 64
// two, so that four workgroups fit a CU; above, what the 256 VGPRs of two
// waves per SIMD leave).
template <int D>
struct Geo {
    static constexpr int kQk = D / 32;
    static constexpr int kVpl = D / 16;
    static constexpr int kDT = D / 16;
    static constexpr int kVDw = kVpl / 2;            // dwords of V per lane and token
    static constexpr int kFlight = D == 64 ? 2 : D == 128 ? 3 : 1;
    // head_dim 256: the Q^T operands (D/8 VGPRs) are read from LDS for each
    // tile instead of held, so that two waves fit a SIMD
    static constexpr bool kQInLds = D >= 256;
    // head_dim 64: K is read with adjacent lanes contiguous (kLpt lanes per
    // token row, whole 128-byte rows per load) and moved into the QK operand
    // layout (token lane % 16, 16 bytes per lane group) through the wave's
    // LDS slice.  Read in the operand layout, each load took 64 bytes of 16
    // rows, the other half of each line falling to the next load: 176.4 ->
    // 169.9 us per call on 512 sequences (mean of six runs in turn).  At 128
    // the same read gained nothing; at 256 its addresses spilled registers.
    static constexpr bool kKLds = D == 64;
    static constexpr int kLpt = D / 8;
    static constexpr int kQPitch = D + 8;            // halves per staged Q row (16 bytes of padding)
};

// The Q^T operands of the lane's query row: held in registers, or read
// from the workgroup's staged copy in LDS.
template <int D, bool kLds = Geo<D>::kQInLds>
struct QOperands;

template <int D>
struct QOperands<D, false> {
    half8_t v[Geo<D>::kQk];
    __device__ __forceinline__ half8_t operator[](int c) const { return v[c]; }
};

typedef __attribute__((address_space(3))) const half8_t* lds_half8_ptr;

template <int D>
struct QOperands<D, true> {
    uint32_t addr;                           // LDS byte address of this lane's query row, at d = 8j
    __device__ __forceinline__ half8_t operator[](int c) const {
        // the empty asm hides the address from loop-invariant code motion,
        // which would otherwise hoist the reads out of the tile loop and hold
        // the operands in registers after all; the address stays an LDS one
        uint32_t a = addr + 64u * (uint32_t)c;
        asm volatile("" : "+v"(a));
        return *reinterpret_cast<lds_half8_ptr>((size_t)a);
    }
};

// One 16-token tile as this lane holds it.
template <int D>
struct Tile {
    u32x4 k[Geo<D>::kQk];                   // K row (token n), d = 32c + 8j .. +7
    uint32_t v[4][Geo<D>::kVDw];            // V rows (tokens 4j + i), d = vcol(n, c) for c = 0 .. kVpl-1
    bool valid[4];                          // tokens 4j + i: inside the context and the pool
};

template <int D>
struct Softmax {
    float m, l;                             // running max (base 2) and sum of query n
    float4_t o[Geo<D>::kDT];                // O[query 4j + i][d = vcol(n, c)] in o[c][i]
};

// Head-dim index of PV output column n of d-tile c.  Up to head_dim 128 a
// lane's kVpl values are contiguous, d = kVpl*n + c: one load per token
// covers the whole row across the 16 lanes.  At 256 they are two runs of
// 8, d = 128*(c/8) + 8n + c%8, so that each 16-byte load of the 16 lanes
// reads one contiguous 256-byte half of the row; with one run of 16 each
// load would read 16-byte pieces 32 bytes apart, touching every cache line
// of the row in both loads.
template <int D>
__device__ __forceinline__ int vcol(int n, int c) {
    if constexpr (D >= 256) return 128 * (c / 8) + 8 * n + (c % 8);
    else return Geo<D>::kVpl * n + c;
}

template <int D>
__device__ __forceinline__ void load_v_row(uint32_t (&dst)[Geo<D>::kVDw], const _Float16* row, int n) {
    if constexpr (Geo<D>::kVDw == 2) {
        const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(row + vcol<D>(n, 0)));
        dst[0] = x[0];
        dst[1] = x[1];
    } else {
#pragma unroll
        for (int w = 0; w < Geo<D>::kVDw / 4; ++w) {
            const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + vcol<D>(n, 8 * w)));
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[4 * w + e] = x[e];
        }
    }
}

// Tile loads when a tile lies inside one block (B >= 16): `phys` is the
// block's table entry, read ahead by the caller with a scalar load.  Rows
// past the context read the context's last row again (the same cache lines:
// no extra HBM bytes) and are masked later.
template <int D, int B>
__device__ __forceinline__ void load_tile_block(Tile<D>& t, int t0, int end, int32_t phys,
                                                const _Float16* __restrict__ kbase,
                                                const _Float16* __restrict__ vbase, int64_t blk_stride,
                                                int32_t num_blocks, int lane) {
    using G = Geo<D>;
    const int n = lane & 15;
    const int j = lane >> 4;
    const bool ok = (uint32_t)phys < (uint32_t)num_blocks;
    const int64_t base = (int64_t)(ok ? phys : 0) * blk_stride + (int64_t)(t0 % B) * D;
    const int lim = end - 1 - t0;
    if constexpr (G::kKLds) {
        // load c: token c*(64/kLpt) + lane/kLpt, 16-byte chunk lane % kLpt
#pragma unroll
        for (int c = 0; c < G::kQk; ++c) {
            const int tk = c * (64 / G::kLpt) + lane / G::kLpt;
            const int rk = tk < lim ? tk : lim;
            t.k[c] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(kbase + base + rk * D + 8 * (lane % G::kLpt)));
        }
    } else {
        const int rk = n < lim ? n : lim;
#pragma unroll
        for (int c = 0; c < G::kQk; ++c)
            t.k[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + base + rk * D + 32 * c + 8 * j));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rv = 4 * j + i < lim ? 4 * j + i : lim;
        t.valid[i] = ok && t0 + 4 * j + i < end;
        load_v_row<D>(t.v[i], vbase + base + rv * D, n);
    }
}

// Tile loads when a tile spans several blocks (B < 16): every row looks up
// its own table entry.
template <int D, int B>
__device__ __forceinline__ void load_tile_rows(Tile<D>& t, int t0, int end, const int32_t* __restrict__ trow,
                                               const _Float16* __restrict__ kbase,
                                               const _Float16* __restrict__ vbase, int64_t blk_stride,
                                               int32_t num_blocks, int lane) {
    using G = Geo<D>;
    const int n = lane & 15;
    const int j = lane >> 4;
    {
        const int tk = t0 + n;
        const int tc = tk < end ? tk : end - 1;        // keeps the table index inside the sequence
        const int32_t phys = trow[tc / B];
        const bool ok = (uint32_t)phys < (uint32_t)num_blocks;
        const int64_t row = (int64_t)(ok ? phys : 0) * blk_stride + (int64_t)(tc % B) * D;
#pragma unroll
        for (int c = 0; c < G::kQk; ++c)
            t.k[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + row + 32 * c + 8 * j));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int tv = t0 + 4 * j + i;
        const int tc = tv < end ? tv : end - 1;
        const int32_t phys = trow[tc / B];
        const bool ok = (uint32_t)phys < (uint32_t)num_blocks;
        t.valid[i] = tv < end && ok;
        const int64_t row = (int64_t)(ok ? phys : 0) * blk_stride + (int64_t)(tc % B) * D;
        load_v_row<D>(t.v[i], vbase + row, n);
    }
}

// keep[i]: token 4j + i takes part (inside the context and the pool);
// t.valid[i]: its V row holds data (zeroed by select otherwise).
// kKRows: t.k holds K as load_tile_block reads it when Geo<D>::kKLds
// (whole rows); it goes through the wave's LDS slice `kslice` into the
// operand layout first.
template <int D, bool kKRows = false>
__device__ __forceinline__ void consume_tile(Softmax<D>& st, Tile<D>& t, const QOperands<D>& qb,
                                             float scale_log2, int lane, u32x4* kslice = nullptr) {
    using G = Geo<D>;
    const int j = lane >> 4;
    if constexpr (kKRows) {
        // t.k[c] holds token c*(64/kLpt) + lane/kLpt, chunk lane % kLpt: into
        // the slice (chunk q of token r at position q ^ (r % kLpt), so that the
        // 16 tokens of one operand read fall in distinct banks), then back as
        // MFMA c's operand: token lane % 16, chunk 4c + j
#pragma unroll
        for (int c = 0; c < G::kQk; ++c) {
            const int r = c * (64 / G::kLpt) + lane / G::kLpt;
            const int q = lane % G::kLpt;
            kslice[r * G::kLpt + (q ^ (r & (G::kLpt - 1)))] = t.k[c];
        }
        const int m = lane & 15;
#pragma unroll
        for (int c = 0; c < G::kQk; ++c) t.k[c] = kslice[m * G::kLpt + ((4 * c + j) ^ (m & (G::kLpt - 1)))];
    }
    // S^T = K Q^T: lane holds S^T[token 4j+i][query n]
    float4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < G::kQk; ++c) s = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(t.k[c]), qb[c], s, 0, 0, 0);
    // online softmax of query n over the tile's 16 tokens (4 per lane, 4 lanes)
    float sc[4];
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        sc[i] = t.valid[i] ? s[i] * scale_log2 : -INFINITY;
        mt = fmaxf(mt, sc[i]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(st.m, mt);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(st.m - m_use);
    half4_t p;
    float lt = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p[i] = (_Float16)fast_exp2(sc[i] - m_use);
        lt += (float)p[i];                     // the weights the matrix core sees
    }
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    st.l = st.l * alpha + lt;
    st.m = m_new;
    // Rescale O rows (queries 4j+i) by their query's alpha, held by lane
    // 4j+i -- only when some running max moved: once the maxima settle most
    // tiles skip it, and skipping a multiply by exactly 1 changes no bit.
    if (__any(alpha != 1.f)) {
        float ar[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * j + i);
#pragma unroll
        for (int c = 0; c < G::kDT; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) st.o[c][i] *= ar[i];
    }
    // O += P V per d-tile.  Rows of masked tokens may hold anything (NaN in
    // an unused tail row): in a tile with any masked row they are zeroed by
    // select first (in the tile's own registers, which are reloaded next),
    // since a zero weight times NaN is still NaN.
    if (!__all(t.valid[0] && t.valid[1] && t.valid[2] && t.valid[3])) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int w = 0; w < G::kVDw; ++w) t.v[i][w] = t.valid[i] ? t.v[i][w] : 0u;
    }
#pragma unroll
    for (int c = 0; c < G::kDT; ++c) {
        half4_t b;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w = t.v[i][c / 2];
            b[i] = __builtin_bit_cast(_Float16, (uint16_t)((c & 1) ? w >> 16 : w & 0xffffu));
        }
        st.o[c] = __builtin_amdgcn_mfma_f32_16x16x16f16(p, b, st.o[c], 0, 0, 0);
    }
}

// kAppend: the last position n - 1 of every sequence holds the token of
// this step, whose K/V come from new_k / new_v (token s, KV head h at s *
// new_stride + h * D) instead of the cache; the workgroup whose partition
// holds it folds it in as a one-token tile and writes it into the cache
// through k_write / v_write.  The cache is read for positions < n - 1 only.
// Workgroups per CU: 4 at head_dim 64 (two tiles in flight per wave, ~120
// VGPRs: more resident workgroups hide each one's start and drain better
// than deeper pipelines -- 8 tiles in flight at 2 workgroups per CU ran 11-14%
// slower), 2 at 128 (3 tiles in flight; 1 tile at 3 workgroups per CU
// measured within 1%), 2 at 256 with tiles in one block, 1 otherwise.
template <int D, int B, bool kAppend>
__global__ void __launch_bounds__(kThreads, D == 64 ? 4 : (D >= 256 && B < kTile) ? 1 : 2)
decode_gqa_mfma_kernel(_Float16* __restrict__ out, float* __restrict__ ws_ml, float* __restrict__ ws_acc,
                       const int32_t* __restrict__ order, const _Float16* __restrict__ q, const _Float16* __restrict__ k_cache,
                       const _Float16* __restrict__ v_cache, const int32_t* __restrict__ tables,
                       int32_t max_blocks, const int32_t* __restrict__ lens, int32_t num_heads,
                       int32_t num_kv_heads, int32_t num_blocks, float scale_log2, int32_t part_size,
                       int32_t num_parts, int64_t len_cap, const _Float16* __restrict__ new_k,
                       const _Float16* __restrict__ new_v, int64_t new_stride, _Float16* __restrict__ k_write,
                       _Float16* __restrict__ v_write) {
    using G = Geo<D>;
    const int kvh = blockIdx.x;
    const int s = order ? order[blockIdx.y] : (int)blockIdx.y;   // longest sequences first
    if ((uint32_t)s >= gridDim.y) return;                         // not a sequence: nothing to do
    const int part = blockIdx.z;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = num_heads / num_kv_heads;
    const int nl = lane & 15;
    const int jl = lane >> 4;

    const int32_t n_raw = lens[s];
    const bool bad_len = n_raw < 0 || (int64_t)n_raw > len_cap;
    const int n = bad_len ? 0 : n_raw;
    const int start = part * part_size;
    if (part > 0 && start >= n) return;
    const int cached = kAppend && n > 0 ? n - 1 : n;   // positions read from the cache
    const int end = min(start + part_size, cached);
    const int np = (n + part_size - 1) / part_size;

    // Q^T operands of query head kvh*g + n (zero past g): MFMA c takes
    // d = 32c + 8j .. +7
    QOperands<D> qb;
    const _Float16* qgroup = q + ((int64_t)s * num_heads + (int64_t)kvh * g) * D;
    if constexpr (G::kQInLds) {
        __shared__ __attribute__((aligned(16))) _Float16 s_q[16 * G::kQPitch];
        for (int idx = threadIdx.x; idx < 16 * (D / 8); idx += kThreads) {
            const int qi = idx / (D / 8);
            const int ch = idx - qi * (D / 8);
            const u32x4 z = {0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(s_q + qi * G::kQPitch + 8 * ch) =
                qi < g ? *reinterpret_cast<const u32x4*>(qgroup + (int64_t)qi * D + 8 * ch) : z;
        }
        __syncthreads();
        qb.addr = (uint32_t)(size_t)(__attribute__((address_space(3))) const _Float16*)(s_q + nl * G::kQPitch +
                                                                                         8 * jl);
    } else {
        const bool live = nl < g;
        const _Float16* qrow = qgroup + (int64_t)(live ? nl : 0) * D;
#pragma unroll
        for (int c = 0; c < G::kQk; ++c) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            qb.v[c] = as_h8(live ? *reinterpret_cast<const u32x4*>(qrow + 32 * c + 8 * jl) : z);
        }
    }

    const int32_t* trow = tables + (int64_t)s * max_blocks;
    const int64_t slab = (int64_t)B * D;
    const _Float16* kbase = k_cache + (int64_t)kvh * slab;
    const _Float16* vbase = v_cache + (int64_t)kvh * slab;
    const int64_t blk_stride = (int64_t)num_kv_heads * slab;

    Softmax<D> st;
    st.m = -INFINITY;
    st.l = 0.f;
#pragma unroll
    for (int c = 0; c < G::kDT; ++c) st.o[c] = float4_t{0.f, 0.f, 0.f, 0.f};

    // append mode: the workgroup whose partition holds position n - 1 loads
    // the new token's K and V rows now (lane i < D/8: K chunk i, the next D/8
    // lanes the V chunks), issued ahead of the first tiles so that its
    // latency hides under theirs, and parks them in LDS once those are
    // issued: no registers are held through the main loop
    __shared__ __attribute__((aligned(16))) unsigned char s_new[64 * 16];
    const int pos_new = n - 1;
    const bool holds_new = kAppend && n > 0 && pos_new >= start && pos_new < start + part_size;
    const bool new_wave = holds_new && wave == kWaves - 1;
    u32x4 new_row = {0u, 0u, 0u, 0u};
    if constexpr (kAppend) {
        constexpr int kChunks = D / 8;
        if (new_wave && lane < 2 * kChunks) {
            const _Float16* src = lane < kChunks ? new_k + (int64_t)s * new_stride + (int64_t)kvh * D + 8 * lane
                                                 : new_v + (int64_t)s * new_stride + (int64_t)kvh * D +
                                                       8 * (lane - kChunks);
            new_row = *reinterpret_cast<const u32x4*>(src);
        }
    }
    auto park_new = [&]() {
        if constexpr (kAppend)
            if (new_wave && lane < 2 * (D / 8)) *reinterpret_cast<u32x4*>(s_new + 16 * lane) = new_row;
    };

    const int ntok = end > start ? end - start : 0;
    const int nsteps = (ntok + kTile - 1) / kTile;
    __shared__ u32x4 s_kt[kWaves][G::kKLds ? 16 * G::kLpt : 1];   // each wave's K slice (head_dim 64)
    u32x4* kslice = s_kt[wave];
    if (wave < nsteps) {
        if constexpr (B >= kTile) {
            // One table entry per tile, read with scalar loads a tile ahead of
            // its issue; kFlight tiles in flight per wave beside the one being
            // consumed (kFlight + 1 buffers rotate).  Every step issues a tile
            // -- past the last step one that is never consumed, every lane
            // reading the same bytes of the last tile's block (one cache line
            // per load) -- so the count of loads is the same on every path and
            // the wait before a consume leaves the newer tiles in flight.
            constexpr int NF = G::kFlight;
            Tile<D> buf[NF + 1];
            auto clamp = [&](int stp) { return stp < nsteps ? stp : nsteps - 1; };
            auto entry = [&](int stp) { return trow[(start + clamp(stp) * kTile) / B]; };
            auto issue = [&](Tile<D>& t, int stp, int32_t phys) {
                load_tile_block<D, B>(t, start + clamp(stp) * kTile, end, phys, kbase, vbase, blk_stride, num_blocks,
                                      stp < nsteps ? lane : 0);
            };
            int stp = wave;
#pragma unroll
            for (int r = 0; r < NF; ++r) issue(buf[r], stp + r * kWaves, entry(stp + r * kWaves));
            park_new();
            int32_t tnext = entry(stp + NF * kWaves);
            // The loads of every step are issued unconditionally and the exit
            // test follows the consume (loads under a branch would make the
            // compiler wait for all of them before each consume).
            for (;;) {
#pragma unroll
                for (int r = 0; r < NF + 1; ++r) {
                    // the tile NF steps ahead goes into the buffer consumed last
                    const int32_t cur = tnext;
                    tnext = entry(stp + (NF + 1) * kWaves);
                    issue(buf[(r + NF) % (NF + 1)], stp + NF * kWaves, cur);
                    consume_tile<D, G::kKLds>(st, buf[r], qb, scale_log2, lane, kslice);
                    stp += kWaves;
                    if (stp >= nsteps) goto walked;
                }
            }
        walked:;
        } else {
            Tile<D> A, Bt;
            int stp = wave;
            load_tile_rows<D, B>(A, start + stp * kTile, end, trow, kbase, vbase, blk_stride, num_blocks, lane);
            park_new();
            for (;;) {
                int nx = stp + kWaves;
                if (nx >= nsteps) { consume_tile<D>(st, A, qb, scale_log2, lane); break; }
                load_tile_rows<D, B>(Bt, start + nx * kTile, end, trow, kbase, vbase, blk_stride, num_blocks, lane);
                consume_tile<D>(st, A, qb, scale_log2, lane);
                stp = nx;
                nx = stp + kWaves;
                if (nx >= nsteps) { consume_tile<D>(st, Bt, qb, scale_log2, lane); break; }
                load_tile_rows<D, B>(A, start + nx * kTile, end, trow, kbase, vbase, blk_stride, num_blocks, lane);
                consume_tile<D>(st, Bt, qb, scale_log2, lane);
                stp = nx;
            }
        }
    }

    if constexpr (kAppend) {
        if (new_wave) {
            if (wave >= nsteps) park_new();       // a wave without tiles parks the row here
            const int32_t phys = trow[pos_new / B];
            const bool ok = (uint32_t)phys < (uint32_t)num_blocks;   // as a cached row behind a skipped id
            const u32x4 z = {0u, 0u, 0u, 0u};
            Tile<D> t;
            // K row of token n (d = 32c + 8j ..): token 0 only
#pragma unroll
            for (int c = 0; c < G::kQk; ++c)
                t.k[c] = nl == 0 ? *reinterpret_cast<const u32x4*>(s_new + 16 * (4 * c + jl)) : z;
            // V rows of tokens 4j + i (d = vcol(n, c)): token 0 is i = 0 of lane group 0
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int w = 0; w < G::kVDw; ++w)
                    t.v[i][w] = i == 0 && jl == 0
                                    ? *reinterpret_cast<const uint32_t*>(s_new + 2 * D + 2 * vcol<D>(nl, 2 * w))
                                    : 0u;
#pragma unroll
            for (int i = 0; i < 4; ++i) t.valid[i] = ok && jl == 0 && i == 0;
            consume_tile<D>(st, t, qb, scale_log2, lane);
            if (ok && lane < 2 * (D / 8)) {
                // the staged row goes to the cache: lane i < D/8 writes K chunk
                // i, the next D/8 lanes the V chunks
                const int64_t row = (int64_t)kvh * slab + (int64_t)phys * blk_stride + (int64_t)(pos_new % B) * D;
                const u32x4 x = *reinterpret_cast<const u32x4*>(s_new + 16 * lane);
                if (lane < D / 8) *reinterpret_cast<u32x4*>(k_write + row + 8 * lane) = x;
                else *reinterpret_cast<u32x4*>(v_write + row + 8 * (lane - D / 8)) = x;
            }
        }
    }

    if constexpr (D <= 128) {
        // Merge the 4 waves' states through LDS in one round: every wave
        // leaves (m, l, O) there, then all 256 threads form the outputs (or
        // the partition's partial state), one column each.
        __shared__ float s_m[kWaves][16];
        __shared__ float s_l[kWaves][16];
        __shared__ float s_o[kWaves][16][D];
        if (jl == 0) {
            s_m[wave][nl] = st.m;
            s_l[wave][nl] = st.l;
        }
#pragma unroll
        for (int c = 0; c < G::kDT; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) s_o[wave][4 * jl + i][vcol<D>(nl, c)] = st.o[c][i];
        __syncthreads();
        for (int idx = threadIdx.x; idx < g * D; idx += kThreads) {
            const int qi = idx / D;
            const int d = idx - qi * D;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][qi]);
            float L = 0.f, o = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float mw = s_m[w][qi];
                const float wt = mw == -INFINITY ? 0.f : fast_exp2(mw - M);
                L = fmaf(wt, s_l[w][qi], L);
                o = fmaf(wt, s_o[w][qi][d], o);
            }
            const int64_t head_row = (int64_t)s * num_heads + (int64_t)kvh * g + qi;
            if (bad_len) {
                out[head_row * D + d] = (_Float16)NAN;
            } else if (np <= 1) {
                out[head_row * D + d] = L > 0.f ? (_Float16)(o / L) : (_Float16)0.f;
            } else {
                const int64_t slot = head_row * num_parts + part;
                ws_acc[slot * D + d] = o;
                if (d == 0) {
                    ws_ml[2 * slot] = M;
                    ws_ml[2 * slot + 1] = L;
                }
            }
        }
        return;
    } else {
        // head_dim 256: merge as a tree, so that LDS holds two states of O,
        // not four (2 x 16 x D floats): waves 2, 3 hand theirs to waves 0,
        // 1, then wave 1 to wave 0; each receiver rescales both states to
        // the larger maximum and adds.  Wave 0 then writes the result from
        // its registers: lane (n, j) holds O[query 4j + i][d = vcol(n, c)].
        // (Up to head_dim 128 the one-round merge is faster: measured 1.2%
        // per call on the 256-sequence batch at g = 8.)
        __shared__ float s_m[2][16];
        __shared__ float s_l[2][16];
        __shared__ __attribute__((aligned(16))) float s_o[2][16][D];
        for (int half = kWaves / 2; half >= 1; half /= 2) {
            if (wave >= half && wave < 2 * half) {
                const int slot = wave - half;
                if (jl == 0) {
                    s_m[slot][nl] = st.m;
                    s_l[slot][nl] = st.l;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int c = 0; c < G::kDT; ++c) s_o[slot][4 * jl + i][G::kVpl * nl + c] = st.o[c][i];
            }
            __syncthreads();
            if (wave < half) {
                const float pm = s_m[wave][nl];
                const float m = fmaxf(st.m, pm);
                const float a_self = st.m == -INFINITY ? 0.f : fast_exp2(st.m - m);
                const float a_other = pm == -INFINITY ? 0.f : fast_exp2(pm - m);
                st.l = st.l * a_self + s_l[wave][nl] * a_other;
                st.m = m;
                float as[4], ao[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    as[i] = __shfl(a_self, 4 * jl + i);
                    ao[i] = __shfl(a_other, 4 * jl + i);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int c = 0; c < G::kDT; ++c)
                        st.o[c][i] = st.o[c][i] * as[i] + s_o[wave][4 * jl + i][G::kVpl * nl + c] * ao[i];
            }
            if (half > 1) __syncthreads();
        }
        if (wave != 0) return;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int qi = 4 * jl + i;
            const float L = __shfl(st.l, qi);
            const float M = __shfl(st.m, qi);
            if (qi >= g) continue;
            const int64_t head_row = (int64_t)s * num_heads + (int64_t)kvh * g + qi;
            if (bad_len || np <= 1) {
                _Float16 h[G::kDT];
#pragma unroll
                for (int c = 0; c < G::kDT; ++c)
                    h[c] = bad_len ? (_Float16)NAN : L > 0.f ? (_Float16)(st.o[c][i] / L) : (_Float16)0.f;
                _Float16* dst = out + head_row * D;
#pragma unroll
                for (int c = 0; c < G::kDT; c += 4)
                    *reinterpret_cast<half4_t*>(dst + vcol<D>(nl, c)) = half4_t{h[c], h[c + 1], h[c + 2], h[c + 3]};
            } else {
                const int64_t slot = head_row * num_parts + part;
                float* acc = ws_acc + slot * D;
#pragma unroll
                for (int c = 0; c < G::kDT; c += 4)
                    *reinterpret_cast<float4_t*>(acc + vcol<D>(nl, c)) =
                        float4_t{st.o[c][i], st.o[c + 1][i], st.o[c + 2][i], st.o[c + 3][i]};
                if (nl == 0) {
                    ws_ml[2 * slot] = M;
                    ws_ml[2 * slot + 1] = L;
                }
            }
        }

    }
}

using GqaFn = void (*)(_Float16*, float*, float*, const int32_t*, const _Float16*, const _Float16*, const _Float16*,
                       const int32_t*, int32_t, const int32_t*, int32_t, int32_t, int32_t, float, int32_t,
                       int32_t, int64_t, const _Float16*, const _Float16*, int64_t, _Float16*, _Float16*);

template <int D, bool kAppend>
GqaFn pick(int32_t b) {
    switch (b) {
        case 1: return decode_gqa_mfma_kernel<D, 1, kAppend>;
        case 2: return decode_gqa_mfma_kernel<D, 2, kAppend>;
        case 4: return decode_gqa_mfma_kernel<D, 4, kAppend>;
        case 8: return decode_gqa_mfma_kernel<D, 8, kAppend>;
        case 16: return decode_gqa_mfma_kernel<D, 16, kAppend>;
        case 32: return decode_gqa_mfma_kernel<D, 32, kAppend>;
        case 64: return decode_gqa_mfma_kernel<D, 64, kAppend>;
        case 128: return decode_gqa_mfma_kernel<D, 128, kAppend>;
        default: return nullptr;
    }
}

template <bool kAppend>
GqaFn pick(int32_t d, int32_t b) {
    switch (d) {
        case 64: return pick<64, kAppend>(b);
        case 128: return pick<128, kAppend>(b);
        case 256: return pick<256, kAppend>(b);
        default: return nullptr;
    }
}

}  // namespace

namespace pa {

bool gqa_mfma_supported(int32_t head_dim, int32_t block_size, int32_t group) {
    return group >= 2 && group <= 16 && pick<false>(head_dim, block_size) != nullptr;
}

hipError_t launch_gqa_mfma(const DecodeLaunch& a) {
    const bool app = a.new_k != nullptr;
    GqaFn fn = app ? pick<true>(a.head_dim, a.block_size) : pick<false>(a.head_dim, a.block_size);
    // in append mode the cache pointers double as write pointers: the kernel
    // writes only the row of each sequence's last position, which no
    // workgroup reads from the cache
    hipLaunchKernelGGL(fn, dim3((unsigned)a.num_kv_heads, (unsigned)a.num_seqs, (unsigned)a.num_parts),
                       dim3(kThreads), 0, a.stream, a.out, a.ws_ml, a.ws_acc, a.order, a.q, a.k_cache, a.v_cache,
                       a.tables, a.max_blocks, a.lens, a.num_heads, a.num_kv_heads, a.num_blocks, a.scale_log2,
                       a.part_size, a.num_parts, a.len_cap, a.new_k, a.new_v, a.new_stride,
                       app ? const_cast<_Float16*>(a.k_cache) : nullptr,
                       app ? const_cast<_Float16*>(a.v_cache) : nullptr);
    return hipGetLastError();
}

}  // namespace pa

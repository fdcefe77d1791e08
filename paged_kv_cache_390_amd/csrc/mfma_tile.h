// MFMA building blocks shared by the matrix-core attention kernels of the
// library (grouped-query decode, paged prefill): one 16-token K/V tile as a
// lane holds it, its loads through the block table, and the consumption of
// a tile by 16 query rows -- S^T = K Q^T on v_mfma_f32_16x16x16_f16, the
// online softmax in the accumulator layout, O += P V.  Lane layouts (checked
// on the GPU against a host product): A[m][k] in lane m + 16*(k/4), B[k][n]
// in lane n + 16*(k/4), C[m][n] in lane n + 16*(m/4).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;                // head_dim served here
constexpr int kTile = 16;              // tokens per wave step
constexpr int kQkSteps = kD / 16;      // MFMAs per QK tile (k = 16 each)
constexpr int kDTiles = kD / 16;       // output column tiles of 16

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ half8_t as_h8(u32x4 u) { return __builtin_bit_cast(half8_t, u); }

// One 16-token tile as this lane holds it.
struct Tile {
    u32x4 k[4];        // K row (token l%16), d = 8*(4u + l/16) .. +7
    u32x4 v[4];        // V rows (tokens 4*(l/16) + i), d = 8*(l%16) .. +7
    bool valid[4];     // tokens 4*(l/16) + i: inside the context and the pool
};

struct Softmax {
    float m, l;        // running max (base 2) and sum of query l%16
    float4_t o[kDTiles];   // O[query 4*(l/16) + i][d = 8*(l%16) + c] in o[c][i]
};

// Tile loads when a tile lies inside one block (B >= 16): `phys` is the
// block's table entry, read ahead by the caller with a scalar load.
template <int B>
__device__ __forceinline__ void load_tile_block(Tile& t, int t0, int end, int32_t phys,
                                                const _Float16* __restrict__ kbase,
                                                const _Float16* __restrict__ vbase, int64_t blk_stride,
                                                int32_t num_blocks, int lane) {
    const int n = lane & 15;
    const int j = lane >> 4;
    const bool ok = (uint32_t)phys < (uint32_t)num_blocks;
    const int64_t base = (int64_t)(ok ? phys : 0) * blk_stride + (int64_t)(t0 % B) * kD;
    // rows past the context read the context's last row again (the same
    // cache lines: no extra HBM bytes) and are masked later
    const int lim = end - 1 - t0;
    const int rk = n < lim ? n : lim;
#pragma unroll
    for (int u = 0; u < 4; ++u)
        t.k[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + base + rk * kD + 8 * (4 * u + j)));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rv = 4 * j + i < lim ? 4 * j + i : lim;
        t.valid[i] = ok && t0 + 4 * j + i < end;
        t.v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vbase + base + rv * kD + 8 * n));
    }
}

// Tile loads when a tile spans several blocks (B < 16): every row looks up
// its own table entry.
template <int B>
__device__ __forceinline__ void load_tile_rows(Tile& t, int t0, int end, const int32_t* __restrict__ trow,
                                               const _Float16* __restrict__ kbase,
                                               const _Float16* __restrict__ vbase, int64_t blk_stride,
                                               int32_t num_blocks, int lane) {
    const int n = lane & 15;
    const int j = lane >> 4;
    {
        const int tk = t0 + n;
        const int tc = tk < end ? tk : end - 1;        // keeps the table index inside the sequence
        const int32_t phys = trow[tc / B];
        const bool ok = (uint32_t)phys < (uint32_t)num_blocks;
        const int64_t row = (int64_t)(ok ? phys : 0) * blk_stride + (int64_t)(tc % B) * kD;
#pragma unroll
        for (int u = 0; u < 4; ++u)
            t.k[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + row + 8 * (4 * u + j)));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int tv = t0 + 4 * j + i;
        const int tc = tv < end ? tv : end - 1;
        const int32_t phys = trow[tc / B];
        const bool ok = (uint32_t)phys < (uint32_t)num_blocks;
        t.valid[i] = tv < end && ok;
        const int64_t row = (int64_t)(ok ? phys : 0) * blk_stride + (int64_t)(tc % B) * kD;
        t.v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vbase + row + 8 * n));
    }
}

// keep[i]: token 4*(l/16) + i takes part for this lane's query row (inside
// the context and the pool, and -- for prefill -- not after the row's own
// position); t.valid[i]: its V row holds data (zeroed by select otherwise).
__device__ __forceinline__ void consume_tile(Softmax& st, const Tile& t, const half4_t (&qb)[kQkSteps],
                                             float scale_log2, int lane, const bool (&keep)[4]) {
    const int j = lane >> 4;
    // S^T = K Q^T: lane holds S^T[token 4j+i][query l%16]
    float4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kQkSteps; ++c) {
        const half8_t kk = as_h8(t.k[c >> 1]);
        const half4_t a = (c & 1) ? half4_t{kk[4], kk[5], kk[6], kk[7]} : half4_t{kk[0], kk[1], kk[2], kk[3]};
        s = __builtin_amdgcn_mfma_f32_16x16x16f16(a, qb[c], s, 0, 0, 0);
    }
    // online softmax of query l%16 over the tile's 16 tokens (4 per lane, 4 lanes)
    float sc[4];
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        sc[i] = keep[i] ? s[i] * scale_log2 : -INFINITY;
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
        for (int c = 0; c < kDTiles; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) st.o[c][i] *= ar[i];
    }
    // O += P V per d-tile.  Rows of masked tokens may hold anything (NaN in
    // an unused tail row): in a tile with any masked row they are zeroed by
    // select first, since a zero weight times NaN is still NaN.
    auto pv = [&](const u32x4 (&v)[4]) {
        const half8_t v0 = as_h8(v[0]), v1 = as_h8(v[1]), v2 = as_h8(v[2]), v3 = as_h8(v[3]);
#pragma unroll
        for (int c = 0; c < kDTiles; ++c) {
            const half4_t b = {v0[c], v1[c], v2[c], v3[c]};
            st.o[c] = __builtin_amdgcn_mfma_f32_16x16x16f16(p, b, st.o[c], 0, 0, 0);
        }
    };
    if (__all(t.valid[0] && t.valid[1] && t.valid[2] && t.valid[3])) {
        pv(t.v);
    } else {
        const u32x4 z = {0u, 0u, 0u, 0u};
        const u32x4 vz[4] = {t.valid[0] ? t.v[0] : z, t.valid[1] ? t.v[1] : z, t.valid[2] ? t.v[2] : z,
                             t.valid[3] ? t.v[3] : z};
        pv(vz);
    }
}

// Q^T operands of this lane's query row (zero if !live): for MFMA c = 2u +
// (c & 1) the lane holds d = 8*(4u + l/16) + 4*(c & 1) + 0..3.
__device__ __forceinline__ void load_q_operands(half4_t (&qb)[kQkSteps], const _Float16* __restrict__ qrow,
                                                bool live, int lane) {
    const int j = lane >> 4;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        const half8_t h = as_h8(live ? *reinterpret_cast<const u32x4*>(qrow + 8 * (4 * u + j)) : z);
        qb[2 * u] = half4_t{h[0], h[1], h[2], h[3]};
        qb[2 * u + 1] = half4_t{h[4], h[5], h[6], h[7]};
    }
}

}  // namespace

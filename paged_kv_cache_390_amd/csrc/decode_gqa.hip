// Grouped-query paged decode attention on the CDNA4 matrix cores (gfx950).
//
// What is computed is the same as for every other pa_decode shape: each
// query head attends to its sequence's n cached keys/values through the
// block table, textbook softmax attention over the logically contiguous K/V
// (lpnh.cn/news/1824136, 2.2 and 3.2 step 4; lpnh.cn/news/2758356, 2.1 for
// the KV-head dimension of a block).  This kernel serves the case where g =
// num_heads / num_kv_heads query heads share one KV head (2 <= g <= 16,
// head_dim 128): then every K/V element read from HBM meets g queries, and
// the two products are small dense contractions,
//     S^T[t, q] = sum_d K[t, d] Q[q, d]        (16 tokens x 16 queries x 128)
//     O[q, d]  += sum_t P[q, t] V[t, d]         (16 queries x 128 x 16 tokens)
// which run on v_mfma_f32_16x16x16_f16 (fp16 inputs, fp32 accumulation).
// The kernel is still HBM-bound: about 4g flops per 2 bytes of K/V, far
// below the matrix cores' ridge, so the design serves the loads.
//
// Layout (one 256-thread workgroup = 4 wave64s per (KV head, sequence,
// context partition); KV head fastest in the grid so every XCD streams the
// same bytes; a wave step is one 16-token tile, steps dealt round-robin to
// the waves, three tiles in flight per wave when a tile lies in one block):
//  * MFMA 16x16x16 lane layout: A[m][k] is held by lane m + 16*(k/4),
//    B[k][n] by lane n + 16*(k/4), C[m][n] by lane n + 16*(m/4).
//  * QK: A = K tile (m = token), B = Q^T (n = query head of the group,
//    zero-padded past g).  The contraction index k is mapped onto head_dim so
//    that lane (m, j) reads 64 contiguous bytes of token m's row with four
//    16-byte loads -- for load u, d = 8*(4u + j) .. +7 -- and each half of a
//    load is one MFMA operand: no register shuffles.
//  * The result S^T lands with lane (n, j) holding tokens 4j..4j+3 of query
//    n: exactly the A-operand layout of P for the PV product, so the online
//    softmax (running max / sum per query, base 2, log2(e) folded into the
//    scale) runs in place and P goes to the matrix core as fp16.
//  * PV: B = V tile.  Output column n of d-tile c is mapped to d = 8n + c, so
//    lane (n, j) loads 16 contiguous bytes (d = 8n .. 8n+7) of tokens
//    4j..4j+3 -- four 16-byte loads that together read every V row whole --
//    and element c of the four loads is the B operand of d-tile c.
//  * Masking by select: a token past the context, or behind a table entry
//    outside the pool, gets S = -inf and V = 0, so NaN in unused rows cannot
//    reach the sums (0 * NaN would).
//  * Normalisation uses the same fp16-rounded weights the matrix core saw,
//    so each output is an exact convex combination of V rows up to fp32
//    rounding.
//  * The 4 waves' (m, l, O) are merged through LDS; rows split over several
//    partitions leave (m, l, O) in the workspace for the shared reduce
//    kernel, in the same layout as the one-query-per-KV-head kernel.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "decode_internal.h"
#include "mfma_tile.h"

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;

// kAppend: the last position n - 1 of every sequence holds the token of
// this step, whose K/V come from new_k / new_v (token s, KV head h at s *
// new_stride + h * 128) instead of the cache; the workgroup whose partition
// holds it folds it in as a one-token tile and writes it into the cache
// through k_write / v_write.  The cache is read for positions < n - 1 only.
template <int B, bool kAppend>
__global__ void __launch_bounds__(kThreads)
decode_gqa_mfma_kernel(_Float16* __restrict__ out, float* __restrict__ ws_ml, float* __restrict__ ws_acc,
                       const int32_t* __restrict__ order, const _Float16* __restrict__ q, const _Float16* __restrict__ k_cache,
                       const _Float16* __restrict__ v_cache, const int32_t* __restrict__ tables,
                       int32_t max_blocks, const int32_t* __restrict__ lens, int32_t num_heads,
                       int32_t num_kv_heads, int32_t num_blocks, float scale_log2, int32_t part_size,
                       int32_t num_parts, int64_t len_cap, const _Float16* __restrict__ new_k,
                       const _Float16* __restrict__ new_v, int64_t new_stride, _Float16* __restrict__ k_write,
                       _Float16* __restrict__ v_write) {
    const int kvh = blockIdx.x;
    const int s = order ? order[blockIdx.y] : (int)blockIdx.y;   // longest sequences first
    if ((uint32_t)s >= gridDim.y) return;                         // not a sequence: nothing to do
    const int part = blockIdx.z;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = num_heads / num_kv_heads;

    const int32_t n_raw = lens[s];
    const bool bad_len = n_raw < 0 || (int64_t)n_raw > len_cap;
    const int n = bad_len ? 0 : n_raw;
    const int start = part * part_size;
    if (part > 0 && start >= n) return;
    const int cached = kAppend && n > 0 ? n - 1 : n;   // positions read from the cache
    const int end = min(start + part_size, cached);
    const int np = (n + part_size - 1) / part_size;

    // Q^T operands of query head kvh*g + l%16 (zero past g)
    half4_t qb[kQkSteps];
    {
        const int qi = lane & 15;
        const bool live = qi < g;
        load_q_operands(qb, q + ((int64_t)s * num_heads + (int64_t)kvh * g + (live ? qi : 0)) * kD, live, lane);
    }

    const int32_t* trow = tables + (int64_t)s * max_blocks;
    const int64_t slab = (int64_t)B * kD;
    const _Float16* kbase = k_cache + (int64_t)kvh * slab;
    const _Float16* vbase = v_cache + (int64_t)kvh * slab;
    const int64_t blk_stride = (int64_t)num_kv_heads * slab;

    Softmax st;
    st.m = -INFINITY;
    st.l = 0.f;
#pragma unroll
    for (int c = 0; c < kDTiles; ++c) st.o[c] = float4_t{0.f, 0.f, 0.f, 0.f};

    // append mode: the new token's K/V pieces this lane would hold as token
    // 0 of a tile, loaded now by every lane (a valid address for all) so
    // that the load hides under the main loop
    u32x4 new_kf[4], new_vf;
    if constexpr (kAppend) {
        const _Float16* kn = new_k + (int64_t)s * new_stride + (int64_t)kvh * kD;
#pragma unroll
        for (int u = 0; u < 4; ++u) new_kf[u] = *reinterpret_cast<const u32x4*>(kn + 8 * (4 * u + (lane >> 4)));
        new_vf = *reinterpret_cast<const u32x4*>(new_v + (int64_t)s * new_stride + (int64_t)kvh * kD + 8 * (lane & 15));
    }

    const int ntok = end > start ? end - start : 0;
    const int nsteps = (ntok + kTile - 1) / kTile;
    if (wave < nsteps) {
        Tile A, Bt;
        if constexpr (B >= kTile) {
            // One table entry per tile, read with scalar loads a tile ahead of
            // its issue; three tiles in flight per wave beside the one being
            // consumed (A, Bt, C, D rotate).  Every step issues a tile -- past
            // the last step one that is never consumed, every lane reading the
            // same 16 bytes of the last tile's block (one cache line per load)
            // -- so the count of loads is the same on every path and the wait
            // before a consume leaves the three newer tiles in flight.
            Tile C, D;
            auto clamp = [&](int stp) { return stp < nsteps ? stp : nsteps - 1; };
            auto entry = [&](int stp) { return trow[(start + clamp(stp) * kTile) / B]; };
            auto issue = [&](Tile& t, int stp, int32_t phys) {
                load_tile_block<B>(t, start + clamp(stp) * kTile, end, phys, kbase, vbase, blk_stride, num_blocks,
                                   stp < nsteps ? lane : 0);
            };
            int stp = wave;
            issue(A, stp, entry(stp));
            issue(Bt, stp + kWaves, entry(stp + kWaves));
            issue(C, stp + 2 * kWaves, entry(stp + 2 * kWaves));
            int32_t tnext = entry(stp + 3 * kWaves);
            // before each consume: the tile 3 steps ahead is issued, the entry 4 steps ahead read
            auto advance = [&](Tile& t, int st) {
                const int ahead = st + 3 * kWaves;
                const int32_t cur = tnext;
                tnext = entry(ahead + kWaves);
                issue(t, ahead, cur);
            };
            for (;;) {
                advance(D, stp);
                consume_tile(st, A, qb, scale_log2, lane, A.valid);
                stp += kWaves;
                if (stp >= nsteps) break;
                advance(A, stp);
                consume_tile(st, Bt, qb, scale_log2, lane, Bt.valid);
                stp += kWaves;
                if (stp >= nsteps) break;
                advance(Bt, stp);
                consume_tile(st, C, qb, scale_log2, lane, C.valid);
                stp += kWaves;
                if (stp >= nsteps) break;
                advance(C, stp);
                consume_tile(st, D, qb, scale_log2, lane, D.valid);
                stp += kWaves;
                if (stp >= nsteps) break;
            }
        } else {
            int stp = wave;
            load_tile_rows<B>(A, start + stp * kTile, end, trow, kbase, vbase, blk_stride, num_blocks, lane);
            for (;;) {
                int nx = stp + kWaves;
                if (nx >= nsteps) { consume_tile(st, A, qb, scale_log2, lane, A.valid); break; }
                load_tile_rows<B>(Bt, start + nx * kTile, end, trow, kbase, vbase, blk_stride, num_blocks, lane);
                consume_tile(st, A, qb, scale_log2, lane, A.valid);
                stp = nx;
                nx = stp + kWaves;
                if (nx >= nsteps) { consume_tile(st, Bt, qb, scale_log2, lane, Bt.valid); break; }
                load_tile_rows<B>(A, start + nx * kTile, end, trow, kbase, vbase, blk_stride, num_blocks, lane);
                consume_tile(st, Bt, qb, scale_log2, lane, Bt.valid);
                stp = nx;
            }
        }
    }

    if constexpr (kAppend) {
        const int pos = n - 1;                  // the new token, as token 0 of a tile
        if (n > 0 && pos >= start && pos < start + part_size && wave == kWaves - 1) {
            const int32_t phys = trow[pos / B];
            const bool ok = (uint32_t)phys < (uint32_t)num_blocks;   // as a cached row behind a skipped id
            const int nn = lane & 15;
            const int j = lane >> 4;
            const u32x4 z = {0u, 0u, 0u, 0u};
            Tile t;
            // K row of token l%16 (d = 8*(4u + l/16) ..): token 0 only
#pragma unroll
            for (int u = 0; u < 4; ++u) t.k[u] = nn == 0 ? new_kf[u] : z;
            // V rows of tokens 4*(l/16) + i (d = 8*(l%16) ..): token 0 is i = 0 of lane group 0
            t.v[0] = j == 0 ? new_vf : z;
#pragma unroll
            for (int i = 1; i < 4; ++i) t.v[i] = z;
#pragma unroll
            for (int i = 0; i < 4; ++i) t.valid[i] = ok && j == 0 && i == 0;
            consume_tile(st, t, qb, scale_log2, lane, t.valid);
            if (ok) {
                const int64_t row = (int64_t)kvh * slab + (int64_t)phys * blk_stride + (int64_t)(pos % B) * kD;
                if (nn == 0)
#pragma unroll
                    for (int u = 0; u < 4; ++u) *reinterpret_cast<u32x4*>(k_write + row + 8 * (4 * u + j)) = t.k[u];
                if (j == 0) *reinterpret_cast<u32x4*>(v_write + row + 8 * nn) = t.v[0];
            }
        }
    }

    // Merge the 4 waves.  s_o[w][q][d] holds wave w's unnormalised output.
    __shared__ float s_m[kWaves][16];
    __shared__ float s_l[kWaves][16];
    __shared__ float s_o[kWaves][16][kD];
    {
        const int ncol = lane & 15;
        const int j = lane >> 4;
        if (j == 0) {
            s_m[wave][ncol] = st.m;
            s_l[wave][ncol] = st.l;
        }
#pragma unroll
        for (int c = 0; c < kDTiles; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) s_o[wave][4 * j + i][8 * ncol + c] = st.o[c][i];
    }
    __syncthreads();

    for (int idx = threadIdx.x; idx < g * kD; idx += kThreads) {
        const int qi = idx / kD;
        const int d = idx - qi * kD;
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
            out[head_row * kD + d] = (_Float16)NAN;
        } else if (np <= 1) {
            out[head_row * kD + d] = L > 0.f ? (_Float16)(o / L) : (_Float16)0.f;
        } else {
            const int64_t slot = head_row * num_parts + part;
            ws_acc[slot * kD + d] = o;
            if (d == 0) {
                ws_ml[2 * slot] = M;
                ws_ml[2 * slot + 1] = L;
            }
        }
    }
}

using GqaFn = void (*)(_Float16*, float*, float*, const int32_t*, const _Float16*, const _Float16*, const _Float16*,
                       const int32_t*, int32_t, const int32_t*, int32_t, int32_t, int32_t, float, int32_t,
                       int32_t, int64_t, const _Float16*, const _Float16*, int64_t, _Float16*, _Float16*);

template <bool kAppend>
GqaFn pick(int32_t b) {
    switch (b) {
        case 1: return decode_gqa_mfma_kernel<1, kAppend>;
        case 2: return decode_gqa_mfma_kernel<2, kAppend>;
        case 4: return decode_gqa_mfma_kernel<4, kAppend>;
        case 8: return decode_gqa_mfma_kernel<8, kAppend>;
        case 16: return decode_gqa_mfma_kernel<16, kAppend>;
        case 32: return decode_gqa_mfma_kernel<32, kAppend>;
        case 64: return decode_gqa_mfma_kernel<64, kAppend>;
        case 128: return decode_gqa_mfma_kernel<128, kAppend>;
        default: return nullptr;
    }
}

}  // namespace

namespace pa {

bool gqa_mfma_supported(int32_t head_dim, int32_t block_size, int32_t group) {
    return head_dim == kD && group >= 2 && group <= 16 && pick<false>(block_size) != nullptr;
}

hipError_t launch_gqa_mfma(const DecodeLaunch& a) {
    const bool app = a.new_k != nullptr;
    GqaFn fn = app ? pick<true>(a.block_size) : pick<false>(a.block_size);
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

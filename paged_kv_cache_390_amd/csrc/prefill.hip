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
// K/V tile meets every later query of its sequence, so the work runs on
// v_mfma_f32_16x16x16_f16 and is bound by the matrix cores and the softmax
// around them, not by HBM.
//  * Query rows: the m new tokens x g query heads of one KV head, token
//    major (row r = token r / g, head r % g).  A wave owns 16 rows -- the N
//    side of the MFMA tiles -- and walks the K/V tiles 0 .. its last row's
//    position on its own: no cross-wave merge.  A 256-thread workgroup is 4
//    such waves (64 rows) of one (KV head, sequence); grid x = KV head
//    (fastest, for XCD balance), y = sequence, z = row tile, issued last row
//    tile first so the longest causal ranges start earliest.
//  * A tile is consumed exactly as in grouped-query decode (shared code):
//    S^T = K Q^T, online softmax per row in the accumulator layout, O += P V,
//    two tiles in flight per wave, table entries read ahead with scalar
//    loads when B >= 16.  The causal mask is a select on each score.
//  * The wave writes its 16 rows itself: each lane holds 8 consecutive
//    output columns of 4 rows, normalised by the row sums it fetches with a
//    cross-lane shuffle, and stores 16 bytes per row.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "mfma_tile.h"
#include "pa.h"
#include "pa_internal.h"

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 16;
constexpr int kRowsPerGroup = kWaves * kRowsPerWave;
constexpr double kLog2e = 1.4426950408889634073599246810019;

template <int B>
__global__ void __launch_bounds__(kThreads)
prefill_mfma_kernel(_Float16* __restrict__ out, const _Float16* __restrict__ q, int32_t num_tokens,
                    const _Float16* __restrict__ k_cache, const _Float16* __restrict__ v_cache,
                    const int32_t* __restrict__ tables, int32_t max_blocks, const int32_t* __restrict__ lens,
                    const int32_t* __restrict__ query_start, int32_t num_heads, int32_t num_kv_heads,
                    int32_t num_blocks, float scale_log2, int32_t max_query_len, int64_t len_cap) {
    const int kvh = blockIdx.x;
    const int s = blockIdx.y;
    const int rtile = gridDim.z - 1 - blockIdx.z;          // last row tile first
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = num_heads / num_kv_heads;

    const int32_t q0 = query_start[s];
    const int32_t q1 = query_start[s + 1];
    // rows outside [0, num_tokens) are never touched: a sequence whose range
    // is not inside it is skipped
    if (q0 < 0 || q1 < q0 || q1 > num_tokens) return;
    const int32_t m_raw = q1 - q0;
    const int32_t n_raw = lens[s];
    const int rows_all = (m_raw < max_query_len ? m_raw : max_query_len) * g;
    const int row0 = rtile * kRowsPerGroup + wave * kRowsPerWave;   // first row of this wave
    if (row0 >= rows_all) return;
    const bool bad = m_raw > max_query_len || n_raw < m_raw || (int64_t)n_raw > len_cap;
    const int rows = min(rows_all - row0, kRowsPerWave);             // live rows of this wave

    const int nrow = lane & 15;                 // this lane's query row (MFMA column)
    const int jg = lane >> 4;                   // its token group within a tile
    if (bad) {                                  // the sequence's rows come out as NaN
        if (jg == 0 && nrow < rows) {
            const int r = row0 + nrow;
            const int64_t orow = ((int64_t)q0 + r / g) * num_heads + (int64_t)kvh * g + r % g;
            for (int d = 0; d < kD; ++d) out[orow * kD + d] = (_Float16)NAN;
        }
        return;
    }
    const int n = n_raw, m = m_raw;
    const int base_pos = n - m;                 // position of new token 0

    // this lane's row: token, head, position
    const bool live = nrow < rows;
    const int r = row0 + (live ? nrow : 0);
    const int pos = base_pos + r / g;
    half4_t qb[kQkSteps];
    load_q_operands(qb, q + (((int64_t)q0 + r / g) * num_heads + (int64_t)kvh * g + r % g) * kD, live, lane);

    // the position of the wave's last live row bounds its causal range
    const int pos_hi = base_pos + (row0 + rows - 1) / g;
    const int ntiles = pos_hi / kTile + 1;

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

    auto consume = [&](const Tile& t, int k) {
        const int t0 = k * kTile;
        bool keep[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) keep[i] = live && t.valid[i] && t0 + 4 * jg + i <= pos;   // causal
        consume_tile(st, t, qb, scale_log2, lane, keep);
    };

    Tile A, Bt;
    if constexpr (B >= kTile) {
        auto entry = [&](int k) { return trow[(k * kTile) / B]; };
        int k = 0;
        int32_t tnext = k + 1 < ntiles ? entry(k + 1) : 0;
        load_tile_block<B>(A, 0, n, entry(0), kbase, vbase, blk_stride, num_blocks, lane);
        for (;;) {
            if (k + 1 >= ntiles) { consume(A, k); break; }
            int32_t tcur = tnext;
            tnext = k + 2 < ntiles ? entry(k + 2) : 0;
            load_tile_block<B>(Bt, (k + 1) * kTile, n, tcur, kbase, vbase, blk_stride, num_blocks, lane);
            consume(A, k);
            ++k;
            if (k + 1 >= ntiles) { consume(Bt, k); break; }
            tcur = tnext;
            tnext = k + 2 < ntiles ? entry(k + 2) : 0;
            load_tile_block<B>(A, (k + 1) * kTile, n, tcur, kbase, vbase, blk_stride, num_blocks, lane);
            consume(Bt, k);
            ++k;
        }
    } else {
        int k = 0;
        load_tile_rows<B>(A, 0, n, trow, kbase, vbase, blk_stride, num_blocks, lane);
        for (;;) {
            if (k + 1 >= ntiles) { consume(A, k); break; }
            load_tile_rows<B>(Bt, (k + 1) * kTile, n, trow, kbase, vbase, blk_stride, num_blocks, lane);
            consume(A, k);
            ++k;
            if (k + 1 >= ntiles) { consume(Bt, k); break; }
            load_tile_rows<B>(A, (k + 1) * kTile, n, trow, kbase, vbase, blk_stride, num_blocks, lane);
            consume(Bt, k);
            ++k;
        }
    }

    // Rows 4*jg + i of the wave live in this lane's o[c][i] at column 8*nrow
    // + c; their sums sit in lanes 4*jg + i.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rr = 4 * jg + i;
        const float L = __shfl(st.l, rr);
        if (rr >= rows) continue;
        const int rw = row0 + rr;
        const int64_t orow = ((int64_t)q0 + rw / g) * num_heads + (int64_t)kvh * g + rw % g;
        const float inv = L > 0.f ? 1.f / L : 0.f;
        half8_t h;
#pragma unroll
        for (int c = 0; c < kDTiles; ++c) h[c] = (_Float16)(st.o[c][i] * inv);
        *reinterpret_cast<half8_t*>(out + orow * kD + 8 * nrow) = h;
    }
}

using PrefillFn = void (*)(_Float16*, const _Float16*, int32_t, const _Float16*, const _Float16*, const int32_t*,
                           int32_t, const int32_t*, const int32_t*, int32_t, int32_t, int32_t, float, int32_t,
                           int64_t);

PrefillFn pick(int32_t b) {
    switch (b) {
        case 1: return prefill_mfma_kernel<1>;
        case 2: return prefill_mfma_kernel<2>;
        case 4: return prefill_mfma_kernel<4>;
        case 8: return prefill_mfma_kernel<8>;
        case 16: return prefill_mfma_kernel<16>;
        case 32: return prefill_mfma_kernel<32>;
        case 64: return prefill_mfma_kernel<64>;
        case 128: return prefill_mfma_kernel<128>;
        default: return nullptr;
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" int pa_prefill(void* out, const void* q, int32_t num_tokens, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                          const int32_t* query_start, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                          int32_t max_query_len, int32_t dtype, void* stream) {
    if (dtype != PA_DTYPE_F16) return pa::fail(PA_ERR_UNSUPPORTED, "pa_prefill: dtype %d", dtype);
    if (head_dim != kD) return pa::fail(PA_ERR_UNSUPPORTED, "pa_prefill: head_dim %d (only %d)", head_dim, kD);
    if (!pick(block_size)) return pa::fail(PA_ERR_UNSUPPORTED, "pa_prefill: block_size %d", block_size);
    if (num_seqs < 0 || num_tokens < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 ||
        num_blocks <= 0 || max_blocks_per_seq < 0 || max_query_len < 0)
        return pa::fail(PA_ERR_INVALID, "pa_prefill: bad sizes (S=%d H=%d Hkv=%d NB=%d W=%d max_q=%d)", num_seqs,
                        num_heads, num_kv_heads, num_blocks, max_blocks_per_seq, max_query_len);
    if (num_seqs > 65535 || num_kv_heads > 65535)
        return pa::fail(PA_ERR_INVALID, "pa_prefill: num_seqs and num_kv_heads must be <= 65535");
    if (!std::isfinite(scale)) return pa::fail(PA_ERR_INVALID, "pa_prefill: scale is not finite");
    if (num_seqs == 0 || max_query_len == 0 || num_tokens == 0) return PA_OK;
    if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
        return pa::fail(PA_ERR_INVALID, "pa_prefill: null pointer");
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
        return pa::fail(PA_ERR_INVALID, "pa_prefill: out, q and caches must be 16-byte aligned");
    const int64_t g = num_heads / num_kv_heads;
    const int64_t row_tiles = ((int64_t)max_query_len * g + kRowsPerGroup - 1) / kRowsPerGroup;
    if (row_tiles > 65535)
        return pa::fail(PA_ERR_INVALID, "pa_prefill: max_query_len %d x %lld heads needs %lld row tiles (limit 65535)",
                        max_query_len, (long long)g, (long long)row_tiles);
    const int64_t len_cap = (int64_t)max_blocks_per_seq * block_size;
    const float scale_log2 = (float)((double)scale * kLog2e);
    hipLaunchKernelGGL(pick(block_size), dim3((unsigned)num_kv_heads, (unsigned)num_seqs, (unsigned)row_tiles),
                       dim3(kThreads), 0, static_cast<hipStream_t>(stream), static_cast<_Float16*>(out),
                       static_cast<const _Float16*>(q), num_tokens, static_cast<const _Float16*>(k_cache),
                       static_cast<const _Float16*>(v_cache), block_tables, max_blocks_per_seq, context_lens,
                       query_start, num_heads, num_kv_heads, num_blocks, scale_log2, max_query_len, len_cap);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return pa::fail(PA_ERR_HIP, "pa_prefill: %s", hipGetErrorString(e));
    return PA_OK;
}

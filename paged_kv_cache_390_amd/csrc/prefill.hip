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
//    major (row r = token r / g, head r % g).  A wave owns 16 rows -- the N
//    side of the MFMA tiles.  A 512-thread workgroup is 8 such waves (128
//    rows) of one (KV head, sequence); grid x = KV head (fastest, for XCD
//    balance), y = sequence, z = row tile, issued last row tile first so the
//    longest causal ranges start earliest.
//  * K/V tiles of 32 tokens are staged through LDS once per workgroup and
//    read by all 8 waves: each thread fetches 16 bytes of one token row of K
//    and of V (table lookup per row, nontemporal loads) two tiles ahead into
//    registers, and stores them one tile ahead into the other of two LDS
//    buffers; one barrier per tile.  Rows are padded to 272 bytes so that
//    the 16 rows one operand read touches fall in different banks.
//  * QK as S^T = K Q^T: MFMA c takes head_dim 32c + 8*(l/16) + 0..7 in lane
//    l, one 16-byte LDS read of K per MFMA; Q^T operands stay in registers.
//    S^T lands with each lane holding 8 scores of one row (tokens 4j..4j+3
//    and 16+4j..16+4j+3 of the tile) -- exactly that lane's A operand of P
//    for the 32-token PV product, so the online softmax (base 2, causal and
//    validity masks by select) runs in place and P goes to the matrix core
//    as fp16; the row sum adds the same rounded weights.
//  * PV: output column n of d-tile c is d = 8n + c; the lane reads its 8
//    token rows' columns 8n..8n+7 and builds each B operand with 4
//    v_perm_b32 (an 8 x 8 transpose of halves).
//  * Each wave walks the tiles up to its own last row's position and writes
//    its rows itself: 16 bytes per row, normalised by the row sums fetched
//    with a cross-lane shuffle.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "mfma_tile.h"
#include "pa.h"
#include "pa_internal.h"

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 16;
constexpr int kRowsPerGroup = kWaves * kRowsPerWave;
constexpr double kLog2e = 1.4426950408889634073599246810019;

// One K/V tile in LDS: kKvTile token rows of K and of V, kPitch bytes each
// (256 bytes of data + 16 of padding, so the 16 rows one MFMA operand read
// touches fall in different banks), plus a flag per token (inside the
// context and the pool).
constexpr int kKvTile = 32;
constexpr int kPitch = kD * 2 + 16;
constexpr int kTileBytes = kKvTile * kPitch;

typedef _Float16 half8_t_ __attribute__((ext_vector_type(8)));

// One thread's share of a K/V tile in flight: 16 bytes (columns 8*col ..
// 8*col+7) of kStageRows token rows -- tok, tok + kThreads/16, ... with tok
// = thread / 16 -- of K and of V.
constexpr int kStageRows = kKvTile * 16 / kThreads;
static_assert(kStageRows >= 1 && kKvTile * 16 == kStageRows * kThreads, "tile rows must split evenly");

struct Staged {
    u32x4 k[kStageRows], v[kStageRows];
    bool ok[kStageRows];
};

// Fetch tile k (tokens 32k .. 32k+31) from HBM into registers.
template <int B>
__device__ __forceinline__ void fetch_tile(Staged& st, int k, int n, const int32_t* __restrict__ trow,
                                           const _Float16* __restrict__ kbase, const _Float16* __restrict__ vbase,
                                           int64_t blk_stride, int32_t num_blocks) {
    const int tok = (int)threadIdx.x / 16;
    const int col = (int)threadIdx.x % 16;
#pragma unroll
    for (int i = 0; i < kStageRows; ++i) {
        const int t = k * kKvTile + tok + (kThreads / 16) * i;
        const int tc = t < n ? t : n - 1;
        const int32_t phys = trow[tc / B];
        const bool ok = t < n && (uint32_t)phys < (uint32_t)num_blocks;
        const int64_t off = (int64_t)(ok ? phys : 0) * blk_stride + (int64_t)(tc % B) * kD + col * 8;
        const u32x4 z = {0u, 0u, 0u, 0u};
        st.k[i] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + off)) : z;
        st.v[i] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vbase + off)) : z;
        st.ok[i] = ok;
    }
}

__device__ __forceinline__ void store_tile(const Staged& st, unsigned char* buf, unsigned char* flags) {
    const int tok = (int)threadIdx.x / 16;
    const int col = (int)threadIdx.x % 16;
#pragma unroll
    for (int i = 0; i < kStageRows; ++i) {
        const int row = tok + (kThreads / 16) * i;
        *reinterpret_cast<u32x4*>(buf + row * kPitch + col * 16) = st.k[i];
        *reinterpret_cast<u32x4*>(buf + kTileBytes + row * kPitch + col * 16) = st.v[i];
        if (col == 0) flags[row] = st.ok[i];
    }
}

// Runtime flags of one wave's rows.
struct Rows {
    bool live;       // this lane's row (l % 16) exists
    int pos;         // its position
};

// Consume one LDS tile for the wave's 16 rows on v_mfma_f32_16x16x32_f16.
//   QK, per 16-token half h: S^T[token][row] = sum_d K[token][d] Q[row][d];
//     MFMA c takes d = 32c + 8*(l/16) + 0..7 in lane l (one 16-byte LDS read).
//   PV: k = 32 tokens; lane (n, j) supplies P[row n][tokens 4j..4j+3 and
//     16+4j..16+4j+3] -- exactly the scores it holds -- and V rows of the
//     same tokens at columns 8n..8n+7; output column n of d-tile c is d = 8n+c.
__device__ __forceinline__ void consume_lds_tile(Softmax& st, const unsigned char* buf, const unsigned char* flags,
                                                 int t0, const half8_t_ (&qb)[4], float scale_log2, int lane,
                                                 const Rows& rw) {
    constexpr int NS = kKvTile / 32;            // 32-token sub-tiles (one PV MFMA k-slab each)
    const int n = lane & 15;
    const int j = lane >> 4;
    const unsigned char* kb = buf;
    const unsigned char* vb = buf + kTileBytes;
    float4_t s2[2 * NS];
#pragma unroll
    for (int h = 0; h < 2 * NS; ++h) {
        float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const half8_t_ a = __builtin_bit_cast(half8_t_, *reinterpret_cast<const u32x4*>(
                                                               kb + (16 * h + n) * kPitch + 64 * c + 16 * j));
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qb[c], acc, 0, 0, 0);
        }
        s2[h] = acc;
    }
    // flags of this lane's tokens 16h + 4j .. 16h + 4j + 3: one dword per half
    float sc[8 * NS];
    float mt = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2 * NS; ++h) {
        const uint32_t fl = *reinterpret_cast<const uint32_t*>(flags + 16 * h + 4 * j);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int tok = 16 * h + 4 * j + e;
            const bool keep = rw.live && ((fl >> (8 * e)) & 0xffu) && t0 + tok <= rw.pos;
            sc[4 * h + e] = keep ? s2[h][e] * scale_log2 : -INFINITY;
            mt = fmaxf(mt, sc[4 * h + e]);
        }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(st.m, mt);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(st.m - m_use);
    half8_t_ p[NS];
    float lt = 0.f;
#pragma unroll
    for (int i = 0; i < 8 * NS; ++i) {
        // sub-tile u = i / 8 takes halves 2u (k 0..3 of each lane group) and 2u+1 (k 4..7)
        const _Float16 w = (_Float16)fast_exp2(sc[i] - m_use);
        p[i / 8][i % 8] = w;
        lt += (float)w;
    }
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    st.l = st.l * alpha + lt;
    st.m = m_new;
    if (__any(alpha != 1.f)) {
        float ar[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) ar[e] = __shfl(alpha, 4 * j + e);
#pragma unroll
        for (int c = 0; c < kDTiles; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) st.o[c][e] *= ar[e];
    }
    // V rows of the lane's 8 tokens of each sub-tile, columns 8n..8n+7; the
    // B operand of d-tile c is element c of each -- an 8 x 8 transpose of
    // halves, one v_perm_b32 per output dword (byte selectors: low halves of
    // two dwords, or high halves)
#pragma unroll
    for (int u = 0; u < NS; ++u) {
        u32x4 vv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int tok = 32 * u + ((i < 4) ? 4 * j + i : 16 + 4 * j + (i - 4));
            vv[i] = *reinterpret_cast<const u32x4*>(vb + tok * kPitch + 16 * n);
        }
#pragma unroll
        for (int c = 0; c < kDTiles; ++c) {
            const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
            const int dw = c >> 1;
            const u32x4 b = {__builtin_amdgcn_perm(vv[1][dw], vv[0][dw], sel),
                             __builtin_amdgcn_perm(vv[3][dw], vv[2][dw], sel),
                             __builtin_amdgcn_perm(vv[5][dw], vv[4][dw], sel),
                             __builtin_amdgcn_perm(vv[7][dw], vv[6][dw], sel)};
            st.o[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(p[u], __builtin_bit_cast(half8_t_, b), st.o[c], 0, 0, 0);
        }
    }
}

template <int B>
__global__ void __launch_bounds__(kThreads)
prefill_mfma_kernel(_Float16* __restrict__ out, const _Float16* __restrict__ q, int32_t num_tokens,
                    const _Float16* __restrict__ k_cache, const _Float16* __restrict__ v_cache,
                    const int32_t* __restrict__ tables, int32_t max_blocks, const int32_t* __restrict__ lens,
                    const int32_t* __restrict__ query_start, int32_t num_heads, int32_t num_kv_heads,
                    int32_t num_blocks, float scale_log2, int32_t max_query_len, int64_t len_cap) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[2][2 * kTileBytes];
    __shared__ __attribute__((aligned(4))) unsigned char lds_flags[2][kKvTile];
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
    const int grow0 = rtile * kRowsPerGroup;               // first row of the workgroup
    if (grow0 >= rows_all) return;                         // uniform over the workgroup
    const bool bad = m_raw > max_query_len || n_raw < m_raw || (int64_t)n_raw > len_cap;
    const int row0 = grow0 + wave * kRowsPerWave;          // first row of this wave
    const int rows = max(0, min(rows_all - row0, kRowsPerWave));
    const int nrow = lane & 15;
    const int jg = lane >> 4;
    if (bad) {                                             // the sequence's rows come out as NaN
        if (jg == 0 && nrow < rows) {
            const int r = row0 + nrow;
            const int64_t orow = ((int64_t)q0 + r / g) * num_heads + (int64_t)kvh * g + r % g;
            for (int d = 0; d < kD; ++d) out[orow * kD + d] = (_Float16)NAN;
        }
        return;                                            // uniform: bad depends on the sequence only
    }
    const int n = n_raw, m = m_raw;
    const int base_pos = n - m;

    Rows rw;
    rw.live = nrow < rows;
    const int r = row0 + (rw.live ? nrow : 0);
    rw.pos = base_pos + r / g;
    half8_t_ qb[4];
    {
        const _Float16* qrow = q + (((int64_t)q0 + r / g) * num_heads + (int64_t)kvh * g + r % g) * kD;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            qb[c] = __builtin_bit_cast(half8_t_, rw.live ? *reinterpret_cast<const u32x4*>(qrow + 32 * c + 8 * jg) : z);
        }
    }
    // the workgroup walks the tiles up to its last row's position; a wave
    // computes only up to its own last row's
    const int wg_rows = min(rows_all - grow0, kRowsPerGroup);
    const int ntiles = (base_pos + (grow0 + wg_rows - 1) / g) / kKvTile + 1;
    const int my_tiles = rows > 0 ? (base_pos + (row0 + rows - 1) / g) / kKvTile + 1 : 0;

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

    // Pipeline: tile k is consumed from LDS while tile k+1 waits in
    // registers and tile k+2 is being fetched -- each fetch has two tile
    // periods to land.  Registers sets R0/R1 alternate; LDS buffers too.
    Staged R0, R1;
    fetch_tile<B>(R0, 0, n, trow, kbase, vbase, blk_stride, num_blocks);
    if (ntiles > 1) fetch_tile<B>(R1, 1, n, trow, kbase, vbase, blk_stride, num_blocks);
    store_tile(R0, lds[0], lds_flags[0]);
    __syncthreads();
    auto step = [&](int k, Staged& fetch_into, const Staged& next) {
        const int cur = k & 1;
        if (k + 2 < ntiles) fetch_tile<B>(fetch_into, k + 2, n, trow, kbase, vbase, blk_stride, num_blocks);
        if (k < my_tiles) consume_lds_tile(st, lds[cur], lds_flags[cur], k * kKvTile, qb, scale_log2, lane, rw);
        if (k + 1 < ntiles) store_tile(next, lds[cur ^ 1], lds_flags[cur ^ 1]);
        __syncthreads();
    };
    for (int k = 0; k < ntiles; k += 2) {
        step(k, R0, R1);                    // R0 (tile k, now in LDS) refills with k+2; R1 holds k+1
        if (k + 1 < ntiles) step(k + 1, R1, R0);
    }

    // Rows 4*jg + e of the wave live in this lane's o[c][e] at column 8*nrow
    // + c; their sums sit in lanes 4*jg + e.
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int rr = 4 * jg + e;
        const float L = __shfl(st.l, rr);
        if (rr >= rows) continue;
        const int rwi = row0 + rr;
        const int64_t orow = ((int64_t)q0 + rwi / g) * num_heads + (int64_t)kvh * g + rwi % g;
        const float inv = L > 0.f ? 1.f / L : 0.f;
        half8_t h;
#pragma unroll
        for (int c = 0; c < kDTiles; ++c) h[c] = (_Float16)(st.o[c][e] * inv);
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

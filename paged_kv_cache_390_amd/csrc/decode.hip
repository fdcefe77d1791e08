// Single-query paged decode attention for gfx950 (CDNA4).
//
// What is computed: for every sequence s and query head h, the new token's
// query attends to the sequence's n cached keys/values, found through its
// block table; paging is invisible to the result, which is plain softmax
// attention over the logically contiguous K/V (lpnh.cn/news/1824136, 2.2 and
// 3.2 step 4; lpnh.cn/news/2758356, 2.2; the formula itself is not on the
// pages and is taken as textbook scaled dot-product attention).
//
// Design (MI355X first; the pages describe no kernel):
//  * Decode with one query per KV head is a GEMV: about one flop per byte of
//    K/V, far below the HBM ridge, so the work runs on VALU, not MFMA, and
//    every choice serves HBM streaming.
//  * Grid: one 256-thread workgroup (4 wave64s) per (query head, sequence,
//    context partition).  A partition is partition_size consecutive
//    tokens; sequences longer than one partition are split so that long
//    contexts still spread over all 256 CUs, and a second kernel merges the
//    partial softmax states.  Sequences that fit one partition are finished
//    by the first kernel directly.
//  * Longest first: grid row y works on sequence order[y], a permutation
//    that sorts the sequences by length (order_by_length_kernel, once per
//    step via pa_decode_order or inside the call).  Workgroups start in grid
//    order, and with a couple of workgroups per resident slot a long
//    sequence that started last would run alone through the drain; longest
//    processing time first keeps the drain short.
//  * XCD balance: workgroups are dealt round-robin to the 8 XCDs in linear
//    order, so the query head is the fastest grid dimension: every XCD then
//    gets the same heads of every (sequence, partition), i.e. the same bytes
//    to stream.  (With the partition fastest, a partition count sharing a
//    factor with 8 sends every sequence's first partition to the same XCDs
//    and only the long sequences' last ones to the others: measured 25%
//    slower on the Llama-2-7B batch.)
//  * Lane mapping: a token's head_dim fp16 values are 2*D bytes, read by
//    D/8 lanes with one 16-byte load each, so one wave load moves 1 KiB of
//    consecutive rows of a block's [block_size, head_dim] slab -- fully
//    coalesced however the blocks are scattered.  A wave step issues 4 such
//    loads for K and 4 for V before any math, keeping 8 KiB in flight per
//    wave.  Steps are dealt round-robin to the 4 waves.
//  * q.k: the lane's 8 fp16 products are summed with v_dot2_f32_f16 (fp32
//    accumulate) and the D/8-lane partial sums are combined with DPP
//    row/quad permutations (no LDS traffic).
//  * Softmax: online (running max m and sum l, in base-2 units with log2(e)
//    folded into the scale), kept separately per token row of the wave, so
//    the inner loop needs no cross-row communication; the 4 x (64*8/D) row
//    states of a workgroup are merged once through LDS at the end.
//  * Masking uses selects, never a multiply by zero, so garbage or NaN in
//    the unused rows of a tail block cannot leak; loads of masked rows are
//    not issued at all.
//  * The block table is read with wave-uniform (scalar) loads whenever the
//    rows of one wave load share a block (head_dim * block_size >= 512
//    elements); otherwise each lane looks up its own block.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "decode_internal.h"
#include "pa.h"
#include "pa_internal.h"

namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // one 16-byte load

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kLoadsPerStep = 4;          // 16-byte loads per lane per step, each for K and V
constexpr int kPartitionQuantum = 128;    // partition_size granularity (a multiple of every step)
constexpr double kLog2e = 1.4426950408889634073599246810019;

// DPP controls (GFX9 encoding).
constexpr int kDppQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <- lane 7-i within each 8
constexpr int kDppRowMirror = 0x140;      // lane i <- lane 15-i within each 16

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of G lanes; every lane of a group ends with the
// same bits (each stage adds two equal-bit partial sums in swapped order).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (G >= 2) v += dpp<kDppQuadXor1>(v);
    if constexpr (G >= 4) v += dpp<kDppQuadXor2>(v);
    if constexpr (G >= 8) v += dpp<kDppRowHalfMirror>(v);
    if constexpr (G >= 16) v += dpp<kDppRowMirror>(v);
    if constexpr (G >= 32) v += __shfl_xor(v, 16);
    return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

struct Frag {
    half2_t h[4];
};

__device__ __forceinline__ Frag as_frag(u32x4 u) { return __builtin_bit_cast(Frag, u); }

// Static geometry of one (head_dim, block_size) instance.
template <int D, int B>
struct Geo {
    static constexpr int LPT = D / 8;                   // lanes per token row (16 B each)
    static constexpr int TPL = 64 / LPT;                // token rows per wave load
    static constexpr int CH = TPL * kLoadsPerStep;      // tokens per wave step
    static constexpr bool kUniform = TPL <= B;          // a load's rows share one block
    static constexpr int NT = !kUniform ? kLoadsPerStep : (B >= CH ? 1 : CH / B);   // table reads per step
    static constexpr int LPB = B >= CH ? kLoadsPerStep : B / TPL;   // loads per table read (uniform case)
    static constexpr int64_t SLAB = (int64_t)B * D;     // elements of one (block, head) slab
};

// The K/V fragments of one step plus the validity of each load's row.
struct StepBuf {
    u32x4 k[kLoadsPerStep];
    u32x4 v[kLoadsPerStep];
    bool valid[kLoadsPerStep];
};

// Online-softmax state of one token row (identical in its D/8 lanes).
struct RowState {
    float m, l, acc[8];
};

template <int D>
__device__ __forceinline__ void consume(RowState& r, const StepBuf& b, const Frag& qf, float scale_log2) {
    constexpr int LPT = D / 8;
    float sc[kLoadsPerStep];
#pragma unroll
    for (int j = 0; j < kLoadsPerStep; ++j) {
        const Frag kh = as_frag(b.k[j]);
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) a = __builtin_amdgcn_fdot2(qf.h[i], kh.h[i], a, false);
        sc[j] = a;
    }
#pragma unroll
    for (int j = 0; j < kLoadsPerStep; ++j) sc[j] = group_sum<LPT>(sc[j]);
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kLoadsPerStep; ++j) {
        sc[j] = b.valid[j] ? sc[j] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, sc[j]);
    }
    const float m_new = fmaxf(r.m, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(r.m - m_use);
    r.l *= alpha;
#pragma unroll
    for (int i = 0; i < 8; ++i) r.acc[i] *= alpha;
#pragma unroll
    for (int j = 0; j < kLoadsPerStep; ++j) {
        const float p = fast_exp2(sc[j] - m_use);
        r.l += p;
        // a masked row was loaded as zeros (tail) or from a clamped block
        // (skipped id): select, so its values never reach the sum
        const Frag vh = as_frag(b.v[j]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float v0 = b.valid[j] ? (float)vh.h[i].x : 0.f;
            const float v1 = b.valid[j] ? (float)vh.h[i].y : 0.f;
            r.acc[2 * i] = fmaf(p, v0, r.acc[2 * i]);
            r.acc[2 * i + 1] = fmaf(p, v1, r.acc[2 * i + 1]);
        }
    }
    r.m = m_new;
}

// kAppend: the last position n - 1 of every sequence holds the token of
// this step, whose K/V come from new_k / new_v (token s, KV head h at s *
// new_stride + h * D) instead of the cache; the workgroup whose partition
// holds it folds it in as a one-row step and -- for the first query head of
// its KV head -- writes it into the cache through k_write / v_write.  The
// cache is read for positions < n - 1 only, so no workgroup reads the row
// being written.
template <int D, int B, bool kAppend>
__global__ void __launch_bounds__(kThreads)
decode_partition_kernel(_Float16* __restrict__ out, float* __restrict__ ws_ml, float* __restrict__ ws_acc,
                        const int32_t* __restrict__ order, const _Float16* __restrict__ q, const _Float16* __restrict__ k_cache,
                        const _Float16* __restrict__ v_cache, const int32_t* __restrict__ tables,
                        int32_t max_blocks, const int32_t* __restrict__ lens, int32_t num_heads,
                        int32_t num_kv_heads, int32_t num_blocks, float scale_log2, int32_t part_size,
                        int32_t num_parts, int64_t len_cap, const _Float16* __restrict__ new_k,
                        const _Float16* __restrict__ new_v, int64_t new_stride, _Float16* __restrict__ k_write,
                        _Float16* __restrict__ v_write) {
    using G = Geo<D, B>;
    constexpr int LPT = G::LPT;
    constexpr int TPL = G::TPL;
    constexpr int CH = G::CH;
    constexpr int NT = G::NT;
    constexpr int NSTATE = kWaves * TPL;        // softmax states per workgroup

    const int h = blockIdx.x;
    const int s = order ? order[blockIdx.y] : (int)blockIdx.y;   // longest sequences first
    if ((uint32_t)s >= gridDim.y) return;                         // not a sequence: nothing to do
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform by construction
    const int row = lane / LPT;
    const int col = lane % LPT;

    const int32_t n_raw = lens[s];
    const bool bad_len = n_raw < 0 || (int64_t)n_raw > len_cap;
    const int n = bad_len ? 0 : n_raw;
    const int part = blockIdx.z;
    const int start = part * part_size;
    if (part > 0 && start >= n) return;
    const int cached = kAppend && n > 0 ? n - 1 : n;   // positions read from the cache
    const int end = min(start + part_size, cached);
    const int np = (n + part_size - 1) / part_size;   // partitions of this sequence
    const int kvh = h / (num_heads / num_kv_heads);

    const Frag qf = as_frag(*reinterpret_cast<const u32x4*>(q + ((int64_t)s * num_heads + h) * D + col * 8));

    const int32_t* trow = tables + (int64_t)s * max_blocks;
    const _Float16* kbase = k_cache + (int64_t)kvh * G::SLAB;
    const _Float16* vbase = v_cache + (int64_t)kvh * G::SLAB;
    const int64_t blk_stride = (int64_t)num_kv_heads * G::SLAB;

    RowState r;
    r.m = -INFINITY;
    r.l = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) r.acc[i] = 0.f;

    // append mode: the new token's K/V, loaded now by every lane (a valid
    // address for all) so that the load hides under the main loop
    u32x4 new_kf = {0u, 0u, 0u, 0u}, new_vf = {0u, 0u, 0u, 0u};
    if constexpr (kAppend) {
        const int64_t src = (int64_t)s * new_stride + (int64_t)kvh * D + col * 8;
        new_kf = *reinterpret_cast<const u32x4*>(new_k + src);
        new_vf = *reinterpret_cast<const u32x4*>(new_v + src);
    }

    const int ntok = end > start ? end - start : 0;
    const int nsteps = ntok / CH;               // steps whose CH tokens are all < end
    const bool tail = ntok % CH != 0;

    // ---- full steps: unconditional loads, table prefetched one step ahead
    if constexpr (G::kUniform) {
        int32_t tnext[NT];                     // table entries of the next step to issue
        auto fetch = [&](int st, int32_t (&t)[NT]) {
#pragma unroll
            for (int k = 0; k < NT; ++k) t[k] = trow[(start + st * CH) / B + k];
        };
        auto issue = [&](StepBuf& b, int st) {
            const int t0 = start + st * CH;
            int32_t cur[NT];
#pragma unroll
            for (int k = 0; k < NT; ++k) cur[k] = tnext[k];
            const int nx = st + kWaves;
            if (nx < nsteps) fetch(nx, tnext);
#pragma unroll
            for (int k = 0; k < NT; ++k) {
                const bool ok = (uint32_t)cur[k] < (uint32_t)num_blocks;
                const int64_t blk = ok ? cur[k] : 0;   // a skipped id reads block 0, masked below
#pragma unroll
                for (int u = 0; u < G::LPB; ++u) {
                    const int j = k * G::LPB + u;
                    const int rowoff = (B >= CH ? t0 % B : 0) + u * TPL;
                    const int64_t off = blk * blk_stride + (int64_t)rowoff * D + lane * 8;
                    b.k[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + off));
                    b.v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vbase + off));
                    b.valid[j] = ok;
                }
            }
        };
        if (wave < nsteps) {
            fetch(wave, tnext);
            StepBuf A, Bf;
            int st = wave;
            issue(A, st);
            for (;;) {
                int nx = st + kWaves;
                if (nx >= nsteps) { consume<D>(r, A, qf, scale_log2); break; }
                issue(Bf, nx);
                consume<D>(r, A, qf, scale_log2);
                st = nx;
                nx = st + kWaves;
                if (nx >= nsteps) { consume<D>(r, Bf, qf, scale_log2); break; }
                issue(A, nx);
                consume<D>(r, Bf, qf, scale_log2);
                st = nx;
            }
        }
    } else {
        // rows of one load lie in several blocks: every lane looks up its own
        for (int st = wave; st < nsteps; st += kWaves) {
            const int t0 = start + st * CH;
            StepBuf b;
#pragma unroll
            for (int j = 0; j < kLoadsPerStep; ++j) {
                const int t = t0 + j * TPL + row;
                const int32_t phys = trow[t / B];
                const bool ok = (uint32_t)phys < (uint32_t)num_blocks;
                const int64_t off = (int64_t)(ok ? phys : 0) * blk_stride + (int64_t)(t % B) * D + col * 8;
                b.k[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + off));
                b.v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vbase + off));
                b.valid[j] = ok;
            }
            consume<D>(r, b, qf, scale_log2);
        }
    }

    // ---- the partial last step: per-row masks, loads of masked rows skipped
    if (tail && wave == nsteps % kWaves) {
        const int t0 = start + nsteps * CH;
        StepBuf b;
#pragma unroll
        for (int j = 0; j < kLoadsPerStep; ++j) {
            const int t = t0 + j * TPL + row;
            const bool in = t < end;
            const int tc = in ? t : end - 1;   // keeps the table index inside the sequence
            const int32_t phys = trow[tc / B];
            const bool ok = (uint32_t)phys < (uint32_t)num_blocks;
            b.valid[j] = in && ok;
            b.k[j] = u32x4{0, 0, 0, 0};
            b.v[j] = u32x4{0, 0, 0, 0};
            if (b.valid[j]) {
                const int64_t off = (int64_t)phys * blk_stride + (int64_t)(tc % B) * D + col * 8;
                b.k[j] = *reinterpret_cast<const u32x4*>(kbase + off);
                b.v[j] = *reinterpret_cast<const u32x4*>(vbase + off);
            }
        }
        consume<D>(r, b, qf, scale_log2);
    }
    if constexpr (kAppend) {
        const int pos = n - 1;                  // the new token
        if (n > 0 && pos >= start && pos < start + part_size && wave == kWaves - 1) {
            const int32_t phys = trow[pos / B];
            const bool ok = (uint32_t)phys < (uint32_t)num_blocks;   // as a cached row behind a skipped id
            StepBuf b;
#pragma unroll
            for (int j = 0; j < kLoadsPerStep; ++j) {
                b.k[j] = u32x4{0, 0, 0, 0};
                b.v[j] = u32x4{0, 0, 0, 0};
                b.valid[j] = false;
            }
            if (row == 0) {
                b.k[0] = new_kf;
                b.v[0] = new_vf;
                b.valid[0] = ok;
            }
            consume<D>(r, b, qf, scale_log2);
            if (row == 0 && ok && h % (num_heads / num_kv_heads) == 0) {
                const int64_t off = (int64_t)kvh * G::SLAB + (int64_t)phys * blk_stride + (int64_t)(pos % B) * D + col * 8;
                *reinterpret_cast<u32x4*>(k_write + off) = b.k[0];
                *reinterpret_cast<u32x4*>(v_write + off) = b.v[0];
            }
        }
    }
    const float m = r.m, l = r.l;
    const float* acc = r.acc;

    // Merge the NSTATE row states of the workgroup.  State k = wave*TPL+row
    // owns s_acc[k*D .. k*D+D); this lane's 8 values sit at (wave*64+lane)*8.
    __shared__ float s_m[NSTATE];
    __shared__ float s_l[NSTATE];
    __shared__ __attribute__((aligned(16))) float s_acc[NSTATE * D];
    {
        float4* dst = reinterpret_cast<float4*>(s_acc + (wave * 64 + lane) * 8);
        dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
        if (col == 0) {
            s_m[wave * TPL + row] = m;
            s_l[wave * TPL + row] = l;
        }
    }
    __syncthreads();

    float M = -INFINITY;
#pragma unroll 8
    for (int k = 0; k < NSTATE; ++k) M = fmaxf(M, s_m[k]);

    const int64_t head_row = (int64_t)s * num_heads + h;
    for (int d = threadIdx.x; d < D; d += kThreads) {
        float L = 0.f, o = 0.f;
#pragma unroll 8
        for (int k = 0; k < NSTATE; ++k) {
            const float mk = s_m[k];
            const float w = mk == -INFINITY ? 0.f : fast_exp2(mk - M);
            L = fmaf(w, s_l[k], L);
            o = fmaf(w, s_acc[k * D + d], o);
        }
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
}

// Merge the partitions of every sequence longer than one partition.
template <int D>
__global__ void __launch_bounds__(D < 64 ? 64 : D)
decode_reduce_kernel(_Float16* __restrict__ out, const float* __restrict__ ws_ml,
                     const float* __restrict__ ws_acc, const int32_t* __restrict__ order,
                     const int32_t* __restrict__ lens, int32_t num_heads, int32_t part_size, int32_t num_parts,
                     int64_t len_cap) {
    const int h = blockIdx.x;
    const int s = order ? order[blockIdx.y] : (int)blockIdx.y;   // the sequences the first kernel did
    if ((uint32_t)s >= gridDim.y) return;
    const int32_t n = lens[s];
    if (n < 0 || (int64_t)n > len_cap) return;   // written as NaN by the first kernel
    const int np = (n + part_size - 1) / part_size;
    if (np <= 1) return;
    const int64_t head_row = (int64_t)s * num_heads + h;
    const int64_t base = head_row * num_parts;
    float M = -INFINITY;
    for (int p = 0; p < np; ++p) M = fmaxf(M, ws_ml[2 * (base + p)]);
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
        float L = 0.f, o = 0.f;
        for (int p = 0; p < np; ++p) {
            const float mp = ws_ml[2 * (base + p)];
            const float w = mp == -INFINITY ? 0.f : fast_exp2(mp - M);
            L = fmaf(w, ws_ml[2 * (base + p) + 1], L);
            o = fmaf(w, ws_acc[(base + p) * D + d], o);
        }
        out[head_row * D + d] = L > 0.f ? (_Float16)(o / L) : (_Float16)0.f;
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_head_dim(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128 || d == 256; }

bool supported_block_size(int32_t b) {
    return b == 1 || b == 2 || b == 4 || b == 8 || b == 16 || b == 32 || b == 64 || b == 128;
}

// Longest-first order of the sequences: a counting sort of the lengths into
// kOrderClasses classes of `width` tokens, longest class first.  Workgroups
// start in grid order, so handing the longest sequences to the first ones
// keeps a long sequence from starting last and running alone through the
// drain.  Within a class the order is whatever the atomics give: every order
// computes the same outputs (each workgroup's work depends only on which
// sequence it takes), it only changes when each one starts.
constexpr int kOrderClasses = 1024;

__global__ void __launch_bounds__(kOrderClasses)
order_by_length_kernel(int32_t* __restrict__ order, const int32_t* __restrict__ lens, int32_t num_seqs,
                       int32_t width) {
    __shared__ int32_t count[kOrderClasses];
    __shared__ int32_t scan[2][kOrderClasses];
    const int t = threadIdx.x;
    auto cls = [&](int32_t n) {
        const int32_t c = n < 0 ? 0 : n / width;
        return c < kOrderClasses - 1 ? c : kOrderClasses - 1;
    };
    count[t] = 0;
    __syncthreads();
    for (int s = t; s < num_seqs; s += kOrderClasses) atomicAdd(&count[cls(lens[s])], 1);
    __syncthreads();
    // first slot of class c = sequences in the classes above it: an inclusive
    // scan over the classes taken longest first, minus the class's own count
    const int rc = kOrderClasses - 1 - t;
    int cur = 0;
    scan[0][t] = count[rc];
    __syncthreads();
    for (int off = 1; off < kOrderClasses; off <<= 1) {
        scan[cur ^ 1][t] = scan[cur][t] + (t >= off ? scan[cur][t - off] : 0);
        cur ^= 1;
        __syncthreads();
    }
    count[rc] = scan[cur][t] - count[rc];               // thread t alone owns entry rc
    __syncthreads();
    for (int s = t; s < num_seqs; s += kOrderClasses) order[atomicAdd(&count[cls(lens[s])], 1)] = s;
}

void launch_order(int32_t* order, const int32_t* lens, int32_t num_seqs, int32_t max_context_len, hipStream_t st) {
    const int32_t width = max_context_len / kOrderClasses + 1;
    hipLaunchKernelGGL(order_by_length_kernel, dim3(1), dim3(kOrderClasses), 0, st, order, lens, num_seqs, width);
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace: the longest-first sequence order (int32 per sequence, when
// there are two or more), then for split sequences the partial (m, l) and
// the partial O of every (sequence, head, partition); each region aligned to
// 256 bytes.
struct Layout {
    int32_t part_size;
    int32_t num_parts;
    size_t order_bytes;
    size_t ml_bytes;
    size_t total;
};

Layout workspace_layout(int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t max_context_len,
                        int32_t part_size) {
    Layout L{};
    L.part_size = part_size;
    const int64_t np = max_context_len > 0 ? ((int64_t)max_context_len + part_size - 1) / part_size : 1;
    L.num_parts = (int32_t)(np > 0 ? np : 1);
    L.order_bytes = num_seqs > 1 ? align_up((size_t)num_seqs * sizeof(int32_t), 256) : 0;
    L.total = L.order_bytes;
    if (L.num_parts <= 1) return L;
    const size_t rows = (size_t)num_seqs * num_heads * L.num_parts;
    L.ml_bytes = align_up(rows * 2 * sizeof(float), 256);
    L.total += L.ml_bytes + align_up(rows * head_dim * sizeof(float), 256);
    return L;
}

using MainFn = void (*)(_Float16*, float*, float*, const int32_t*, const _Float16*, const _Float16*, const _Float16*,
                        const int32_t*, int32_t, const int32_t*, int32_t, int32_t, int32_t, float, int32_t,
                        int32_t, int64_t, const _Float16*, const _Float16*, int64_t, _Float16*, _Float16*);
using ReduceFn = void (*)(_Float16*, const float*, const float*, const int32_t*, const int32_t*, int32_t, int32_t,
                          int32_t, int64_t);

template <int D, bool kAppend>
MainFn pick_main(int32_t b) {
    switch (b) {
        case 1: return decode_partition_kernel<D, 1, kAppend>;
        case 2: return decode_partition_kernel<D, 2, kAppend>;
        case 4: return decode_partition_kernel<D, 4, kAppend>;
        case 8: return decode_partition_kernel<D, 8, kAppend>;
        case 16: return decode_partition_kernel<D, 16, kAppend>;
        case 32: return decode_partition_kernel<D, 32, kAppend>;
        case 64: return decode_partition_kernel<D, 64, kAppend>;
        case 128: return decode_partition_kernel<D, 128, kAppend>;
        default: return nullptr;
    }
}

template <bool kAppend>
MainFn pick_main(int32_t d, int32_t b) {
    switch (d) {
        case 16: return pick_main<16, kAppend>(b);
        case 32: return pick_main<32, kAppend>(b);
        case 64: return pick_main<64, kAppend>(b);
        case 128: return pick_main<128, kAppend>(b);
        case 256: return pick_main<256, kAppend>(b);
        default: return nullptr;
    }
}

ReduceFn pick_reduce(int32_t d) {
    switch (d) {
        case 16: return decode_reduce_kernel<16>;
        case 32: return decode_reduce_kernel<32>;
        case 64: return decode_reduce_kernel<64>;
        case 128: return decode_reduce_kernel<128>;
        case 256: return decode_reduce_kernel<256>;
        default: return nullptr;
    }
}

bool uses_mfma(int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size) {
    const int32_t group = num_kv_heads > 0 ? num_heads / num_kv_heads : 1;
    return pa::gqa_mfma_supported(head_dim, block_size, group);
}

// workgroups per partition index: one per (sequence, query head), or per
// (sequence, KV head) on the grouped-query kernel
int64_t grid_rows(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size) {
    return (int64_t)num_seqs * (uses_mfma(num_heads, num_kv_heads, head_dim, block_size) ? num_kv_heads : num_heads);
}

// workgroups resident at once: 256 CUs x 4 (vector kernel, 108 VGPRs) or,
// for the grouped-query kernel, as many as its registers allow
int64_t resident_slots(int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size) {
    if (!uses_mfma(num_heads, num_kv_heads, head_dim, block_size)) return 256LL * 4;
    // the matrix-core kernel's registers: 4 workgroups per CU at head_dim 64,
    // 1 at head_dim 256 with tiles across blocks, 2 otherwise
    if (head_dim == 64) return 256LL * 4;
    if (block_size < 16 && head_dim == 256) return 256LL * 1;
    return 256LL * 2;
}

// Default partition.  Rows are the workgroups one partition index gives
// (grid_rows), slots the workgroups resident at once (resident_slots), and
// "cover" the bound rounded up to the partition quantum: one partition for
// every context, no partial states, no merge kernel.
//  * At least half a round and at most one round of rows (rows in [slots/2,
//    slots]): cover.  Every workgroup is resident at once, so nothing waits
//    behind a long sequence, and splitting only adds the merge.
//  * More than one round: cover when its workgroups fill the slots a whole
//    number of times or leave the last round at least 3/4 full; with the
//    sequences dispatched longest first the drain is then short.  A last
//    round mostly empty would run its few workgroups alone when the lengths
//    are alike, so then the longest of 2048 / 1024 / 512 / 256 tokens that
//    gives at least four workgroups per slot, counting full partitions of a
//    longest sequence (the bound may exceed every actual length).
//  * Fewer rows than half a round: the context is cut into enough parts for
//    one workgroup per compute unit (256), parts of at least 256 tokens.
// Measured (decode call, same process, interleaved; U[1, bound] contexts
// unless stated): 64 x 32 heads at bounds 2600 / 3072 / 4096: 2048-token
// partitions 3.2 / 3.3 / 4.1% slower than cover; 16 x 4096 uniform (half a
// round): 512 2.6% slower than cover; 32 / 64 sequences of 8 KV heads x 8
// query heads (half / one round on the matrix-core kernel): 256 / 512 5 / 11%
// slower than cover; 4 x 4096 uniform (1/8 round): two parts of 2048 take
// 19% less time than cover; 100 requests of 1001..1200 tokens sharing a
// 1000-token prompt (3.1 rounds): 512 gives 10% more than cover.  Cover is
// 5% slower than 512 in one measured case: 16 sequences with contexts
// U[1, 4096] (the few longest sequences' workgroups then set the pace).
int32_t default_partition(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t max_context_len) {
    const int64_t rows = grid_rows(num_seqs, num_heads, num_kv_heads, head_dim, block_size);
    const int64_t slots = resident_slots(num_heads, num_kv_heads, head_dim, block_size);
    const int64_t bound = max_context_len > 0 ? max_context_len : 1;
    const int64_t cover64 = (bound + kPartitionQuantum - 1) / kPartitionQuantum * kPartitionQuantum;
    const int32_t cover = (int32_t)(cover64 < 0x7fffff80 ? cover64 : 0x7fffff80);
    if (rows <= 0) return cover;
    if (2 * rows >= slots && rows <= slots) return cover;
    if (rows > slots) {
        const int64_t tail = rows % slots;
        if (tail == 0 || 4 * tail >= 3 * slots) return cover;
        const int32_t cands[] = {2048, 1024, 512, 256};
        for (int32_t p : cands) {
            const int64_t parts = bound / p > 0 ? bound / p : 1;
            if (rows * parts >= 4 * slots) return p;
        }
        return 256;
    }
    // fewer rows than half a round: one workgroup per compute unit
    const int64_t parts = (256 + rows - 1) / rows;
    int64_t p = (bound + parts - 1) / parts;
    p = (p + kPartitionQuantum - 1) / kPartitionQuantum * kPartitionQuantum;
    return (int32_t)(p < 256 ? 256 : p);
}

bool bad_geometry(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                  int32_t max_context_len, int32_t partition_size) {
    return num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 ||
           !supported_head_dim(head_dim) || max_context_len < 0 || partition_size < 0 ||
           partition_size % kPartitionQuantum != 0;
}

}  // namespace

extern "C" int32_t pa_decode_default_partition(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                               int32_t head_dim, int32_t block_size, int32_t max_context_len) {
    if (bad_geometry(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len, 0) ||
        !supported_block_size(block_size))
        return -1;
    return default_partition(num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_context_len);
}

extern "C" size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size, int32_t max_context_len,
                                           int32_t partition_size) {
    if (bad_geometry(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len, partition_size) ||
        !supported_block_size(block_size))
        return (size_t)-1;
    const int32_t p = partition_size ? partition_size
                                     : default_partition(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                                         max_context_len);
    return workspace_layout(num_seqs, num_heads, head_dim, max_context_len, p).total;
}

extern "C" int pa_decode_order(int32_t* seq_order, const int32_t* context_lens, int32_t num_seqs,
                               int32_t max_context_len, void* stream) {
    if (num_seqs < 0 || num_seqs > 65535 || max_context_len < 0)
        return pa::fail(PA_ERR_INVALID, "pa_decode_order: bad sizes (S=%d max_len=%d)", num_seqs, max_context_len);
    if (num_seqs == 0) return PA_OK;
    if (!seq_order || !context_lens) return pa::fail(PA_ERR_INVALID, "pa_decode_order: null pointer");
    launch_order(seq_order, context_lens, num_seqs, max_context_len, static_cast<hipStream_t>(stream));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return pa::fail(PA_ERR_HIP, "pa_decode_order: %s", hipGetErrorString(e));
    return PA_OK;
}

namespace {

// The step's new tokens when pa_decode_append folds their write into the
// call (null otherwise).
struct Append {
    const _Float16* key;
    const _Float16* value;
    int64_t stride;
};

int decode_impl(const char* fn, void* out, const void* q, const void* k_cache, const void* v_cache,
                const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                int32_t num_blocks, float scale, int32_t max_context_len, int32_t partition_size, void* workspace,
                size_t workspace_bytes, const int32_t* seq_order, int32_t dtype, void* stream, const Append* app) {
    if (dtype != PA_DTYPE_F16) return pa::fail(PA_ERR_UNSUPPORTED, "%s: dtype %d", fn, dtype);
    if (!supported_head_dim(head_dim)) return pa::fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d", fn, head_dim);
    if (!supported_block_size(block_size))
        return pa::fail(PA_ERR_UNSUPPORTED, "%s: block_size %d", fn, block_size);
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 ||
        num_blocks <= 0 || max_blocks_per_seq < 0 || max_context_len < 0 || partition_size < 0)
        return pa::fail(PA_ERR_INVALID, "%s: bad sizes (S=%d H=%d Hkv=%d NB=%d W=%d max_len=%d P=%d)", fn,
                        num_seqs, num_heads, num_kv_heads, num_blocks, max_blocks_per_seq, max_context_len,
                        partition_size);
    if (partition_size % kPartitionQuantum != 0)
        return pa::fail(PA_ERR_INVALID, "%s: partition_size %d is not a multiple of %d", fn, partition_size,
                        kPartitionQuantum);
    if (num_seqs > 65535 || num_heads > 65535)
        return pa::fail(PA_ERR_INVALID, "%s: num_seqs and num_heads must be <= 65535", fn);
    if (!std::isfinite(scale)) return pa::fail(PA_ERR_INVALID, "%s: scale is not finite", fn);
    if (num_seqs == 0) return PA_OK;
    if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
        return pa::fail(PA_ERR_INVALID, "%s: null pointer", fn);
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
        return pa::fail(PA_ERR_INVALID, "%s: out, q and caches must be 16-byte aligned", fn);
    if (app) {
        if (!app->key || !app->value) return pa::fail(PA_ERR_INVALID, "%s: null key or value", fn);
        if (!aligned16(app->key) || !aligned16(app->value) || app->stride % 8 != 0)
            return pa::fail(PA_ERR_INVALID, "%s: key, value and kv_token_stride must be 16-byte aligned", fn);
        if (app->stride < (int64_t)num_kv_heads * head_dim)
            return pa::fail(PA_ERR_INVALID, "%s: kv_token_stride %lld < num_kv_heads * head_dim", fn,
                            (long long)app->stride);
    }

    const int32_t p = partition_size ? partition_size
                                     : default_partition(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                                         max_context_len);
    const Layout L = workspace_layout(num_seqs, num_heads, head_dim, max_context_len, p);
    if (L.num_parts > 1) {
        if (!workspace) return pa::fail(PA_ERR_INVALID, "%s: workspace of %zu bytes required", fn, L.total);
        if (workspace_bytes < L.total)
            return pa::fail(PA_ERR_INVALID, "%s: workspace %zu < %zu bytes", fn, workspace_bytes, L.total);
    }
    if (workspace && !aligned16(workspace))
        return pa::fail(PA_ERR_INVALID, "%s: workspace must be 16-byte aligned", fn);
    // the caller's order if given; else one computed here into the
    // workspace (with one partition the workspace only holds that order, and
    // without one -- NULL or smaller -- the sequences run in index order).
    // When every workgroup is resident at once the order cannot matter, and
    // the small kernel is skipped.
    const bool compute_order = !seq_order && L.order_bytes > 0 && workspace && workspace_bytes >= L.total &&
                               (int64_t)grid_rows(num_seqs, num_heads, num_kv_heads, head_dim, block_size) *
                                       L.num_parts > resident_slots(num_heads, num_kv_heads, head_dim, block_size);
    if (L.num_parts > 65535)
        return pa::fail(PA_ERR_INVALID, "%s: max_context_len %d needs %d partitions of %d (limit 65535)", fn,
                        max_context_len, L.num_parts, p);
    // a row is computed only when its length fits the table, the grid and
    // the caller's bound; any other row comes out as NaN
    int64_t len_cap = (int64_t)max_blocks_per_seq * block_size;
    if ((int64_t)L.num_parts * p < len_cap) len_cap = (int64_t)L.num_parts * p;
    if ((int64_t)max_context_len < len_cap) len_cap = max_context_len;

    if (pa::validate_enabled())
        if (int rc = pa::validate_tables(fn, block_tables, max_blocks_per_seq, context_lens, num_seqs, block_size,
                                         num_blocks, max_context_len, stream))
            return rc;

    char* wsb = static_cast<char*>(workspace);
    int32_t* own_order = compute_order ? reinterpret_cast<int32_t*>(wsb) : nullptr;
    const int32_t* order = seq_order ? seq_order : own_order;
    float* ws_ml = L.num_parts > 1 ? reinterpret_cast<float*>(wsb + L.order_bytes) : nullptr;
    float* ws_acc = L.num_parts > 1 ? reinterpret_cast<float*>(wsb + L.order_bytes + L.ml_bytes) : nullptr;
    const float scale_log2 = (float)((double)scale * kLog2e);
    auto st = static_cast<hipStream_t>(stream);

    hipError_t e;
    if (own_order) {
        launch_order(own_order, context_lens, num_seqs, max_context_len, st);
        e = hipGetLastError();
        if (e != hipSuccess) return pa::fail(PA_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
    }

    const int32_t group = num_heads / num_kv_heads;
    if (pa::gqa_mfma_supported(head_dim, block_size, group)) {
        // several query heads per KV head: the products are contractions -> matrix cores
        pa::DecodeLaunch a{static_cast<_Float16*>(out), ws_ml, ws_acc, order, static_cast<const _Float16*>(q),
                           static_cast<const _Float16*>(k_cache), static_cast<const _Float16*>(v_cache),
                           block_tables, max_blocks_per_seq, context_lens, num_seqs, num_heads, num_kv_heads,
                           num_blocks, block_size, head_dim, scale_log2, p, L.num_parts, len_cap, st,
                           app ? app->key : nullptr, app ? app->value : nullptr, app ? app->stride : 0};
        e = pa::launch_gqa_mfma(a);
    } else {
        MainFn main_fn = app ? pick_main<true>(head_dim, block_size) : pick_main<false>(head_dim, block_size);
        // the cache pointers double as write pointers in append mode: the
        // kernel writes only the row of each sequence's last position, which
        // no workgroup reads from the cache
        hipLaunchKernelGGL(main_fn, dim3((unsigned)num_heads, (unsigned)num_seqs, (unsigned)L.num_parts),
                           dim3(kThreads), 0, st, static_cast<_Float16*>(out), ws_ml, ws_acc, order,
                           static_cast<const _Float16*>(q), static_cast<const _Float16*>(k_cache),
                           static_cast<const _Float16*>(v_cache), block_tables, max_blocks_per_seq, context_lens,
                           num_heads, num_kv_heads, num_blocks, scale_log2, p, L.num_parts, len_cap,
                           app ? app->key : nullptr, app ? app->value : nullptr, app ? app->stride : (int64_t)0,
                           app ? static_cast<_Float16*>(const_cast<void*>(k_cache)) : nullptr,
                           app ? static_cast<_Float16*>(const_cast<void*>(v_cache)) : nullptr);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return pa::fail(PA_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
    if (L.num_parts > 1) {
        const unsigned threads = head_dim < 64 ? 64u : (unsigned)head_dim;
        hipLaunchKernelGGL(pick_reduce(head_dim), dim3((unsigned)num_heads, (unsigned)num_seqs), dim3(threads), 0,
                           st, static_cast<_Float16*>(out), (const float*)ws_ml, (const float*)ws_acc, order,
                           context_lens, num_heads, p, L.num_parts, len_cap);
        e = hipGetLastError();
        if (e != hipSuccess) return pa::fail(PA_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
    }
    return PA_OK;
}

}  // namespace

extern "C" int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                         float scale, int32_t max_context_len, int32_t partition_size, void* workspace,
                         size_t workspace_bytes, const int32_t* seq_order, int32_t dtype, void* stream) {
    return decode_impl("pa_decode", out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, max_context_len,
                       partition_size, workspace, workspace_bytes, seq_order, dtype, stream, nullptr);
}

extern "C" int pa_decode_append(void* out, const void* q, const void* key, const void* value,
                                int64_t kv_token_stride, void* k_cache, void* v_cache, const int32_t* block_tables,
                                int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                                int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                int32_t num_blocks, float scale, int32_t max_context_len, int32_t partition_size,
                                void* workspace, size_t workspace_bytes, const int32_t* seq_order, int32_t dtype,
                                void* stream) {
    const Append app{static_cast<const _Float16*>(key), static_cast<const _Float16*>(value), kv_token_stride};
    return decode_impl("pa_decode_append", out, q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                       max_context_len, partition_size, workspace, workspace_bytes, seq_order, dtype, stream, &app);
}

// ---------------------------------------------------------------------------
// pa_decode_noalloc: pa_decode with its workspace held by the library, for
// callers that cannot allocate device memory.  The workspace lives in a
// file-scope device array (one copy per GPU, kept until the process ends);
// its device address is looked up once per device with that device current
// and kept, and only that address is ever handed to kernels.  Nothing in it
// has to start at zero: the order kernel writes every entry it later reads,
// and the partition kernel writes every partial state before the merge
// kernel reads it.
namespace {

constexpr size_t kScratchBytes = PA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(const char* fn, void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return pa::fail(PA_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return pa::fail(PA_ERR_HIP, "%s: device %d out of range", fn, dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return pa::fail(PA_ERR_HIP, "%s: hipGetSymbolAddress: %s", fn, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return PA_OK;
}

}  // namespace

extern "C" int pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                 float scale, int32_t max_context_len, int32_t partition_size,
                                 const int32_t* seq_order, int32_t dtype, void* stream) {
    const char* fn = "pa_decode_noalloc";
    // the same argument checks and workspace layout as pa_decode; sizes
    // that pa_decode would refuse are refused by decode_impl below
    if (!bad_geometry(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len, partition_size) &&
        supported_block_size(block_size) && num_seqs > 0) {
        const int32_t p = partition_size ? partition_size
                                         : default_partition(num_seqs, num_heads, num_kv_heads, head_dim,
                                                             block_size, max_context_len);
        const size_t need = workspace_layout(num_seqs, num_heads, head_dim, max_context_len, p).total;
        if (need > kScratchBytes)
            return pa::fail(PA_ERR_INVALID,
                            "%s: these sizes need %zu bytes of workspace, above the library's %zu-byte scratch; "
                            "call pa_decode with a workspace instead (or a longer partition_size)",
                            fn, need, kScratchBytes);
    }
    void* ws = nullptr;
    if (num_seqs > 0) {
        const int rc = scratch_address(fn, &ws);
        if (rc != PA_OK) return rc;
    }
    return decode_impl(fn, out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                       num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, max_context_len,
                       partition_size, ws, ws ? kScratchBytes : 0, seq_order, dtype, stream, nullptr);
}

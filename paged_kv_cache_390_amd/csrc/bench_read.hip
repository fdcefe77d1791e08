// Read-only streaming kernels: measurement aids that give the same-chip
// ceiling the decode kernels are judged against.  They compute nothing of
// the method -- every byte is loaded once with the decode kernels' load form
// (16 bytes per lane, nontemporal) and folded into an XOR so that no load
// can be dropped -- and write one 32-bit word per workgroup.
//
//  * stream_read_kernel: consecutive 1 MiB pieces of one buffer, one piece
//    per workgroup (the plainest streaming read).
//  * block_read_kernel: the decode access pattern without its arithmetic --
//    one workgroup per (KV head, sequence) reads the K and the V slab of
//    every block its table lists for the sequence's n tokens (whole blocks),
//    in table order, scattered over the pool however the table scatters
//    them, on the decode kernel's schedule (1 KiB wave loads, 4 K + 4 V per
//    wave step, two steps in flight).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa_bench.h"
#include "pa_internal.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kInFlight = 16;                       // 16-byte loads per lane before any is used
constexpr int64_t kPiece = 1 << 20;                 // bytes per workgroup (stream_read_kernel)
constexpr int64_t kPieceUnits = kPiece / 16;

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

__device__ __forceinline__ void store_folded(uint32_t* sink, uint32_t x) {
    __shared__ uint32_t part[kThreads / 64];
    for (int o = 32; o > 0; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int w = 0; w < kThreads / 64; ++w) r ^= part[w];
        sink[blockIdx.x] = r;
    }
}

__global__ void __launch_bounds__(kThreads)
stream_read_kernel(const u32x4* __restrict__ src, int64_t units, uint32_t* __restrict__ sink) {
    const int64_t begin = (int64_t)blockIdx.x * kPieceUnits;
    const int64_t end = begin + kPieceUnits < units ? begin + kPieceUnits : units;
    uint32_t x = 0;
    int64_t i = begin + threadIdx.x;
    // whole rounds: kInFlight loads per lane issued before the first is used
    for (; i + (kInFlight - 1) * kThreads < end; i += kInFlight * kThreads) {
        u32x4 v[kInFlight];
#pragma unroll
        for (int j = 0; j < kInFlight; ++j) v[j] = __builtin_nontemporal_load(src + i + j * kThreads);
#pragma unroll
        for (int j = 0; j < kInFlight; ++j) x ^= fold(v[j]);
    }
    for (; i < end; i += kThreads) x ^= fold(__builtin_nontemporal_load(src + i));
    store_folded(sink, x);
}

// Grid: x = KV head fastest, then sequence (order as pa_decode's vector
// kernel deals its heads to the XCDs).  A (block, head) slab of slab_units
// sixteen-byte units is cut into chunks of 64 units (1 KiB: one wave load);
// the chunks of a sequence, in table order, are grouped in steps of 4, and
// wave w takes steps w, w + 4, ... -- the decode kernel's schedule -- with
// the next step's 4 K and 4 V loads issued before the current step's are
// used (two steps in flight per wave).
constexpr int kWaves = kThreads / 64;
constexpr int kChunksPerStep = 4;

struct StepLoads {
    u32x4 k[kChunksPerStep], v[kChunksPerStep];
};

__global__ void __launch_bounds__(kThreads)
block_read_kernel(const u32x4* __restrict__ k_cache, const u32x4* __restrict__ v_cache,
                  const int32_t* __restrict__ tables, int32_t max_blocks, const int32_t* __restrict__ lens,
                  int32_t num_kv_heads, int32_t block_size, int32_t num_blocks, int32_t slab_units,
                  int32_t chunk_shift, uint32_t* __restrict__ sink) {
    const int h = blockIdx.x % num_kv_heads;
    const int s = blockIdx.x / num_kv_heads;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int32_t n = lens[s];
    if (n < 0) n = 0;
    int32_t nblk = (n + block_size - 1) / block_size;
    if (nblk > max_blocks) nblk = max_blocks;
    const int32_t* trow = tables + (int64_t)s * max_blocks;
    const int64_t blk_units = (int64_t)num_kv_heads * slab_units;
    const u32x4* kb = k_cache + (int64_t)h * slab_units + lane;
    const u32x4* vb = v_cache + (int64_t)h * slab_units + lane;
    const int32_t chunks = nblk << chunk_shift;
    const int32_t steps = (chunks + kChunksPerStep - 1) / kChunksPerStep;
    const int32_t cmask = (1 << chunk_shift) - 1;
    auto issue = [&](StepLoads& b, int32_t st) {
#pragma unroll
        for (int c = 0; c < kChunksPerStep; ++c) {
            int32_t ci = st * kChunksPerStep + c;
            if (ci >= chunks) ci = chunks - 1;                // past the end: the last chunk again
            int32_t phys = trow[ci >> chunk_shift];
            if ((uint32_t)phys >= (uint32_t)num_blocks) phys = 0;
            const int64_t off = (int64_t)phys * blk_units + (int64_t)(ci & cmask) * 64;
            b.k[c] = __builtin_nontemporal_load(kb + off);
            b.v[c] = __builtin_nontemporal_load(vb + off);
        }
    };
    uint32_t x = 0;
    auto use = [&](const StepLoads& b) {
#pragma unroll
        for (int c = 0; c < kChunksPerStep; ++c) x ^= fold(b.k[c]) ^ fold(b.v[c]);
    };
    if (wave < steps) {
        StepLoads A, Bf;
        int32_t st = wave;
        issue(A, st);
        for (;;) {
            int32_t nx = st + kWaves;
            if (nx >= steps) { use(A); break; }
            issue(Bf, nx);
            use(A);
            st = nx;
            nx = st + kWaves;
            if (nx >= steps) { use(Bf); break; }
            issue(A, nx);
            use(Bf);
            st = nx;
        }
    }
    store_folded(sink, x);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" int64_t pa_bench_stream_read_groups(size_t bytes) {
    return (int64_t)((bytes + kPiece - 1) / kPiece);
}

extern "C" int pa_bench_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    if (!buf || !sink) return pa::fail(PA_ERR_INVALID, "pa_bench_stream_read: null pointer");
    if (!aligned16(buf) || bytes % 16 != 0)
        return pa::fail(PA_ERR_INVALID, "pa_bench_stream_read: buffer must be 16-byte aligned and sized");
    const int64_t groups = pa_bench_stream_read_groups(bytes);
    if (groups == 0) return PA_OK;
    if (groups > 0x7fffffff) return pa::fail(PA_ERR_INVALID, "pa_bench_stream_read: buffer too large");
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)groups), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(buf), (int64_t)(bytes / 16), sink);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return pa::fail(PA_ERR_HIP, "pa_bench_stream_read: %s", hipGetErrorString(e));
    return PA_OK;
}

extern "C" int pa_bench_block_read(const void* k_cache, const void* v_cache, const int32_t* block_tables,
                                   int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                   uint32_t* sink, void* stream) {
    if (num_seqs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0 ||
        max_blocks_per_seq < 0)
        return pa::fail(PA_ERR_INVALID, "pa_bench_block_read: bad sizes");
    const int64_t su = (int64_t)block_size * head_dim * 2 / 16;
    if (((int64_t)block_size * head_dim * 2) % 16 != 0 || su < 64 || su > (1 << 20) || (su & (su - 1)) != 0)
        return pa::fail(PA_ERR_INVALID,
                        "pa_bench_block_read: a slab must be a power-of-two number of KiB (block_size * head_dim "
                        ">= 512)");
    if ((int64_t)max_blocks_per_seq * (su / 64) > 0x7fffffff)
        return pa::fail(PA_ERR_INVALID, "pa_bench_block_read: table too wide");
    const int64_t groups = (int64_t)num_seqs * num_kv_heads;
    if (groups == 0) return PA_OK;
    if (groups > 0x7fffffff) return pa::fail(PA_ERR_INVALID, "pa_bench_block_read: grid too large");
    if (!k_cache || !v_cache || !block_tables || !context_lens || !sink)
        return pa::fail(PA_ERR_INVALID, "pa_bench_block_read: null pointer");
    if (!aligned16(k_cache) || !aligned16(v_cache))
        return pa::fail(PA_ERR_INVALID, "pa_bench_block_read: caches must be 16-byte aligned");
    const int32_t slab_units = (int32_t)su;
    const int32_t chunk_shift = __builtin_ctzll((unsigned long long)(su / 64));
    hipLaunchKernelGGL(block_read_kernel, dim3((unsigned)groups), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(k_cache), static_cast<const u32x4*>(v_cache), block_tables,
                       max_blocks_per_seq, context_lens, num_kv_heads, block_size, num_blocks, slab_units, chunk_shift,
                       sink);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return pa::fail(PA_ERR_HIP, "pa_bench_block_read: %s", hipGetErrorString(e));
    return PA_OK;
}

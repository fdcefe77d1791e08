// Slot-mapped cache write and whole-block copy for gfx950.
//
// Both are pure data movement: every lane moves 16 bytes (8 fp16 values)
// per load/store when the addresses allow it, else 2 bytes.  Neither needs
// LDS or MFMA; they are bound by launch latency at decode batch sizes
// (reshape) or by HBM bandwidth (block copy).
//
// Sources (pages named by address, sections as they number them):
//   [lpnh-1824136]  lpnh.cn/news/1824136, 3.1: results are scattered back
//                   into the proper blocks
//   [lpnh-2758356]  lpnh.cn/news/2758356, 2.2 (slot = block id * block size
//                   + row), 4.2 third step (copy the whole shared block into
//                   the new one), 4.3 (that copy costs bandwidth)
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa.h"
#include "pa_internal.h"

namespace {

constexpr int kThreads = 256;

// One lane per (token, head, VEC-element chunk); K and V move together.
template <int VEC>
__global__ void __launch_bounds__(kThreads)
scatter_kv_kernel(const uint16_t* __restrict__ key, const uint16_t* __restrict__ value,
                  int64_t token_stride, const int64_t* __restrict__ slots, int64_t work,
                  uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache,
                  int64_t pool_slots, int32_t num_kv_heads, int32_t block_size,
                  int32_t head_dim) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= work) return;
    const int32_t chunks = head_dim / VEC;
    const int64_t per_token = (int64_t)num_kv_heads * chunks;
    const int64_t t = i / per_token;
    const int32_t r = (int32_t)(i - t * per_token);
    const int32_t h = r / chunks;
    const int32_t c = r - h * chunks;
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= pool_slots) return;            // padding / outside the pool
    const int64_t blk = slot / block_size;
    const int64_t row = slot - blk * block_size;
    const int64_t src = t * token_stride + (int64_t)h * head_dim + (int64_t)c * VEC;
    const int64_t dst = ((blk * num_kv_heads + h) * block_size + row) * head_dim + (int64_t)c * VEC;
    if constexpr (VEC == 8) {
        *reinterpret_cast<uint4*>(k_cache + dst) = *reinterpret_cast<const uint4*>(key + src);
        *reinterpret_cast<uint4*>(v_cache + dst) = *reinterpret_cast<const uint4*>(value + src);
    } else {
        k_cache[dst] = key[src];
        v_cache[dst] = value[src];
    }
}

constexpr int kMaxLayersPerLaunch = 64;
constexpr int kCopyUnroll = 4;

struct LayerPtrs {
    void* k[kMaxLayersPerLaunch];
    void* v[kMaxLayersPerLaunch];
};

// grid: x = chunk of the block, y = pair, z = 2 * layer + (0: K, 1: V)
template <typename T>
__global__ void __launch_bounds__(kThreads)
copy_blocks_kernel(LayerPtrs layers, const int64_t* __restrict__ pairs, int64_t num_blocks,
                   int64_t units_per_block) {
    const int64_t src = pairs[2 * (int64_t)blockIdx.y];
    const int64_t dst = pairs[2 * (int64_t)blockIdx.y + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
    T* base = static_cast<T*>((blockIdx.z & 1) ? layers.v[blockIdx.z >> 1] : layers.k[blockIdx.z >> 1]);
    const T* s = base + src * units_per_block;
    T* d = base + dst * units_per_block;
    const int64_t first = (int64_t)blockIdx.x * (kThreads * kCopyUnroll) + threadIdx.x;
    T tmp[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const int64_t k = first + (int64_t)u * kThreads;
        if (k < units_per_block) tmp[u] = s[k];
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const int64_t k = first + (int64_t)u * kThreads;
        if (k < units_per_block) d[k] = tmp[u];
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_head_dim(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128 || d == 256; }

}  // namespace

extern "C" int pa_reshape_and_cache(const void* key, const void* value, int64_t kv_token_stride,
                                    const int64_t* slot_mapping, int32_t num_tokens, void* k_cache,
                                    void* v_cache, int32_t num_blocks, int32_t num_kv_heads,
                                    int32_t block_size, int32_t head_dim, int32_t dtype,
                                    void* stream) {
    if (dtype != PA_DTYPE_F16) return pa::fail(PA_ERR_UNSUPPORTED, "pa_reshape_and_cache: dtype %d", dtype);
    if (!supported_head_dim(head_dim))
        return pa::fail(PA_ERR_UNSUPPORTED, "pa_reshape_and_cache: head_dim %d", head_dim);
    if (num_tokens < 0 || num_blocks < 0 || num_kv_heads <= 0 || block_size <= 0)
        return pa::fail(PA_ERR_INVALID, "pa_reshape_and_cache: bad sizes");
    if (kv_token_stride < (int64_t)num_kv_heads * head_dim)
        return pa::fail(PA_ERR_INVALID, "pa_reshape_and_cache: kv_token_stride %lld < num_kv_heads * head_dim",
                        (long long)kv_token_stride);
    if (num_tokens == 0) return PA_OK;
    if (!key || !value || !slot_mapping || !k_cache || !v_cache)
        return pa::fail(PA_ERR_INVALID, "pa_reshape_and_cache: null pointer");

    const bool vec = aligned16(key) && aligned16(value) && aligned16(k_cache) && aligned16(v_cache) &&
                     kv_token_stride % 8 == 0;
    const int vecw = vec ? 8 : 1;
    const int64_t work = (int64_t)num_tokens * num_kv_heads * (head_dim / vecw);
    const int64_t blocks = (work + kThreads - 1) / kThreads;
    if (blocks > 0x7fffffff) return pa::fail(PA_ERR_INVALID, "pa_reshape_and_cache: too many tokens");
    const int64_t pool_slots = (int64_t)num_blocks * block_size;
    auto st = static_cast<hipStream_t>(stream);
    if (vec)
        hipLaunchKernelGGL(scatter_kv_kernel<8>, dim3((unsigned)blocks), dim3(kThreads), 0, st,
                           static_cast<const uint16_t*>(key), static_cast<const uint16_t*>(value),
                           kv_token_stride, slot_mapping, work, static_cast<uint16_t*>(k_cache),
                           static_cast<uint16_t*>(v_cache), pool_slots, num_kv_heads, block_size, head_dim);
    else
        hipLaunchKernelGGL(scatter_kv_kernel<1>, dim3((unsigned)blocks), dim3(kThreads), 0, st,
                           static_cast<const uint16_t*>(key), static_cast<const uint16_t*>(value),
                           kv_token_stride, slot_mapping, work, static_cast<uint16_t*>(k_cache),
                           static_cast<uint16_t*>(v_cache), pool_slots, num_kv_heads, block_size, head_dim);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return pa::fail(PA_ERR_HIP, "pa_reshape_and_cache: %s", hipGetErrorString(e));
    return PA_OK;
}

extern "C" int pa_copy_blocks(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                              const int64_t* src_dst_pairs, int32_t num_pairs, int32_t num_blocks,
                              int64_t block_elems, int32_t dtype, void* stream) {
    if (dtype != PA_DTYPE_F16) return pa::fail(PA_ERR_UNSUPPORTED, "pa_copy_blocks: dtype %d", dtype);
    if (num_layers < 0 || num_pairs < 0 || num_blocks < 0 || block_elems <= 0)
        return pa::fail(PA_ERR_INVALID, "pa_copy_blocks: bad sizes");
    if (num_pairs == 0 || num_layers == 0) return PA_OK;
    if (!k_caches || !v_caches || !src_dst_pairs) return pa::fail(PA_ERR_INVALID, "pa_copy_blocks: null pointer");
    if (num_pairs > 65535) return pa::fail(PA_ERR_INVALID, "pa_copy_blocks: more than 65535 pairs in one call");
    bool vec = block_elems % 8 == 0;
    for (int32_t l = 0; l < num_layers; ++l) {
        if (!k_caches[l] || !v_caches[l]) return pa::fail(PA_ERR_INVALID, "pa_copy_blocks: null cache of layer %d", l);
        vec = vec && aligned16(k_caches[l]) && aligned16(v_caches[l]);
    }
    auto st = static_cast<hipStream_t>(stream);
    const int64_t units = vec ? block_elems / 8 : block_elems;
    const int64_t chunks = (units + kThreads * kCopyUnroll - 1) / (kThreads * kCopyUnroll);
    if (chunks > 0x7fffffff) return pa::fail(PA_ERR_INVALID, "pa_copy_blocks: block too large");
    for (int32_t l0 = 0; l0 < num_layers; l0 += kMaxLayersPerLaunch) {
        const int32_t nl = num_layers - l0 < kMaxLayersPerLaunch ? num_layers - l0 : kMaxLayersPerLaunch;
        LayerPtrs lp{};
        for (int32_t i = 0; i < nl; ++i) {
            lp.k[i] = k_caches[l0 + i];
            lp.v[i] = v_caches[l0 + i];
        }
        const dim3 grid((unsigned)chunks, (unsigned)num_pairs, (unsigned)(2 * nl));
        if (vec)
            hipLaunchKernelGGL(copy_blocks_kernel<uint4>, grid, dim3(kThreads), 0, st, lp, src_dst_pairs,
                               (int64_t)num_blocks, units);
        else
            hipLaunchKernelGGL(copy_blocks_kernel<uint16_t>, grid, dim3(kThreads), 0, st, lp, src_dst_pairs,
                               (int64_t)num_blocks, units);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return pa::fail(PA_ERR_HIP, "pa_copy_blocks: %s", hipGetErrorString(e));
    }
    return PA_OK;
}

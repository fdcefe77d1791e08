// Slot-mapped cache write and whole-block copy for gfx950.
//
// Both are pure data movement: every lane moves 16 bytes (8 fp16 values)
// per load/store when the addresses allow it, else 2 bytes.  Neither needs
// LDS or MFMA; they are bound by launch latency at decode batch sizes
// (reshape) or by HBM bandwidth (block copy).
//
// A third operation moves whole blocks between a device cache and a pinned
// host cache (swap out / in) with the same copy loop: the kernel reads or
// writes the host side through its device mapping over PCIe, one launch for
// every block and layer of a group.
//
// Sources (pages named by address, sections as they number them):
//   [lpnh-1824136]  lpnh.cn/news/1824136, 3.1: results are scattered back
//                   into the proper blocks
//   [lpnh-2758356]  lpnh.cn/news/2758356, 2.2 (slot = block id * block size
//                   + row), 4.2 third step (copy the whole shared block into
//                   the new one), 4.3 (that copy costs bandwidth)
//   [lpnh-1824136]  lpnh.cn/news/1824136, 4.2: KV blocks can be swapped out
//                   to host memory, at a large latency cost
#include <hip/hip_runtime.h>

#include <type_traits>

#include <cstdint>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

namespace {

constexpr int kThreads = 256;

// One lane per (head, VEC-element chunk) of a token; K and V move together.
// Grid x = token, y = group of lanes (64 to kThreads per workgroup) over the
// token's (head, chunk) pairs: the token's slot is read once per workgroup (a uniform, scalar
// load), and the chunk count and -- when it is a power of two -- the block
// size turn divisions into shifts, so the stores wait on one load only.
template <int VEC>
__global__ void __launch_bounds__(kThreads)
scatter_kv_kernel(const uint16_t* __restrict__ key, const uint16_t* __restrict__ value,
                  int64_t token_stride, const int64_t* __restrict__ slots,
                  uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache,
                  int64_t pool_slots, int32_t per_token, int32_t chunk_shift, int32_t block_size,
                  int32_t block_shift, int32_t head_dim) {
    const int64_t t = blockIdx.x;
    const int32_t r = (int32_t)(blockIdx.y * blockDim.x + threadIdx.x);
    if (r >= per_token) return;
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= pool_slots) return;            // padding / outside the pool
    const int64_t blk = block_shift >= 0 ? slot >> block_shift : slot / block_size;
    const int64_t row = slot - blk * block_size;
    const int32_t h = r >> chunk_shift;
    const int32_t c = r - (h << chunk_shift);
    const int32_t num_kv_heads = per_token >> chunk_shift;
    const int64_t src = t * token_stride + (int64_t)h * head_dim + (int64_t)c * VEC;
    const int64_t dst = ((blk * num_kv_heads + h) * block_size + row) * head_dim + (int64_t)c * VEC;
    if constexpr (VEC == 8) {
        // nontemporal both ways: each byte is moved once (15360 prompt tokens
        // at 32 x 128 heads: 96 instead of 102 us)
        typedef unsigned u32x4_nt __attribute__((ext_vector_type(4)));
        const u32x4_nt kv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(key + src));
        const u32x4_nt vv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(value + src));
        __builtin_nontemporal_store(kv, reinterpret_cast<u32x4_nt*>(k_cache + dst));
        __builtin_nontemporal_store(vv, reinterpret_cast<u32x4_nt*>(v_cache + dst));
    } else {
        k_cache[dst] = key[src];
        v_cache[dst] = value[src];
    }
}

constexpr int kMaxCachesPerLaunch = 128;   // cache tensors (K or V of one layer) per launch

// Source and destination tensor of each cache in one launch: the same
// tensor for copy-on-write copies, a device and a host tensor for swaps.
struct CachePtrs {
    const void* src[kMaxCachesPerLaunch];
    void* dst[kMaxCachesPerLaunch];
};

// grid: x = chunk of the block, y = pair, z = cache; pairs[i] = (src id, dst id).
// One unit (16 bytes when vectorised) per thread, so a 128 KiB block is 32
// workgroups of 4 KiB: on 4096 pairs of 128 KiB blocks this moves 6.14 TB/s
// (read + write), against 5.27 with 2 units per thread and 4.9 with 4 (fewer,
// larger workgroups leave the copy's tail to fewer CUs); swaps over PCIe are
// the same either way.
template <typename T>
__global__ void __launch_bounds__(kThreads)
block_copy_kernel(CachePtrs caches, const int64_t* __restrict__ pairs, int64_t src_blocks, int64_t dst_blocks,
                  int64_t units_per_block) {
    const int64_t src = pairs[2 * (int64_t)blockIdx.y];
    const int64_t dst = pairs[2 * (int64_t)blockIdx.y + 1];
    if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
    const T* s = static_cast<const T*>(caches.src[blockIdx.z]) + src * units_per_block;
    T* d = static_cast<T*>(caches.dst[blockIdx.z]) + dst * units_per_block;
    const int64_t k = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    // stores bypass the L2's keep policy (nontemporal): the destination is
    // not read back by this kernel; +1.3% on 4096 pairs of 128 KiB blocks
    typedef unsigned u32x4_nt __attribute__((ext_vector_type(4)));
    using U = typename std::conditional<sizeof(T) == 16, u32x4_nt, uint16_t>::type;
    if (k < units_per_block)
        __builtin_nontemporal_store(reinterpret_cast<const U*>(s)[k], reinterpret_cast<U*>(d) + k);
}

// Enqueue block copies for caches [0, n): src[i] -> dst[i] per pair.
int launch_block_copies(const std::vector<const void*>& src, const std::vector<void*>& dst,
                        const int64_t* pairs, int32_t num_pairs, int64_t src_blocks, int64_t dst_blocks,
                        int64_t block_elems, bool vec, hipStream_t st, const char* what) {
    const int64_t units = vec ? block_elems / 8 : block_elems;
    const int64_t chunks = (units + kThreads - 1) / kThreads;
    if (chunks > 0x7fffffff) return pa::fail(PA_ERR_INVALID, "%s: block too large", what);
    const int32_t n = (int32_t)src.size();
    for (int32_t c0 = 0; c0 < n; c0 += kMaxCachesPerLaunch) {
        const int32_t nc = n - c0 < kMaxCachesPerLaunch ? n - c0 : kMaxCachesPerLaunch;
        CachePtrs cp{};
        for (int32_t i = 0; i < nc; ++i) {
            cp.src[i] = src[c0 + i];
            cp.dst[i] = dst[c0 + i];
        }
        const dim3 grid((unsigned)chunks, (unsigned)num_pairs, (unsigned)nc);
        if (vec)
            hipLaunchKernelGGL(block_copy_kernel<uint4>, grid, dim3(kThreads), 0, st, cp, pairs, src_blocks,
                               dst_blocks, units);
        else
            hipLaunchKernelGGL(block_copy_kernel<uint16_t>, grid, dim3(kThreads), 0, st, cp, pairs, src_blocks,
                               dst_blocks, units);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return pa::fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    }
    return PA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_head_dim(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128 || d == 256; }

// Device address of pinned host memory (hipHostMalloc / torch pin_memory),
// or null if `p` is not pinned, mapped host memory.
void* host_device_address(void* p) {
    hipPointerAttribute_t a{};
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    if (a.type != hipMemoryTypeHost || !a.devicePointer || !a.hostPointer) return nullptr;
    return static_cast<char*>(a.devicePointer) + (static_cast<char*>(p) - static_cast<char*>(a.hostPointer));
}

bool is_device_memory(const void* p) {
    hipPointerAttribute_t a{};
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return a.type == hipMemoryTypeDevice;
}

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
    const int64_t per_token = (int64_t)num_kv_heads * (head_dim / vecw);
    int32_t threads = 64;                                  // lanes per workgroup: up to one per pair
    while (threads < kThreads && threads < per_token) threads *= 2;
    const int64_t groups = (per_token + threads - 1) / threads;
    if (groups > 65535)
        return pa::fail(PA_ERR_INVALID, "pa_reshape_and_cache: num_kv_heads * head_dim too large");
    const int32_t chunk_shift = __builtin_ctz((unsigned)(head_dim / vecw));   // head_dim / vecw: a power of two
    const int32_t block_shift = (block_size & (block_size - 1)) == 0 ? __builtin_ctz((unsigned)block_size) : -1;
    const int64_t pool_slots = (int64_t)num_blocks * block_size;
    if (pa::validate_enabled())
        if (int rc = pa::validate_slots("pa_reshape_and_cache", slot_mapping, num_tokens, pool_slots, stream)) return rc;
    auto st = static_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)num_tokens, (unsigned)groups);
    if (vec)
        hipLaunchKernelGGL(scatter_kv_kernel<8>, grid, dim3((unsigned)threads), 0, st, static_cast<const uint16_t*>(key),
                           static_cast<const uint16_t*>(value), kv_token_stride, slot_mapping,
                           static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache), pool_slots,
                           (int32_t)per_token, chunk_shift, block_size, block_shift, head_dim);
    else
        hipLaunchKernelGGL(scatter_kv_kernel<1>, grid, dim3((unsigned)threads), 0, st, static_cast<const uint16_t*>(key),
                           static_cast<const uint16_t*>(value), kv_token_stride, slot_mapping,
                           static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache), pool_slots,
                           (int32_t)per_token, chunk_shift, block_size, block_shift, head_dim);
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
    std::vector<const void*> src;
    std::vector<void*> dst;
    for (int32_t l = 0; l < num_layers; ++l) {
        if (!k_caches[l] || !v_caches[l]) return pa::fail(PA_ERR_INVALID, "pa_copy_blocks: null cache of layer %d", l);
        vec = vec && aligned16(k_caches[l]) && aligned16(v_caches[l]);
        src.push_back(k_caches[l]);
        dst.push_back(k_caches[l]);
        src.push_back(v_caches[l]);
        dst.push_back(v_caches[l]);
    }
    if (pa::validate_enabled())
        if (int rc = pa::validate_pairs("pa_copy_blocks", src_dst_pairs, num_pairs, num_blocks, num_blocks, true,
                                        stream))
            return rc;
    return launch_block_copies(src, dst, src_dst_pairs, num_pairs, num_blocks, num_blocks, block_elems, vec,
                               static_cast<hipStream_t>(stream), "pa_copy_blocks");
}

extern "C" int pa_swap_blocks(void* const* dev_caches, void* const* host_caches, int32_t num_caches,
                              const int64_t* pairs, int32_t num_pairs, int32_t dev_num_blocks,
                              int32_t host_num_blocks, int64_t block_elems, int32_t direction, int32_t dtype,
                              void* stream) {
    if (dtype != PA_DTYPE_F16) return pa::fail(PA_ERR_UNSUPPORTED, "pa_swap_blocks: dtype %d", dtype);
    if (direction != PA_SWAP_OUT && direction != PA_SWAP_IN)
        return pa::fail(PA_ERR_INVALID, "pa_swap_blocks: direction %d", direction);
    if (num_caches < 0 || num_pairs < 0 || dev_num_blocks < 0 || host_num_blocks < 0 || block_elems <= 0)
        return pa::fail(PA_ERR_INVALID, "pa_swap_blocks: bad sizes");
    if (num_pairs == 0 || num_caches == 0) return PA_OK;
    if (!dev_caches || !host_caches || !pairs) return pa::fail(PA_ERR_INVALID, "pa_swap_blocks: null pointer");
    if (num_pairs > 65535) return pa::fail(PA_ERR_INVALID, "pa_swap_blocks: more than 65535 pairs in one call");
    if (!is_device_memory(pairs)) return pa::fail(PA_ERR_INVALID, "pa_swap_blocks: pairs must be device memory");
    // resolve every pointer before anything is enqueued
    bool vec = block_elems % 8 == 0;
    std::vector<const void*> src;
    std::vector<void*> dst;
    for (int32_t i = 0; i < num_caches; ++i) {
        if (!dev_caches[i] || !host_caches[i])
            return pa::fail(PA_ERR_INVALID, "pa_swap_blocks: null cache pointer %d", i);
        if (!is_device_memory(dev_caches[i]))
            return pa::fail(PA_ERR_INVALID, "pa_swap_blocks: cache %d on the device side is not device memory", i);
        void* h = host_device_address(host_caches[i]);
        if (!h) return pa::fail(PA_ERR_INVALID, "pa_swap_blocks: host cache %d is not pinned, mapped host memory", i);
        vec = vec && aligned16(dev_caches[i]) && aligned16(h);
        src.push_back(direction == PA_SWAP_OUT ? dev_caches[i] : h);
        dst.push_back(direction == PA_SWAP_OUT ? h : dev_caches[i]);
    }
    const int64_t src_nb = direction == PA_SWAP_OUT ? dev_num_blocks : host_num_blocks;
    const int64_t dst_nb = direction == PA_SWAP_OUT ? host_num_blocks : dev_num_blocks;
    if (pa::validate_enabled())
        if (int rc = pa::validate_pairs("pa_swap_blocks", pairs, num_pairs, src_nb, dst_nb, false, stream)) return rc;
    return launch_block_copies(src, dst, pairs, num_pairs, src_nb, dst_nb, block_elems, vec,
                               static_cast<hipStream_t>(stream), "pa_swap_blocks");
}

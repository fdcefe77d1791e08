// Launch interface shared by the decode kernels of the library (not part of
// the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pa {

// Everything one pa_decode partition-kernel launch needs; pointers are
// device pointers, the workspace pointers null when no sequence is split.
// `order` (null: grid order) lists the sequences longest first: grid row y
// works on sequence order[y].
struct DecodeLaunch {
    _Float16* out;
    float* ws_ml;
    float* ws_acc;
    const int32_t* order;
    const _Float16* q;
    const _Float16* k_cache;
    const _Float16* v_cache;
    const int32_t* tables;
    int32_t max_blocks;
    const int32_t* lens;
    int32_t num_seqs;
    int32_t num_heads;
    int32_t num_kv_heads;
    int32_t num_blocks;
    int32_t block_size;
    int32_t head_dim;
    float scale_log2;
    int32_t part_size;
    int32_t num_parts;
    int64_t len_cap;
    hipStream_t stream;
    // append mode (pa_decode_append): the new token of sequence s, KV head
    // h at s * new_stride + h * head_dim; null otherwise.  The kernel then
    // writes it into k_cache / v_cache at the sequence's last position.
    const _Float16* new_k;
    const _Float16* new_v;
    int64_t new_stride;
};

// Grouped-query decode on the matrix cores: head_dim 64, 128 or 256, 2 <= group <= 16.
bool gqa_mfma_supported(int32_t head_dim, int32_t block_size, int32_t group);
hipError_t launch_gqa_mfma(const DecodeLaunch& a);

}  // namespace pa

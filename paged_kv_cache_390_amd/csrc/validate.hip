// Opt-in host validation of device-resident indices (PA_VALIDATE set to
// anything but "0" in the environment).
//
// The GPU calls take slots, copy pairs, block tables and lengths in device
// memory and cannot check them without a device-to-host copy, so by default
// the kernels only skip ids outside the pool.  With PA_VALIDATE set, a call
// first copies those arrays to the host on its stream, waits for them, and
// refuses (PA_ERR_INVALID, nothing enqueued) what the block manager would
// never produce:
//   * pa_reshape_and_cache: a slot past the pool, or two tokens of one call
//     writing one slot (their writes would race);
//   * pa_copy_blocks / pa_swap_blocks: an id outside its pool, two pairs
//     with one destination, or (copy-on-write copies within one tensor) a
//     destination that is also a source of the call -- all pairs of a call
//     are copied at once ([lpnh-2758356] 4.2: the copy goes to a new block);
//   * the decode and prefill calls: a length above the call's bound or the
//     table width, a table entry outside the pool for a position below the
//     length, and (prefill) query ranges that are not ordered and inside
//     the batch.
// Validation synchronises the stream, so it is a debugging aid: it must not
// be enabled while a caller captures the stream into a graph.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <unordered_set>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

namespace {

template <typename T>
int fetch(const char* fn, std::vector<T>& host, const T* dev, size_t n, void* stream) {
    host.resize(n);
    if (n == 0) return PA_OK;
    auto st = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(host.data(), dev, n * sizeof(T), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return pa::fail(PA_ERR_HIP, "%s: validation copy: %s", fn, hipGetErrorString(e));
    return PA_OK;
}

}  // namespace

namespace pa {

bool validate_enabled() {
    const char* v = std::getenv("PA_VALIDATE");
    return v && v[0] && std::strcmp(v, "0") != 0;
}

int validate_slots(const char* fn, const int64_t* slots, int32_t n, int64_t pool_slots, void* stream) {
    std::vector<int64_t> h;
    if (int rc = fetch(fn, h, slots, (size_t)n, stream)) return rc;
    std::unordered_set<int64_t> seen;
    seen.reserve(h.size() * 2);
    for (int32_t t = 0; t < n; ++t) {
        const int64_t s = h[t];
        if (s < 0) continue;                                  // padding: skipped by the kernel
        if (s >= pool_slots)
            return fail(PA_ERR_INVALID, "%s: slot %lld of token %d is outside the pool of %lld slots", fn,
                        (long long)s, t, (long long)pool_slots);
        if (!seen.insert(s).second)
            return fail(PA_ERR_INVALID, "%s: slot %lld is written by two tokens of the call (token %d)", fn,
                        (long long)s, t);
    }
    return PA_OK;
}

int validate_pairs(const char* fn, const int64_t* pairs, int32_t n, int64_t src_blocks, int64_t dst_blocks,
                   bool one_pool, void* stream) {
    std::vector<int64_t> h;
    if (int rc = fetch(fn, h, pairs, 2 * (size_t)n, stream)) return rc;
    std::unordered_set<int64_t> dsts, srcs;
    for (int32_t i = 0; i < n; ++i) {
        const int64_t s = h[2 * i], d = h[2 * i + 1];
        if (s < 0 || s >= src_blocks || d < 0 || d >= dst_blocks)
            return fail(PA_ERR_INVALID, "%s: pair %d (%lld -> %lld) has an id outside its pool", fn, i, (long long)s,
                        (long long)d);
        if (!dsts.insert(d).second)
            return fail(PA_ERR_INVALID, "%s: block %lld is the destination of two pairs", fn, (long long)d);
        srcs.insert(s);
    }
    if (one_pool)
        for (int64_t d : dsts)
            if (srcs.count(d))
                return fail(PA_ERR_INVALID, "%s: block %lld is both a destination and a source of the call", fn,
                            (long long)d);
    return PA_OK;
}

int validate_tables(const char* fn, const int32_t* tables, int32_t width, const int32_t* lens, int32_t num_seqs,
                    int32_t block_size, int32_t num_blocks, int64_t max_len, void* stream) {
    std::vector<int32_t> ht, hl;
    if (int rc = fetch(fn, hl, lens, (size_t)num_seqs, stream)) return rc;
    if (int rc = fetch(fn, ht, tables, (size_t)num_seqs * width, stream)) return rc;
    const int64_t cap = (int64_t)width * block_size < max_len ? (int64_t)width * block_size : max_len;
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int64_t n = hl[s];
        if (n < 0 || n > cap)
            return fail(PA_ERR_INVALID, "%s: sequence %d has length %lld outside [0, %lld]", fn, s, (long long)n,
                        (long long)cap);
        const int64_t nb = (n + block_size - 1) / block_size;
        for (int64_t j = 0; j < nb; ++j) {
            const int32_t b = ht[(size_t)s * width + j];
            if (b < 0 || b >= num_blocks)
                return fail(PA_ERR_INVALID, "%s: table entry %lld of sequence %d is %d, outside the pool of %d", fn,
                            (long long)j, s, b, num_blocks);
        }
    }
    return PA_OK;
}

int validate_queries(const char* fn, const int32_t* query_start, int32_t num_seqs, int32_t num_tokens,
                     const int32_t* lens, int32_t max_query_len, void* stream) {
    std::vector<int32_t> hq, hl;
    if (int rc = fetch(fn, hq, query_start, (size_t)num_seqs + 1, stream)) return rc;
    if (int rc = fetch(fn, hl, lens, (size_t)num_seqs, stream)) return rc;
    if (hq[0] != 0 || hq[num_seqs] != num_tokens)
        return fail(PA_ERR_INVALID, "%s: query_start must run from 0 to num_tokens (%d .. %d given)", fn, hq[0],
                    hq[num_seqs]);
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int32_t m = hq[s + 1] - hq[s];
        if (m < 0 || m > max_query_len || m > hl[s])
            return fail(PA_ERR_INVALID, "%s: sequence %d has %d new tokens (bound %d, length %d)", fn, s, m,
                        max_query_len, hl[s]);
    }
    return PA_OK;
}

}  // namespace pa

// Internal helpers shared by the library's translation units (not part of
// the C ABI).
#pragma once

#include <cstdarg>
#include <cstdint>

namespace pa {

// Record a message for pa_last_error() on the calling thread.
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));

// Record a message and return `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Clear the calling thread's message.
void clear_error();

// Opt-in host validation of device-resident indices (PA_VALIDATE set and not
// "0"): each copies its arrays to the host on `stream`, waits, and returns
// PA_OK or PA_ERR_INVALID with a message.
bool validate_enabled();
int validate_slots(const char* fn, const int64_t* slots, int32_t n, int64_t pool_slots, void* stream);
int validate_pairs(const char* fn, const int64_t* pairs, int32_t n, int64_t src_blocks, int64_t dst_blocks,
                   bool one_pool, void* stream);
int validate_tables(const char* fn, const int32_t* tables, int32_t width, const int32_t* lens, int32_t num_seqs,
                    int32_t block_size, int32_t num_blocks, int64_t max_len, void* stream);
int validate_queries(const char* fn, const int32_t* query_start, int32_t num_seqs, int32_t num_tokens,
                     const int32_t* lens, int32_t max_query_len, void* stream);

}  // namespace pa

// Host block manager: free list, per-block holder counts and per-sequence
// block tables.  Builds what the GPU calls consume: int32 tables, int32
// lengths, int64 slots and int64 copy-on-write pairs.
//
// Sources (pages named by address, sections as they number them):
//   [5688vip]       5688vip.com, "4、PagedAttention：显存管理、分页机制、块大小选择",
//                   section 分页机制 (append a block when the last one is full)
//   [n1n]           explore.n1n.ai, "PagedAttention 对比传统 KV 缓存", section
//                   实现逻辑代码示例 (free list popped from its end; failure
//                   when it is empty)
//   [lpnh-2758356]  lpnh.cn/news/2758356: 3.1 (grow on demand), 3.2 (status,
//                   count and address per block; release walks the table),
//                   4.2 (fork shares blocks; writing into a shared block that
//                   is not full copies it; a full one is never copied), 4.3
//                   (count updates must be atomic)
//   [lpnh-1824136]  lpnh.cn/news/1824136, 4.2 (KV blocks can be swapped out
//                   to host memory, at a large latency cost)
//
// Design: the state is a vector of counts, a vector used as the free stack
// and a hash map from sequence id to (table, length).  Every public call
// validates first, then mutates, so a failing call changes nothing.  One
// mutex serialises calls.  A second pool (host blocks, its own counts and
// free stack) receives the blocks of swapped-out sequences; a group of
// sequences is swapped together so that blocks shared by forks stay shared:
// each distinct block, in order of first appearance, gets one block on the
// other side whose count is the number of group members holding it.
// Prefix sharing across requests ([n1n] 前缀缓存; [lpnh-1824136] 3.2 second
// step): full prompt blocks are indexed by (previous block id or -1, their
// token ids) -- the previous block's id stands for the whole prefix before
// it -- and a new prompt takes every leading full block it finds there.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

namespace {

struct Seq {
    std::vector<int32_t> table;   // device ids, or host ids while swapped
    int64_t len = 0;
    bool swapped = false;
};

// Index key of a full block: the block before it (-1 for the first) and
// its token ids.  Exact: equality compares every token.
struct PrefixKey {
    int32_t prev;
    std::vector<int32_t> toks;
    bool operator==(const PrefixKey& o) const { return prev == o.prev && toks == o.toks; }
};

struct PrefixKeyHash {
    size_t operator()(const PrefixKey& k) const {
        uint64_t h = 1469598103934665603ull ^ (uint32_t)k.prev;   // FNV-1a over the ids
        for (int32_t t : k.toks) {
            h ^= (uint32_t)t;
            h *= 1099511628211ull;
        }
        return (size_t)h;
    }
};

struct Pool {
    std::vector<int32_t> free_stack;   // allocation pops from the back
    std::vector<int32_t> count;        // holders per block

    void init(int32_t n) {
        free_stack.resize(n);
        for (int32_t i = 0; i < n; ++i) free_stack[i] = i;
        count.assign(n, 0);
    }
};

}  // namespace

struct pa_bm {
    int32_t num_blocks;
    int32_t block_size;
    std::vector<int32_t> free_stack;   // allocation pops from the back
    std::vector<int32_t> count;        // holders per block
    std::unordered_map<int64_t, Seq> seqs;
    Pool host;                         // swap target
    std::unordered_map<PrefixKey, int32_t, PrefixKeyHash> prefix_index;
    std::unordered_map<int32_t, PrefixKey> block_key;
    std::mutex mu;

    // A device block whose count reached 0: back on the free stack and out
    // of the prefix index.
    void release(int32_t b) {
        free_stack.push_back(b);
        auto it = block_key.find(b);
        if (it != block_key.end()) {
            prefix_index.erase(it->second);
            block_key.erase(it);
        }
    }

    int64_t blocks_for(int64_t n) const { return (n + block_size - 1) / block_size; }

    int32_t pop_free() {
        int32_t b = free_stack.back();
        free_stack.pop_back();
        count[b] = 1;
        return b;
    }

    int64_t slot_of(const Seq& s, int64_t pos) const {
        return (int64_t)s.table[pos / block_size] * block_size + pos % block_size;
    }

    // Append one token; assumes seq exists.  Fails with OOM before mutating.
    int append(Seq& s, int64_t* slot, int64_t* src, int64_t* dst) {
        *src = -1;
        *dst = -1;
        const int64_t n = s.len;
        int rc = PA_OK;
        if (n % block_size == 0) {
            // no block yet, or the last block is full: a fresh block
            if (free_stack.empty()) return PA_ERR_OOM;
            s.table.push_back(pop_free());
        } else {
            const int32_t last = s.table.back();
            if (count[last] > 1) {
                // shared and not full: copy on write
                if (free_stack.empty()) return PA_ERR_OOM;
                const int32_t fresh = pop_free();
                count[last] -= 1;
                s.table.back() = fresh;
                *src = last;
                *dst = fresh;
                rc = PA_COW;
            }
        }
        s.len = n + 1;
        *slot = slot_of(s, n);
        return rc;
    }

    // Swap a group between the device pool and the host pool (out: device
    // -> host).  Validates everything first; changes nothing on failure.
    int move(const int64_t* ids, int32_t n, bool out, int64_t* pairs, int32_t cap, int32_t* npairs,
             const char* what) {
        std::vector<Seq*> group;
        group.reserve(n);
        std::unordered_set<int64_t> seen;
        for (int32_t i = 0; i < n; ++i) {
            auto it = seqs.find(ids[i]);
            if (it == seqs.end())
                return pa::fail(PA_ERR_STATE, "%s: unknown sequence %lld", what, (long long)ids[i]);
            if (!seen.insert(ids[i]).second)
                return pa::fail(PA_ERR_STATE, "%s: sequence %lld appears twice", what, (long long)ids[i]);
            if (it->second.swapped == out)
                return pa::fail(PA_ERR_STATE, "%s: sequence %lld is already %s", what, (long long)ids[i],
                                out ? "swapped out" : "resident");
            group.push_back(&it->second);
        }
        std::vector<int32_t>& src_count = out ? count : host.count;
        std::vector<int32_t>& src_free = out ? free_stack : host.free_stack;
        std::vector<int32_t>& dst_count = out ? host.count : count;
        std::vector<int32_t>& dst_free = out ? host.free_stack : free_stack;
        std::vector<int32_t> order;
        std::unordered_map<int32_t, int32_t> holders;
        for (Seq* q : group)
            for (int32_t b : q->table)
                if (holders[b]++ == 0) order.push_back(b);
        if (order.size() > dst_free.size())
            return pa::fail(PA_ERR_OOM, "%s: %zu blocks needed, %zu free", what, order.size(), dst_free.size());
        if ((int64_t)order.size() > cap)
            return pa::fail(PA_ERR_INVALID, "%s: %zu pairs, room for %d", what, order.size(), cap);
        std::unordered_map<int32_t, int32_t> moved;
        for (size_t i = 0; i < order.size(); ++i) {
            const int32_t b = order[i];
            const int32_t d = dst_free.back();
            dst_free.pop_back();
            dst_count[d] = holders[b];
            moved[b] = d;
            pairs[2 * i] = b;
            pairs[2 * i + 1] = d;
            src_count[b] -= holders[b];
            if (src_count[b] == 0) {
                if (out)
                    release(b);
                else
                    src_free.push_back(b);
            }
        }
        for (Seq* q : group) {
            for (int32_t& b : q->table) b = moved[b];
            q->swapped = out;
        }
        *npairs = (int32_t)order.size();
        return PA_OK;
    }
};

extern "C" {

pa_bm* pa_bm_create(int32_t num_blocks, int32_t block_size) { return pa_bm_create_with_host(num_blocks, block_size, 0); }

pa_bm* pa_bm_create_with_host(int32_t num_blocks, int32_t block_size, int32_t num_host_blocks) {
    if (num_blocks < 0 || block_size <= 0 || num_host_blocks < 0) {
        pa::set_error("pa_bm_create: num_blocks >= 0, num_host_blocks >= 0 and block_size > 0 required");
        return nullptr;
    }
    pa_bm* bm = new (std::nothrow) pa_bm();
    if (!bm) {
        pa::set_error("pa_bm_create: out of host memory");
        return nullptr;
    }
    try {
        bm->num_blocks = num_blocks;
        bm->block_size = block_size;
        bm->free_stack.resize(num_blocks);
        for (int32_t i = 0; i < num_blocks; ++i) bm->free_stack[i] = i;
        bm->count.assign(num_blocks, 0);
        bm->host.init(num_host_blocks);
    } catch (...) {
        delete bm;
        pa::set_error("pa_bm_create: out of host memory");
        return nullptr;
    }
    return bm;
}

void pa_bm_destroy(pa_bm* bm) { delete bm; }

int pa_bm_add_sequence(pa_bm* bm, int64_t seq, int32_t n_tokens, int64_t* slots_out) {
    if (!bm || n_tokens < 0) return pa::fail(PA_ERR_INVALID, "pa_bm_add_sequence: bad argument");
    std::lock_guard<std::mutex> g(bm->mu);
    if (bm->seqs.count(seq)) return pa::fail(PA_ERR_STATE, "pa_bm_add_sequence: sequence %lld exists", (long long)seq);
    const int64_t need = bm->blocks_for(n_tokens);
    if (need > (int64_t)bm->free_stack.size())
        return pa::fail(PA_ERR_OOM, "pa_bm_add_sequence: need %lld blocks, %zu free", (long long)need, bm->free_stack.size());
    Seq s;
    s.table.reserve(need);
    for (int64_t i = 0; i < need; ++i) s.table.push_back(bm->pop_free());
    s.len = n_tokens;
    if (slots_out)
        for (int64_t p = 0; p < n_tokens; ++p) slots_out[p] = bm->slot_of(s, p);
    bm->seqs.emplace(seq, std::move(s));
    return PA_OK;
}

int pa_bm_set_table(pa_bm* bm, int64_t seq, const int32_t* blocks, int32_t nblk, int32_t n_tokens) {
    if (!bm || n_tokens < 0 || nblk < 0 || (nblk > 0 && !blocks))
        return pa::fail(PA_ERR_INVALID, "pa_bm_set_table: bad argument");
    std::lock_guard<std::mutex> g(bm->mu);
    if (nblk != bm->blocks_for(n_tokens))
        return pa::fail(PA_ERR_INVALID, "pa_bm_set_table: %d blocks given, %lld needed", nblk, (long long)bm->blocks_for(n_tokens));
    if (bm->seqs.count(seq)) return pa::fail(PA_ERR_STATE, "pa_bm_set_table: sequence %lld exists", (long long)seq);
    std::unordered_set<int32_t> taken;
    for (int32_t i = 0; i < nblk; ++i) {
        const int32_t b = blocks[i];
        if (b < 0 || b >= bm->num_blocks || bm->count[b] != 0 || !taken.insert(b).second)
            return pa::fail(PA_ERR_STATE, "pa_bm_set_table: block %d is not free (or repeated)", b);
    }
    // a block with count 0 is on the free list; drop the taken ones, keep order
    bm->free_stack.erase(std::remove_if(bm->free_stack.begin(), bm->free_stack.end(),
                                        [&](int32_t b) { return taken.count(b) != 0; }),
                         bm->free_stack.end());
    Seq s;
    s.table.assign(blocks, blocks + nblk);
    s.len = n_tokens;
    for (int32_t b : s.table) bm->count[b] = 1;
    bm->seqs.emplace(seq, std::move(s));
    return PA_OK;
}

int pa_bm_fork(pa_bm* bm, int64_t parent, int64_t child) {
    if (!bm) return pa::fail(PA_ERR_INVALID, "pa_bm_fork: null manager");
    std::lock_guard<std::mutex> g(bm->mu);
    auto it = bm->seqs.find(parent);
    if (it == bm->seqs.end()) return pa::fail(PA_ERR_STATE, "pa_bm_fork: unknown parent %lld", (long long)parent);
    if (it->second.swapped) return pa::fail(PA_ERR_STATE, "pa_bm_fork: parent %lld is swapped out", (long long)parent);
    if (bm->seqs.count(child)) return pa::fail(PA_ERR_STATE, "pa_bm_fork: sequence %lld exists", (long long)child);
    Seq c = it->second;
    for (int32_t b : c.table) bm->count[b] += 1;
    bm->seqs.emplace(child, std::move(c));
    return PA_OK;
}

int pa_bm_append_token(pa_bm* bm, int64_t seq, int64_t* slot_out, int64_t* cow_src, int64_t* cow_dst) {
    if (!bm) return pa::fail(PA_ERR_INVALID, "pa_bm_append_token: null manager");
    std::lock_guard<std::mutex> g(bm->mu);
    auto it = bm->seqs.find(seq);
    if (it == bm->seqs.end()) return pa::fail(PA_ERR_STATE, "pa_bm_append_token: unknown sequence %lld", (long long)seq);
    if (it->second.swapped) return pa::fail(PA_ERR_STATE, "pa_bm_append_token: sequence %lld is swapped out", (long long)seq);
    int64_t slot, src, dst;
    const int rc = bm->append(it->second, &slot, &src, &dst);
    if (rc == PA_ERR_OOM) return pa::fail(PA_ERR_OOM, "pa_bm_append_token: no free block");
    if (slot_out) *slot_out = slot;
    if (cow_src) *cow_src = src;
    if (cow_dst) *cow_dst = dst;
    return rc;
}

int pa_bm_append_tokens(pa_bm* bm, const int64_t* seqs, int32_t n, int64_t* slots_out,
                        int64_t* cow_pairs_out, int32_t* num_cow_out, int32_t* num_done_out) {
    if (num_cow_out) *num_cow_out = 0;
    if (num_done_out) *num_done_out = 0;
    if (!bm || n < 0 || (n > 0 && (!seqs || !slots_out || !cow_pairs_out)))
        return pa::fail(PA_ERR_INVALID, "pa_bm_append_tokens: bad argument");
    std::lock_guard<std::mutex> g(bm->mu);
    int32_t ncow = 0;
    for (int32_t i = 0; i < n; ++i) {
        auto it = bm->seqs.find(seqs[i]);
        if (it == bm->seqs.end())
            return pa::fail(PA_ERR_STATE, "pa_bm_append_tokens: unknown sequence %lld", (long long)seqs[i]);
        if (it->second.swapped)
            return pa::fail(PA_ERR_STATE, "pa_bm_append_tokens: sequence %lld is swapped out", (long long)seqs[i]);
        int64_t src, dst;
        const int rc = bm->append(it->second, &slots_out[i], &src, &dst);
        if (rc == PA_ERR_OOM) return pa::fail(PA_ERR_OOM, "pa_bm_append_tokens: no free block at entry %d", i);
        if (rc == PA_COW) {
            cow_pairs_out[2 * ncow] = src;
            cow_pairs_out[2 * ncow + 1] = dst;
            ++ncow;
            if (num_cow_out) *num_cow_out = ncow;
        }
        if (num_done_out) *num_done_out = i + 1;
    }
    return PA_OK;
}

int pa_bm_free_sequence(pa_bm* bm, int64_t seq) {
    if (!bm) return pa::fail(PA_ERR_INVALID, "pa_bm_free_sequence: null manager");
    std::lock_guard<std::mutex> g(bm->mu);
    auto it = bm->seqs.find(seq);
    if (it == bm->seqs.end()) return pa::fail(PA_ERR_STATE, "pa_bm_free_sequence: unknown sequence %lld", (long long)seq);
    for (int32_t b : it->second.table) {
        if (it->second.swapped) {
            if (--bm->host.count[b] == 0) bm->host.free_stack.push_back(b);
        } else {
            if (--bm->count[b] == 0) bm->release(b);
        }
    }
    bm->seqs.erase(it);
    return PA_OK;
}

int pa_bm_add_sequence_cached(pa_bm* bm, int64_t seq, const int32_t* token_ids, int32_t n_tokens,
                              int64_t* slots_out, int32_t* num_cached_out) {
    if (num_cached_out) *num_cached_out = 0;
    if (!bm || n_tokens < 0 || (n_tokens > 0 && !token_ids))
        return pa::fail(PA_ERR_INVALID, "pa_bm_add_sequence_cached: bad argument");
    std::lock_guard<std::mutex> g(bm->mu);
    if (bm->seqs.count(seq))
        return pa::fail(PA_ERR_STATE, "pa_bm_add_sequence_cached: sequence %lld exists", (long long)seq);
    const int32_t B = bm->block_size;
    const int64_t nfull = n_tokens / B;
    std::vector<int32_t> hits;
    PrefixKey key{-1, {}};
    for (int64_t i = 0; i < nfull; ++i) {
        key.toks.assign(token_ids + i * B, token_ids + (i + 1) * B);
        auto f = bm->prefix_index.find(key);
        if (f == bm->prefix_index.end()) break;
        hits.push_back(f->second);
        key.prev = f->second;
    }
    const int64_t total = bm->blocks_for(n_tokens);
    const int64_t need = total - (int64_t)hits.size();
    if (need > (int64_t)bm->free_stack.size())
        return pa::fail(PA_ERR_OOM, "pa_bm_add_sequence_cached: need %lld blocks, %zu free", (long long)need,
                        bm->free_stack.size());
    Seq s;
    s.table.reserve(total);
    for (int32_t b : hits) {
        bm->count[b] += 1;
        s.table.push_back(b);
    }
    for (int64_t i = (int64_t)hits.size(); i < total; ++i) {
        const int32_t b = bm->pop_free();
        s.table.push_back(b);
        if (i < nfull) {                       // a full prompt block: index it
            PrefixKey k{i > 0 ? s.table[i - 1] : -1, std::vector<int32_t>(token_ids + i * B, token_ids + (i + 1) * B)};
            bm->block_key[b] = k;
            bm->prefix_index.emplace(std::move(k), b);
        }
    }
    s.len = n_tokens;
    if (slots_out)
        for (int64_t p = 0; p < n_tokens; ++p) slots_out[p] = bm->slot_of(s, p);
    if (num_cached_out) *num_cached_out = (int32_t)hits.size() * B;
    bm->seqs.emplace(seq, std::move(s));
    return PA_OK;
}

int32_t pa_bm_num_cached_blocks(pa_bm* bm) {
    if (!bm) return -1;
    std::lock_guard<std::mutex> g(bm->mu);
    return (int32_t)bm->prefix_index.size();
}

int pa_bm_swap_out(pa_bm* bm, const int64_t* seqs, int32_t n, int64_t* pairs_out, int32_t cap,
                   int32_t* num_pairs_out) {
    if (num_pairs_out) *num_pairs_out = 0;
    if (!bm || n < 0 || cap < 0 || (n > 0 && !seqs) || (cap > 0 && !pairs_out) || !num_pairs_out)
        return pa::fail(PA_ERR_INVALID, "pa_bm_swap_out: bad argument");
    std::lock_guard<std::mutex> g(bm->mu);
    return bm->move(seqs, n, true, pairs_out, cap, num_pairs_out, "pa_bm_swap_out");
}

int pa_bm_swap_in(pa_bm* bm, const int64_t* seqs, int32_t n, int64_t* pairs_out, int32_t cap,
                  int32_t* num_pairs_out) {
    if (num_pairs_out) *num_pairs_out = 0;
    if (!bm || n < 0 || cap < 0 || (n > 0 && !seqs) || (cap > 0 && !pairs_out) || !num_pairs_out)
        return pa::fail(PA_ERR_INVALID, "pa_bm_swap_in: bad argument");
    std::lock_guard<std::mutex> g(bm->mu);
    return bm->move(seqs, n, false, pairs_out, cap, num_pairs_out, "pa_bm_swap_in");
}

int32_t pa_bm_is_swapped(pa_bm* bm, int64_t seq) {
    if (!bm) return -1;
    std::lock_guard<std::mutex> g(bm->mu);
    auto it = bm->seqs.find(seq);
    return it == bm->seqs.end() ? -1 : (it->second.swapped ? 1 : 0);
}

int32_t pa_bm_host_refcount(pa_bm* bm, int32_t hblk) {
    if (!bm) return -1;
    std::lock_guard<std::mutex> g(bm->mu);
    if (hblk < 0 || hblk >= (int32_t)bm->host.count.size()) return -1;
    return bm->host.count[hblk];
}

int32_t pa_bm_host_free_list(pa_bm* bm, int32_t* out, int32_t cap) {
    if (!bm) return -1;
    std::lock_guard<std::mutex> g(bm->mu);
    const int32_t n = (int32_t)bm->host.free_stack.size();
    const int32_t k = std::min(n, std::max(cap, 0));
    if (out && k) std::memcpy(out, bm->host.free_stack.data(), (size_t)k * sizeof(int32_t));
    return n;
}

int pa_bm_get_tables(pa_bm* bm, const int64_t* seqs, int32_t n, int32_t* tables_out,
                     int32_t max_blocks, int32_t* lens_out) {
    if (!bm || n < 0 || max_blocks < 0 || (n > 0 && (!seqs || (!tables_out && max_blocks > 0))))
        return pa::fail(PA_ERR_INVALID, "pa_bm_get_tables: bad argument");
    std::lock_guard<std::mutex> g(bm->mu);
    for (int32_t i = 0; i < n; ++i) {
        auto it = bm->seqs.find(seqs[i]);
        if (it == bm->seqs.end()) return pa::fail(PA_ERR_STATE, "pa_bm_get_tables: unknown sequence %lld", (long long)seqs[i]);
        if (it->second.swapped)
            return pa::fail(PA_ERR_STATE, "pa_bm_get_tables: sequence %lld is swapped out", (long long)seqs[i]);
        if ((int64_t)it->second.table.size() > max_blocks)
            return pa::fail(PA_ERR_INVALID, "pa_bm_get_tables: table of %lld has %zu blocks > %d",
                            (long long)seqs[i], it->second.table.size(), max_blocks);
    }
    for (int32_t i = 0; i < n; ++i) {
        const Seq& s = bm->seqs.find(seqs[i])->second;
        int32_t* row = tables_out + (int64_t)i * max_blocks;
        const size_t k = s.table.size();
        if (k) std::memcpy(row, s.table.data(), k * sizeof(int32_t));
        for (int64_t j = (int64_t)k; j < max_blocks; ++j) row[j] = -1;
        if (lens_out) lens_out[i] = (int32_t)s.len;
    }
    return PA_OK;
}

int pa_bm_get_slots(pa_bm* bm, int64_t seq, int32_t pos_begin, int32_t count, int64_t* slots_out) {
    if (!bm || pos_begin < 0 || count < 0 || (count > 0 && !slots_out))
        return pa::fail(PA_ERR_INVALID, "pa_bm_get_slots: bad argument");
    std::lock_guard<std::mutex> g(bm->mu);
    auto it = bm->seqs.find(seq);
    if (it == bm->seqs.end()) return pa::fail(PA_ERR_STATE, "pa_bm_get_slots: unknown sequence %lld", (long long)seq);
    if (it->second.swapped) return pa::fail(PA_ERR_STATE, "pa_bm_get_slots: sequence %lld is swapped out", (long long)seq);
    const Seq& s = it->second;
    if ((int64_t)pos_begin + count > (int64_t)s.table.size() * bm->block_size)
        return pa::fail(PA_ERR_INVALID, "pa_bm_get_slots: positions beyond the table");
    for (int32_t i = 0; i < count; ++i) slots_out[i] = bm->slot_of(s, (int64_t)pos_begin + i);
    return PA_OK;
}

int32_t pa_bm_refcount(pa_bm* bm, int32_t blk) {
    if (!bm) return -1;
    std::lock_guard<std::mutex> g(bm->mu);
    if (blk < 0 || blk >= bm->num_blocks) return -1;
    return bm->count[blk];
}

int32_t pa_bm_num_free(pa_bm* bm) {
    if (!bm) return -1;
    std::lock_guard<std::mutex> g(bm->mu);
    return (int32_t)bm->free_stack.size();
}

int32_t pa_bm_free_list(pa_bm* bm, int32_t* out, int32_t cap) {
    if (!bm) return -1;
    std::lock_guard<std::mutex> g(bm->mu);
    const int32_t n = (int32_t)bm->free_stack.size();
    const int32_t k = std::min(n, std::max(cap, 0));
    if (out && k) std::memcpy(out, bm->free_stack.data(), (size_t)k * sizeof(int32_t));
    return n;
}

int32_t pa_bm_seq_len(pa_bm* bm, int64_t seq) {
    if (!bm) return -1;
    std::lock_guard<std::mutex> g(bm->mu);
    auto it = bm->seqs.find(seq);
    return it == bm->seqs.end() ? -1 : (int32_t)it->second.len;
}

int32_t pa_bm_seq_table(pa_bm* bm, int64_t seq, int32_t* out, int32_t cap) {
    if (!bm) return -1;
    std::lock_guard<std::mutex> g(bm->mu);
    auto it = bm->seqs.find(seq);
    if (it == bm->seqs.end()) return -1;
    const int32_t n = (int32_t)it->second.table.size();
    const int32_t k = std::min(n, std::max(cap, 0));
    if (out && k) std::memcpy(out, it->second.table.data(), (size_t)k * sizeof(int32_t));
    return n;
}

int32_t pa_bm_seq_blocks(pa_bm* bm, int64_t seq) {
    if (!bm) return -1;
    std::lock_guard<std::mutex> g(bm->mu);
    auto it = bm->seqs.find(seq);
    return it == bm->seqs.end() ? -1 : (int32_t)it->second.table.size();
}

}  // extern "C"

// Multi-threaded stress of the host block manager through its C ABI (test
// infrastructure: built and run by tests/test_bm_concurrency.py, with and
// without ThreadSanitizer).
//
// lpnh.cn/news/2758356 section 4.3: when several sequences share blocks,
// updates of the holder counts must be atomic.  Here every thread forks
// children off one shared parent sequence (counts of the parent's blocks go
// up from many threads at once), appends to them (the first append into the
// shared, partly filled tail copies it: that count goes down while other
// threads raise it), forks its own children, adds and frees sequences, and
// reads tables and slots -- all at the same time, against one pool.  Every
// thread checks what each call returns on its own sequences; at the end the
// main thread checks the pool: the parent's blocks are held once, every
// other block is free, the free list has every id exactly once.
//
// Usage: bm_stress [threads] [iterations per thread]; prints "ok ..." and
// exits 0, or prints the first violation and exits 1.
#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <thread>
#include <vector>

#include "pa.h"

namespace {

std::atomic<int> g_failed{0};

#define CHECK(cond, ...)                                  \
    do {                                                  \
        if (!(cond)) {                                    \
            if (g_failed.fetch_add(1) == 0) {             \
                std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
                std::fprintf(stderr, __VA_ARGS__);        \
                std::fprintf(stderr, "\n");               \
            }                                             \
            return;                                       \
        }                                                 \
    } while (0)

struct Rng {                 // splitmix64
    uint64_t s;
    uint64_t next() {
        uint64_t z = (s += 0x9e3779b97f4a7c15ull);
        z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
        z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
        return z ^ (z >> 31);
    }
    int below(int n) { return (int)(next() % (uint64_t)n); }
};

constexpr int32_t kPool = 6000;
constexpr int32_t kB = 16;
constexpr int64_t kParent = 1;
constexpr int32_t kParentLen = 100;            // 6 full blocks + 4 tokens: a partly filled tail
constexpr int kMaxLive = 24;

struct Mine {
    int64_t id;
    int64_t len;
};

// The slot of the sequence's last position agrees with its table.
bool slot_agrees(pa_bm* bm, int64_t seq, int64_t len, int64_t slot) {
    int32_t tab[512];
    const int32_t nb = pa_bm_seq_table(bm, seq, tab, 512);
    if (nb != (len + kB - 1) / kB || nb > 512) return false;
    const int64_t p = len - 1;
    return slot == (int64_t)tab[p / kB] * kB + p % kB;
}

void worker(pa_bm* bm, int t, int iters) {
    Rng rng{0x1234567ull * (uint64_t)(t + 1)};
    std::vector<Mine> live;
    int64_t next_id = 1000000ll * (t + 1);
    for (int it = 0; it < iters && g_failed.load() == 0; ++it) {
        const int r = rng.below(100);
        if (r < 20 && (int)live.size() < kMaxLive) {
            // fork the shared parent: its blocks' counts rise under contention
            const int64_t c = next_id++;
            const int rc = pa_bm_fork(bm, kParent, c);
            CHECK(rc == PA_OK, "fork of the parent: %d", rc);
            CHECK(pa_bm_seq_len(bm, c) == kParentLen, "child length");
            live.push_back({c, kParentLen});
        } else if (r < 30 && !live.empty() && (int)live.size() < kMaxLive) {
            // fork one of this thread's own sequences
            const Mine& p = live[rng.below((int)live.size())];
            const int64_t c = next_id++;
            const int rc = pa_bm_fork(bm, p.id, c);
            CHECK(rc == PA_OK, "fork: %d", rc);
            live.push_back({c, p.len});
        } else if (r < 40 && (int)live.size() < kMaxLive) {
            const int32_t n = rng.below(80);
            const int64_t c = next_id++;
            std::vector<int64_t> slots(n > 0 ? n : 1);
            const int rc = pa_bm_add_sequence(bm, c, n, slots.data());
            if (rc == PA_ERR_OOM) continue;
            CHECK(rc == PA_OK, "add: %d", rc);
            for (int32_t p = 0; p < n; ++p) CHECK(slots[p] >= 0 && slots[p] < (int64_t)kPool * kB, "slot range");
            live.push_back({c, n});
        } else if (r < 85 && !live.empty()) {
            Mine& m = live[rng.below((int)live.size())];
            int64_t slot = -1, src = -1, dst = -1;
            const int rc = pa_bm_append_token(bm, m.id, &slot, &src, &dst);
            if (rc == PA_ERR_OOM) continue;
            CHECK(rc == PA_OK || rc == PA_COW, "append: %d", rc);
            m.len += 1;
            CHECK(pa_bm_seq_len(bm, m.id) == m.len, "length after append");
            CHECK(slot_agrees(bm, m.id, m.len, slot), "slot of seq %lld", (long long)m.id);
            if (rc == PA_COW) {
                // the copy goes to a fresh block this sequence alone holds;
                // the source stays held by the others
                CHECK(src != dst && src >= 0 && dst >= 0, "cow pair %lld -> %lld", (long long)src, (long long)dst);
                CHECK(slot / kB == dst, "the written block is the copy");
                CHECK(pa_bm_refcount(bm, (int32_t)dst) == 1, "copy held once");
            } else {
                CHECK(src == -1 && dst == -1, "no pair without a copy");
            }
        } else if (!live.empty()) {
            const int k = rng.below((int)live.size());
            const int rc = pa_bm_free_sequence(bm, live[k].id);
            CHECK(rc == PA_OK, "free: %d", rc);
            CHECK(pa_bm_seq_len(bm, live[k].id) == -1, "freed sequence still known");
            live[k] = live.back();
            live.pop_back();
        }
    }
    for (const Mine& m : live) {
        const int rc = pa_bm_free_sequence(bm, m.id);
        CHECK(rc == PA_OK, "final free: %d", rc);
    }
}

// Readers: the pool-wide queries take the same lock.
void reader(pa_bm* bm, std::atomic<bool>* stop) {
    std::vector<int32_t> fl(kPool);
    while (!stop->load()) {
        const int32_t nf = pa_bm_num_free(bm);
        CHECK(nf >= 0 && nf <= kPool, "num_free %d", nf);
        const int32_t got = pa_bm_free_list(bm, fl.data(), kPool);
        CHECK(got >= 0 && got <= kPool, "free list length %d", got);
        for (int32_t b = 0; b < kPool; b += 97) CHECK(pa_bm_refcount(bm, b) >= 0, "count of %d", b);
    }
}

}  // namespace

int main(int argc, char** argv) {
    const int threads = argc > 1 ? std::atoi(argv[1]) : 8;
    const int iters = argc > 2 ? std::atoi(argv[2]) : 4000;
    pa_bm* bm = pa_bm_create(kPool, kB);
    if (!bm) {
        std::fprintf(stderr, "create failed\n");
        return 1;
    }
    if (pa_bm_add_sequence(bm, kParent, kParentLen, nullptr) != PA_OK) {
        std::fprintf(stderr, "parent add failed\n");
        return 1;
    }
    int32_t ptab[16];
    const int32_t pn = pa_bm_seq_table(bm, kParent, ptab, 16);
    std::atomic<bool> stop{false};
    std::thread rd(reader, bm, &stop);
    std::vector<std::thread> ws;
    for (int t = 0; t < threads; ++t) ws.emplace_back(worker, bm, t, iters);
    for (auto& w : ws) w.join();
    stop.store(true);
    rd.join();
    if (g_failed.load()) return 1;

    // the pool after everything but the parent is gone
    int bad = 0;
    std::vector<char> in_parent(kPool, 0);
    for (int32_t i = 0; i < pn; ++i) in_parent[ptab[i]] = 1;
    for (int32_t b = 0; b < kPool; ++b) {
        const int32_t want = in_parent[b] ? 1 : 0;
        if (pa_bm_refcount(bm, b) != want) {
            if (!bad++) std::fprintf(stderr, "FAIL: block %d held %d times, want %d\n", b, pa_bm_refcount(bm, b), want);
        }
    }
    std::vector<int32_t> fl(kPool);
    const int32_t nf = pa_bm_free_list(bm, fl.data(), kPool);
    std::vector<char> seen(kPool, 0);
    for (int32_t i = 0; i < nf; ++i) {
        if (fl[i] < 0 || fl[i] >= kPool || seen[fl[i]] || in_parent[fl[i]]) {
            if (!bad++) std::fprintf(stderr, "FAIL: free list entry %d\n", fl[i]);
        } else {
            seen[fl[i]] = 1;
        }
    }
    if (nf != kPool - pn && !bad++) std::fprintf(stderr, "FAIL: %d free, want %d\n", nf, kPool - pn);
    if (pa_bm_free_sequence(bm, kParent) != PA_OK || pa_bm_num_free(bm) != kPool) {
        if (!bad++) std::fprintf(stderr, "FAIL: pool not whole after the parent's release\n");
    }
    pa_bm_destroy(bm);
    if (bad) return 1;
    std::printf("ok threads=%d iterations=%d\n", threads, iters);
    return 0;
}

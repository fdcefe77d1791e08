/*
 * pa.h -- C ABI of the paged-KV-cache hot path for AMD Instinct MI355X
 * (gfx950).  Library: paged_kv_cache_390_amd/libpa.so.
 *
 * Sources cited below (pages named by address, sections as they number them):
 *   [5688vip]       5688vip.com, "4、PagedAttention：显存管理、分页机制、块大小选择"
 *   [n1n]           explore.n1n.ai, "PagedAttention 对比传统 KV 缓存：vLLM 如何重塑
 *                   LLM 推理的 GPU 显存管理"
 *   [lpnh-2758356]  lpnh.cn/news/2758356 (block mapping, on-demand allocation,
 *                   copy-on-write), sections 1-5
 *   [lpnh-1824136]  lpnh.cn/news/1824136 (the SOSP 2023 paper and vLLM),
 *                   sections 1-4
 *
 * Conventions shared by every GPU call
 *   - Cache layout: one K and one V tensor per layer, each
 *     [num_blocks, num_kv_heads, block_size, head_dim], fp16, contiguous.
 *     A physical block id indexes every layer's tensors, so one block table
 *     serves all layers ([lpnh-2758356] 2.1: per-block shape block_size x
 *     kv heads x head_dim, layers with their own block sets of one size).
 *   - Token position p of a sequence lives at slot table[p / B] * B + p % B,
 *     i.e. block table[p / B], row p % B ([5688vip] 分页机制 figure;
 *     [lpnh-2758356] 2.2).
 *   - All device buffers belong to the caller; the library never allocates
 *     device memory.  Pointers marked "device" must be device-accessible;
 *     every other pointer is host memory.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is
 *     the null stream).  The call returns once the kernels are enqueued.
 *   - Argument errors are found before anything is enqueued and leave every
 *     output untouched.  Device-resident indices (slots, table entries, copy
 *     pairs) cannot be checked without a device-to-host copy; instead the
 *     kernels skip any that fall outside the pool, so a bad index is never
 *     dereferenced (see each call for what the output then holds).
 *   - dtype: PA_DTYPE_F16 is the only element type.
 *   - head_dim in {16, 32, 64, 128, 256} (pa_prefill: 64, 128, 256); the attention
 *     calls take block_size in {1, 2, 4, 8, 16, 32, 64, 128}
 *     (PA_ERR_UNSUPPORTED otherwise); pa_reshape_and_cache and the block
 *     copies take any block size.
 *
 * Every function returns PA_OK (0) or a negative PA_ERR_* code, except where
 * stated.  pa_last_error() gives a message for the calling thread's last
 * failure.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    PA_OK = 0,
    PA_COW = 1,               /* append: a copy-on-write pair was produced   */
    PA_ERR_INVALID = -1,      /* null pointer, bad size or inconsistent dims */
    PA_ERR_UNSUPPORTED = -2,  /* dtype, head_dim or block_size not built     */
    PA_ERR_HIP = -3,          /* the HIP runtime reported an error           */
    PA_ERR_OOM = -4,          /* block manager: no free block                */
    PA_ERR_STATE = -5         /* block manager: unknown / duplicate sequence,
                                 block not free                              */
};

enum { PA_DTYPE_F16 = 0 };

/* Message for the calling thread's most recent failed call ("" if none). */
const char *pa_last_error(void);

/* ------------------------------------------------------------------------
 * Slot-mapped cache write ("reshape and cache").
 * The new tokens' K and V vectors are written into the blocks their tables
 * assign ([lpnh-1824136] 3.1: results are scattered back into the proper
 * blocks; [5688vip] 分页机制: a token goes into the current block while it
 * has room).
 *
 *   key, value     device, fp16, token t head h at element
 *                  t * kv_token_stride + h * head_dim (head_dim contiguous)
 *   kv_token_stride elements between consecutive tokens (>= Hkv * head_dim)
 *   slot_mapping   device, int64 [num_tokens]; token t goes to block
 *                  slot / block_size, row slot % block_size.  A negative
 *                  slot, or one >= num_blocks * block_size, is skipped.
 *                  Slots within one call must be distinct.
 *   k_cache, v_cache  device, fp16 [num_blocks, num_kv_heads, block_size,
 *                  head_dim]; updated in place, bit-exact copies.
 * num_tokens == 0 enqueues nothing.
 * ------------------------------------------------------------------------ */
int pa_reshape_and_cache(const void *key, const void *value,
                         int64_t kv_token_stride,
                         const int64_t *slot_mapping, int32_t num_tokens,
                         void *k_cache, void *v_cache, int32_t num_blocks,
                         int32_t num_kv_heads, int32_t block_size,
                         int32_t head_dim, int32_t dtype, void *stream);

/* ------------------------------------------------------------------------
 * Single-query decode attention over the paged cache.
 * Each sequence's new token attends to all of its cached K/V, read through
 * its block table ([lpnh-1824136] 2.2 and 3.2 step 4: the kernel looks up
 * the table and reads history K/V from scattered blocks; [lpnh-2758356] 2.2:
 * the result is that of ordinary attention over the logically contiguous
 * K/V).  The pages give no formula; computed is scaled dot-product softmax
 * attention, out = softmax(scale * K q) V over positions [0, n), with
 * fp32 accumulation and fp16 (round to nearest even) output.
 *
 *   out            device, fp16 [num_seqs, num_heads, head_dim], written
 *   q              device, fp16 [num_seqs, num_heads, head_dim]
 *   k_cache, v_cache  device, fp16 [num_blocks, num_kv_heads, block_size,
 *                  head_dim]
 *   block_tables   device, int32 [num_seqs, max_blocks_per_seq]; entries past
 *                  ceil(n / block_size) are never read
 *   context_lens   device, int32 [num_seqs]; n for each sequence, including
 *                  the token just written.  n == 0 gives an all-zero row.
 *   num_heads      query heads; num_heads % num_kv_heads == 0 and query head
 *                  h reads KV head h / (num_heads / num_kv_heads).  When 2 to
 *                  16 query heads share a KV head and head_dim is 64, 128 or
 *                  256, the products run on the matrix cores (one workgroup
 *                  reads each K/V block once for the whole group); otherwise
 *                  on the vector ALUs, one workgroup per query head.
 *   scale          multiplies q.k (1/sqrt(head_dim) in the usual model)
 *   max_context_len  host-known upper bound on every n; it sizes the grid so
 *                  that no device-to-host read is needed.  A row whose n
 *                  exceeds it, or exceeds max_blocks_per_seq * block_size,
 *                  comes out as NaN.
 *   partition_size tokens per context partition, a multiple of 128 (0 picks
 *                  a default).  Sequences longer than one partition are split
 *                  across workgroups and merged by a second kernel.
 *   workspace      device scratch of at least pa_decode_workspace_size()
 *                  bytes, 16-byte aligned.  It holds the partial results
 *                  when a sequence is split and, when seq_order is NULL, the
 *                  longest-first dispatch order (written by a small kernel
 *                  launched first).  With one partition it may be NULL (or
 *                  smaller): without seq_order the sequences then run in
 *                  index order, with the same results.  Contents on entry are
 *                  ignored; calls sharing a workspace must be stream-ordered.
 *   seq_order      device, int32 [num_seqs], or NULL: the order in which
 *                  the sequences are dispatched, as pa_decode_order writes
 *                  it (longest first, so that no long sequence starts last
 *                  and runs alone at the end).  Every layer of a step shares
 *                  one order: computing it once per step saves the small
 *                  kernel on every call.  The order never changes a result;
 *                  an entry outside [0, num_seqs) is skipped, and a sequence
 *                  the array leaves out keeps its output rows untouched.
 * Table entries outside [0, num_blocks) are skipped: their tokens take no
 * part in the softmax.
 * ------------------------------------------------------------------------ */
int pa_decode(void *out, const void *q, const void *k_cache,
              const void *v_cache, const int32_t *block_tables,
              int32_t max_blocks_per_seq, const int32_t *context_lens,
              int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
              int32_t head_dim, int32_t block_size, int32_t num_blocks,
              float scale, int32_t max_context_len, int32_t partition_size,
              void *workspace, size_t workspace_bytes,
              const int32_t *seq_order, int32_t dtype, void *stream);

/* ------------------------------------------------------------------------
 * Decode with the step's cache write folded in: pa_reshape_and_cache of one
 * new token per sequence followed by pa_decode, in one launch (the write
 * scatters the token into its block, [lpnh-1824136] 3.1; the attention is
 * pa_decode's).  Sequence s's new token sits at position n - 1 (n =
 * context_lens[s], which counts it):
 *
 *   key, value     device, fp16; the token of sequence s, KV head h at
 *                  element s * kv_token_stride + h * head_dim (head_dim
 *                  contiguous); 16-byte aligned
 *   kv_token_stride elements between consecutive sequences' tokens, a
 *                  multiple of 8 and >= num_kv_heads * head_dim
 *   k_cache, v_cache  as for pa_decode, and written: the token goes to
 *                  block block_tables[s][(n-1) / block_size], row (n-1) %
 *                  block_size -- the slot the block manager's append
 *                  reserved -- bit for bit.  A table entry outside
 *                  [0, num_blocks) writes nothing and, as in pa_decode,
 *                  the token takes no part in the softmax.
 * Every other argument, the output and the error behaviour are those of
 * pa_decode.  The cache is read for positions < n - 1 only; the new token's
 * K/V come from key / value, so the result does not depend on the slot's
 * contents before the call.  Sequences with n == 0, or with n above
 * max_context_len or the table width, write nothing, and so does a
 * sequence that seq_order leaves out (its output rows stay untouched, as
 * in pa_decode).  The written block
 * must not be shared with another sequence of the call (the block
 * manager's copy-on-write guarantees that for the last block of a
 * sequence).
 * ------------------------------------------------------------------------ */
int pa_decode_append(void *out, const void *q, const void *key,
                     const void *value, int64_t kv_token_stride,
                     void *k_cache, void *v_cache,
                     const int32_t *block_tables, int32_t max_blocks_per_seq,
                     const int32_t *context_lens, int32_t num_seqs,
                     int32_t num_heads, int32_t num_kv_heads,
                     int32_t head_dim, int32_t block_size, int32_t num_blocks,
                     float scale, int32_t max_context_len,
                     int32_t partition_size, void *workspace,
                     size_t workspace_bytes, const int32_t *seq_order,
                     int32_t dtype, void *stream);

/* ------------------------------------------------------------------------
 * pa_decode without a caller workspace, for callers that cannot allocate
 * device memory (code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid allocation).  The library keeps the workspace in a
 * device array of PA_NOALLOC_SCRATCH_BYTES bytes (1 MiB) per GPU, reserved
 * when the library's code is loaded on that GPU and held until the process
 * ends; the call itself allocates nothing.  (The array is kept small: the
 * HIP runtime was measured to spend about 1.5 us per MiB of such static
 * device arrays on every blocking host-to-device copy of the process.)
 * 1 MiB holds the dispatch order of any batch and the partial states of
 * about 2000 (sequence, head, partition) rows at head_dim 128; the default
 * partition needs none for batches of at least half a round of
 * workgroups.
 *
 * Arguments, results and error behaviour are those of pa_decode with
 * workspace = that array.  PA_ERR_INVALID, before anything is enqueued, when
 * the sizes need more workspace than the array holds
 * (pa_decode_workspace_size() > PA_NOALLOC_SCRATCH_BYTES).  Every call on
 * one GPU shares its array: calls that may overlap on a GPU (different
 * streams without ordering between them, or several host threads) race and
 * must be serialised by the caller.  Nothing in the array needs to be
 * cleared between calls.
 * ------------------------------------------------------------------------ */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)1 << 20)

int pa_decode_noalloc(void *out, const void *q, const void *k_cache,
                      const void *v_cache, const int32_t *block_tables,
                      int32_t max_blocks_per_seq, const int32_t *context_lens,
                      int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t num_blocks,
                      float scale, int32_t max_context_len,
                      int32_t partition_size, const int32_t *seq_order,
                      int32_t dtype, void *stream);

/* Longest-first dispatch order for pa_decode and pa_prefill: seq_order
 * (device, int32 [num_seqs], written) becomes a permutation of 0 ..
 * num_seqs - 1 with the sequences sorted by context_lens into 1024 classes of
 * max_context_len / 1024 + 1 tokens, longest class first (order within a
 * class unspecified).  Stream-ordered with the calls that use it. */
int pa_decode_order(int32_t *seq_order, const int32_t *context_lens,
                    int32_t num_seqs, int32_t max_context_len, void *stream);

/* ------------------------------------------------------------------------
 * Paged prefill / chunked prefill: several new tokens per sequence, each
 * attending causally to the cached positions up to its own.  This is the
 * prompt path of a request ([lpnh-1824136] 3.2, second step) over the paged
 * cache, which a contiguous-memory attention kernel cannot read ([n1n]
 * 权衡与局限性); the result is textbook softmax attention, and one new token
 * per sequence is exactly pa_decode.
 *
 *   out, q         device, fp16 [num_tokens, num_heads, head_dim]: the new
 *                  tokens of all sequences packed in sequence order
 *   query_start    device, int32 [num_seqs + 1]: sequence s owns rows
 *                  query_start[s] .. query_start[s+1] - 1 (m_s of them); a
 *                  sequence whose range is not inside [0, num_tokens) is
 *                  skipped (its rows are left untouched)
 *   context_lens   device, int32 [num_seqs]: n_s cached tokens INCLUDING the
 *                  m_s new ones, whose K/V must already be in the cache
 *                  (pa_reshape_and_cache); row query_start[s] + i is the
 *                  token at position n_s - m_s + i
 *   block_tables, k_cache, v_cache, num_blocks, block_size, scale: as for
 *                  pa_decode
 *   max_query_len  host-known bound on every m_s; it sizes the grid.  A
 *                  sequence with m_s > max_query_len, m_s > n_s or n_s beyond
 *                  its table gets its first max_query_len rows as NaN.
 *   workspace      device scratch of pa_prefill_workspace_size() bytes,
 *                  16-byte aligned, or NULL.  When the batch gives too few
 *                  workgroups to fill the GPU (few sequences or KV heads,
 *                  short chunks over long contexts) and the context bound
 *                  max_blocks_per_seq * block_size is at least 8 times
 *                  max_query_len (2 times when the row tiles give at most
 *                  128 workgroups), the context is split
 *                  into parts whose partial results it holds, merged by a
 *                  second kernel; when it gives more than one round of
 *                  resident workgroups, one query head per KV head and at
 *                  least 1024 query rows (8 row tiles at head_dim 64 and
 *                  128, 16 at 256) per (KV head, sequence), its first 256
 *                  bytes hold the counters
 *                  from which one round of persistent workgroups takes the
 *                  row tiles (zeroed by the call itself, in a kernel ahead
 *                  of the attention on the same stream).  Without it (NULL
 *                  or smaller) the context is not split and every row tile
 *                  gets a workgroup of its own; the results are the same
 *                  bit for bit.  Contents on entry are ignored; calls
 *                  sharing a workspace must be stream-ordered.
 *   seq_order      device, int32 [num_seqs], or NULL (index order): the
 *                  order in which the sequences' row tiles are dispatched,
 *                  as pa_decode_order writes it from context_lens (longest
 *                  first, so that no long prompt's row tiles start last and
 *                  run alone at the end).  Every layer of a step shares one
 *                  order.  The order never changes a result; an entry
 *                  outside [0, num_seqs) is skipped, and a sequence the array
 *                  leaves out keeps its output rows untouched.
 * head_dim 64, 128 or 256 (PA_ERR_UNSUPPORTED otherwise); any num_heads
 * multiple of num_kv_heads.  Runs on the matrix cores
 * (v_mfma_f32_16x16x32_f16, fp32 accumulation).
 * ------------------------------------------------------------------------ */
int pa_prefill(void *out, const void *q, int32_t num_tokens,
               const void *k_cache, const void *v_cache,
               const int32_t *block_tables, int32_t max_blocks_per_seq,
               const int32_t *context_lens, const int32_t *query_start,
               int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
               int32_t head_dim, int32_t block_size, int32_t num_blocks,
               float scale, int32_t max_query_len, void *workspace,
               size_t workspace_bytes, const int32_t *seq_order,
               int32_t dtype, void *stream);

/* ------------------------------------------------------------------------
 * pa_reshape_and_cache of the new tokens followed by pa_prefill, in one
 * call (the prompt path of a request, [lpnh-1824136] 3.2 second step: the
 * prompt's K/V are stored into the blocks while its attention runs).
 *
 *   key, value     device, fp16; new token row i (the row of q holding it)
 *                  and KV head h at element i * kv_token_stride + h *
 *                  head_dim (head_dim contiguous); 16-byte aligned
 *   kv_token_stride elements between consecutive token rows, a multiple of
 *                  8 and >= num_kv_heads * head_dim
 *   k_cache, v_cache  as for pa_prefill, and written: new token i of
 *                  sequence s (position p = n_s - m_s + i) goes to block
 *                  block_tables[s][p / block_size], row p % block_size, bit
 *                  for bit.  A table entry outside [0, num_blocks) writes
 *                  nothing and the token takes no part in any softmax.
 * Every other argument, the output and the error behaviour are those of
 * pa_prefill.  The cache is read for positions < n_s - m_s only; the new
 * tokens' K/V come from key / value, so the result does not depend on their
 * slots' contents before the call.  A sequence that pa_prefill skips or
 * answers with NaN writes nothing.  The blocks written must not be shared
 * with another sequence of the call (the block manager gives a sequence
 * its own blocks for new tokens).
 * ------------------------------------------------------------------------ */
int pa_prefill_append(void *out, const void *q, int32_t num_tokens,
                      const void *key, const void *value,
                      int64_t kv_token_stride, void *k_cache, void *v_cache,
                      const int32_t *block_tables, int32_t max_blocks_per_seq,
                      const int32_t *context_lens, const int32_t *query_start,
                      int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t num_blocks,
                      float scale, int32_t max_query_len, void *workspace,
                      size_t workspace_bytes, const int32_t *seq_order,
                      int32_t dtype, void *stream);

/* Bytes of workspace pa_prefill uses for these sizes: when the context is
 * split, (2 + head_dim) x 4 bytes per (token, head, context part), in two
 * 256-byte aligned regions; otherwise 256 (the persistent grid's counters)
 * when the batch has more than 256 row-tile workgroups, else 0.  The context
 * bound is max_blocks_per_seq x block_size.  (size_t)-1 for invalid
 * arguments. */
size_t pa_prefill_workspace_size(int32_t num_tokens, int32_t num_seqs,
                                 int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size,
                                 int32_t max_blocks_per_seq,
                                 int32_t max_query_len);

/* Bytes of workspace pa_decode uses for these sizes: the dispatch order
 * (4 bytes per sequence, rounded up to 256; none for a single sequence) plus,
 * when a sequence can span several partitions, the partial results.
 * partition_size as for pa_decode (0 = default).  Returns (size_t)-1 for
 * invalid arguments. */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_heads,
                                int32_t num_kv_heads, int32_t head_dim,
                                int32_t block_size, int32_t max_context_len,
                                int32_t partition_size);

/* The partition size pa_decode uses when given 0.  With rows =
 * num_seqs x num_heads (x num_kv_heads on the matrix-core path), slots = the
 * workgroups of the serving kernel resident at once (1024 on the vector
 * path, 512 on the matrix-core path with blocks of 16 or more tokens) and
 * cover = max_context_len rounded up to a multiple of 128 (one partition
 * for every context, no merge kernel):
 *   - cover when rows fill half a round to one round of slots, or more than
 *     one round a whole number of times or with the last round at least 3/4
 *     full;
 *   - above one round otherwise, the longest of 2048, 1024, 512 and 256
 *     tokens that gives at least four workgroups per slot counting full
 *     partitions of a max_context_len sequence (256 when none does);
 *   - below half a round, the bound cut into enough parts for one workgroup
 *     per compute unit (256 of them), parts of at least 256 tokens.
 * -1 for invalid arguments. */
int32_t pa_decode_default_partition(int32_t num_seqs, int32_t num_heads,
                                    int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size,
                                    int32_t max_context_len);

/* ------------------------------------------------------------------------
 * Whole-block copies for copy-on-write.
 * A writer holding a shared block that still has free rows gets a new block
 * holding a copy of the shared one ([lpnh-2758356] 4.2, third step; 4.3 on
 * the bandwidth this costs).
 *
 *   k_caches, v_caches  HOST arrays of num_layers device pointers, each a
 *                  cache tensor of num_blocks blocks of block_elems fp16
 *   src_dst_pairs  device, int64 [num_pairs, 2]; row i copies block
 *                  pairs[i][0] onto block pairs[i][1] in every layer, K and V.
 *                  Destinations must be distinct and never also a source (a
 *                  source may repeat).  A pair with an id outside
 *                  [0, num_blocks) is skipped.
 *   block_elems    elements per block = num_kv_heads * block_size * head_dim
 * num_pairs == 0 or num_layers == 0 enqueues nothing.
 * ------------------------------------------------------------------------ */
int pa_copy_blocks(void *const *k_caches, void *const *v_caches,
                   int32_t num_layers, const int64_t *src_dst_pairs,
                   int32_t num_pairs, int32_t num_blocks, int64_t block_elems,
                   int32_t dtype, void *stream);

/* ------------------------------------------------------------------------
 * Whole-block copies between the device cache and a host cache ("swap").
 * Under memory pressure a sequence's KV blocks can be moved out to host
 * memory and back later, at a large latency cost ([lpnh-1824136] 4.2).  The
 * block manager's pa_bm_swap_out / pa_bm_swap_in produce the pairs.
 *
 *   dev_caches     HOST array of num_caches device pointers: cache tensors of
 *                  dev_num_blocks blocks of block_elems fp16 each (list the K
 *                  and the V tensor of every layer)
 *   host_caches    HOST array of num_caches pointers to pinned, device-mapped
 *                  host memory (hipHostMalloc, or a pinned torch tensor) of
 *                  host_num_blocks blocks each; host_caches[i] mirrors
 *                  dev_caches[i]
 *   pairs          device, int64 [num_pairs, 2]: (source id, destination id);
 *                  PA_SWAP_OUT copies device block pairs[i][0] to host block
 *                  pairs[i][1], PA_SWAP_IN host block pairs[i][0] to device
 *                  block pairs[i][1].  Destinations must be distinct.  A pair
 *                  with an id outside its pool is skipped.
 * The copy runs as one kernel per 128 caches that reads or writes the host
 * side through its device mapping (PCIe).  PA_ERR_INVALID, before anything is
 * enqueued, if a device pointer is not device memory or a host pointer is not
 * pinned, mapped host memory.  The caller orders it on the stream before
 * anything that reuses the source blocks (pa_bm_swap_out frees them at once).
 * ------------------------------------------------------------------------ */
enum { PA_SWAP_OUT = 0, PA_SWAP_IN = 1 };

int pa_swap_blocks(void *const *dev_caches, void *const *host_caches,
                   int32_t num_caches, const int64_t *pairs, int32_t num_pairs,
                   int32_t dev_num_blocks, int32_t host_num_blocks,
                   int64_t block_elems, int32_t direction, int32_t dtype,
                   void *stream);

/* ------------------------------------------------------------------------
 * Host block manager: free list, reference counts, per-sequence tables.
 * Host memory only; every call takes an internal lock, so calls from
 * several threads are serialised ([lpnh-2758356] 4.3: count updates must be
 * atomic).
 *
 * Rules ([n1n] 实现逻辑代码示例; [5688vip] 分页机制; [lpnh-2758356] 3.1, 3.2, 4.2):
 *   - the pool starts as ids 0..num_blocks-1 on a free list; an allocation
 *     takes the id at its end; a freed id is pushed on its end;
 *   - a new block is appended to a table only when the sequence has none or
 *     its last block is full;
 *   - every allocated block has a count of holders; fork adds one per block;
 *   - appending into a shared block (count > 1) that still has free rows
 *     first copies it: a new block replaces it in this table, the old count
 *     drops by one and the pair (old, new) is reported for pa_copy_blocks;
 *     a shared block that is full is never copied;
 *   - freeing a sequence drops each of its blocks' counts and returns blocks
 *     whose count reaches 0.
 * Any call that fails (OOM included) leaves the state unchanged, except the
 * batched append, which applies the appends before the failing one.
 * ------------------------------------------------------------------------ */
typedef struct pa_bm pa_bm;

/* NULL on bad sizes or out of host memory.  pa_bm_create has no host pool
 * (num_host_blocks = 0). */
pa_bm *pa_bm_create(int32_t num_blocks, int32_t block_size);
pa_bm *pa_bm_create_with_host(int32_t num_blocks, int32_t block_size,
                              int32_t num_host_blocks);
void pa_bm_destroy(pa_bm *bm);

/* New sequence with n_tokens tokens: ceil(n_tokens / B) blocks taken from
 * the free list in logical order.  slots_out (may be NULL) receives the
 * n_tokens slots.  PA_ERR_STATE if seq exists, PA_ERR_OOM if short of
 * blocks. */
int pa_bm_add_sequence(pa_bm *bm, int64_t seq, int32_t n_tokens,
                       int64_t *slots_out);

/* New sequence given its prompt's token ids (host int32 [n_tokens]),
 * sharing the blocks of a common prefix with sequences already there
 * ([n1n] 前缀缓存: requests with one long system prompt share its physical
 * blocks; [lpnh-1824136] 3.2, second step).  Every full block of a prompt
 * added this way is indexed by (the id of the block before it, or -1; its
 * B token ids); a new prompt takes each leading full block whose key it
 * finds (count + 1) and allocates the rest.  A partial last block is never
 * shared this way.  An indexed block leaves the index when its count
 * reaches 0.  slots_out (may be NULL) receives all n_tokens slots;
 * *num_cached_out the number of leading positions whose K/V are already in
 * shared blocks -- the caller computes and writes only the rest.
 * PA_ERR_STATE if seq exists, PA_ERR_OOM (state unchanged) if short of
 * blocks. */
int pa_bm_add_sequence_cached(pa_bm *bm, int64_t seq, const int32_t *token_ids,
                              int32_t n_tokens, int64_t *slots_out,
                              int32_t *num_cached_out);
/* Number of full blocks currently in the prefix index. */
int32_t pa_bm_num_cached_blocks(pa_bm *bm);

/* New sequence with an explicit table: nblk == ceil(n_tokens / B) distinct
 * ids, each currently free; they leave the free list (the rest keep their
 * order) with a count of 1. */
int pa_bm_set_table(pa_bm *bm, int64_t seq, const int32_t *blocks,
                    int32_t nblk, int32_t n_tokens);

/* child shares every block of parent (counts + 1) and its length. */
int pa_bm_fork(pa_bm *bm, int64_t parent, int64_t child);

/* Reserve the slot of seq's next token.  Returns PA_OK, or PA_COW when the
 * shared last block had to be copied (then *cow_src / *cow_dst hold the
 * pair; otherwise they are set to -1).  Output pointers may be NULL. */
int pa_bm_append_token(pa_bm *bm, int64_t seq, int64_t *slot_out,
                       int64_t *cow_src, int64_t *cow_dst);

/* Batched append, in the order given.  slots_out[n]; cow_pairs_out receives
 * up to n (src, dst) rows and *num_cow_out their count; *num_done_out the
 * number of appends applied.  Stops at the first failure and returns its
 * code (the appends before it stay applied). */
int pa_bm_append_tokens(pa_bm *bm, const int64_t *seqs, int32_t n,
                        int64_t *slots_out, int64_t *cow_pairs_out,
                        int32_t *num_cow_out, int32_t *num_done_out);

/* Release seq: counts - 1, ids reaching 0 pushed on the free list in
 * logical order (the host pool's, for a swapped-out sequence). */
int pa_bm_free_sequence(pa_bm *bm, int64_t seq);

/* Swap a group of n distinct sequences out to the host pool, or back in.
 * Every distinct block of the group, in order of first appearance
 * (sequence order, then table order), gets one block of the other pool
 * (allocated from the end of its free list) whose count is the number of
 * group members holding it, so blocks shared by forks stay shared; the old
 * block's count drops by that number and it is freed at 0.  pairs_out
 * receives (old id, new id) rows -- (device, host) for swap_out, (host,
 * device) for swap_in -- and *num_pairs_out their number.  A swapped-out
 * sequence can only be swapped in or freed (other calls: PA_ERR_STATE).
 * PA_ERR_OOM if the other pool has too few free blocks, PA_ERR_INVALID if
 * cap is too small: both leave the state unchanged. */
int pa_bm_swap_out(pa_bm *bm, const int64_t *seqs, int32_t n,
                   int64_t *pairs_out, int32_t cap, int32_t *num_pairs_out);
int pa_bm_swap_in(pa_bm *bm, const int64_t *seqs, int32_t n,
                  int64_t *pairs_out, int32_t cap, int32_t *num_pairs_out);
/* 1 if seq is swapped out, 0 if resident, -1 if unknown. */
int32_t pa_bm_is_swapped(pa_bm *bm, int64_t seq);
/* Holders of host block hblk (0 if free); -1 if outside the host pool. */
int32_t pa_bm_host_refcount(pa_bm *bm, int32_t hblk);
/* Like pa_bm_free_list, for the host pool. */
int32_t pa_bm_host_free_list(pa_bm *bm, int32_t *out, int32_t cap);
/* Copies min(len, cap) ids of seq's table (host ids while swapped out) into
 * out; returns the table length, or -1 if seq is unknown. */
int32_t pa_bm_seq_table(pa_bm *bm, int64_t seq, int32_t *out, int32_t cap);

/* Pack tables of the given sequences into tables_out[n, max_blocks] (padding
 * -1) and their lengths into lens_out[n] (may be NULL).  PA_ERR_INVALID if a
 * table is longer than max_blocks. */
int pa_bm_get_tables(pa_bm *bm, const int64_t *seqs, int32_t n,
                     int32_t *tables_out, int32_t max_blocks,
                     int32_t *lens_out);

/* Slots of positions [pos_begin, pos_begin + count) of seq; every position
 * must lie inside its table (< table length * B). */
int pa_bm_get_slots(pa_bm *bm, int64_t seq, int32_t pos_begin, int32_t count,
                    int64_t *slots_out);

/* Holders of block blk (0 if free); -1 if blk is outside the pool. */
int32_t pa_bm_refcount(pa_bm *bm, int32_t blk);
/* Number of free blocks. */
int32_t pa_bm_num_free(pa_bm *bm);
/* Copies min(count, cap) free ids, bottom of the list first, into out;
 * returns count. */
int32_t pa_bm_free_list(pa_bm *bm, int32_t *out, int32_t cap);
/* Length of seq, or -1 if unknown. */
int32_t pa_bm_seq_len(pa_bm *bm, int64_t seq);
/* Table length of seq, or -1 if unknown. */
int32_t pa_bm_seq_blocks(pa_bm *bm, int64_t seq);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */

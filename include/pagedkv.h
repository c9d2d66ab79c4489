/*
 * pagedkv.h -- C ABI of the MI355X (gfx950) paged KV-cache library.
 *
 * Three operations form the decode hot path of a paged KV cache:
 *   pkv_paged_attention_decode  single-query attention read through block tables
 *   pkv_reshape_and_cache       write each new token's K/V into its slot
 *   pkv_copy_blocks             copy whole blocks (copy-on-write)
 * plus pkv_paged_attention_decode_append (a decode step's append and attention in
 * one call), the same calls over 8-bit (FP8 E4M3) caches, attention of several query
 * tokens per sequence (pkv_paged_attention_chunk: prefill chunks, draft
 * verification), a decode that reads prefix blocks shared by several sequences once
 * (pkv_paged_attention_decode_grouped), block swaps between GPU and pinned host pools
 * (pkv_swap_blocks), workspace sizing and initialisation, version and error strings.
 *
 * Pages cited (titles as published):
 *   [P1] "vLLM 源码解析：PagedAttention 如何让大模型推理提速 10 倍"
 *   [P2] "vLLM 核心源码深度解析：PagedAttention 的 KV Cache 管理、Scheduler 调度引擎与
 *         Continuous Batching 实现全解"
 *   [P3] "论文专题讲解：vLLM / PagedAttention：为什么 KV cache 需要分页管理"
 *
 * Common rules for every call:
 *  - All array pointers are DEVICE memory owned by the caller (pkv_swap_blocks also
 *    takes pinned host memory); the library never allocates, frees or retains them.
 *    Arrays are dense, row-major, contiguous.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream) and the
 *    call returns before it completes. Nothing synchronises inside a call unless
 *    the environment variable PKV_VALIDATE=1 is set (see below).
 *  - Return value: PKV_OK (0), or a negative PKV_E_* code for errors the host can
 *    see (NULL pointers, bad sizes, unsupported shapes, a too-small workspace, a
 *    launch failure). Nothing is enqueued when a call returns an error.
 *  - Contents of index arrays (block IDs, context lengths, slots, pairs) are the
 *    caller's contract and are not checked on the host. The kernels never access
 *    memory outside the arrays described by the size arguments: an out-of-range
 *    block ID is skipped, a context longer than its table row is cut to the row,
 *    a negative context counts as empty, an out-of-range slot or pair writes
 *    nothing. Results for such inputs are unspecified.
 *  - PKV_VALIDATE=1: before enqueuing, the index arrays are copied to the host
 *    (a synchronising copy on `stream`) and checked; violations return
 *    PKV_E_INDEX and enqueue nothing.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, out, k/v and the caches (all share one type, except in the
 * *_fp8 calls, whose caches hold OCP FP8 E4M3 codes). */
typedef enum {
    PKV_FLOAT32 = 0,
    PKV_BFLOAT16 = 1,
    PKV_FLOAT16 = 2
} pkv_dtype;

enum {
    PKV_OK = 0,
    PKV_E_NULL = -1,         /* a required pointer is NULL */
    PKV_E_SHAPE = -2,        /* a size is negative/zero where it must be positive, or inconsistent */
    PKV_E_HEADS = -3,        /* num_heads is not a multiple of num_kv_heads, or the group is too large */
    PKV_E_UNSUPPORTED = -4,  /* dtype / head_dim / block_size combination not supported */
    PKV_E_WORKSPACE = -5,    /* workspace NULL or smaller than pkv_paged_attention_workspace_size() */
    PKV_E_LAUNCH = -6,       /* the HIP runtime reported an error when enqueuing */
    PKV_E_INDEX = -7,        /* PKV_VALIDATE=1 only: an index array holds an out-of-range entry */
    PKV_E_DEVICE = -8,       /* no current HIP device could be queried */
    PKV_E_NOSPACE = -9,      /* block manager: no free or evictable block for the request */
    PKV_E_SEQUENCE = -10,    /* block manager: unknown sequence id, or the id is taken */
    PKV_E_SCRATCH = -11      /* the call needs more scratch than PKV_NOALLOC_SCRATCH_BYTES */
};

/* A hipStream_t passed as an opaque pointer. */
typedef void* pkv_stream_t;

/* Library version string, e.g. "pagedkv 0.1.0 gfx950". Static storage. */
const char* pkv_version(void);

/* Human-readable text for a PKV_* code. Static storage; never NULL. */
const char* pkv_strerror(int code);

/*
 * Bytes of device workspace pkv_paged_attention_decode needs for these sizes and
 * this partition_size (same meaning as in the decode call). The value depends only
 * on its arguments (no device query), so it can be computed once per shape bucket;
 * it can be 0. Returns 0 for invalid sizes as well; the decode call then reports
 * the error.
 */
size_t pkv_paged_attention_workspace_size(int num_seqs, int num_heads, int num_kv_heads,
                                          int head_dim, int block_size,
                                          int max_blocks_per_seq, int partition_size);

/*
 * Where a decode call with a partition size keeps its per-partition results in the
 * workspace. A long context is cut into partitions; each partition's attention is
 * reduced to a log-sum-exp record, and the reduction kernel merges the records of a
 * row ([P1] section 四: per-block partial attention, merged at the end). The same
 * records are what two devices holding different parts of one context would need to
 * exchange.
 *
 * Arguments are those of the decode call (dtype included: it selects the kernel).
 * Returns P, the partitions per (sequence, query head) row, and fills offsets[0..2]
 * with the byte offsets in the workspace of three float32 arrays, record index
 * r = (b * num_heads + h) * P + p:
 *   m [r]             the partition's reference score, in base-2 units (score =
 *                     scale * q.k * log2 e): at most the partition's largest score
 *                     and less than 8 below it
 *   l [r]             sum over the partition's tokens of 2^(score - m)
 *   o [r, head_dim]   sum of 2^(score - m) * v over those tokens, divided by l
 *                     (and multiplied by v_scale for 8-bit caches)
 * Records exist after the call completes, for the sequences whose context spans more
 * than one partition; partitions past a context's end are not written. Returns 0
 * (offsets zero) when the call keeps no records (no partition size, or at most one
 * partition per context); a negative PKV_E_* for sizes the decode call would refuse.
 * Host only: no device access.
 */
int pkv_paged_attention_partials_layout(int num_seqs, int num_heads, int num_kv_heads,
                                        int head_dim, int block_size, int max_blocks_per_seq,
                                        int partition_size, pkv_dtype dtype,
                                        size_t offsets[3]);

/*
 * Zero-fill a workspace with a kernel on `stream` (no memset node, so the call can
 * sit inside a captured graph). A workspace must be zero-filled once before its
 * first use; every decode call leaves its bookkeeping zeroed again on completion,
 * so later calls need no re-initialisation. Decode calls that run concurrently must
 * use distinct workspaces.
 */
int pkv_workspace_init(void* workspace, size_t workspace_bytes, pkv_stream_t stream);

/*
 * Paged decode attention (one query token per sequence).
 *
 * Defined by [P1] section 四 (the kernel walks, per query, the physical blocks of
 * its page table, attends each block and merges the partial results) and [P3]
 * section "PagedAttention：逻辑连续，物理不必连续" (the query at position i attends
 * tokens 1..i; the keys/values of logical block j are tokens (j-1)B+1..jB). Token
 * position t of sequence b is read from physical block block_tables[b][t / bs] at
 * offset t % bs ([P2] section "Block Table 数据结构"). Per-block partial results are
 * merged with an online softmax; long contexts are split into partitions whose
 * (max, sum, output) are merged by a log-sum-exp reduction.
 *
 *   out[b,h,:] = sum_t softmax_t(scale * q[b,h,:] . K_b[t,:]) * V_b[t,:],
 *   t = 0 .. context_lens[b]-1, K_b/V_b read from KV head h / (num_heads/num_kv_heads).
 *
 * out           [num_seqs, num_heads, head_dim]                 written
 * q             [num_seqs, num_heads, head_dim]                 read
 * k_cache       [num_blocks, num_kv_heads, block_size, head_dim] read
 * v_cache       [num_blocks, num_kv_heads, block_size, head_dim] read
 * block_tables  int32 [num_seqs, max_blocks_per_seq]; entries at or beyond
 *               ceil(context_lens[b] / block_size) are never read (pad with -1)
 * context_lens  int32 [num_seqs]; the tokens each query attends, the new token
 *               included; 0 gives an all-zero output row
 * scale         multiplier of q.k (typically 1/sqrt(head_dim))
 * dtype         element type of out, q and the caches; accumulation is float32,
 *               the output is rounded to nearest-even
 * partition_size  0: the library chooses how to split the work (recommended;
 *               a context far longer than the batch's average is cut across
 *               several workgroups, their results merged through the workspace);
 *               >0: split every context into partitions of this many tokens
 *               (a multiple of block_size), one partial result per partition,
 *               merged by a separate reduction kernel
 * workspace     device scratch of at least pkv_paged_attention_workspace_size()
 *               bytes, zero-filled before first use (pkv_workspace_init); may be
 *               NULL only when that size is 0
 * Supported: head_dim in {64, 128, 256}; block_size in {1, 2, 4, 8, 16, 32};
 * num_heads / num_kv_heads <= 16 (group sizes above 8 need bfloat16/float16,
 * block_size 16, head_dim 128). Deterministic: the same inputs give
 * bit-identical outputs.
 */
int pkv_paged_attention_decode(void* out, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_tables,
                               const int32_t* context_lens, float scale, int num_seqs,
                               int num_heads, int num_kv_heads, int head_dim, int block_size,
                               int max_blocks_per_seq, int num_blocks, pkv_dtype dtype,
                               int partition_size, void* workspace, size_t workspace_bytes,
                               pkv_stream_t stream);

/*
 * pkv_paged_attention_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid allocation. It runs the same kernels as
 * pkv_paged_attention_decode (bit-identical results); their scratch (merge counters,
 * partial results, per-partition records) is a fixed array of
 * PKV_NOALLOC_SCRATCH_BYTES in device memory that the library holds on every GPU it
 * runs on until the process ends. The call never allocates or frees device memory.
 *
 * Arguments, supported shapes, results and errors are those of
 * pkv_paged_attention_decode, plus PKV_E_SCRATCH (nothing enqueued) when the call's
 * scratch, pkv_paged_attention_workspace_size() for its shape and partition_size,
 * exceeds PKV_NOALLOC_SCRATCH_BYTES. The library's own split (partition_size 0)
 * fits at every supported size; fixed partitions fit while
 * num_seqs * num_heads * partitions * (head_dim + 2) * 4 bytes stay below about
 * 71 MiB (e.g. 8 sequences x 32 heads x 256 partitions of 512 tokens at head_dim 128).
 *
 * The first call on a device finds that device's copy of the array and clears its
 * counter region on `stream`. Every call on one GPU shares that GPU's array, and
 * each call leaves its counters zeroed for the next. Calls whose work may overlap on
 * one GPU (different streams, or different host threads) race on the array and give
 * undefined results: serialise them on one stream.
 */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)72 << 20)
int pkv_paged_attention_decode_noalloc(void* out, const void* q, const void* k_cache,
                                       const void* v_cache, const int32_t* block_tables,
                                       const int32_t* context_lens, float scale, int num_seqs,
                                       int num_heads, int num_kv_heads, int head_dim,
                                       int block_size, int max_blocks_per_seq, int num_blocks,
                                       pkv_dtype dtype, int partition_size,
                                       pkv_stream_t stream);

/*
 * One whole decode step in one call: append each sequence's newest token, then attend.
 * The step follows [P3] section "Block table：为什么它能减少碎片": the token just
 * generated goes into the free slot of its sequence's last block, or into a newly
 * taken block, and the query then attends over the context including that token. Its
 * slot is the block-table walk of [P2] section "Block Table 数据结构" applied to
 * position context_lens[b] - 1.
 *
 * The result is the same as two calls:
 *   pkv_reshape_and_cache(new_k, new_v, k_cache, v_cache, slot_mapping, num_seqs, ...)
 *   pkv_paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens, ...)
 * with slot_mapping[b] = block_tables[b][(n-1)/block_size] * block_size
 * + (n-1) % block_size, where n = context_lens[b], and -1 (skip) when n == 0.
 *
 * On the matrix-core paths the append runs inside the decode kernel, so the step is
 * one launch. The workgroup that reads a sequence's last block writes the new row
 * before it loads that block. On other paths a small append kernel runs first.
 *
 * new_k, new_v  [num_seqs, num_kv_heads, head_dim], dtype; read. Must be non-NULL when
 *               num_seqs > 0.
 * k_cache, v_cache  read and written: only the slot at position context_lens[b] - 1
 *               of each sequence changes, and it receives a bit-exact copy.
 * All other arguments, the workspace rules and the errors are those of
 * pkv_paged_attention_decode.
 *
 * Caller contract:
 *  - No two sequences may append into the same slot.
 *  - The slot a sequence writes must lie in a block that no other sequence of the
 *    batch reads. Copy-on-write guarantees this: a shared block is copied before a
 *    writer touches it. Where the contract is broken, the other sequence may see the
 *    old or the new row.
 */
int pkv_paged_attention_decode_append(void* out, const void* q, const void* new_k,
                                      const void* new_v, void* k_cache, void* v_cache,
                                      const int32_t* block_tables, const int32_t* context_lens,
                                      float scale, int num_seqs, int num_heads,
                                      int num_kv_heads, int head_dim, int block_size,
                                      int max_blocks_per_seq, int num_blocks, pkv_dtype dtype,
                                      int partition_size, void* workspace,
                                      size_t workspace_bytes, pkv_stream_t stream);

/*
 * 8-bit KV caches. [P2] lists an FP8 KV cache among the engine's milestones (section
 * "vLLM 的发展里程碑"), and [P3]'s KV-size formula notes that quantisation lowers the
 * bytes per element. The format and the scales are this library's reading, since the
 * pages fix neither.
 *  - Each cache element is one byte, an OCP FP8 E4M3 code: 1 sign bit, 4 exponent bits
 *    with bias 7, 3 mantissa bits, no infinities, S.1111.111 = NaN, largest finite 448.
 *  - Each cache has one scale, so key = decode(code) * k_scale and
 *    value = decode(code) * v_scale. Both scales must be positive and finite
 *    (PKV_E_SHAPE otherwise).
 *  - Appending stores code = E4M3(float(x) * (1.0f / scale)): one binary32 product with
 *    the binary32 reciprocal, rounded to the nearest code (ties to an even mantissa).
 *    Magnitudes of 448 or more saturate to +-448; NaN stays NaN.
 *  - q, out and the appended rows keep their 16-bit dtype. Every E4M3 value is exact
 *    in bfloat16 and float16, so the attention arithmetic is that of the 16-bit calls.
 *  - Supported: dtype bfloat16/float16, head_dim 128, block_size 16 (the matrix-core
 *    kernels); other shapes return PKV_E_UNSUPPORTED.
 * Caches are [num_blocks, num_kv_heads, block_size, head_dim] bytes. pkv_copy_blocks
 * serves them unchanged, with block_bytes = num_kv_heads * block_size * head_dim.
 */

/* pkv_paged_attention_decode over 8-bit caches (arguments as there, plus the scales). */
int pkv_paged_attention_decode_fp8(void* out, const void* q, const void* k_cache,
                                   const void* v_cache, float k_scale, float v_scale,
                                   const int32_t* block_tables, const int32_t* context_lens,
                                   float scale, int num_seqs, int num_heads, int num_kv_heads,
                                   int head_dim, int block_size, int max_blocks_per_seq,
                                   int num_blocks, pkv_dtype dtype, int partition_size,
                                   void* workspace, size_t workspace_bytes,
                                   pkv_stream_t stream);

/* pkv_paged_attention_decode_append over 8-bit caches: new_k/new_v ([num_seqs,
 * num_kv_heads, head_dim], dtype) are quantised as described above into the slot of
 * each sequence's last context position, then attended. Same caller contract. */
int pkv_paged_attention_decode_append_fp8(void* out, const void* q, const void* new_k,
                                          const void* new_v, void* k_cache, void* v_cache,
                                          float k_scale, float v_scale,
                                          const int32_t* block_tables,
                                          const int32_t* context_lens, float scale,
                                          int num_seqs, int num_heads, int num_kv_heads,
                                          int head_dim, int block_size, int max_blocks_per_seq,
                                          int num_blocks, pkv_dtype dtype, int partition_size,
                                          void* workspace, size_t workspace_bytes,
                                          pkv_stream_t stream);

/*
 * Decode of a batch whose sequences share prefix blocks, reading each shared block
 * once per group instead of once per sequence. [P1] section 五 and [P3] section
 * "共享前缀和 copy-on-write" describe the sharing: the samples of one prompt (parallel
 * sampling, beam search, requests under one system prompt) point their block tables at
 * the same physical blocks of the prompt, and only the block that one of them writes
 * is copied. The result is that of pkv_paged_attention_decode (new_k == NULL) or
 * pkv_paged_attention_decode_append (new_k != NULL) on the same arguments; only the
 * order in which partial results are merged differs, so results agree with those calls
 * within rounding, not bit for bit.
 *
 * Groups: group i is the consecutive sequences group_start[i] .. group_start[i+1]-1,
 * whose block tables hold the same physical blocks in entries 0 .. group_prefix[i]-1.
 * The groups cover the batch in order: group_start[0] = 0, non-decreasing,
 * group_start[num_groups] = num_seqs (a sequence that shares nothing is a group of one
 * with prefix 0). pkv_prefix_groups derives such groups from the tables on the host.
 *
 * How it runs: the members of a group are the columns of the matrix-core tiles (a
 * tile of 16 columns holds 16 / G whole members, G = num_heads / num_kv_heads). One
 * workgroup per (group, KV head, tile) reads each prefix block once for all of its
 * members, then each member's own blocks, and writes the members' output rows. A
 * prefix longer than 128 blocks is cut into parts of 128 blocks, one workgroup each,
 * whose log-sum-exp records go to the workspace and are merged by a second kernel. A
 * member attends the prefix blocks before its own context end; with new_k != NULL the
 * block of its newest token is always read as one of its own blocks, after the
 * workgroup has written the token, even when the group's prefix covers it.
 *
 * group_start   int32 [num_groups + 1], device
 * group_prefix  int32 [num_groups], device; each in [0, max_prefix_blocks]
 * num_groups    >= 1 when num_seqs > 0
 * max_group_size  the largest group_start[i+1] - group_start[i] (at least 1)
 * max_prefix_blocks  an upper bound of group_prefix (<= max_blocks_per_seq); sizes
 *               the workspace and the grid
 * new_k, new_v  NULL (plain decode) or [num_seqs, num_kv_heads, head_dim] rows appended
 *               at position context_lens[b] - 1 before the attention, as in
 *               pkv_paged_attention_decode_append; both NULL or both non-NULL
 *               (PKV_E_NULL otherwise)
 * workspace     device scratch of at least pkv_paged_attention_grouped_workspace_size()
 *               bytes, which is 0 (NULL allowed) when max_prefix_blocks <= 128; no
 *               initialisation needed; its first MiB is left untouched, so the
 *               workspace of pkv_paged_attention_decode can serve when large enough
 * All other arguments as in pkv_paged_attention_decode (no partition_size).
 * Supported: dtype bfloat16/float16, head_dim 128, block_size 16, num_heads /
 * num_kv_heads <= 16 (PKV_E_UNSUPPORTED / PKV_E_HEADS otherwise). Errors: PKV_E_WORKSPACE for a missing or small workspace;
 * the common rules otherwise. With PKV_VALIDATE=1 the groups are also checked (cover
 * the batch in order, sizes and prefixes within their bounds, members' table entries
 * equal over the prefix): PKV_E_INDEX. Groups that break these rules without
 * PKV_VALIDATE give unspecified results but no access outside the arrays.
 * Caller contract: that of pkv_paged_attention_decode_append when appending.
 * Deterministic: the same inputs give bit-identical outputs.
 */
size_t pkv_paged_attention_grouped_workspace_size(int num_seqs, int num_heads,
                                                  int max_prefix_blocks);
int pkv_paged_attention_decode_grouped(void* out, const void* q, const void* new_k,
                                       const void* new_v, void* k_cache, void* v_cache,
                                       const int32_t* block_tables, const int32_t* context_lens,
                                       const int32_t* group_start, const int32_t* group_prefix,
                                       int num_groups, int max_group_size,
                                       int max_prefix_blocks, float scale, int num_seqs,
                                       int num_heads, int num_kv_heads, int head_dim,
                                       int block_size, int max_blocks_per_seq, int num_blocks,
                                       pkv_dtype dtype, void* workspace,
                                       size_t workspace_bytes, pkv_stream_t stream);

/* pkv_paged_attention_decode_grouped over 8-bit caches (scales and quantised append as
 * in pkv_paged_attention_decode_append_fp8). */
int pkv_paged_attention_decode_grouped_fp8(
    void* out, const void* q, const void* new_k, const void* new_v, void* k_cache,
    void* v_cache, float k_scale, float v_scale, const int32_t* block_tables,
    const int32_t* context_lens, const int32_t* group_start, const int32_t* group_prefix,
    int num_groups, int max_group_size, int max_prefix_blocks, float scale, int num_seqs,
    int num_heads, int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
    int num_blocks, pkv_dtype dtype, void* workspace, size_t workspace_bytes,
    pkv_stream_t stream);

/*
 * Host helper for the grouped decode: groups of consecutive sequences that share prefix
 * blocks, read from HOST copies of the block tables and context lengths (no device
 * work). A group is a maximal run of sequences whose first table entry is the same
 * non-negative block and that each hold at least one full block; its prefix is the
 * number of leading entries on which all members agree and that are full blocks
 * (context_lens / block_size, rounded down) of every member. Every other sequence is a
 * group of one with prefix 0.
 * block_tables [num_seqs, max_blocks_per_seq], context_lens [num_seqs]: host, read.
 * group_start  host, written: num_groups + 1 entries (room for num_seqs + 1).
 * group_prefix host, written: num_groups entries (room for num_seqs).
 * num_groups, max_group_size, max_prefix_blocks: written (0 for an empty batch).
 * Errors: PKV_E_SHAPE (negative sizes, block_size <= 0), PKV_E_NULL.
 */
int pkv_prefix_groups(const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                      int max_blocks_per_seq, int block_size, int32_t* group_start,
                      int32_t* group_prefix, int* num_groups, int* max_group_size,
                      int* max_prefix_blocks);

/* pkv_reshape_and_cache into 8-bit caches: key/value ([num_tokens, num_kv_heads,
 * head_dim] of dtype float32, bfloat16 or float16) are quantised as described above.
 * head_dim must be a multiple of 16 (PKV_E_UNSUPPORTED otherwise). Slots as in
 * pkv_reshape_and_cache. */
int pkv_reshape_and_cache_fp8(const void* key, const void* value, void* k_cache,
                              void* v_cache, const int64_t* slot_mapping, float k_scale,
                              float v_scale, int num_tokens, int num_kv_heads, int head_dim,
                              int block_size, int num_blocks, pkv_dtype dtype,
                              pkv_stream_t stream);

/*
 * Attention of several new query tokens per sequence: a prefill chunk, or draft tokens
 * verified in one pass. [P3] section "PagedAttention：逻辑连续，物理不必连续" states
 * that the query at position i attends tokens 1..i, read block by block through the
 * block table; [P2] section "vLLM 的发展里程碑" names chunked prefill and speculative
 * decoding, the two users of such a call.
 *
 * Sequence b owns query rows query_start[b] .. query_start[b+1]-1 (T_b rows). They are
 * the LAST T_b tokens of its context of n = context_lens[b] tokens, which already hold
 * their K and V (written by pkv_reshape_and_cache). Row query_start[b] + j sits at
 * position n - T_b + j and attends the first n - T_b + j + 1 tokens. A row whose
 * position is negative (T_b > n) attends nothing and gets a zero output.
 *
 * out, q        [num_query_tokens, num_heads, head_dim], dtype bfloat16 or float16;
 *               out written (only rows owned by a sequence), q read.
 * k_cache, v_cache, block_tables, context_lens, scale: as in pkv_paged_attention_decode.
 * query_start   int32 [num_seqs + 1] on the device: query_start[0] = 0, non-decreasing,
 *               query_start[num_seqs] = num_query_tokens.
 * max_query_len host value >= every T_b; sizes the launch (one workgroup per 16 / G
 *               query tokens, KV head and sequence, G = num_heads / num_kv_heads).
 * Supported: bfloat16/float16, head_dim 128, block_size 16, G <= 16
 * (PKV_E_UNSUPPORTED / PKV_E_HEADS otherwise); no workspace.
 * Errors: PKV_E_SHAPE for negative sizes, PKV_E_NULL for missing pointers. Under
 * PKV_VALIDATE=1 a query_start that breaks the rules above, or a T_b above
 * max_query_len, returns PKV_E_INDEX. Without it the kernel skips a sequence whose
 * query_start entries fall outside [0, num_query_tokens] or decrease, and rows past
 * max_query_len are not written.
 */
int pkv_paged_attention_chunk(void* out, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* block_tables,
                              const int32_t* context_lens, const int32_t* query_start,
                              float scale, int num_seqs, int num_query_tokens,
                              int max_query_len, int num_heads, int num_kv_heads, int head_dim,
                              int block_size, int max_blocks_per_seq, int num_blocks,
                              pkv_dtype dtype, pkv_stream_t stream);

/* pkv_paged_attention_chunk over 8-bit (E4M3) caches with their scales. */
int pkv_paged_attention_chunk_fp8(void* out, const void* q, const void* k_cache,
                                  const void* v_cache, float k_scale, float v_scale,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  const int32_t* query_start, float scale, int num_seqs,
                                  int num_query_tokens, int max_query_len, int num_heads,
                                  int num_kv_heads, int head_dim, int block_size,
                                  int max_blocks_per_seq, int num_blocks, pkv_dtype dtype,
                                  pkv_stream_t stream);

/*
 * Slot-mapped append of new tokens' K and V ([P3] section "Block table：为什么它能
 * 减少碎片": a decoded token goes into the free slot of its last block, or into a
 * newly taken block; section "Continuous batching 为什么离不开内存管理": generated
 * K/V are written back into their block).
 *
 * key, value    [num_tokens, num_kv_heads, head_dim] read
 * k_cache, v_cache [num_blocks, num_kv_heads, block_size, head_dim] written at the
 *               addressed slots only
 * slot_mapping  int64 [num_tokens]; slot = physical_block * block_size + offset;
 *               a negative slot skips the token. Two tokens with the same slot are a
 *               caller error (which one lands is unspecified).
 * The copy is bit-exact (no conversion). num_tokens may be 0 (nothing enqueued).
 */
int pkv_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                          const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                          int head_dim, int block_size, int num_blocks, pkv_dtype dtype,
                          pkv_stream_t stream);

/*
 * Whole-block copies inside one pool, as copy-on-write needs them ([P1] section 五:
 * a shared block is copied to a newly allocated one before a writer changes it;
 * [P3] section "共享前缀和 copy-on-write").
 *
 * cache         one pool of num_blocks blocks of block_bytes bytes each (call once
 *               for the K pool and once for the V pool)
 * src_dst_pairs int32 [num_pairs, 2] of (src, dst) block IDs. Destinations must be
 *               distinct and no destination may also be a source (caller contract);
 *               under that contract the result does not depend on the order.
 * block_bytes   a multiple of 4 (16 for the vectorised path); num_pairs may be 0.
 * Bit-exact.
 */
int pkv_copy_blocks(void* cache, const int32_t* src_dst_pairs, int num_pairs, int num_blocks,
                    size_t block_bytes, pkv_stream_t stream);

/*
 * Whole-block copies between two pools of the same block layout, for swapping blocks
 * between GPU memory and host memory ([P2] section "BlockAllocator 源码核心：vLLM 的
 * 显存管理心脏": the CPU/GPU two-tier allocator moves cold blocks to CPU memory when GPU
 * blocks run short and back when they are needed). Swap-out passes the GPU pool as
 * src_pool and the host pool as dst_pool; swap-in the reverse. Two device pools work
 * too.
 *
 * dst_pool, src_pool  num_dst_blocks / num_src_blocks blocks of block_bytes bytes. Each
 *               is device memory or PINNED host memory (hipHostMalloc, or a torch tensor
 *               made with pin_memory=True); the kernel reads and writes host memory
 *               directly through its device mapping, one launch for all pairs. Any other
 *               pointer (pageable host memory) returns PKV_E_UNSUPPORTED before anything
 *               is enqueued. Pools must not overlap.
 * src_dst_pairs int32 [num_pairs, 2] of (source block, destination block); device or
 *               pinned host memory. Destinations must be distinct (caller contract;
 *               checked under PKV_VALIDATE=1, like the ranges).
 * block_bytes   a multiple of 4 (16 for the vectorised path); num_pairs may be 0.
 * Bit-exact. Pairs with an index outside its pool are skipped.
 */
int pkv_swap_blocks(void* dst_pool, const void* src_pool, const int32_t* src_dst_pairs,
                    int num_pairs, int num_src_blocks, int num_dst_blocks, size_t block_bytes,
                    pkv_stream_t stream);

/*
 * Host block manager (plain host code, no device work): decides which physical block
 * and slot every token of every sequence uses, and produces the block tables, context
 * lengths, slot mappings and copy-on-write pairs the device calls take.
 *  - Token position p of a sequence lives in logical block p / bs at offset p % bs of
 *    its table ([P2] section "Block Table 数据结构"); slot = physical * bs + offset.
 *  - Free blocks form a stack: allocation pops, release pushes ([P2] section "内存分配
 *    与回收流程"). A new manager hands out order[0], order[1], ... (order NULL: 0, 1, ...).
 *  - Blocks are taken on demand: ceil(n / bs) for an n-token prompt, one more when a
 *    decoded token finds the last block full ([P3] section "Block table：为什么它能减少
 *    碎片"; [P1] section 六).
 *  - Reference counts; appending into a block shared with another sequence first
 *    copies it to a fresh block (copy-on-write) and reports the (src, dst) pair, which
 *    the caller copies on the device (pkv_copy_blocks) before writing the token
 *    ([P3] section "共享前缀和 copy-on-write"; [P1] section 五).
 *  - Prefix caching ([P2] section "Copy-on-Write 与 Prefix Caching"): full blocks of
 *    sequences added with token ids are cached under their whole token prefix (a
 *    64-bit chained key, confirmed on a hit by the block's own tokens and its parent's
 *    key); a prompt whose leading full blocks are cached references them.
 *  - A cached block nobody references stays cold; with no free block, allocation
 *    evicts the least recently released cold block ([P2] section "BlockAllocator
 *    源码核心：vLLM 的显存管理心脏"). Sequences release their blocks last first.
 *  - Each call checks that its blocks are available before changing anything and
 *    returns PKV_E_NOSPACE otherwise.
 * Not thread-safe; one manager per scheduler thread. Sequence ids are any int64.
 */
typedef struct pkv_block_manager pkv_block_manager;

/* A manager over num_blocks blocks of block_size tokens; order (NULL or a permutation
 * of 0..num_blocks-1) is the hand-out order of the initial free list. NULL on bad
 * arguments or out of memory. */
pkv_block_manager* pkv_bm_create(int num_blocks, int block_size, const int32_t* order);
void pkv_bm_destroy(pkv_block_manager* bm);

/* Free plus cold (evictable) blocks. */
int pkv_bm_available(const pkv_block_manager* bm);

/* 1 if a prompt of num_tokens tokens fits (ignoring prefix hits), else 0. */
int pkv_bm_can_allocate(const pkv_block_manager* bm, int num_tokens);

/* Place a new sequence's prompt of num_tokens tokens. token_ids (NULL: no prefix
 * caching for this sequence) are host int32 [num_tokens]; *cached_tokens (may be NULL)
 * receives the number of prompt tokens whose blocks were found in the cache (their
 * K/V need not be computed again). */
int pkv_bm_add_sequence(pkv_block_manager* bm, int64_t seq_id, int num_tokens,
                        const int32_t* token_ids, int* cached_tokens);

/* child_id shares every block of parent_id (parallel sampling, beam search). */
int pkv_bm_fork(pkv_block_manager* bm, int64_t parent_id, int64_t child_id);

/* Place the next token of seq_id: *slot receives its slot; *copy_src / *copy_dst the
 * copy-on-write pair, or -1 / -1. token_id feeds the prefix cache of tracked
 * sequences. */
int pkv_bm_append_token(pkv_block_manager* bm, int64_t seq_id, int32_t token_id,
                        int64_t* slot, int32_t* copy_src, int32_t* copy_dst);

/* One decode step of a batch: pkv_bm_append_token for seq_ids[0..n-1] in order
 * (token_ids may be NULL). slots int64 [n]; copy_pairs int32 [n, 2] (may be NULL),
 * (-1, -1) where no copy is needed. Returns how many sequences were placed: n, or
 * fewer when blocks ran out (the rest are untouched), or a negative error. */
int pkv_bm_append_tokens(pkv_block_manager* bm, const int64_t* seq_ids,
                         const int32_t* token_ids, int n, int64_t* slots,
                         int32_t* copy_pairs);

/* Release a finished sequence's blocks. */
int pkv_bm_free_sequence(pkv_block_manager* bm, int64_t seq_id);

/* Tokens placed for seq_id, or a negative error. */
int64_t pkv_bm_num_tokens(const pkv_block_manager* bm, int64_t seq_id);

/* The block table of seq_id: writes min(count, capacity) entries to out (may be NULL)
 * and returns count, or a negative error. */
int pkv_bm_block_table(const pkv_block_manager* bm, int64_t seq_id, int32_t* out,
                       int capacity);

/* Reference count of a block (0 for free and cold blocks). */
int pkv_bm_refcount(const pkv_block_manager* bm, int32_t block);

/* Block tables of seq_ids as host int32 rows of `width` entries padded with -1, and
 * their context lengths (host int32 [num_seqs]): the block_tables / context_lens
 * arguments of the attention calls. PKV_E_SHAPE if a table is wider than width;
 * nothing is written on error. */
int pkv_bm_build_tables(const pkv_block_manager* bm, const int64_t* seq_ids, int num_seqs,
                        int width, int32_t* tables, int32_t* context_lens);

/*
 * Device-bandwidth probe (diagnostic; not part of the attention path). Reads num_tiles
 * tiles of tile_bytes bytes, tile i starting at byte offsets[i] of base, each read once
 * with the non-temporal hint the decode kernels use for K and V, and computes nothing
 * from them. Timing it on the tiles a decode call reads gives the gather bandwidth the
 * device reaches for the decode's access pattern (whole 2 or 4 KiB tiles at scattered
 * addresses): [P3] section "它没有解决什么" notes that paging leaves attention bound by
 * memory bandwidth, and this is that bound as measured, next to the HBM peak.
 *
 * base        device memory of base_bytes bytes; a tile that does not lie wholly inside
 *             it, or whose offset is negative or not a multiple of 16, is skipped
 * offsets     device int64 [num_tiles], byte offsets into base
 * tile_bytes  2048 or 4096
 * workgroups  1..65535 workgroups of four waves; wave w reads tiles w, w + W, ... (W the
 *             number of waves)
 * tiles_in_flight  1, 2 or 4 tiles whose loads one wave issues before using any
 * sink        device uint32 [workgroups * 256]: written only in the (practically
 *             impossible) case that a wave's XOR of its data equals a fixed word, which
 *             keeps the loads from being optimised away
 * Errors: PKV_E_SHAPE, PKV_E_UNSUPPORTED, PKV_E_NULL, PKV_E_LAUNCH; nothing is enqueued
 * on error.
 */
int pkv_read_tiles(const void* base, size_t base_bytes, const int64_t* offsets, int num_tiles,
                   int tile_bytes, int workgroups, int tiles_in_flight, uint32_t* sink,
                   pkv_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */

// Internal launch entry points (host functions that enqueue kernels). Each returns 0
// on success or -1 if the HIP runtime rejected a launch.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

#include "plan.h"

namespace pkv {

int launch_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                             const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                             int head_dim, int block_size, int num_blocks, int elt_bytes,
                             hipStream_t stream);

int launch_copy_blocks(void* cache, const int32_t* pairs, int num_pairs, int num_blocks,
                       size_t block_bytes, hipStream_t stream);

// Whole-block copies between two pools of one block layout; dst and src are addresses
// the device can dereference (device memory, or pinned host memory's device mapping).
int launch_swap_blocks(void* dst, const void* src, const int32_t* pairs, int num_pairs,
                       int num_src_blocks, int num_dst_blocks, size_t block_bytes,
                       hipStream_t stream);

int launch_zero(void* p, size_t bytes, hipStream_t stream);

// Gather-bandwidth probe: reads num_tiles tiles of tile_bytes (2048 or 4096) bytes at
// base + offsets[i], with `workgroups` workgroups of four waves and `unroll` (1, 2, 4)
// tiles in flight per wave; tiles outside [0, base_bytes) are skipped.
int launch_read_tiles(const void* base, size_t base_bytes, const int64_t* offsets,
                      int num_tiles, int tile_bytes, int workgroups, int unroll, uint32_t* sink,
                      hipStream_t stream);

struct DecodeArgs {
    void* out;
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;
    const int32_t* context_lens;
    float scale;
    DecodeShape shape;
    void* workspace;
    // Fused append (both NULL for a plain decode): new K/V rows [num_seqs, Hkv, D]
    // written at each sequence's last context position before it is attended.
    const void* new_k = nullptr;
    const void* new_v = nullptr;
    // 8-bit caches (OCP FP8 E4M3 codes): key = code value * k_scale, value = code value
    // * v_scale; q, out and appended rows keep the 16-bit dtype of `shape`.
    int kv_fp8 = 0;
    float k_scale = 1.f;
    float v_scale = 1.f;
};

// Slot-mapped append into 8-bit caches: each element of key/value (elt_bytes 2 or 4,
// dtype bf16/f16/f32) becomes the E4M3 code of float(x) * inv_scale.
int launch_reshape_and_cache_fp8(const void* key, const void* value, void* k_cache,
                                 void* v_cache, const int64_t* slot_mapping, int num_tokens,
                                 int num_kv_heads, int head_dim, int block_size,
                                 int num_blocks, int src_dtype, float k_inv, float v_inv,
                                 hipStream_t stream);

// The append half of a fused decode step as its own kernel (paths whose decode kernel
// does not fuse it): new_k/new_v[b] go to position context_lens[b] - 1 of sequence b.
int launch_append_at_context_end(const DecodeArgs& a, hipStream_t stream);

// VALU kernel over fixed partitions (+ reduction when a context spans several).
int launch_decode_generic(const DecodeArgs& a, const DecodePlan& plan, hipStream_t stream);

// Log-sum-exp merge of per-partition partial results (shared by the fixed-partition
// paths).
int launch_partition_reduce(const DecodeArgs& a, const DecodePlan& plan, hipStream_t stream);

// Several query tokens per sequence, causal within each sequence's chunk: rows
// query_start[b] .. query_start[b+1]-1 of q/out ([num_query_tokens, num_heads,
// head_dim]) are the last tokens of sequence b's context.
struct ChunkArgs {
    void* out;
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_tables;
    const int32_t* context_lens;
    const int32_t* query_start;
    float scale;
    int num_seqs, num_query_tokens, max_query_len;
    int num_heads, num_kv_heads, head_dim, block_size, max_blocks, num_blocks, dtype;
    int kv_fp8 = 0;
    float k_scale = 1.f;
    float v_scale = 1.f;
};

// Matrix-core chunk kernel (bfloat16/float16 queries, head_dim 128, block_size 16,
// group <= 16).
int launch_chunk_mfma(const ChunkArgs& a, hipStream_t stream);

// Grouped decode: sequences group_start[i] .. group_start[i+1]-1 share their first
// group_prefix[i] (<= max_prefix) table entries; groups cover the batch in order.
struct GroupArgs {
    const int32_t* group_start;    // [num_groups + 1], device
    const int32_t* group_prefix;   // [num_groups], device
    int num_groups, max_group_size, max_prefix;
};

// Matrix-core grouped decode (each shared prefix block read once per tile of a group's
// members, then the members' own blocks); the workspace is laid out by plan_grouped.
int launch_decode_grouped(const DecodeArgs& a, const GroupArgs& ga, const GroupPlan& gp,
                          hipStream_t stream);

// Matrix-core kernels (bfloat16/float16, block_size 16).
int launch_decode_mfma(const DecodeArgs& a, const DecodePlan& plan, int num_cus,
                       hipStream_t stream);

}  // namespace pkv

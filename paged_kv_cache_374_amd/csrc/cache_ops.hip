// Cache companions of paged decode attention: slot-mapped append (into 16/32-bit
// caches, or quantising into 8-bit ones), the decode step's append at each context end
// (for paths whose decode kernel does not fuse it) and block copy.
//
// Both are pure data movement. Each thread moves one 16-byte (or 4-byte) chunk per
// loop trip; consecutive threads take consecutive chunks of a row, so a wavefront's
// stores cover contiguous runs of a KV row. Bounds are checked per chunk so that
// no index array content can push an access outside the pools.
#include "device_common.h"
#include "launchers.h"
#include "pagedkv.h"

namespace pkv {

namespace {

// key/value [T, Hkv, D]; caches [num_blocks, Hkv, bs, D]; rows of row_chunks chunks.
template <typename Chunk>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const Chunk* __restrict__ key, const Chunk* __restrict__ value, Chunk* __restrict__ k_cache,
    Chunk* __restrict__ v_cache, const int64_t* __restrict__ slot_mapping, int num_tokens,
    int num_kv_heads, int row_chunks, int block_size, int num_blocks) {
    const int64_t per_token = (int64_t)num_kv_heads * row_chunks;
    const int64_t total = (int64_t)num_tokens * per_token;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = i / per_token;
        const int64_t rem = i - t * per_token;          // h * row_chunks + c
        const int64_t slot = slot_mapping[t];
        if (slot < 0) continue;
        const int64_t blk = slot / block_size;
        if (blk >= num_blocks) continue;
        const int64_t off = slot - blk * block_size;
        const int64_t h = rem / row_chunks;
        const int64_t c = rem - h * row_chunks;
        const int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * row_chunks + c;
        k_cache[dst] = key[i];
        v_cache[dst] = value[i];
    }
}

// Slot-mapped append into 8-bit caches: each thread takes 16 consecutive elements of a
// K or V row (bf16/f16/f32 source S) and stores their 16 E4M3 codes with one 16-byte
// store: code = E4M3(float(x) * inv_scale), nearest-even, saturating at 448.
template <typename S>
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(
    const S* __restrict__ key, const S* __restrict__ value, uint8_t* __restrict__ k_cache,
    uint8_t* __restrict__ v_cache, const int64_t* __restrict__ slot_mapping, int num_tokens,
    int num_kv_heads, int head_dim, int block_size, int num_blocks, float k_inv, float v_inv) {
    constexpr int kPer = Vec16<S>::N;            // source elements per 16-byte load
    const int chunks = head_dim / 16;
    const int64_t per_token = (int64_t)num_kv_heads * chunks;
    const int64_t total = (int64_t)num_tokens * per_token;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = i / per_token;
        const int64_t rem = i - t * per_token;   // h * chunks + c
        const int64_t slot = slot_mapping[t];
        if (slot < 0) continue;
        const int64_t blk = slot / block_size;
        if (blk >= num_blocks) continue;
        const int64_t off = slot - blk * block_size;
        const int64_t h = rem / chunks;
        const int64_t c = rem - h * chunks;
        const int64_t src = (t * num_kv_heads + h) * head_dim + 16 * c;
        const int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * head_dim + 16 * c;
#pragma unroll
        for (int kind = 0; kind < 2; ++kind) {
            const uint4* sp = reinterpret_cast<const uint4*>((kind ? value : key) + src);
            const float inv = kind ? v_inv : k_inv;
            float f[16];
#pragma unroll
            for (int k = 0; k < 16 / kPer; ++k) Vec16<S>::unpack(sp[k], f + k * kPer);
            uint32_t w[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                w[k] = fp8_e4m3_code(f[4 * k] * inv) | fp8_e4m3_code(f[4 * k + 1] * inv) << 8 |
                       fp8_e4m3_code(f[4 * k + 2] * inv) << 16 |
                       fp8_e4m3_code(f[4 * k + 3] * inv) << 24;
            *reinterpret_cast<uint4*>((kind ? v_cache : k_cache) + dst) =
                make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
}

// The append of a decode step with slots taken from the block tables: row (b, h) of
// key/value goes to position context_lens[b] - 1 of sequence b, i.e. physical block
// tables[b][(n - 1) / block_size] at offset (n - 1) % block_size. Empty contexts and
// out-of-range table entries write nothing.
template <typename Chunk>
__global__ __launch_bounds__(256) void append_at_context_end_kernel(
    const Chunk* __restrict__ key, const Chunk* __restrict__ value, Chunk* __restrict__ k_cache,
    Chunk* __restrict__ v_cache, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ ctx_lens, int num_seqs, int num_kv_heads, int row_chunks,
    int block_size, int max_blocks, int num_blocks) {
    const int64_t per_seq = (int64_t)num_kv_heads * row_chunks;
    const int64_t total = (int64_t)num_seqs * per_seq;
    const int64_t cap = (int64_t)max_blocks * block_size;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t b = i / per_seq;
        int64_t n = ctx_lens[b];
        n = n > cap ? cap : n;
        if (n <= 0) continue;
        const int64_t j = (n - 1) / block_size;
        const int64_t blk = tables[b * max_blocks + j];
        if (blk < 0 || blk >= num_blocks) continue;
        const int64_t rem = i - b * per_seq;            // h * row_chunks + c
        const int64_t h = rem / row_chunks;
        const int64_t c = rem - h * row_chunks;
        const int64_t off = (n - 1) - j * block_size;
        const int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * row_chunks + c;
        k_cache[dst] = key[i];
        v_cache[dst] = value[i];
    }
}

// One block pair per grid row; threads stride over the block's chunks.
template <typename Chunk>
__global__ __launch_bounds__(256) void copy_blocks_kernel(Chunk* __restrict__ cache,
                                                          const int32_t* __restrict__ pairs,
                                                          int num_pairs, int num_blocks,
                                                          int64_t block_chunks) {
    for (int pi = blockIdx.y; pi < num_pairs; pi += gridDim.y) {
        const int src = pairs[2 * pi];
        const int dst = pairs[2 * pi + 1];
        if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) continue;
        const Chunk* s = cache + (int64_t)src * block_chunks;
        Chunk* d = cache + (int64_t)dst * block_chunks;
        for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < block_chunks;
             c += (int64_t)gridDim.x * blockDim.x)
            d[c] = s[c];
    }
}

// Whole-block copies from one pool to another of the same block layout: a device pool
// and a pinned host pool mapped into the device's address space, in either direction,
// or two device pools ([P2] section "BlockAllocator 源码核心：vLLM 的显存管理心脏": the
// CPU/GPU two-tier allocator moves cold blocks to host memory and back). One block pair
// per grid row. Each thread issues U loads before its U stores, so every wave keeps
// U KiB in flight: reads of host memory cross the host link with microsecond latency.
template <typename Chunk, int U>
__global__ __launch_bounds__(256) void swap_blocks_kernel(Chunk* __restrict__ dst,
                                                          const Chunk* __restrict__ src,
                                                          const int32_t* __restrict__ pairs,
                                                          int num_pairs, int num_src,
                                                          int num_dst, int64_t block_chunks) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int pi = blockIdx.y; pi < num_pairs; pi += gridDim.y) {
        const int from = pairs[2 * pi];
        const int to = pairs[2 * pi + 1];
        if (from < 0 || from >= num_src || to < 0 || to >= num_dst) continue;
        const Chunk* s = src + (int64_t)from * block_chunks;
        Chunk* d = dst + (int64_t)to * block_chunks;
        for (int64_t c0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c0 < block_chunks;
             c0 += stride * U) {
            Chunk v[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (c0 + u * stride < block_chunks) v[u] = s[c0 + u * stride];
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (c0 + u * stride < block_chunks) d[c0 + u * stride] = v[u];
        }
    }
}

int grid_for(int64_t items, int threads, int cap) {
    int64_t g = (items + threads - 1) / threads;
    if (g < 1) g = 1;
    return (int)(g > cap ? cap : g);
}

}  // namespace

int launch_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                             const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                             int head_dim, int block_size, int num_blocks, int elt_bytes,
                             hipStream_t stream) {
    const int row_bytes = head_dim * elt_bytes;
    const int64_t rows = (int64_t)num_tokens * num_kv_heads;
    if (row_bytes % 16 == 0) {
        const int rc = row_bytes / 16;
        hipLaunchKernelGGL(reshape_and_cache_kernel<uint4>, dim3(grid_for(rows * rc, 256, 65536)),
                           dim3(256), 0, stream, (const uint4*)key, (const uint4*)value,
                           (uint4*)k_cache, (uint4*)v_cache, slot_mapping, num_tokens,
                           num_kv_heads, rc, block_size, num_blocks);
    } else {
        const int rc = row_bytes / 4;
        hipLaunchKernelGGL(reshape_and_cache_kernel<uint32_t>,
                           dim3(grid_for(rows * rc, 256, 65536)), dim3(256), 0, stream,
                           (const uint32_t*)key, (const uint32_t*)value, (uint32_t*)k_cache,
                           (uint32_t*)v_cache, slot_mapping, num_tokens, num_kv_heads, rc,
                           block_size, num_blocks);
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_reshape_and_cache_fp8(const void* key, const void* value, void* k_cache,
                                 void* v_cache, const int64_t* slot_mapping, int num_tokens,
                                 int num_kv_heads, int head_dim, int block_size,
                                 int num_blocks, int src_dtype, float k_inv, float v_inv,
                                 hipStream_t stream) {
    const int64_t items = (int64_t)num_tokens * num_kv_heads * (head_dim / 16);
    const dim3 grid(grid_for(items, 256, 65536)), block(256);
    switch (src_dtype) {
        case PKV_FLOAT32:
            hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<float>, grid, block, 0, stream,
                               (const float*)key, (const float*)value, (uint8_t*)k_cache,
                               (uint8_t*)v_cache, slot_mapping, num_tokens, num_kv_heads,
                               head_dim, block_size, num_blocks, k_inv, v_inv);
            break;
        case PKV_BFLOAT16:
            hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<bf16_t>, grid, block, 0, stream,
                               (const bf16_t*)key, (const bf16_t*)value, (uint8_t*)k_cache,
                               (uint8_t*)v_cache, slot_mapping, num_tokens, num_kv_heads,
                               head_dim, block_size, num_blocks, k_inv, v_inv);
            break;
        case PKV_FLOAT16:
            hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<f16_t>, grid, block, 0, stream,
                               (const f16_t*)key, (const f16_t*)value, (uint8_t*)k_cache,
                               (uint8_t*)v_cache, slot_mapping, num_tokens, num_kv_heads,
                               head_dim, block_size, num_blocks, k_inv, v_inv);
            break;
        default:
            return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_append_at_context_end(const DecodeArgs& a, hipStream_t stream) {
    const DecodeShape& s = a.shape;
    const int elt = s.dtype == PKV_FLOAT32 ? 4 : 2;
    const int row_bytes = s.head_dim * elt;
    const int64_t rows = (int64_t)s.num_seqs * s.num_kv_heads;
    if (rows == 0 || s.max_blocks == 0) return 0;
    if (row_bytes % 16 == 0) {
        const int rc = row_bytes / 16;
        hipLaunchKernelGGL(append_at_context_end_kernel<uint4>,
                           dim3(grid_for(rows * rc, 256, 65536)), dim3(256), 0, stream,
                           (const uint4*)a.new_k, (const uint4*)a.new_v, (uint4*)a.k_cache,
                           (uint4*)a.v_cache, a.block_tables, a.context_lens, s.num_seqs,
                           s.num_kv_heads, rc, s.block_size, s.max_blocks, s.num_blocks);
    } else {
        const int rc = row_bytes / 4;
        hipLaunchKernelGGL(append_at_context_end_kernel<uint32_t>,
                           dim3(grid_for(rows * rc, 256, 65536)), dim3(256), 0, stream,
                           (const uint32_t*)a.new_k, (const uint32_t*)a.new_v,
                           (uint32_t*)a.k_cache, (uint32_t*)a.v_cache, a.block_tables,
                           a.context_lens, s.num_seqs, s.num_kv_heads, rc, s.block_size,
                           s.max_blocks, s.num_blocks);
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_copy_blocks(void* cache, const int32_t* pairs, int num_pairs, int num_blocks,
                       size_t block_bytes, hipStream_t stream) {
    const int gy = num_pairs > 65535 ? 65535 : num_pairs;
    if (block_bytes % 16 == 0) {
        const int64_t chunks = (int64_t)(block_bytes / 16);
        hipLaunchKernelGGL(copy_blocks_kernel<uint4>, dim3(grid_for(chunks, 256, 64), gy),
                           dim3(256), 0, stream, (uint4*)cache, pairs, num_pairs, num_blocks,
                           chunks);
    } else {
        const int64_t chunks = (int64_t)(block_bytes / 4);
        hipLaunchKernelGGL(copy_blocks_kernel<uint32_t>, dim3(grid_for(chunks, 256, 64), gy),
                           dim3(256), 0, stream, (uint32_t*)cache, pairs, num_pairs, num_blocks,
                           chunks);
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_swap_blocks(void* dst, const void* src, const int32_t* pairs, int num_pairs,
                       int num_src_blocks, int num_dst_blocks, size_t block_bytes,
                       hipStream_t stream) {
    constexpr int U = 8;
    const int gy = num_pairs > 65535 ? 65535 : num_pairs;
    if (block_bytes % 16 == 0) {
        const int64_t chunks = (int64_t)(block_bytes / 16);
        hipLaunchKernelGGL((swap_blocks_kernel<uint4, U>), dim3(grid_for(chunks, 256 * U, 64), gy),
                           dim3(256), 0, stream, (uint4*)dst, (const uint4*)src, pairs,
                           num_pairs, num_src_blocks, num_dst_blocks, chunks);
    } else {
        const int64_t chunks = (int64_t)(block_bytes / 4);
        hipLaunchKernelGGL((swap_blocks_kernel<uint32_t, U>),
                           dim3(grid_for(chunks, 256 * U, 64), gy), dim3(256), 0, stream,
                           (uint32_t*)dst, (const uint32_t*)src, pairs, num_pairs,
                           num_src_blocks, num_dst_blocks, chunks);
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Zero-fill with a kernel (graph-capture friendly: no memset node).
__global__ __launch_bounds__(256) void zero_kernel(uint32_t* __restrict__ p, int64_t words) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

int launch_zero(void* p, size_t bytes, hipStream_t stream) {
    const int64_t words = (int64_t)(bytes / 4);
    if (words == 0) return 0;
    hipLaunchKernelGGL(zero_kernel, dim3(grid_for(words, 256, 4096)), dim3(256), 0, stream,
                       (uint32_t*)p, words);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace pkv

// C ABI of the paged KV-cache library: argument checks, optional index validation,
// path selection and kernel launches. See include/pagedkv.h for the contract.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <mutex>
#include <vector>

#include "launchers.h"
#include "pagedkv.h"
#include "plan.h"

namespace {

bool validate_enabled() {
    static const int on = [] {
        const char* e = std::getenv("PKV_VALIDATE");
        return (e && e[0] == '1') ? 1 : 0;
    }();
    return on != 0;
}

// Compute units of the current device (cached per device ordinal).
int current_device_cus() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    if (dev >= 0 && dev < 64 && cache[dev] > 0) return cache[dev];
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return -1;
    if (dev >= 0 && dev < 64) cache[dev] = n;
    return n;
}

template <typename T>
bool fetch(std::vector<T>& host, const T* dev, size_t n, hipStream_t stream) {
    host.resize(n);
    if (n == 0) return true;
    if (hipMemcpyAsync(host.data(), dev, n * sizeof(T), hipMemcpyDeviceToHost, stream) !=
        hipSuccess)
        return false;
    return hipStreamSynchronize(stream) == hipSuccess;
}

// The address at which the current device reaches `p`: p itself for device memory, the
// device mapping for pinned host memory. nullptr for memory the device cannot reach
// (pageable host memory, unknown pointers); the failed query's error is cleared so a
// later launch check does not see it.
const void* device_view(const void* p) {
    hipPointerAttribute_t attr{};
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    if (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged) return p;
    if (attr.type == hipMemoryTypeHost && attr.devicePointer) {
        if (!attr.hostPointer) return attr.devicePointer;
        return (const char*)attr.devicePointer + ((const char*)p - (const char*)attr.hostPointer);
    }
    return nullptr;
}

// A cache scale must be a positive, finite binary32 value.
bool scale_ok(float s) { return s > 0.f && s <= 3.4028235e38f; }

int validate_tables(const pkv::DecodeShape& s, const int32_t* tables, const int32_t* ctx,
                    hipStream_t stream) {
    std::vector<int32_t> ht, hc;
    if (!fetch(hc, ctx, (size_t)s.num_seqs, stream) ||
        !fetch(ht, tables, (size_t)s.num_seqs * s.max_blocks, stream))
        return PKV_E_LAUNCH;
    for (int b = 0; b < s.num_seqs; ++b) {
        const long long n = hc[b];
        if (n < 0 || n > (long long)s.max_blocks * s.block_size) return PKV_E_INDEX;
        const long long nb = (n + s.block_size - 1) / s.block_size;
        for (long long j = 0; j < nb; ++j) {
            const int32_t p = ht[(size_t)b * s.max_blocks + j];
            if (p < 0 || p >= s.num_blocks) return PKV_E_INDEX;
        }
    }
    return PKV_OK;
}

// Scratch of pkv_paged_attention_decode_noalloc: one copy per device, zero at load.
// Host code never names it directly (on the host the name is only a stand-in); it
// uses the device address that hipGetSymbolAddress reports for the current device.
static __device__ __align__(256) uint8_t scratch[PKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's `scratch`, found once per device. On that
// first call the counter region is cleared on `stream` with a fill kernel (the array
// is zero at load already; every decode leaves its counters zeroed again).
int noalloc_scratch(hipStream_t stream, void** ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return PKV_E_DEVICE;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return PKV_E_LAUNCH;
        }
        if (pkv::launch_zero(p, pkv::kCounterBytes, stream) != 0) return PKV_E_LAUNCH;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return PKV_OK;
}

}  // namespace

extern "C" {

const char* pkv_version(void) { return "pagedkv 0.1.0 (gfx950)"; }

const char* pkv_strerror(int code) {
    switch (code) {
        case PKV_OK: return "success";
        case PKV_E_NULL: return "a required pointer is NULL";
        case PKV_E_SHAPE: return "invalid or inconsistent sizes";
        case PKV_E_HEADS: return "num_heads must be a multiple of num_kv_heads within the supported group size";
        case PKV_E_UNSUPPORTED: return "unsupported dtype / head_dim / block_size";
        case PKV_E_WORKSPACE: return "workspace missing or too small";
        case PKV_E_LAUNCH: return "the HIP runtime rejected a launch or copy";
        case PKV_E_INDEX: return "an index array holds an out-of-range entry (PKV_VALIDATE)";
        case PKV_E_DEVICE: return "no current HIP device";
        case PKV_E_NOSPACE: return "no free or evictable block for the request";
        case PKV_E_SEQUENCE: return "unknown sequence id, or the id is already in use";
        case PKV_E_SCRATCH: return "the call needs more scratch than the library's fixed array (PKV_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown pagedkv error";
    }
}

int pkv_workspace_init(void* workspace, size_t workspace_bytes, pkv_stream_t stream) {
    if (workspace_bytes == 0) return PKV_OK;
    if (!workspace) return PKV_E_NULL;
    return pkv::launch_zero(workspace, workspace_bytes, (hipStream_t)stream) == 0 ? PKV_OK
                                                                              : PKV_E_LAUNCH;
}

}  // extern "C"

namespace {

// Shared by the plain and the fused (append + decode) entry points; new_k/new_v are
// NULL for the plain decode.
// kv_fp8: the caches hold E4M3 codes with scales k_scale / v_scale.
int decode_call(void* out, const void* q, const void* new_k, const void* new_v,
                const void* k_cache, const void* v_cache, int kv_fp8, float k_scale,
                float v_scale, const int32_t* block_tables, const int32_t* context_lens,
                float scale, int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                int block_size, int max_blocks_per_seq, int num_blocks, pkv_dtype dtype,
                int partition_size, void* workspace, size_t workspace_bytes,
                pkv_stream_t stream) {
    pkv::DecodeShape s{num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                       max_blocks_per_seq, num_blocks, (int)dtype, partition_size};
    pkv::DecodePlan plan{};
    const int rc = pkv::plan_decode(s, &plan);
    if (rc != PKV_OK) return rc;
    // 8-bit caches run on the matrix-core kernels only
    if (kv_fp8 && plan.path == pkv::Path::Generic) return PKV_E_UNSUPPORTED;
    if (kv_fp8 && !(scale_ok(k_scale) && scale_ok(v_scale))) return PKV_E_SHAPE;
    if (num_seqs == 0) return PKV_OK;
    if (num_seqs > 65535) return PKV_E_SHAPE;
    if (!out || !q || !context_lens) return PKV_E_NULL;
    if (max_blocks_per_seq > 0 && (!k_cache || !v_cache || !block_tables)) return PKV_E_NULL;
    if (plan.bytes > 0 && (!workspace || workspace_bytes < plan.bytes)) return PKV_E_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    if (validate_enabled()) {
        const int v = validate_tables(s, block_tables, context_lens, st);
        if (v != PKV_OK) return v;
    }
    pkv::DecodeArgs a{out, q, k_cache, v_cache, block_tables, context_lens, scale, s, workspace};
    a.new_k = new_k;
    a.new_v = new_v;
    a.kv_fp8 = kv_fp8;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    int lr;
    if (plan.path == pkv::Path::Generic) {
        // the VALU kernel does not fuse the append: run it as its own kernel first
        lr = new_k ? pkv::launch_append_at_context_end(a, st) : 0;
        if (lr == 0) lr = pkv::launch_decode_generic(a, plan, st);
    } else {
        const int cus = current_device_cus();
        if (cus <= 0) return PKV_E_DEVICE;
        lr = pkv::launch_decode_mfma(a, plan, cus, st);
    }
    return lr == 0 ? PKV_OK : PKV_E_LAUNCH;
}

// Host check of a grouped decode's groups (PKV_VALIDATE=1): they cover the batch in
// order, no group exceeds max_group_size, every prefix lies in [0, max_prefix], and
// the members of a group hold the same table entries over its prefix.
int validate_groups(const pkv::DecodeShape& s, const int32_t* tables, const int32_t* start,
                    const int32_t* prefix, int num_groups, int max_group_size, int max_prefix,
                    hipStream_t stream) {
    std::vector<int32_t> hs, hp, ht;
    if (!fetch(hs, start, (size_t)num_groups + 1, stream) ||
        !fetch(hp, prefix, (size_t)num_groups, stream) ||
        !fetch(ht, tables, (size_t)s.num_seqs * s.max_blocks, stream))
        return PKV_E_LAUNCH;
    if (hs[0] != 0 || hs[num_groups] != s.num_seqs) return PKV_E_INDEX;
    for (int i = 0; i < num_groups; ++i) {
        const int a = hs[i], b = hs[i + 1], p = hp[i];
        if (b < a || b - a > max_group_size || p < 0 || p > max_prefix) return PKV_E_INDEX;
        for (int m = a + 1; m < b; ++m)
            for (int j = 0; j < p; ++j)
                if (ht[(size_t)m * s.max_blocks + j] != ht[(size_t)a * s.max_blocks + j])
                    return PKV_E_INDEX;
    }
    return PKV_OK;
}

// Shared by the 16-bit and 8-bit grouped decode entry points.
int grouped_call(void* out, const void* q, const void* new_k, const void* new_v,
                 const void* k_cache, const void* v_cache, int kv_fp8, float k_scale,
                 float v_scale, const int32_t* block_tables, const int32_t* context_lens,
                 const int32_t* group_start, const int32_t* group_prefix, int num_groups,
                 int max_group_size, int max_prefix_blocks, float scale, int num_seqs,
                 int num_heads, int num_kv_heads, int head_dim, int block_size,
                 int max_blocks_per_seq, int num_blocks, pkv_dtype dtype, void* workspace,
                 size_t workspace_bytes, pkv_stream_t stream) {
    pkv::DecodeShape s{num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                       max_blocks_per_seq, num_blocks, (int)dtype, 0};
    pkv::GroupPlan gp{};
    const int rc = pkv::plan_grouped(s, num_groups, max_group_size, max_prefix_blocks, &gp);
    if (rc != PKV_OK) return rc;
    if (kv_fp8 && !(scale_ok(k_scale) && scale_ok(v_scale))) return PKV_E_SHAPE;
    if ((new_k == nullptr) != (new_v == nullptr)) return PKV_E_NULL;
    if (num_seqs == 0) return PKV_OK;
    if (!out || !q || !context_lens || !group_start || !group_prefix) return PKV_E_NULL;
    if (max_blocks_per_seq > 0 && (!k_cache || !v_cache || !block_tables)) return PKV_E_NULL;
    if (gp.bytes > 0 && (!workspace || workspace_bytes < gp.bytes)) return PKV_E_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    if (validate_enabled()) {
        int v = validate_tables(s, block_tables, context_lens, st);
        if (v == PKV_OK)
            v = validate_groups(s, block_tables, group_start, group_prefix, num_groups,
                                max_group_size, max_prefix_blocks, st);
        if (v != PKV_OK) return v;
    }
    pkv::DecodeArgs a{out, q, k_cache, v_cache, block_tables, context_lens, scale, s, workspace};
    a.new_k = new_k;
    a.new_v = new_v;
    a.kv_fp8 = kv_fp8;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    const pkv::GroupArgs ga{group_start, group_prefix, num_groups, max_group_size,
                            max_prefix_blocks};
    return pkv::launch_decode_grouped(a, ga, gp, st) == 0 ? PKV_OK : PKV_E_LAUNCH;
}

// Shared by the 16-bit and 8-bit chunk entry points.
int chunk_call(void* out, const void* q, const void* k_cache, const void* v_cache, int kv_fp8,
               float k_scale, float v_scale, const int32_t* block_tables,
               const int32_t* context_lens, const int32_t* query_start, float scale,
               int num_seqs, int num_query_tokens, int max_query_len, int num_heads,
               int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
               int num_blocks, pkv_dtype dtype, pkv_stream_t stream) {
    if (num_seqs < 0 || num_query_tokens < 0 || max_query_len < 0 || num_heads <= 0 ||
        num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || max_blocks_per_seq < 0 ||
        num_blocks < 0)
        return PKV_E_SHAPE;
    if (num_heads % num_kv_heads != 0 || num_heads / num_kv_heads > pkv::kMaxGroup)
        return PKV_E_HEADS;
    // matrix-core kernel only: bfloat16/float16 queries, head_dim 128, block_size 16
    if (!pkv::mfma_eligible((int)dtype, head_dim, block_size, num_heads / num_kv_heads))
        return PKV_E_UNSUPPORTED;
    if (kv_fp8 && !(scale_ok(k_scale) && scale_ok(v_scale))) return PKV_E_SHAPE;
    if (num_seqs > 65535 || num_kv_heads > 65535) return PKV_E_SHAPE;
    if (num_seqs == 0 || num_query_tokens == 0 || max_query_len == 0) return PKV_OK;
    // byte offsets into q and out are 32-bit in the kernels
    if ((long long)num_query_tokens * num_heads * head_dim * 2 > 0x7fffffffLL) return PKV_E_SHAPE;
    if (!out || !q || !context_lens || !query_start) return PKV_E_NULL;
    if (max_blocks_per_seq > 0 && (!k_cache || !v_cache || !block_tables)) return PKV_E_NULL;
    hipStream_t st = (hipStream_t)stream;
    if (validate_enabled()) {
        pkv::DecodeShape s{num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                           max_blocks_per_seq, num_blocks, (int)dtype, 0};
        const int v = validate_tables(s, block_tables, context_lens, st);
        if (v != PKV_OK) return v;
        std::vector<int32_t> hq;
        if (!fetch(hq, query_start, (size_t)num_seqs + 1, st)) return PKV_E_LAUNCH;
        if (hq[0] != 0 || hq[num_seqs] != num_query_tokens) return PKV_E_INDEX;
        for (int b = 0; b < num_seqs; ++b)
            if (hq[b + 1] < hq[b] || hq[b + 1] - hq[b] > max_query_len) return PKV_E_INDEX;
    }
    pkv::ChunkArgs a{out, q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
                     num_seqs, num_query_tokens, max_query_len, num_heads, num_kv_heads,
                     head_dim, block_size, max_blocks_per_seq, num_blocks, (int)dtype};
    a.kv_fp8 = kv_fp8;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    return pkv::launch_chunk_mfma(a, st) == 0 ? PKV_OK : PKV_E_LAUNCH;
}

}  // namespace

extern "C" {

int pkv_paged_attention_decode(void* out, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_tables,
                               const int32_t* context_lens, float scale, int num_seqs,
                               int num_heads, int num_kv_heads, int head_dim, int block_size,
                               int max_blocks_per_seq, int num_blocks, pkv_dtype dtype,
                               int partition_size, void* workspace, size_t workspace_bytes,
                               pkv_stream_t stream) {
    return decode_call(out, q, nullptr, nullptr, k_cache, v_cache, 0, 1.f, 1.f, block_tables,
                       context_lens, scale, num_seqs, num_heads, num_kv_heads, head_dim,
                       block_size, max_blocks_per_seq, num_blocks, dtype, partition_size,
                       workspace, workspace_bytes, stream);
}

int pkv_paged_attention_decode_noalloc(void* out, const void* q, const void* k_cache,
                                       const void* v_cache, const int32_t* block_tables,
                                       const int32_t* context_lens, float scale, int num_seqs,
                                       int num_heads, int num_kv_heads, int head_dim,
                                       int block_size, int max_blocks_per_seq, int num_blocks,
                                       pkv_dtype dtype, int partition_size,
                                       pkv_stream_t stream) {
    pkv::DecodeShape s{num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                       max_blocks_per_seq, num_blocks, (int)dtype, partition_size};
    pkv::DecodePlan plan{};
    const int rc = pkv::plan_decode(s, &plan);
    if (rc != PKV_OK) return rc;
    if (plan.bytes > PKV_NOALLOC_SCRATCH_BYTES) return PKV_E_SCRATCH;
    void* ws = nullptr;
    if (plan.bytes > 0 && num_seqs > 0) {
        const int sr = noalloc_scratch((hipStream_t)stream, &ws);
        if (sr != PKV_OK) return sr;
    }
    return decode_call(out, q, nullptr, nullptr, k_cache, v_cache, 0, 1.f, 1.f, block_tables,
                       context_lens, scale, num_seqs, num_heads, num_kv_heads, head_dim,
                       block_size, max_blocks_per_seq, num_blocks, dtype, partition_size, ws,
                       ws ? PKV_NOALLOC_SCRATCH_BYTES : 0, stream);
}

int pkv_paged_attention_decode_append(void* out, const void* q, const void* new_k,
                                      const void* new_v, void* k_cache, void* v_cache,
                                      const int32_t* block_tables, const int32_t* context_lens,
                                      float scale, int num_seqs, int num_heads,
                                      int num_kv_heads, int head_dim, int block_size,
                                      int max_blocks_per_seq, int num_blocks, pkv_dtype dtype,
                                      int partition_size, void* workspace,
                                      size_t workspace_bytes, pkv_stream_t stream) {
    if (num_seqs > 0 && (!new_k || !new_v)) return PKV_E_NULL;
    return decode_call(out, q, new_k, new_v, k_cache, v_cache, 0, 1.f, 1.f, block_tables,
                       context_lens, scale, num_seqs, num_heads, num_kv_heads, head_dim,
                       block_size, max_blocks_per_seq, num_blocks, dtype, partition_size,
                       workspace, workspace_bytes, stream);
}

int pkv_paged_attention_decode_fp8(void* out, const void* q, const void* k_cache,
                                   const void* v_cache, float k_scale, float v_scale,
                                   const int32_t* block_tables, const int32_t* context_lens,
                                   float scale, int num_seqs, int num_heads, int num_kv_heads,
                                   int head_dim, int block_size, int max_blocks_per_seq,
                                   int num_blocks, pkv_dtype dtype, int partition_size,
                                   void* workspace, size_t workspace_bytes,
                                   pkv_stream_t stream) {
    return decode_call(out, q, nullptr, nullptr, k_cache, v_cache, 1, k_scale, v_scale,
                       block_tables, context_lens, scale, num_seqs, num_heads, num_kv_heads,
                       head_dim, block_size, max_blocks_per_seq, num_blocks, dtype,
                       partition_size, workspace, workspace_bytes, stream);
}

int pkv_paged_attention_decode_append_fp8(void* out, const void* q, const void* new_k,
                                          const void* new_v, void* k_cache, void* v_cache,
                                          float k_scale, float v_scale,
                                          const int32_t* block_tables,
                                          const int32_t* context_lens, float scale,
                                          int num_seqs, int num_heads, int num_kv_heads,
                                          int head_dim, int block_size, int max_blocks_per_seq,
                                          int num_blocks, pkv_dtype dtype, int partition_size,
                                          void* workspace, size_t workspace_bytes,
                                          pkv_stream_t stream) {
    if (num_seqs > 0 && (!new_k || !new_v)) return PKV_E_NULL;
    return decode_call(out, q, new_k, new_v, k_cache, v_cache, 1, k_scale, v_scale,
                       block_tables, context_lens, scale, num_seqs, num_heads, num_kv_heads,
                       head_dim, block_size, max_blocks_per_seq, num_blocks, dtype,
                       partition_size, workspace, workspace_bytes, stream);
}

int pkv_paged_attention_decode_grouped(void* out, const void* q, const void* new_k,
                                       const void* new_v, void* k_cache, void* v_cache,
                                       const int32_t* block_tables, const int32_t* context_lens,
                                       const int32_t* group_start, const int32_t* group_prefix,
                                       int num_groups, int max_group_size,
                                       int max_prefix_blocks, float scale, int num_seqs,
                                       int num_heads, int num_kv_heads, int head_dim,
                                       int block_size, int max_blocks_per_seq, int num_blocks,
                                       pkv_dtype dtype, void* workspace,
                                       size_t workspace_bytes, pkv_stream_t stream) {
    return grouped_call(out, q, new_k, new_v, k_cache, v_cache, 0, 1.f, 1.f, block_tables,
                        context_lens, group_start, group_prefix, num_groups, max_group_size,
                        max_prefix_blocks, scale, num_seqs, num_heads, num_kv_heads, head_dim,
                        block_size, max_blocks_per_seq, num_blocks, dtype, workspace,
                        workspace_bytes, stream);
}

int pkv_paged_attention_decode_grouped_fp8(
    void* out, const void* q, const void* new_k, const void* new_v, void* k_cache,
    void* v_cache, float k_scale, float v_scale, const int32_t* block_tables,
    const int32_t* context_lens, const int32_t* group_start, const int32_t* group_prefix,
    int num_groups, int max_group_size, int max_prefix_blocks, float scale, int num_seqs,
    int num_heads, int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
    int num_blocks, pkv_dtype dtype, void* workspace, size_t workspace_bytes,
    pkv_stream_t stream) {
    return grouped_call(out, q, new_k, new_v, k_cache, v_cache, 1, k_scale, v_scale,
                        block_tables, context_lens, group_start, group_prefix, num_groups,
                        max_group_size, max_prefix_blocks, scale, num_seqs, num_heads,
                        num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                        dtype, workspace, workspace_bytes, stream);
}

int pkv_paged_attention_chunk(void* out, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* block_tables,
                              const int32_t* context_lens, const int32_t* query_start,
                              float scale, int num_seqs, int num_query_tokens,
                              int max_query_len, int num_heads, int num_kv_heads, int head_dim,
                              int block_size, int max_blocks_per_seq, int num_blocks,
                              pkv_dtype dtype, pkv_stream_t stream) {
    return chunk_call(out, q, k_cache, v_cache, 0, 1.f, 1.f, block_tables, context_lens,
                      query_start, scale, num_seqs, num_query_tokens, max_query_len, num_heads,
                      num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, dtype,
                      stream);
}

int pkv_paged_attention_chunk_fp8(void* out, const void* q, const void* k_cache,
                                  const void* v_cache, float k_scale, float v_scale,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  const int32_t* query_start, float scale, int num_seqs,
                                  int num_query_tokens, int max_query_len, int num_heads,
                                  int num_kv_heads, int head_dim, int block_size,
                                  int max_blocks_per_seq, int num_blocks, pkv_dtype dtype,
                                  pkv_stream_t stream) {
    return chunk_call(out, q, k_cache, v_cache, 1, k_scale, v_scale, block_tables,
                      context_lens, query_start, scale, num_seqs, num_query_tokens,
                      max_query_len, num_heads, num_kv_heads, head_dim, block_size,
                      max_blocks_per_seq, num_blocks, dtype, stream);
}

int pkv_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                          const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                          int head_dim, int block_size, int num_blocks, pkv_dtype dtype,
                          pkv_stream_t stream) {
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        num_blocks < 0)
        return PKV_E_SHAPE;
    int elt;
    switch (dtype) {
        case PKV_FLOAT32: elt = 4; break;
        case PKV_BFLOAT16:
        case PKV_FLOAT16: elt = 2; break;
        default: return PKV_E_UNSUPPORTED;
    }
    if ((head_dim * elt) % 4 != 0) return PKV_E_UNSUPPORTED;
    if (num_tokens == 0) return PKV_OK;
    if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PKV_E_NULL;
    hipStream_t st = (hipStream_t)stream;
    if (validate_enabled()) {
        std::vector<int64_t> hs;
        if (!fetch(hs, slot_mapping, (size_t)num_tokens, st)) return PKV_E_LAUNCH;
        for (int64_t x : hs)
            if (x >= (int64_t)num_blocks * block_size) return PKV_E_INDEX;
    }
    return pkv::launch_reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, num_tokens,
                                         num_kv_heads, head_dim, block_size, num_blocks, elt,
                                         st) == 0
               ? PKV_OK
               : PKV_E_LAUNCH;
}

int pkv_reshape_and_cache_fp8(const void* key, const void* value, void* k_cache,
                              void* v_cache, const int64_t* slot_mapping, float k_scale,
                              float v_scale, int num_tokens, int num_kv_heads, int head_dim,
                              int block_size, int num_blocks, pkv_dtype dtype,
                              pkv_stream_t stream) {
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        num_blocks < 0 || !scale_ok(k_scale) || !scale_ok(v_scale))
        return PKV_E_SHAPE;
    if ((dtype != PKV_FLOAT32 && dtype != PKV_BFLOAT16 && dtype != PKV_FLOAT16) ||
        head_dim % 16 != 0)
        return PKV_E_UNSUPPORTED;
    if (num_tokens == 0) return PKV_OK;
    if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PKV_E_NULL;
    hipStream_t st = (hipStream_t)stream;
    if (validate_enabled()) {
        std::vector<int64_t> hs;
        if (!fetch(hs, slot_mapping, (size_t)num_tokens, st)) return PKV_E_LAUNCH;
        for (int64_t x : hs)
            if (x >= (int64_t)num_blocks * block_size) return PKV_E_INDEX;
    }
    return pkv::launch_reshape_and_cache_fp8(key, value, k_cache, v_cache, slot_mapping,
                                             num_tokens, num_kv_heads, head_dim, block_size,
                                             num_blocks, (int)dtype, 1.f / k_scale,
                                             1.f / v_scale, st) == 0
               ? PKV_OK
               : PKV_E_LAUNCH;
}

int pkv_copy_blocks(void* cache, const int32_t* src_dst_pairs, int num_pairs, int num_blocks,
                    size_t block_bytes, pkv_stream_t stream) {
    if (num_pairs < 0 || num_blocks < 0) return PKV_E_SHAPE;
    if (block_bytes % 4 != 0) return PKV_E_UNSUPPORTED;
    if (num_pairs == 0 || block_bytes == 0) return PKV_OK;
    if (!cache || !src_dst_pairs) return PKV_E_NULL;
    hipStream_t st = (hipStream_t)stream;
    if (validate_enabled()) {
        std::vector<int32_t> hp;
        if (!fetch(hp, src_dst_pairs, (size_t)num_pairs * 2, st)) return PKV_E_LAUNCH;
        std::vector<char> role((size_t)num_blocks, 0);   // 1 = source, 2 = destination
        for (int i = 0; i < num_pairs; ++i) {
            const int32_t a = hp[2 * i], b = hp[2 * i + 1];
            if (a < 0 || a >= num_blocks || b < 0 || b >= num_blocks) return PKV_E_INDEX;
            if (role[b] != 0 || role[a] == 2) return PKV_E_INDEX;
            role[a] = 1;
            role[b] = 2;
        }
    }
    return pkv::launch_copy_blocks(cache, src_dst_pairs, num_pairs, num_blocks, block_bytes,
                                   st) == 0
               ? PKV_OK
               : PKV_E_LAUNCH;
}

int pkv_read_tiles(const void* base, size_t base_bytes, const int64_t* offsets, int num_tiles,
                   int tile_bytes, int workgroups, int tiles_in_flight, uint32_t* sink,
                   pkv_stream_t stream) {
    if (num_tiles < 0 || workgroups < 1 || workgroups > 65535) return PKV_E_SHAPE;
    if ((tile_bytes != 2048 && tile_bytes != 4096) ||
        (tiles_in_flight != 1 && tiles_in_flight != 2 && tiles_in_flight != 4))
        return PKV_E_UNSUPPORTED;
    if (num_tiles == 0) return PKV_OK;
    if (!base || !offsets || !sink) return PKV_E_NULL;
    return pkv::launch_read_tiles(base, base_bytes, offsets, num_tiles, tile_bytes, workgroups,
                                  tiles_in_flight, sink, (hipStream_t)stream) == 0
               ? PKV_OK
               : PKV_E_LAUNCH;
}

int pkv_swap_blocks(void* dst_pool, const void* src_pool, const int32_t* src_dst_pairs,
                    int num_pairs, int num_src_blocks, int num_dst_blocks, size_t block_bytes,
                    pkv_stream_t stream) {
    if (num_pairs < 0 || num_src_blocks < 0 || num_dst_blocks < 0) return PKV_E_SHAPE;
    if (block_bytes % 4 != 0) return PKV_E_UNSUPPORTED;
    if (num_pairs == 0 || block_bytes == 0) return PKV_OK;
    if (!dst_pool || !src_pool || !src_dst_pairs) return PKV_E_NULL;
    // Both pools must be reachable from the device: device memory, or pinned host memory
    // through its device mapping. Anything else is refused before any launch.
    void* dst = const_cast<void*>(device_view(dst_pool));
    const void* src = device_view(src_pool);
    const int32_t* pairs = static_cast<const int32_t*>(device_view(src_dst_pairs));
    if (!dst || !src || !pairs) return PKV_E_UNSUPPORTED;
    hipStream_t st = (hipStream_t)stream;
    if (validate_enabled()) {
        std::vector<int32_t> hp;
        if (!fetch(hp, src_dst_pairs, (size_t)num_pairs * 2, st)) return PKV_E_LAUNCH;
        std::vector<char> seen((size_t)num_dst_blocks, 0);
        for (int i = 0; i < num_pairs; ++i) {
            const int32_t a = hp[2 * i], b = hp[2 * i + 1];
            if (a < 0 || a >= num_src_blocks || b < 0 || b >= num_dst_blocks || seen[b])
                return PKV_E_INDEX;
            seen[b] = 1;
        }
    }
    return pkv::launch_swap_blocks(dst, src, pairs, num_pairs, num_src_blocks,
                                   num_dst_blocks, block_bytes, st) == 0
               ? PKV_OK
               : PKV_E_LAUNCH;
}

}  // extern "C"

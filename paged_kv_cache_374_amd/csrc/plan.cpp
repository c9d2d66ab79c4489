// Host-side validation and launch planning for paged decode attention (no HIP calls).
#include "plan.h"

#include "pagedkv.h"

namespace pkv {

namespace {

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool head_dim_ok(int d) { return d == 64 || d == 128 || d == 256; }


bool block_size_ok(int bs) {
    return bs == 1 || bs == 2 || bs == 4 || bs == 8 || bs == 16 || bs == 32;
}

}  // namespace

bool mfma_eligible(int dtype, int head_dim, int block_size, int group) {
    return (dtype == PKV_BFLOAT16 || dtype == PKV_FLOAT16) && block_size == kMfmaBlockSize &&
           head_dim == kMfmaHeadDim && group >= 1 && group <= kMaxGroup;
}

int balanced_workers(const DecodeShape& s, int num_cus, int wg_per_cu) {
    if (num_cus <= 0 || wg_per_cu <= 0) return 0;
    const long long blocks = (long long)s.num_seqs * s.num_kv_heads * s.max_blocks;
    long long w = (long long)num_cus * wg_per_cu;
    const long long need = (blocks + kShareMax - 1) / kShareMax;
    if (need > w) w = need;
    w = (w + 7) / 8 * 8;
    return w > kMaxWorkers ? 0 : (int)w;
}

int plan_decode(const DecodeShape& s, DecodePlan* plan) {
    if (s.num_seqs < 0 || s.num_heads <= 0 || s.num_kv_heads <= 0 || s.head_dim <= 0 ||
        s.block_size <= 0 || s.max_blocks < 0 || s.num_blocks < 0 || s.partition_size < 0)
        return PKV_E_SHAPE;
    if (s.num_heads % s.num_kv_heads != 0) return PKV_E_HEADS;
    const int group = s.num_heads / s.num_kv_heads;
    if (group > kMaxGroup) return PKV_E_HEADS;
    if (s.dtype != PKV_FLOAT32 && s.dtype != PKV_BFLOAT16 && s.dtype != PKV_FLOAT16)
        return PKV_E_UNSUPPORTED;
    if (!head_dim_ok(s.head_dim) || !block_size_ok(s.block_size)) return PKV_E_UNSUPPORTED;
    if (s.partition_size > 0 && s.partition_size % s.block_size != 0) return PKV_E_SHAPE;
    const long long max_ctx = (long long)s.max_blocks * s.block_size;
    if (max_ctx > (1LL << 30)) return PKV_E_SHAPE;

    const bool mfma = mfma_eligible(s.dtype, s.head_dim, s.block_size, group);
    if (!mfma && group > kMaxGroupGeneric) return PKV_E_HEADS;

    DecodePlan p{};
    p.group = group;
    // The balanced path needs every sequence's length in LDS and at most kMaxWorkers
    // workgroups of at most kShareMax blocks each.
    const long long all_blocks = (long long)s.num_seqs * s.num_kv_heads * s.max_blocks;
    const bool fits = s.num_seqs <= kMaxSeqsBalanced &&
                      all_blocks <= (long long)kMaxWorkers * kShareMax &&
                      (size_t)s.num_seqs * s.num_kv_heads * sizeof(int32_t) <= kCounterBytes;
    // Automatic choice on the matrix-core path: one workgroup per (sequence, KV head),
    // long contexts paired with short ones on a CU, when there are enough units for two
    // per CU and no context can be longer than kPerUnitMaxBlocks blocks (which bounds
    // what one long unit can cost). It needs no workspace and no merges between
    // workgroups. Otherwise the balanced split, which evens out any length mix.
    const bool per_unit = mfma && s.partition_size == 0 && s.num_seqs <= kPerUnitMaxSeqs &&
                          (long long)s.num_seqs * s.num_kv_heads >= kPerUnitMinUnits &&
                          s.max_blocks <= kPerUnitMaxBlocks;
    if (per_unit) {
        p.path = Path::MfmaPartitioned;
        p.partition_tokens = s.max_blocks * s.block_size;
        p.max_partitions = 1;
        // pieces of long units: a counter per unit, records for every piece (at most
        // one per helper plus one per long unit), byte offsets within 32 bits
        const size_t rec = (size_t)balanced_slot_floats(mfma_gmax(group)) * sizeof(float);
        const size_t per_head = (size_t)kPerUnitMaxHelpers + (size_t)s.num_seqs;
        const size_t rec_bytes = (size_t)s.num_kv_heads * per_head * rec;
        if ((size_t)s.num_seqs * s.num_kv_heads * sizeof(int32_t) <= kCounterBytes &&
            rec_bytes <= 0x7fffffffULL) {
            p.helpers = kPerUnitMaxHelpers;
            p.rec_per_head = (int)per_head;
            p.off_counters = 0;
            p.off_partials = kCounterBytes;
            p.bytes = kCounterBytes + rec_bytes;
        }
    } else if (mfma && s.partition_size == 0 && fits) {
        p.path = Path::MfmaBalanced;
        p.max_workers = kMaxWorkers;
        const size_t slot = (size_t)balanced_slot_floats(mfma_gmax(group)) * sizeof(float);
        p.off_counters = 0;
        p.off_partials = kCounterBytes;
        p.bytes = p.off_partials + (size_t)2 * kMaxWorkers * slot;
        if (s.num_seqs == 0) p.bytes = 0;
    } else {
        p.path = mfma ? Path::MfmaPartitioned : Path::Generic;
        p.partition_tokens = s.partition_size > 0 ? s.partition_size : kDefaultPartition;
        // the matrix-core partition kernel stages one partition's blocks in LDS
        if (mfma && p.partition_tokens / s.block_size > kShareMax) p.path = Path::Generic;
        if (p.path == Path::Generic && group > kMaxGroupGeneric) return PKV_E_HEADS;
        p.max_partitions = (int)((max_ctx + p.partition_tokens - 1) / p.partition_tokens);
        if (p.max_partitions < 1) p.max_partitions = 1;
        if (p.max_partitions > 1 && s.num_seqs > 0) {
            const size_t rows = (size_t)s.num_seqs * s.num_heads * p.max_partitions;
            p.off_m = kCounterBytes;
            p.off_l = p.off_m + align_up(rows * sizeof(float), 256);
            p.off_o = p.off_l + align_up(rows * sizeof(float), 256);
            p.bytes = p.off_o + rows * s.head_dim * sizeof(float);
        }
    }
    *plan = p;
    return PKV_OK;
}

}  // namespace pkv

extern "C" size_t pkv_paged_attention_workspace_size(int num_seqs, int num_heads,
                                                     int num_kv_heads, int head_dim,
                                                     int block_size, int max_blocks_per_seq,
                                                     int partition_size) {
    // The dtype only matters for eligibility of the matrix-core path; size for the
    // larger of the two layouts so one workspace serves every dtype.
    size_t best = 0;
    for (int dtype : {PKV_FLOAT32, PKV_BFLOAT16}) {
        pkv::DecodeShape s{num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                           max_blocks_per_seq, 0, dtype, partition_size};
        pkv::DecodePlan p{};
        if (pkv::plan_decode(s, &p) == PKV_OK && p.bytes > best) best = p.bytes;
    }
    return best;
}

extern "C" int pkv_paged_attention_partials_layout(int num_seqs, int num_heads,
                                                   int num_kv_heads, int head_dim,
                                                   int block_size, int max_blocks_per_seq,
                                                   int partition_size, pkv_dtype dtype,
                                                   size_t offsets[3]) {
    if (!offsets) return PKV_E_NULL;
    pkv::DecodeShape s{num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                       max_blocks_per_seq, 0, (int)dtype, partition_size};
    pkv::DecodePlan p{};
    const int rc = pkv::plan_decode(s, &p);
    if (rc != PKV_OK) return rc;
    offsets[0] = offsets[1] = offsets[2] = 0;
    // only the fixed-partition paths keep per-partition records, and only when a
    // context can span more than one partition
    if (p.path == pkv::Path::MfmaBalanced || p.max_partitions <= 1 || p.bytes == 0) return 0;
    offsets[0] = p.off_m;
    offsets[1] = p.off_l;
    offsets[2] = p.off_o;
    return p.max_partitions;
}

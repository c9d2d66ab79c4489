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

int plan_grouped(const DecodeShape& s, int num_groups, int max_group_size, int max_prefix,
                 GroupPlan* plan) {
    if (s.num_seqs < 0 || s.num_heads <= 0 || s.num_kv_heads <= 0 || s.max_blocks < 0 ||
        s.num_blocks < 0 || num_groups < 0 || max_group_size < 0 || max_prefix < 0)
        return PKV_E_SHAPE;
    if (s.num_heads % s.num_kv_heads != 0) return PKV_E_HEADS;
    const int group = s.num_heads / s.num_kv_heads;
    if (group > kMaxGroup) return PKV_E_HEADS;
    if (!mfma_eligible(s.dtype, s.head_dim, s.block_size, group)) return PKV_E_UNSUPPORTED;
    if ((long long)s.max_blocks * s.block_size > (1LL << 30) || max_prefix > s.max_blocks)
        return PKV_E_SHAPE;
    if (s.num_seqs > 65535 || num_groups > 65535 || s.num_kv_heads > 65535) return PKV_E_SHAPE;
    // every sequence belongs to a group
    if (s.num_seqs > 0 && (num_groups == 0 || max_group_size == 0)) return PKV_E_SHAPE;
    if (max_group_size > s.num_seqs) return PKV_E_SHAPE;
    // query byte offsets within a group (and up to a tile past it) are 32-bit in the
    // tile kernel
    if ((long long)(max_group_size + 16) * s.num_heads * s.head_dim * 2 > 0x7fffffffLL)
        return PKV_E_SHAPE;
    GroupPlan p{};
    p.parts = max_prefix > kGroupPartBlocks
                  ? (max_prefix + kGroupPartBlocks - 1) / kGroupPartBlocks : 1;
    p.members_per_tile = 16 / group;
    const int per_set = p.members_per_tile * kGroupTilesPerWorkgroup;
    p.tiles = (max_group_size + per_set - 1) / per_set;
    const long long units8 = ((long long)p.parts * s.num_kv_heads * num_groups + 7) / 8 * 8;
    if (units8 * p.tiles > 0x7fffffffLL) return PKV_E_SHAPE;
    if (s.num_seqs > 0 && p.parts > 1) {
        const size_t recs = (size_t)s.num_seqs * s.num_heads * p.parts;
        p.off_prefix = kCounterBytes;
        p.off_m = p.off_prefix + align_up((size_t)s.num_seqs * sizeof(int32_t), 256);
        p.off_l = p.off_m + align_up(recs * sizeof(float), 256);
        p.off_o = p.off_l + align_up(recs * sizeof(float), 256);
        p.bytes = p.off_o + recs * s.head_dim * sizeof(float);
    }
    *plan = p;
    return PKV_OK;
}

}  // namespace pkv

extern "C" size_t pkv_paged_attention_grouped_workspace_size(int num_seqs, int num_heads,
                                                             int max_prefix_blocks) {
    // records only when a prefix needs several parts
    if (num_seqs <= 0 || num_heads <= 0 || max_prefix_blocks <= pkv::kGroupPartBlocks)
        return 0;
    const size_t parts =
        ((size_t)max_prefix_blocks + pkv::kGroupPartBlocks - 1) / pkv::kGroupPartBlocks;
    const size_t recs = (size_t)num_seqs * num_heads * parts;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    return pkv::kCounterBytes + up((size_t)num_seqs * sizeof(int32_t)) +
           2 * up(recs * sizeof(float)) + recs * pkv::kMfmaHeadDim * sizeof(float);
}

extern "C" int pkv_prefix_groups(const int32_t* block_tables, const int32_t* context_lens,
                                 int num_seqs, int max_blocks_per_seq, int block_size,
                                 int32_t* group_start, int32_t* group_prefix, int* num_groups,
                                 int* max_group_size, int* max_prefix_blocks) {
    if (num_seqs < 0 || max_blocks_per_seq < 0 || block_size <= 0) return PKV_E_SHAPE;
    if (!num_groups || !max_group_size || !max_prefix_blocks) return PKV_E_NULL;
    if (num_seqs > 0 && (!context_lens || !group_start || !group_prefix)) return PKV_E_NULL;
    if (num_seqs > 0 && max_blocks_per_seq > 0 && !block_tables) return PKV_E_NULL;
    const size_t W = (size_t)max_blocks_per_seq;
    // blocks of sequence b that are full (shared blocks are only ever full ones)
    auto full = [&](int b) {
        const long long n = context_lens[b];
        const long long f = n <= 0 ? 0 : n / block_size;
        return (int)(f < max_blocks_per_seq ? f : max_blocks_per_seq);
    };
    int ng = 0, gmax = 0, pmax = 0;
    int b = 0;
    while (b < num_seqs) {
        // a run of sequences whose first full block is the same physical block
        int e = b + 1;
        int pfx = full(b);
        if (pfx > 0 && block_tables[(size_t)b * W] >= 0) {
            while (e < num_seqs && full(e) > 0 &&
                   block_tables[(size_t)e * W] == block_tables[(size_t)b * W])
                ++e;
        }
        if (e - b < 2) {
            pfx = 0;
        } else {
            // leading entries that every member holds in full and all agree on
            for (int m = b + 1; m < e; ++m) {
                const int f = full(m);
                if (f < pfx) pfx = f;
                int j = 0;
                while (j < pfx &&
                       block_tables[(size_t)m * W + j] == block_tables[(size_t)b * W + j])
                    ++j;
                pfx = j;
            }
        }
        group_start[ng] = b;
        group_prefix[ng] = pfx;
        ++ng;
        if (e - b > gmax) gmax = e - b;
        if (pfx > pmax) pmax = pfx;
        b = e;
    }
    if (num_seqs > 0) group_start[ng] = num_seqs;
    *num_groups = ng;
    *max_group_size = gmax;
    *max_prefix_blocks = pmax;
    return PKV_OK;
}

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

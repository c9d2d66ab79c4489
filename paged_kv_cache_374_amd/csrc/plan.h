// Host-side validation and launch planning for paged decode attention.
// Plain C++ (no HIP calls): every decision here depends only on sizes, so it can be
// exercised without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>

namespace pkv {

enum class Path {
    Generic,          // VALU kernel, fixed partitions + reduction kernel
    MfmaBalanced,     // matrix-core kernel, equal-share work split, in-kernel merge
    MfmaPartitioned,  // matrix-core kernel, fixed partitions + reduction kernel
};

struct DecodeShape {
    int num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks, num_blocks;
    int dtype;           // pkv_dtype
    int partition_size;  // 0 = library's choice
};

// Workspace layout (byte offsets into the caller's workspace).
struct DecodePlan {
    Path path;
    int group;              // num_heads / num_kv_heads
    int partition_tokens;   // fixed-partition paths: tokens per partition
    int max_partitions;     // fixed-partition paths: ceil(max_blocks*block_size / partition)
    int max_workers;        // balanced path: upper bound on workers (partial slots = 2 per worker)
    size_t off_m, off_l, off_o;          // fixed-partition partial results
    size_t off_counters, off_partials;   // balanced path; per-unit path's long units
    int helpers;            // per-unit path: most helper workgroups per KV head (0: none)
    int rec_per_head;       // per-unit path: piece records per KV head
    size_t bytes;                        // total workspace bytes
};

// Largest number of workers the balanced path launches; sizes its partial slots.
constexpr int kMaxWorkers = 4096;
// Every workspace starts with this many bytes of merge counters, used only by the
// balanced path and left zeroed by it; all other scratch lies above, so calls of any
// path and shape can share one workspace without clobbering the counters.
constexpr size_t kCounterBytes = size_t(1) << 20;
// Largest share of blocks one balanced-path workgroup stages in LDS.
constexpr int kShareMax = 2048;
// head_dim and block_size of the matrix-core kernels.
constexpr int kMfmaHeadDim = 128;
constexpr int kMfmaBlockSize = 16;
// Partition length the generic path uses when the caller passes 0.
constexpr int kDefaultPartition = 512;
// Largest grouped-query factor any path supports.
constexpr int kMaxGroup = 16;
// Largest group the generic (VALU) kernel supports.
constexpr int kMaxGroupGeneric = 8;
// Sequences the balanced path scans in its prologue (LDS-resident prefix sums).
constexpr int kMaxSeqsBalanced = 4096;
// The automatic choice of one workgroup per (sequence, KV head) on the matrix-core
// path: at least this many units (two per CU of a 256-CU MI355X, the grid that is
// resident at once), at most this many blocks per table row (4096 tokens at block
// size 16), and at most this many sequences (every workgroup ranks the batch's
// lengths, four per lane of a wave).
constexpr int kPerUnitMinUnits = 512;
constexpr int kPerUnitMaxBlocks = 256;
constexpr int kPerUnitMaxSeqs = 256;
// Most helper workgroups per KV head that the per-unit grid adds for the pieces of
// units too long for one workgroup (the launch takes one per workgroup slot of the
// device, two per CU, spread over the KV heads); they return at once when the batch
// has none.
constexpr int kPerUnitMaxHelpers = 64;

// Validate sizes and choose a path. Returns 0 or a negative PKV_E_* code.
int plan_decode(const DecodeShape& s, DecodePlan* plan);

// Grouped decode (sequences sharing prefix blocks): blocks of a shared prefix per
// workgroup; a longer prefix is cut into parts whose records a merge kernel combines.
constexpr int kGroupPartBlocks = 128;
// Tiles of 16 columns (16 / group whole members each) that one workgroup of the
// grouped decode folds every shared block into.
constexpr int kGroupTilesPerWorkgroup = 2;

// Grouped decode launch sizes and workspace layout (byte offsets; everything lies above
// the kCounterBytes of merge counters that start every workspace). No workspace when
// every prefix fits one part.
struct GroupPlan {
    int parts;              // most parts of a prefix: max(1, ceil(max_prefix / kGroupPartBlocks))
    int members_per_tile;   // 16 / group: a tile's 16 columns hold whole members
    int tiles;              // workgroups per (part, KV head, group): tile sets of the
                            // largest group, kGroupTilesPerWorkgroup tiles each
    size_t off_prefix, off_m, off_l, off_o;
    size_t bytes;           // total workspace bytes (0 with one part or an empty batch)
};

// Validate the grouped decode's sizes (matrix-core shapes only) and lay out its
// workspace. Returns 0 or a negative PKV_E_* code.
int plan_grouped(const DecodeShape& s, int num_groups, int max_group_size, int max_prefix,
                 GroupPlan* plan);

// True when the matrix-core kernel supports this dtype / head_dim / block_size / group.
bool mfma_eligible(int dtype, int head_dim, int block_size, int group);

// Query heads per KV head that a matrix-core kernel instance is built for (4, 8, 16).
constexpr int mfma_gmax(int group) { return group <= 4 ? 4 : group <= 8 ? 8 : 16; }

// Floats of one balanced-path partial slot: o[gmax][128], m[gmax], l[gmax], padded to
// a multiple of 64 floats.
constexpr int balanced_slot_floats(int gmax) {
    return ((gmax * kMfmaHeadDim + 2 * gmax) + 63) / 64 * 64;
}

// Workgroups the balanced path launches: wg_per_cu per compute unit, at least enough
// that no share exceeds kShareMax blocks, rounded up to a multiple of 8 (one per
// XCD). Returns 0 when that exceeds kMaxWorkers.
int balanced_workers(const DecodeShape& s, int num_cus, int wg_per_cu);

}  // namespace pkv

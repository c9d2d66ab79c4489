// Paged decode attention on the matrix cores (bfloat16 / float16 KV, block_size 16,
// head_dim 128, up to 16 query heads per KV head).
//
// What is computed: for every sequence b and query head h, attention of q[b,h] over
// the first context_lens[b] tokens of the sequence, whose keys and values sit in the
// physical blocks listed by block_tables[b] (token t in block table[t / 16] at offset
// t % 16; "vLLM 核心源码深度解析…", section "Block Table 数据结构"). The walk visits
// the physical blocks one at a time, forms the block's partial attention and folds it
// into a running result with an online softmax ("vLLM 源码解析：PagedAttention 如何让大
// 模型推理提速 10 倍", section 四: per-block local attention, merged at the end).
//
// Mapping onto CDNA4 (one wavefront = one 16-token KV block at a time):
//   * QK^T of a block is one 16x16 tile: rows = the block's 16 tokens, columns = the
//     query heads of the KV head (G <= 16, unused columns see a zero query). K arrives
//     in whole 128-byte lines and passes through a per-wave LDS tile (chunk c of row t
//     stored at slot c ^ t: conflict-free writes and operand reads) into the A
//     operand of v_mfma_f32_16x16x32; Q is the B operand with the same dim assignment.
//   * The score tile comes out with lane l holding tokens 4(l/16)+r (r = 0..3) of
//     head l%16, which is exactly the A-operand layout of v_mfma_f32_16x16x16 for
//     P (rows = heads, k = tokens). The probabilities are rounded to the KV type.
//   * PV: lane l loads V rows 4(l/16)+r, dims 8(l%16) .. +7. The n-th of the eight
//     16x16x16 products takes element n of those four rows as its B operand, so
//     output column j of product n is dim 8j + n; the repack is a byte permute per
//     register, no LDS transpose.
//   * Exact online softmax per head in base-2 units (scale * log2 e folded in).
//
// Work split ("balanced" path): all (sequence, KV head) units are laid end to end as
// one list of blocks, and every workgroup (one per CU, one wave per SIMD) takes an
// equal contiguous share of it. Each wave streams one contiguous quarter of the share
// through a ring of register buffers. A unit a wave sees whole is written out by that
// wave; pieces cut between waves merge through LDS; a unit cut by share boundaries
// leaves one partial (m, l, unnormalised o) per workgroup, and the last workgroup to
// finish it (atomic counter) merges them:
//   M = max_w m_w,  L = sum_w l_w 2^(m_w - M),  out = sum_w o_w 2^(m_w - M) / L,
// in fixed workgroup order (deterministic), and zeroes the counter for the next call.
//
// "Partitioned" path (caller asks for a partition size): one workgroup per
// (partition, KV head, sequence); each leaves (m, l, o/l) per partition for the
// shared reduction kernel, or writes the output when the context has one partition.
//
// Both kernels can also perform the append of a decode step (see "fused append").
#include <type_traits>

#include "device_common.h"
#include "launchers.h"
#include "pagedkv.h"

namespace pkv {

namespace {

constexpr int kD = kMfmaHeadDim;
constexpr int kBS = kMfmaBlockSize;
constexpr int kTile = kBS * kD;  // elements of one (block, KV head) tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTabMax = kShareMax;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr uint32_t kNoTile = 0xffffffffu;
// Blocks of a shared prefix that one workgroup of the grouped decode attends.
constexpr int kGroupPart = kGroupPartBlocks;
// Register buffers per wave in the balanced kernel: while one block is folded, the
// next one is in flight. Measured on the Llama-3-8B-shaped batch (four waves per CU):
// 2 buffers 53.6 us, 3 buffers 55.7, 4 buffers 56.4, 6 buffers 58. The memory
// system is saturated either way, and more outstanding requests only add contention.
constexpr int kRing = 2;
// s_waitcnt immediate that waits for vmcnt == 0 only (expcnt 7 and lgkmcnt 15 are the
// "don't wait" values of their fields on gfx9-class parts).
constexpr int kWaitVmcnt0 = 0x0F70;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

template <typename T> struct Mma;
template <> struct Mma<bf16_t> {
    static __device__ __forceinline__ f32x4_t qk(const uint4& a, const uint4& b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                      __builtin_bit_cast(bf16x8_t, b), c, 0, 0,
                                                      0);
    }
    static __device__ __forceinline__ f32x4_t pv(const uint2& a, const uint2& b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                        __builtin_bit_cast(i16x4_t, b), c, 0, 0,
                                                        0);
    }
    // Two floats rounded to nearest even, packed low/high.
    static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
        bf16x2_t v = {(__bf16)lo, (__bf16)hi};
        return __builtin_bit_cast(uint32_t, v);
    }
    // acc + the two packed values (one dot-product instruction)
    static __device__ __forceinline__ float add_pair(uint32_t packed, float acc) {
        const bf16x2_t one = {(__bf16)1.f, (__bf16)1.f};
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, packed), one, acc,
                                               false);
    }
};
template <> struct Mma<f16_t> {
    static __device__ __forceinline__ f32x4_t qk(const uint4& a, const uint4& b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                     __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4_t pv(const uint2& a, const uint2& b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                    __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
        f16x2_t v = {(_Float16)lo, (_Float16)hi};
        return __builtin_bit_cast(uint32_t, v);
    }
    static __device__ __forceinline__ float add_pair(uint32_t packed, float acc) {
        const f16x2_t one = {(_Float16)1.f, (_Float16)1.f};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, packed), one, acc, false);
    }
};

// 16-bit element n (0..7) of each of two 16-byte rows, packed (row a low, row b high).
template <int N>
__device__ __forceinline__ uint32_t pick(const uint4& a, const uint4& b) {
    const uint32_t wa = N / 2 == 0 ? a.x : N / 2 == 1 ? a.y : N / 2 == 2 ? a.z : a.w;
    const uint32_t wb = N / 2 == 0 ? b.x : N / 2 == 1 ? b.y : N / 2 == 2 ? b.z : b.w;
    // v_perm_b32 selector bytes: 0-3 address the second source, 4-7 the first.
    constexpr uint32_t sel = (N % 2 == 0) ? 0x05040100u : 0x07060302u;
    return __builtin_amdgcn_perm(wb, wa, sel);
}

// Per-wave online-softmax state. Lane l: m, lsum for head l%16 (lsum over the tokens
// this lane saw); o[n][r] = unnormalised output of head 4(l/16)+r, dim 8(l%16)+n.
struct WaveState {
    float m;
    float lsum;
    f32x4_t o[8];
};

__device__ __forceinline__ void reset(WaveState& s) {
    s.m = kNegInf;
    s.lsum = 0.f;
#pragma unroll
    for (int n = 0; n < 8; ++n) s.o[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

// Keeps the loads issued before it ahead of those issued after it. The ring loops wait
// for a block with a vector-memory count that assumes the prologue issued the ring's
// buffers in order; the count at the loop head must hold on the entry path and on the
// back edge alike, and a prologue the scheduler had reordered made the compiler settle
// on a count that waited for both buffers in every other step.
__device__ __forceinline__ void issue_order() { asm volatile("" ::: "memory"); }

// Word 3 of a raw (untyped, stride 0) buffer descriptor on gfx9-class parts.
constexpr int kRawBufferWord3 = 0x00020000;

// Cache policy of the K/V loads: non-temporal. Every KV byte is read once per call,
// and keeping it out of L2 and the Infinity Cache measured ~8% more gather bandwidth
// (6.3 vs 5.8 TB/s for 285 MB of 4 KiB tiles) and 12-14% shorter decode kernels.
// Blocks that several sequences of the batch reference are the exception: the
// per-unit kernel reads those sequences with kShared, the default policy, so that the
// neighbours that read the same blocks find them in L2.
constexpr int kStream = 2;
constexpr int kShared = 0;

template <int AUX = 0>
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, int offset) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, offset, 0, AUX));
}
template <int AUX = 0>
__device__ __forceinline__ uint2 buffer_load8(__amdgpu_buffer_rsrc_t r, int offset) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, offset, 0, AUX));
}

// Per-wave LDS tile that turns the line-coalesced K rows into MFMA operand order.
// 16-byte chunk ch of token row t (0..15) sits at slot ch ^ t of the row. Every row
// starts on the same bank, so an operand read (one chunk from each of the 16 rows)
// must find 16 different slots: with ch ^ (t & 7), rows t and t + 8 shared a slot,
// and the LDS counters showed 19% (16-bit caches) and 39% (8-bit) of active LDS cycles
// lost to bank conflicts. Row-wise writes stay a permutation of the row's slots.
struct KTile {
    uint4 chunk[kBS][kD / 8];
};

// The query of the block's unit in QK B-operand order (lane l: column l%16, dims
// 32kk + 8(l/16) .. +7). It travels with every block so the loop carries no per-unit
// registers (an L1/L2 hit after a unit's first block). `qrow` is the unit's first query
// row, `qbytes` the size of the buffer over its rows and `qlane` the byte offset of the
// lane's column row from the first; columns past the unit fall outside the buffer and
// read zeros. A padding block (past the wave's range) passes qbytes 0: its loads are all
// zero-record, so none of them waits on memory when the wave drains its ring.
//   decode: column c is head c of the group: qlane = c * D * elt, qbytes = G * D * elt.
//   query chunks: column c is token c / G, head c % G of the chunk's rows.
template <typename T>
__device__ __forceinline__ void issue_query(uint4 (&qv)[4], const T* __restrict__ q, int qrow,
                                            int qbytes, int qlane, int lane) {
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(q + (size_t)qrow * kD), 0, qbytes, kRawBufferWord3);
    const int qoff = qlane + 8 * (lane >> 4) * (int)sizeof(T);
#pragma unroll
    for (int i = 0; i < 4; ++i) qv[i] = buffer_load16(rq, qoff + 32 * i * (int)sizeof(T));
}

// ---- KV formats: how one (block, KV head) tile of K and V is fetched and widened to
// the MFMA type T. Every block issues exactly the format's loads, with no branches: a
// block whose table entry is out of range gets buffers of zero records (the hardware
// returns zeros). A fixed count lets the compiler wait for just this block's loads
// while later blocks' loads stay in flight.

// Caches of T itself (bfloat16 / float16). Both tiles come in whole 128-byte lines: K
// load i covers rows 4i..4i+3 (one contiguous KiB; lane l takes row 4i + l/16, 16-byte
// chunk l%16), V load r covers rows r, 4+r, 8+r, 12+r (lane l takes row 4(l/16)+r,
// chunk l%16). (Loading K straight in MFMA operand order would touch 16 half lines per
// instruction, which measured ~20% slower as a gather.)
template <typename T>
struct KvNative {
    using Elem = T;
    static constexpr int kWaves = 4;   // balanced-kernel waves per workgroup
    struct Regs {
        uint4 k[4];
        uint4 v[4];
        uint4 q[4];
    };
    // AUX: cache policy of the K/V loads (kStream when every byte is read once).
    // WITH_Q false: the caller keeps the query in its own registers (r.q unused).
    template <int AUX = kStream, bool WITH_Q = true>
    static __device__ __forceinline__ void issue(Regs& r, const T* k_cache, const T* v_cache,
                                                 const T* __restrict__ q, uint32_t tile,
                                                 int qrow, int qbytes, int qlane, int lane) {
        tile = __builtin_amdgcn_readfirstlane(tile);
        qrow = __builtin_amdgcn_readfirstlane(qrow);
        const bool ok = tile != kNoTile;
        const size_t base = (size_t)(ok ? tile : 0u) * kTile;
        const int bytes = ok ? kTile * (int)sizeof(T) : 0;
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(k_cache + base), 0, bytes, kRawBufferWord3);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(v_cache + base), 0, bytes, kRawBufferWord3);
        const int c = lane & 15, grp = lane >> 4;
        const int koff = (grp * kD + 8 * c) * (int)sizeof(T);
        const int voff = (4 * grp * kD + 8 * c) * (int)sizeof(T);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            r.k[i] = buffer_load16<AUX>(rk, koff + i * 4 * kD * (int)sizeof(T));
#pragma unroll
        for (int i = 0; i < 4; ++i)
            r.v[i] = buffer_load16<AUX>(rv, voff + i * kD * (int)sizeof(T));
        if constexpr (WITH_Q) issue_query(r.q, q, qrow, ok ? qbytes : 0, qlane, lane);
    }
    static __device__ __forceinline__ void stage_k(KTile& kt, const Regs& r, int lane) {
        const int c = lane & 15, grp = lane >> 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 4 * i + grp;
            kt.chunk[t][c ^ (t & 15)] = r.k[i];
        }
    }
    static __device__ __forceinline__ void widen_v(const Regs& r, uint4 (&v)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = r.v[e];
    }
    // Append: chunk c (16 bytes) of the new K (kind 0) or V (kind 1) row of unit (b, g)
    // goes to position n - 1 of the sequence, bit for bit. It comes in two halves so a
    // caller can issue the source loads early and store once the destination tile (the
    // unit's last block, phys * Hkv + g, or kNoTile when its table entry is out of
    // range) is known.
    static constexpr int kAppendChunks = kD * (int)sizeof(T) / 16;
    struct AppendSrc {
        uint4 val;
    };
    static __device__ __forceinline__ void append_load(AppendSrc& a, const T* __restrict__ new_k,
                                                       const T* __restrict__ new_v, int b,
                                                       int g, int Hkv, int kind, int c) {
        const size_t src = ((size_t)b * Hkv + g) * kD;
        a.val = reinterpret_cast<const uint4*>((kind ? new_v : new_k) + src)[c];
    }
    static __device__ __forceinline__ void append_store(const AppendSrc& a, T* k_cache,
                                                        T* v_cache, uint32_t tile, int pos,
                                                        int kind, int c, float, float) {
        if (tile == kNoTile) return;
        const size_t dst = ((size_t)tile * kBS + pos) * kD;
        reinterpret_cast<uint4*>((kind ? v_cache : k_cache) + dst)[c] = a.val;
    }
    static __device__ __forceinline__ void append(T* k_cache, T* v_cache,
                                                  const T* __restrict__ new_k,
                                                  const T* __restrict__ new_v,
                                                  const int32_t* __restrict__ table, int b,
                                                  int g, int Hkv, int n, int num_blocks,
                                                  int kind, int c, float k_inv, float v_inv) {
        AppendSrc a;
        append_load(a, new_k, new_v, b, g, Hkv, kind, c);
        const int j = (n - 1) / kBS;
        const int phys = table[j];
        const bool ok = phys >= 0 && phys < num_blocks;
        append_store(a, k_cache, v_cache, ok ? (uint32_t)phys * Hkv + g : kNoTile,
                     n - 1 - j * kBS, kind, c, k_inv, v_inv);
    }
};

// Two E4M3 codes (the low or the high byte pair of a word) widened exactly to T,
// packed low/high (the lower byte becomes the lower element).
template <typename T> struct WidenFp8;
template <> struct WidenFp8<bf16_t> {
    template <bool HI>
    static __device__ __forceinline__ uint32_t pair(uint32_t w) {
        return __builtin_bit_cast(uint32_t,
                                  __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI));
    }
};
template <> struct WidenFp8<f16_t> {
    template <bool HI>
    static __device__ __forceinline__ uint32_t pair(uint32_t w) {
        return __builtin_bit_cast(uint32_t,
                                  __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, HI));
    }
};
template <typename T>
__device__ __forceinline__ uint4 widen8(uint32_t lo, uint32_t hi) {   // 8 codes -> 8 T
    using W = WidenFp8<T>;
    return make_uint4(W::template pair<false>(lo), W::template pair<true>(lo),
                      W::template pair<false>(hi), W::template pair<true>(hi));
}

// 8-bit caches (OCP FP8 E4M3 codes, one byte per element). Every E4M3 value is exact
// in bfloat16 and float16, so widening loses nothing; the caches' scales are applied
// outside the tile (the key scale folds into the softmax scale, the value scale into
// the final normalisation). K load i covers rows 8i..8i+7 (one contiguous KiB; lane l
// takes row 8i + l/8, codes 16(l%8) .. +15); V load r covers rows r, 4+r, 8+r, 12+r
// (lane l takes row 4(l/16)+r, codes 8(l%16) .. +7: 8 bytes, four half lines per
// instruction).
template <typename T>
struct KvFp8 {
    using Elem = uint8_t;
    // Two waves per SIMD: with half the bytes per block the fold's own latency weighs
    // more, and a second wave hides it (35.1 vs 37.8 us on the 8B-shaped batch).
    static constexpr int kWaves = 8;
    struct Regs {
        uint4 k[2];
        uint2 v[4];
        uint4 q[4];
    };
    template <int AUX = kStream, bool WITH_Q = true>
    static __device__ __forceinline__ void issue(Regs& r, const uint8_t* k_cache,
                                                 const uint8_t* v_cache,
                                                 const T* __restrict__ q, uint32_t tile,
                                                 int qrow, int qbytes, int qlane, int lane) {
        tile = __builtin_amdgcn_readfirstlane(tile);
        qrow = __builtin_amdgcn_readfirstlane(qrow);
        const bool ok = tile != kNoTile;
        const size_t base = (size_t)(ok ? tile : 0u) * kTile;
        const int bytes = ok ? kTile : 0;
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(k_cache + base), 0, bytes, kRawBufferWord3);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(v_cache + base), 0, bytes, kRawBufferWord3);
        const int koff = (lane >> 3) * kD + 16 * (lane & 7);
        const int voff = 4 * (lane >> 4) * kD + 8 * (lane & 15);
#pragma unroll
        for (int i = 0; i < 2; ++i) r.k[i] = buffer_load16<AUX>(rk, koff + i * 8 * kD);
#pragma unroll
        for (int i = 0; i < 4; ++i) r.v[i] = buffer_load8<AUX>(rv, voff + i * kD);
        if constexpr (WITH_Q) issue_query(r.q, q, qrow, ok ? qbytes : 0, qlane, lane);
    }
    // Lane l holds chunks 2(l%8) and 2(l%8)+1 of its row. Lanes with l%8 >= 4 store
    // their odd chunk first, so each eight-lane group of a store covers all eight
    // 16-byte slots of a 128-byte bank period instead of only the even (or odd) ones.
    static __device__ __forceinline__ void stage_k(KTile& kt, const Regs& r, int lane) {
        const int c2 = 2 * (lane & 7);   // the lane's first 8-dim chunk
        const int odd = (lane >> 2) & 1;  // 1: odd chunk first
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int t = 8 * i + (lane >> 3);
            const uint32_t a0 = odd ? r.k[i].z : r.k[i].x, a1 = odd ? r.k[i].w : r.k[i].y;
            const uint32_t b0 = odd ? r.k[i].x : r.k[i].z, b1 = odd ? r.k[i].y : r.k[i].w;
            kt.chunk[t][(c2 + odd) ^ (t & 15)] = widen8<T>(a0, a1);
            kt.chunk[t][(c2 + 1 - odd) ^ (t & 15)] = widen8<T>(b0, b1);
        }
    }
    static __device__ __forceinline__ void widen_v(const Regs& r, uint4 (&v)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = widen8<T>(r.v[e].x, r.v[e].y);
    }
    // Append: chunk c (4 elements) of the new K or V row is quantised (binary32 product
    // with the reciprocal scale, then E4M3 nearest-even, saturating) into 4 codes at
    // position n - 1 of the sequence. Split into source loads and the quantising store
    // as for 16-bit caches. Four elements per thread spread a row pair over a whole wave:
    // the quantiser is about 20 VALU instructions per element, and with 16 elements per
    // thread it held up the workgroup's first loads by ~0.7 us.
    static constexpr int kAppendChunks = kD / 4;
    struct AppendSrc {
        uint2 v;
    };
    static __device__ __forceinline__ void append_load(AppendSrc& a, const T* __restrict__ new_k,
                                                       const T* __restrict__ new_v, int b,
                                                       int g, int Hkv, int kind, int c) {
        a.v = *reinterpret_cast<const uint2*>((kind ? new_v : new_k) +
                                              ((size_t)b * Hkv + g) * kD + 4 * c);
    }
    static __device__ __forceinline__ void append_store(const AppendSrc& a, uint8_t* k_cache,
                                                        uint8_t* v_cache, uint32_t tile, int pos,
                                                        int kind, int c, float k_inv,
                                                        float v_inv) {
        if (tile == kNoTile) return;
        float f[8];
        Vec16<T>::unpack(make_uint4(a.v.x, a.v.y, 0u, 0u), f);
        const float inv = kind ? v_inv : k_inv;
        const uint32_t w = fp8_e4m3_code(f[0] * inv) | fp8_e4m3_code(f[1] * inv) << 8 |
                           fp8_e4m3_code(f[2] * inv) << 16 | fp8_e4m3_code(f[3] * inv) << 24;
        const size_t dst = ((size_t)tile * kBS + pos) * kD + 4 * c;
        *reinterpret_cast<uint32_t*>((kind ? v_cache : k_cache) + dst) = w;
    }
    static __device__ __forceinline__ void append(uint8_t* k_cache, uint8_t* v_cache,
                                                  const T* __restrict__ new_k,
                                                  const T* __restrict__ new_v,
                                                  const int32_t* __restrict__ table, int b,
                                                  int g, int Hkv, int n, int num_blocks,
                                                  int kind, int c, float k_inv, float v_inv) {
        AppendSrc a;
        append_load(a, new_k, new_v, b, g, Hkv, kind, c);
        const int j = (n - 1) / kBS;
        const int phys = table[j];
        const bool ok = phys >= 0 && phys < num_blocks;
        append_store(a, k_cache, v_cache, ok ? (uint32_t)phys * Hkv + g : kNoTile,
                     n - 1 - j * kBS, kind, c, k_inv, v_inv);
    }
};

// A operand of QK product kk for lane l: token l%16, dims 32kk + 8(l/16) .. +7.
__device__ __forceinline__ uint4 k_operand(const KTile& kt, int kk, int lane) {
    const int c = lane & 15, grp = lane >> 4;
    return kt.chunk[c][(4 * kk + grp) ^ c];
}

// Largest sum of one lane's 4 weights of a block that stands: each weight then lies at
// most this far above the column's reference (2^8), far inside the range of binary32
// sums and of the bfloat16 / float16 operands of the PV product.
constexpr float kWeightBound = 256.f;

// The query-dependent half of a fold: scores of one 16-column tile against the block's
// K operand `ka` (k_operand order), masked to the first `lim` tokens for the lane's
// column, the online-softmax update, and the PV product with the block's V rows `v`.
template <typename T>
__device__ __forceinline__ void fold_tile(WaveState& s, const uint4 (&ka)[4],
                                          const uint4 (&qv)[4], const uint4 (&v)[4], int lim,
                                          float scale_log2, int lane) {
    const int grp = lane >> 4;
    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) sc = Mma<T>::qk(ka[i], qv[i], sc);
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = (4 * grp + e < lim) ? sc[e] * scale_log2 : kNegInf;
    // Weights against the column's reference s.m (the final ratio o / l cancels it).
    // A lane's sum of its 4 weights bounds each of them, so a sum within kWeightBound
    // keeps the reference in place with no column maximum taken (most blocks). It fails
    // (also as infinity or NaN on a column's first block, s.m = -inf) when some score
    // passes the reference by more than log2(kWeightBound / 4): then the reference
    // moves to the column's maximum, o and l are rescaled (a wave-uniform branch), and
    // the weights are taken again, at most 1 each (up to rounding), so that pass
    // stands. Either way the reference stays within 8 (base 2) below the maximum of
    // the scores so far, as the merges of partial results assume.
    float p[4];
    float ps;
    auto weights = [&](float mu) {
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = fast_exp2(x[e] - mu);
        ps = (p[0] + p[1]) + (p[2] + p[3]);
    };
    weights(s.m);
    if (__ballot(!(ps <= kWeightBound)) != 0) {
        float mb = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        mb = fmaxf(mb, __shfl_xor(mb, 16));
        mb = max_xor32(mb);
        const float mn = fmaxf(s.m, mb);
        const float alpha = (s.m == kNegInf) ? 0.f : fast_exp2(s.m - mn);
        s.lsum *= alpha;
        s.m = mn;
        // o[.][e] belongs to head 4(l/16)+e, whose factor lives in lane 4(l/16)+e.
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float a = __shfl(alpha, 4 * grp + e);
#pragma unroll
            for (int n = 0; n < 8; ++n) s.o[n][e] *= a;
        }
        // a column with no token yet in view takes its weights against 0 (zeros, not NaN)
        weights(mn == kNegInf ? 0.f : mn);
    }
    s.lsum += ps;
    const uint2 pa = make_uint2(Mma<T>::pack(p[0], p[1]), Mma<T>::pack(p[2], p[3]));
#define PKV_PV_STEP(N)                                                                  \
    s.o[N] = Mma<T>::pv(pa, make_uint2(pick<N>(v[0], v[1]), pick<N>(v[2], v[3])), s.o[N]);
    PKV_PV_STEP(0) PKV_PV_STEP(1) PKV_PV_STEP(2) PKV_PV_STEP(3)
    PKV_PV_STEP(4) PKV_PV_STEP(5) PKV_PV_STEP(6) PKV_PV_STEP(7)
#undef PKV_PV_STEP
}

// The query-independent half: K through the wave's LDS tile into operand order (ka),
// V widened to T with the rows past the context cleared. `valid` = tokens of the block
// inside the context. Slots past the context hold stale data (possibly NaN); a zero
// weight does not cancel a NaN inside the product, so their V rows are cleared, and
// their scores are replaced by -inf in fold_tile (a select), so stale K never reaches
// the softmax.
template <typename T, typename KV>
__device__ __forceinline__ void stage_block(const typename KV::Regs& r, KTile& kt, int valid,
                                            int lane, uint4 (&ka)[4], uint4 (&v)[4]) {
    const int grp = lane >> 4;
    KV::stage_k(kt, r, lane);
    KV::widen_v(r, v);
    if (valid < kBS) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (4 * grp + e >= valid) v[e] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) ka[i] = k_operand(kt, i, lane);
}

// Fold one block into the wave's state. `valid` = tokens of the block inside the
// context (0 masks the whole block); `lim` <= valid = tokens that count for the lane's
// column (decode: lim = valid; query chunks: the column's causal limit).
template <typename T, typename KV>
__device__ __forceinline__ void fold_block(WaveState& s, typename KV::Regs& r, KTile& kt,
                                           int valid, int lim, float scale_log2, int lane) {
    uint4 ka[4], v[4];
    stage_block<T, KV>(r, kt, valid, lane, ka, v);
    fold_tile<T>(s, ka, r.q, v, lim, scale_log2, lane);
}

__device__ __forceinline__ float weight(float m, float M) {
    return m == kNegInf ? 0.f : fast_exp2(m - M);
}

template <typename T>
__device__ __forceinline__ void store4(T* p, float4 v) {
    uint2 w;
    w.x = Mma<T>::pack(v.x, v.y);
    w.y = Mma<T>::pack(v.z, v.w);
    *reinterpret_cast<uint2*>(p) = w;
}

// Cache policy of the partial-result traffic between workgroups: the device-scope
// coherence bit (sc1), as device-scope atomics use it, on plain wide accesses, so the
// stores write through to the point of coherence shared by all XCDs and the loads
// skip stale cache copies, while the compiler still batches them freely.
constexpr int kCoherent = 16;

__device__ __forceinline__ void publish4(__amdgpu_buffer_rsrc_t r, int byte_off, float4 v) {
    typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, byte_off, 0,
                                           kCoherent);
}
__device__ __forceinline__ void publish1(__amdgpu_buffer_rsrc_t r, int byte_off, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, byte_off, 0,
                                          kCoherent);
}
__device__ __forceinline__ float4 fetch4(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return __builtin_bit_cast(float4,
                              __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kCoherent));
}
__device__ __forceinline__ float fetch1(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, kCoherent));
}

// Partial result of one unit: o[GMAX][D] (unnormalised), then m[GMAX], l[GMAX]. The
// same layout serves a wave's piece in LDS and a workgroup's piece in the workspace.
template <int GMAX>
struct Part {
    static constexpr int kM = GMAX * kD;
    static constexpr int kL = GMAX * kD + GMAX;
    static constexpr int kFloats = balanced_slot_floats(GMAX);
};

// The wave's softmax denominator of head (lane & 15), in every lane of that head.
__device__ __forceinline__ float head_lsum(const WaveState& s) {
    float ls = s.lsum;
    ls += __shfl_xor(ls, 16);
    return sum_xor32(ls);
}

// A wave's state -> partial record P (LDS).
template <int GMAX>
__device__ __forceinline__ void wave_to_part(float* P, const WaveState& s, int lane, int group) {
    const int c = lane & 15, grp = lane >> 4;
    const float ls = head_lsum(s);
    if (grp == 0 && c < group) {
        P[Part<GMAX>::kM + c] = s.m;
        P[Part<GMAX>::kL + c] = ls;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int h = 4 * grp + e;
        if (h < group) {
            float4* dst = reinterpret_cast<float4*>(P + h * kD + 8 * c);
            dst[0] = make_float4(s.o[0][e], s.o[1][e], s.o[2][e], s.o[3][e]);
            dst[1] = make_float4(s.o[4][e], s.o[5][e], s.o[6][e], s.o[7][e]);
        }
    }
}

// A wave's state -> normalised output rows (the wave saw the whole unit). `rows`
// points at head 0 of the unit's group; each lane stores 16 bytes per head.
template <typename T>
__device__ __forceinline__ void wave_to_out(T* rows, const WaveState& s, int lane, int group,
                                            float out_scale) {
    const int c = lane & 15, grp = lane >> 4;
    const float ls = head_lsum(s);
    const float inv = ls > 0.f ? out_scale / ls : 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int h = 4 * grp + e;
        const float iv = __shfl(inv, h);
        if (h < group) {
            uint4 w;
            w.x = Mma<T>::pack(s.o[0][e] * iv, s.o[1][e] * iv);
            w.y = Mma<T>::pack(s.o[2][e] * iv, s.o[3][e] * iv);
            w.z = Mma<T>::pack(s.o[4][e] * iv, s.o[5][e] * iv);
            w.w = Mma<T>::pack(s.o[6][e] * iv, s.o[7][e] * iv);
            *reinterpret_cast<uint4*>(rows + h * kD + 8 * c) = w;
        }
    }
}

// Merge n (1 <= n <= NMAX) LDS partial records for head h, dims d0..d0+3. Records are
// addressed by index into the LDS array (not through generic pointers, which would
// compile to flat loads that also wait for outstanding global stores). The trip count
// is fixed and records past n are masked, so every LDS read of a call is independent
// of the others and they all go out before the first wait.
template <int GMAX, int NREC, int NMAX>
__device__ __forceinline__ void merge_parts(const float (&rec)[NREC][Part<GMAX>::kFloats],
                                            const int* idx, int n, int h, int d0, float& M,
                                            float& L, float4& o) {
    // idx[i] must be a valid record for every i < NMAX (callers repeat a valid one
    // past n), so the reads need no branch and all go out together.
    float m[NMAX], l[NMAX];
    float4 v[NMAX];
#pragma unroll
    for (int i = 0; i < NMAX; ++i) {
        const float* r = rec[idx[i]];
        m[i] = i < n ? r[Part<GMAX>::kM + h] : kNegInf;
        l[i] = r[Part<GMAX>::kL + h];
        v[i] = *reinterpret_cast<const float4*>(r + h * kD + d0);
    }
    M = m[0];
#pragma unroll
    for (int i = 1; i < NMAX; ++i) M = fmaxf(M, m[i]);
    L = 0.f;
    o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < NMAX; ++i) {
        const float wt = weight(m[i], M);
        L += l[i] * wt;
        o.x += v[i].x * wt;
        o.y += v[i].y * wt;
        o.z += v[i].z * wt;
        o.w += v[i].w * wt;
    }
}

// A value every lane of the wave holds (read from LDS, say) moved to a scalar register,
// so that branches on it are scalar and the compiler sees straight control flow.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Largest sequence b with Hkv * pref[b] <= x (x below the total, wave-uniform; pref in
// LDS). Such a sequence is never empty: an empty one shares its prefix with the next.
// Since pref is non-decreasing, b is a count: a ballot over every k-th entry
// (k = ceil(num_seqs / 64)) finds the stretch of k sequences that holds b, a second
// ballot counts inside it. One or two LDS round trips, where a binary search over 64
// sequences takes six in a row.
__device__ __forceinline__ int seq_of(const int* pref, int num_seqs, int Hkv, int x) {
    const int lane = __lane_id();
    const int k = (num_seqs + 63) >> 6;
    const int s = lane * k;
    const bool le = s < num_seqs && Hkv * pref[s] <= x;
    const int base = (__popcll(__ballot(le)) - 1) * k;
    if (k == 1) return base;
    const int s2 = base + 1 + lane;
    const bool le2 = lane < k - 1 && s2 < num_seqs && Hkv * pref[s2] <= x;
    return base + __popcll(__ballot(le2));
}

// The unit after (b, g): next KV head, else the first KV head of the next non-empty
// sequence.
__device__ __forceinline__ void next_unit(const int* pref, int num_seqs, int Hkv, int b, int g,
                                          int& bn, int& gn) {
    bn = b;
    gn = g + 1;
    if (gn == Hkv) {
        gn = 0;
        ++bn;
        while (bn < num_seqs && uni(pref[bn + 1]) == uni(pref[bn])) ++bn;
    }
}

// ------------------------------------------------------------------ fused append
// A decode step first writes each sequence's newest token (position n - 1) into the
// free slot of its last block, then attends over all n tokens ([P3] section "Block
// table：为什么它能减少碎片": a decoded token fills the last block's free slot or a
// newly taken block; the slot is found by the block-table walk of [P2] section
// "Block Table 数据结构"). Fused into the decode, the workgroup that reads a unit's
// last block writes that unit's new K and V rows during staging; the workgroup
// barrier before its waves start loading orders those stores before the loads.
// ------------------------------------------------------------------ balanced kernel
// Equal shares of the block list: worker w (logical index) covers [w*C, (w+1)*C)
// clipped to the list, C = ceil(total / W). Every workgroup derives the same map from
// `total`, so share boundaries, and with them the results, do not depend on scheduling.
// (Per-XCD streaming speeds differ by a few per cent, but the pattern changes from
// machine to machine; a fixed skew between XCDs did not shorten the kernel.)
struct ShareMap {
    int C, total;
    __device__ ShareMap(int total_, int W) : C((total_ + W - 1) / W), total(total_) {}
    // First block of worker w's share (w = W gives the end of the list).
    __device__ int start(int w) const {
        const long long s = (long long)w * C;
        return s < total ? (int)s : total;
    }
    // The worker whose share holds block t (0 <= t < total).
    __device__ int owner(int t) const { return t / C; }
};

// How the workgroup finishes one unit that its waves saw in pieces: merge LDS records
// rec[0..n-1] (n = 0: nothing to do), then write query rows row.. of the output, or,
// when the unit crosses the share's edge, publish the merged piece at float offset
// `slot` of the partials.
template <int NW>
struct MergePlan {
    int rec[NW];
    int n, cross, row, slot;
};

template <int GMAX, int NW>
struct BalancedLds {
    int pref[kMaxSeqsBalanced + 1];   // blocks per sequence, exclusive prefix
    int ctx[kMaxSeqsBalanced];        // context length per sequence (clipped to the table)
    uint32_t tile[kTabMax];           // (physical block * Hkv + kv head), or kNoTile
    int qrow[kTabMax];                // first query row of the block's unit
    uint8_t valid[kTabMax];           // tokens of the block inside the context
    KTile ktile[NW];
    float part[NW * 2][Part<GMAX>::kFloats];   // wave v: [2v] first, [2v+1] last unit piece
    MergePlan<NW> plan[NW + 1];                // candidate units of the end phase
    int nplan;                                 // how many of them have work
    int4 cross[2];                             // units crossing the share's edges (b, g, su, ue)
    int ncross;                                // how many
    int flag[2];
};

// End-phase plan of a share [x0, x1) cut into quarters of Cw blocks (run by one wave;
// sb0..sb1 are the sequences the share touches). Candidate k is the first unit of
// quarter k (k < nq) or the share's last unit (k = nq); lane k finds it. Units cut
// between waves or between workgroups are all among the candidates, and at most two
// of them (the share's first and last unit) cross its edges. For each candidate with
// work, the plan names the LDS records of its pieces and where the merged result goes:
// output rows for a unit inside the share, this workgroup's partial slot for a crossing
// one (published for the count round).
template <int GMAX, int NW>
__device__ __forceinline__ void plan_end_phase(BalancedLds<GMAX, NW>& S, int sb0, int sb1,
                                               int Hkv, int x0, int x1, int Cw, int w,
                                               int num_heads, int group, int lane) {
    const int nq = (x1 - x0 + Cw - 1) / Cw;   // non-empty quarters
    const int k = lane;
    int b = 0, g = 0, su = 0, ue = 0;
    if (k <= nq) {
        const int pos = k < nq ? x0 + k * Cw : x1 - 1;
        int lo = sb0, hi = sb1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (Hkv * S.pref[mid] <= pos) lo = mid; else hi = mid - 1;
        }
        b = lo;
        const int nb = S.pref[b + 1] - S.pref[b];
        g = (pos - Hkv * S.pref[b]) / nb;
        su = Hkv * S.pref[b] + g * nb;
        ue = su + nb;
    }
    const int prev_su = __shfl(su, k > 0 ? k - 1 : 0);
    // the crossing units: the first candidate if it starts before the share or ends
    // after it, the last if it differs and ends after it
    const int fb = __shfl(b, 0), fg = __shfl(g, 0), fs = __shfl(su, 0), fe = __shfl(ue, 0);
    const int lb = __shfl(b, nq), lg = __shfl(g, nq), ls = __shfl(su, nq),
              le = __shfl(ue, nq);
    if (k == 0) {
        int n = 0;
        if (fs < x0 || fe > x1) S.cross[n++] = make_int4(fb, fg, fs, fe);
        if (ls != fs && le > x1) S.cross[n++] = make_int4(lb, lg, ls, le);
        S.ncross = n;
    }
    if (k <= nq) {
        MergePlan<NW> pl;
        const int lo = su > x0 ? su : x0, hi = ue < x1 ? ue : x1;
        const int wlo = (lo - x0) / Cw, whi = (hi - 1 - x0) / Cw;
        const bool crosses = su < x0 || ue > x1;
        pl.cross = crosses;
        // same unit as the previous candidate, or one wave saw all of it (written)
        pl.n = ((k > 0 && prev_su == su) || (wlo == whi && !crosses)) ? 0 : whi - wlo + 1;
#pragma unroll
        for (int j = 0; j < NW; ++j) {
            const int v = wlo + j < whi ? wlo + j : whi;
            pl.rec[j] = 2 * v + (su <= x0 + v * Cw ? 0 : 1);
        }
        pl.row = b * num_heads + g * group;
        pl.slot = (2 * w + (su <= x0 ? 0 : 1)) * Part<GMAX>::kFloats;
        // keep only the candidates with work, packed to the front
        const unsigned long long act = __ballot(pl.n > 0);
        if (pl.n > 0) S.plan[__popcll(act & ((1ull << k) - 1))] = pl;
        if (k == 0) S.nplan = __popcll(act);
    }
}

// NW waves per workgroup, one workgroup per CU. 16-bit caches use one wave per SIMD:
// with two waves on a SIMD the older one was measured to stream ~1.5x faster than the
// younger, which breaks equal static shares, and eight waves per CU were no faster
// (52.9 vs 53.0 us on the 8B-shaped batch). 8-bit caches use two waves per SIMD.
//
// KV: the cache format (KvNative<T> or KvFp8<T>). scale_log2 = scale * key scale *
// log2(e); out_scale = value scale (1 for native caches) multiplies each normalised
// output; k_inv, v_inv are the reciprocal scales an 8-bit append quantises with.
template <typename T, typename KV, int GMAX, int NW>
__global__ __launch_bounds__(64 * NW) void decode_mfma_balanced_kernel(
    T* __restrict__ out, const T* __restrict__ q, typename KV::Elem* k_cache,
    typename KV::Elem* v_cache, const T* __restrict__ new_k, const T* __restrict__ new_v,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ ctx_lens, float scale_log2,
    float out_scale, float k_inv, float v_inv, int num_seqs, int num_heads,
    int num_kv_heads, int group, int max_blocks, int num_blocks, int32_t* __restrict__ counters,
    float* __restrict__ partials) {
    __shared__ BalancedLds<GMAX, NW> S;
    constexpr int kThreads = 64 * NW;
    constexpr int kWaves = NW;
    // wave index via readfirstlane: the compiler cannot tell that tid >> 6 is uniform,
    // and everything derived from it (share bounds, loop counters) must be scalar
    const int tid = threadIdx.x, lane = tid & 63, wave = uni(tid >> 6);
    const int W = gridDim.x;
    // Logical worker index: consecutive shares (which may cut one unit) go to
    // workgroups that the dispatcher places on the same XCD (round-robin over 8).
    const int w = (W % 8 == 0) ? (blockIdx.x % 8) * (W / 8) + blockIdx.x / 8 : blockIdx.x;
    const int cap = max_blocks * kBS;
    const int Hkv = num_kv_heads;

    // ---- prologue: context lengths, blocks per sequence and their prefix sums
    for (int i = tid; i < num_seqs; i += kThreads) {
        int n = ctx_lens[i];
        n = n < 0 ? 0 : (n > cap ? cap : n);
        S.ctx[i] = n;
        S.pref[i + 1] = (n + kBS - 1) / kBS;
    }
    if (tid == 0) S.pref[0] = 0;
    __syncthreads();
    if (wave == 0) {
        int carry = 0;
        for (int base = 0; base < num_seqs; base += 64) {
            const int i = base + lane;
            int v = i < num_seqs ? S.pref[i + 1] : 0;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int u = __shfl_up(v, off);
                if (lane >= off) v += u;
            }
            if (i < num_seqs) S.pref[i + 1] = v + carry;
            carry += __shfl(v, 63);
        }
    }
    __syncthreads();
    // Empty contexts produce zero rows; sequences are dealt out round-robin.
    for (int b = w; b < num_seqs; b += W) {
        if (S.pref[b + 1] == S.pref[b]) {
            T* o = out + (size_t)b * num_heads * kD;
            for (int i = tid * 4; i < num_heads * kD; i += kThreads * 4)
                store4(o + i, make_float4(0.f, 0.f, 0.f, 0.f));
        }
    }
    // Block indices of all units laid end to end fit in 32 bits: the plan admits at
    // most kMaxWorkers * kShareMax blocks of tables.
    const int total = Hkv * uni(S.pref[num_seqs]);
    if (total == 0) return;
    const ShareMap shares(total, W);
    const int x0 = shares.start(w);
    const int x1 = shares.start(w + 1);
    if (x0 >= x1) return;

    // ---- fused append, first half. The units whose last block lies in the share are
    // consecutive: from the unit of the share's first block through the unit of its
    // last block (that one only when it ends inside the share). Item `it` is unit
    // au0 + it / (2 * chunks), its K (kind 0) or V row, chunk it % chunks. Each
    // thread loads its first item's source now, so those loads overlap the table loads
    // of the staging below; the destination comes from the staged table entry.
    // The sequences of the share's first and last blocks bound every search below.
    const int sb0 = seq_of(S.pref, num_seqs, Hkv, x0);
    const int sb1 = seq_of(S.pref, num_seqs, Hkv, x1 - 1);
    int au0 = 0, aitems = 0;
    if (new_k != nullptr) {
        const int p0 = uni(S.pref[sb0]), p1 = uni(S.pref[sb1]);
        const int g0 = (x0 - Hkv * p0) / (uni(S.pref[sb0 + 1]) - p0);
        const int g1 = (x1 - 1 - Hkv * p1) / (uni(S.pref[sb1 + 1]) - p1);
        au0 = sb0 * Hkv + g0;
        aitems = (sb1 * Hkv + g1 - au0 + 1) * 2 * KV::kAppendChunks;
    }
    // Item `it`: its unit (b, g), row kind and chunk c; returns the index in the share
    // of the unit's last block, or -1 when that block lies past the share (or the
    // sequence is empty).
    auto item = [&](int it, int& b, int& g, int& kind, int& c) -> int {
        const int u = au0 + it / (2 * KV::kAppendChunks);
        b = u / Hkv;
        g = u - b * Hkv;
        kind = (it / KV::kAppendChunks) & 1;
        c = it % KV::kAppendChunks;
        const int nb = S.pref[b + 1] - S.pref[b];
        const int last = Hkv * S.pref[b] + (g + 1) * nb - 1;
        return (nb > 0 && last < x1) ? last - x0 : -1;
    };
    typename KV::AppendSrc a0;
    int ai0 = -1, ab = 0, ag = 0, ak = 0, ac = 0;
    if (tid < aitems) {
        ai0 = item(tid, ab, ag, ak, ac);
        KV::append_load(a0, new_k, new_v, ab, ag, Hkv, ak, ac);
    }

    // ---- stage (tile, query row, valid tokens) of every block of the share. Each
    // thread finds its block's sequence by binary search over the prefix sums, so the
    // table loads of the whole share go out together.
    for (int xx = x0 + tid; xx < x1; xx += kThreads) {
        int lo = sb0, hi = sb1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (Hkv * S.pref[mid] <= xx) lo = mid; else hi = mid - 1;
        }
        // the largest such sequence is never empty (an empty one shares its prefix
        // with the next), so nb > 0
        const int b = lo;
        const int nb = S.pref[b + 1] - S.pref[b];
        const int r = xx - Hkv * S.pref[b];
        const int g = r / nb, j = r - g * nb;
        const int phys = tables[(size_t)b * max_blocks + j];
        const int left = S.ctx[b] - j * kBS;
        const bool ok = phys >= 0 && phys < num_blocks;
        S.tile[xx - x0] = ok ? (uint32_t)phys * (uint32_t)Hkv + (uint32_t)g : kNoTile;
        S.qrow[xx - x0] = b * num_heads + g * group;
        S.valid[xx - x0] = (uint8_t)(ok ? (left < kBS ? left : kBS) : 0);
    }
    __syncthreads();
    // ---- fused append, second half: the stores, to the staged tile of each unit's last
    // block (kNoTile for an out-of-range table entry: nothing is written). The workgroup
    // barrier below orders them before the waves' loads of that block.
    if (ai0 >= 0)
        KV::append_store(a0, k_cache, v_cache, S.tile[ai0], (S.ctx[ab] - 1) % kBS, ak, ac,
                         k_inv, v_inv);
    for (int it = tid + kThreads; it < aitems; it += kThreads) {
        int b, g, kind, c;
        const int i = item(it, b, g, kind, c);
        if (i < 0) continue;
        typename KV::AppendSrc a;
        KV::append_load(a, new_k, new_v, b, g, Hkv, kind, c);
        KV::append_store(a, k_cache, v_cache, S.tile[i], (S.ctx[b] - 1) % kBS, kind, c, k_inv,
                         v_inv);
    }
    __syncthreads();

    // ---- each wave streams one contiguous quarter of the share; no barriers inside
    const int Cw = (x1 - x0 + kWaves - 1) / kWaves;
    const int xa = x0 + wave * Cw;
    const int xb = xa + Cw < x1 ? xa + Cw : x1;
    if (xa < xb) {
        int b = seq_of(S.pref, num_seqs, Hkv, xa);
        int nb = uni(S.pref[b + 1]) - uni(S.pref[b]);
        int g = (xa - Hkv * uni(S.pref[b])) / nb;
        int su = Hkv * uni(S.pref[b]) + g * nb;
        int ue = su + nb;
        int bn, gn;
        next_unit(S.pref, num_seqs, Hkv, b, g, bn, gn);
        // Every step issues one block (a zero-record buffer past the quarter's end), so
        // the number of loads in flight never depends on the path taken.
        const int qbytes = group * kD * (int)sizeof(T), qlane = (lane & 15) * kD * (int)sizeof(T);
        auto issue = [&](typename KV::Regs& R, int xi) {
            const int i = (int)((xi < xb ? xi : xb - 1) - x0);
            KV::issue(R, k_cache, v_cache, q, xi < xb ? S.tile[i] : kNoTile, S.qrow[i], qbytes,
                      qlane, lane);
        };
        // kRing register buffers in fixed roles (the loop is unrolled kRing times): a
        // block's loads land where the fold reads them (no copies), and kRing - 1
        // blocks stay in flight behind the one being folded.
        static_assert(kRing == 2, "the loop below is unrolled for two buffers");
        typename KV::Regs R0, R1;
        issue(R0, xa);
        issue_order();
        issue(R1, xa + 1);
        // While the first blocks are in flight, wave 0 plans the end phase: it depends
        // only on where the quarters and units begin and end, not on the data.
        if (wave == 0) plan_end_phase(S, sb0, sb1, Hkv, x0, x1, Cw, w, num_heads, group, lane);
        WaveState st;
        reset(st);
        int x = xa;
        // Finish the current unit: the wave saw all of it -> output; else its piece
        // goes to the wave's first (unit began at or before xa) or last LDS record.
        auto flush = [&]() {
            if (su >= xa && ue <= xb)
                wave_to_out(out + ((size_t)b * num_heads + (size_t)g * group) * kD, st, lane,
                            group, out_scale);
            else
                wave_to_part<GMAX>(S.part[2 * wave + (su <= xa ? 0 : 1)], st, lane, group);
        };
        auto advance = [&]() {
            flush();
            b = bn;
            g = gn;
            nb = S.pref[b + 1] - S.pref[b];
            su = Hkv * S.pref[b] + (int)g * nb;
            ue = su + nb;
            next_unit(S.pref, num_seqs, Hkv, b, g, bn, gn);
            reset(st);
        };
#define PKV_STEP(R)                                                                       \
        if (x >= xb) break;                                                               \
        if (x >= ue) advance();                                                           \
        {                                                                                 \
            const int vd = uni(S.valid[x - x0]);                                          \
            fold_block<T, KV>(st, R, S.ktile[wave], vd, vd, scale_log2, lane);            \
        }                                                                                 \
        issue(R, x + kRing);                                                              \
        ++x;
        while (true) {
            PKV_STEP(R0)
            PKV_STEP(R1)
        }
#undef PKV_STEP
        // Retire the padding loads still in flight before the last unit's stores go
        // out. Their registers are reused below, and the memory counter retires loads
        // and stores in order, so waiting after the stores would also wait for the
        // stores to complete (slow while other workgroups saturate the memory system).
        // The padding loads touch no memory, so this wait is short.
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        flush();
    }
    __syncthreads();

    // ---- units cut between waves or between workgroups (planned by wave 0 before its
    // loop: plan_end_phase). Pieces of a crossing unit outside the share belong to other
    // workgroups.
    const __amdgpu_buffer_rsrc_t R = __builtin_amdgcn_make_buffer_rsrc(
        partials, 0, 2 * kMaxWorkers * Part<GMAX>::kFloats * (int)sizeof(float),
        kRawBufferWord3);
    // The crossing units and the merge plan were written before the loop (by wave 0).
    const int ncross = uni(S.ncross);
    const int cb0 = uni(S.cross[0].x), cg0 = uni(S.cross[0].y), cs0 = uni(S.cross[0].z),
              ce0 = uni(S.cross[0].w);
    const int cb1 = uni(S.cross[1].x), cg1 = uni(S.cross[1].y), cs1 = uni(S.cross[1].z),
              ce1 = uni(S.cross[1].w);
    constexpr int kCols = kD / 4;   // float4 columns of a head's row
    for (int it = tid; it < S.nplan * group * kCols; it += kThreads) {
        const int k = it / (group * kCols), i = it - k * (group * kCols);
        const MergePlan<NW> pl = S.plan[k];   // one copy: all fields load together
        const int h = i / kCols, d0 = (i % kCols) * 4;
        float M, Ls;
        float4 o;
        merge_parts<GMAX, NW * 2, NW>(S.part, pl.rec, pl.n, h, d0, M, Ls, o);
        if (!pl.cross) {
            const float inv = Ls > 0.f ? out_scale / Ls : 0.f;
            store4(out + ((size_t)pl.row + h) * kD + d0,
                   make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv));
        } else {
            // this workgroup's piece, with write-through stores (see kCoherent)
            publish4(R, 4 * (pl.slot + h * kD + d0), o);
            if (d0 == 0) {
                publish1(R, 4 * (pl.slot + Part<GMAX>::kM + h), M);
                publish1(R, 4 * (pl.slot + Part<GMAX>::kL + h), Ls);
            }
        }
    }
    if (ncross == 0) return;
    // The wait and barrier complete every published store before the counters move.
    // (A release fence here would write back whole L2 caches: measured slower than the
    // attention itself.) Wave k counts crossing unit k.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (lane == 0 && wave < ncross) {
        const int su = wave ? cs1 : cs0, ue = wave ? ce1 : ce0;
        const int u = (wave ? cb1 : cb0) * Hkv + (wave ? cg1 : cg0);
        const int done = __hip_atomic_fetch_add(&counters[u], 1, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
        S.flag[wave] = (done == shares.owner(ue - 1) - shares.owner(su));
    }
    __syncthreads();
    // A last contributor reads every workgroup's piece back (coherent loads) and merges
    // them in workgroup order; the two crossing units use separate thread halves.
    const int span = kThreads / ncross;
    const int k = tid / span, t = tid - k * span;
    if (S.flag[k]) {
        const int b = k ? cb1 : cb0, g = k ? cg1 : cg0;
        const int su = k ? cs1 : cs0, ue = k ? ce1 : ce0;
        const int wf = shares.owner(su), wl = shares.owner(ue - 1);
        T* rows = out + ((size_t)b * num_heads + (size_t)g * group) * kD;
        for (int i = t; i < group * kCols; i += span) {
            const int h = i / kCols, d0 = (i % kCols) * 4;
            // Online merge in workgroup order. The loads of unrolled iterations do not
            // depend on the running state, so they go out together: one round trip.
            float M = kNegInf, Ls = 0.f;
            float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
            for (int v = wf; v <= wl; ++v) {
                const int sl = (2 * v + ((v > wf || su == shares.start(v)) ? 0 : 1)) *
                               Part<GMAX>::kFloats;
                const float m = fetch1(R, 4 * (sl + Part<GMAX>::kM + h));
                const float l = fetch1(R, 4 * (sl + Part<GMAX>::kL + h));
                const float4 pv = fetch4(R, 4 * (sl + h * kD + d0));
                const float Mn = fmaxf(M, m);
                const float a = weight(M, Mn), c = weight(m, Mn);
                Ls = Ls * a + l * c;
                o.x = o.x * a + pv.x * c;
                o.y = o.y * a + pv.y * c;
                o.z = o.z * a + pv.z * c;
                o.w = o.w * a + pv.w * c;
                M = Mn;
            }
            const float inv = Ls > 0.f ? out_scale / Ls : 0.f;
            store4(rows + h * kD + d0, make_float4(o.x * inv, o.y * inv, o.z * inv,
                                                   o.w * inv));
        }
        if (t == 0)
            __hip_atomic_store(&counters[b * Hkv + g], 0, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ------------------------------------------------------------------ long with short
// Kernels that give each (sequence, KV head) its own workgroup launch a grid of
// (x, KV head, sequence) with two workgroups per CU. When the grid is resident at once
// (at most kPerUnitMinUnits workgroups), the dispatcher hands every CU one workgroup of
// the grid's first half, then one of its second half, so a CU that drew two long
// contexts would set the kernel's time. The first half therefore takes the sequences
// in decreasing order of context length and the second half in increasing order: long
// pairs with short. A larger grid runs in rounds and takes them longest first
// throughout, so the longest start earliest. Batches above kPerUnitMaxSeqs keep their
// order.
__device__ __forceinline__ bool ranks_lengths(int nseq) {
    return nseq > 1 && nseq <= kPerUnitMaxSeqs;
}

// Lane u holds the clipped lengths of sequences u, u + 64, u + 128 and u + 192 and
// their block counts (-1 past the batch). nseq <= kPerUnitMaxSeqs.
struct LengthKeys {
    int len[4];
    int key[4];   // blocks: the work a sequence's unit holds
};

__device__ __forceinline__ LengthKeys load_lengths(const int32_t* __restrict__ ctx_lens,
                                                   int nseq, int cap, int lane) {
    static_assert(kPerUnitMaxSeqs <= 256, "four lengths per lane");
    // all loads first (a wave-uniform test per round, indices clamped into the batch),
    // then one wait: a test per lane around each load made the compiler wait for each
    // round before issuing the next
    const int nr = (nseq + 63) >> 6;
    int raw[4] = {0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < 4; ++r)
        if (r < nr) raw[r] = ctx_lens[min(lane + 64 * r, nseq - 1)];
    LengthKeys k;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int u = lane + 64 * r;
        int x = -1;   // no sequence: never counted
        if (u < nseq) x = raw[r] < 0 ? 0 : (raw[r] > cap ? cap : raw[r]);
        k.len[r] = x;
        k.key[r] = x < 0 ? -1 : (x + kBS - 1) / kBS;
    }
    return k;
}

// The clipped length of sequence u (wave-uniform u < nseq).
__device__ __forceinline__ int length_of(const LengthKeys& k, int u) {
    const int l = u & 63, r = u >> 6;
    const int v0 = __builtin_amdgcn_readlane(k.len[0], l), v1 = __builtin_amdgcn_readlane(k.len[1], l);
    const int v2 = __builtin_amdgcn_readlane(k.len[2], l), v3 = __builtin_amdgcn_readlane(k.len[3], l);
    return r == 0 ? v0 : r == 1 ? v1 : r == 2 ? v2 : v3;
}

// Wave-wide maximum of x (every lane's value), with row-local DPP steps (lanes ^1, ^2,
// then rotations by 4 and 8 within each row of 16) and one read of each row.
__device__ __forceinline__ int wave_max(int x) {
    x = max(x, __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false));    // quad [1,0,3,2]
    x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false));    // quad [2,3,0,1]
    x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x124, 0xF, 0xF, false));   // row_ror:4
    x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x128, 0xF, 0xF, false));   // row_ror:8
    return max(max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
               max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}

// Wave-wide sum of x, with the same steps as wave_max.
__device__ __forceinline__ int wave_sum(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x124, 0xF, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false);
    return (__builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16)) +
           (__builtin_amdgcn_readlane(x, 32) + __builtin_amdgcn_readlane(x, 48));
}

// Longest and shortest of the lengths (wave-uniform).
__device__ __forceinline__ void length_range(const LengthKeys& k, int cap, int& hi, int& lo) {
    int h = -1, neg_lo = -cap;   // minimum through the maximum of negated lengths
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        h = max(h, k.len[r]);
        if (k.len[r] >= 0) neg_lo = max(neg_lo, -k.len[r]);
    }
    hi = wave_max(h);
    lo = -wave_max(neg_lo);
}

// True when every length lies within an eighth of the longest.
__device__ __forceinline__ bool narrow_range(int hi, int lo) { return 8 * (hi - lo) <= hi; }

// The sequence at position `want` when the units are ordered by block count, most
// first, equal counts by index; its length goes to `len`. Blocks are the work a unit
// holds, and counting them rather than tokens shortens the search: `lo` and `hi` bound
// the counts (the batch's shortest and longest). Every wave finds it on its own, with
// no LDS and no barrier: a binary search over the count counts the larger ones with
// ballots (the answer is the smallest x with at most `want` counts above it), and the
// position among the units of exactly that count picks one of them. want < nseq.
__device__ __forceinline__ int select_by_length(const LengthKeys& k, int nseq, int want,
                                                int lo, int hi, int& len) {
    const int nr = (nseq + 63) >> 6;
    auto above = [&](int x) {
        int c = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (r < nr) c += __popcll(__ballot(k.key[r] > x));
        return c;
    };
    // above(hi) == 0 <= want, above(lo - 1) == nseq > want
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (above(mid) <= want)
            hi = mid;
        else
            lo = mid + 1;
    }
    int t = want - above(lo);   // position among the units of lo blocks
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        if (r >= nr) break;
        unsigned long long m = __ballot(k.key[r] == lo);
        const int c = __popcll(m);
        if (t < c) {
            for (int i = 0; i < t; ++i) m &= m - 1;
            const int u = 64 * r + __ffsll(m) - 1;
            len = length_of(k, u);
            return u;
        }
        t -= c;
    }
    len = 0;
    return 0;   // not reached for want < nseq
}

// Position of sequence u in the order select_by_length uses (most blocks first, equal
// counts by index): the units with more blocks, plus those with as many and a smaller
// index. u < nseq, wave-uniform.
__device__ __forceinline__ int rank_of(const LengthKeys& k, int nseq, int u) {
    const int nr = (nseq + 63) >> 6;
    const int l = u & 63, ru = u >> 6;
    const int k0 = __builtin_amdgcn_readlane(k.key[0], l), k1 = __builtin_amdgcn_readlane(k.key[1], l);
    const int k2 = __builtin_amdgcn_readlane(k.key[2], l), k3 = __builtin_amdgcn_readlane(k.key[3], l);
    const int ku = ru == 0 ? k0 : ru == 1 ? k1 : ru == 2 ? k2 : k3;
    const int lane = (int)__lane_id();
    int c = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r)
        if (r < nr)
            c += __popcll(__ballot(k.key[r] > ku || (k.key[r] == ku && 64 * r + lane < u)));
    return c;
}

// Ranks remembered between calls. A serving loop decodes the same batch step after step,
// and a unit's position in the order changes only when block counts change it, so each
// workgroup first tries the sequence that held its position last time: rank_of checks
// it exactly against the current lengths (a few ballots instead of the search), and only
// a failed check runs the search and remembers its answer. A wrong or stale guess costs
// nothing but that search, so the result never depends on the table. Slots are chosen by
// the address of the lengths array (a loop keeps reusing its buffer; calls with other
// buffers take other slots); concurrent launches may overwrite each other's entries,
// which is again only a failed check.
constexpr int kRankSlots = 32;
__device__ int rank_memo[kRankSlots][kPerUnitMaxSeqs];

__device__ __forceinline__ int rank_slot(const int32_t* ctx_lens) {
    // Fibonacci hashing of the address (its top five bits after the multiply)
    const uint64_t a = reinterpret_cast<uint64_t>(ctx_lens) >> 8;
    return (int)((a * 0x9E3779B97F4A7C15ull) >> 59);
}

// Position in the longest-first order of the sequence that workgroup (.., .., b) takes.
// More workgroups than two per CU: longest first throughout (the grid runs in rounds,
// and the longest should start earliest); else the second half runs shortest first.
__device__ __forceinline__ int pairing_position(int nseq, int b) {
    const int half = (nseq + 1) / 2;
    const bool rounds = (long long)nseq * gridDim.y * gridDim.x > kPerUnitMinUnits;
    return (rounds || b < half) ? b : nseq - 1 - (b - half);
}

// The sequence workgroup (.., .., b) takes, and its clipped length in `len`. Lengths
// that all lie within an eighth of the longest keep the caller's order: pairing or
// ranking them would even out the CUs' shares by at most that eighth, while the
// caller's order keeps neighbours together, which is where sequences that share prefix
// blocks sit (the samples of one prompt), so that one XCD reads a shared block for
// several of them while it is still in its L2.
__device__ __forceinline__ int paired_sequence(const int32_t* __restrict__ ctx_lens, int nseq,
                                               int b, int cap, int lane, int& len) {
    auto own = [&] {
        const int x = ctx_lens[b];
        len = x < 0 ? 0 : (x > cap ? cap : x);
        return b;
    };
    if (!ranks_lengths(nseq)) return own();
    // the remembered sequence of this position (see rank_memo), read with the lengths
    const int want = pairing_position(nseq, b);
    int* memo = &rank_memo[rank_slot(ctx_lens)][0];
    const int guess = __builtin_amdgcn_raw_buffer_load_b32(
        __builtin_amdgcn_make_buffer_rsrc((void*)memo, 0, kPerUnitMaxSeqs * 4, kRawBufferWord3),
        want * 4, 0, 0);
    const LengthKeys k = load_lengths(ctx_lens, nseq, cap, lane);
    int hi, lo;
    length_range(k, cap, hi, lo);
    if (narrow_range(hi, lo)) return own();
    const int gu = __builtin_amdgcn_readfirstlane(guess);
    if (gu >= 0 && gu < nseq && rank_of(k, nseq, gu) == want) {
        len = length_of(k, gu);
        return gu;
    }
    const int u = select_by_length(k, nseq, want, (lo + kBS - 1) / kBS, (hi + kBS - 1) / kBS,
                                   len);
    if (lane == 0 && (int)(threadIdx.x >> 6) == 0) memo[want] = u;
    return u;
}

// ------------------------------------------------------------------ long units
// One workgroup per (sequence, KV head) cannot finish before its longest unit does.
// With S the blocks of all units over the workgroup slots (two per CU), a unit of more
// than 2S blocks outlasts any pairing of it with a short one, so it is cut into pieces
// of P >= S/2 blocks (S rounded up; half a slot's share measured best, S/3 and S
// slower): its own workgroup folds the first piece, and helper workgroups (placed
// first in the grid when some unit is cut, so that they start with the first round)
// fold the others, each long unit's pieces in turn, in sequence order.
// Every piece's partial result goes to a workspace record; the last piece to finish
// (a device-scope counter per unit) merges them all in piece order. P grows when the
// pieces would outnumber the helpers.
struct UnitWork {
    int b = 0, n = 0;     // sequence and its clipped length
    int j0 = 0, j1 = 0;   // blocks this workgroup folds
    int pieces = 1;       // workgroups that share the unit
    int piece = 0;        // this workgroup's piece
    int rec = 0;          // record of the unit's first piece (per KV head)
};

// The work of workgroup z of a per-unit grid of nseq + helpers workgroups per KV head;
// false when it has none (a helper with no piece to fold).
__device__ __forceinline__ bool unit_work(const int32_t* __restrict__ ctx_lens, int nseq, int z,
                                          int cap, int lane, int slots, int helpers, int hkv,
                                          UnitWork& w) {
    if (!ranks_lengths(nseq)) {
        if (z >= nseq) return false;
        const int x = ctx_lens[z];
        w.b = z;
        w.n = x < 0 ? 0 : (x > cap ? cap : x);
        w.j1 = (w.n + kBS - 1) / kBS;
        return true;
    }
    // this workgroup's remembered sequence, read alongside the lengths (a vector load,
    // so that scalar waits do not wait for it)
    const int want = z < nseq ? pairing_position(nseq, z) : 0;
    int* memo = &rank_memo[rank_slot(ctx_lens)][0];
    const int guess = __builtin_amdgcn_raw_buffer_load_b32(
        __builtin_amdgcn_make_buffer_rsrc((void*)memo, 0, kPerUnitMaxSeqs * 4, kRawBufferWord3),
        want * 4, 0, 0);
    const LengthKeys k = load_lengths(ctx_lens, nseq, cap, lane);
    auto own = [&](int b) {
        w.b = b;
        w.n = length_of(k, b);
        w.j1 = (w.n + kBS - 1) / kBS;
    };
    int nbk[4], sum = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        nbk[r] = k.key[r] > 0 ? k.key[r] : 0;
        sum += nbk[r];
    }
    int hi, lo;
    length_range(k, cap, hi, lo);
    // A unit is long when it holds more than twice the blocks of an average slot:
    // blocks * slots > 2 * (blocks of all units). At most kPerUnitMaxBlocks blocks per
    // unit, and helpers come with at most one merge counter per unit (2^18 units):
    // 32-bit safe.
    const int all = helpers > 0 ? wave_sum(sum) * hkv : 0;
    auto is_long = [&](int nb) { return nb * slots > 2 * all; };
    int P = 0;   // piece length; 0: no unit is cut
    if (helpers > 0 && is_long((hi + kBS - 1) / kBS)) {
        int S = (all + slots - 1) / slots;   // blocks of an average slot
        if (S < 1) S = 1;
        int bl = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) bl += is_long(nbk[r]) ? nbk[r] : 0;
        bl = wave_sum(bl);
        P = max((S + 1) / 2, (bl + helpers - 1) / helpers);
    }
    // When some unit is cut, the helpers come first in the grid: the dispatcher starts
    // them with the first round instead of after short units free their slots, so the
    // pieces of a long unit run alongside the rest (every workgroup derives P from the
    // same lengths, so all agree on the order).
    if (P > 0 && helpers > 0) z = z < helpers ? nseq + z : z - helpers;
    // Long units in sequence order: visit(u, blocks, pieces, first record) returns true
    // to stop. Lanes past the batch hold 0 blocks, so they are never long.
    auto walk = [&](auto visit) {
        int c = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            unsigned long long m = __ballot(is_long(nbk[r]));
            while (m) {
                const int l = __ffsll(m) - 1;
                m &= m - 1;
                const int nb = __builtin_amdgcn_readlane(nbk[r], l);
                const int kk = (nb + P - 1) / P;
                if (visit(64 * r + l, nb, kk, c)) return;
                c += kk;
            }
        }
    };
    if (z >= nseq) {
        if (P == 0) return false;
        int h = z - nseq;   // extra piece h of the whole batch
        bool found = false;
        walk([&](int u, int nb, int kk, int c) {
            if (h >= kk - 1) {
                h -= kk - 1;
                return false;
            }
            own(u);
            w.pieces = kk;
            w.piece = h + 1;
            w.j0 = w.piece * P;
            w.j1 = min(nb, w.j0 + P);
            w.rec = c;
            found = true;
            return true;
        });
        return found;
    }
    if (narrow_range(hi, lo)) {
        own(z);
    } else {
        const int pos = pairing_position(nseq, z);   // z may have moved past the helpers
        const int gu = uni(guess);
        if (pos == want && gu >= 0 && gu < nseq && rank_of(k, nseq, gu) == pos) {
            own(gu);
        } else {
            int len;
            const int b = select_by_length(k, nseq, pos, (lo + kBS - 1) / kBS,
                                           (hi + kBS - 1) / kBS, len);
            w.b = b;
            w.n = len;
            w.j1 = (len + kBS - 1) / kBS;
            if (lane == 0 && (int)(threadIdx.x >> 6) == 0) memo[pos] = b;
        }
    }
    if (P > 0 && is_long(w.j1) && w.j1 > P) {
        const int b = w.b;
        walk([&](int u, int nb, int kk, int c) {
            if (u != b) return false;
            w.pieces = kk;
            w.j1 = P;
            w.rec = c;
            return true;
        });
    }
    return true;
}

// True when sequence b's first block is also the first block of sequence b - 1 or
// b + 1 (the samples of one prompt, forked from it, sit next to each other and
// reference its blocks).
__device__ __forceinline__ bool shares_first_block(const int32_t* __restrict__ tables, int b,
                                                   int nseq, int max_blocks) {
    const int first = tables[(size_t)b * max_blocks];
    const int prev = b > 0 ? tables[(size_t)(b - 1) * max_blocks] : -1;
    const int next = b + 1 < nseq ? tables[(size_t)(b + 1) * max_blocks] : -1;
    return first >= 0 && (first == prev || first == next);
}

// ------------------------------------------------------------------ partitioned kernel
template <int GMAX>
struct PartLds {
    uint32_t tile[kTabMax];
    uint8_t valid[kTabMax];
    int shared;   // shares_first_block for the workgroup's sequence
    int last;     // this workgroup merges the pieces of its unit
    KTile ktile[kWaves];
    float part[kWaves][Part<GMAX>::kFloats];
};

template <typename T, typename KV, int GMAX, bool PATCH>
__global__ __launch_bounds__(kThreads) void decode_mfma_partition_kernel(
    T* __restrict__ out, const T* __restrict__ q, typename KV::Elem* k_cache,
    typename KV::Elem* v_cache, const T* __restrict__ new_k, const T* __restrict__ new_v,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ ctx_lens, float scale_log2,
    float out_scale, float k_inv, float v_inv, int num_heads, int num_kv_heads,
    int group, int max_blocks, int num_blocks, int part_blocks, int max_parts,
    float* __restrict__ ws_m, float* __restrict__ ws_l, float* __restrict__ ws_o, int num_seqs,
    int slots, int32_t* __restrict__ counters, float* __restrict__ records, int rec_per_head) {
    __shared__ PartLds<GMAX> S;
    const int p = blockIdx.x, g = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = uni(tid >> 6);
    const int cap = max_blocks * kBS;
    // one partition per context: one workgroup per (sequence, KV head), long paired
    // with short on a CU, long units cut into pieces (unit_work)
    UnitWork w;
    if (gridDim.x == 1) {
        if (!unit_work(ctx_lens, num_seqs, blockIdx.z, cap, lane, slots,
                       (int)gridDim.z - num_seqs, num_kv_heads, w))
            return;
    } else {
        w.b = blockIdx.z;
        const int x = ctx_lens[w.b];
        w.n = x < 0 ? 0 : (x > cap ? cap : x);
        const int nbw = (w.n + kBS - 1) / kBS;
        w.j0 = p * part_blocks;
        w.j1 = min(nbw, w.j0 + part_blocks);
    }
    const int b = uni(w.b), n = uni(w.n), pieces = uni(w.pieces);
    const int nb = (n + kBS - 1) / kBS;
    if (n == 0) {
        if (p == 0)
            for (int i = tid * 4; i < group * kD; i += kThreads * 4)
                store4(out + ((size_t)b * num_heads + g * group) * kD + i,
                       make_float4(0.f, 0.f, 0.f, 0.f));
        return;
    }
    const int j0 = uni(w.j0);
    if (j0 >= nb) return;
    const int j1 = uni(w.j1);
    const int nparts = (nb + part_blocks - 1) / part_blocks;
    for (int j = j0 + tid; j < j1; j += kThreads) {
        const int phys = tables[(size_t)b * max_blocks + j];
        const bool ok = phys >= 0 && phys < num_blocks;
        const int left = n - j * kBS;
        S.tile[j - j0] = ok ? (uint32_t)phys * (uint32_t)num_kv_heads + (uint32_t)g : kNoTile;
        S.valid[j - j0] = (uint8_t)(ok ? (left < kBS ? left : kBS) : 0);
    }
    // the cache policy's test reads beside the table (its latency hides behind it)
    if (tid == kThreads - 1) S.shared = shares_first_block(tables, b, num_seqs, max_blocks);
    // Fused append: the partition holding the newest token writes its K and V rows.
    // The plain form appends here, and the barrier below orders the stores before this
    // workgroup's loads. The PATCH form (16-bit caches, chosen for grids that start
    // every unit at once, where this barrier is on the launch's critical path) has no
    // wait for them: the wave that folds the unit's last block takes the new rows from
    // new_k / new_v into that block's load registers itself (the bytes the cache will
    // hold) and stores them to the cache then; no load in this kernel reads them back.
    static_assert(!PATCH || sizeof(typename KV::Elem) == sizeof(T), "16-bit caches only");
    const int last = (n - 1) / kBS;                  // the unit's last block
    const bool appends = new_k != nullptr && last >= j0 && last < j1;
    if (!PATCH && appends && tid < 2 * KV::kAppendChunks)
        KV::append(k_cache, v_cache, new_k, new_v, tables + (size_t)b * max_blocks, b, g,
                   num_kv_heads, n, num_blocks, tid / KV::kAppendChunks,
                   tid % KV::kAppendChunks, k_inv, v_inv);
    __syncthreads();
    const bool shared = uni(S.shared) != 0;
    WaveState st;
    reset(st);
    // waves take every fourth block; two register buffers in fixed roles
    const int qrow = b * num_heads + g * group;
    // every step issues one block (a zero-record buffer past the end): the loads in
    // flight never depend on the path taken
    const int qbytes = group * kD * (int)sizeof(T), qlane = (lane & 15) * kD * (int)sizeof(T);
    // PATCH: wave (last - j0) % 4 folds the last block (waves take every fourth block);
    // every wave loads chunk (lane % 16) of the new K and V rows, from zero-record
    // buffers unless it is that wave, so that all waves issue the same loads.
    const bool patches = PATCH && appends && wave == (last - j0) % kWaves;
    uint4 nk = make_uint4(0, 0, 0, 0), nv = nk;
    if constexpr (PATCH) {
        const size_t row = ((size_t)b * num_kv_heads + g) * kD;
        const int rb = patches ? kD * (int)sizeof(T) : 0;
        nk = buffer_load16(__builtin_amdgcn_make_buffer_rsrc((void*)(new_k + (patches ? row : 0)),
                                                             0, rb, kRawBufferWord3),
                           (lane & 15) * 16);
        nv = buffer_load16(__builtin_amdgcn_make_buffer_rsrc((void*)(new_v + (patches ? row : 0)),
                                                             0, rb, kRawBufferWord3),
                           (lane & 15) * 16);
    }
    // Row t of the last block sits in K register t / 4 of the lanes of row group t % 4,
    // and in V register t % 4 of the lanes of row group t / 4 (the layouts of
    // KvNative::issue); the new chunks replace whatever the block's loads returned there.
    auto patch = [&](typename KV::Regs& R) {
        if constexpr (PATCH) {
            const int t = (n - 1) & (kBS - 1), grp = lane >> 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (e == (t >> 2) && grp == (t & 3)) R.k[e] = nk;
                if (e == (t & 3) && grp == (t >> 2)) R.v[e] = nv;
            }
            if (lane < 16) {
                typename KV::AppendSrc a;
                a.val = nk;
                KV::append_store(a, k_cache, v_cache, S.tile[last - j0], t, 0, lane, 0.f, 0.f);
                a.val = nv;
                KV::append_store(a, k_cache, v_cache, S.tile[last - j0], t, 1, lane, 0.f, 0.f);
            }
        }
    };
    auto stream_blocks = [&](auto policy) {
        constexpr int AUX = decltype(policy)::value;
        auto issue = [&](typename KV::Regs& R, int ji) {
            KV::template issue<AUX>(R, k_cache, v_cache, q,
                                    ji < j1 ? S.tile[ji - j0] : kNoTile, qrow, qbytes, qlane,
                                    lane);
        };
        int j = j0 + wave;
        typename KV::Regs A, B;
        issue(A, j);
        issue_order();
        issue(B, j + kWaves);
#define PKV_STEP(R)                                                                          \
    if (j >= j1) break;                                                                      \
    if (PATCH && patches && j == last) patch(R);                                             \
    fold_block<T, KV>(st, R, S.ktile[wave], S.valid[j - j0], S.valid[j - j0], scale_log2,    \
                      lane);                                                                 \
    issue(R, j + 2 * kWaves);                                                                \
    j += kWaves;
        while (true) {
            PKV_STEP(A)
            PKV_STEP(B)
        }
#undef PKV_STEP
    };
    if (shared)
        stream_blocks(std::integral_constant<int, kShared>{});
    else
        stream_blocks(std::integral_constant<int, kStream>{});

    wave_to_part<GMAX>(S.part[wave], st, lane, group);
    __syncthreads();
    int P[kWaves];
    for (int v = 0; v < kWaves; ++v) P[v] = v;
    constexpr int kCols = kD / 4;   // float4 columns of a head's row
    // pieces of a long unit: records of kFloats floats, rec_per_head per KV head
    const __amdgpu_buffer_rsrc_t R = __builtin_amdgcn_make_buffer_rsrc(
        records, 0, pieces > 1 ? num_kv_heads * rec_per_head * Part<GMAX>::kFloats * 4 : 0,
        kRawBufferWord3);
    const int rec0 = (g * rec_per_head + uni(w.rec)) * Part<GMAX>::kFloats;
    for (int i = tid; i < group * kCols; i += kThreads) {
        const int h = i / kCols, d0 = (i % kCols) * 4;
        float M, Ls;
        float4 o;
        merge_parts<GMAX, kWaves, kWaves>(S.part, P, kWaves, h, d0, M, Ls, o);
        if (pieces > 1) {
            // this piece, with write-through stores (see kCoherent)
            const int sl = rec0 + uni(w.piece) * Part<GMAX>::kFloats;
            publish4(R, 4 * (sl + h * kD + d0), o);
            if (d0 == 0) {
                publish1(R, 4 * (sl + Part<GMAX>::kM + h), M);
                publish1(R, 4 * (sl + Part<GMAX>::kL + h), Ls);
            }
            continue;
        }
        const float inv = Ls > 0.f ? out_scale / Ls : 0.f;
        o.x *= inv; o.y *= inv; o.z *= inv; o.w *= inv;
        const size_t hrow = (size_t)b * num_heads + g * group + h;
        if (nparts == 1) {
            store4(out + hrow * kD + d0, o);
        } else {
            const size_t pr = hrow * max_parts + p;
            *reinterpret_cast<float4*>(ws_o + pr * kD + d0) = o;
            if (d0 == 0) {
                ws_m[pr] = M;
                ws_l[pr] = Ls;
            }
        }
    }
    if (pieces == 1) return;
    // The wait and barrier complete every published store before the counter moves;
    // the last piece to arrive reads all of them back (coherent loads) and merges them
    // in piece order, then leaves the counter at zero for the next call.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const int done = __hip_atomic_fetch_add(&counters[b * num_kv_heads + g], 1,
                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        S.last = done == pieces - 1;
    }
    __syncthreads();
    if (!uni(S.last)) return;
    T* rows = out + ((size_t)b * num_heads + (size_t)g * group) * kD;
    for (int i = tid; i < group * kCols; i += kThreads) {
        const int h = i / kCols, d0 = (i % kCols) * 4;
        float M = kNegInf, Ls = 0.f;
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
        for (int v = 0; v < pieces; ++v) {
            const int sl = rec0 + v * Part<GMAX>::kFloats;
            const float m = fetch1(R, 4 * (sl + Part<GMAX>::kM + h));
            const float l = fetch1(R, 4 * (sl + Part<GMAX>::kL + h));
            const float4 pv = fetch4(R, 4 * (sl + h * kD + d0));
            const float Mn = fmaxf(M, m);
            const float a = weight(M, Mn), c = weight(m, Mn);
            Ls = Ls * a + l * c;
            o.x = o.x * a + pv.x * c;
            o.y = o.y * a + pv.y * c;
            o.z = o.z * a + pv.z * c;
            o.w = o.w * a + pv.w * c;
            M = Mn;
        }
        const float inv = Ls > 0.f ? out_scale / Ls : 0.f;
        store4(rows + h * kD + d0, make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv));
    }
    if (tid == 0)
        __hip_atomic_store(&counters[b * num_kv_heads + g], 0, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ query chunks
// Several new query tokens per sequence: a prefill chunk, or draft tokens to verify in
// one pass. The query at position i attends tokens 1..i, read block by block ([P3]
// section "PagedAttention：逻辑连续，物理不必连续"). Sequence b's query rows
// query_start[b] .. query_start[b+1]-1 are its last T tokens, so its row j sits at
// position n - T + j of an n-token context.
//
// The 16 MFMA columns of a wave hold TQ = 16 / G query tokens times the G heads of one
// KV head: column c is token c / G, head c % G (a tile). Each lane masks the scores of
// its own column: token t of a block that starts at position s counts for column c
// when s + t <= (position of the tile's first row) + c / G. Two kernels spread a
// (sequence, KV head) over workgroups: chunk_split_kernel for short chunks (up to four
// tiles, e.g. draft verification) and chunk_tiles_kernel for long ones (prefill).
// Tables are staged in windows of kTabMax blocks, so the context length is not
// limited by LDS.
struct ChunkLds {
    uint32_t tile[kTabMax];
    uint8_t valid[kTabMax];
    KTile ktile[kWaves];
    float part[kWaves][Part<16>::kFloats];
};

// A wave's state -> normalised output rows for columns c < ncols, column c going to
// row row0 + (c / group) * num_heads + c % group.
template <typename T>
__device__ __forceinline__ void wave_to_rows(T* out, int row0, const WaveState& s, int lane,
                                             int ncols, int group, int num_heads,
                                             float out_scale) {
    const int c = lane & 15, grp = lane >> 4;
    const float ls = head_lsum(s);
    const float inv = ls > 0.f ? out_scale / ls : 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int h = 4 * grp + e;
        const float iv = __shfl(inv, h);
        if (h < ncols) {
            uint4 w;
            w.x = Mma<T>::pack(s.o[0][e] * iv, s.o[1][e] * iv);
            w.y = Mma<T>::pack(s.o[2][e] * iv, s.o[3][e] * iv);
            w.z = Mma<T>::pack(s.o[4][e] * iv, s.o[5][e] * iv);
            w.w = Mma<T>::pack(s.o[6][e] * iv, s.o[7][e] * iv);
            const size_t row = (size_t)row0 + (h / group) * num_heads + h % group;
            *reinterpret_cast<uint4*>(out + row * kD + 8 * c) = w;
        }
    }
}

// Rows of a workgroup whose rows all lie before the context: zero output. `row0` is
// the query/output row of column 0 and `ntok` the workgroup's query tokens.
template <typename T>
__device__ __forceinline__ void zero_rows(T* out, int row0, int ntok, int group, int num_heads,
                                          int tid) {
    constexpr int kCols = kD / 4;
    for (int i = tid; i < ntok * group * kCols; i += kThreads) {
        const int h = i / kCols;
        store4(out + ((size_t)row0 + (h / group) * num_heads + h % group) * kD + (i % kCols) * 4,
               make_float4(0.f, 0.f, 0.f, 0.f));
    }
}

// Table entries of blocks w0 .. w1-1 of sequence b into the workgroup's LDS window.
__device__ __forceinline__ void stage_window(uint32_t* tile, uint8_t* valid,
                                             const int32_t* __restrict__ tables, int b, int g,
                                             int n, int w0, int w1, int max_blocks,
                                             int num_blocks, int num_kv_heads, int tid) {
    for (int j = w0 + tid; j < w1; j += kThreads) {
        const int phys = tables[(size_t)b * max_blocks + j];
        const bool ok = phys >= 0 && phys < num_blocks;
        const int left = n - j * kBS;
        tile[j - w0] = ok ? (uint32_t)phys * (uint32_t)num_kv_heads + (uint32_t)g : kNoTile;
        valid[j - w0] = (uint8_t)(ok ? (left < kBS ? left : kBS) : 0);
    }
}

// Short chunks: one tile per workgroup; its waves take every fourth block and their
// pieces merge through LDS.
template <typename T, typename KV>
__global__ __launch_bounds__(kThreads) void chunk_split_kernel(
    T* __restrict__ out, const T* __restrict__ q, const typename KV::Elem* k_cache,
    const typename KV::Elem* v_cache, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ ctx_lens, const int32_t* __restrict__ query_start,
    float scale_log2, float out_scale, int num_query_tokens, int num_heads, int num_kv_heads,
    int group, int tq, int max_blocks, int num_blocks) {
    __shared__ ChunkLds S;
    const int g = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = uni(tid >> 6);
    // long contexts paired with short ones on a CU (paired_sequence)
    const int cap = max_blocks * kBS;
    int n = 0;
    const int b = paired_sequence(ctx_lens, gridDim.z, blockIdx.z, cap, lane, n);
    const int r0 = query_start[b], r1 = query_start[b + 1];
    // rows outside the query array or a decreasing start: nothing is read or written
    if (r0 < 0 || r1 < r0 || r1 > num_query_tokens) return;
    const int T_b = r1 - r0;
    const int tok0 = blockIdx.x * tq;
    if (tok0 >= T_b) return;
    const int ntok = min(tq, T_b - tok0);
    const int first = n - T_b + tok0;                   // position of the tile's first row
    const int nb = first + ntok - 1 < 0 ? 0 : (first + ntok - 1) / kBS + 1;
    const int ncols = ntok * group;
    const int row0 = (r0 + tok0) * num_heads + g * group;   // query/output row of column 0
    if (nb == 0) {
        zero_rows(out, row0, ntok, group, num_heads, tid);
        return;
    }
    // The lane's column: token ctok, head c % G. Columns past the tile (c >= ncols)
    // point past the query buffer and read zeros; they are never written.
    const int c = lane & 15, ctok = c / group;
    const int qlane = (ctok * num_heads + c % group) * kD * (int)sizeof(T);
    const int qbytes = ((ntok - 1) * num_heads + group) * kD * (int)sizeof(T);
    const int lim0 = first + ctok + 1;   // context tokens the lane's column sees

    WaveState st;
    reset(st);
    for (int w0 = 0; w0 < nb; w0 += kTabMax) {
        const int w1 = min(nb, w0 + kTabMax);
        __syncthreads();   // the previous window's entries are no longer read
        stage_window(S.tile, S.valid, tables, b, g, n, w0, w1, max_blocks, num_blocks,
                     num_kv_heads, tid);
        __syncthreads();
        // every step issues one block (a zero-record buffer past the window), so the
        // loads in flight never depend on the path taken
        auto issue = [&](typename KV::Regs& R, int ji) {
            KV::issue(R, k_cache, v_cache, q, ji < w1 ? S.tile[ji - w0] : kNoTile, row0,
                      qbytes, qlane, lane);
        };
        int j = w0 + wave;
        typename KV::Regs A, B;
        issue(A, j);
        issue_order();
        issue(B, j + kWaves);
#define PKV_STEP(R)                                                                          \
        if (j >= w1) break;                                                                  \
        {                                                                                    \
            const int vd = S.valid[j - w0];                                                  \
            int lim = lim0 - j * kBS;                                                        \
            lim = lim < 0 ? 0 : (lim > vd ? vd : lim);                                       \
            fold_block<T, KV>(st, R, S.ktile[wave], vd, lim, scale_log2, lane);              \
        }                                                                                    \
        issue(R, j + 2 * kWaves);                                                            \
        j += kWaves;
        while (true) {
            PKV_STEP(A)
            PKV_STEP(B)
        }
#undef PKV_STEP
    }
    wave_to_part<16>(S.part[wave], st, lane, ncols);
    __syncthreads();
    int P[kWaves];
    for (int v = 0; v < kWaves; ++v) P[v] = v;
    constexpr int kCols = kD / 4;
    for (int i = tid; i < ncols * kCols; i += kThreads) {
        const int h = i / kCols, d0 = (i % kCols) * 4;
        float M, Ls;
        float4 o;
        merge_parts<16, kWaves, kWaves>(S.part, P, kWaves, h, d0, M, Ls, o);
        const float inv = Ls > 0.f ? out_scale / Ls : 0.f;
        store4(out + ((size_t)row0 + (h / group) * num_heads + h % group) * kD + d0,
               make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv));
    }
}

// ------------------------------------------------------------------ shared prefixes
// Sequences that share their leading blocks (the samples of one prompt, forked from it:
// [P1] section 五, [P3] section "共享前缀和 copy-on-write") can be decoded as groups:
// consecutive sequences group_start[i] .. group_start[i+1]-1 whose first
// group_prefix[i] table entries are the same physical blocks. The members of a group are
// the columns of the matrix-core tiles: a tile holds mpt = 16 / G members (column c:
// member c / G of the tile, head c % G, as the query chunks lay out their tokens), and
// each column is masked to its own context. A tile's workgroup reads each prefix block
// once for all of its members, then each member's own blocks (columns of other members
// masked), so a block shared by the group is read once per tile instead of once per
// member. A prefix longer than kGroupPart blocks is cut into parts, one workgroup each;
// the last part also takes the members' own blocks. A group of one part writes its
// output directly; otherwise each part leaves a log-sum-exp record (m, l, unnormalised
// o) per (member, query head) and group_merge_kernel combines them.
//
// A member's share of the prefix is prefix_blocks(): the group's prefix, but never the
// block of its newest token when the step appends it (the workgroup writes that token
// first, so it must read the block after the write), and never past its context.
__device__ __forceinline__ int prefix_blocks(int pfx, int n, int appending) {
    if (n <= 0) return 0;
    const int own = appending ? (n - 1) / kBS : (n + kBS - 1) / kBS;
    return pfx < own ? pfx : own;
}

// Table entries a tile's workgroup stages at a time: its list of blocks (the part's
// prefix blocks, then each member's own blocks) goes through LDS in windows.
constexpr int kGroupWindow = 1024;
// Tiles (of 16 columns) a workgroup folds every prefix block into, and its waves.
constexpr int kGroupTiles = kGroupTilesPerWorkgroup;
constexpr int kGroupWaves = 4;
// Most members of one workgroup (16 columns per tile, at least one column per member).
constexpr int kGroupMembers = 16 * kGroupTiles;
static_assert(kGroupMembers <= 64, "members of a workgroup are the lanes of one wave");

template <int NW>
struct GroupLds {
    uint32_t tile[kGroupWindow];
    uint8_t valid[kGroupWindow];
    int8_t owner[kGroupWindow];   // -1: a prefix block; else the member (in the workgroup) it belongs to
    int priv[kGroupMembers + 1];  // members' own blocks, exclusive prefix sums
    int mn[kGroupMembers];        // members' context lengths
    int me[kGroupMembers];        // and prefix shares
    KTile ktile[NW];
    float part[NW][Part<16>::kFloats];
};

// One-dimensional grid over (tile set, unit), a unit being (part, KV head, group): unit
// u = part + parts * (g + Hkv * group index), units padded to a multiple of 8. Each
// workgroup takes NT tiles of a group (NT * mpt members): its waves fold every staged
// prefix block into all NT tiles (the K and V registers shared) and each member's own
// block into that member's tile. Workgroup L takes tile set (L / 8) % sets of unit
// (L / 8 / sets) * 8 + L % 8, so the tile sets of one unit sit 8 workgroups apart in
// dispatch order, which places them on one XCD (workgroups go to the XCDs in turn):
// all but the first read the prefix blocks from that XCD's L2.
template <typename T, typename KV, int NT, int NW>
__global__ __launch_bounds__(64 * NW) void group_tile_kernel(
    T* __restrict__ out, const T* __restrict__ q, typename KV::Elem* k_cache,
    typename KV::Elem* v_cache, const T* __restrict__ new_k, const T* __restrict__ new_v,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ ctx_lens,
    const int32_t* __restrict__ group_start, const int32_t* __restrict__ group_prefix,
    float scale_log2, float out_scale, float k_inv, float v_inv, int num_seqs, int num_heads,
    int num_kv_heads, int group, int mpt, int sets, int units, int max_blocks,
    int num_blocks, int max_prefix, int parts_max, int32_t* __restrict__ seq_prefix,
    float* __restrict__ rec_m, float* __restrict__ rec_l, float* __restrict__ rec_o) {
    __shared__ GroupLds<NW> S;
    constexpr int kT = 64 * NW;
    const int L = blockIdx.x, hi = L >> 3;
    const int set = hi % sets, u = (hi / sets) * 8 + (L & 7);
    if (u >= units) return;
    const int part = u % parts_max, g = (u / parts_max) % num_kv_heads;
    const int gi = u / parts_max / num_kv_heads;
    const int tid = threadIdx.x, lane = tid & 63, wave = uni(tid >> 6);
    const int s0 = uni(group_start[gi]), s1 = uni(group_start[gi + 1]);
    // a group outside the batch or with a decreasing start: nothing is read or written
    if (s0 < 0 || s1 < s0 || s1 > num_seqs) return;
    const int k = s1 - s0;
    int pfx = uni(group_prefix[gi]);
    pfx = pfx < 0 ? 0 : (pfx > max_prefix ? max_prefix : pfx);
    const int parts = pfx > 0 ? (pfx + kGroupPart - 1) / kGroupPart : 1;
    // the merge kernel learns each member's prefix
    if (seq_prefix != nullptr && part == 0 && g == 0 && set == 0)
        for (int m = tid; m < k; m += kT) seq_prefix[s0 + m] = pfx;
    const int m0 = set * NT * mpt;   // the workgroup's first member
    if (part >= parts || m0 >= k) return;
    const int nm = min(NT * mpt, k - m0);    // members of this workgroup
    const int nt = (nm + mpt - 1) / mpt;     // tiles holding them
    const bool last = part == parts - 1;
    const int appending = new_k != nullptr;
    const int cap = max_blocks * kBS;
    // members' lengths, prefix shares and (last part) own block counts
    if (wave == 0) {
        int n = 0, e = 0, own = 0;
        if (lane < nm) {
            n = ctx_lens[s0 + m0 + lane];
            n = n < 0 ? 0 : (n > cap ? cap : n);
            e = prefix_blocks(pfx, n, appending);
            own = last ? (n + kBS - 1) / kBS - e : 0;
        }
        int incl = own;   // inclusive prefix sum over the lanes
#pragma unroll
        for (int d = 1; d < kGroupMembers; d <<= 1) {
            const int y = __shfl_up(incl, d);
            if (lane >= d) incl += y;
        }
        if (lane < kGroupMembers) {
            S.mn[lane] = n;
            S.me[lane] = e;
            S.priv[lane + 1] = incl;
        }
        if (lane == 0) S.priv[0] = 0;
    }
    // fused append (last part): each member's newest row, before any block is read
    if (appending && last)
        for (int i = tid; i < nm * 2 * KV::kAppendChunks; i += kT) {
            const int mi = i / (2 * KV::kAppendChunks), r = i % (2 * KV::kAppendChunks);
            const int b = s0 + m0 + mi;
            int n = ctx_lens[b];
            n = n < 0 ? 0 : (n > cap ? cap : n);
            if (n > 0)
                KV::append(k_cache, v_cache, new_k, new_v, tables + (size_t)b * max_blocks, b, g,
                           num_kv_heads, n, num_blocks, r / KV::kAppendChunks,
                           r % KV::kAppendChunks, k_inv, v_inv);
        }
    __syncthreads();
    // The lane's column in tile t: member t * mpt + c / G of the workgroup, head c % G.
    // Columns past the members point past their query rows and read zeros; they are
    // never written.
    const int c = lane & 15, cm = c / group;
    const int row0 = (s0 + m0) * num_heads + g * group;   // query row of member 0, head 0
    int lim0[NT];     // prefix tokens the lane's column of tile t attends
    uint4 qv[NT][4];  // its query, loaded once
    int pmax = 0;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int mi = t * mpt + cm;
        const bool live = c < mpt * group && mi < nm;
        lim0[t] = live ? min(S.mn[mi], S.me[mi] * kBS) : 0;
        pmax = max(pmax, lim0[t]);
        const int tm = min(mpt, max(0, nm - t * mpt));   // members of tile t
        const int qrow = row0 + t * mpt * num_heads;
        const int qbytes = tm > 0 ? ((tm - 1) * num_heads + group) * kD * (int)sizeof(T) : 0;
        issue_query(qv[t], q, qrow, qbytes, (cm * num_heads + c % group) * kD * (int)sizeof(T),
                    lane);
    }
    // prefix blocks of this part that some column attends; slots past all of them are
    // cleared like the slots past a context (they may never have been written)
    const int nmax = wave_max(pmax);
    const int j0 = part * kGroupPart;
    const int np = max(0, min(min(pfx, j0 + kGroupPart), (nmax + kBS - 1) / kBS) - j0);
    const int total = np + uni(S.priv[nm]);
    WaveState st[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) reset(st[t]);
    for (int w0 = 0; w0 < total; w0 += kGroupWindow) {
        const int w1 = min(total, w0 + kGroupWindow);
        __syncthreads();   // the previous window's entries are no longer read
        for (int x = w0 + tid; x < w1; x += kT) {
            int b, j, n, own = -1;
            if (x < np) {   // a prefix block, from the first member's table
                b = s0;
                j = j0 + x;
                n = nmax;
            } else {        // member own's block
                const int y = x - np;
                own = 0;
                while (own < nm - 1 && S.priv[own + 1] <= y) ++own;
                b = s0 + m0 + own;
                j = S.me[own] + (y - S.priv[own]);
                n = S.mn[own];
            }
            const int phys = tables[(size_t)b * max_blocks + j];
            const bool ok = phys >= 0 && phys < num_blocks;
            const int left = n - j * kBS;
            S.tile[x - w0] = ok ? (uint32_t)phys * (uint32_t)num_kv_heads + (uint32_t)g : kNoTile;
            S.valid[x - w0] = (uint8_t)(ok ? (left < kBS ? left : kBS) : 0);
            S.owner[x - w0] = (int8_t)own;
        }
        __syncthreads();
        // every step issues one block (a zero-record buffer past the window)
        auto issue = [&](typename KV::Regs& R, int xi) {
            KV::template issue<kStream, false>(R, k_cache, v_cache, q,
                                               xi < w1 ? S.tile[xi - w0] : kNoTile, 0, 0, 0,
                                               lane);
        };
        int x = w0 + wave;
        typename KV::Regs A, B;
        issue(A, x);
        issue_order();
        issue(B, x + NW);
#define PKV_STEP(R)                                                                          \
        if (x >= w1) break;                                                                  \
        {                                                                                    \
            const int vd = S.valid[x - w0], ow = uni(S.owner[x - w0]);                       \
            uint4 ka[4], v[4];                                                               \
            stage_block<T, KV>(R, S.ktile[wave], vd, lane, ka, v);                           \
            _Pragma("unroll") for (int t = 0; t < NT; ++t) {                                 \
                if (t >= nt) break;                                                          \
                int lim;                                                                     \
                if (ow < 0) {                                                                \
                    lim = lim0[t] - (j0 + x) * kBS;                                          \
                    lim = lim < 0 ? 0 : (lim > vd ? vd : lim);                               \
                } else {                                                                     \
                    if (ow / mpt != t) continue;                                             \
                    lim = (c < mpt * group && t * mpt + cm == ow) ? vd : 0;                  \
                }                                                                            \
                fold_tile<T>(st[t], ka, qv[t], v, lim, scale_log2, lane);                    \
            }                                                                                \
        }                                                                                    \
        issue(R, x + 2 * NW);                                                            \
        x += NW;
        while (true) {
            PKV_STEP(A)
            PKV_STEP(B)
        }
#undef PKV_STEP
    }
    int P[NW];
    for (int v = 0; v < NW; ++v) P[v] = v;
    constexpr int kCols = kD / 4;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if (t >= nt) break;
        const int ncols = min(mpt, nm - t * mpt) * group;
        if (t > 0) __syncthreads();   // the previous tile's records are no longer read
        wave_to_part<16>(S.part[wave], st[t], lane, ncols);
        __syncthreads();
        for (int i = tid; i < ncols * kCols; i += kT) {
            const int h = i / kCols, d0 = (i % kCols) * 4;
            float M, Ls;
            float4 o;
            merge_parts<16, NW, NW>(S.part, P, NW, h, d0, M, Ls, o);
            const size_t row =
                (size_t)row0 + (t * mpt + h / group) * num_heads + h % group;
            if (parts == 1) {
                const float inv = Ls > 0.f ? out_scale / Ls : 0.f;
                store4(out + row * kD + d0,
                       make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv));
            } else {
                const size_t r = row * parts_max + part;
                *reinterpret_cast<float4*>(rec_o + r * kD + d0) = o;
                if (d0 == 0) {
                    rec_m[r] = M;
                    rec_l[r] = Ls;
                }
            }
        }
    }
}

// Output rows of the members of groups with several prefix parts: the parts' records
// merged in part order, normalised. One thread per (query row, four dims).
template <typename T>
__global__ __launch_bounds__(kThreads) void group_merge_kernel(
    T* __restrict__ out, const int32_t* __restrict__ seq_prefix, const float* __restrict__ rec_m,
    const float* __restrict__ rec_l, const float* __restrict__ rec_o, float out_scale,
    int num_rows, int num_heads, int max_prefix, int parts_max) {
    constexpr int kCols = kD / 4;
    const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
    if (i >= (long long)num_rows * kCols) return;
    const int row = (int)(i / kCols), d0 = (int)(i % kCols) * 4;
    int pfx = seq_prefix[row / num_heads];
    pfx = pfx < 0 ? 0 : (pfx > max_prefix ? max_prefix : pfx);
    const int parts = (pfx + kGroupPart - 1) / kGroupPart;
    if (parts <= 1) return;   // written by the tile kernel
    float M = kNegInf, Ls = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int p = 0; p < parts; ++p) {
        const size_t r = (size_t)row * parts_max + p;
        const float m = rec_m[r], l = rec_l[r];
        const float4 v = *reinterpret_cast<const float4*>(rec_o + r * kD + d0);
        const float Mn = fmaxf(M, m);
        const float a = weight(M, Mn), cw = weight(m, Mn);
        Ls = Ls * a + l * cw;
        o.x = o.x * a + v.x * cw;
        o.y = o.y * a + v.y * cw;
        o.z = o.z * a + v.z * cw;
        o.w = o.w * a + v.w * cw;
        M = Mn;
    }
    const float inv = Ls > 0.f ? out_scale / Ls : 0.f;
    store4(out + (size_t)row * kD + d0, make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv));
}

// ------------------------------------------------------------------ prefill chunks
// Long chunks on 32x32 matrix-core tiles, flash-attention style. A workgroup takes
// 4 x 32 query rows of one (sequence, KV head): each wave 32 rows, row r being query
// token r / G and head r % G of the wave's tokens. Each step brings 32 context tokens
// (two blocks) into LDS once for all four waves, straight from HBM (buffer loads that
// write LDS), K and V both row-major with their 16-byte chunks permuted per token; the
// PV operand comes from transposing LDS reads. Per step and wave:
//   S^T = K Q^T  (32 tokens x 32 rows, eight 32x32x16 products; Q stays in registers)
//   online softmax per row: a lane's column is its row, so the max and the rescale of
//   the accumulator stay in the lane (one exchange with the lane 32 apart)
//   O^T += V^T P^T  (128 dims x 32 rows, eight 32x32x16 products; P^T is the score
//   tile's own register layout)
// The 32x32 layouts (checked on gfx950): A holds row l%32, k = K/2*(l/32) .. ; B holds
// column l%32, the same k; D element v of lane l is row 8(v/4) + 4(l/32) + v%4, column
// l%32. Slots past the context are loaded as zeros (a zero weight does not cancel a
// NaN) and masked in S.
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <typename T> struct Mma32;
template <> struct Mma32<bf16_t> {
    static __device__ __forceinline__ f32x16_t mma(const uint4& a, const uint4& b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                      __builtin_bit_cast(bf16x8_t, b), c, 0, 0,
                                                      0);
    }
};
template <> struct Mma32<f16_t> {
    static __device__ __forceinline__ f32x16_t mma(const uint4& a, const uint4& b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                     __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
};

constexpr int kFaRows = 32;      // query rows per wave (the 32 columns of S^T)
constexpr int kFaStep = 32;      // context tokens per step: two blocks of 16
constexpr int kFaRing = 3;       // LDS slots: the step being multiplied and two in flight
constexpr int kFaTab = 512;      // table entries staged per window (256 steps)
// Largest sum of one lane's 16 weights of a step that stands: every weight then lies
// below it (weights are not negative), and the final division cancels the reference the
// weights are taken against.
constexpr float kFaBound = 256.f;

// Batches up to this many sequences run their heaviest work first (see chunk_fa_kernel).
constexpr int kFaSortMax = kFaTab;

// K and V rows of a step in LDS, both [token][16-byte chunk] with the chunks of a row
// permuted: K chunk c of token t sits at c ^ (t % 16) (the 16-byte score-operand reads
// of 32 tokens hit distinct banks), V chunk c at c ^ 4 (t % 4) (the transposing 8-byte
// reads of the PV operand, four tokens x 32 dims per half-wave, hit distinct banks).
struct FaLds {
    uint32_t tile[kFaTab];
    int seq;
    uint4 k[kFaRing][kFaStep][kD / 8];
    uint4 v[kFaRing][kFaStep][kD / 8];
};

// 16 bytes per lane from a raw buffer straight into LDS: lane l writes lds_addr + 16 l
// (gfx950). Written as assembly so that the compiler's wait insertion does not treat
// every later LDS read as dependent on it (that would drain all loads in flight); the
// code orders it with explicit vector-memory counter waits and barriers instead. M0
// holds the LDS address and needs one wait state before the load; the leading five
// wait states cover descriptor words just written by v_readfirstlane (the compiler's
// hazard checks do not look inside assembly). M0 is a register the compiler reserves,
// so the statement leaves it as it found it: the old value is kept in a scalar
// temporary and put back after the load has issued (the load takes its LDS address at
// issue), followed by one wait state for any M0 reader the compiler places next.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void lds_load16(i32x4_t rsrc, uint32_t lds_addr, int voffset) {
    uint32_t saved_m0;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_nop 4\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0"
        : "=&s"(saved_m0)
        : "s"(lds_addr), "v"(voffset), "s"(rsrc)
        : "memory");
}
// A raw buffer descriptor (stride 0, num_records bytes) as four scalar words.
__device__ __forceinline__ i32x4_t raw_rsrc_words(const void* base, int bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4_t w;
    w.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    w.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xffff);
    w.z = __builtin_amdgcn_readfirstlane(bytes);
    w.w = kRawBufferWord3;
    return w;
}
__device__ __forceinline__ uint32_t lds_address(const void* p) {
    return (uint32_t)reinterpret_cast<uintptr_t>(
        (const __attribute__((address_space(3))) void*)p);
}
// Workgroup barrier that orders memory operations in the compiler only; the waits that
// the data needs are explicit before it.
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmem() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <typename T>
__global__ __launch_bounds__(kThreads) void chunk_fa_kernel(
    T* __restrict__ out, const T* __restrict__ q, const T* __restrict__ k_cache,
    const T* __restrict__ v_cache, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ ctx_lens, const int32_t* __restrict__ query_start,
    float scale_log2, int num_query_tokens, int num_heads, int num_kv_heads, int group,
    int max_blocks, int num_blocks, int groups) {
    __shared__ FaLds S;
    // (sequence, KV head) pair p with all its row groups on XCD p % 8 (see
    // chunk_tiles_kernel)
    const int pairs = gridDim.x / groups;
    int pair, sg;
    if (pairs % 8 == 0) {
        const int x = blockIdx.x % 8, k = blockIdx.x / 8;
        pair = x + 8 * (k / groups);
        sg = k % groups;
    } else {
        pair = blockIdx.x / groups;
        sg = blockIdx.x % groups;
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = uni(tid >> 6);
    // Heaviest work first, so that the longest workgroups do not start last: pair ranks
    // go to the sequences in decreasing order of context length (ties by index), and a
    // pair's row groups run from the last (which sees the most context) to the first.
    // Every workgroup ranks the context lengths itself (staged in LDS).
    const int nseq = pairs / num_kv_heads, g = pair % num_kv_heads;
    int b = pair / num_kv_heads;
    sg = groups - 1 - sg;
    if (nseq <= kFaSortMax) {
        const int cap0 = max_blocks * kBS;
        for (int u = tid; u < nseq; u += kThreads) {
            const int x = ctx_lens[u];
            S.tile[u] = (uint32_t)(x < 0 ? 0 : (x > cap0 ? cap0 : x));
        }
        __syncthreads();
        for (int u = tid; u < nseq; u += kThreads) {
            const uint32_t key = S.tile[u];
            int rank = 0;
            for (int v = 0; v < nseq; ++v) {
                const uint32_t kv = S.tile[v];
                rank += (kv > key || (kv == key && v < u)) ? 1 : 0;
            }
            if (rank == b) S.seq = u;
        }
        __syncthreads();
        b = S.seq;
    }
    // b and everything derived from it are wave-uniform; saying so lets the compiler
    // branch on them (the causal mask below is then skipped outright on whole steps)
    b = uni(b);
    const int r0 = uni(query_start[b]), r1 = uni(query_start[b + 1]);
    if (r0 < 0 || r1 < r0 || r1 > num_query_tokens) return;
    const int T_b = r1 - r0;
    const int tqw = kFaRows / group;                 // query tokens per wave
    const int tok_wg = sg * kWaves * tqw;
    if (tok_wg >= T_b) return;
    const int cap = max_blocks * kBS;
    int n = uni(ctx_lens[b]);
    n = n < 0 ? 0 : (n > cap ? cap : n);
    const int ntok_wg = min(kWaves * tqw, T_b - tok_wg);
    const int last_wg = n - T_b + tok_wg + ntok_wg - 1;   // position of the last row
    if (last_wg < 0) {
        zero_rows(out, (r0 + tok_wg) * num_heads + g * group, ntok_wg, group, num_heads, tid);
        return;
    }
    const int steps = last_wg / kFaStep + 1;
    const int nb_ctx = (n + kBS - 1) / kBS;
    const int h = lane >> 5, r = lane & 31;
    const int tok_w = tok_wg + wave * tqw;           // this wave's first query token
    const int rtok = r / group, rhead = r % group;
    const bool row_ok = r < tqw * group && tok_w + rtok < T_b;
    const int pos = n - T_b + tok_w + rtok;          // the lane's row position
    const int last_w = n - T_b + min(T_b, tok_w + tqw) - 1;   // the wave's last row

    // the lane's query row, dims 16s + 8h .. +7 for k-step s (zeros past the chunk)
    uint4 qv[kD / 16];
    {
        const int qbytes = (r1 - r0) * num_heads * kD * (int)sizeof(T);
        const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(q + (size_t)r0 * num_heads * kD), 0, qbytes, kRawBufferWord3);
        const int qoff = row_ok
            ? (((tok_w + rtok) * num_heads + g * group + rhead) * kD + 8 * h) * (int)sizeof(T)
            : qbytes;
#pragma unroll
        for (int s = 0; s < kD / 16; ++s)
            qv[s] = buffer_load16(rq, qoff + 16 * s * (int)sizeof(T));
    }
    f32x16_t acc[kD / 32];
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt) acc[dt] = f32x16_t{};
    float m = kNegInf, lsum = 0.f;

    // Global -> LDS without registers: buffer loads that write LDS directly, lane l of a
    // wave to the wave's LDS base + 16 l. For block bi of a step, thread tid fills row
    // bi * 16 + tid / 16, position tid % 16, so it fetches the chunk that the row's
    // permutation puts there. A block's descriptor covers only its tokens inside the
    // context (none for a missing block): loads past it write zeros, which keeps
    // anything beyond the context out of the PV products (a zero weight does not cancel
    // a NaN).
    int w0 = 0, w1 = 0;
    const int tt = tid / 16, tc = tid % 16;
    const int koff = (tt * (kD / 8) + (tc ^ tt)) * 16;
    const int voff = (tt * (kD / 8) + (tc ^ (4 * (tt % 4)))) * 16;
    auto issue = [&](int st, auto slot) {
        constexpr int sl = decltype(slot)::value;
#pragma unroll
        for (int bi = 0; bi < 2; ++bi) {
            const int jb = 2 * st + bi;
            const uint32_t tl = uni(jb < w1 ? (int)S.tile[jb - w0] : (int)kNoTile);
            const int nv = min(kBS, max(0, n - jb * kBS));
            const bool ok = tl != kNoTile;
            const size_t base = (size_t)(ok ? tl : 0u) * kTile;
            const int bytes = ok ? nv * kD * (int)sizeof(T) : 0;
            lds_load16(raw_rsrc_words(k_cache + base, bytes),
                       uni(lds_address(&S.k[sl][bi * kBS + 4 * wave][0])), koff);
            lds_load16(raw_rsrc_words(v_cache + base, bytes),
                       uni(lds_address(&S.v[sl][bi * kBS + 4 * wave][0])), voff);
        }
    };
    // PV operand reads: ds_read_tr16_b64 gives lane m of each 16-lane group element j of
    // source lane 4j + m / 4 at position m % 4. Source lane 4j + q of group G points at
    // token 16s + 8e + 4h + j, dims 32dt + 16(G % 2) + 4q .. +3, so lane m receives dim
    // 32dt + 16(G % 2) + m = 32dt + lane % 32 of tokens 16s + 8e + 4h + 0..3: the row and
    // k order of the score registers that form the other operand.
    const int tj = (lane % 16) / 4, tq = lane % 4, tg = (lane / 16) % 2;
    auto v_operand = [&](auto slot, int s, int dt) {
        constexpr int sl = decltype(slot)::value;
        uint2 part[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int tok = 16 * s + 8 * e + 4 * h + tj;
            const int chunk = (4 * dt + 2 * tg + tq / 2) ^ (4 * tj);
            const char* p = reinterpret_cast<const char*>(&S.v[sl][tok][chunk]) + 8 * (tq % 2);
            part[e] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4_t*)(p)));
        }
        return make_uint4(part[0].x, part[0].y, part[1].x, part[1].y);
    };
    auto compute = [&](int st, auto slot) {
        constexpr int sl = decltype(slot)::value;
        const int tp0 = st * kFaStep;
        if (tp0 > last_w) return;                    // none of the wave's rows sees it
        f32x16_t sc = f32x16_t{};
#pragma unroll
        for (int s = 0; s < kD / 16; ++s)
            sc = Mma32<T>::mma(S.k[sl][r][(2 * s + h) ^ (r & 15)], qv[s], sc);
        // The VALU, not the matrix cores, bounds this loop (a wave64 VALU op takes four
        // cycles): steps that every row of the wave sees whole skip the mask, the scale
        // enters through one FMA before the exp, and no step takes a row maximum unless
        // its weights fail the bound below.
        const bool whole = tp0 + kFaStep - 1 <= n - T_b + tok_w && tp0 + kFaStep <= n;
        if (!whole) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int tp = tp0 + 8 * (v / 4) + 4 * h + (v % 4);
                sc[v] = (tp <= pos && tp < n) ? sc[v] : kNegInf;
            }
        }
        // Weights against the row's reference m, and the row sum that adds them as
        // rounded for the PV product (a dot product with ones per packed pair: half the
        // instructions of the float adds), so that the numerator and the denominator
        // see the same weights. Two partial sums keep the chain short.
        uint2 pb[4];
        float ps;
        auto weights = [&](float mu) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                float p[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    p[e] = fast_exp2(__builtin_fmaf(sc[4 * s + e], scale_log2, -mu));
                pb[s] = make_uint2(Mma<T>::pack(p[0], p[1]), Mma<T>::pack(p[2], p[3]));
            }
            float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                ps0 = Mma<T>::add_pair(pb[s].x, ps0);
                ps1 = Mma<T>::add_pair(pb[s].y, ps1);
            }
            ps = ps0 + ps1;
        };
        weights(m);
        // A lane's sum bounds each of its weights, so a sum within kFaBound keeps them
        // all below it without a maximum. It fails (also as infinity or NaN, on a row's
        // first step, where m = -inf) when some score passes m by more than
        // log2(kFaBound / 16): then m moves to the row's maximum, the accumulator and
        // sum are rescaled, and the weights are taken again. None of them then exceeds
        // 1 (up to rounding), so the second pass stands. A row that sees no token (m
        // still -inf: its position lies before the context, which is shorter than the
        // chunk) takes its weights against 0, so that its masked scores give zeros
        // instead of NaN.
        if (__any(!(ps <= kFaBound))) {
            float mraw = kNegInf;
#pragma unroll
            for (int v = 0; v < 16; ++v) mraw = fmaxf(mraw, sc[v]);
            const float mn = fmaxf(m, max_xor32(mraw) * scale_log2);
            const float alpha = (m == kNegInf) ? 0.f : fast_exp2(m - mn);
            lsum *= alpha;
#pragma unroll
            for (int dt = 0; dt < kD / 32; ++dt) acc[dt] *= alpha;
            m = mn;
            weights(m == kNegInf ? 0.f : m);
        }
        lsum += ps;
        // PV on 32x32x16 products over 16 tokens each. The k order inside a product is
        // free as long as both operands use it: lane l supplies its own score registers
        // (tokens 16s + 4h + 0..3 and 16s + 8 + 4h + 0..3), and the V operand is read in
        // the same order.
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const uint4 pbk = make_uint4(pb[2 * s].x, pb[2 * s].y, pb[2 * s + 1].x, pb[2 * s + 1].y);
#pragma unroll
            for (int dt = 0; dt < kD / 32; ++dt)
                acc[dt] = Mma32<T>::mma(v_operand(slot, s, dt), pbk, acc[dt]);
        }
    };

    // Per table window: the loads of step st + kFaRing - 1 go out once every wave is past
    // step st - 1 (whose slot they refill), so kFaRing - 1 steps are in flight while
    // step st is computed; one barrier per step. The vector-memory counter wait before
    // the barrier leaves the loads of later steps (four per thread and step) in flight.
    const int nbl = 2 * steps;                       // blocks the steps cover
    static_assert(kFaRing == 3, "the waits below assume one later step in flight");
    for (w0 = 0; w0 < nbl; w0 += kFaTab) {
        w1 = min(nbl, w0 + kFaTab);
        __syncthreads();                             // the previous window is done
        for (int j = w0 + tid; j < w1; j += kThreads) {
            int phys = j < nb_ctx ? tables[(size_t)b * max_blocks + j] : -1;
            const bool ok = phys >= 0 && phys < num_blocks;
            S.tile[j - w0] = ok ? (uint32_t)phys * (uint32_t)num_kv_heads + (uint32_t)g
                                : kNoTile;
        }
        // no load of the compiler's own (the query row, the table) may be outstanding
        // in the loop below, or its waits would also drain the LDS loads in flight
        wait_vmem<0>();
        __syncthreads();
        const int s0 = w0 / 2, ns = w1 / 2 - s0;
        using Slot0 = std::integral_constant<int, 0>;
        using Slot1 = std::integral_constant<int, 1>;
        using Slot2 = std::integral_constant<int, 2>;
        issue(s0, Slot0{});
        if (1 < ns) issue(s0 + 1, Slot1{});
        // step i computes from slot i % 3 and refills slot (i + 2) % 3; the loop is
        // unrolled over the three slots so that every LDS address is a constant offset
        auto step = [&](int i, auto slot, auto refill) {
            if (i + 1 < ns) wait_vmem<4>(); else wait_vmem<0>();
            barrier_only();
            if (i + 2 < ns) issue(s0 + i + 2, refill);
            compute(s0 + i, slot);
        };
        for (int i = 0; i < ns; i += 3) {
            step(i, Slot0{}, Slot2{});
            if (i + 1 < ns) step(i + 1, Slot1{}, Slot0{});
            if (i + 2 < ns) step(i + 2, Slot2{}, Slot1{});
        }
    }
    const float lt = sum_xor32(lsum);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (row_ok) {
        T* orow = out + ((size_t)(r0 + tok_w + rtok) * num_heads + g * group + rhead) * kD;
#pragma unroll
        for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                uint2 w;
                w.x = Mma<T>::pack(acc[dt][4 * q4] * inv, acc[dt][4 * q4 + 1] * inv);
                w.y = Mma<T>::pack(acc[dt][4 * q4 + 2] * inv, acc[dt][4 * q4 + 3] * inv);
                *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * q4 + 4 * h) = w;
            }
    }
}

// Register buffers per wave in chunk_tiles_kernel (its loads mostly hit L2).
constexpr int kChunkRing = 2;

// Long chunks: each wave owns NT consecutive tiles (NT * TQ tokens) and streams every
// block its last row sees. A block is staged once (K through LDS into operand order, V
// widened) and folded into all NT tiles; the queries stay in registers. The four waves
// of a workgroup take consecutive spans and read the same lines close together in time
// (cached loads: the lines are also reused by the sequence's other workgroups).
struct ChunkTilesLds {
    uint32_t tile[kTabMax];
    uint8_t valid[kTabMax];
    KTile ktile[kWaves];
};

template <typename T, typename KV, int NT>
__global__ __launch_bounds__(kThreads) void chunk_tiles_kernel(
    T* __restrict__ out, const T* __restrict__ q, const typename KV::Elem* k_cache,
    const typename KV::Elem* v_cache, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ ctx_lens, const int32_t* __restrict__ query_start,
    float scale_log2, float out_scale, int num_query_tokens, int num_heads, int num_kv_heads,
    int group, int tq, int max_blocks, int num_blocks, int groups) {
    __shared__ ChunkTilesLds S;
    // One-dimensional grid over (sequence, KV head) pairs times span groups. The
    // dispatcher deals workgroups round-robin over the 8 XCDs (workgroup i to XCD i % 8).
    // Pair p goes to XCD p % 8 with all its span groups, so the workgroups that read the
    // same lines share one L2, and every XCD gets a mix of sequences.
    const int pairs = gridDim.x / groups;                   // num_seqs * Hkv
    int pair, sg;
    if (pairs % 8 == 0) {
        const int x = blockIdx.x % 8, k = blockIdx.x / 8;
        pair = x + 8 * (k / groups);
        sg = k % groups;
    } else {
        pair = blockIdx.x / groups;
        sg = blockIdx.x % groups;
    }
    const int g = pair % num_kv_heads, b = pair / num_kv_heads;
    const int tid = threadIdx.x, lane = tid & 63, wave = uni(tid >> 6);
    const int r0 = query_start[b], r1 = query_start[b + 1];
    if (r0 < 0 || r1 < r0 || r1 > num_query_tokens) return;
    const int T_b = r1 - r0;
    const int span = NT * tq;                               // tokens per wave
    const int tok_wg = sg * kWaves * span;
    if (tok_wg >= T_b) return;
    const int cap = max_blocks * kBS;
    int n = ctx_lens[b];
    n = n < 0 ? 0 : (n > cap ? cap : n);
    const int ntok_wg = min(kWaves * span, T_b - tok_wg);
    const int last_wg = n - T_b + tok_wg + ntok_wg - 1;   // position of the last row
    const int nb_wg = last_wg < 0 ? 0 : last_wg / kBS + 1;
    if (nb_wg == 0) {
        zero_rows(out, (r0 + tok_wg) * num_heads + g * group, ntok_wg, group, num_heads, tid);
        return;
    }
    const int tok_w = tok_wg + wave * span;                 // this wave's first token
    const int ntok_w = max(0, min(span, T_b - tok_w));
    const int last_w = n - T_b + tok_w + ntok_w - 1;
    const int nb_w = (ntok_w == 0 || last_w < 0) ? 0 : last_w / kBS + 1;
    const int c = lane & 15, ctok = c / group;
    const int qlane = (ctok * num_heads + c % group) * kD * (int)sizeof(T);
    uint4 qv[NT][4];
    WaveState st[NT];
    int lim0[NT], row0[NT], ncols[NT], tlast[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int tok0 = tok_w + t * tq;
        const int ntok = max(0, min(tq, T_b - tok0));
        row0[t] = (r0 + tok0) * num_heads + g * group;
        ncols[t] = ntok * group;
        lim0[t] = n - T_b + tok0 + ctok + 1;
        tlast[t] = ntok > 0 ? n - T_b + tok0 + ntok - 1 : -1;   // the tile's last position
        issue_query(qv[t], q, ntok > 0 ? row0[t] : 0,
                    ntok > 0 ? ((ntok - 1) * num_heads + group) * kD * (int)sizeof(T) : 0,
                    qlane, lane);
        reset(st[t]);
    }
    for (int w0 = 0; w0 < nb_wg; w0 += kTabMax) {
        const int w1 = min(nb_wg, w0 + kTabMax);
        __syncthreads();
        stage_window(S.tile, S.valid, tables, b, g, n, w0, w1, max_blocks, num_blocks,
                     num_kv_heads, tid);
        __syncthreads();
        const int jend = min(w1, nb_w);
        auto issue = [&](typename KV::Regs& R, int ji) {
            KV::template issue<0, false>(R, k_cache, v_cache, q,
                                         ji < jend ? S.tile[ji - w0] : kNoTile, 0, 0, 0, lane);
        };
        // kChunkRing register buffers in fixed roles, the loop unrolled over them. The
        // loop runs whole rounds: steps past the end fold an empty block (no valid
        // tokens, zero-record loads: the state does not change). With no branch around
        // a fold or an exit inside a round, the compiler keeps each buffer's loads where
        // they are issued and waits for exactly the block being folded.
        constexpr int kR = kChunkRing;
        static_assert(kR >= 2 && kR <= 4, "2 to 4 buffers");
        int j = w0;
        typename KV::Regs B0, B1, B2, B3;
        issue(B0, j);
        issue_order();
        issue(B1, j + 1);
        if constexpr (kR > 2) {
            issue_order();
            issue(B2, j + 2);
        }
        if constexpr (kR > 3) {
            issue_order();
            issue(B3, j + 3);
        }
#define PKV_STEP(R)                                                                          \
        {                                                                                    \
            const int vd = j < jend ? (int)S.valid[j - w0] : 0;                              \
            uint4 ka[4], v[4];                                                               \
            stage_block<T, KV>(R, S.ktile[wave], vd, lane, ka, v);                           \
            _Pragma("unroll")                                                                \
            for (int t = 0; t < NT; ++t) {                                                   \
                /* a tile that sees nothing of the block skips it (uniform) */               \
                if (NT > 1 && j * kBS > tlast[t]) continue;                                  \
                int lim = lim0[t] - j * kBS;                                                 \
                lim = lim < 0 ? 0 : (lim > vd ? vd : lim);                                   \
                fold_tile<T>(st[t], ka, qv[t], v, lim, scale_log2, lane);                    \
            }                                                                                \
        }                                                                                    \
        issue(R, j + kR);                                                                    \
        ++j;
        if (jend > w0) {
            do {
                PKV_STEP(B0)
                PKV_STEP(B1)
                if constexpr (kR > 2) { PKV_STEP(B2) }
                if constexpr (kR > 3) { PKV_STEP(B3) }
            } while (j < jend);
        }
#undef PKV_STEP
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
        wave_to_rows(out, row0[t], st[t], lane, ncols[t], group, num_heads, out_scale);
}

// Scale arguments of a launch: the key scale folds into the softmax scale, the value
// scale into the output normalisation; reciprocals (one binary32 division each) for
// the 8-bit append.
struct Scales {
    float scale_log2, out_scale, k_inv, v_inv;
};
inline Scales scales_of(const DecodeArgs& a) {
    const bool fp8 = a.kv_fp8 != 0;
    return Scales{a.scale * (fp8 ? a.k_scale : 1.f) * kLog2e, fp8 ? a.v_scale : 1.f,
                  fp8 ? 1.f / a.k_scale : 1.f, fp8 ? 1.f / a.v_scale : 1.f};
}

template <typename T, typename KV, int GMAX, int NW>
int launch_balanced(const DecodeArgs& a, const DecodePlan& plan, int workers,
                    hipStream_t stream) {
    const DecodeShape& s = a.shape;
    char* ws = (char*)a.workspace;
    using E = typename KV::Elem;
    const Scales sc = scales_of(a);
    hipLaunchKernelGGL((decode_mfma_balanced_kernel<T, KV, GMAX, NW>), dim3(workers),
                       dim3(64 * NW), 0, stream, (T*)a.out, (const T*)a.q, (E*)a.k_cache,
                       (E*)a.v_cache, (const T*)a.new_k, (const T*)a.new_v, a.block_tables,
                       a.context_lens, sc.scale_log2, sc.out_scale, sc.k_inv, sc.v_inv,
                       s.num_seqs, s.num_heads, s.num_kv_heads, plan.group,
                       s.max_blocks, s.num_blocks, (int32_t*)(ws + plan.off_counters),
                       (float*)(ws + plan.off_partials));
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <typename T, typename KV, int GMAX>
int launch_partitioned(const DecodeArgs& a, const DecodePlan& plan, int num_cus,
                       hipStream_t stream) {
    const DecodeShape& s = a.shape;
    char* ws = (char*)a.workspace;
    const bool split = plan.max_partitions > 1;
    // helpers only on the per-unit grid (one partition per context): one per workgroup
    // slot (two per CU), spread over the KV heads
    int helpers = split ? 0 : max(1, 2 * num_cus / s.num_kv_heads);
    if (helpers > plan.helpers) helpers = plan.helpers;
    using E = typename KV::Elem;
    const Scales sc = scales_of(a);
    // the patching form of the fused step (16-bit caches, a grid that starts every unit
    // at once: there the append's wait lies on the launch's critical path; in a grid run
    // in rounds the extra work in the loop costs more than it saves)
    auto kernel = decode_mfma_partition_kernel<T, KV, GMAX, false>;
    if constexpr (sizeof(E) == sizeof(T)) {
        if (a.new_k != nullptr && !split &&
            (long long)s.num_seqs * s.num_kv_heads <= kPerUnitMinUnits)
            kernel = decode_mfma_partition_kernel<T, KV, GMAX, true>;
    }
    hipLaunchKernelGGL(kernel,
                       dim3(plan.max_partitions, s.num_kv_heads, s.num_seqs + helpers),
                       dim3(kThreads), 0, stream, (T*)a.out, (const T*)a.q, (E*)a.k_cache,
                       (E*)a.v_cache, (const T*)a.new_k, (const T*)a.new_v, a.block_tables,
                       a.context_lens, sc.scale_log2, sc.out_scale, sc.k_inv, sc.v_inv,
                       s.num_heads, s.num_kv_heads, plan.group, s.max_blocks, s.num_blocks,
                       plan.partition_tokens / kBS, plan.max_partitions,
                       split ? (float*)(ws + plan.off_m) : nullptr,
                       split ? (float*)(ws + plan.off_l) : nullptr,
                       split ? (float*)(ws + plan.off_o) : nullptr, s.num_seqs, 2 * num_cus,
                       helpers ? (int32_t*)(ws + plan.off_counters) : nullptr,
                       helpers ? (float*)(ws + plan.off_partials) : nullptr,
                       plan.rec_per_head);
    if (hipGetLastError() != hipSuccess) return -1;
    return split ? launch_partition_reduce(a, plan, stream) : 0;
}

// Grouped decode: the tile kernel over every group (its prefix parts and its members'
// own blocks), then, when some prefix has several parts, the merge kernel.
template <typename T, typename KV>
int launch_grouped_t(const DecodeArgs& a, const GroupArgs& ga, const GroupPlan& gp,
                     hipStream_t stream) {
    const DecodeShape& s = a.shape;
    char* ws = (char*)a.workspace;
    using E = typename KV::Elem;
    const Scales sc = scales_of(a);
    const int G = s.num_heads / s.num_kv_heads;
    const long long units = (long long)gp.parts * s.num_kv_heads * ga.num_groups;
    const long long units8 = (units + 7) / 8 * 8;
    if (units == 0) return 0;
    if (units8 * gp.tiles > 0x7fffffffLL) return -1;
    const bool merge = gp.parts > 1;
    int32_t* seq_prefix = merge ? (int32_t*)(ws + gp.off_prefix) : nullptr;
    float* rm = merge ? (float*)(ws + gp.off_m) : nullptr;
    float* rl = merge ? (float*)(ws + gp.off_l) : nullptr;
    float* ro = merge ? (float*)(ws + gp.off_o) : nullptr;
    hipLaunchKernelGGL((group_tile_kernel<T, KV, kGroupTiles, kGroupWaves>),
                       dim3((unsigned)(units8 * gp.tiles)), dim3(64 * kGroupWaves), 0, stream, (T*)a.out, (const T*)a.q, (E*)a.k_cache,
                       (E*)a.v_cache, (const T*)a.new_k, (const T*)a.new_v, a.block_tables,
                       a.context_lens, ga.group_start, ga.group_prefix, sc.scale_log2,
                       sc.out_scale, sc.k_inv, sc.v_inv, s.num_seqs, s.num_heads,
                       s.num_kv_heads, G, gp.members_per_tile, gp.tiles, (int)units,
                       s.max_blocks, s.num_blocks, ga.max_prefix, gp.parts, seq_prefix, rm, rl,
                       ro);
    if (hipGetLastError() != hipSuccess) return -1;
    if (merge) {
        const long long threads = (long long)s.num_seqs * s.num_heads * (kD / 4);
        hipLaunchKernelGGL((group_merge_kernel<T>),
                           dim3((unsigned)((threads + kThreads - 1) / kThreads)),
                           dim3(kThreads), 0, stream, (T*)a.out, seq_prefix, rm, rl, ro,
                           sc.out_scale, s.num_seqs * s.num_heads, s.num_heads, ga.max_prefix,
                           gp.parts);
        if (hipGetLastError() != hipSuccess) return -1;
    }
    return 0;
}

template <typename T, typename KV>
int launch_chunk(const ChunkArgs& a, hipStream_t stream) {
    const int G = a.num_heads / a.num_kv_heads;
    const int tq = 16 / G;   // query tokens per workgroup (G <= 16)
    const int tiles = (a.max_query_len + tq - 1) / tq;
    if (tiles == 0 || a.num_seqs == 0) return 0;
    using E = typename KV::Elem;
    const bool fp8 = a.kv_fp8 != 0;
    const float scale_log2 = a.scale * (fp8 ? a.k_scale : 1.f) * kLog2e;
    const float out_scale = fp8 ? a.v_scale : 1.f;
    // Long chunks (more than four tiles): each wave folds NT tiles per staged
    // block. Short ones: one tile per workgroup, its waves splitting the blocks.
    constexpr int NT = 1;
    if (tiles > kWaves && !fp8 && a.scale > 0.f) {
        // 16-bit caches: 32x32 tiles, K/V shared through LDS by the workgroup's waves
        const int tqw = 32 / G;
        const int groups = (a.max_query_len + kWaves * tqw - 1) / (kWaves * tqw);
        const long long items = (long long)groups * a.num_kv_heads * a.num_seqs;
        if (items > 0x7fffffffLL) return -1;
        hipLaunchKernelGGL((chunk_fa_kernel<T>), dim3((unsigned)items), dim3(kThreads), 0, stream,
                           (T*)a.out, (const T*)a.q, (const T*)a.k_cache, (const T*)a.v_cache,
                           a.block_tables, a.context_lens, a.query_start, scale_log2,
                           a.num_query_tokens, a.num_heads, a.num_kv_heads, G, a.max_blocks,
                           a.num_blocks, groups);
    } else if (tiles > kWaves)
    {
        // one-dimensional grid of (span group, KV head, sequence) items
        const int groups = (tiles + kWaves * NT - 1) / (kWaves * NT);
        const long long items = (long long)groups * a.num_kv_heads * a.num_seqs;
        if (items > 0x7fffffffLL) return -1;
        hipLaunchKernelGGL((chunk_tiles_kernel<T, KV, NT>), dim3((unsigned)items),
                           dim3(kThreads), 0, stream, (T*)a.out, (const T*)a.q,
                           (const E*)a.k_cache, (const E*)a.v_cache, a.block_tables,
                           a.context_lens, a.query_start, scale_log2, out_scale,
                           a.num_query_tokens, a.num_heads, a.num_kv_heads, G, tq, a.max_blocks,
                           a.num_blocks, groups);
    }
    else
        hipLaunchKernelGGL((chunk_split_kernel<T, KV>),
                           dim3(tiles, a.num_kv_heads, a.num_seqs), dim3(kThreads), 0, stream,
                           (T*)a.out, (const T*)a.q, (const E*)a.k_cache, (const E*)a.v_cache,
                           a.block_tables, a.context_lens, a.query_start, scale_log2, out_scale,
                           a.num_query_tokens, a.num_heads, a.num_kv_heads, G, tq, a.max_blocks,
                           a.num_blocks);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <typename T, typename KV>
int launch_format(const DecodeArgs& a, const DecodePlan& plan, int num_cus,
                  hipStream_t stream) {
    const int G = plan.group;
    if (plan.path == Path::MfmaBalanced) {
        // one workgroup per CU
        const int workers = balanced_workers(a.shape, num_cus, 1);
        if (workers <= 0 || workers > plan.max_workers) return -1;
        // Waves per workgroup: KV::kWaves (two per SIMD for 8-bit caches) while the
        // merge records fit in LDS (groups up to 8), else four.
        constexpr int NW = KV::kWaves;
        if (G <= 4) return launch_balanced<T, KV, 4, NW>(a, plan, workers, stream);
        if (G <= 8) return launch_balanced<T, KV, 8, NW>(a, plan, workers, stream);
        return launch_balanced<T, KV, 16, 4>(a, plan, workers, stream);
    }
    if (G <= 4) return launch_partitioned<T, KV, 4>(a, plan, num_cus, stream);
    if (G <= 8) return launch_partitioned<T, KV, 8>(a, plan, num_cus, stream);
    return launch_partitioned<T, KV, 16>(a, plan, num_cus, stream);
}

template <typename T>
int launch_typed(const DecodeArgs& a, const DecodePlan& plan, int num_cus, hipStream_t stream) {
    return a.kv_fp8 ? launch_format<T, KvFp8<T>>(a, plan, num_cus, stream)
                    : launch_format<T, KvNative<T>>(a, plan, num_cus, stream);
}

}  // namespace

int launch_chunk_mfma(const ChunkArgs& a, hipStream_t stream) {
    if (a.dtype == PKV_BFLOAT16)
        return a.kv_fp8 ? launch_chunk<bf16_t, KvFp8<bf16_t>>(a, stream)
                        : launch_chunk<bf16_t, KvNative<bf16_t>>(a, stream);
    if (a.dtype == PKV_FLOAT16)
        return a.kv_fp8 ? launch_chunk<f16_t, KvFp8<f16_t>>(a, stream)
                        : launch_chunk<f16_t, KvNative<f16_t>>(a, stream);
    return -1;
}

int launch_decode_grouped(const DecodeArgs& a, const GroupArgs& ga, const GroupPlan& gp,
                          hipStream_t stream) {
    if (a.shape.num_kv_heads <= 0 || a.shape.num_heads % a.shape.num_kv_heads != 0) return -1;
    switch (a.shape.dtype) {
        case PKV_BFLOAT16:
            return a.kv_fp8 ? launch_grouped_t<bf16_t, KvFp8<bf16_t>>(a, ga, gp, stream)
                            : launch_grouped_t<bf16_t, KvNative<bf16_t>>(a, ga, gp, stream);
        case PKV_FLOAT16:
            return a.kv_fp8 ? launch_grouped_t<f16_t, KvFp8<f16_t>>(a, ga, gp, stream)
                            : launch_grouped_t<f16_t, KvNative<f16_t>>(a, ga, gp, stream);
        default: return -1;
    }
}

int launch_decode_mfma(const DecodeArgs& a, const DecodePlan& plan, int num_cus,
                       hipStream_t stream) {
    switch (a.shape.dtype) {
        case PKV_BFLOAT16: return launch_typed<bf16_t>(a, plan, num_cus, stream);
        case PKV_FLOAT16: return launch_typed<f16_t>(a, plan, num_cus, stream);
        default: return -1;
    }
}

}  // namespace pkv

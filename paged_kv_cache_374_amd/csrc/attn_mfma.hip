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
//     query heads of the KV head (G <= 16, unused columns see a zero query). K is
//     loaded straight from HBM into the A operand of v_mfma_f32_16x16x32 (16-byte
//     loads; lane l holds token l%16, dims 32kk + 8(l/16) .. +7), Q sits in the B
//     operand with the same dim assignment, so the contraction pairs equal dims.
//   * The score tile comes out with lane l holding tokens 4(l/16)+r (r = 0..3) of
//     head l%16, which is exactly the A-operand layout of v_mfma_f32_16x16x16 for
//     P (rows = heads, k = tokens). The probabilities are rounded to the KV type.
//   * PV: lane l loads V rows 4(l/16)+r, dims 8(l%16) .. +7. The n-th of the eight
//     16x16x16 products takes element n of those four rows as its B operand, so
//     output column j of product n is dim 8j + n; the repack is a byte permute per
//     register, no LDS transpose.
//   * Online softmax per head in base-2 units (scale * log2 e folded in). The running
//     max is raised lazily: the accumulators are rescaled only when a block's max
//     exceeds the running max by more than 2^8, so most blocks skip the rescale.
//
// Work split ("balanced" path): all (sequence, KV head) units are laid end to end as
// one list of blocks, and every workgroup takes an equal contiguous share of it
// (the grid is a fixed multiple of the CU count). Its four waves take every fourth
// block of the share, each keeping its own softmax state, merged through LDS at each
// unit boundary. A unit covered by one workgroup is written out directly; a unit cut
// by share boundaries leaves one partial (m, l, unnormalised o) per workgroup, and
// the last workgroup to finish it (atomic counter) merges them:
//   M = max_w m_w,  L = sum_w l_w 2^(m_w - M),  out = sum_w o_w 2^(m_w - M) / L,
// in fixed workgroup order (deterministic), and zeroes the counter for the next call.
//
// "Partitioned" path (caller asks for a partition size): one workgroup per
// (partition, KV head, sequence); each leaves (m, l, o/l) per partition for the
// shared reduction kernel, or writes the output when the context has one partition.
#include <cstdlib>

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
constexpr float kLazy = 8.0f;    // rescale only when the max grows by more than 2^8
constexpr uint32_t kNoTile = 0xffffffffu;

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

// One wave's KV registers for one block: K in QK operand order, V rows for PV.
struct BlockRegs {
    uint4 k[4];
    uint4 v[4];
};

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

template <typename T>
__device__ __forceinline__ void issue_block(BlockRegs& r, const T* __restrict__ k_cache,
                                            const T* __restrict__ v_cache, uint32_t tile,
                                            int lane) {
    if (tile == kNoTile) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            r.k[i] = make_uint4(0, 0, 0, 0);
            r.v[i] = make_uint4(0, 0, 0, 0);
        }
        return;
    }
    const size_t base = (size_t)tile * kTile;
    const int c = lane & 15, grp = lane >> 4;
    const T* kp = k_cache + base + c * kD + 8 * grp;
    const T* vp = v_cache + base + (4 * grp) * kD + 8 * c;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.k[i] = load16(kp + 32 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) r.v[i] = load16(vp + i * kD);
}

// Fold one block into the wave's state. `valid` = tokens of the block that count
// (0 masks the whole block); qop = the query in QK B-operand order.
template <typename T>
__device__ __forceinline__ void fold_block(WaveState& s, BlockRegs& r, const uint4 (&qop)[4],
                                           int valid, float scale_log2, int group, int lane) {
    const int c = lane & 15, grp = lane >> 4;
    if (valid < kBS) {
        // Slots past the context hold stale data (possibly NaN); a zero weight does not
        // cancel a NaN inside the product, so their V rows are cleared. Their scores are
        // replaced by -inf below (a select), so stale K never reaches the softmax.
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (4 * grp + e >= valid) r.v[e] = make_uint4(0, 0, 0, 0);
    }
    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) sc = Mma<T>::qk(r.k[i], qop[i], sc);
    float x[4];
    float mb = kNegInf;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[e] = (4 * grp + e < valid) ? sc[e] * scale_log2 : kNegInf;
        mb = fmaxf(mb, x[e]);
    }
    mb = fmaxf(mb, __shfl_xor(mb, 16));
    mb = fmaxf(mb, __shfl_xor(mb, 32));
    const bool raise = (c < group) && (mb > s.m + kLazy);
    if (__any(raise)) {
        const float mn = fmaxf(s.m, mb);
        const float alpha = (s.m == kNegInf) ? 0.f : fast_exp2(s.m - mn);
        s.lsum *= alpha;
        s.m = mn;
        // o[.][r] belongs to head 4(l/16)+r, whose factor lives in lane 4(l/16)+r.
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float a = __shfl(alpha, 4 * grp + e);
#pragma unroll
            for (int n = 0; n < 8; ++n) s.o[n][e] *= a;
        }
    }
    const float mu = (s.m == kNegInf) ? 0.f : s.m;
    float p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        p[e] = fast_exp2(x[e] - mu);
        s.lsum += p[e];
    }
    const uint2 pa = make_uint2(Mma<T>::pack(p[0], p[1]), Mma<T>::pack(p[2], p[3]));
#define PKV_PV_STEP(N)                                                                  \
    s.o[N] = Mma<T>::pv(pa, make_uint2(pick<N>(r.v[0], r.v[1]), pick<N>(r.v[2], r.v[3])), \
                        s.o[N]);
    PKV_PV_STEP(0) PKV_PV_STEP(1) PKV_PV_STEP(2) PKV_PV_STEP(3)
    PKV_PV_STEP(4) PKV_PV_STEP(5) PKV_PV_STEP(6) PKV_PV_STEP(7)
#undef PKV_PV_STEP
}

template <typename T>
__device__ __forceinline__ void load_query(uint4 (&qop)[4], const T* __restrict__ q, int b,
                                           int g, int num_heads, int group, int lane) {
    const int c = lane & 15, grp = lane >> 4;
    if (c < group) {
        const T* qp = q + ((size_t)b * num_heads + g * group + c) * kD + 8 * grp;
#pragma unroll
        for (int i = 0; i < 4; ++i) qop[i] = load16(qp + 32 * i);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) qop[i] = make_uint4(0, 0, 0, 0);
    }
}

// LDS used to merge the four waves' states of one unit.
template <int GMAX>
struct MergeLds {
    float m[kWaves][GMAX];
    float l[kWaves][GMAX];
    float o[kWaves][GMAX][kD];
};

// Wave -> LDS (every wave calls it; caller syncs afterwards).
template <int GMAX>
__device__ __forceinline__ void stash_state(MergeLds<GMAX>& L, WaveState& s, int wave, int lane,
                                            int group) {
    const int c = lane & 15, grp = lane >> 4;
    float ls = s.lsum;
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    if (grp == 0 && c < group) {
        L.m[wave][c] = s.m;
        L.l[wave][c] = ls;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int h = 4 * grp + e;
        if (h < group) {
            float4* dst = reinterpret_cast<float4*>(&L.o[wave][h][8 * c]);
            dst[0] = make_float4(s.o[0][e], s.o[1][e], s.o[2][e], s.o[3][e]);
            dst[1] = make_float4(s.o[4][e], s.o[5][e], s.o[6][e], s.o[7][e]);
        }
    }
}

__device__ __forceinline__ float weight(float m, float M) {
    return m == kNegInf ? 0.f : fast_exp2(m - M);
}

// Merge the four waves for head h, dims d0..d0+3: returns M, L and four o values.
template <int GMAX>
__device__ __forceinline__ void merge_waves(const MergeLds<GMAX>& L, int h, int d0, float& M,
                                            float& Lsum, float4& o) {
    M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, L.m[w][h]);
    Lsum = 0.f;
    o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const float wt = weight(L.m[w][h], M);
        Lsum += L.l[w][h] * wt;
        const float4 v = *reinterpret_cast<const float4*>(&L.o[w][h][d0]);
        o.x += v.x * wt;
        o.y += v.y * wt;
        o.z += v.z * wt;
        o.w += v.w * wt;
    }
}

template <typename T>
__device__ __forceinline__ void store4(T* p, float4 v) {
    uint2 w;
    w.x = Mma<T>::pack(v.x, v.y);
    w.y = Mma<T>::pack(v.z, v.w);
    *reinterpret_cast<uint2*>(p) = w;
}

// Device-scope relaxed atomic store / load of one float (coherent across XCDs).
__device__ __forceinline__ void publish(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float fetch(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Partial-result slot of the balanced path: o[GMAX][D], then m[GMAX], l[GMAX].
template <int GMAX>
struct Slot {
    static constexpr int kFloats = balanced_slot_floats(GMAX);
};

// ------------------------------------------------------------------ balanced kernel
template <typename T, int GMAX>
struct BalancedLds {
    int pref[kMaxSeqsBalanced + 1];   // blocks per sequence, exclusive prefix
    uint32_t tile[kTabMax];           // (physical block * Hkv + kv head), or kNoTile
    uint8_t valid[kTabMax];           // tokens of the block inside the context
    MergeLds<GMAX> merge;
    int flag;
};

template <typename T, int GMAX>
__global__ __launch_bounds__(kThreads) void decode_mfma_balanced_kernel(
    T* __restrict__ out, const T* __restrict__ q, const T* __restrict__ k_cache,
    const T* __restrict__ v_cache, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ ctx_lens, float scale_log2, int num_seqs, int num_heads,
    int num_kv_heads, int group, int max_blocks, int num_blocks, int32_t* __restrict__ counters,
    float* __restrict__ partials) {
    __shared__ BalancedLds<T, GMAX> S;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int W = gridDim.x;
    // Logical worker index: consecutive shares (which may cut one unit) go to
    // workgroups that the dispatcher places on the same XCD (round-robin over 8).
    const int w = (W % 8 == 0) ? (blockIdx.x % 8) * (W / 8) + blockIdx.x / 8 : blockIdx.x;
    const int cap = max_blocks * kBS;
    const int Hkv = num_kv_heads;

    // ---- prologue: blocks per sequence and their prefix sums
    for (int i = tid; i < num_seqs; i += kThreads) {
        int n = ctx_lens[i];
        n = n < 0 ? 0 : (n > cap ? cap : n);
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
    const long long total = (long long)Hkv * S.pref[num_seqs];
    if (total == 0) return;
    const long long C = (total + W - 1) / W;
    const long long x0 = (long long)w * C;
    const long long x1 = x0 + C < total ? x0 + C : total;
    if (x0 >= x1) return;

    // ---- first sequence of the share: largest b with Hkv * pref[b] <= x0
    int b0;
    {
        int lo = 0, hi = num_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if ((long long)Hkv * S.pref[mid] <= x0) lo = mid; else hi = mid - 1;
        }
        b0 = lo;
    }

    // ---- stage (tile, valid tokens) of every block of the share
    {
        long long x = x0;
        int b = b0;
        while (x < x1) {
            const long long base = (long long)Hkv * S.pref[b];
            const int nb = S.pref[b + 1] - S.pref[b];
            const long long end = base + (long long)Hkv * nb;
            const long long stop = end < x1 ? end : x1;
            int n = ctx_lens[b];
            n = n < 0 ? 0 : (n > cap ? cap : n);
            for (long long xx = x + tid; xx < stop; xx += kThreads) {
                const int r = (int)(xx - base);
                const int g = r / nb, j = r - g * nb;
                const int phys = tables[(size_t)b * max_blocks + j];
                const int left = n - j * kBS;
                const bool ok = phys >= 0 && phys < num_blocks;
                S.tile[xx - x0] = ok ? (uint32_t)phys * (uint32_t)Hkv + (uint32_t)g : kNoTile;
                S.valid[xx - x0] = (uint8_t)(ok ? (left < kBS ? left : kBS) : 0);
            }
            x = stop;
            ++b;
            while (b < num_seqs && S.pref[b + 1] == S.pref[b]) ++b;
        }
    }
    __syncthreads();

    // ---- walk the units of the share
    long long xw = x0 + wave;          // this wave's next block
    BlockRegs cur;
    if (xw < x1) issue_block(cur, k_cache, v_cache, S.tile[xw - x0], lane);
    int b = b0;
    long long ubase = (long long)Hkv * S.pref[b];
    int nb = S.pref[b + 1] - S.pref[b];
    int g = (int)((x0 - ubase) / nb);
    uint4 qop[4];
    load_query(qop, q, b, g, num_heads, group, lane);
    long long x = x0;
    WaveState st;
    while (x < x1) {
        const long long su = ubase + (long long)g * nb;   // first block of unit (b, g)
        const long long ue = su + nb;
        const long long stop = ue < x1 ? ue : x1;
        reset(st);
        // next unit (for the query prefetch)
        int bn = b, gn = g + 1;
        if (gn == Hkv) {
            gn = 0;
            ++bn;
            while (bn < num_seqs && S.pref[bn + 1] == S.pref[bn]) ++bn;
        }
        uint4 qnext[4];
        const bool more = stop < x1;
        if (more) load_query(qnext, q, bn, gn, num_heads, group, lane);
        while (xw < stop) {
            const long long xn = xw + kWaves;
            BlockRegs nxt;
            if (xn < x1) issue_block(nxt, k_cache, v_cache, S.tile[xn - x0], lane);
            fold_block<T>(st, cur, qop, S.valid[xw - x0], scale_log2, group, lane);
            cur = nxt;
            xw = xn;
        }
        // ---- merge the waves for unit (b, g)
        stash_state(S.merge, st, wave, lane, group);
        __syncthreads();
        const bool whole = su >= x0 && ue <= x1;
        const int u = b * Hkv + g;
        if (whole) {
            for (int i = tid; i < group * (kD / 4); i += kThreads) {
                const int h = i / (kD / 4), d0 = (i % (kD / 4)) * 4;
                float M, Ls;
                float4 o;
                merge_waves(S.merge, h, d0, M, Ls, o);
                const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
                o.x *= inv; o.y *= inv; o.z *= inv; o.w *= inv;
                store4(out + ((size_t)b * num_heads + g * group + h) * kD + d0, o);
            }
        } else {
            // Publish this workgroup's partial. Every word goes out as a device-scope
            // atomic store, coherent across the XCDs' L2s on its own, so no fence has to
            // write back or invalidate whole caches (measured: such fences cost more than
            // the attention itself). __syncthreads waits for those stores to complete
            // before thread 0 bumps the unit's counter.
            const int slot = 2 * w + (su <= x0 ? 0 : 1);
            float* P = partials + (size_t)slot * Slot<GMAX>::kFloats;
            for (int i = tid; i < group * (kD / 4); i += kThreads) {
                const int h = i / (kD / 4), d0 = (i % (kD / 4)) * 4;
                float M, Ls;
                float4 o;
                merge_waves(S.merge, h, d0, M, Ls, o);
                publish(P + h * kD + d0, o.x);
                publish(P + h * kD + d0 + 1, o.y);
                publish(P + h * kD + d0 + 2, o.z);
                publish(P + h * kD + d0 + 3, o.w);
                if (d0 == 0) {
                    publish(P + GMAX * kD + h, M);
                    publish(P + GMAX * kD + GMAX + h, Ls);
                }
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            const long long wf = su / C, wl = (ue - 1) / C;
            if (tid == 0) {
                const int done = __hip_atomic_fetch_add(&counters[u], 1, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
                S.flag = (done == (int)(wl - wf));
            }
            __syncthreads();
            if (S.flag) {
                // Last contributor: read every partial back with device-scope atomic
                // loads (they bypass stale cache copies) and merge in workgroup order.
                for (int i = tid; i < group * (kD / 4); i += kThreads) {
                    const int h = i / (kD / 4), d0 = (i % (kD / 4)) * 4;
                    float M = kNegInf;
                    for (long long v = wf; v <= wl; ++v) {
                        const int sl = 2 * (int)v + ((v > wf || su == v * C) ? 0 : 1);
                        const float* Q = partials + (size_t)sl * Slot<GMAX>::kFloats;
                        M = fmaxf(M, fetch(Q + GMAX * kD + h));
                    }
                    float Ls = 0.f;
                    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
                    for (long long v = wf; v <= wl; ++v) {
                        const int sl = 2 * (int)v + ((v > wf || su == v * C) ? 0 : 1);
                        const float* Q = partials + (size_t)sl * Slot<GMAX>::kFloats;
                        const float wt = weight(fetch(Q + GMAX * kD + h), M);
                        Ls += fetch(Q + GMAX * kD + GMAX + h) * wt;
                        o.x += fetch(Q + h * kD + d0) * wt;
                        o.y += fetch(Q + h * kD + d0 + 1) * wt;
                        o.z += fetch(Q + h * kD + d0 + 2) * wt;
                        o.w += fetch(Q + h * kD + d0 + 3) * wt;
                    }
                    const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
                    o.x *= inv; o.y *= inv; o.z *= inv; o.w *= inv;
                    store4(out + ((size_t)b * num_heads + g * group + h) * kD + d0, o);
                }
                if (tid == 0)
                    __hip_atomic_store(&counters[u], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        __syncthreads();   // the merge LDS is reused by the next unit
        x = stop;
        if (more) {
            b = bn;
            g = gn;
            ubase = (long long)Hkv * S.pref[b];
            nb = S.pref[b + 1] - S.pref[b];
#pragma unroll
            for (int i = 0; i < 4; ++i) qop[i] = qnext[i];
        }
    }
}

// ------------------------------------------------------------------ partitioned kernel
template <int GMAX>
struct PartLds {
    uint32_t tile[kTabMax];
    uint8_t valid[kTabMax];
    MergeLds<GMAX> merge;
};

template <typename T, int GMAX>
__global__ __launch_bounds__(kThreads) void decode_mfma_partition_kernel(
    T* __restrict__ out, const T* __restrict__ q, const T* __restrict__ k_cache,
    const T* __restrict__ v_cache, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ ctx_lens, float scale_log2, int num_heads, int num_kv_heads,
    int group, int max_blocks, int num_blocks, int part_blocks, int max_parts,
    float* __restrict__ ws_m, float* __restrict__ ws_l, float* __restrict__ ws_o) {
    __shared__ PartLds<GMAX> S;
    const int p = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cap = max_blocks * kBS;
    int n = ctx_lens[b];
    n = n < 0 ? 0 : (n > cap ? cap : n);
    const int nb = (n + kBS - 1) / kBS;
    if (n == 0) {
        if (p == 0)
            for (int i = tid * 4; i < group * kD; i += kThreads * 4)
                store4(out + ((size_t)b * num_heads + g * group) * kD + i,
                       make_float4(0.f, 0.f, 0.f, 0.f));
        return;
    }
    const int j0 = p * part_blocks;
    if (j0 >= nb) return;
    const int j1 = min(nb, j0 + part_blocks);
    const int nparts = (nb + part_blocks - 1) / part_blocks;
    for (int j = j0 + tid; j < j1; j += kThreads) {
        const int phys = tables[(size_t)b * max_blocks + j];
        const bool ok = phys >= 0 && phys < num_blocks;
        const int left = n - j * kBS;
        S.tile[j - j0] = ok ? (uint32_t)phys * (uint32_t)num_kv_heads + (uint32_t)g : kNoTile;
        S.valid[j - j0] = (uint8_t)(ok ? (left < kBS ? left : kBS) : 0);
    }
    __syncthreads();
    uint4 qop[4];
    load_query(qop, q, b, g, num_heads, group, lane);
    WaveState st;
    reset(st);
    int jw = j0 + wave;
    BlockRegs cur;
    if (jw < j1) issue_block(cur, k_cache, v_cache, S.tile[jw - j0], lane);
    while (jw < j1) {
        const int jn = jw + kWaves;
        BlockRegs nxt;
        if (jn < j1) issue_block(nxt, k_cache, v_cache, S.tile[jn - j0], lane);
        fold_block<T>(st, cur, qop, S.valid[jw - j0], scale_log2, group, lane);
        cur = nxt;
        jw = jn;
    }
    stash_state(S.merge, st, wave, lane, group);
    __syncthreads();
    for (int i = tid; i < group * (kD / 4); i += kThreads) {
        const int h = i / (kD / 4), d0 = (i % (kD / 4)) * 4;
        float M, Ls;
        float4 o;
        merge_waves(S.merge, h, d0, M, Ls, o);
        const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
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
}

template <typename T, int GMAX>
int launch_balanced(const DecodeArgs& a, const DecodePlan& plan, int workers,
                    hipStream_t stream) {
    const DecodeShape& s = a.shape;
    char* ws = (char*)a.workspace;
    hipLaunchKernelGGL((decode_mfma_balanced_kernel<T, GMAX>), dim3(workers), dim3(kThreads), 0,
                       stream, (T*)a.out, (const T*)a.q, (const T*)a.k_cache,
                       (const T*)a.v_cache, a.block_tables, a.context_lens, a.scale * kLog2e,
                       s.num_seqs, s.num_heads, s.num_kv_heads, plan.group, s.max_blocks,
                       s.num_blocks, (int32_t*)(ws + plan.off_counters),
                       (float*)(ws + plan.off_partials));
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <typename T, int GMAX>
int launch_partitioned(const DecodeArgs& a, const DecodePlan& plan, hipStream_t stream) {
    const DecodeShape& s = a.shape;
    char* ws = (char*)a.workspace;
    const bool split = plan.max_partitions > 1;
    hipLaunchKernelGGL((decode_mfma_partition_kernel<T, GMAX>),
                       dim3(plan.max_partitions, s.num_kv_heads, s.num_seqs), dim3(kThreads), 0,
                       stream, (T*)a.out, (const T*)a.q, (const T*)a.k_cache,
                       (const T*)a.v_cache, a.block_tables, a.context_lens, a.scale * kLog2e,
                       s.num_heads, s.num_kv_heads, plan.group, s.max_blocks, s.num_blocks,
                       plan.partition_tokens / kBS, plan.max_partitions,
                       split ? (float*)(ws + plan.off_m) : nullptr,
                       split ? (float*)(ws + plan.off_l) : nullptr,
                       split ? (float*)(ws + plan.off_o) : nullptr);
    if (hipGetLastError() != hipSuccess) return -1;
    return split ? launch_partition_reduce(a, plan, stream) : 0;
}

template <typename T>
int launch_typed(const DecodeArgs& a, const DecodePlan& plan, int workers, hipStream_t stream) {
    const int G = plan.group;
    if (plan.path == Path::MfmaBalanced) {
        if (G <= 4) return launch_balanced<T, 4>(a, plan, workers, stream);
        if (G <= 8) return launch_balanced<T, 8>(a, plan, workers, stream);
        return launch_balanced<T, 16>(a, plan, workers, stream);
    }
    if (G <= 4) return launch_partitioned<T, 4>(a, plan, stream);
    if (G <= 8) return launch_partitioned<T, 8>(a, plan, stream);
    return launch_partitioned<T, 16>(a, plan, stream);
}

}  // namespace

int wg_per_cu() {
    static const int v = [] {
        const char* e = std::getenv("PKV_WG_PER_CU");
        const int n = e ? std::atoi(e) : 0;
        return n > 0 && n <= 16 ? n : kWgPerCu;
    }();
    return v;
}

int launch_decode_mfma(const DecodeArgs& a, const DecodePlan& plan, int num_cus,
                       hipStream_t stream) {
    int workers = 0;
    if (plan.path == Path::MfmaBalanced) {
        workers = balanced_workers(a.shape, num_cus, wg_per_cu());
        if (workers <= 0 || workers > plan.max_workers) return -1;
    }
    switch (a.shape.dtype) {
        case PKV_BFLOAT16: return launch_typed<bf16_t>(a, plan, workers, stream);
        case PKV_FLOAT16: return launch_typed<f16_t>(a, plan, workers, stream);
        default: return -1;
    }
}

}  // namespace pkv

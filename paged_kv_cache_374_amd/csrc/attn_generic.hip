// Paged decode attention, vector-ALU kernel for every supported dtype and shape.
//
// One workgroup (256 threads) per (partition, KV head, sequence). A "token group"
// of TG = head_dim*elt/16 lanes owns one token row at a time: each lane loads a
// 16-byte chunk of the row's K and V, forms its part of q.k for every query head
// of the group, and the partial dots are summed across the TG lanes with xor
// shuffles. Each token group keeps its own online-softmax state (running max m,
// running sum l, unnormalised output acc) over the tokens it visits; at the end
// the states are merged across token groups (shuffles), then across the four
// waves (LDS). Scores are kept in base-2 units (scale * log2 e folded in) so the
// exponentials are the native exp2.
//
// A context that fits one partition is written straight to the output; otherwise
// each partition leaves (m, l, acc/l) in the workspace and a reduction kernel
// merges them:  M = max_p m_p,  w_p = l_p 2^(m_p - M),  out = sum_p w_p o_p / sum_p w_p.
//
// The walk follows the pages' description of the kernel: per query, visit the
// physical blocks named by its block table, attend each, merge ([P1] "vLLM 源码解析：
// PagedAttention 如何让大模型推理提速 10 倍", section 四); token t of a sequence is
// in block table[t / block_size] at offset t % block_size ([P2] "vLLM 核心源码深度
// 解析…", section "Block Table 数据结构").
#include "device_common.h"
#include "launchers.h"
#include "pagedkv.h"

namespace pkv {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

// Weight 2^(m - M) of a state whose max is m, inside a merge whose max is M; an empty
// state (m = -inf) weighs nothing, also when every state is empty.
__device__ __forceinline__ float merge_weight(float m, float M) {
    return m == kNegInf ? 0.f : fast_exp2(m - M);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_generic_kernel(
    T* __restrict__ out, const T* __restrict__ q, const T* __restrict__ k_cache,
    const T* __restrict__ v_cache, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ ctx_lens, float scale_log2, int num_heads, int num_kv_heads,
    int group, int block_size, int max_blocks, int num_blocks, int part_tokens, int max_parts,
    float* __restrict__ ws_m, float* __restrict__ ws_l, float* __restrict__ ws_o) {
    constexpr int VEC = Vec16<T>::N;
    constexpr int TG = D / VEC;          // lanes per token row
    constexpr int NTG = 256 / TG;        // token groups per workgroup
    constexpr int MAXG = kMaxGroupGeneric;
    static_assert(TG >= 1 && TG <= 64 && 64 % TG == 0, "token row must tile a wavefront");
    __shared__ float s_m[4][MAXG];
    __shared__ float s_l[4][MAXG];
    __shared__ float s_acc[4][MAXG][D];

    const int p = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int cap = max_blocks * block_size;
    int ctx = ctx_lens[b];
    ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
    const int tid = threadIdx.x;
    const int li = tid % TG, gi = tid / TG;
    const int h0 = kvh * group;

    if (ctx == 0) {  // empty context: zero output (written once, by partition 0)
        if (p == 0)
            for (int i = tid; i < group * D; i += 256)
                out[((size_t)b * num_heads + h0 + i / D) * D + i % D] = Elt<T>::from_float(0.f);
        return;
    }
    const int t0 = p * part_tokens;
    if (t0 >= ctx) return;
    const int t1 = min(ctx, t0 + part_tokens);
    const int nparts = (ctx + part_tokens - 1) / part_tokens;

    float qv[MAXG][VEC];
#pragma unroll
    for (int g = 0; g < MAXG; ++g) {
        if (g < group) {
            Vec16<T>::unpack(load16(q + ((size_t)b * num_heads + h0 + g) * D + li * VEC), qv[g]);
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) qv[g][e] = 0.f;
        }
    }
    float m[MAXG], l[MAXG], acc[MAXG][VEC];
#pragma unroll
    for (int g = 0; g < MAXG; ++g) {
        m[g] = kNegInf;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[g][e] = 0.f;
    }

    const int32_t* table = tables + (size_t)b * max_blocks;
    for (int t = t0 + gi; t < t1; t += NTG) {
        const int phys = table[t / block_size];
        if (phys < 0 || phys >= num_blocks) continue;  // uniform within the token group
        const size_t row =
            (((size_t)phys * num_kv_heads + kvh) * block_size + (t % block_size)) * D + li * VEC;
        float kf[VEC], vf[VEC];
        Vec16<T>::unpack(load16(k_cache + row), kf);
        Vec16<T>::unpack(load16(v_cache + row), vf);
#pragma unroll
        for (int g = 0; g < MAXG; ++g) {
            if (g < group) {
                float s = 0.f;
#pragma unroll
                for (int e = 0; e < VEC; ++e) s += qv[g][e] * kf[e];
#pragma unroll
                for (int off = TG / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, TG);
                s *= scale_log2;
                const float mn = fmaxf(m[g], s);
                const float a = fast_exp2(m[g] - mn);   // m = -inf on the first token: 0
                const float pe = fast_exp2(s - mn);
                l[g] = l[g] * a + pe;
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[g][e] = acc[g][e] * a + pe * vf[e];
                m[g] = mn;
            }
        }
    }

    // Merge token groups inside the wavefront (lanes with equal li hold equal dims).
#pragma unroll
    for (int off = TG; off < 64; off <<= 1) {
#pragma unroll
        for (int g = 0; g < MAXG; ++g) {
            if (g < group) {
                const float mo = __shfl_xor(m[g], off);
                const float lo = __shfl_xor(l[g], off);
                const float M = fmaxf(m[g], mo);
                const float wa = merge_weight(m[g], M), wb = merge_weight(mo, M);
                l[g] = l[g] * wa + lo * wb;
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float ao = __shfl_xor(acc[g][e], off);
                    acc[g][e] = acc[g][e] * wa + ao * wb;
                }
                m[g] = M;
            }
        }
    }
    const int wave = tid / 64, lane = tid % 64;
    if (lane < TG) {
#pragma unroll
        for (int g = 0; g < MAXG; ++g) {
            if (g < group) {
                if (lane == 0) {
                    s_m[wave][g] = m[g];
                    s_l[wave][g] = l[g];
                }
#pragma unroll
                for (int e = 0; e < VEC; ++e) s_acc[wave][g][lane * VEC + e] = acc[g][e];
            }
        }
    }
    __syncthreads();

    // Merge the four waves and write the result (or this partition's partial).
    for (int i = tid; i < group * D; i += 256) {
        const int g = i / D, d = i % D;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w][g]);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float wt = merge_weight(s_m[w][g], M);
            L += s_l[w][g] * wt;
            O += s_acc[w][g][d] * wt;
        }
        const float o = L > 0.f ? O / L : 0.f;
        const size_t hrow = (size_t)b * num_heads + h0 + g;
        if (nparts == 1) {
            out[hrow * D + d] = Elt<T>::from_float(o);
        } else {
            const size_t pr = hrow * max_parts + p;
            ws_o[pr * D + d] = o;
            if (d == 0) {
                ws_m[pr] = M;
                ws_l[pr] = L;
            }
        }
    }
}

// One workgroup per (query head, sequence) merges that row's partitions:
//   M = max_p m_p,  w_p = l_p 2^(m_p - M),  out = sum_p w_p o_p / sum_p w_p
// (o_p is partition p's normalised output). Threads split the partitions into
// interleaved sets and the dims into float4 columns, so every load of a thread is
// independent of the others; the sets are then added in LDS in a fixed order
// (deterministic).
constexpr int kReduceThreads = 256;

template <typename T>
__global__ __launch_bounds__(kReduceThreads) void partition_reduce_kernel(
    T* __restrict__ out, const int32_t* __restrict__ ctx_lens, int num_heads, int head_dim,
    int max_blocks, int block_size, int part_tokens, int max_parts,
    const float* __restrict__ ws_m, const float* __restrict__ ws_l,
    const float* __restrict__ ws_o) {
    __shared__ float4 acc_s[kReduceThreads];
    __shared__ float w_s[kReduceThreads];
    __shared__ float max_s[kReduceThreads / 64];
    const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int cap = max_blocks * block_size;
    int ctx = ctx_lens[b];
    ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
    const int nparts = (ctx + part_tokens - 1) / part_tokens;
    if (nparts <= 1) return;   // written directly by the partition kernel
    const size_t row = (size_t)b * num_heads + h;
    const float* m = ws_m + row * max_parts;
    const float* l = ws_l + row * max_parts;
    const float* o = ws_o + row * max_parts * head_dim;
    float M = kNegInf;
    for (int p = tid; p < nparts; p += kReduceThreads) M = fmaxf(M, m[p]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    if ((tid & 63) == 0) max_s[tid >> 6] = M;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kReduceThreads / 64; ++i) M = fmaxf(M, max_s[i]);
    const int cols = head_dim / 4;               // 16, 32 or 64
    const int sets = kReduceThreads / cols;      // 16, 8 or 4
    const int c = tid % cols, set = tid / cols;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float W = 0.f;
#pragma unroll 4
    for (int p = set; p < nparts; p += sets) {
        const float w = l[p] * merge_weight(m[p], M);
        const float4 v = reinterpret_cast<const float4*>(o + (size_t)p * head_dim)[c];
        acc.x += w * v.x;
        acc.y += w * v.y;
        acc.z += w * v.z;
        acc.w += w * v.w;
        W += w;
    }
    acc_s[tid] = acc;
    w_s[tid] = W;
    __syncthreads();
    if (set == 0) {
        float4 t = acc;
        float wt = W;
        for (int k = 1; k < sets; ++k) {
            const float4 u = acc_s[k * cols + c];
            t.x += u.x;
            t.y += u.y;
            t.z += u.z;
            t.w += u.w;
            wt += w_s[k * cols];
        }
        const float inv = wt > 0.f ? 1.f / wt : 0.f;
        T* dst = out + row * head_dim + 4 * c;
        dst[0] = Elt<T>::from_float(t.x * inv);
        dst[1] = Elt<T>::from_float(t.y * inv);
        dst[2] = Elt<T>::from_float(t.z * inv);
        dst[3] = Elt<T>::from_float(t.w * inv);
    }
}

template <typename T, int D>
int launch_generic_typed(const DecodeArgs& a, const DecodePlan& plan, hipStream_t stream) {
    const DecodeShape& s = a.shape;
    char* ws = (char*)a.workspace;
    float* wm = plan.max_partitions > 1 ? (float*)(ws + plan.off_m) : nullptr;
    float* wl = plan.max_partitions > 1 ? (float*)(ws + plan.off_l) : nullptr;
    float* wo = plan.max_partitions > 1 ? (float*)(ws + plan.off_o) : nullptr;
    hipLaunchKernelGGL((decode_generic_kernel<T, D>),
                       dim3(plan.max_partitions, s.num_kv_heads, s.num_seqs), dim3(256), 0,
                       stream, (T*)a.out, (const T*)a.q, (const T*)a.k_cache,
                       (const T*)a.v_cache, a.block_tables, a.context_lens, a.scale * kLog2e,
                       s.num_heads, s.num_kv_heads, plan.group, s.block_size, s.max_blocks,
                       s.num_blocks, plan.partition_tokens, plan.max_partitions, wm, wl, wo);
    if (hipGetLastError() != hipSuccess) return -1;
    if (plan.max_partitions > 1) return launch_partition_reduce(a, plan, stream);
    return 0;
}

template <typename T>
int launch_reduce_typed(const DecodeArgs& a, const DecodePlan& plan, hipStream_t stream) {
    const DecodeShape& s = a.shape;
    const char* ws = (const char*)a.workspace;
    hipLaunchKernelGGL(partition_reduce_kernel<T>, dim3(s.num_heads, s.num_seqs),
                       dim3(kReduceThreads), 0,
                       stream, (T*)a.out, a.context_lens, s.num_heads, s.head_dim, s.max_blocks,
                       s.block_size, plan.partition_tokens, plan.max_partitions,
                       (const float*)(ws + plan.off_m), (const float*)(ws + plan.off_l),
                       (const float*)(ws + plan.off_o));
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <typename T>
int dispatch_head_dim(const DecodeArgs& a, const DecodePlan& plan, hipStream_t stream) {
    switch (a.shape.head_dim) {
        case 64: return launch_generic_typed<T, 64>(a, plan, stream);
        case 128: return launch_generic_typed<T, 128>(a, plan, stream);
        case 256: return launch_generic_typed<T, 256>(a, plan, stream);
        default: return -1;
    }
}

}  // namespace

int launch_decode_generic(const DecodeArgs& a, const DecodePlan& plan, hipStream_t stream) {
    switch (a.shape.dtype) {
        case PKV_FLOAT32: return dispatch_head_dim<float>(a, plan, stream);
        case PKV_BFLOAT16: return dispatch_head_dim<bf16_t>(a, plan, stream);
        case PKV_FLOAT16: return dispatch_head_dim<f16_t>(a, plan, stream);
        default: return -1;
    }
}

int launch_partition_reduce(const DecodeArgs& a, const DecodePlan& plan, hipStream_t stream) {
    switch (a.shape.dtype) {
        case PKV_FLOAT32: return launch_reduce_typed<float>(a, plan, stream);
        case PKV_BFLOAT16: return launch_reduce_typed<bf16_t>(a, plan, stream);
        case PKV_FLOAT16: return launch_reduce_typed<f16_t>(a, plan, stream);
        default: return -1;
    }
}

}  // namespace pkv

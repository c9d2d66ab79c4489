/*
 * oracle.c -- plain, slow, fp64 CPU reference for paged decode attention and the
 * two KV-cache companions (slot-mapped append, whole-block copy).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call
 * this code; it exists so that tests, the smoke check and the benchmark's CPU
 * baseline can compare the GPU library with an independent implementation. It
 * shares no source, header, table or helper with the GPU library.
 *
 * Pages followed (titles as published):
 *   [P1] "vLLM 源码解析：PagedAttention 如何让大模型推理提速 10 倍"
 *   [P2] "vLLM 核心源码深度解析：PagedAttention 的 KV Cache 管理、Scheduler 调度引擎与
 *         Continuous Batching 实现全解"
 *   [P3] "论文专题讲解：vLLM / PagedAttention：为什么 KV cache 需要分页管理"
 *
 * What is computed is the plain definition, not an algorithm replica: paged
 * attention gives exactly the attention of the query over its whole context; only
 * where the keys and values sit in memory differs ([P3] "PagedAttention：逻辑连续，
 * 物理不必连续": the query at position i attends tokens 1..i, read block by block;
 * [P1] section 四: per query, walk its physical blocks through the page table).
 * So for each sequence b and query head h:
 *   token t (0-based) of b lives in physical block tables[b][t / bs] at offset
 *   t % bs ([P2] "Block Table 数据结构": block number = position // block_size,
 *   offset = position % block_size, physical = block_table[block number]);
 *   s[t]  = scale * sum_d q[b,h,d] * K[t,d]
 *   out   = sum_t exp(s[t] - max s) V[t,:] / sum_t exp(s[t] - max s)
 * evaluated in double precision in two passes. Readings where the pages are
 * silent: KV pools are laid out [num_blocks, num_kv_heads, block_size, head_dim];
 * query head h reads KV head h / (num_heads / num_kv_heads); a zero-length
 * context yields a zero output; the scale is an input.
 *
 * reshape_and_cache: a token with slot s >= 0 is written at block s / bs, offset
 * s % bs, for every KV head ([P3] "Block table：为什么它能减少碎片": the new token
 * goes into the free slot of the last block, or into a newly taken block; the
 * flat slot encoding block * bs + offset is the reading taken for the mapping).
 * copy_blocks: each (src, dst) pair copies a whole block ([P1] section 五,
 * copy-on-write copies the shared block to the new one before the write).
 *
 * 8-bit KV cache. [P2] lists an FP8 KV cache among the engine's milestones
 * ("vLLM 的发展里程碑"), and [P3]'s KV-size formula notes that quantisation lowers
 * the bytes per element. The format and scales are a reading, since the pages fix
 * neither. Elements are OCP FP8 E4M3 (1 sign bit, 4 exponent bits with bias 7, 3
 * mantissa bits; no infinities; S.1111.111 is NaN; largest finite 448). Each cache
 * has one scale: value = decode(code) * scale. Appending a value x stores
 * code = round_e4m3(float(x) * inv_scale). The multiply is a binary32 product, and
 * rounding goes to nearest with ties to an even mantissa; magnitudes of 448 or more
 * (infinity included) saturate to 448, and NaN stays NaN.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F16 = 2, ORACLE_FP8 = 3 };

/* IEEE 754 binary16 -> double, from the format's definition. */
static double half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -24);
    } else if (expo == 31) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexp(1024.0 + (double)frac, expo - 25);
    }
    return sign ? -v : v;
}

/* bfloat16 is the upper half of a binary32: widen the bits and reinterpret. */
static double bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP FP8 E4M3 -> double, from the format's definition. */
static double fp8_to_double(uint8_t c) {
    int sign = c >> 7, expo = (c >> 3) & 15, mant = c & 7;
    double v;
    if (expo == 15 && mant == 7) {
        v = NAN;
    } else if (expo == 0) {
        v = ldexp((double)mant, -9);                 /* subnormal: mant/8 * 2^(1-7) */
    } else {
        v = ldexp(8.0 + (double)mant, expo - 10);    /* (1 + mant/8) * 2^(expo-7) */
    }
    return sign ? -v : v;
}

/* binary32 -> OCP FP8 E4M3: nearest, ties to even mantissa, saturating at 448. */
static uint8_t fp8_from_float(float y) {
    const uint8_t sign = signbit(y) ? 0x80 : 0x00;
    const double a = fabs((double)y);
    if (isnan(y)) return sign | 0x7F;
    if (a >= 448.0) return sign | 0x7E;
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: multiples of 2^-9; a result of 8 is the code of 2^-6,
           the smallest normal value */
        return sign | (uint8_t)nearbyint(ldexp(a, 9));
    }
    int e;
    const double f = frexp(a, &e);                   /* a = f * 2^e, 0.5 <= f < 1 */
    int expo = e - 1;                                /* a = (1 + mant/8) * 2^expo */
    int mant = (int)nearbyint((2.0 * f - 1.0) * 8.0);
    if (mant == 8) {
        mant = 0;
        expo += 1;
    }
    return sign | (uint8_t)(((expo + 7) << 3) | mant);
}

static double elem(const void* base, size_t i, int dtype) {
    if (dtype == ORACLE_F32) return (double)((const float*)base)[i];
    if (dtype == ORACLE_FP8) return fp8_to_double(((const uint8_t*)base)[i]);
    uint16_t bits = ((const uint16_t*)base)[i];
    return dtype == ORACLE_BF16 ? bf16_to_double(bits) : half_to_double(bits);
}

/* Exposed for the tests: decode n raw elements to double. */
int oracle_decode(double* out, const void* src, long n, int dtype) {
    if (dtype < 0 || dtype > 3) return -1;
    for (long i = 0; i < n; ++i) out[i] = elem(src, (size_t)i, dtype);
    return 0;
}

/* Exposed for the tests: quantise n elements (dtype F32, BF16 or F16) to E4M3 codes,
   code[i] = fp8_from_float(float(src[i]) * inv_scale). */
int oracle_quantize_fp8(uint8_t* out, const void* src, long n, int dtype, float inv_scale) {
    if (dtype < 0 || dtype > 2) return -1;
    for (long i = 0; i < n; ++i) {
        const float x = (float)elem(src, (size_t)i, dtype);   /* exact widening */
        const float y = x * inv_scale;                        /* one binary32 product */
        out[i] = fp8_from_float(y);
    }
    return 0;
}

/*
 * out:          double [B, Hq, D]
 * q:            [B, Hq, D]            (q_dtype)
 * k_cache:      [num_blocks, Hkv, bs, D]   (kv_dtype; key = element * k_scale)
 * v_cache:      [num_blocks, Hkv, bs, D]   (kv_dtype; value = element * v_scale)
 * block_tables: int32 [B, max_blocks]
 * context_lens: int32 [B]
 * rows:         optional int32 [num_rows, 2] of (b, h) to evaluate; NULL = all.
 *               With rows given, out is [num_rows, D].
 * Returns 0, or -1 for inconsistent sizes, -2 for a table entry outside the pool
 * inside the used part of a table, -3 for a context longer than its table.
 */
/* Attention of one query row against the first n tokens of sequence b through KV head
 * g: the two-pass walk described at the top. qoff is the element offset of the row's D
 * values in q. Writes o[0..D-1]; returns 0, or -1 when scratch memory runs out. */
static int attend_row(double* o, const void* q, size_t qoff, int q_dtype,
                      const void* k_cache, const void* v_cache, int kv_dtype, double k_scale,
                      double v_scale, const int32_t* block_tables, int b, int g, int n,
                      double scale, int Hkv, int D, int bs, int max_blocks) {
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    if (n <= 0) return 0;
    double* s = (double*)malloc(sizeof(double) * (size_t)n);
    size_t* at = (size_t*)malloc(sizeof(size_t) * (size_t)n);
    if (!s || !at) { free(s); free(at); return -1; }
    /* pass 1: scores, token by token through the block table */
    double mx = -INFINITY;
    for (int t = 0; t < n; ++t) {
        int phys = block_tables[(long)b * max_blocks + t / bs];
        at[t] = (((size_t)phys * Hkv + g) * bs + (size_t)(t % bs)) * D;
        double acc = 0.0;
        for (int d = 0; d < D; ++d)
            acc += elem(q, qoff + d, q_dtype) * (elem(k_cache, at[t] + d, kv_dtype) * k_scale);
        s[t] = scale * acc;
        if (s[t] > mx) mx = s[t];
    }
    /* pass 2: normalised weights applied to the values */
    double denom = 0.0;
    for (int t = 0; t < n; ++t) {
        s[t] = exp(s[t] - mx);
        denom += s[t];
    }
    for (int t = 0; t < n; ++t)
        for (int d = 0; d < D; ++d)
            o[d] += s[t] * (elem(v_cache, at[t] + d, kv_dtype) * v_scale);
    for (int d = 0; d < D; ++d) o[d] /= denom;
    free(s);
    free(at);
    return 0;
}

/* Checks shared by the attention entry points: sizes, contexts within their tables,
 * table entries inside the pool over the used part. */
static int check_tables(const int32_t* block_tables, const int32_t* context_lens, int B,
                        int max_blocks, int num_blocks, int bs) {
    for (int b = 0; b < B; ++b) {
        int n = context_lens[b];
        if (n < 0 || (long)n > (long)max_blocks * bs) return -3;
        for (int j = 0; j < (n + bs - 1) / bs; ++j) {
            int p = block_tables[(long)b * max_blocks + j];
            if (p < 0 || p >= num_blocks) return -2;
        }
    }
    return 0;
}

int oracle_paged_attention_kv(double* out, const void* q, int q_dtype, const void* k_cache,
                              const void* v_cache, int kv_dtype, double k_scale,
                              double v_scale, const int32_t* block_tables,
                              const int32_t* context_lens, double scale, int B, int Hq,
                              int Hkv, int D, int bs, int max_blocks, int num_blocks,
                              const int32_t* rows, int num_rows, int nthreads) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || bs <= 0 || Hq % Hkv != 0) return -1;
    if (q_dtype < 0 || q_dtype > 2 || kv_dtype < 0 || kv_dtype > 3) return -1;
    const int G = Hq / Hkv;
    const int bad = check_tables(block_tables, context_lens, B, max_blocks, num_blocks, bs);
    if (bad) return bad;
    const long work = rows ? num_rows : (long)B * Hq;
    int status = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (long w = 0; w < work; ++w) {
        int b = rows ? rows[2 * w] : (int)(w / Hq);
        int h = rows ? rows[2 * w + 1] : (int)(w % Hq);
        if (b < 0 || b >= B || h < 0 || h >= Hq) { status = -1; continue; }
        int g = h / G;
        if (attend_row(out + w * D, q, ((size_t)b * Hq + h) * D, q_dtype, k_cache, v_cache,
                       kv_dtype, k_scale, v_scale, block_tables, b, g, context_lens[b],
                       scale, Hkv, D, bs, max_blocks))
            status = -1;
    }
    return status;
}

/*
 * Several new query tokens per sequence (a prefill chunk, or draft tokens to verify):
 * [P3] "PagedAttention：逻辑连续，物理不必连续" states that the query at position i
 * attends tokens 1..i, read block by block. Sequence b owns query rows
 * query_start[b] .. query_start[b+1]-1, which are its last T_b = query_start[b+1] -
 * query_start[b] tokens: row query_start[b] + j sits at position
 * context_lens[b] - T_b + j (0-based) and so attends the first
 * context_lens[b] - T_b + j + 1 tokens (none if that count is not positive).
 *
 * out: double [NQ, Hq, D]; q: [NQ, Hq, D] (q_dtype); query_start: int32 [B + 1] with
 * query_start[0] = 0, non-decreasing, query_start[B] = NQ. The caches' new tokens are
 * already written. Returns 0, or the codes of oracle_paged_attention_kv, or -4 for an
 * inconsistent query_start.
 */
int oracle_paged_attention_chunk(double* out, const void* q, int q_dtype,
                                 const void* k_cache, const void* v_cache, int kv_dtype,
                                 double k_scale, double v_scale, const int32_t* block_tables,
                                 const int32_t* context_lens, const int32_t* query_start,
                                 double scale, int B, int NQ, int Hq, int Hkv, int D, int bs,
                                 int max_blocks, int num_blocks, int nthreads) {
    if (B < 0 || NQ < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || bs <= 0 || Hq % Hkv != 0)
        return -1;
    if (q_dtype < 0 || q_dtype > 2 || kv_dtype < 0 || kv_dtype > 3) return -1;
    if (query_start[0] != 0 || query_start[B] != NQ) return -4;
    for (int b = 0; b < B; ++b)
        if (query_start[b + 1] < query_start[b]) return -4;
    const int bad = check_tables(block_tables, context_lens, B, max_blocks, num_blocks, bs);
    if (bad) return bad;
    const int G = Hq / Hkv;
    int status = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (long w = 0; w < (long)NQ * Hq; ++w) {
        const int r = (int)(w / Hq), h = (int)(w % Hq);
        int b = 0;                                  /* the sequence that owns row r */
        while (query_start[b + 1] <= r) ++b;
        const int T = query_start[b + 1] - query_start[b];
        const int j = r - query_start[b];
        const int n = context_lens[b] - T + j + 1;  /* tokens 0 .. position */
        if (attend_row(out + w * D, q, ((size_t)r * Hq + h) * D, q_dtype, k_cache, v_cache,
                       kv_dtype, k_scale, v_scale, block_tables, b, h / G, n, scale, Hkv, D,
                       bs, max_blocks))
            status = -1;
    }
    return status;
}

/* The same walk with q and the caches in one 16/32-bit type and unit scales. */
int oracle_paged_attention(double* out, const void* q, const void* k_cache,
                           const void* v_cache, int dtype, const int32_t* block_tables,
                           const int32_t* context_lens, double scale, int B, int Hq,
                           int Hkv, int D, int bs, int max_blocks, int num_blocks,
                           const int32_t* rows, int num_rows, int nthreads) {
    if (dtype < 0 || dtype > 2) return -1;
    return oracle_paged_attention_kv(out, q, dtype, k_cache, v_cache, dtype, 1.0, 1.0,
                                     block_tables, context_lens, scale, B, Hq, Hkv, D, bs,
                                     max_blocks, num_blocks, rows, num_rows, nthreads);
}

/*
 * k, v:          [T, Hkv, D] raw elements of elt_bytes each
 * k_cache, v_cache: [num_blocks, Hkv, bs, D], updated in place
 * slot_mapping:  int64 [T]; a negative slot skips the token
 * Returns 0, or -2 if a slot points outside the pool.
 */
int oracle_reshape_and_cache(const void* k, const void* v, void* k_cache, void* v_cache,
                             const int64_t* slot_mapping, int T, int Hkv, int D, int bs,
                             int num_blocks, int elt_bytes) {
    const size_t row = (size_t)D * elt_bytes;
    for (int t = 0; t < T; ++t) {
        int64_t slot = slot_mapping[t];
        if (slot < 0) continue;
        int64_t blk = slot / bs, off = slot % bs;
        if (blk >= num_blocks) return -2;
        for (int h = 0; h < Hkv; ++h) {
            size_t dst = (((size_t)blk * Hkv + h) * bs + (size_t)off) * row;
            size_t src = ((size_t)t * Hkv + h) * row;
            memcpy((char*)k_cache + dst, (const char*)k + src, row);
            memcpy((char*)v_cache + dst, (const char*)v + src, row);
        }
    }
    return 0;
}

/*
 * cache: one pool of num_blocks blocks of block_bytes each, updated in place.
 * pairs: int32 [n, 2] of (src, dst), applied in order.
 * Returns 0, or -2 for an ID outside the pool.
 */
/*
 * The append into an 8-bit cache: the same slot walk, each element quantised.
 * k, v:          [T, Hkv, D] elements of src_dtype (F32, BF16 or F16)
 * k_cache, v_cache: uint8 [num_blocks, Hkv, bs, D] E4M3 codes, updated in place
 * k_inv_scale, v_inv_scale: the binary32 reciprocals of the caches' scales
 */
int oracle_reshape_and_cache_fp8(const void* k, const void* v, uint8_t* k_cache,
                                 uint8_t* v_cache, const int64_t* slot_mapping, int T,
                                 int Hkv, int D, int bs, int num_blocks, int src_dtype,
                                 float k_inv_scale, float v_inv_scale) {
    if (src_dtype < 0 || src_dtype > 2) return -1;
    for (int t = 0; t < T; ++t) {
        const int64_t slot = slot_mapping[t];
        if (slot >= (int64_t)num_blocks * bs) return -2;
        if (slot >= 0) for (int h = 0; h < Hkv; ++h) {
            /* slot = block * bs + offset */
            const int64_t block = slot / bs, offset = slot - block * bs;
            size_t dst = (((size_t)block * Hkv + h) * bs + (size_t)offset) * D;
            size_t src = ((size_t)t * Hkv + h) * D;
            for (int d = 0; d < D; ++d) {
                k_cache[dst + d] =
                    fp8_from_float((float)elem(k, src + d, src_dtype) * k_inv_scale);
                v_cache[dst + d] =
                    fp8_from_float((float)elem(v, src + d, src_dtype) * v_inv_scale);
            }
        }
    }
    return 0;
}

int oracle_copy_blocks(void* cache, const int32_t* pairs, int n, int num_blocks,
                       long block_bytes) {
    for (int i = 0; i < n; ++i) {
        int src = pairs[2 * i], dst = pairs[2 * i + 1];
        if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return -2;
        memmove((char*)cache + (size_t)dst * block_bytes,
                (const char*)cache + (size_t)src * block_bytes, (size_t)block_bytes);
    }
    return 0;
}

/*
 * Swap between two pools of the same block layout (a GPU pool and a host pool): each
 * (src, dst) pair copies block src of src_pool over block dst of dst_pool
 * ([P2] "BlockAllocator 源码核心：vLLM 的显存管理心脏", CpuGpuBlockAllocator: when
 * GPU blocks run short, cold blocks move to CPU memory and move back when they are
 * needed again). Returns 0, or -2 for an index outside its pool.
 */
int oracle_swap_blocks(void* dst_pool, const void* src_pool, const int32_t* pairs, int n,
                       int num_src_blocks, int num_dst_blocks, long block_bytes) {
    for (int i = 0; i < n; ++i) {
        const int from = pairs[2 * i], to = pairs[2 * i + 1];
        if (from < 0 || from >= num_src_blocks || to < 0 || to >= num_dst_blocks) return -2;
        memcpy((char*)dst_pool + (size_t)to * block_bytes,
               (const char*)src_pool + (size_t)from * block_bytes, (size_t)block_bytes);
    }
    return 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

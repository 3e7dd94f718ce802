/*
 * fp64 CPU oracle for draft-block paged attention.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the library path may call, link or load
 * this; only the tests, the smoke check and the benchmark's CPU-baseline leg
 * use it. It shares no code with the GPU library.
 */
#ifndef ORACLE_H
#define ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct oracle_params {
    int32_t batch;             /* B requests */
    int32_t block_size;        /* K draft queries per request */
    int32_t num_q_heads;       /* Hq */
    int32_t num_kv_heads;      /* Hkv, divides Hq */
    int32_t head_dim;          /* D */
    int32_t page_size;         /* P tokens per page */
    int32_t page_table_stride; /* entries per page-table row */
    int32_t num_pages;         /* pages in each pool; every page id read must lie below it */
    int32_t window_left;       /* -1: no left limit; W >= 1: keys (p - W, p] on the causal side */
    int32_t window_right;      /* -1: every later block key; 0: none; > 0: at most that many */
    double sm_scale;
    int32_t kv_dtype;          /* ORACLE_KV_BF16 or ORACLE_KV_FP8_E4M3: element type of both pools */
    double k_scale;            /* a stored key element stands for k_scale times its decoded value */
    double v_scale;            /* likewise for values */
    const uint16_t* k_block;   /* NULL, or bf16 bits [B, K, Hkv, D]: the block's keys, read from here (as
                                  they are, no scale) instead of the cache for positions N_b - K .. N_b - 1 */
    const uint16_t* v_block;   /* likewise for values; given together with k_block */
} oracle_params;

enum { ORACLE_KV_BF16 = 0, ORACLE_KV_FP8_E4M3 = 1 };

enum { ORACLE_PART_ALL = 0, ORACLE_PART_CAUSAL = 1, ORACLE_PART_FUTURE = 2 };

/*
 * Attention of every query row over its key set, straight from the definition.
 * q: bf16 bits [B, K, Hq, D]; k_pool, v_pool: [pages, Hkv, P, D] elements of
 * kv_dtype (bf16 bits or OCP fp8 e4m3 bytes), scaled by k_scale / v_scale;
 * page_table: int32 [B, stride]; seq_lens: int32 [B] (context + K keys).
 * pairs: optional list of n_pairs (b, h_kv) int32 pairs; when NULL every pair
 * is computed. out: double [B, K, Hq, D]; lse2: double [B, K, Hq] (base-2
 * log-sum-exp of the scaled logits). Rows outside the chosen pairs are left
 * untouched. An empty key set gives out = 0, lse2 = -inf.
 * Returns 0, or -1 on invalid arguments.
 */
int oracle_attention(const oracle_params* prm, int part, const uint16_t* q, const void* k_pool,
                     const void* v_pool, const int32_t* page_table, const int32_t* seq_lens,
                     const int32_t* pairs, int n_pairs, double* out, double* lse2, int threads);

/* Log-sum-exp merge of two normalised attention results over disjoint key sets. */
void oracle_merge(int64_t rows, int32_t head_dim, const double* out_a, const double* lse_a, const double* out_b,
                  const double* lse_b, double* out, double* lse);

/* Exact bf16 -> double widening used by the oracle (exported for its tests). */
double oracle_bf16_to_double(uint16_t bits);

/* Exact OCP fp8 e4m3 -> double decoding used by the oracle (exported for its tests). */
double oracle_fp8_e4m3_to_double(uint8_t code);

/*
 * The cache element that appending the bf16 value `bits` to a pool of kv_dtype with
 * `scale` stores: q = fp32(value) / fp32(scale) in IEEE fp32 (correctly rounded),
 * then bf16 or OCP E4M3 by round-to-nearest-even; E4M3 saturates at +-448 and maps
 * NaN to 0x7F. Returns the bf16 bits or the E4M3 byte.
 */
uint16_t oracle_encode_kv(int kv_dtype, float scale, uint16_t bits);

#ifdef __cplusplus
}
#endif

#endif

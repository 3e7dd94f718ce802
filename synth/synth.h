/* Seeded synthetic inputs (see synth.c for the generator's definition). */
#ifndef SYNTH_H
#define SYNTH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    SYNTH_TENSOR_Q = 1,
    SYNTH_TENSOR_K = 2,
    SYNTH_TENSOR_V = 3,
    SYNTH_TENSOR_PERM = 4,
    SYNTH_TENSOR_CTX = 5,
    SYNTH_TENSOR_OUTLIER = 6,
    SYNTH_TENSOR_K_BLOCK = 7,  /* dense block keys [B, K, Hkv, D] */
    SYNTH_TENSOR_V_BLOCK = 8
};

uint64_t synth_key(uint64_t seed, uint64_t tensor);
uint64_t synth_draw(uint64_t key, uint64_t n);
double synth_uniform(uint64_t key, uint64_t n);
double synth_normal(uint64_t key, uint64_t n);
uint16_t synth_bf16_from_double(double x);

/* q[count] bf16 N(0,1), element n drawn from stream (seed, q). */
void synth_fill_q(uint64_t seed, int64_t count, uint16_t* q, int threads);
/* count N(0, 1) draws of stream (seed, tensor_id), rounded to bf16 (q uses SYNTH_TENSOR_Q) */
void synth_fill_normal(uint64_t seed, int tensor_id, int64_t count, uint16_t* dst, int threads);

/* out[b] uniform integer in [lo, hi] from stream (seed, context lengths). */
void synth_context_lengths(uint64_t seed, int batch, int lo, int hi, int32_t* out);

/* Pages a pool needs for these lengths: sum of ceil(len/P) plus one fill page. */
int64_t synth_pages_needed(int batch, const int32_t* seq_lens, int page_size);

/* Disjoint shuffled page ranges; rows padded with the fill page id. 0 on success. */
int synth_page_table(uint64_t seed, int batch, const int32_t* seq_lens, int page_size, int stride,
                     int32_t* page_table);

/* Fill a [num_pages, Hkv, P, D] pool with element j of token t, kv head h drawn
 * N(0,1), divided by the pool's scale (inv_scale = 1 / scale) and stored as bf16
 * (fp8 = 0) or OCP fp8 E4M3 bytes (fp8 = 1). For tensor_id == K, each
 * (b, token) is an outlier with probability outlier_rate and its keys are
 * multiplied by outlier_scale. Unused slots get `fill` (its low byte for fp8). */
int synth_fill_kv(uint64_t seed, int tensor_id, int batch, const int32_t* seq_lens, int num_kv_heads, int head_dim,
                  int page_size, int stride, const int32_t* page_table, int64_t num_pages, double outlier_rate,
                  double outlier_scale, int fp8, double inv_scale, uint16_t fill, void* pool, int threads);

/* OCP fp8 E4M3 encoding by round-to-nearest-even, saturating at +-448. */
uint8_t synth_e4m3_from_double(double x);

#ifdef __cplusplus
}
#endif

#endif

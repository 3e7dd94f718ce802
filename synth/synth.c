/*
 * Seeded synthetic inputs for draft-block paged attention.
 *
 * This module only draws numbers and lays them out; it holds none of the
 * attention arithmetic. Both the fp64 oracle and the GPU library consume what
 * it writes, so it is the single source of every test and benchmark input.
 *
 * Generator (counter based, so any element can be drawn on its own):
 *   mix(z)        the SplitMix64 finaliser (Steele, Lea, Flood, "Fast
 *                 splittable pseudorandom number generators", OOPSLA 2014;
 *                 the 64-bit variant published by Vigna as splitmix64.c)
 *   key(s, t)     mix(s * G + mix(t + T0)) for seed s and tensor id t
 *   draw(k, n)    mix(k + (n + 1) * G), the n-th 64-bit word of stream k
 *   normal(k, n)  Box-Muller on the pair of words (2*(n/2), 2*(n/2)+1):
 *                 u1 = (w0 >> 11 + 1) 2^-53 in (0,1], u2 = (w1 >> 11) 2^-53,
 *                 r = sqrt(-2 ln u1); cos(2 pi u2) r for even n, sin for odd n
 *   to bf16       fp64 -> fp32 (round to nearest) -> bf16 (round to nearest even)
 *
 * Tensor ids: q = 1, k = 2, v = 3, page permutation = 4, context lengths = 5,
 * outlier tokens = 6. Logical element indices:
 *   q[b, i, h, d]            ((b*K + i)*Hq + h)*D + d
 *   k, v at (b, j, h_kv, d)  ((b*2^24 + j)*Hkv + h_kv)*D + d
 *   outlier flag of (b, j)   b*2^24 + j
 *
 * Paged layout ("HND"): each pool is [num_pages, Hkv, P, D] bf16. The logical
 * key j of request b lives in page page_table[b, j / P], slot j % P. Pages are
 * dealt from one seeded Fisher-Yates permutation of all used page ids, in
 * consecutive slices to b = 0, 1, ..., so page ranges are disjoint and in
 * random order. The pool holds one extra page (the last id) filled with the
 * fill value; page-table entries past a request's last page point at it, and
 * the unused slots of each request's last page hold the fill value too.
 */
#include "synth.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#define SYNTH_G 0x9E3779B97F4A7C15ULL
#define SYNTH_T0 0x632BE59BD9B4E019ULL
#define SYNTH_TOKEN_SPAN (1ULL << 24)

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, uint64_t tensor) {
    return mix64(seed * SYNTH_G + mix64(tensor + SYNTH_T0));
}

uint64_t synth_draw(uint64_t key, uint64_t n) { return mix64(key + (n + 1) * SYNTH_G); }

double synth_uniform(uint64_t key, uint64_t n) {
    return (double)(synth_draw(key, n) >> 11) * 0x1.0p-53;
}

double synth_normal(uint64_t key, uint64_t n) {
    const uint64_t pair = n >> 1;
    const double u1 = (double)((synth_draw(key, 2 * pair) >> 11) + 1) * 0x1.0p-53;
    const double u2 = (double)(synth_draw(key, 2 * pair + 1) >> 11) * 0x1.0p-53;
    const double r = sqrt(-2.0 * log(u1));
    const double th = 6.283185307179586476925286766559 * u2;
    return (n & 1) ? r * sin(th) : r * cos(th);
}

uint16_t synth_bf16_from_double(double x) {
    float f = (float)x;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* OCP fp8 E4M3 (bias 7, 3 mantissa bits, no infinity, S.1111.111 = NaN) by
 * round-to-nearest-even, saturating at +-448. Input data preparation only. */
uint8_t synth_e4m3_from_double(double x) {
    if (isnan(x)) return 0x7F;
    const uint8_t s = signbit(x) ? 0x80 : 0x00;
    double a = fabs(x);
    if (a >= 448.0) return s | 0x7E;
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: multiples of 2^-9; 8 * 2^-9 is the smallest normal (code 0x08) */
        const double q = nearbyint(ldexp(a, 9));
        return s | (uint8_t)q;
    }
    int e;
    frexp(a, &e); /* a = f * 2^e, f in [0.5, 1): the leading bit is 2^(e-1) */
    e -= 1;
    double q = nearbyint(ldexp(a, 3 - e)); /* 8..16 steps of 2^(e-3) */
    if (q >= 16.0) {
        q = 8.0;
        e += 1;
    }
    if (e > 8 || (e == 8 && q > 14.0)) return s | 0x7E;
    return s | (uint8_t)(((e + 7) << 3) | ((int)q - 8));
}

/* ---------------- q ---------------- */

typedef struct {
    uint64_t key;
    uint16_t* dst;
    uint64_t lo, hi;
} q_job;

static void* q_worker(void* arg) {
    q_job* j = (q_job*)arg;
    for (uint64_t n = j->lo; n < j->hi; ++n) j->dst[n] = synth_bf16_from_double(synth_normal(j->key, n));
    return NULL;
}

static int clamp_threads(int threads) {
    if (threads < 1) return 1;
    if (threads > 256) return 256;
    return threads;
}

void synth_fill_q(uint64_t seed, int64_t count, uint16_t* q, int threads) {
    synth_fill_normal(seed, SYNTH_TENSOR_Q, count, q, threads);
}

void synth_fill_normal(uint64_t seed, int tensor_id, int64_t count, uint16_t* q, int threads) {
    threads = clamp_threads(threads);
    const uint64_t key = synth_key(seed, (uint64_t)tensor_id);
    pthread_t tid[256];
    q_job jobs[256];
    for (int t = 0; t < threads; ++t) {
        jobs[t].key = key;
        jobs[t].dst = q;
        jobs[t].lo = (uint64_t)count * (uint64_t)t / (uint64_t)threads;
        jobs[t].hi = (uint64_t)count * (uint64_t)(t + 1) / (uint64_t)threads;
        pthread_create(&tid[t], NULL, q_worker, &jobs[t]);
    }
    for (int t = 0; t < threads; ++t) pthread_join(tid[t], NULL);
}

/* ---------------- lengths and page tables ---------------- */

void synth_context_lengths(uint64_t seed, int batch, int lo, int hi, int32_t* out) {
    const uint64_t key = synth_key(seed, SYNTH_TENSOR_CTX);
    const uint64_t span = (uint64_t)(hi - lo + 1);
    for (int b = 0; b < batch; ++b) out[b] = lo + (int32_t)(synth_draw(key, (uint64_t)b) % span);
}

int64_t synth_pages_needed(int batch, const int32_t* seq_lens, int page_size) {
    int64_t total = 0;
    for (int b = 0; b < batch; ++b) total += ((int64_t)seq_lens[b] + page_size - 1) / page_size;
    return total + 1; /* + the fill page */
}

int synth_page_table(uint64_t seed, int batch, const int32_t* seq_lens, int page_size, int stride,
                     int32_t* page_table) {
    const int64_t used = synth_pages_needed(batch, seq_lens, page_size) - 1;
    if (used > 0x7FFFFFFF - 1) return -1;
    int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)(used > 0 ? used : 1));
    if (!perm) return -1;
    for (int64_t n = 0; n < used; ++n) perm[n] = (int32_t)n;
    const uint64_t key = synth_key(seed, SYNTH_TENSOR_PERM);
    for (int64_t s = used - 1; s >= 1; --s) {
        const int64_t j = (int64_t)(synth_draw(key, (uint64_t)s) % (uint64_t)(s + 1));
        const int32_t tmp = perm[s];
        perm[s] = perm[j];
        perm[j] = tmp;
    }
    const int32_t fill_page = (int32_t)used;
    int64_t off = 0;
    for (int b = 0; b < batch; ++b) {
        const int64_t np = ((int64_t)seq_lens[b] + page_size - 1) / page_size;
        if (np > stride) {
            free(perm);
            return -2;
        }
        for (int64_t p = 0; p < stride; ++p)
            page_table[(int64_t)b * stride + p] = p < np ? perm[off + p] : fill_page;
        off += np;
    }
    free(perm);
    return 0;
}

/* ---------------- k / v pools ---------------- */

typedef struct {
    uint64_t key, outlier_key;
    double outlier_rate, outlier_scale, inv_scale;
    int batch, num_kv_heads, head_dim, page_size, stride, fp8;
    const int32_t* seq_lens;
    const int32_t* page_table;
    uint16_t fill;
    void* pool;
    int64_t num_pages;
    int32_t* owner_b;  /* per page: request, or -1 for unused pages */
    int32_t* owner_lp; /* per page: logical page index within the request */
    int64_t lo, hi;    /* page range of this worker */
} kv_job;

static void put(const kv_job* j, size_t idx, uint16_t bits) {
    if (j->fp8)
        ((uint8_t*)j->pool)[idx] = (uint8_t)bits;
    else
        ((uint16_t*)j->pool)[idx] = bits;
}

static void* kv_worker(void* arg) {
    kv_job* j = (kv_job*)arg;
    const int P = j->page_size, D = j->head_dim, H = j->num_kv_heads;
    for (int64_t pid = j->lo; pid < j->hi; ++pid) {
        const size_t page = (size_t)pid * (size_t)H * P * D;
        const int b = j->owner_b[pid];
        if (b < 0) {
            for (size_t e = 0; e < (size_t)H * P * D; ++e) put(j, page + e, j->fill);
            continue;
        }
        const int64_t n_b = j->seq_lens[b];
        for (int slot = 0; slot < P; ++slot) {
            const int64_t tok = (int64_t)j->owner_lp[pid] * P + slot;
            int outlier = 0;
            if (tok < n_b && j->outlier_rate > 0.0)
                outlier = synth_uniform(j->outlier_key, (uint64_t)b * SYNTH_TOKEN_SPAN + (uint64_t)tok) < j->outlier_rate;
            for (int h = 0; h < H; ++h) {
                const size_t row = page + ((size_t)h * P + slot) * D;
                if (tok >= n_b) {
                    for (int d = 0; d < D; ++d) put(j, row + d, j->fill);
                    continue;
                }
                const uint64_t base = (((uint64_t)b * SYNTH_TOKEN_SPAN + (uint64_t)tok) * (uint64_t)H + (uint64_t)h) * (uint64_t)D;
                for (int d = 0; d < D; ++d) {
                    double x = synth_normal(j->key, base + (uint64_t)d);
                    if (outlier) x *= j->outlier_scale;
                    x *= j->inv_scale;
                    put(j, row + d, j->fp8 ? synth_e4m3_from_double(x) : synth_bf16_from_double(x));
                }
            }
        }
    }
    return NULL;
}

int synth_fill_kv(uint64_t seed, int tensor_id, int batch, const int32_t* seq_lens, int num_kv_heads, int head_dim,
                  int page_size, int stride, const int32_t* page_table, int64_t num_pages, double outlier_rate,
                  double outlier_scale, int fp8, double inv_scale, uint16_t fill, void* pool, int threads) {
    threads = clamp_threads(threads);
    int32_t* owner_b = (int32_t*)malloc(sizeof(int32_t) * (size_t)num_pages);
    int32_t* owner_lp = (int32_t*)malloc(sizeof(int32_t) * (size_t)num_pages);
    if (!owner_b || !owner_lp) {
        free(owner_b);
        free(owner_lp);
        return -1;
    }
    for (int64_t p = 0; p < num_pages; ++p) owner_b[p] = -1, owner_lp[p] = 0;
    for (int b = 0; b < batch; ++b) {
        const int64_t np = ((int64_t)seq_lens[b] + page_size - 1) / page_size;
        for (int64_t lp = 0; lp < np; ++lp) {
            const int32_t pid = page_table[(int64_t)b * stride + lp];
            if (pid < 0 || pid >= num_pages) {
                free(owner_b);
                free(owner_lp);
                return -2;
            }
            owner_b[pid] = b;
            owner_lp[pid] = (int32_t)lp;
        }
    }
    pthread_t tid[256];
    kv_job jobs[256];
    for (int t = 0; t < threads; ++t) {
        kv_job* j = &jobs[t];
        j->key = synth_key(seed, (uint64_t)tensor_id);
        j->outlier_key = synth_key(seed, SYNTH_TENSOR_OUTLIER);
        j->outlier_rate = tensor_id == SYNTH_TENSOR_K ? outlier_rate : 0.0;
        j->outlier_scale = outlier_scale;
        j->inv_scale = inv_scale;
        j->fp8 = fp8;
        j->batch = batch;
        j->num_kv_heads = num_kv_heads;
        j->head_dim = head_dim;
        j->page_size = page_size;
        j->stride = stride;
        j->seq_lens = seq_lens;
        j->page_table = page_table;
        j->fill = fill;
        j->pool = pool;
        j->num_pages = num_pages;
        j->owner_b = owner_b;
        j->owner_lp = owner_lp;
        j->lo = num_pages * t / threads;
        j->hi = num_pages * (t + 1) / threads;
        pthread_create(&tid[t], NULL, kv_worker, j);
    }
    for (int t = 0; t < threads; ++t) pthread_join(tid[t], NULL);
    free(owner_b);
    free(owner_lp);
    return 0;
}

/*
 * fp64 CPU oracle for draft-block paged attention.
 *
 * TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
 * CPU-baseline leg are its only users. It shares no code, header, table or
 * helper with the GPU library, and the library never calls it.
 *
 * What it computes, written out from the pages' definitions (plain loops, no
 * split-KV, no online softmax, no merge tricks):
 *
 *  - Key set of a draft query. TensorRT-LLM PR #20374 ("non-causal unwindowed
 *    DFlash block attention as decode rows"), Description: with no mask every
 *    query of a request's block attends the same seq_lens_after keys, i.e. the
 *    whole paged context plus the block's own K keys, which were appended to
 *    the cache before attention (the B > 1 comment's "Layer adds the K/V
 *    append"). So request b holds N_b = C_b + K keys and block query i sits at
 *    absolute position p = C_b + i.
 *
 *  - Windowed non-causal form. TensorRT-LLM PR #21130 (DSpark non-causal
 *    windowed draft layer), Description: a causal windowed decode plus a
 *    log-sum-exp merge of the block keys that follow each query. Its key set is
 *    therefore the causal window of p joined with the later block keys:
 *    j in [max(0, p - W + 1), p] and j in (p, min(N_b - 1, p + W_r)], W_r
 *    unbounded when -1. A window of W keys counts p itself; window_right = 0
 *    leaves only the causal part.
 *
 *  - Scores s_j = sm_scale * <q, k_j> in fp64; out = softmax(s) V; the LSE is
 *    base 2, as the decode's LSE that PR #21130's merge updates in place:
 *    lse2 = log2 sum_j exp(s_j) = (m + ln sum_j exp(s_j - m)) / ln 2.
 *
 *  - The merge (PR #21130, Description and its formulation table): two
 *    normalised results over disjoint key sets combine as
 *    lse = log2(2^a + 2^b), out = 2^(a - lse) out_a + 2^(b - lse) out_b.
 *
 *  - Paged reads (PR #20374 sweep setup: page 32, "HND" layout): key j of
 *    request b is slot j mod P of page page_table[b, j / P]; a pool is
 *    [pages, Hkv, P, D]. Query head h reads kv head h / (Hq / Hkv).
 *
 *  - The dense block (TensorRT-LLM PR #16150, the DFlash context kernel fuses the
 *    dense suffix of block keys into the same softmax as the paged context; its
 *    "fused block K/V append" writes them into the pages). With k_block / v_block
 *    given, the K block keys are read from those bf16 arrays instead of the cache;
 *    the key set does not change.
 *
 *  - fp8 context storage (TensorRT-LLM PR #16150, paged DFlash context read from
 *    the target KV cache manager's pool: the kernel supports fp8 context storage,
 *    with bf16 dots and fp32 accumulation). The pages fix no format; read here as
 *    OCP E4M3 bytes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
 *    exponent field 0 encodes subnormals m * 2^-9; S.1111.111 is NaN, there is no
 *    infinity), each standing for scale * value, one scale per pool.
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

double oracle_bf16_to_double(uint16_t bits) {
    const uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double oracle_fp8_e4m3_to_double(uint8_t code) {
    const int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    const double v = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return sign ? -v : v;
}

uint16_t oracle_encode_kv(int kv_dtype, float scale, uint16_t bits) {
    const float x = (float)oracle_bf16_to_double(bits);
    const float q = x / scale; /* IEEE fp32 division */
    if (kv_dtype == ORACLE_KV_FP8_E4M3) {
        /* nearest E4M3 value, ties to the even code, by search over the finite codes */
        if (isnan(q)) return 0x7F;
        const double a = fabs((double)q);
        const uint16_t sign = signbit(q) ? 0x80 : 0x00;
        if (a >= 448.0) return sign | 0x7E;
        int best = 0;
        double best_err = INFINITY;
        for (int c = 0; c <= 0x7E; ++c) {
            const double err = fabs(oracle_fp8_e4m3_to_double((uint8_t)c) - a);
            if (err < best_err || (err == best_err && (c & 1) == 0)) {
                best = c;
                best_err = err;
            }
        }
        return sign | (uint16_t)best;
    }
    /* bf16 of q by round-to-nearest-even (IEEE 754 roundTiesToEven into 8 significand
       bits): the nearer of the two bf16 values around q, the one with an even code on a
       tie. lo is q cut to bf16 and hi the next code away from zero. Past the largest
       finite bf16 (0x7F7F) the next step is infinity, which rounding weighs as the value
       2^128: a magnitude at or beyond the midpoint 2^128 (1 - 2^-9) becomes infinity.
       Every NaN becomes the one quiet NaN 0x7FC0. */
    if (isnan(q)) return 0x7FC0;
    uint32_t u;
    memcpy(&u, &q, sizeof u);
    const uint16_t lo = (uint16_t)(u >> 16), hi = (uint16_t)(lo + 1);
    const double dq = (double)q, dlo = oracle_bf16_to_double(lo);
    const double dhi = (hi & 0x7F80) == 0x7F80 ? copysign(ldexp(1.0, 128), dq) : oracle_bf16_to_double(hi);
    if ((u & 0xFFFFu) == 0) return lo;
    const double elo = fabs(dq - dlo), ehi = fabs(dhi - dq);
    if (elo < ehi) return lo;
    if (ehi < elo) return hi;
    return (lo & 1) ? hi : lo;
}

/* Element d of a K or V row, decoded and scaled. */
static double kv_elem(const oracle_params* prm, const void* pool, int64_t row_elem, int d, double scale) {
    if (prm->kv_dtype == ORACLE_KV_FP8_E4M3) return scale * oracle_fp8_e4m3_to_double(((const uint8_t*)pool)[row_elem + d]);
    return scale * oracle_bf16_to_double(((const uint16_t*)pool)[row_elem + d]);
}

typedef struct {
    const oracle_params* prm;
    int part;
    const uint16_t* q;
    const void *k, *v;
    const int32_t *pt, *lens;
    const int32_t* rows; /* triples (b, i, h) */
    int64_t n_rows;
    double *out, *lse2;
    int64_t next;
    pthread_mutex_t lock;
    int64_t max_keys;
} oracle_job;

/* Element index of the first element of key j's row (kv head hk) in a pool. */
static int64_t key_row(const oracle_params* prm, const int32_t* pt, int b, int hk, int64_t j) {
    const int64_t page = pt[(int64_t)b * prm->page_table_stride + j / prm->page_size];
    const int64_t slot = j % prm->page_size;
    return ((page * prm->num_kv_heads + hk) * prm->page_size + slot) * prm->head_dim;
}

static void one_row(oracle_job* job, int b, int i, int h, double* s) {
    const oracle_params* prm = job->prm;
    const int K = prm->block_size, D = prm->head_dim, Hq = prm->num_q_heads;
    const int g = prm->num_q_heads / prm->num_kv_heads;
    const int hk = h / g;
    const int64_t n = job->lens[b];
    const int64_t p = n - K + i;

    int64_t lo = prm->window_left < 0 ? 0 : p - prm->window_left + 1;
    if (lo < 0) lo = 0;
    int64_t hi = prm->window_right < 0 ? n - 1 : p + prm->window_right;
    if (hi > n - 1) hi = n - 1;
    if (job->part == ORACLE_PART_CAUSAL && hi > p) hi = p;
    if (job->part == ORACLE_PART_FUTURE && lo < p + 1) lo = p + 1;

    const int64_t row = ((int64_t)b * K + i) * Hq + h;
    double* o = job->out + row * D;
    if (lo > hi) {
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        job->lse2[row] = -INFINITY;
        return;
    }

    const uint16_t* qr = job->q + row * D;
    double qd[1024];
    for (int d = 0; d < D; ++d) qd[d] = oracle_bf16_to_double(qr[d]);

    double m = -INFINITY;
    for (int64_t j = lo; j <= hi; ++j) {
        double dot = 0.0;
        if (prm->k_block && j >= n - K) {
            const uint16_t* kb = prm->k_block + (((int64_t)b * K + (j - (n - K))) * prm->num_kv_heads + hk) * D;
            for (int d = 0; d < D; ++d) dot += qd[d] * oracle_bf16_to_double(kb[d]);
        } else {
            const int64_t kr = key_row(prm, job->pt, b, hk, j);
            for (int d = 0; d < D; ++d) dot += qd[d] * kv_elem(prm, job->k, kr, d, prm->k_scale);
        }
        s[j - lo] = prm->sm_scale * dot;
        if (s[j - lo] > m) m = s[j - lo];
    }
    double z = 0.0;
    double acc[1024];
    for (int d = 0; d < D; ++d) acc[d] = 0.0;
    for (int64_t j = lo; j <= hi; ++j) {
        const double e = exp(s[j - lo] - m);
        z += e;
        if (prm->v_block && j >= n - K) {
            const uint16_t* vb = prm->v_block + (((int64_t)b * K + (j - (n - K))) * prm->num_kv_heads + hk) * D;
            for (int d = 0; d < D; ++d) acc[d] += e * oracle_bf16_to_double(vb[d]);
        } else {
            const int64_t vr = key_row(prm, job->pt, b, hk, j);
            for (int d = 0; d < D; ++d) acc[d] += e * kv_elem(prm, job->v, vr, d, prm->v_scale);
        }
    }
    for (int d = 0; d < D; ++d) o[d] = acc[d] / z;
    job->lse2[row] = (m + log(z)) / log(2.0);
}

static void* worker(void* arg) {
    oracle_job* job = (oracle_job*)arg;
    double* s = (double*)malloc(sizeof(double) * (size_t)(job->max_keys > 0 ? job->max_keys : 1));
    if (!s) return NULL;
    for (;;) {
        pthread_mutex_lock(&job->lock);
        const int64_t r = job->next++;
        pthread_mutex_unlock(&job->lock);
        if (r >= job->n_rows) break;
        one_row(job, job->rows[3 * r], job->rows[3 * r + 1], job->rows[3 * r + 2], s);
    }
    free(s);
    return NULL;
}

int oracle_attention(const oracle_params* prm, int part, const uint16_t* q, const void* k_pool,
                     const void* v_pool, const int32_t* page_table, const int32_t* seq_lens,
                     const int32_t* pairs, int n_pairs, double* out, double* lse2, int threads) {
    if (!prm || !q || !k_pool || !v_pool || !page_table || !seq_lens || !out || !lse2) return -1;
    if (prm->batch < 1 || prm->block_size < 1 || prm->num_kv_heads < 1 || prm->num_q_heads < 1 ||
        prm->num_q_heads % prm->num_kv_heads != 0 || prm->head_dim < 1 || prm->head_dim > 1024 ||
        prm->page_size < 1 || prm->page_table_stride < 1 || prm->num_pages < 1)
        return -1;
    if (part < ORACLE_PART_ALL || part > ORACLE_PART_FUTURE) return -1;
    if (prm->kv_dtype != ORACLE_KV_BF16 && prm->kv_dtype != ORACLE_KV_FP8_E4M3) return -1;
    if (!isfinite(prm->k_scale) || !isfinite(prm->v_scale)) return -1;
    if ((prm->k_block == NULL) != (prm->v_block == NULL)) return -1;
    if (prm->window_left == 0 || prm->window_left < -1 || prm->window_right < -1) return -1;

    int64_t max_keys = 0;
    for (int b = 0; b < prm->batch; ++b) {
        const int64_t n = seq_lens[b];
        if (n < prm->block_size) return -1;
        const int64_t np = (n + prm->page_size - 1) / prm->page_size;
        if (np > prm->page_table_stride) return -1;
        for (int64_t lp = 0; lp < np; ++lp) {
            const int32_t pid = page_table[(int64_t)b * prm->page_table_stride + lp];
            if (pid < 0 || pid >= prm->num_pages) return -1;
        }
        if (n > max_keys) max_keys = n;
    }

    const int g = prm->num_q_heads / prm->num_kv_heads;
    const int64_t per_pair = (int64_t)prm->block_size * g;
    const int64_t np_all = (int64_t)prm->batch * prm->num_kv_heads;
    const int64_t npairs = pairs ? n_pairs : np_all;
    int32_t* rows = (int32_t*)malloc(sizeof(int32_t) * 3 * (size_t)(npairs * per_pair > 0 ? npairs * per_pair : 1));
    if (!rows) return -1;
    int64_t nr = 0;
    for (int64_t pi = 0; pi < npairs; ++pi) {
        const int b = pairs ? pairs[2 * pi] : (int)(pi / prm->num_kv_heads);
        const int hk = pairs ? pairs[2 * pi + 1] : (int)(pi % prm->num_kv_heads);
        if (b < 0 || b >= prm->batch || hk < 0 || hk >= prm->num_kv_heads) {
            free(rows);
            return -1;
        }
        for (int i = 0; i < prm->block_size; ++i)
            for (int l = 0; l < g; ++l) {
                rows[3 * nr] = b;
                rows[3 * nr + 1] = i;
                rows[3 * nr + 2] = hk * g + l;
                ++nr;
            }
    }

    oracle_job job;
    job.prm = prm;
    job.part = part;
    job.q = q;
    job.k = k_pool;
    job.v = v_pool;
    job.pt = page_table;
    job.lens = seq_lens;
    job.rows = rows;
    job.n_rows = nr;
    job.out = out;
    job.lse2 = lse2;
    job.next = 0;
    job.max_keys = max_keys;
    pthread_mutex_init(&job.lock, NULL);

    if (threads < 1) threads = 1;
    if (threads > 256) threads = 256;
    pthread_t tid[256];
    for (int t = 0; t < threads; ++t) pthread_create(&tid[t], NULL, worker, &job);
    for (int t = 0; t < threads; ++t) pthread_join(tid[t], NULL);
    pthread_mutex_destroy(&job.lock);
    free(rows);
    return 0;
}

void oracle_merge(int64_t rows, int32_t head_dim, const double* out_a, const double* lse_a, const double* out_b,
                  const double* lse_b, double* out, double* lse) {
    for (int64_t r = 0; r < rows; ++r) {
        const double a = lse_a[r], b = lse_b[r];
        double l;
        if (a == -INFINITY && b == -INFINITY)
            l = -INFINITY;
        else
            l = (a > b ? a : b) + log2(1.0 + exp2(-fabs(a - b)));
        const double wa = a == -INFINITY ? 0.0 : exp2(a - l);
        const double wb = b == -INFINITY ? 0.0 : exp2(b - l);
        for (int d = 0; d < head_dim; ++d)
            out[r * head_dim + d] = wa * out_a[r * head_dim + d] + wb * out_b[r * head_dim + d];
        lse[r] = l;
    }
}

/*
 * blockattn: draft-block attention over a paged bf16 KV cache, for MI355X (gfx950).
 *
 * A speculative-decoding drafter proposes a block of K draft tokens per
 * request. Each of the K block queries (times the GQA group, so R = K * Hq/Hkv
 * query rows per KV head, any number) attends to the request's paged context
 * plus the K block keys, which are already appended to the cache.
 *
 *  - blockattn_forward: the non-causal unwindowed form. Every block query of a
 *    request sees the same N_b = seq_lens[b] keys (TensorRT-LLM PR #20374, on
 *    unwindowed DFlash block attention, Description: without a mask every block
 *    query attends to all keys present after the append).
 *  - blockattn_windowed_forward: the non-causal windowed form: a causal
 *    windowed decode with a base-2 LSE, and the log-sum-exp merge of the block
 *    keys that follow each query (TensorRT-LLM PR #21130, DSpark non-causal
 *    windowed draft layer, Description items 1-2). Those keys lie in the tiles
 *    the decode already streams, so the merge is done by the decode's own online
 *    softmax update rather than by a second pass. With K = 1 or window_right = 0
 *    no block key follows any query and the causal result is returned as is.
 *  - blockattn_forward_block: either form with the block's own keys and values
 *    taken from dense arrays, optionally appended to the cache in the same call.
 *  - blockattn_merge: the log-sum-exp merge of partial results over disjoint key
 *    sets, such as the shards of a context split across GPUs.
 *
 * Definitions (p = N_b - K + i is the absolute position of block query i):
 *   s_j  = sm_scale * <q[b,i,h,:], k_j>, with k_j read through the page table
 *   key set, unwindowed: j in [0, N_b)
 *   key set, windowed:   j in [max(0, p - W + 1), p]  (the causal window, W keys
 *                        including p) joined with j in (p, min(N_b - 1, p + W_r)]
 *                        (W_r = -1: every later block key)
 *   out[b,i,h,:] = sum_j softmax(s)_j v_j,   lse[b,i,h] = log2 sum_j exp(s_j)
 *
 * Layouts (all contiguous, row-major, device memory unless stated):
 *   q, out      bf16 [B, K, Hq, D]
 *   k_cache,    [num_pages, Hkv, P, D] each ("HND" pages, PR #20374 sweep
 *   v_cache          setup) of bf16, or of fp8 E4M3 bytes (kv_dtype); key j of
 *                    request b is slot j % P of page page_table[b, j / P]; a
 *                    stored key stands for k_scale * k, a value for v_scale * v
 *   page_table  int32 [B, page_table_stride]; entries past ceil(N_b / P) are
 *               never read
 *   seq_lens    int32 [B] = C_b + K, context plus the appended block
 *   lse         fp32 [B, K, Hq], base 2
 *   Query head h uses kv head h / (Hq / Hkv).
 *
 * Ownership: the caller owns every device buffer, the workspace and the stream.
 * The library owns only the plan (a host object). Nothing is allocated on the
 * device by a forward call, and a forward call never synchronises the host, so
 * it can be captured in a HIP graph.
 *
 * Errors: every entry point returns a blockattn_status. On any error nothing is
 * launched, and blockattn_last_error() (thread-local) names the offending field
 * and how to fix it.
 */
#ifndef BLOCKATTN_H
#define BLOCKATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum blockattn_status {
    BLOCKATTN_OK = 0,
    BLOCKATTN_ERR_INVALID_ARGUMENT = 1,  /* a shape, length, pointer or window out of range */
    BLOCKATTN_ERR_UNSUPPORTED = 2,       /* a valid shape the library has no kernel for (D, P, R) */
    BLOCKATTN_ERR_WORKSPACE_TOO_SMALL = 3,
    BLOCKATTN_ERR_PLAN_MISMATCH = 4,     /* forward kind or workspace differs from the plan's */
    BLOCKATTN_ERR_HIP = 5                /* the HIP runtime reported an error */
} blockattn_status;

typedef struct blockattn_params {
    int32_t batch;             /* B >= 1 requests */
    int32_t block_size;        /* K draft queries per request, 1..16 */
    int32_t num_q_heads;       /* Hq, a multiple of Hkv */
    int32_t num_kv_heads;      /* Hkv >= 1 */
    int32_t head_dim;          /* D: 64 or 128 */
    int32_t page_size;         /* P tokens per page: 16, 32, 64, 128 or 256 */
    int32_t page_table_stride; /* int32 entries per page-table row, >= ceil(N_b / P) */
    int32_t num_pages;         /* pages in each pool; page ids must lie in [0, num_pages) */
    int32_t window_left;       /* -1: unwindowed form; W >= 1: windowed form, causal window of W keys */
    int32_t window_right;      /* windowed form: -1 every later block key, 0 none, > 0 at most that many.
                                  Must be -1 for the unwindowed form. */
    float sm_scale;            /* softmax scale, finite and > 0 (usually 1/sqrt(D)) */
    int32_t splits_override;   /* 0: automatic split count. > 0: exactly that many KV splits per
                                  (request, kv head), clamped to the request's 32-token tile count
                                  (for testing split invariance and tuning) */
    int32_t waves_override;    /* 0: automatic. > 0: wavefronts per workgroup (1..8): token groups when
                                  R <= 32, row-waves (one or two row blocks each) when R > 32; at
                                  D = 128 with seven or eight 16-row blocks, a count above the block
                                  count selects two token groups of four two-block waves, and with
                                  three blocks two token groups of four one-block waves, one of them
                                  rowless (tuning). Automatic at D = 128: two token groups for seven
                                  or eight blocks once the batch holds at least 8 tiles per CU; four
                                  waves (one rowless) at three blocks, as two token groups with fp8
                                  pools once the batch holds at least 64 tiles per CU */
    int32_t kv_dtype;          /* element type of k_cache and v_cache: BLOCKATTN_KV_BF16, or
                                  BLOCKATTN_KV_FP8_E4M3 (OCP fp8 E4M3 bytes: 1 sign, 4 exponent bits
                                  with bias 7, 3 mantissa bits, S.1111.111 = NaN; TensorRT-LLM PR #16150,
                                  the paged DFlash context kernel supports fp8 context storage) */
    float k_scale;             /* finite and > 0: a stored key element stands for k_scale times its
                                  value (1 for an unscaled cache) */
    float v_scale;             /* finite: a stored value element stands for v_scale times its value */
    int32_t combine_mode;      /* how the splits of a split request are combined (TensorRT-LLM PR #20374,
                                  Description: the multi-CTA split-KV decode combines its splits through
                                  counter buffers): BLOCKATTN_COMBINE_AUTO (0) lets the plan choose (the
                                  combine kernel, the faster of the two wherever measured on MI355X);
                                  BLOCKATTN_COMBINE_KERNEL (1) launches a separate combine kernel;
                                  BLOCKATTN_COMBINE_LAST_ARRIVER (2) has the last split of each
                                  (request, kv head) to finish combine them inside the attention kernel,
                                  found by a per-(request, kv head) arrival counter in the workspace
                                  (any split count; that unit reads every partial of its pair, so it
                                  pays off only at few, narrow splits) */
} blockattn_params;

enum { BLOCKATTN_COMBINE_AUTO = 0, BLOCKATTN_COMBINE_KERNEL = 1, BLOCKATTN_COMBINE_LAST_ARRIVER = 2 };

enum { BLOCKATTN_KV_BF16 = 0, BLOCKATTN_KV_FP8_E4M3 = 1 };

typedef struct blockattn_plan_s* blockattn_plan_t;

typedef struct blockattn_plan_info {
    int32_t kind;              /* 0 unwindowed, 1 windowed */
    int32_t units;             /* work units (workgroups) of the split-KV partial kernel */
    int32_t max_splits;        /* largest split count of any (request, kv head) */
    int32_t merge_active;      /* 1 when block keys after a query join its key set (windowed, K > 1,
                                  window_right != 0) */
    int32_t waves_per_unit;    /* wavefronts per workgroup of the partial kernel */
    int32_t token_groups;      /* wavefronts streaming different tiles inside one workgroup */
    int32_t row_waves;         /* wavefronts sharing one tile, each owning some query rows */
    int32_t uploaded;          /* 1 once the work list has been copied into a workspace */
    int32_t combine_launch;    /* 1: a combine kernel follows the attention kernel (some request has
                                  more than one split); 0: every split wrote its output directly */
    int32_t shared_tiles;      /* 1: each workgroup loads a tile once into LDS for all its row waves
                                  (R > 32); 0: each wave streams its own tiles */
    int32_t row_groups;        /* work units per (request, kv head, split): 1 up to 128 query rows per
                                  kv head; above that the rows are split into this many groups of at
                                  most 128, each reading the kv head's keys */
    int32_t fused_combine;     /* 1: split requests are combined inside the attention kernel by the last
                                  split to finish (no combine launch); 0: by the combine kernel, if any */
    size_t workspace_bytes;    /* bytes the plan needs */
} blockattn_plan_info_t;

/*
 * Exact workspace bytes needed for these parameters and host lengths: the
 * split-KV work list, the per-(request, kv head) table and arrival counters, the
 * input-error word and the fp32 partial softmax states (acc, m, l) of every work
 * unit. The size is
 * computed from the same plan a forward runs, so the softmax statistics can never
 * outgrow their carve (TensorRT-LLM PR #21130, Description item 3: the workspace
 * must hold the stats, and a launch is refused when it is too small).
 * seq_lens_host: int32 [B] on the host. Returns BLOCKATTN_OK and sets *bytes;
 * invalid parameters give the same errors as blockattn_plan.
 */
int blockattn_workspace_size(const blockattn_params* params, const int32_t* seq_lens_host, size_t* bytes);

/*
 * Validate, choose the split-KV decomposition for gfx950 and lay out the
 * workspace: the planning step of the pages' multi-CTA split-KV decode
 * (TensorRT-LLM PR #20374, Description: decode rows take the paged split-KV
 * path with its counter buffers; PR #16150, commit list: the split count of the
 * paged context kernel is a runtime argument). seq_lens_host fixes the split
 * counts; forward reads the live lengths from device memory, so the lengths may
 * change between forwards (for example under graph replay) as long as every
 * N_b stays in [K, page_table_stride * P]. A live length outside that range is
 * clamped into it and recorded in the input-error word (blockattn_input_errors).
 * workspace: device buffer of workspace_bytes, or NULL for a host-only plan
 * (info and validation only; such a plan cannot run). With a workspace, one
 * asynchronous host-to-device copy of the work list is enqueued on stream
 * (a hipStream_t, NULL = default stream). The plan must outlive that copy;
 * blockattn_plan_destroy waits for it.
 * Streams: a forward on that same stream is ordered after the copy by the
 * stream. A forward on another stream first waits for the copy on the device
 * (an event wait, no host synchronisation). A forward captured into a graph on
 * another stream cannot wait on the copy's event: the copy must have completed
 * before such a capture begins (for example after synchronising the plan's
 * stream; torch.cuda.graph synchronises the device when capture starts).
 * A plan is not safe for concurrent use from several host threads.
 * On success *plan holds a new plan owned by the caller.
 */
int blockattn_plan(const blockattn_params* params, const int32_t* seq_lens_host, void* workspace,
                   size_t workspace_bytes, void* stream, blockattn_plan_t* plan);

/*
 * Non-causal unwindowed block attention (the plan must have window_left = -1).
 * q: bf16, k_cache and v_cache: kv_dtype device buffers (layouts above); page_table,
 * seq_lens: int32 device buffers; workspace: the buffer given to the plan;
 * out: bf16 [B, K, Hq, D]; lse: fp32 [B, K, Hq] or NULL; stream: hipStream_t.
 * Launch only: no allocation, no host synchronisation.
 * Out-of-range device inputs never lead to reads outside the caller's buffers:
 * a page id outside [0, num_pages) is clamped into that range and a length
 * outside [K, page_table_stride * P] into that one. The result is then not the
 * one the inputs describe, and the clamp is recorded in the workspace's
 * input-error word, which blockattn_input_errors reads.
 */
int blockattn_forward(blockattn_plan_t plan, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* page_table, const int32_t* seq_lens, void* workspace, void* out, float* lse,
                      void* stream);

/*
 * Non-causal windowed block attention (the plan must have window_left >= 1):
 * the causal windowed split-KV decode with the block keys after each query
 * folded into the same online softmax (the log-sum-exp merge, applied to the
 * running state), then the split combine. Same arguments as blockattn_forward;
 * lse is required and receives the final, merged base-2 LSE.
 */
int blockattn_windowed_forward(blockattn_plan_t plan, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* page_table, const int32_t* seq_lens, void* workspace, void* out,
                               float* lse, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): blockattn_forward or
 * blockattn_windowed_forward, whichever the plan's kind is, with no workspace
 * argument. The work list and the partial softmax states go to a library-owned
 * device array of BLOCKATTN_SCRATCH_BYTES on each GPU, laid out as a workspace and
 * held until the process ends. The call allocates nothing: the array's address is
 * looked up once per device (when a plan is made, or at the first call there).
 *   plan     from blockattn_plan, with or without a workspace; its workspace_bytes
 *            (blockattn_plan_info) must not exceed BLOCKATTN_SCRATCH_BYTES, else
 *            BLOCKATTN_ERR_WORKSPACE_TOO_SMALL and nothing is launched
 *   others   as for blockattn_forward (lse required for a windowed plan)
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap on one GPU (on concurrent streams, or graph replays
 * running at the same time) race and give wrong results; order them. A plan whose
 * requests have different split counts copies its work list (a few KB) from the
 * plan's pinned host copy into the array on `stream` at each call, so such a plan
 * must outlive every call and every replay of a graph that captured one. The
 * array's input-error word is not reported (blockattn_input_errors reads a
 * workspace).
 */
#define BLOCKATTN_SCRATCH_BYTES ((size_t)32 << 20)
int blockattn_forward_scratch(blockattn_plan_t plan, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* page_table, const int32_t* seq_lens, void* out, float* lse,
                              void* stream);

/*
 * Block attention with the block's own keys and values given as dense bf16
 * arrays, either plan kind (TensorRT-LLM PR #16150: the paged DFlash context
 * kernel fuses the dense suffix of block keys into the same softmax, and the
 * K/V of the block are appended to the cache just before attention).
 *   k_block, v_block  bf16 [B, K, Hkv, D]: the keys and values at positions
 *                     C_b .. C_b + K - 1, read from here instead of the cache
 *                     (unscaled); the key set is the same as the plan kind's.
 *   append            0: the cache is only read (its block slots may hold
 *                     anything). 1: the call also stores the block into its
 *                     cache slots (page_table[b, j / P], slot j % P), each element
 *                     as fp32(x) / fp32(scale) rounded to the pool's type (bf16,
 *                     or E4M3 by nearest-even saturating at +-448), so the next
 *                     step finds it there.
 * Other arguments as for blockattn_forward / blockattn_windowed_forward (lse
 * required for a windowed plan). k_cache and v_cache are written only with
 * append = 1, and only at the block slots. Requires v_scale != 0 with a finite
 * fp32 reciprocal (the block values join the scaled cache values as v / v_scale:
 * each probability of a block key is multiplied by 1 / v_scale before its bf16
 * rounding, which is exact when v_scale is a power of two).
 */
int blockattn_forward_block(blockattn_plan_t plan, const void* q, const void* k_block, const void* v_block,
                            void* k_cache, void* v_cache, const int32_t* page_table, const int32_t* seq_lens,
                            void* workspace, void* out, float* lse, int32_t append, void* stream);

/*
 * Merge G partial results of the same rows computed over disjoint key sets, such as
 * the shards of a context split across GPUs, after gathering each shard's out and LSE
 * (the log-sum-exp merge of TensorRT-LLM PR #21130, Description item 1, taken over G
 * parts): M = max_g lse_g, w_g = 2^(lse_g - M), out = sum_g w_g out_g / sum_g w_g,
 * lse = M + log2 sum_g w_g. A part with lse = -inf holds no keys and weighs 0.
 *   parts      G >= 1 (at most 4096)
 *   rows       rows per part (B * K * Hq for forward results); 0 launches nothing
 *   head_dim   64 or 128
 *   part_out   bf16 [G, rows, head_dim], each part normalised (as forward returns it)
 *   part_lse   fp32 [G, rows], base 2
 *   out        bf16 [rows, head_dim]; must not overlap part_out
 *   lse        fp32 [rows] or NULL
 * Device pointers; launch only on stream (hipStream_t, NULL = default): no allocation,
 * no host synchronisation.
 */
int blockattn_merge(int32_t parts, int64_t rows, int32_t head_dim, const void* part_out, const float* part_lse,
                    void* out, float* lse, void* stream);

/*
 * Describe the plan: the path taken (kernel, units, splits, whether a combine
 * launch follows, whether the block keys after each query are merged). Tests use it
 * to assert which path runs, as the pages' tests count the calls of each
 * path (TensorRT-LLM PR #20374, Test Coverage: the row path is checked by counting
 * which kernels a step calls). Returns BLOCKATTN_ERR_INVALID_ARGUMENT for NULL
 * arguments; reads only the host plan.
 */
int blockattn_plan_info(blockattn_plan_t plan, blockattn_plan_info_t* info);

/*
 * Profiling aid: per-phase timestamps of the split-KV partial kernel. With a
 * device buffer of at least units * 8 uint64 (units from blockattn_plan_info),
 * every later forward on this plan has each work unit (workgroup) write, after
 * its memory operations in flight have completed, the 100 MHz constant GPU clock
 * at: [0] kernel entry, [1] its sequence length loaded, [2] its first window of
 * page ids staged, [3] token group 0's tile loop done, [4] all token groups done
 * (multi-group units only), [5] its output or partial stored; [6] and [7] are
 * unused. Entry u * 8 + k is unit u's phase k. The waits make traced calls a
 * little slower. NULL stops tracing. Not for use during graph capture.
 * Returns BLOCKATTN_ERR_WORKSPACE_TOO_SMALL when the buffer is too small.
 */
int blockattn_plan_set_phase_trace(blockattn_plan_t plan, void* trace, size_t bytes);

/* Bits of the input-error word. */
enum {
    BLOCKATTN_INPUT_BAD_LENGTH = 1, /* a device seq_lens entry was outside [K, page_table_stride * P] */
    BLOCKATTN_INPUT_BAD_PAGE = 2    /* a page-table entry a call read was outside [0, num_pages) */
};

/*
 * Checked mode for debugging callers: report which out-of-range device inputs the
 * forwards on this plan's workspace met since the last call (or since the plan
 * was made), then clear the record. The forwards clamp such inputs so that no read
 * leaves the caller's buffers. The pages ask that a bad shape raise a clear,
 * actionable error (TensorRT-LLM PR #16150, commit list); this is that rule for the
 * inputs only the device sees.
 *   workspace  the buffer given to the plan
 *   stream     the stream the forwards ran on (hipStream_t); the call is ordered
 *              after them, waits on the host for the read-back, and must not be
 *              made during graph capture
 *   flags      receives BLOCKATTN_INPUT_BAD_LENGTH | BLOCKATTN_INPUT_BAD_PAGE, or 0
 */
int blockattn_input_errors(blockattn_plan_t plan, void* workspace, void* stream, int32_t* flags);

/*
 * Profiling aid. When before/after are non-NULL hipEvent_t handles, every later
 * forward on this plan records `before` on its stream right before the split-KV
 * partial kernel and `after` right after it, so a caller can time that kernel
 * alone with hipEventElapsedTime. Pass NULL, NULL to stop. Adds no device work.
 */
int blockattn_plan_set_profile_events(blockattn_plan_t plan, void* before, void* after);

/*
 * Measurement aid: the read-only streaming reference. Reads every byte of src once
 * with the 16-byte non-temporal vector loads the attention kernels use for K and V
 * and XOR-folds the words into *result (so no load is dropped); writes nothing
 * else. Timed over a buffer far larger than the caches (2 GiB), it gives the HBM
 * read rate a plain kernel reaches, the yardstick for the attention kernels' KV
 * read rate.
 *   src         device buffer, 16-byte aligned
 *   bytes       a positive multiple of 16
 *   result      device uint32; the caller zeroes it first if it wants the fold's value
 *   workgroups  256-thread workgroups, each reading one contiguous range (0: 1024)
 *   stream      hipStream_t. Launch only: no allocation, no host synchronisation.
 */
int blockattn_stream_read(const void* src, size_t bytes, uint32_t* result, int32_t workgroups, void* stream);

/* Wait for the plan's pending work-list copy, then free it. NULL is ignored. */
void blockattn_plan_destroy(blockattn_plan_t plan);

/* Message of the last error on the calling thread ("" if none). */
const char* blockattn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BLOCKATTN_H */

// Host side of blockattn: validation, the gfx950 split-KV plan, workspace layout
// and the C ABI declared in include/blockattn.h.
//
// The plan replaces two host decisions of the pages' designs: the batch-size
// gate between decode rows and context FMHA (TensorRT-LLM PR #20374,
// Description: the row form wins at small batch because it gives multi-CTA
// split-KV), and the split count of the paged split-KV kernel (PR #16150, commit
// list: a flash-decoding style rework whose split count became a runtime
// argument). Here one kernel covers every batch: the plan picks the tiles per
// split that minimise an estimated makespan on the 256 gfx950 compute units (each
// CU's tiles at its own rate, a fixed cost per round of resident units, and the
// combine launch when any request is split), so every split keeps enough keys that
// its fp32 partial state stays small next to the KV bytes it reads. The workspace is
// sized exactly and checked before anything launches, the lesson of PR #21130's
// workspace item 3 (a stats carve that outgrew its buffer).
#include "blockattn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "internal.h"

using namespace blockattn;

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
    g_last_error = msg;
    return code;
}

constexpr int kNumCUs = 256;
constexpr size_t kReadback = 256;  // pinned bytes after the staged head, for reading the error word back
constexpr size_t kLdsPerCU = 160 * 1024;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace sections, each 256-byte aligned. The head (work list, pair table and the
// input-error word) is what the plan uploads; the partials follow it.
struct Layout {
    size_t work = 0, pairs = 0, cnt = 0, err = 0, m = 0, l = 0, acc = 0, total = 0;
};


}  // namespace

int blockattn::record_error(int code, const char* msg) { return fail(code, msg); }

struct blockattn_plan_s {
    blockattn_params prm{};
    int kind = 0;
    int g = 1, R = 1, NB = 1;  // R: query rows per work unit (NB 16-row blocks)
    int R_all = 1, G = 1;      // query rows per kv head, split into G row groups of R
    KernelShape shape{};
    bool merge_active = false;
    bool fused = false;  // split pairs combined in the attention kernel by their last unit
    int units = 0, max_splits = 0;
    int uniform_splits = 0;  // > 0 when every (request, kv head) has this split count
    std::vector<WorkItem> work;
    std::vector<int32_t> pair_table;
    Layout lay;
    void* ws = nullptr;
    bool uploaded = false;
    void* stage = nullptr;             // pinned host copy of the workspace head, then 256 bytes of read-back
    hipEvent_t copy_done = nullptr;    // recorded after the head's upload on upload_stream
    hipStream_t upload_stream = nullptr;
    bool upload_seen_done = false;     // copy_done has been observed complete: no stream needs to wait on it
    hipEvent_t scratch_copy_done = nullptr;  // recorded after each copy of the stage into the scratch array
    hipEvent_t prof_before = nullptr, prof_after = nullptr;
    uint64_t* trace = nullptr;  // per-unit phase timestamps (profiling aid), or NULL
};

namespace {

int validate(const blockattn_params* p, const int32_t* lens) {
    if (!p) return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "params is NULL");
    if (!lens) return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "seq_lens_host is NULL; pass the host copy of the lengths");
    if (p->batch < 1) return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "batch must be >= 1");
    if (p->block_size < 1 || p->block_size > 16)
        return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "block_size must be in [1, 16]");
    if (p->num_kv_heads < 1 || p->num_q_heads < 1 || p->num_q_heads % p->num_kv_heads != 0)
        return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "num_q_heads must be a positive multiple of num_kv_heads >= 1");
    if (p->head_dim != 64 && p->head_dim != 128)
        return fail(BLOCKATTN_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (the gfx950 kernels are built for those)");
    // Any power of two from 16 (half a 32-token tile, so a half never spans two pages) to
    // 256 (a target pool's page size when the draft context lives in the target's pool).
    if (p->page_size < 16 || p->page_size > 256 || (p->page_size & (p->page_size - 1)) != 0)
        return fail(BLOCKATTN_ERR_UNSUPPORTED, "page_size must be 16, 32, 64, 128 or 256 tokens");
    const int g = p->num_q_heads / p->num_kv_heads;
    (void)g;  // any row count: more than 128 rows per kv head run as several row groups
    if (p->page_table_stride < 1) return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "page_table_stride must be >= 1");
    if (p->num_pages < 1) return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "num_pages must be >= 1");
    if ((int64_t)p->num_pages * p->num_kv_heads > INT32_MAX)
        return fail(BLOCKATTN_ERR_UNSUPPORTED, "num_pages * num_kv_heads must stay below 2^31 (pool slabs are int32)");
    if (!(std::isfinite(p->sm_scale) && p->sm_scale > 0.f))
        return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "sm_scale must be finite and > 0");
    if (p->kv_dtype != BLOCKATTN_KV_BF16 && p->kv_dtype != BLOCKATTN_KV_FP8_E4M3)
        return fail(BLOCKATTN_ERR_UNSUPPORTED, "kv_dtype must be BLOCKATTN_KV_BF16 (0) or BLOCKATTN_KV_FP8_E4M3 (1)");
    if (!(std::isfinite(p->k_scale) && p->k_scale > 0.f))
        return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "k_scale must be finite and > 0 (1 for an unscaled cache)");
    if (!std::isfinite(p->v_scale))
        return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "v_scale must be finite (1 for an unscaled cache)");
    if (!(std::isfinite((double)p->sm_scale * p->k_scale * 1.4426950408889634) &&
          (float)((double)p->sm_scale * p->k_scale * 1.4426950408889634) > 0.f))
        return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "sm_scale * k_scale must stay a finite, non-zero fp32 value");
    if (p->window_left == 0 || p->window_left < -1)
        return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "window_left must be -1 (unwindowed) or >= 1 keys");
    if (p->window_right < -1) return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "window_right must be >= -1");
    if (p->window_left == -1 && p->window_right != -1)
        return fail(BLOCKATTN_ERR_INVALID_ARGUMENT,
                    "window_right must be -1 for the unwindowed form (window_left = -1)");
    if (p->splits_override < 0) return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "splits_override must be >= 0");
    if (p->waves_override < 0 || p->waves_override > kMaxWaves)
        return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "waves_override must be in [0, 8]");
    if (p->combine_mode < BLOCKATTN_COMBINE_AUTO || p->combine_mode > BLOCKATTN_COMBINE_LAST_ARRIVER)
        return fail(BLOCKATTN_ERR_INVALID_ARGUMENT,
                    "combine_mode must be BLOCKATTN_COMBINE_AUTO (0), _KERNEL (1) or _LAST_ARRIVER (2)");
    const long max_keys = (long)p->page_table_stride * p->page_size;
    if (max_keys > (1L << 30))
        return fail(BLOCKATTN_ERR_UNSUPPORTED, "page_table_stride * page_size must be <= 2^30 keys");
    for (int b = 0; b < p->batch; ++b) {
        if (lens[b] < p->block_size) {
            char buf[160];
            snprintf(buf, sizeof buf, "seq_lens[%d] = %d is below block_size %d: lengths count context + block keys",
                     b, lens[b], p->block_size);
            return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, buf);
        }
        if ((long)lens[b] > max_keys) {
            char buf[160];
            snprintf(buf, sizeof buf, "seq_lens[%d] = %d needs more than page_table_stride = %d pages of %d tokens",
                     b, lens[b], p->page_table_stride, p->page_size);
            return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, buf);
        }
    }
    return BLOCKATTN_OK;
}

// Key tiles a request needs: 32-token tiles covering the union of its rows' key sets
// (for the windowed form the causal windows and the block keys after each query).
int tiles_for(const blockattn_params* p, int n) {
    const int c = n - p->block_size;
    const int lo = p->window_left > 0 ? std::max(0, c - p->window_left + 1) : 0;
    return (n + kTileTokens - 1) / kTileTokens - lo / kTileTokens;
}

KernelShape choose_shape(int D, int NB, int R, int waves_override, long total_tiles, bool fp8) {
    // Each wave owns up to two 16-row blocks of the R query rows. With one row-wave
    // (R <= 32), WT token groups of the workgroup stream different tiles, each wave
    // loading its own (stream_kernel). With WR > 1 row-waves the workgroup loads each
    // tile once into an LDS ring that every row-wave reads (shared_kernel). D = 64
    // allows 8 waves per workgroup; D = 128 keeps 4 so a wave may use the whole
    // register file (one wave per SIMD).
    KernelShape s{};
    s.head_dim = D;
    s.nbw = std::min(NB, 2);
    s.row_waves = (NB + s.nbw - 1) / s.nbw;
    s.all_on = NB % s.nbw == 0;
    s.waves_per_simd = D == 64 ? 2 : 1;
    const int max_waves = D == 64 ? kMaxWaves : 4;
    // More than one row-wave: the workgroup shares each tile through LDS, one token stream.
    s.shared = s.row_waves > 1;
    // Token groups: as many as the workgroup allows. At D = 64 eight groups beat four by
    // 0.5-4 % over the unwindowed batches measured (one 8-wave workgroup per CU instead
    // of two of 4 waves) and tie on the wider ones.
    s.token_groups = s.shared ? 1 : std::max(1, max_waves / s.row_waves);
    const bool many_tiles = total_tiles >= 8L * kNumCUs;
    if (s.shared && D == 128 && NB >= 7 && (waves_override > NB || (waves_override == 0 && many_tiles))) {
        // Seven or eight row blocks and at least 8 tiles per CU: two token groups, each
        // of four waves with two row blocks per wave and its own ring (8 waves, two per
        // SIMD within 256 registers each). Two blocks per wave halve the LDS reads per
        // row, and the second group keeps two waves on every SIMD. Measured at seven
        // blocks (windowed, W = 4096, D = 128), per call against seven one-block waves:
        // 64 requests x 4 kv heads of 2K-16K keys 131 against 145 us; one kv head, 64
        // requests of 2K, 8K, 16K keys 35.8 / 50.0 / 48.4 against 39.4 / 53.9 / 52.2 us;
        // 8 requests of 16K keys (about 4 tiles per CU) 27.3 against 24.4 us, so
        // smaller batches keep the one-group shape.
        s.nbw = 2;
        s.row_waves = (NB + 1) / 2;
        s.all_on = NB % 2 == 0;
        s.token_groups = 2;
        s.waves_per_simd = 2;
    } else if (s.shared && D == 128) {
        // One row block per wave, up to 8 waves (two per SIMD, each within 256
        // registers), so two waves per SIMD hide each other's latency. Measured on the
        // windowed mixed batch: at three row blocks, three waves of one block beat two
        // waves of two (121 against 138 us per call); at seven, seven waves beat four
        // (151 against 197 us). waves_override picks the waves per workgroup: rows per
        // wave = ceil(blocks / waves), 1 or 2; above the row blocks (three, or seven or
        // more), two token groups.
        int wv = NB;
        if (waves_override > 0) wv = std::max((NB + 1) / 2, std::min(waves_override, NB));
        s.nbw = (NB + wv - 1) / wv;
        s.row_waves = (NB + s.nbw - 1) / s.nbw;
        s.all_on = NB % s.nbw == 0;
        s.waves_per_simd = s.nbw == 1 ? 2 : 1;
        if (NB == 3 && (waves_override == 0 || waves_override > NB)) {
            // A fourth wave with no rows: each of the four 16-row halves of a K or V tile
            // is then moved by one wave through one buffer resource. Measured against three
            // waves: 7 % less per call at 1 and 8 requests of 16K keys, 0-1 % less at 64
            // requests and on the mixed batch (2 % with fp8 pools).
            s.row_waves = 4;
            s.all_on = false;
            // fp8 pools with at least 64 tiles per CU (or a count above the blocks): two
            // token groups of these four waves. The loading waves also widen the keys and
            // values there, and one wave per SIMD leaves nothing to overlap that with; on
            // the mixed batch at K = 3 this took 72 against 90 us per call. bf16 pools keep
            // one group (85 against 88 us), as do smaller batches (64 requests of 2K keys
            // with fp8 pools: 24.1 against 25.3 us).
            if (waves_override > NB || (waves_override == 0 && fp8 && total_tiles >= 64L * kNumCUs))
                s.token_groups = 2;
        }
    } else if (waves_override > 0 && !s.shared) {
        s.token_groups = std::max(1, std::min(waves_override, max_waves / s.row_waves));
    }
    s.lds_bytes = attention_lds_bytes(s, R);
    while (s.lds_bytes > kLdsPerCU && s.token_groups > 1) {
        --s.token_groups;
        s.lds_bytes = attention_lds_bytes(s, R);
    }
    return s;
}

int build_plan(const blockattn_params* p, const int32_t* lens, blockattn_plan_s* pl) {
    int rc = validate(p, lens);
    if (rc) return rc;
    pl->prm = *p;
    pl->kind = p->window_left == -1 ? 0 : 1;
    pl->g = p->num_q_heads / p->num_kv_heads;
    // More than 128 query rows per kv head: G row groups of equal 16-row blocks, each its
    // own work unit that reads the kv head's keys again.
    pl->R_all = p->block_size * pl->g;
    const int blocks_all = (pl->R_all + 15) / 16;
    pl->G = (blocks_all + kMaxRowBlocks - 1) / kMaxRowBlocks;
    pl->NB = (blocks_all + pl->G - 1) / pl->G;
    pl->R = pl->G == 1 ? pl->R_all : 16 * pl->NB;
    pl->merge_active = pl->kind == 1 && p->block_size > 1 && p->window_right != 0;

    const int B = p->batch, H = p->num_kv_heads * pl->G;  // (kv head, row group) pairs per request
    std::vector<int> nt(B);
    long total = 0;
    for (int b = 0; b < B; ++b) {
        nt[b] = tiles_for(p, lens[b]);
        total += (long)nt[b] * H;
    }
    pl->shape = choose_shape(p->head_dim, pl->NB, pl->R, p->waves_override, total, p->kv_dtype == BLOCKATTN_KV_FP8_E4M3);
    pl->shape.fp8 = p->kv_dtype == BLOCKATTN_KV_FP8_E4M3;
    // Workgroups resident per CU, from the kernel's waves per SIMD and its LDS.
    const int waves = pl->shape.row_waves * pl->shape.token_groups;
    const int waves_per_cu = 4 * pl->shape.waves_per_simd;
    int wg_per_cu = (int)std::max<size_t>(1, kLdsPerCU / std::max<size_t>(pl->shape.lds_bytes, 1));
    wg_per_cu = std::max(1, std::min(wg_per_cu, waves_per_cu / waves));
    const long slots = (long)kNumCUs * wg_per_cu;
    // Tiles per unit (at least two per wave of the streaming kernel at D = 64 and one at
    // D = 128, 16 KiB of bf16 keys and values either way: one D = 128 tile per wave took
    // 5-10 % off the windowed K = 1 batches of 1 and 8 requests, one D = 64 tile per wave
    // added 4-7 % at one 32K request; two for the shared-tile kernel, whose prologue
    // stages two tiles): the value that minimises an
    // estimate of the makespan, in tiles. Workgroups resident on one CU share its
    // throughput, so the tiles cost the largest unit's count once per unit a CU
    // receives (units / CUs, rounded up), whether they run side by side or one after
    // another. The fixed start-up and epilogue cost is paid once per round of `slots`
    // resident workgroups (co-resident units overlap theirs), and splitting any request
    // adds the combine launch.
    constexpr long kUnitCost = 8, kCombineCost = 8;
    const long wt = pl->shape.token_groups;
    long max_nt = 1;
    for (int b = 0; b < B; ++b) max_nt = std::max<long>(max_nt, nt[b]);
    long per_unit = std::max(pl->shape.shared ? 2 : (p->head_dim == 64 ? 2 : 1) * wt, (total + slots - 1) / slots);
    if (p->splits_override <= 0 && per_unit < max_nt) {
        long best = -1, best_cost = 0;
        for (long pu = per_unit;; pu = std::min(max_nt, std::max(pu + 1, pu * 9 / 8))) {
            long units = 0, largest = 0;
            bool split = false;
            for (int b = 0; b < B; ++b) {
                const long S = std::max(1L, std::min<long>((nt[b] + pu - 1) / pu, nt[b]));
                units += S * H;
                largest = std::max(largest, (nt[b] + S - 1) / S);
                split = split || S > 1;
            }
            const long cost = (units + kNumCUs - 1) / kNumCUs * largest + (units + slots - 1) / slots * kUnitCost +
                              (split ? kCombineCost : 0);
            if (best < 0 || cost < best_cost) {
                best = pu;
                best_cost = cost;
            }
            if (pu >= max_nt) break;
        }
        per_unit = best;
    }

    pl->work.clear();
    pl->pair_table.assign((size_t)B * H * 2, 0);
    pl->max_splits = 0;
    for (int b = 0; b < B; ++b) {
        int S = p->splits_override > 0 ? p->splits_override : (int)((nt[b] + per_unit - 1) / per_unit);
        S = std::max(1, std::min(S, nt[b]));
        pl->max_splits = std::max(pl->max_splits, S);
        for (int h = 0; h < H; ++h) {
            const size_t pair = (size_t)b * H + h;
            pl->pair_table[2 * pair] = (int32_t)pl->work.size();
            pl->pair_table[2 * pair + 1] = S;
            for (int s = 0; s < S; ++s) pl->work.push_back(WorkItem{b, h, s, S});
        }
    }
    if (pl->work.size() > 0x7FFFFFFFu / 2)
        return fail(BLOCKATTN_ERR_UNSUPPORTED, "too many work units; lower batch or splits_override");
    pl->units = (int)pl->work.size();
    pl->uniform_splits = pl->max_splits;
    for (size_t pr = 0; pr < (size_t)B * H; ++pr)
        if (pl->pair_table[2 * pr + 1] != pl->max_splits) pl->uniform_splits = 0;

    // Split combine: by the combine kernel, or in the attention kernel by each pair's last unit.
    // The automatic choice is the combine kernel: on MI355X it measured faster at every batch of
    // the Kimi-style rank at 128K (B = 1 ... 16), because the last arriver alone reads all of its
    // pair's partials through device-scope loads while the combine kernel spreads them over
    // many workgroups.
    pl->fused = false;
    // (Its only LDS is one arrival flag, which every kernel shape has: each item folds its
    // splits in registers.)
    if (pl->max_splits > 1 && p->combine_mode == BLOCKATTN_COMBINE_LAST_ARRIVER) pl->fused = true;

    Layout& L = pl->lay;
    L.work = 0;
    L.pairs = align_up(L.work + pl->work.size() * sizeof(WorkItem), 256);
    L.cnt = align_up(L.pairs + pl->pair_table.size() * sizeof(int32_t), 256);
    L.err = align_up(L.cnt + (size_t)B * H * sizeof(uint32_t), 256);
    L.m = align_up(L.err + sizeof(uint32_t), 256);
    L.l = align_up(L.m + (size_t)pl->units * pl->R * sizeof(float), 256);
    L.acc = align_up(L.l + (size_t)pl->units * pl->R * sizeof(float), 256);
    L.total = align_up(L.acc + (size_t)pl->units * pl->R * p->head_dim * sizeof(float), 256);
    return BLOCKATTN_OK;
}

int check_forward(blockattn_plan_t plan, int kind, const void* q, const void* k, const void* v, const int32_t* pt,
                  const int32_t* lens, void* ws, void* out, float* lse) {
    if (!plan) return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "plan is NULL");
    if (plan->kind != kind)
        return fail(BLOCKATTN_ERR_PLAN_MISMATCH,
                    kind == 0 ? "plan is windowed (window_left >= 1); call blockattn_windowed_forward"
                              : "plan is unwindowed (window_left = -1); call blockattn_forward");
    if (!plan->uploaded)
        return fail(BLOCKATTN_ERR_PLAN_MISMATCH, "plan was made without a workspace; plan again with one");
    if (ws != plan->ws)
        return fail(BLOCKATTN_ERR_PLAN_MISMATCH, "workspace differs from the one the plan was uploaded to");
    if (!q || !k || !v || !pt || !lens || !out)
        return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "q, k_cache, v_cache, page_table, seq_lens and out are required");
    if (kind == 1 && !lse)
        return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "the windowed forward returns the merged LSE: lse is required");
    return BLOCKATTN_OK;
}

// A forward on a stream other than the one the plan uploaded its work list on must not
// start before that copy has landed. Outside graph capture it waits on the copy's event
// (on the device, no host wait) until the copy has once been seen complete. A stream
// being captured cannot wait on an event recorded outside the capture; the header makes
// the copy's completion before such a capture the caller's part.
hipError_t order_after_upload(blockattn_plan_t plan, hipStream_t st) {
    if (plan->upload_seen_done || st == plan->upload_stream) return hipSuccess;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(st, &cs);
    if (e != hipSuccess || cs != hipStreamCaptureStatusNone) return e;
    e = hipEventQuery(plan->copy_done);
    if (e == hipSuccess) {
        plan->upload_seen_done = true;
        return hipSuccess;
    }
    if (e != hipErrorNotReady) return e;
    return hipStreamWaitEvent(st, plan->copy_done, 0);
}

// ws: the plan's workspace, or (from_scratch) the library's device scratch array, laid out the same.
int run_forward(blockattn_plan_t plan, const void* q, const void* k, const void* v, const int32_t* pt,
                const int32_t* lens, void* ws, void* out, float* lse, void* stream, const void* k_block = nullptr,
                const void* v_block = nullptr, int append = 0, bool from_scratch = false) {
    const blockattn_params& p = plan->prm;
    char* base = static_cast<char*>(ws);
    hipStream_t st = static_cast<hipStream_t>(stream);

    KernelArgs ka{};
    ka.k_block = static_cast<const uint16_t*>(k_block);
    ka.v_block = static_cast<const uint16_t*>(v_block);
    ka.append = append ? 1 : 0;
    ka.k_scale = p.k_scale;
    ka.q = static_cast<const uint16_t*>(q);
    ka.kc = k;
    ka.vc = v;
    ka.page_table = pt;
    ka.seq_lens = lens;
    ka.work = reinterpret_cast<const WorkItem*>(base + plan->lay.work);
    ka.pair_table = reinterpret_cast<const int32_t*>(base + plan->lay.pairs);
    ka.part_m = reinterpret_cast<float*>(base + plan->lay.m);
    ka.part_l = reinterpret_cast<float*>(base + plan->lay.l);
    ka.part_acc = reinterpret_cast<float*>(base + plan->lay.acc);
    ka.err = reinterpret_cast<uint32_t*>(base + plan->lay.err);
    ka.counters = reinterpret_cast<uint32_t*>(base + plan->lay.cnt);
    ka.fused_combine = plan->fused ? 1 : 0;
    ka.out = static_cast<uint16_t*>(out);
    ka.lse = lse;
    ka.K = p.block_size;
    ka.Hq = p.num_q_heads;
    ka.Hkv = p.num_kv_heads;
    ka.g = plan->g;
    ka.R = plan->R;
    ka.R_all = plan->R_all;
    ka.row_groups = plan->G;
    ka.P = p.page_size;
    ka.p_shift = __builtin_ctz((unsigned)p.page_size);
    ka.stride = p.page_table_stride;
    ka.num_pages = p.num_pages;
    ka.window_left = p.window_left;
    ka.window_right = p.window_right;
    ka.row_waves = plan->shape.row_waves;
    ka.token_groups = plan->shape.token_groups;
    ka.uniform_splits = plan->uniform_splits;
    // A stored key stands for k_scale * k: the logits take k_scale with sm_scale.
    ka.scale_log2 = (float)((double)p.sm_scale * p.k_scale * 1.4426950408889634);
    ka.v_scale = p.v_scale;
    ka.block_scale_log2 = (float)((double)p.sm_scale * 1.4426950408889634);
    ka.block_p_mul = 1.0f / p.v_scale;
    ka.trace = plan->trace;

    hipError_t e = from_scratch ? hipSuccess : order_after_upload(plan, st);
    if (e != hipSuccess) return fail(BLOCKATTN_ERR_HIP, std::string("ordering after the work-list upload: ") + hipGetErrorString(e));
    if (plan->prof_before) e = hipEventRecord(plan->prof_before, st);
    if (e == hipSuccess) e = launch_attention(plan->shape, plan->kind == 1, plan->units, ka, st);
    if (e == hipSuccess && plan->prof_after) e = hipEventRecord(plan->prof_after, st);
    if (e != hipSuccess) return fail(BLOCKATTN_ERR_HIP, std::string("attention kernel launch: ") + hipGetErrorString(e));
    if (plan->max_splits > 1 && !plan->fused) {
        const int rows = p.batch * p.num_kv_heads * plan->R_all;
        e = launch_combine(p.head_dim, rows, plan->max_splits, ka, st);
        if (e != hipSuccess)
            return fail(BLOCKATTN_ERR_HIP, std::string("combine kernel launch: ") + hipGetErrorString(e));
    }
    return BLOCKATTN_OK;
}

}  // namespace

extern "C" {

int blockattn_workspace_size(const blockattn_params* params, const int32_t* seq_lens_host, size_t* bytes) {
    if (!bytes) return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "bytes is NULL");
    blockattn_plan_s tmp;
    int rc = build_plan(params, seq_lens_host, &tmp);
    if (rc) return rc;
    *bytes = tmp.lay.total;
    g_last_error.clear();
    return BLOCKATTN_OK;
}

int blockattn_plan(const blockattn_params* params, const int32_t* seq_lens_host, void* workspace,
                   size_t workspace_bytes, void* stream, blockattn_plan_t* plan) {
    if (!plan) return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "plan is NULL");
    *plan = nullptr;
    blockattn_plan_s* pl = new (std::nothrow) blockattn_plan_s();
    if (!pl) return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "out of host memory");
    int rc = build_plan(params, seq_lens_host, pl);
    if (rc) {
        delete pl;
        return rc;
    }
    if (workspace && workspace_bytes < pl->lay.total) {
        char buf[200];
        snprintf(buf, sizeof buf, "workspace has %zu bytes but this plan needs %zu (blockattn_workspace_size)",
                 workspace_bytes, pl->lay.total);
        delete pl;
        return fail(BLOCKATTN_ERR_WORKSPACE_TOO_SMALL, buf);
    }
    // The head (work list, pair table, zeroed arrival counters and input-error word), staged in pinned host
    // memory: the workspace's upload copies it now, blockattn_forward_scratch at each call. A
    // host-only plan made where no GPU is visible keeps no stage.
    const size_t head = pl->lay.m;
    hipError_t e = hipHostMalloc(&pl->stage, head + kReadback, hipHostMallocDefault);
    if (e != hipSuccess) {
        pl->stage = nullptr;
        if (workspace) {
            delete pl;
            return fail(BLOCKATTN_ERR_HIP, std::string("hipHostMalloc: ") + hipGetErrorString(e));
        }
        (void)hipGetLastError();
    } else {
        std::memset(pl->stage, 0, head);
        std::memcpy(static_cast<char*>(pl->stage) + pl->lay.work, pl->work.data(), pl->work.size() * sizeof(WorkItem));
        std::memcpy(static_cast<char*>(pl->stage) + pl->lay.pairs, pl->pair_table.data(),
                    pl->pair_table.size() * sizeof(int32_t));
        // Set-up for blockattn_forward_scratch: the current device's scratch address, looked
        // up once per device.
        void* scratch = nullptr;
        if (scratch_address(&scratch) != hipSuccess) (void)hipGetLastError();
        if (hipEventCreateWithFlags(&pl->scratch_copy_done, hipEventDisableTiming) != hipSuccess) {
            pl->scratch_copy_done = nullptr;
            (void)hipGetLastError();
        }
    }
    if (workspace) {
        hipStream_t st = static_cast<hipStream_t>(stream);
        e = hipMemcpyAsync(workspace, pl->stage, head, hipMemcpyHostToDevice, st);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&pl->copy_done, hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventRecord(pl->copy_done, st);
        if (e != hipSuccess) {
            blockattn_plan_destroy(pl);
            return fail(BLOCKATTN_ERR_HIP, std::string("work-list upload: ") + hipGetErrorString(e));
        }
        pl->ws = workspace;
        pl->uploaded = true;
        pl->upload_stream = st;
    }
    *plan = pl;
    g_last_error.clear();
    return BLOCKATTN_OK;
}

int blockattn_forward(blockattn_plan_t plan, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* page_table, const int32_t* seq_lens, void* workspace, void* out, float* lse,
                      void* stream) {
    int rc = check_forward(plan, 0, q, k_cache, v_cache, page_table, seq_lens, workspace, out, lse);
    if (rc) return rc;
    return run_forward(plan, q, k_cache, v_cache, page_table, seq_lens, workspace, out, lse, stream);
}

int blockattn_windowed_forward(blockattn_plan_t plan, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* page_table, const int32_t* seq_lens, void* workspace, void* out,
                               float* lse, void* stream) {
    int rc = check_forward(plan, 1, q, k_cache, v_cache, page_table, seq_lens, workspace, out, lse);
    if (rc) return rc;
    return run_forward(plan, q, k_cache, v_cache, page_table, seq_lens, workspace, out, lse, stream);
}

int blockattn_forward_block(blockattn_plan_t plan, const void* q, const void* k_block, const void* v_block,
                            void* k_cache, void* v_cache, const int32_t* page_table, const int32_t* seq_lens,
                            void* workspace, void* out, float* lse, int32_t append, void* stream) {
    if (!plan) return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "plan is NULL");
    if (!k_block || !v_block)
        return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "k_block and v_block (bf16 [B, K, Hkv, D]) are required");
    // The accumulator is kept in stored units (the epilogue multiplies by v_scale), so
    // the block's unscaled values join it divided by v_scale.
    if (!std::isfinite(1.0f / plan->prm.v_scale))
        return fail(BLOCKATTN_ERR_INVALID_ARGUMENT,
                    "dense block values need v_scale != 0 with a finite fp32 reciprocal (they join as v / v_scale)");
    if (!std::isfinite((float)((double)plan->prm.sm_scale * 1.4426950408889634)))
        return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "sm_scale * log2(e) must stay a finite fp32 value");
    int rc = check_forward(plan, plan->kind, q, k_cache, v_cache, page_table, seq_lens, workspace, out, lse);
    if (rc) return rc;
    return run_forward(plan, q, k_cache, v_cache, page_table, seq_lens, workspace, out, lse, stream, k_block, v_block,
                       append);
}

int blockattn_forward_scratch(blockattn_plan_t plan, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* page_table, const int32_t* seq_lens, void* out, float* lse,
                              void* stream) {
    if (!plan) return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "plan is NULL");
    if (plan->lay.total > kScratchBytes) {
        char buf[240];
        snprintf(buf, sizeof buf,
                 "this plan needs %zu bytes of work list and partials, more than the %zu-byte scratch array; "
                 "use blockattn_forward / blockattn_windowed_forward with a workspace, or fewer splits",
                 plan->lay.total, kScratchBytes);
        return fail(BLOCKATTN_ERR_WORKSPACE_TOO_SMALL, buf);
    }
    if (!q || !k_cache || !v_cache || !page_table || !seq_lens || !out)
        return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "q, k_cache, v_cache, page_table, seq_lens and out are required");
    if (plan->kind == 1 && !lse)
        return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "the windowed form returns the merged LSE: lse is required");
    if (!plan->stage)
        return fail(BLOCKATTN_ERR_PLAN_MISMATCH, "plan has no staged work list (it was made with no GPU visible)");
    void* scratch = nullptr;
    hipError_t e = scratch_address(&scratch);
    if (e != hipSuccess) return fail(BLOCKATTN_ERR_HIP, std::string("scratch array address: ") + hipGetErrorString(e));
    if (plan->uniform_splits == 0 || plan->fused) {
        // Requests with different split counts: the kernels read the work list and the pair
        // table; an in-kernel combine: its arrival counters must start at zero, whatever an
        // earlier call left in the array. So this call brings its plan's head (work list, pair
        // table, zeroed counters) into the shared array first. The event lets
        // blockattn_plan_destroy wait until the copy has read the stage.
        if (!plan->scratch_copy_done)
            return fail(BLOCKATTN_ERR_PLAN_MISMATCH, "plan has no event for its work-list copies; plan again");
        hipStream_t st = static_cast<hipStream_t>(stream);
        e = hipMemcpyAsync(scratch, plan->stage, plan->lay.m, hipMemcpyHostToDevice, st);
        if (e == hipSuccess) e = hipEventRecord(plan->scratch_copy_done, st);
        if (e != hipSuccess) return fail(BLOCKATTN_ERR_HIP, std::string("work-list copy: ") + hipGetErrorString(e));
    }
    return run_forward(plan, q, k_cache, v_cache, page_table, seq_lens, scratch, out, lse, stream, nullptr, nullptr, 0,
                       true);
}

int blockattn_merge(int32_t parts, int64_t rows, int32_t head_dim, const void* part_out, const float* part_lse,
                    void* out, float* lse, void* stream) {
    if (parts < 1 || parts > 4096) return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "parts must be in [1, 4096]");
    if (rows < 0) return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "rows must be >= 0");
    if (head_dim != 64 && head_dim != 128)
        return fail(BLOCKATTN_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (the gfx950 kernels are built for those)");
    if (rows > (int64_t)0x7FFFFFFF * (256 / (head_dim / 8)))
        return fail(BLOCKATTN_ERR_UNSUPPORTED, "rows exceed one launch; merge in pieces");
    if (rows == 0) return BLOCKATTN_OK;
    if (!part_out || !part_lse || !out)
        return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "part_out, part_lse and out are required");
    const char* po = static_cast<const char*>(part_out);
    const char* oo = static_cast<const char*>(out);
    const size_t part_bytes = (size_t)parts * rows * head_dim * 2, out_bytes = (size_t)rows * head_dim * 2;
    if (oo < po + part_bytes && po < oo + out_bytes)
        return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "out must not overlap part_out");
    hipError_t e = launch_merge(head_dim, parts, rows, static_cast<const uint16_t*>(part_out), part_lse,
                                static_cast<uint16_t*>(out), lse, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(BLOCKATTN_ERR_HIP, std::string("merge kernel launch: ") + hipGetErrorString(e));
    return BLOCKATTN_OK;
}

int blockattn_plan_info(blockattn_plan_t plan, blockattn_plan_info_t* info) {
    if (!plan || !info) return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "plan and info are required");
    info->kind = plan->kind;
    info->units = plan->units;
    info->max_splits = plan->max_splits;
    info->merge_active = plan->merge_active ? 1 : 0;
    info->waves_per_unit = plan->shape.row_waves * plan->shape.token_groups;
    info->token_groups = plan->shape.token_groups;
    info->row_waves = plan->shape.row_waves;
    info->uploaded = plan->uploaded ? 1 : 0;
    info->combine_launch = plan->max_splits > 1 && !plan->fused ? 1 : 0;
    info->fused_combine = plan->fused ? 1 : 0;
    info->shared_tiles = plan->shape.shared ? 1 : 0;
    info->row_groups = plan->G;
    info->workspace_bytes = plan->lay.total;
    return BLOCKATTN_OK;
}

int blockattn_plan_set_profile_events(blockattn_plan_t plan, void* before, void* after) {
    if (!plan) return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "plan is NULL");
    if ((before == nullptr) != (after == nullptr))
        return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "pass both profiling events or neither");
    plan->prof_before = static_cast<hipEvent_t>(before);
    plan->prof_after = static_cast<hipEvent_t>(after);
    return BLOCKATTN_OK;
}

int blockattn_plan_set_phase_trace(blockattn_plan_t plan, void* trace, size_t bytes) {
    if (!plan) return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "plan is NULL");
    if (trace && bytes < (size_t)plan->units * kTracePoints * sizeof(uint64_t)) {
        char buf[160];
        snprintf(buf, sizeof buf, "trace buffer has %zu bytes; this plan's %d units need %zu", bytes, plan->units,
                 (size_t)plan->units * kTracePoints * sizeof(uint64_t));
        return fail(BLOCKATTN_ERR_WORKSPACE_TOO_SMALL, buf);
    }
    if (trace && (reinterpret_cast<uintptr_t>(trace) & 7u) != 0)
        return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "trace buffer must be 8-byte aligned");
    plan->trace = static_cast<uint64_t*>(trace);
    return BLOCKATTN_OK;
}

int blockattn_input_errors(blockattn_plan_t plan, void* workspace, void* stream, int32_t* flags) {
    if (!plan || !flags) return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "plan and flags are required");
    *flags = 0;
    if (!plan->uploaded || workspace != plan->ws)
        return fail(BLOCKATTN_ERR_PLAN_MISMATCH, "workspace is not the one this plan was uploaded to");
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(st, &cs);
    if (e == hipSuccess && cs != hipStreamCaptureStatusNone)
        return fail(BLOCKATTN_ERR_INVALID_ARGUMENT, "blockattn_input_errors waits on the host: call it outside graph capture");
    uint32_t* host = reinterpret_cast<uint32_t*>(static_cast<char*>(plan->stage) + plan->lay.m);
    char* word = static_cast<char*>(workspace) + plan->lay.err;
    if (e == hipSuccess) e = order_after_upload(plan, st);
    if (e == hipSuccess) e = hipMemcpyAsync(host, word, sizeof(uint32_t), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipMemsetAsync(word, 0, sizeof(uint32_t), st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(BLOCKATTN_ERR_HIP, std::string("reading the input-error word: ") + hipGetErrorString(e));
    *flags = (int32_t)*host;
    return BLOCKATTN_OK;
}

void blockattn_plan_destroy(blockattn_plan_t plan) {
    if (!plan) return;
    if (plan->copy_done) {
        (void)hipEventSynchronize(plan->copy_done);
        (void)hipEventDestroy(plan->copy_done);
    }
    if (plan->scratch_copy_done) {
        (void)hipEventSynchronize(plan->scratch_copy_done);
        (void)hipEventDestroy(plan->scratch_copy_done);
    }
    if (plan->stage) (void)hipHostFree(plan->stage);
    delete plan;
}

const char* blockattn_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

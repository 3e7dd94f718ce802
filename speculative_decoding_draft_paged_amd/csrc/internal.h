// Internal interface between the host plan/C ABI (api.cpp) and the gfx950 kernels (kernels_*.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace blockattn {

constexpr int kTileTokens = 32;   // keys per tile: one MFMA K-step of PV, two 16-token M blocks of QK^T
constexpr int kMaxRowBlocks = 8;  // a work unit holds at most 128 query rows; more rows per kv head are
                                   // split into row groups of at most 128, each its own unit
constexpr int kMaxWaves = 8;      // wavefronts per workgroup of the attention kernels
constexpr int kPidWindow = 2048;     // tiles whose page ids the streaming kernel stages in LDS at a time

// Bits of the input-error word (the values of BLOCKATTN_INPUT_BAD_LENGTH / _BAD_PAGE).
constexpr uint32_t kErrLength = 1u;  // a device length outside [K, stride * P]: clamped into it
constexpr uint32_t kErrPage = 2u;    // a page id read outside [0, num_pages): clamped into it

// One unit of split-KV work. Tiles [lo, hi) of the key range of (b, h_kv) are derived on
// the device from the live sequence length: unit s of S covers tiles tb + s*nt/S ..
// tb + (s+1)*nt/S.
struct WorkItem {
    int32_t b, hk, s, S;  // hk: kv head * row_groups + row group
};

struct KernelArgs {
    const uint16_t* q;
    const void* kc;        // K pool: bf16 or fp8 E4M3 elements
    const void* vc;        // V pool
    const int32_t* page_table;
    const int32_t* seq_lens;
    const WorkItem* work;
    const int32_t* pair_table;  // per (b, h_kv): first unit, split count
    float* part_m;
    float* part_l;
    float* part_acc;
    uint32_t* err;         // input-error word: bits kErrLength / kErrPage are set when a clamp was needed
    uint32_t* counters;    // per (request, kv head, row group): arrivals of its units; zero between calls
    int32_t fused_combine; // split pairs are combined in the attention kernel by their last unit
    uint16_t* out;
    float* lse;
    int32_t K, Hq, Hkv, g, R, P, stride, num_pages;  // R: query rows per work unit (<= 128)
    int32_t R_all;         // query rows per kv head, K * g
    int32_t row_groups;    // units of R rows that cover them: ceil(R_all / R)
    int32_t p_shift;       // log2 P
    int32_t window_left;   // -1: none
    int32_t window_right;  // -1: every later block key
    int32_t row_waves;     // WR: waves streaming the same tiles, each owning NBW row blocks
    int32_t token_groups;  // WT: tile streams per workgroup
    int32_t uniform_splits;  // > 0: every (b, h_kv) has this many splits, unit = pair * S + s (no work list read)
    float scale_log2;      // sm_scale * k_scale * log2(e)
    float v_scale;         // applied to the outputs (a stored value stands for v_scale * v)
    float k_scale;         // pool scales again, for encoding appended block keys and values
    const uint16_t* k_block;  // NULL: the block keys are in the cache; else bf16 [B, K, Hkv, D] read instead
    const uint16_t* v_block;
    int32_t append;        // with k_block: the last split of each (b, h_kv) also stores the block into the cache
    float block_scale_log2;  // sm_scale * log2(e): logit scale of the dense block keys (they are unscaled)
    float block_p_mul;       // 1 / v_scale: the dense block values join the accumulator, which is kept in
                             // stored units, through probabilities multiplied by this
    uint64_t* trace;         // NULL, or kTracePoints timestamps per work unit (profiling aid)
};

// Phase timestamps a traced attention kernel records per work unit (workgroup), in the
// 100 MHz constant clock: kernel entry, length known, page ids staged, this unit's loop done
// (token group 0), all token groups done (epilogue start), stores complete.
constexpr int kTracePoints = 8;
enum TracePoint { kTrEntry = 0, kTrLength = 1, kTrPages = 2, kTrLoop = 3, kTrEpilogue = 4, kTrStored = 5 };

// Chosen kernel shape for a plan.
struct KernelShape {
    int head_dim;      // 64 or 128
    int nbw;           // 16-row blocks per wave (1 or 2)
    bool all_on;       // every wave's row blocks hold live rows (R is a multiple of 16 * nbw)
    int row_waves;     // WR: waves streaming the same tiles, each owning nbw row blocks
    int token_groups;  // WT
    bool shared;       // row_waves > 1: the workgroup loads each tile once into an LDS ring (shared_kernel)
    bool fp8;          // K and V pools hold fp8 E4M3 bytes
    int waves_per_simd;  // occupancy the kernel's register use allows (1 or 2)
    size_t lds_bytes;  // dynamic LDS per workgroup
};

size_t attention_lds_bytes(const KernelShape& s, int R);

hipError_t launch_attention(const KernelShape& shape, bool windowed, int units, const KernelArgs& args,
                            hipStream_t stream);
// fp8 E4M3 KV instantiations (kernels_fp8.hip); launch_attention routes to it when shape.fp8.
hipError_t launch_attention_fp8(const KernelShape& shape, bool windowed, int units, const KernelArgs& args,
                                hipStream_t stream);
// LSE combine of the splits of `rows` output rows; max_splits: the largest split count of any row.
hipError_t launch_combine(int head_dim, int rows, int max_splits, const KernelArgs& args, hipStream_t stream);
// Set the calling thread's last-error text (blockattn_last_error) and return code.
int record_error(int code, const char* msg);

// Bytes of the library's device scratch array (one per GPU, held until the process ends), where
// blockattn_forward_scratch keeps the work list and partial softmax states of callers that cannot
// allocate. Equal to BLOCKATTN_SCRATCH_BYTES.
constexpr size_t kScratchBytes = (size_t)32 << 20;
// Device address of the scratch array on the current device (looked up once per device).
hipError_t scratch_address(void** ptr);

// G-way LSE merge of bf16 partial results [parts, rows, head_dim] with base-2 LSEs [parts, rows].
hipError_t launch_merge(int head_dim, int parts, int64_t rows, const uint16_t* part_out, const float* part_lse,
                        uint16_t* out, float* lse, hipStream_t stream);

}  // namespace blockattn

// Internal interface between the host plan/C ABI (api.cpp) and the gfx950 kernels (kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace blockattn {

constexpr int kTileTokens = 32;  // keys per tile: one MFMA K-step of PV, two 16-token M blocks of QK^T
constexpr int kMaxRowBlocks = 8; // R = K * group <= 128 query rows per kv head
constexpr int kMaxWaves = 8;     // wavefronts per workgroup of the partial kernel

// One unit of split-KV work: tiles [lo, hi) of the key range of (b, h_kv) are
// derived on the device from the live sequence length: unit s of S covers
// tiles tb + s*nt/S .. tb + (s+1)*nt/S.
struct WorkItem {
    int32_t b, hk, s, S;
};

struct PartialArgs {
    const uint16_t* q;
    const uint16_t* kc;
    const uint16_t* vc;
    const int32_t* page_table;
    const int32_t* seq_lens;
    const WorkItem* work;
    float* part_m;
    float* part_l;
    float* part_acc;
    int32_t K, Hq, Hkv, g, R, P, stride, num_pages;
    int32_t window_left;  // -1 none
    int32_t row_waves;    // WR: waves sharing a tile, each owning NBW row blocks
    int32_t token_groups; // WT: tile streams per workgroup
    float scale_log2;     // sm_scale * log2(e)
};

struct CombineArgs {
    const uint16_t* q;
    const uint16_t* kc;
    const uint16_t* vc;
    const int32_t* page_table;
    const int32_t* seq_lens;
    const int32_t* pair_table;  // per (b, h_kv): first unit, split count
    const float* part_m;
    const float* part_l;
    const float* part_acc;
    uint16_t* out;
    float* lse;
    int32_t K, Hq, Hkv, g, R, P, stride, num_pages;
    int32_t window_right;
    float scale_log2;
};

// Chosen kernel shape for a plan.
struct KernelShape {
    int head_dim;     // 64 or 128
    int nbw;          // row blocks per wave (1 or 2)
    int cpw;          // 1-KiB load chunks per wave per tile (4, 8 or 16)
    int row_waves;    // WR
    int token_groups; // WT
    size_t lds_bytes; // dynamic LDS per workgroup
};

size_t partial_lds_bytes(int head_dim, int nbw, int row_waves, int token_groups);

hipError_t launch_partial(const KernelShape& shape, bool windowed, int units, const PartialArgs& args,
                          hipStream_t stream);
hipError_t launch_combine(int head_dim, bool merge, int rows, const CombineArgs& args, hipStream_t stream);

}  // namespace blockattn

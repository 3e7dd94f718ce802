// bf16 KV instantiations of the attention kernels, the split combine and the LDS sizing.
#include "attention_kernels.h"

namespace blockattn {

// Scratch for blockattn_forward_scratch (callers that cannot allocate): work list, pair table,
// input-error word and partial softmax states, laid out as a workspace. Each GPU holds its own
// copy at its own address; host code never passes the array's name to a kernel (on the host it
// is only a stand-in), only the device address scratch_address looked up with that device current.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kScratchDevices];  // static storage: starts at nullptr
}  // namespace

hipError_t scratch_address(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool tracked = dev >= 0 && dev < kScratchDevices;
    if (tracked) {
        void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
        if (p) {
            *ptr = p;
            return hipSuccess;
        }
    }
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    if (tracked) g_scratch_ptr[dev].store(p, std::memory_order_release);
    *ptr = p;
    return hipSuccess;
}

size_t attention_lds_bytes(const KernelShape& s, int R) {
    (void)R;
    const int D = s.head_dim;
    if (s.shared) {
        const size_t pitches = D == 64 ? kKPitch<64> + kVPitch<64> : kKPitch<128> + kVPitch<128>;
        const size_t ring = (size_t)s.token_groups * 3 * kTileTokens * pitches * sizeof(uint16_t) +
                            2 * kPidWindow * sizeof(int);
        const size_t epi = epilogue_floats(D, s.row_waves * s.nbw, s.token_groups) * sizeof(float);
        return ring > epi ? ring : epi;
    }
    const size_t vpitch = D == 64 ? kVPitch<64> : kVPitch<128>;
    const size_t loop = ((size_t)s.token_groups * s.row_waves * kTileTokens) * vpitch * sizeof(uint16_t) +
                        2 * kPidWindow * sizeof(int);
    const size_t epi = epilogue_floats(D, s.row_waves * s.nbw, s.token_groups) * sizeof(float);
    return loop > epi ? loop : epi;
}

hipError_t launch_attention(const KernelShape& shape, bool windowed, int units, const KernelArgs& args,
                            hipStream_t stream) {
    if (shape.fp8) return launch_attention_fp8(shape, windowed, units, args, stream);
    return windowed ? dispatch<true, false>(shape, units, args, stream) : dispatch<false, false>(shape, units, args, stream);
}

hipError_t launch_merge(int head_dim, int parts, int64_t rows, const uint16_t* part_out, const float* part_lse,
                        uint16_t* out, float* lse, hipStream_t stream) {
    const int rpb = 256 / (head_dim / 8);
    const int64_t blocks = (rows + rpb - 1) / rpb;
    if (head_dim == 64)
        hipLaunchKernelGGL(merge_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, stream, parts, rows, part_out,
                           part_lse, out, lse);
    else if (head_dim == 128)
        hipLaunchKernelGGL(merge_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, stream, parts, rows, part_out,
                           part_lse, out, lse);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_combine(int head_dim, int rows, int max_splits, const KernelArgs& args, hipStream_t stream) {
    if (head_dim != 64 && head_dim != 128) return hipErrorInvalidValue;
    const int streams = 256 / (head_dim / 4);  // split streams per 256-thread workgroup
    int sl = 1;                                 // streams per row: each folds at most about 4 splits
    while (sl < streams && sl * 4 < max_splits) sl *= 2;
    const int per_wg = streams / sl;
    const unsigned blocks = (unsigned)((rows + per_wg - 1) / per_wg);
    if (head_dim == 64)
        hipLaunchKernelGGL(combine_kernel<64>, dim3(blocks), dim3(256), 0, stream, args, sl, rows);
    else
        hipLaunchKernelGGL(combine_kernel<128>, dim3(blocks), dim3(256), 0, stream, args, sl, rows);
    return hipGetLastError();
}

}  // namespace blockattn

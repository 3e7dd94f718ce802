// fp8 E4M3 KV instantiations of the attention kernels (compiled on their own to keep builds parallel).
#include "attention_kernels.h"

namespace blockattn {

hipError_t launch_attention_fp8(const KernelShape& shape, bool windowed, int units, const KernelArgs& args,
                                hipStream_t stream) {
    return windowed ? dispatch<true, true>(shape, units, args, stream) : dispatch<false, true>(shape, units, args, stream);
}

}  // namespace blockattn

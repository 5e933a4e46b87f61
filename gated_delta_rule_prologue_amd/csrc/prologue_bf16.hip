// prologue_bf16.hip -- prologue kernels for bf16 inputs: the closed-form kernels without history (every L, channel group width and strip length)
// (kernel template in prologue_kernel.h).
#include "prologue_kernel.h"

namespace prism {

hipError_t launch_prologue_bf16(const PrologueArgs& p, hipStream_t stream)
{
    return launch_T<uint16_t, false>(p, stream);
}

}  // namespace prism

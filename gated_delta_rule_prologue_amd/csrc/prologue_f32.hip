// prologue_f32.hip -- prologue kernels for fp32 inputs: the closed-form kernels without history (every L, channel group width and strip length)
// (kernel template in prologue_kernel.h).
#include "prologue_kernel.h"

namespace prism {

hipError_t launch_prologue_f32(const PrologueArgs& p, hipStream_t stream)
{
    return launch_T<float, false>(p, stream);
}

}  // namespace prism

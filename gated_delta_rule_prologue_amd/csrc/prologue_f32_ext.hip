// prologue_f32_ext.hip -- prologue kernels for fp32 inputs: the kernels with a carried history or the GELU residual chain
// (kernel template in prologue_kernel.h).
#include "prologue_kernel.h"

namespace prism {

hipError_t launch_prologue_f32_ext(const PrologueArgs& p, hipStream_t stream)
{
    return launch_T<float, true>(p, stream);
}

}  // namespace prism

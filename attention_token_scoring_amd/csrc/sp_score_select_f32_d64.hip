// Instantiations of the fused scoring-and-selection kernel for fp32 operands, head dimension 64.
#include "sp_score_kernel.h"

namespace sp {

const void* score_select_kernel_f32_d64(int rows, int G, int tpw, bool dma) {
    return pick_kernel_for<64, false, kLaunchFused>(rows, G, tpw, dma);
}

}  // namespace sp

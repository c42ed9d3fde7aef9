// Instantiations of the scoring kernel for fp32 operands, head dimension 128.
#include "sp_score_kernel.h"

namespace sp {

const void* score_kernel_f32_d128(int rows, int G, int tpw, bool dma) {
    return pick_kernel_for<128, false, kLaunchPlain>(rows, G, tpw, dma);
}

}  // namespace sp

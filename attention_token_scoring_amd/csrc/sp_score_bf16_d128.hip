// Instantiations of the scoring kernel for bf16 operands, head dimension 128.
#include "sp_score_kernel.h"

namespace sp {

const void* score_kernel_bf16_d128(int rows, int G, int tpw, bool dma) {
    return pick_kernel_for<128, true, kLaunchPlain>(rows, G, tpw, dma);
}

}  // namespace sp

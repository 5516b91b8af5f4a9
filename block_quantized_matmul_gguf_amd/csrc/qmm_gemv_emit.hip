// qmm_gemv_emit.hip -- the mode (b) instances of the decode kernel that also write their integer block sums and quantized activations (the traced run).
#include "qmm_gemv_kernel.h"

namespace qmm {

GvKernel gv_kernel_emit(int fmt, int P, int R, int D)
{
    return fmt == FMT_Q8_0 ? gv_pick<FMT_Q8_0, MODE_B, true>(P, R, D) : gv_pick<FMT_Q4_K, MODE_B, true>(P, R, D);
}

}  // namespace qmm

// qmm_gemv_b.hip -- the mode (b) instances of the decode kernel.
#include "qmm_gemv_kernel.h"

namespace qmm {

GvKernel gv_kernel_b(int fmt, int P, int R, int D)
{
    return fmt == FMT_Q8_0 ? gv_pick<FMT_Q8_0, MODE_B, false>(P, R, D) : gv_pick<FMT_Q4_K, MODE_B, false>(P, R, D);
}

}  // namespace qmm

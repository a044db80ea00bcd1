// Mat-vec and dequant kernels for one weight type (instantiations only; the
// device code is in re_kernels.h).
#include "re_kernels.h"

namespace rex {

hipError_t launch_mv_q5_0(const MvArgs &a, uint32_t m, uint32_t nr, dim3 grid, dim3 block, size_t lds,
                         size_t lds_max, hipStream_t s) {
    return launch_mv<kQ5_0>(a, m, nr, grid, block, lds, lds_max, s);
}

hipError_t attributes_mv_q5_0(uint32_t m, uint32_t nr, hipFuncAttributes *attr) {
    return attributes_mv<kQ5_0>(m, nr, attr);
}

hipError_t launch_dq_q5_0(const DqArgs &a, hipStream_t s) { return launch_dq<kQ5_0>(a, s); }

}  // namespace rex

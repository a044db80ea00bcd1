// Mat-vec and dequant kernels for one weight type (instantiations only; the
// device code is in re_kernels.h).
#include "re_kernels.h"

namespace rex {

hipError_t launch_mv_f16(const MvArgs &a, uint32_t m, uint32_t nr, dim3 grid, dim3 block, size_t lds,
                         size_t lds_max, hipStream_t s) {
    return launch_mv<kF16>(a, m, nr, grid, block, lds, lds_max, s);
}

hipError_t attributes_mv_f16(uint32_t m, uint32_t nr, hipFuncAttributes *attr) {
    return attributes_mv<kF16>(m, nr, attr);
}

hipError_t launch_dq_f16(const DqArgs &a, hipStream_t s) { return launch_dq<kF16>(a, s); }

}  // namespace rex

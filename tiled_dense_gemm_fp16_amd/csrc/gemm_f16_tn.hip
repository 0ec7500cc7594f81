// gemm_f16_tn.hip -- kernel configurations of A^T . B (A stored K x M, B stored K x N).
#include "gemm_f16_tile.h"

namespace gemm_f16_impl {

hipError_t launch_tn(int config, const KernelArgs &a, int va, int vb, int64_t grid, hipStream_t s)
{
    return launch_transposed<false, false>(config, a, va, vb, grid, s);
}

} // namespace gemm_f16_impl

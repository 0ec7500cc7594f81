// gemm_f16_tt.hip -- kernel configurations of A^T . B^T (A stored K x M, B stored N x K).
#include "gemm_f16_tile.h"

namespace gemm_f16_impl {

hipError_t launch_tt(int config, const KernelArgs &a, int va, int vb, int64_t grid, hipStream_t s)
{
    return launch_transposed<false, true>(config, a, va, vb, grid, s);
}

} // namespace gemm_f16_impl

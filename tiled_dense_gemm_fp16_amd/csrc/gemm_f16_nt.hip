// gemm_f16_nt.hip -- kernel configurations of A . B^T (A stored M x K, B stored N x K): the pages' transpose_B product.
#include "gemm_f16_tile.h"

namespace gemm_f16_impl {

hipError_t launch_nt(int config, const KernelArgs &a, int va, int vb, int64_t grid, hipStream_t s)
{
    return launch_transposed<true, true>(config, a, va, vb, grid, s);
}

} // namespace gemm_f16_impl

// gemm_f16_nn.hip -- kernel configurations of A . B (A stored M x K, B
// stored K x N), the layout of the pages' tile GEMM.
#include "gemm_f16_tile.h"

namespace gemm_f16_impl {

hipError_t launch_nn(int config, const KernelArgs &a, int va, int vb, int64_t grid, hipStream_t s)
{
    constexpr bool AR = true, BR = false;
    switch (config) {
    case 0: return launch_one<256, 128, 64, 2, 2, 3, true, 8, 8, AR, BR, 1, false, true>(a, grid, s);
    case 1: return launch_one<256, 128, 64, 2, 2, 3, true, 8, 8, AR, BR, 4>(a, grid, s);
    case 2: return launch_one<128, 128, 64, 2, 2, 3, true, 8, 8, AR, BR, 4>(a, grid, s);
    case 3: return launch_staged<128, 128, 32, 2, 2, 2, AR, BR>(a, va, vb, grid, s);
    case 4: return launch_staged<64, 64, 64, 2, 2, 2, AR, BR>(a, va, vb, grid, s);
    case 5: return launch_one<256, 256, 64, 2, 4, 2, true, 8, 8, AR, BR, 2>(a, grid, s);
    case 6: return launch_one<256, 128, 64, 2, 2, 3, true, 2, 2, AR, BR, 1, false, true>(a, grid, s);
    case 7: return launch_one<128, 64, 64, 2, 2, 4, true, 2, 2, AR, BR, 1>(a, grid, s);
    case 8: return launch_one<256, 256, 64, 2, 2, 2, true, 8, 8, AR, BR, GEMM_F16_M16_SPREAD, false, true>(a, grid, s);
    case 9: return launch_one<256, 256, 64, 2, 2, 2, true, 2, 2, AR, BR, GEMM_F16_M16_SPREAD, false, true>(a, grid, s);
    case 10: return launch_one<256, 256, 32, 2, 2, 4, true, 8, 8, AR, BR, 1, false, true>(a, grid, s);
    case 11: return launch_persistent<8, AR, BR>(a, grid, s);
    case 12: return launch_one<64, 64, 64, 2, 2, 4, true, 8, 8, AR, BR, 1>(a, grid, s);
    case 13: return launch_one<128, 128, 64, 2, 2, 4, true, 8, 8, AR, BR, 1, false, true>(a, grid, s);
    case 14: return launch_one<128, 64, 64, 2, 2, 4, true, 8, 8, AR, BR, 1>(a, grid, s);
    case 15: return launch_one<128, 128, 64, 2, 2, 4, true, 2, 2, AR, BR, 1, false, true>(a, grid, s);
    case 16: return launch_one<64, 64, 64, 2, 2, 4, true, 2, 2, AR, BR, 1>(a, grid, s);
    case 17: return launch_staged<128, 128, 64, 2, 2, 2, AR, BR>(a, va, vb, grid, s);
    default: return hipErrorInvalidValue;
    }
}

} // namespace gemm_f16_impl

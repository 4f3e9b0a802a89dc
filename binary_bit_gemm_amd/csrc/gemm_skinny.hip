// Skinny-M path.
#include "lowbit_internal.h"

namespace lowbit {

bool use_skinny(int64_t M, int64_t N, int64_t K) { (void)M; (void)N; (void)K; return false; }

hipError_t launch_gemm_skinny(const GemmProblem& p, int g, int bits, hipStream_t stream) {
    return launch_gemm_tiled(p, g, bits, TILE_64x256, stream);
}

}  // namespace lowbit

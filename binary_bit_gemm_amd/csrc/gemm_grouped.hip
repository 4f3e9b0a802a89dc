// Grouped launch of several independent problems of one (g, bits) class.
#include "lowbit_internal.h"

namespace lowbit {

hipError_t launch_gemm_grouped(const GemmProblem* probs, int count, int g, int bits, hipStream_t stream) {
    for (int i = 0; i < count; ++i) {
        const GemmProblem& p = probs[i];
        hipError_t e = use_skinny(p.M, p.N, p.K, g, bits) ? launch_gemm_skinny(p, g, bits, stream)
                                                 : launch_gemm_tiled(p, g, bits, pick_tile_variant(p.M, p.N, p.K), stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace lowbit

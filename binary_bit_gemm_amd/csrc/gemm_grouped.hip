// Grouped launch of several independent problems of one (g, bits) class: the problems the
// skinny kernel takes go into one launch of it, the rest into one launch of a tile kernel
// (tile chosen for the group as a whole), kMaxGroup problems per launch.  Every output
// element is computed exactly as a single call would compute it.
#include <cstdlib>
#include <cstring>

#include "lowbit_internal.h"

namespace lowbit {
namespace {

// LOWBIT_VARIANT names a tile for A/B runs and tests; -1 when unset or not a tile.
int forced_tile() {
    const char* v = std::getenv("LOWBIT_VARIANT");
    if (v == nullptr) return -1;
    if (std::strcmp(v, "tile256") == 0) return TILE_256x128;
    if (std::strcmp(v, "tile256w") == 0) return TILE_256x256;
    if (std::strcmp(v, "tile128") == 0) return TILE_128x256;
    if (std::strcmp(v, "tile64") == 0) return TILE_64x256;
    if (std::strcmp(v, "tile288") == 0) return TILE_288x192;
    return -1;
}

}  // namespace

hipError_t launch_gemm_grouped(const GemmProblem* probs, int count, int g, int bits, hipStream_t stream) {
    const int forced = forced_tile();
    GemmProblem skinny[kMaxGroup], tiled[kMaxGroup];
    for (int base = 0; base < count; base += kMaxGroup) {
        const int n = count - base < kMaxGroup ? count - base : kMaxGroup;
        int ns = 0, nt = 0;
        for (int i = 0; i < n; ++i) {
            const GemmProblem& p = probs[base + i];
            if (forced < 0 && use_skinny(p.M, p.N, p.K, g, bits)) {
                skinny[ns++] = p;
            } else {
                tiled[nt++] = p;
            }
        }
        if (ns > 0) {
            const hipError_t e = launch_gemm_skinny_group(skinny, ns, g, bits, stream);
            if (e != hipSuccess) return e;
        }
        if (nt > 0) {
            const int variant = forced >= 0 ? forced : pick_tile_variant(tiled, nt, g, bits);
            const hipError_t e = launch_gemm_tiled_group(tiled, nt, g, bits, variant, stream);
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace lowbit

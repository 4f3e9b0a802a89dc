// Grouped launch of several independent problems of one (g, bits) class, kMaxGroup problems
// per launch:
//   * skinny ternary problems the resident kernel covers go into one resident launch per
//     distinct K (split along K through the caller's workspace when the plan asks for it and
//     the workspace is large enough, whole otherwise);
//   * the other skinny problems into one launch of the skinny kernel;
//   * the rest into one launch of a tile kernel (tile chosen for the group as a whole).
// A problem's result does not depend on the other problems of its launch, except that the
// resident kernel's K split is planned for the launch as a whole (so its bits can differ from
// a single call's in the last place; every launch is deterministic).
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
    if (std::strcmp(v, "tile96") == 0) return TILE_96x192;
    if (std::strcmp(v, "tile96k2") == 0) return TILE_96x192K2;
    if (std::strcmp(v, "tile256n") == 0) return TILE_256x192;
    if (std::strcmp(v, "tile64k2") == 0) return TILE_64x128K2;
    if (std::strcmp(v, "tile256sk") == 0) return TILE_256x256SK;
    return -1;
}

// 1: LOWBIT_VARIANT=skinny (no resident launches), 2: LOWBIT_VARIANT=resident (resident
// wherever it applies), 0: the planner decides.
int forced_skinny_kind() {
    const char* v = std::getenv("LOWBIT_VARIANT");
    if (v == nullptr) return 0;
    if (std::strcmp(v, "skinny") == 0) return 1;
    if (std::strcmp(v, "resident") == 0) return 2;
    return 0;
}

// The resident launch (if any) for problems `same` (one K): its plan, or len 0.
ResidentPlan resident_choice(const GemmProblem* same, int n, int g, int kind, void* workspace, size_t ws_bytes) {
    const auto use = [&](const ResidentPlan& pl, bool ws) {
        return pl.len > 0 && (kind == 2 || resident_preferred(same, n, g, ws));
    };
    if (workspace != nullptr) {
        const ResidentPlan pl = plan_resident(same, n, g, true);
        if (use(pl, true) && resident_workspace_bytes(pl) <= ws_bytes) return pl;
    }
    const ResidentPlan pl = plan_resident(same, n, g, false);
    return use(pl, false) ? pl : ResidentPlan{};
}

// Calls f(problems, n, plan) for each same-K subset of `skinny` that goes to the resident
// kernel, and moves the others to the front of `skinny`; returns how many remain.
template <class F>
int take_resident(GemmProblem* skinny, int ns, int g, int bits, int kind, void* workspace, size_t ws_bytes, F&& f) {
    GemmProblem rest[kMaxGroup], same[kMaxGroup];
    bool done[kMaxGroup] = {};
    int nr = 0;
    for (int i = 0; i < ns; ++i) {
        if (done[i]) continue;
        if (kind == 1 || !resident_supported(skinny[i].M, skinny[i].N, skinny[i].K, g, bits)) {
            rest[nr++] = skinny[i];
            continue;
        }
        int nk = 0;
        for (int j = i; j < ns; ++j)
            if (!done[j] && skinny[j].K == skinny[i].K &&
                resident_supported(skinny[j].M, skinny[j].N, skinny[j].K, g, bits)) {
                same[nk++] = skinny[j];
                done[j] = true;
            }
        const ResidentPlan pl = resident_choice(same, nk, g, kind, workspace, ws_bytes);
        if (pl.len > 0) {
            const hipError_t e = f(same, nk, pl);
            if (e != hipSuccess) return -1;
        } else {
            for (int j = 0; j < nk; ++j) rest[nr++] = same[j];
        }
    }
    for (int i = 0; i < nr; ++i) skinny[i] = rest[i];
    return nr;
}

}  // namespace

hipError_t launch_gemm_grouped(const GemmProblem* probs, int count, int g, int bits, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
    const int forced = forced_tile();
    const int kind = forced_skinny_kind();
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
        hipError_t err = hipSuccess;
        ns = take_resident(skinny, ns, g, bits, kind, workspace, workspace_bytes,
                           [&](const GemmProblem* same, int nk, const ResidentPlan& pl) {
                               err = launch_gemm_resident_group(same, nk, g, pl, workspace, stream);
                               return err;
                           });
        if (ns < 0) return err;
        if (ns > 0) {
            const hipError_t e = launch_gemm_skinny_group(skinny, ns, g, bits, stream);
            if (e != hipSuccess) return e;
        }
        if (nt > 0) {
            const int variant = forced >= 0 ? forced : pick_tile_variant(tiled, nt, g, bits);
            if (variant == TILE_256x256SK) {
                // one stream-K launch per problem where the workspace holds its partial tiles
                int rest = 0;
                for (int i = 0; i < nt; ++i) {
                    const size_t need = streamk_workspace_bytes(tiled[i], g, bits);
                    if (need > 0 && workspace != nullptr && need <= workspace_bytes) {
                        const hipError_t e = launch_gemm_streamk(tiled[i], g, bits, workspace, workspace_bytes, stream);
                        if (e != hipSuccess) return e;
                    } else {
                        tiled[rest++] = tiled[i];
                    }
                }
                nt = rest;
                if (nt == 0) continue;
            }
            const hipError_t e = launch_gemm_tiled_group(tiled, nt, g, bits, variant, stream);
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

size_t grouped_workspace_bytes(const GemmProblem* probs, int count, int g, int bits) {
    if (forced_tile() == TILE_256x256SK) {
        size_t need = 0;
        for (int i = 0; i < count; ++i) {
            const size_t b = streamk_workspace_bytes(probs[i], g, bits);
            need = b > need ? b : need;
        }
        return need;
    }
    if (forced_tile() >= 0) return 0;
    const int kind = forced_skinny_kind();
    size_t need = 0;
    GemmProblem skinny[kMaxGroup];
    for (int base = 0; base < count; base += kMaxGroup) {
        const int n = count - base < kMaxGroup ? count - base : kMaxGroup;
        int ns = 0;
        for (int i = 0; i < n; ++i) {
            const GemmProblem& p = probs[base + i];
            if (use_skinny(p.M, p.N, p.K, g, bits)) skinny[ns++] = p;
        }
        // plan with an unbounded workspace and record what the split launches would need
        static char probe;
        take_resident(skinny, ns, g, bits, kind, &probe, size_t(-1),
                      [&](const GemmProblem*, int, const ResidentPlan& pl) {
                          const size_t b = resident_workspace_bytes(pl);
                          need = b > need ? b : need;
                          return hipSuccess;
                      });
    }
    return need;
}

}  // namespace lowbit

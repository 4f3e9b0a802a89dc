// Internal declarations shared by the HIP translation units of liblowbit (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lowbit {

struct GemmProblem {
    const uint16_t* X;  // bf16 [M, K]
    const uint32_t* W;  // packed codes [N, K*bits/32]
    const uint16_t* S;  // fp16 [N, K/g]
    uint16_t* Y;        // bf16 [M, N]
    int M, N, K;
};

// Several independent problems of one (g, bits) class in one launch.  Workgroup w of the
// launch belongs to the first problem i with w < tile_end[i] (inclusive prefix sums of the
// per-problem workgroup counts) and works on its local tile w - tile_end[i - 1].
constexpr int kMaxGroup = 16;
struct ProblemGroup {
    GemmProblem p[kMaxGroup];
    int tile_end[kMaxGroup];
    int count;
};

hipError_t launch_pack(const int8_t* codes, uint32_t* W, int64_t N, int64_t K, int bits,
                       int32_t* bad_count, hipStream_t stream);
hipError_t launch_unpack(const uint32_t* W, int8_t* codes, int64_t N, int64_t K, int bits,
                         hipStream_t stream);

// Tiled MFMA kernels (LDS-staged X, packed weights and scales).  `variant` selects the tile;
// TILE_288x192 is the 16x16x32-block kernel (ternary, g = 64 or 128 only).
enum TileVariant { TILE_256x128 = 0, TILE_256x256 = 1, TILE_128x256 = 2, TILE_64x256 = 3, TILE_288x192 = 4 };
hipError_t launch_gemm_tiled(const GemmProblem& p, int g, int bits, int variant, hipStream_t stream);

// Skinny-M kernel (M <= 32): split-K inside a workgroup, fixed-order LDS reduction.
// Shapes it does not cover (M > 32, K not a whole number of 64-byte row steps, or a
// (g, bits) whose scale group is smaller than the kernel's 16-byte chunk) go to the 64 x 256
// tile.
hipError_t launch_gemm_skinny(const GemmProblem& p, int g, int bits, hipStream_t stream);
bool skinny_supported(int g, int bits);

// Ring kernel (ternary, M <= 16, g = 64 / 128, K % 256 == 0, N % 64 == 0): deep LDS load
// ring, optional split-K across workgroups through a caller-provided workspace.
struct RingArgs {
    GemmProblem p;
    int splits;           // workgroups per column tile along K
    float* ws;            // fp32 partial sums (splits > 1)
    uint32_t* counters;   // one arrival counter per column tile, zero between calls
};
struct RingPlan {
    int nw;      // 16-column blocks per wave (a column tile is 4 * nw blocks)
    int splits;  // workgroups per column tile along K
    int tiles;   // column tiles
};
bool ring_supported(int64_t M, int64_t N, int64_t K, int g, int bits);
RingPlan plan_ring(int64_t N, int64_t K, int max_splits);
size_t ring_workspace_bytes(const RingPlan& plan, int64_t N);
hipError_t launch_gemm_ring(const GemmProblem& p, int g, const RingPlan& plan, void* workspace, hipStream_t stream);

// Grouped launch: problems of one (g, bits) class; one launch per kernel family and per
// kMaxGroup problems.
hipError_t launch_gemm_grouped(const GemmProblem* probs, int count, int g, int bits,
                               hipStream_t stream);
hipError_t launch_gemm_tiled_group(const GemmProblem* probs, int count, int g, int bits, int variant,
                                   hipStream_t stream);
hipError_t launch_gemm_skinny_group(const GemmProblem* probs, int count, int g, int bits, hipStream_t stream);

// Tile for a group of problems: fewest estimated rounds x tile work over the whole group.
int pick_tile_variant(const GemmProblem* probs, int count, int g, int bits);
int pick_tile_variant(int64_t M, int64_t N, int64_t K, int g, int bits);
const char* tile_variant_name(int variant);
bool tile16_supported(int g, int bits);
hipError_t launch_gemm_tile16_group(const GemmProblem* probs, int count, int g, hipStream_t stream);
bool use_skinny(int64_t M, int64_t N, int64_t K, int g, int bits);

}  // namespace lowbit

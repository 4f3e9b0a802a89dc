// Internal declarations shared by the HIP translation units of liblowbit (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdio.h>
#include <stdint.h>

namespace lowbit {

struct GemmProblem {
    const uint16_t* X;  // bf16 [M, K]
    const uint32_t* W;  // packed codes [N, K*bits/32]
    const uint16_t* S;  // fp16 [N, K/g]
    uint16_t* Y;        // bf16 [M, N]
    int M, N, K;
    const uint16_t* R = nullptr;     // gated-residual epilogue only: bf16 residual [M, N] (may be Y)
    const uint16_t* gate = nullptr;  // gated-residual epilogue only: bf16 gate [N]
    const uint16_t* B = nullptr;     // affine 4-bit groups only: fp16 biases [N, K/g]
};

// Epilogues of the 16x16-block tile kernel and of the resident kernel.
constexpr int kEpiPlain = 0;     // Y = X . W^T
constexpr int kEpiSwiglu = 1;    // W holds [gate | up] rows: Y = silu(X . Wg^T) * (X . Wu^T)
constexpr int kEpiResidual = 2;  // Y = R + gate[n] * (X . W^T)

// Tiles of `b` rows or columns over a dimension of n (64-bit: M may be up to 2^31 - 1).
inline int64_t tiles_of(int64_t n, int64_t b) { return (n + b - 1) / b; }

// Several independent problems of one (g, bits) class in one launch.  Workgroup w of the
// launch belongs to the first problem i with w < tile_end[i] (inclusive prefix sums of the
// per-problem workgroup counts) and works on its local tile w - tile_end[i - 1].
constexpr int kMaxGroup = 16;
constexpr int kComputeUnits = 256;  // MI355X
struct ProblemGroup {
    GemmProblem p[kMaxGroup];
    int tile_end[kMaxGroup];
    int count;
};

// LOWBIT_TRACE=1 (read at every launch): one line per GEMM kernel launch on stderr, naming the
// kernel family and its configuration, g, bits, grid and workgroup size, dynamic LDS, and the
// problems (M x N x K) of the launch.
bool trace_enabled();
void trace_launch(const char* family, const char* config, int g, int bits, const GemmProblem* probs, int count,
                  unsigned grid, unsigned block, unsigned lds);

hipError_t launch_pack(const int8_t* codes, uint32_t* W, int64_t N, int64_t K, int bits,
                       int32_t* bad_count, hipStream_t stream);
// Unsigned 4-bit levels 0 .. 15 -> nibble words (levels above 15 pack as 0 and are counted).
hipError_t launch_pack_u4(const uint8_t* levels, uint32_t* W, int64_t N, int64_t K, int32_t* bad_count,
                          hipStream_t stream);
hipError_t launch_unpack(const uint32_t* W, int8_t* codes, int64_t N, int64_t K, int bits,
                         hipStream_t stream);
// Ternary importers (import.hip): the layouts of include/lowbit.h's LOWBIT_LAYOUT_* values.
constexpr int kLayoutGemliteU8T = 1;
constexpr int kLayoutMlxU32 = 2;
hipError_t launch_import(const void* src, int layout, int zero, uint32_t* W, int64_t N, int64_t K,
                         int32_t* bad_count, hipStream_t stream);
hipError_t launch_import_binary_gemlite(const uint8_t* src, uint32_t* W, int64_t N, int64_t K, hipStream_t stream);

// Tiled MFMA kernels (LDS-staged X, packed weights and scales).  `variant` selects the tile;
// TILE_288x192 and TILE_96x192 are the 16x16x32-block kernel (g = 64 or 128 only).
enum TileVariant {
    TILE_256x128 = 0, TILE_256x256 = 1, TILE_128x256 = 2, TILE_64x256 = 3, TILE_288x192 = 4, TILE_96x192 = 5,
    TILE_96x192K2 = 6,  // 96 x 192 with K split between two groups of 4 waves (even step counts)
    TILE_64x128K2 = 7,  // 64 x 128, the same K split (4-bit codes: small output grids)
    TILE_256x192 = 8,   // 256 x 192 in 12 waves of 128 x 32 (M = 4096 in whole rounds at N = 3072)
    TILE_256x256SK = 9  // 256 x 256 stream-K through a workspace (TILE_256x256 where none is given)
};
inline bool is_tile16_variant(int v) {
    return v == TILE_288x192 || v == TILE_96x192 || v == TILE_96x192K2 || v == TILE_64x128K2 || v == TILE_256x192;
}
hipError_t launch_gemm_tiled(const GemmProblem& p, int g, int bits, int variant, hipStream_t stream);
// Stream-K on the 256 x 256 tile (ternary and binary codes): one workgroup per compute unit,
// each a contiguous range of the problem's (tile, 64-element step) units; split tiles are summed
// from fp32 partial tiles in the workspace (its first 4 KiB are arrival counters, zero between
// calls).  0 bytes: the shape is not covered.
size_t streamk_workspace_bytes(const GemmProblem& p, int g, int bits);
hipError_t launch_gemm_streamk(const GemmProblem& p, int g, int bits, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

// Skinny-M kernel (M <= 32): split-K inside a workgroup, fixed-order LDS reduction.
// Shapes it does not cover (M > 32, K not a whole number of 64-byte row steps, or a
// (g, bits) whose scale group is smaller than the kernel's 16-byte chunk) go to the 64 x 256
// tile.
hipError_t launch_gemm_skinny(const GemmProblem& p, int g, int bits, hipStream_t stream);
bool skinny_supported(int g, int bits);

// Resident kernel (ternary, M <= 16, g = 64 / 128, K % 256 == 0): the activations of a
// workgroup's K range in LDS, each wave issues every weight load of its (column block, K
// slice) at once; optionally split along K across workgroups through a caller workspace.
// One launch per group of problems with the same K.
struct ResidentPlan {
    int cb;      // column blocks per workgroup
    int ks;      // K slices per column block inside a workgroup (waves = cb * ks)
    int len;     // most steps of one wave; 0 = shape not covered
    int splits;  // workgroups per column group along K (> 1 needs the workspace)
    int tiles;   // column groups of the launch
};
bool resident_supported(int64_t M, int64_t N, int64_t K, int g, int bits);
ResidentPlan plan_resident(const GemmProblem* probs, int count, int g, bool may_split);
size_t resident_workspace_bytes(const ResidentPlan& plan);
bool resident_preferred(const GemmProblem* probs, int count, int g, bool may_split);
hipError_t launch_gemm_resident_group(const GemmProblem* probs, int count, int g, const ResidentPlan& plan,
                                      void* workspace, hipStream_t stream);
// Fused epilogues on the resident kernel (whole K); hipErrorNotSupported where no plan applies.
hipError_t launch_gemm_resident_epilogue(const GemmProblem& p, int g, int epi, hipStream_t stream);

// Grouped launch: problems of one (g, bits) class; one launch per kernel family and per
// kMaxGroup problems.
hipError_t launch_gemm_grouped(const GemmProblem* probs, int count, int g, int bits, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);
size_t grouped_workspace_bytes(const GemmProblem* probs, int count, int g, int bits);
hipError_t launch_gemm_tiled_group(const GemmProblem* probs, int count, int g, int bits, int variant,
                                   hipStream_t stream);
hipError_t launch_gemm_skinny_group(const GemmProblem* probs, int count, int g, int bits, hipStream_t stream);

// Tile for a group of problems: fewest estimated rounds x tile work over the whole group.
int pick_tile_variant(const GemmProblem* probs, int count, int g, int bits);
int pick_tile_variant(int64_t M, int64_t N, int64_t K, int g, int bits);
const char* tile_variant_name(int variant);
bool tile16_supported(int g, int bits);
// Fused epilogues on the 288 x 192 16x16-block tile (epi = kEpiSwiglu: each problem's W and S
// hold 2N rows, gate rows [0, N) then up rows [N, 2N), Y is [M, N]; epi = kEpiResidual: the
// problem's R and gate are set).
hipError_t launch_gemm_tile16_epilogue(const GemmProblem* probs, int count, int g, int bits, int epi,
                                       hipStream_t stream);
hipError_t launch_gemm_tile16_group(const GemmProblem* probs, int count, int g, int bits, int variant,
                                    hipStream_t stream);
// Affine 4-bit groups (unsigned levels, w = s * q + b with each problem's B set) on a 16x16-block
// tile; `variant` as for 4-bit codes.
hipError_t launch_gemm_tile16_affine(const GemmProblem* probs, int count, int g, int variant, hipStream_t stream);
bool use_skinny(int64_t M, int64_t N, int64_t K, int g, int bits);

}  // namespace lowbit

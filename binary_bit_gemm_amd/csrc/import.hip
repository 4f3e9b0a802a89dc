// Importers of ternary weights packed by other runtimes into this library's word format
// (offline / load-time steps, like lowbit_pack).
//
// Both source layouts hold unsigned 2-bit levels q in {0..3}, least significant field first,
// with the ternary code c = q - zero.  They differ in orientation:
//   GemLite (uint8, transposed): src[K/4][N]; byte (j, n) holds codes k = 4j .. 4j+3 of
//     output row n (the comment thread of the Bonsai-Image-Demo pull request "CPU bring-up":
//     uint8 packed over K with a transpose, (in_features / 4, out_features));
//   MLX (uint32, row-major by output): src[N][K/16]; word (n, j) holds codes k = 16j .. 16j+15
//     ("backend/ -- FastAPI Mac backend", section "Checkpoint layout": uint32 packed weights).
// Codes outside {-1, 0, +1} pack as the 0 field and are counted, as in lowbit_pack.
// Binary weights (the binary model card's GemLite 1-bit format) take the same transposed byte
// layout with 8 codes per byte, src[K/8][N], bit i of byte (j, n) holding code 8j + i (bit 1 ->
// +1): the bytes of a word are then already this library's bits, and only the transpose remains.
#include "lowbit_internal.h"

namespace lowbit {
namespace {

constexpr int kThreads = 256;

// the 2-bit field of this library for level q (00 -> 0, 01 -> +1, 10 -> -1)
__device__ __forceinline__ uint32_t level_field(uint32_t q, int zero, int& bad) {
    const int c = int(q) - zero;
    bad += (c < -1 || c > 1);
    return c == 1 ? 1u : (c == -1 ? 2u : 0u);
}

// 16 source levels (a uint32 of unsigned fields, LSB first) -> one word of this library
__device__ __forceinline__ uint32_t remap_word(uint32_t src, int zero, int& bad) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) w |= level_field((src >> (2 * i)) & 3u, zero, bad) << (2 * i);
    return w;
}

__device__ __forceinline__ void add_bad(int bad, int32_t* bad_count) {
    if (bad_count == nullptr) return;
    if (__ballot(bad != 0) == 0) return;
    int total = bad;
    for (int off = 32; off > 0; off >>= 1) total += __shfl_xor(total, off);
    if ((threadIdx.x & 63) == 0) atomicAdd(bad_count, total);
}

// MLX rows: the same positions, only the field values change.  One thread per word.
__global__ __launch_bounds__(kThreads) void import_mlx_kernel(const uint32_t* __restrict__ src,
                                                              uint32_t* __restrict__ W, int64_t nwords,
                                                              int zero, int32_t* __restrict__ bad_count) {
    const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    int bad = 0;
    if (i < nwords) W[i] = remap_word(src[i], zero, bad);
    add_bad(bad, bad_count);
}

// GemLite transposed bytes: a workgroup turns a 64-row (256 codes along K) x 64-column
// source tile into 64 output rows of 16 words.  The tile goes through LDS so that the
// reads (consecutive n within a source row) and the writes (consecutive words within an
// output row) both stay coalesced.
constexpr int kTileN = 64;      // output rows (source columns) per workgroup
constexpr int kTileJ = 16;      // output words per row per workgroup
constexpr int kTileR = 4 * kTileJ;  // source rows per workgroup

template <int BITS>
__global__ __launch_bounds__(kThreads) void import_gemlite_kernel(const uint8_t* __restrict__ src,
                                                                  uint32_t* __restrict__ W, int64_t N,
                                                                  int64_t K, int zero,
                                                                  int32_t* __restrict__ bad_count) {
    // [source row][4 columns per dword]; one padding dword per row
    __shared__ uint32_t tile[kTileR][kTileN / 4 + 1];
    const int64_t rows = K * BITS / 8, wpr = K * BITS / 32;
    const int64_t n0 = int64_t(blockIdx.x) * kTileN;
    const int64_t r0 = int64_t(blockIdx.y) * kTileR;
    const int t = threadIdx.x;
    // N % 16 == 0: a dword of four columns is wholly in range or wholly out of it
#pragma unroll
    for (int v = 0; v < kTileR * kTileN / 4 / kThreads; ++v) {
        const int d = v * kThreads + t;
        const int r = d / (kTileN / 4), c = d % (kTileN / 4);
        const int64_t gr = r0 + r, gn = n0 + 4 * c;
        uint32_t x = 0;
        if (gr < rows && gn < N) x = *reinterpret_cast<const uint32_t*>(src + gr * N + gn);
        tile[r][c] = x;
    }
    __syncthreads();
    const int n = t / 4;              // output row within the tile
    const int jq = t % 4;             // which four of the tile's 16 words
    const int64_t gn = n0 + n;
    int bad = 0;
    if (gn < N) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = 4 * jq + u;
            const int64_t gj = blockIdx.y * int64_t(kTileJ) + j;
            if (gj >= wpr) break;
            // the four source bytes of this word, in K order, as one uint32 of 16 levels
            uint32_t levels = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) levels |= ((tile[4 * j + i][n / 4] >> (8 * (n % 4))) & 0xFFu) << (8 * i);
            W[gn * wpr + gj] = BITS == 2 ? remap_word(levels, zero, bad) : levels;
        }
    }
    add_bad(bad, bad_count);
}

}  // namespace

hipError_t launch_import(const void* src, int layout, int zero, uint32_t* W, int64_t N, int64_t K,
                         int32_t* bad_count, hipStream_t stream) {
    if (N * K == 0) return hipSuccess;
    if (layout == kLayoutMlxU32) {
        const int64_t nwords = N * K / 16;
        const dim3 grid(unsigned((nwords + kThreads - 1) / kThreads));
        hipLaunchKernelGGL(import_mlx_kernel, grid, dim3(kThreads), 0, stream, static_cast<const uint32_t*>(src), W,
                           nwords, zero, bad_count);
    } else {
        const dim3 grid(unsigned((N + kTileN - 1) / kTileN), unsigned((K / 16 + kTileJ - 1) / kTileJ));
        hipLaunchKernelGGL(import_gemlite_kernel<2>, grid, dim3(kThreads), 0, stream, static_cast<const uint8_t*>(src),
                           W, N, K, zero, bad_count);
    }
    return hipGetLastError();
}

hipError_t launch_import_binary_gemlite(const uint8_t* src, uint32_t* W, int64_t N, int64_t K, hipStream_t stream) {
    if (N * K == 0) return hipSuccess;
    const dim3 grid(unsigned((N + kTileN - 1) / kTileN), unsigned((K / 32 + kTileJ - 1) / kTileJ));
    hipLaunchKernelGGL(import_gemlite_kernel<1>, grid, dim3(kThreads), 0, stream, src, W, N, K, 0,
                       static_cast<int32_t*>(nullptr));
    return hipGetLastError();
}

}  // namespace lowbit

// Large-M packed low-bit GEMM: Y[M,N] = X[M,K] . dequant(W)[N,K]^T on the gfx950 matrix cores.
//
// Workgroup = 4 waves (256 threads) computing a BM x BN tile of Y; each wave owns a
// WM x WN sub-tile made of 32x32 blocks (v_mfma_f32_32x32x16_bf16).  Per K step of
// KS = max(64, g) elements:
//   * X[BM, KS] is copied HBM -> LDS with direct-to-LDS loads (global_load_lds_dwordx4),
//     double-buffered, 16-byte chunks XOR-swizzled by row to keep ds_read_b128 conflict-free;
//   * every lane loads the packed words of its own weight row (one column of Y) straight
//     into registers, together with that row's fp16 group scales, one step ahead;
//   * codes are expanded in registers to bf16 operand dwords (lowbit_device.h);
//   * per scale group: tmp = sum of g/16 MFMAs, then acc += scale * tmp in fp32 -- the
//     group scale multiplies the exact partial sum after the MFMA and is never rounded
//     to bf16 (w = scale_g * b of the binary model card, applied per group);
//   * epilogue: fp32 -> bf16 round-to-nearest-even, store.
//
// Which 8 of a group's codes a lane feeds to one MFMA is a free choice as long as the A
// (activation) and B (weight) operands agree: lane half h (lanes 32h..32h+31) takes the
// h-th half of each group, chunk j takes codes 8j..8j+7 of that half.  Consecutive codes
// in K therefore meet consecutive activations, so X tiles need no reordering.
#include "lowbit_device.h"
#include "lowbit_internal.h"

namespace lowbit {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <int BITS, int G, int BM, int BN, int WAVES_M>
struct TileCfg {
    static constexpr int WAVES_N = kWaves / WAVES_M;
    static constexpr int WM = BM / WAVES_M;
    static constexpr int WN = BN / WAVES_N;
    static constexpr int MB = WM / 32;                 // 32-row blocks per wave
    static constexpr int NB = WN / 32;                 // 32-col blocks per wave
    static constexpr int KS = G > 64 ? G : 64;         // K elements per step
    static constexpr int GPS = KS / G;                 // scale groups per step
    static constexpr int CHUNKS = G / 16;              // MFMAs per group per block
    static constexpr int ROW_BYTES = KS * 2;           // bf16 row of the X tile
    static constexpr int TILE_BYTES = BM * ROW_BYTES;
    static constexpr int CHUNKS_PER_ROW = KS / 8;      // 16-byte chunks per X row
    static constexpr int LOADS = TILE_BYTES / (16 * kThreads);  // global_load_lds per thread per step
    // Packed words of one lane-half of one group: G/2 codes.
    static constexpr int WPH = (G / 2) * BITS / 32 > 0 ? (G / 2) * BITS / 32 : 1;
    static constexpr bool HALF_WORD = (G / 2) * BITS < 32;  // binary g = 32: 16 codes per half
    static_assert(MB >= 1 && NB >= 1, "wave tile too small");
    static_assert(TILE_BYTES % (16 * kThreads) == 0, "tile not a whole number of loads");
};

__device__ __forceinline__ int lds_offset(int row, int chunk, int row_bytes) {
    return row * row_bytes + ((chunk ^ (row & 7)) << 4);
}

template <int BITS, int G, int BM, int BN, int WAVES_M>
__global__ __launch_bounds__(kThreads, 1) void gemm_tiled_kernel(GemmProblem p, int tiles_m, int tiles_n) {
    using C = TileCfg<BITS, G, BM, BN, WAVES_M>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    const int M = p.M, N = p.N, K = p.K;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wave_m = wave % WAVES_M, wave_n = wave / WAVES_M;
    const int half = lane >> 5, col = lane & 31;

    const int tile = xcd_remap(blockIdx.x, tiles_m * tiles_n);
    const int tm = tile / tiles_n, tn = tile % tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;
    const int wm0 = wave_m * C::WM, wn0 = wave_n * C::WN;

    const int kgroups = K / G;
    const int ksteps = (K + C::KS - 1) / C::KS;
    const int words_per_row = K * BITS / 32;

    // ---- X tile loader: thread t handles 16-byte chunk t + i*kThreads of the tile ----
    auto issue_x_loads = [&](int step, int buf) {
        const int k0 = step * C::KS;
#pragma unroll
        for (int i = 0; i < C::LOADS; ++i) {
            const int slot = i * kThreads + threadIdx.x;          // LDS chunk index
            const int r = slot / C::CHUNKS_PER_ROW;
            const int pc = slot % C::CHUNKS_PER_ROW;
            const int c = pc ^ (r & 7);                            // logical chunk stored there
            int gr = m0 + r;
            gr = gr < M ? gr : M - 1;
            int gk = k0 + c * 8;
            gk = gk < K ? gk : K - 8;
            const uint16_t* src = p.X + int64_t(gr) * K + gk;
            // LDS destination of the wave: base + lane*16, contiguous per wave
            unsigned char* dst = smem + buf * C::TILE_BYTES + (i * kThreads + wave * 64) * 16;
            __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
        }
    };

    // ---- per-lane weight rows: column n of Y for each 32-col block of the wave ----
    int wrow[C::NB];
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) {
        int n = n0 + wn0 + nb * 32 + col;
        wrow[nb] = n < N ? n : N - 1;
    }

    uint32_t wcur[C::NB][C::GPS][C::WPH], wnxt[C::NB][C::GPS][C::WPH];
    uint16_t scur[C::NB][C::GPS], snxt[C::NB][C::GPS];

    auto load_w = [&](int step, uint32_t (&wd)[C::NB][C::GPS][C::WPH], uint16_t (&sd)[C::NB][C::GPS]) {
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
#pragma unroll
            for (int q = 0; q < C::GPS; ++q) {
                int grp = step * C::GPS + q;
                grp = grp < kgroups ? grp : kgroups - 1;
                const uint32_t* src = p.W + int64_t(wrow[nb]) * words_per_row;
                if (C::HALF_WORD) {
                    wd[nb][q][0] = src[grp];
                } else {
                    const int off = grp * (2 * C::WPH) + half * C::WPH;
#pragma unroll
                    for (int w = 0; w < C::WPH; ++w) wd[nb][q][w] = src[off + w];
                }
                sd[nb][q] = p.S[int64_t(wrow[nb]) * kgroups + grp];
            }
        }
    };

    f32x16_t acc[C::MB][C::NB];
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.0f;

    issue_x_loads(0, 0);
    load_w(0, wcur, scur);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    const float code_scale = BITS == 2 ? 0.5f : -0.5f;  // operand holds 2c (ternary), -2c (binary)

    for (int step = 0; step < ksteps; ++step) {
        const int buf = step & 1;
        const bool more = step + 1 < ksteps;
        if (more) {
            issue_x_loads(step + 1, buf ^ 1);
            load_w(step + 1, wnxt, snxt);
        }
        const unsigned char* xt = smem + buf * C::TILE_BYTES;

#pragma unroll
        for (int q = 0; q < C::GPS; ++q) {
            if (step * C::GPS + q >= kgroups) break;  // K tail (g = 32 with K % 64 == 32)

            // Expand this group's codes: bfr[nb][j] = operand of MFMA chunk j.
            u32x4_t bfr[C::NB][C::CHUNKS];
            float sc[C::NB];
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb) {
                uint32_t d[C::CHUNKS * 4];
                if (BITS == 2) {
#pragma unroll
                    for (int w = 0; w < C::WPH; ++w) expand_ternary_word(wcur[nb][q][w], d + 8 * w);
                } else if (C::HALF_WORD) {
                    expand_binary_word<8>(wcur[nb][q][0] >> (16 * half), d);
                } else {
#pragma unroll
                    for (int w = 0; w < C::WPH; ++w) expand_binary_word<16>(wcur[nb][q][w], d + 16 * w);
                }
#pragma unroll
                for (int j = 0; j < C::CHUNKS; ++j)
                    bfr[nb][j] = u32x4_t{d[4 * j], d[4 * j + 1], d[4 * j + 2], d[4 * j + 3]};
                sc[nb] = half_bits_to_float(scur[nb][q]) * code_scale;
            }

#pragma unroll
            for (int mb = 0; mb < C::MB; ++mb) {
                const int row = wm0 + mb * 32 + col;
                bf16x8_t afr[C::CHUNKS];
#pragma unroll
                for (int j = 0; j < C::CHUNKS; ++j) {
                    const int chunk = (q * G + half * (G / 2)) / 8 + j;
                    afr[j] = *reinterpret_cast<const bf16x8_t*>(xt + lds_offset(row, chunk, C::ROW_BYTES));
                }
#pragma unroll
                for (int nb = 0; nb < C::NB; ++nb) {
                    f32x16_t tmp = {};
#pragma unroll
                    for (int j = 0; j < C::CHUNKS; ++j)
                        tmp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            afr[j], __builtin_bit_cast(bf16x8_t, bfr[nb][j]), tmp, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[mb][nb][i] = __builtin_fmaf(sc[nb], tmp[i], acc[mb][nb][i]);
                }
            }
        }

        if (more) {
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
                for (int q = 0; q < C::GPS; ++q) {
                    scur[nb][q] = snxt[nb][q];
#pragma unroll
                    for (int w = 0; w < C::WPH; ++w) wcur[nb][q][w] = wnxt[nb][q][w];
                }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }

    // ---- epilogue: lane holds column col of each 32x32 block, rows 8*(i/4) + 4*half + i%4 ----
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
            const int n = n0 + wn0 + nb * 32 + col;
            if (n >= N) continue;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = m0 + wm0 + mb * 32 + 8 * (i / 4) + 4 * half + (i % 4);
                if (m < M) p.Y[int64_t(m) * N + n] = float_to_bf16_bits(acc[mb][nb][i]);
            }
        }
    }
}

template <int BITS, int G, int BM, int BN, int WAVES_M>
hipError_t launch_cfg(const GemmProblem& p, hipStream_t stream) {
    using C = TileCfg<BITS, G, BM, BN, WAVES_M>;
    const int tiles_m = (p.M + BM - 1) / BM;
    const int tiles_n = (p.N + BN - 1) / BN;
    const size_t lds = 2 * size_t(C::TILE_BYTES);
    auto kern = gemm_tiled_kernel<BITS, G, BM, BN, WAVES_M>;
    static bool attr_set = false;  // per instantiation; idempotent if raced
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3(tiles_m * tiles_n), dim3(kThreads), lds, stream, p, tiles_m, tiles_n);
    return hipGetLastError();
}

template <int BITS, int G>
hipError_t launch_bits_g(const GemmProblem& p, int variant, hipStream_t stream) {
    switch (variant) {
        case TILE_256x128: return launch_cfg<BITS, G, 256, 128, 2>(p, stream);
        case TILE_128x128: return launch_cfg<BITS, G, 128, 128, 2>(p, stream);
        default:           return launch_cfg<BITS, G, 64, 128, 2>(p, stream);
    }
}

}  // namespace

int pick_tile_variant(int64_t M, int64_t N, int64_t K) {
    (void)N; (void)K;
    if (M >= 1024) return TILE_256x128;
    if (M >= 256) return TILE_128x128;
    return TILE_64x128;
}

hipError_t launch_gemm_tiled(const GemmProblem& p, int g, int bits, int variant, hipStream_t stream) {
    if (bits == 2) {
        switch (g) {
            case 32: return launch_bits_g<2, 32>(p, variant, stream);
            case 64: return launch_bits_g<2, 64>(p, variant, stream);
            default: return launch_bits_g<2, 128>(p, variant, stream);
        }
    }
    switch (g) {
        case 32: return launch_bits_g<1, 32>(p, variant, stream);
        case 64: return launch_bits_g<1, 64>(p, variant, stream);
        default: return launch_bits_g<1, 128>(p, variant, stream);
    }
}

}  // namespace lowbit

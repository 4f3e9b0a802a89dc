// Skinny-M packed low-bit GEMM (M <= 32 ternary, M <= 16 binary): Y[M,N] = X[M,K] . dequant(W)[N,K]^T.
//
// With 16 or 32 activation rows the work per weight byte is small: every code is expanded
// to a bf16 operand once and meets only M activations.  Each workgroup owns a stripe of NCB
// column blocks of 16 output columns and its waves split K into contiguous step ranges.  The
// partial sums of the waves are combined in LDS in a fixed order (wave 0 first), so the
// result does not depend on timing.  On the way in:
//   * packed weights stream from HBM straight into registers, 16 bytes per lane per column
//     block and step (one 64-byte piece of each of the block's 16 weight rows);
//   * activations (a few hundred KB at most, so L2-resident) are copied per wave and step
//     into LDS for ternary codes and M <= 16, and loaded straight into registers, 16 bytes
//     per lane per MFMA, otherwise;
//   * one step of both is in flight while the previous step is computed.
//
// MFMA: v_mfma_f32_16x16x32_bf16, A = 16 activation rows x 32 K, B = 32 K x 16 weight rows.
// A 16-byte weight load gives lane (q, n) the four words of chunk q of row n (chunk = one
// 16-byte quarter of the step = 64 ternary / 128 binary codes).  Four lane-row swaps
// (v_permlane32_swap, v_permlane16_swap) transpose the 4x4 (lane quarter, word) blocks so
// that register c holds, in lane quarter q, word q of chunk c.  Then each MFMA takes eight
// consecutive codes of every quarter's word of one chunk, so its 32 K positions lie in one
// chunk -- and a chunk lies in one scale group for ternary g = 64 or 128 and binary g = 128.
// A smaller group splits the chunk by lane quarters (ternary g = 32 and binary g = 64: two
// groups, quarters 0-1 and 2-3; binary g = 32: four, one per quarter): each MFMA of the
// chunk then runs once per group, with the activation operand of the other groups'
// quarters set to zero, and each result takes its own group's scale.  The group scale multiplies
// the exact partial sum after the MFMA, in fp32 (w = scale_g * b, model card "Binary
// Weight Representation: 1-bit g128"); the operand holds 2c (ternary) or -2c (binary) and
// the factor +-1/2 is applied once to the final sum.
#include <cstdlib>

#include "lowbit_device.h"
#include "lowbit_internal.h"

namespace lowbit {
namespace {


template <int BITS>
struct SkinnyFmt {
    static constexpr int CPW = 32 / BITS;           // codes per word
    static constexpr int CHUNK = 4 * CPW;           // codes per 16-byte chunk of a row
    static constexpr int STEP = 4 * CHUNK;          // codes per 64-byte step of a row
    static constexpr int MPC = CPW / 8;             // MFMAs per chunk (8 codes per quarter each)
    static constexpr int XPS = 4 * MPC;             // activation operands per step and row block
};

template <int BITS, int G, int MB, int NCB, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 2) void gemm_skinny_kernel(ProblemGroup grp) {
    using F = SkinnyFmt<BITS>;
    constexpr int GPS = F::STEP / G;                      // scale groups per step
    constexpr bool kSplitChunk = F::CHUNK > G;            // groups smaller than a chunk
    constexpr int GPC = kSplitChunk ? F::CHUNK / G : 1;   // scale groups per chunk (1, 2 or 4)
    constexpr int CPG = kSplitChunk ? 1 : G / F::CHUNK;   // chunks per scale group (1 or 2)
    constexpr int SD = GPS / 2;                           // scale dwords per row and step
    static_assert(G % F::CHUNK == 0 || GPC == 2 || GPC == 4, "a chunk lies in 1, 2 or 4 scale groups");
    static_assert(GPS == 2 || GPS == 4 || GPS == 8 || GPS == 16, "scale groups per step");

    // Activations of one step for the ternary single-row-block case go through LDS: each
    // wave copies its own 16 x 256 slice with contiguous 16-byte direct-to-LDS loads (two
    // whole 512-byte rows per instruction) and reads the MFMA operands back with ds_read.
    // Loading the operands straight from global memory would make every instruction touch
    // 16 rows; the vector-memory path pays per row touched, and that cost dominated.
    // Rows are stored with their 16-byte chunk c at position c ^ (row & 15), so that the 16
    // rows one operand read touches fall into 16 different bank groups.
    constexpr bool kXLds = BITS == 2 && MB == 1;
    constexpr int kXRow = F::STEP * 2;                 // bytes of one activation row per step
    constexpr int kXWave = kXLds ? 16 * kXRow : 16;    // bytes per wave and stage
    __shared__ __attribute__((aligned(16))) unsigned char xa[WAVES * kXWave];
    __shared__ __attribute__((aligned(16))) unsigned char xb[WAVES * kXWave];
    __shared__ f32x4_t red[WAVES][MB][NCB][64];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
    const int q = lane >> 4, n = lane & 15;
    int pi = 0;
    while (pi + 1 < grp.count && int(blockIdx.x) >= grp.tile_end[pi]) ++pi;
    const GemmProblem p = grp.p[pi];
    const int stripe = int(blockIdx.x) - (pi > 0 ? grp.tile_end[pi - 1] : 0);
    const int M = p.M, N = p.N, K = p.K;

    // The host guarantees N % (16 * NCB) == 0 and K % STEP == 0 (whole steps, so every
    // row's scales of a step are one aligned 4- or 8-byte piece).
    const int n0 = stripe * (16 * NCB);
    const uint32_t row_bytes = uint32_t(K) * BITS / 8;
    const int kgroups = K / G;
    const uint32_t s_row_bytes = uint32_t(kgroups) * 2u;
    const int steps = K / F::STEP;
    const int s_begin = wave * steps / WAVES, s_end = (wave + 1) * steps / WAVES;

    const unsigned char* w_wg = reinterpret_cast<const unsigned char*>(p.W) + size_t(n0) * row_bytes;
    const unsigned char* s_wg = reinterpret_cast<const unsigned char*>(p.S) + size_t(n0) * s_row_bytes;
    const unsigned char* x_base = reinterpret_cast<const unsigned char*>(p.X);
    const uint32_t w_bytes = uint32_t(16 * NCB) * row_bytes;
    const uint32_t s_bytes = uint32_t(16 * NCB) * s_row_bytes;
    const uint32_t x_bytes = uint32_t(M) * uint32_t(K) * 2u;

    // Per-lane offsets within a step's resources (rebased to the step's first byte; rows of
    // X at or past M read as zero).
    uint32_t w_off[NCB], s_off[NCB], x_off[MB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        w_off[cb] = uint32_t(16 * cb + n) * row_bytes + uint32_t(16 * q);
        s_off[cb] = uint32_t(16 * cb + n) * s_row_bytes;
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) x_off[mb] = (uint32_t(16 * mb + n) * uint32_t(K) + uint32_t(q * F::CPW)) * 2u;
    // LDS staging of X: copy instruction i brings rows 2i, 2i+1; lane l stores position
    // l & 31 of row 2i + (l >> 5), which holds source chunk position ^ (row & 15).
    constexpr int kXCopies = kXLds ? 16 * kXRow / 1024 : 1;
    constexpr int kXChunks = kXRow / 16;
    uint32_t x_dma_off[kXCopies];
    int x_rd[F::XPS];
    if constexpr (kXLds) {
#pragma unroll
        for (int i = 0; i < kXCopies; ++i) {
            const int r = 2 * i + (lane >> 5), pos = lane & 31;
            x_dma_off[i] = uint32_t(r) * uint32_t(K) * 2u + uint32_t((pos ^ (r & 15)) & (kXChunks - 1)) * 16u;
        }
        // operand (c, j) of lane (q, m): logical chunk 8c + 2q + j of row m
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int j = 0; j < F::MPC; ++j) {
                const int ch = (c * F::CHUNK + q * F::CPW + 8 * j) / 8;
                x_rd[c * F::MPC + j] = wave * kXWave + n * kXRow + ((ch ^ n) << 4);
            }
    }

    struct Stage {
        u32x4_t w[NCB];
        bf16x8_t x[MB][F::XPS];
        uint32_t s[NCB][SD];
    };

    // Loads of a step past the wave's range go through empty resources: they are issued (so
    // that both stages are plain loop-carried values without copies) but read nothing.
    auto load = [&](Stage& st, int s, unsigned char* xbuf) {
        // Nothing of the previous compute may move below this point: it read this stage's
        // LDS buffer, which the copies below overwrite.
        __builtin_amdgcn_sched_barrier(0);
        const bool live = s < s_end;
        s = live ? s : s_begin;
        const __amdgpu_buffer_rsrc_t wr = make_rsrc(w_wg + uint32_t(s) * 64u, live ? w_bytes - uint32_t(s) * 64u : 0u);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
            st.w[cb] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(wr, w_off[cb], 0, 0));
        const uint32_t xk = uint32_t(s) * F::STEP * 2u;
        const __amdgpu_buffer_rsrc_t xr = make_rsrc(x_base + xk, live ? x_bytes - xk : 0u);
        if constexpr (kXLds) {
#pragma unroll
            for (int i = 0; i < kXCopies; ++i) dma16(xr, xbuf + wave * kXWave + i * 1024, x_dma_off[i], 0);
        } else {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int j = 0; j < F::MPC; ++j)
                        st.x[mb][c * F::MPC + j] = __builtin_bit_cast(
                            bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(
                                          xr, x_off[mb] + uint32_t(c * F::CHUNK + 8 * j) * 2u, 0, 0));
        }
        const uint32_t sk = uint32_t(s) * GPS * 2u;
        const __amdgpu_buffer_rsrc_t sr = make_rsrc(s_wg + sk, live ? s_bytes - sk : 0u);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            if constexpr (SD >= 4) {
#pragma unroll
                for (int h = 0; h < SD / 4; ++h) {
                    const u32x4_t v = __builtin_bit_cast(
                        u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(sr, s_off[cb] + uint32_t(16 * h), 0, 0));
#pragma unroll
                    for (int e = 0; e < 4; ++e) st.s[cb][4 * h + e] = v[e];
                }
            } else if constexpr (SD == 2) {
                const u32x2_t v = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(sr, s_off[cb], 0, 0));
                st.s[cb][0] = v[0];
                st.s[cb][1] = v[1];
            } else {
                st.s[cb][0] = __builtin_amdgcn_raw_buffer_load_b32(sr, s_off[cb], 0, 0);
            }
        }
        // Keep the scheduler from sinking these loads towards their use (it would trade the
        // prefetch distance for registers).
        __builtin_amdgcn_sched_barrier(0);
    };

    f32x4_t acc[MB][NCB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[mb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto scale_of = [&](const uint32_t (&sv)[SD], int gi) {  // fp16 scale of group gi of the step
        const uint32_t sw = sv[gi >> 1];
        return half_bits_to_float(uint16_t((gi & 1) ? (sw >> 16) : (sw & 0xFFFFu)));
    };
    const int lane_group = q / (4 / GPC);  // split chunks: the chunk group of the lane's codes

    auto compute = [&](Stage& st, const unsigned char* xbuf) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) transpose_words(st.w[cb]);
        if constexpr (kSplitChunk) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                // the chunk's activation operands, one copy per group with the other groups'
                // quarters zeroed (a lane-constant select)
                bf16x8_t xg[GPC][MB][F::MPC];
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int j = 0; j < F::MPC; ++j) {
                        const u32x4_t v = __builtin_bit_cast(
                            u32x4_t, kXLds ? *reinterpret_cast<const bf16x8_t*>(xbuf + x_rd[c * F::MPC + j])
                                           : st.x[mb][c * F::MPC + j]);
#pragma unroll
                        for (int h = 0; h < GPC; ++h) {
                            u32x4_t m;
#pragma unroll
                            for (int e = 0; e < 4; ++e) m[e] = lane_group == h ? v[e] : 0u;
                            xg[h][mb][j] = __builtin_bit_cast(bf16x8_t, m);
                        }
                    }
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    uint32_t d[F::CPW / 2];
                    if constexpr (BITS == 2)
                        expand_ternary_word(st.w[cb][c], d);
                    else
                        expand_binary_word<16>(st.w[cb][c], d);
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
                        for (int h = 0; h < GPC; ++h) {
                            f32x4_t t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int j = 0; j < F::MPC; ++j)
                                t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    xg[h][mb][j],
                                    __builtin_bit_cast(bf16x8_t, u32x4_t{d[4 * j], d[4 * j + 1], d[4 * j + 2], d[4 * j + 3]}),
                                    t, 0, 0, 0);
                            const float sc = scale_of(st.s[cb], GPC * c + h);
#pragma unroll
                            for (int i = 0; i < 4; ++i) acc[mb][cb][i] = __builtin_fmaf(sc, t[i], acc[mb][cb][i]);
                        }
                    }
                }
            }
            return;
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                uint32_t d[F::CPW / 2];
                if constexpr (BITS == 2) {
                    expand_ternary_word(st.w[cb][c], d);
                } else {
                    expand_binary_word<16>(st.w[cb][c], d);
                }
                const float sc = scale_of(st.s[cb], c / CPG);  // group within the step
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    f32x4_t t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int j = 0; j < F::MPC; ++j)
                        t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            kXLds ? *reinterpret_cast<const bf16x8_t*>(xbuf + x_rd[c * F::MPC + j])
                                  : st.x[mb][c * F::MPC + j],
                            __builtin_bit_cast(bf16x8_t, u32x4_t{d[4 * j], d[4 * j + 1], d[4 * j + 2], d[4 * j + 3]}), t,
                            0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[mb][cb][i] = __builtin_fmaf(sc, t[i], acc[mb][cb][i]);
                }
            }
        }
    };

    // Steps in pairs; no branch separates a stage's loads from the compute of the other
    // stage, so the loads stay where they are issued (a step ahead of their use).
    Stage a, b;
    load(a, s_begin, xa);
    int s = s_begin;
    for (; s + 1 < s_end; s += 2) {
        load(b, s + 1, xb);
        compute(a, xa);
        load(a, s + 2, xa);
        compute(b, xb);
    }
    if (s < s_end) compute(a, xa);

    // ---- fixed-order reduction over the waves, then the bf16 epilogue ----
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) red[wave][mb][cb][lane] = acc[mb][cb];
    __syncthreads();

    const float code_scale = BITS == 2 ? 0.5f : -0.5f;  // operand holds 2c (ternary), -2c (binary)
    for (int t = threadIdx.x; t < MB * NCB * 64; t += 64 * WAVES) {
        const int l = t & 63, cb = (t >> 6) % NCB, mb = (t >> 6) / NCB;
        f32x4_t v = red[0][mb][cb][l];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) {
            const f32x4_t u = red[w][mb][cb][l];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] += u[i];
        }
        // 16x16 MFMA result layout: lane l holds column l % 16, rows 4 * (l / 16) + i.
        const int col = n0 + 16 * cb + (l & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 16 * mb + 4 * (l >> 4) + i;
            if (m < M) p.Y[int64_t(m) * N + col] = float_to_bf16_bits(v[i] * code_scale);
        }
    }
}

template <int BITS, int G, int MB, int NCB>
hipError_t launch_cfg(const GemmProblem* probs, int count, hipStream_t stream) {
    constexpr int WAVES = 4;
    ProblemGroup grp{};
    int total = 0;
    for (int i = 0; i < count; ++i) {
        grp.p[i] = probs[i];
        total += probs[i].N / (16 * NCB);
        grp.tile_end[i] = total;
    }
    grp.count = count;
    hipLaunchKernelGGL((gemm_skinny_kernel<BITS, G, MB, NCB, WAVES>), dim3(total), dim3(64 * WAVES), 0, stream, grp);
    const hipError_t e = hipGetLastError();
    if (e == hipSuccess && trace_enabled()) {
        char cfg[64];
        snprintf(cfg, sizeof cfg, "row_blocks=%d column_blocks=%d waves=%d", MB, NCB, WAVES);
        trace_launch("skinny", cfg, G, BITS, probs, count, unsigned(total), 64u * WAVES, 0u);
    }
    return e;
}

// Wider stripes only where the registers allow them: four column blocks for one row block of
// ternary codes, two for binary codes (twice the activation operands per step), one for two
// row blocks and for binary codes with groups of 32 (four masked operand copies per chunk).
template <int BITS, int G, int MB>
hipError_t launch_mb(const GemmProblem* probs, int count, int ncb, hipStream_t stream) {
    if constexpr (MB == 1 && BITS == 2) {
        if (ncb >= 4) return launch_cfg<BITS, G, MB, 4>(probs, count, stream);
    }
    if constexpr (MB == 1 && !(BITS == 1 && G == 32)) {
        if (ncb >= 2) return launch_cfg<BITS, G, MB, 2>(probs, count, stream);
    }
    return launch_cfg<BITS, G, MB, 1>(probs, count, stream);
}

template <int BITS, int G>
hipError_t launch_bits_g(const GemmProblem* probs, int count, int max_m, int ncb, hipStream_t stream) {
    if constexpr (BITS == 1) {
        return launch_mb<BITS, G, 1>(probs, count, ncb, stream);
    } else {
        return max_m <= 16 ? launch_mb<BITS, G, 1>(probs, count, ncb, stream)
                           : launch_mb<BITS, G, 2>(probs, count, ncb, stream);
    }
}

// Column blocks per workgroup: the widest stripe (dividing every N / 16) that still gives
// every compute unit about two workgroups -- X is re-read from L2 once per workgroup, so
// wider stripes read less of it.
int pick_ncb(const GemmProblem* probs, int count) {
    int64_t blocks = 0;
    bool div4 = true, div2 = true;
    for (int i = 0; i < count; ++i) {
        const int64_t b = probs[i].N / 16;
        blocks += b;
        div4 = div4 && b % 4 == 0;
        div2 = div2 && b % 2 == 0;
    }
    int ncb = 1;
    if (div4 && blocks >= 4 * 512) {
        ncb = 4;
    } else if (div2 && blocks >= 2 * 384) {
        ncb = 2;
    }
    if (const char* e = std::getenv("LOWBIT_SKINNY_NCB")) {
        const int v = std::atoi(e);
        if ((v == 1) || (v == 2 && div2) || (v == 4 && div4)) ncb = v;
    }
    return ncb;
}

}  // namespace

bool skinny_supported(int g, int bits) {
    return (bits == 1 || bits == 2) && (g == 32 || g == 64 || g == 128);
}

bool use_skinny(int64_t M, int64_t N, int64_t K, int g, int bits) {
    (void)N;
    const int64_t step = 512 / bits;  // codes in 64 bytes of a packed row
    return M <= (bits == 2 ? 32 : 16) && skinny_supported(g, bits) && K % step == 0;
}

hipError_t launch_gemm_skinny_group(const GemmProblem* probs, int count, int g, int bits, hipStream_t stream) {
    int max_m = 0;
    for (int i = 0; i < count; ++i) max_m = probs[i].M > max_m ? probs[i].M : max_m;
    const int ncb = pick_ncb(probs, count);
    if (bits == 2) {
        switch (g) {
            case 32: return launch_bits_g<2, 32>(probs, count, max_m, ncb, stream);
            case 64: return launch_bits_g<2, 64>(probs, count, max_m, ncb, stream);
            default: return launch_bits_g<2, 128>(probs, count, max_m, ncb, stream);
        }
    }
    switch (g) {
        case 32: return launch_bits_g<1, 32>(probs, count, max_m, ncb, stream);
        case 64: return launch_bits_g<1, 64>(probs, count, max_m, ncb, stream);
        default: return launch_bits_g<1, 128>(probs, count, max_m, ncb, stream);
    }
}

hipError_t launch_gemm_skinny(const GemmProblem& p, int g, int bits, hipStream_t stream) {
    if (!use_skinny(p.M, p.N, p.K, g, bits)) return launch_gemm_tiled(p, g, bits, TILE_64x256, stream);
    return launch_gemm_skinny_group(&p, 1, g, bits, stream);
}

}  // namespace lowbit

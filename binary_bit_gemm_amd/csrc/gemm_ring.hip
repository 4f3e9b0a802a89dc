// Skinny-M ternary GEMM (M <= 16) with a deep load ring and optional split-K across
// workgroups: Y[M,N] = X[M,K] . dequant(W)[N,K]^T.
//
// At M = 16 every code is expanded once and the kernel streams the packed weights from HBM;
// what it needs is many bytes in flight (8 TB/s times a microsecond or two of latency) at
// every compute unit.  The four waves of a workgroup own disjoint column blocks and walk the
// same K steps, so one activation slice per step serves all four:
//   * a ring of D = 4 step stages in LDS holds the activations (16 rows x 256 K, shared),
//     each wave's packed weights (16 rows x 64 bytes per column block) and its scales; all
//     of it arrives by direct-to-LDS copies, three steps ahead of the compute;
//   * one barrier per step: it publishes the step's stage and frees the stage that the
//     previous step used, which the copies issued next overwrite;
//   * packed words are read back with ds_read_b32 in the layout of the 16x16x32 MFMA (lane
//     quarter q takes word q of a chunk), so no lane shuffles are needed.
// The K order inside a step and the scale handling are those of the other kernels: each MFMA
// takes eight consecutive codes of one word per lane quarter, all within one 64-code chunk,
// and the chunk's group scale (g = 64: one group per chunk; g = 128: one group per two
// chunks) multiplies the MFMA's partial sum in fp32 (w = scale_g * b, model card "Binary
// Weight Representation: 1-bit g128").
//
// Split-K: with `splits` > 1 the steps are divided among `splits` workgroups per column
// tile.  Each writes its fp32 partial sums to the workspace, then counts itself in on the
// tile's counter; the workgroup that arrives last adds the partials in split order 0, 1, ...
// (so the result does not depend on which one is last), writes Y and resets the counter.
#include "lowbit_device.h"
#include "lowbit_internal.h"

namespace lowbit {
namespace {

constexpr int kWaves = 4;
constexpr int kD = 4;                        // ring stages
constexpr int kStep = 256;                   // ternary codes per step (64 bytes of a row)
constexpr int kXRow = kStep * 2;             // activation bytes of one row per step
constexpr int kXStage = 16 * kXRow;          // 8 KB: 16 rows
constexpr int kXCopiesPerWave = kXStage / 1024 / kWaves;  // 16-byte copies of 64 lanes

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    // s_waitcnt encoding: vmcnt in bits [3:0] and [15:14], expcnt 7, lgkmcnt 15
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS that keeps the prefetch in flight.  __syncthreads() releases at
// workgroup scope, which on gfx9 waits for every outstanding vector-memory operation --
// including the copies of the three steps ahead.  The ring needs less: each wave has waited
// for its own copies of the step (counted waits), and every LDS read of the previous step
// was consumed before the barrier.  The empty asm statements keep the compiler from moving
// memory operations across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// 4-byte direct-to-LDS copy: lane i's 4 bytes land at lds_wave_base + 4 * i.
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t rs, void* lds_wave_base, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_wave_base, 4, voff, 0,
                                            0, 0);
}

template <int G, int NW>
struct RingCfg {
    static constexpr int GPS = kStep / G;                  // scale groups per step (4 or 2)
    static constexpr int SB = GPS * 2;                     // scale bytes of one row per step
    static constexpr int SDW = SB / 4;                     // ... in dwords
    static constexpr int W_WAVE = NW * 1024;               // packed bytes per wave and stage
    static constexpr int S_WAVE = 256;                     // one 4-byte copy of 64 lanes
    static constexpr int PER_STAGE = kXCopiesPerWave + NW + 1;  // copies per wave and stage
    static_assert(NW * 16 * SDW <= 64, "a wave's scales fit one copy");
};

template <int G, int NW>
__global__ __launch_bounds__(64 * kWaves, 2) void gemm_ring_kernel(RingArgs a) {
    using C = RingCfg<G, NW>;
    __shared__ __attribute__((aligned(16))) unsigned char x0[kXStage], x1[kXStage], x2[kXStage], x3[kXStage];
    __shared__ __attribute__((aligned(16))) unsigned char w0[kWaves * C::W_WAVE], w1[kWaves * C::W_WAVE],
        w2[kWaves * C::W_WAVE], w3[kWaves * C::W_WAVE];
    __shared__ __attribute__((aligned(16))) unsigned char s0[kWaves * C::S_WAVE], s1[kWaves * C::S_WAVE],
        s2[kWaves * C::S_WAVE], s3[kWaves * C::S_WAVE];
    __shared__ int last_flag;

    const GemmProblem& p = a.p;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
    const int q = lane >> 4, l16 = lane & 15;
    const int M = p.M, N = p.N, K = p.K;
    const int splits = a.splits;
    const int tile = int(blockIdx.x) / splits, split = int(blockIdx.x) % splits;

    const int n_wave = tile * (kWaves * NW * 16) + wave * (NW * 16);  // first column of this wave
    const uint32_t row_bytes = uint32_t(K) / 4u;
    const uint32_t s_row_bytes = uint32_t(K / G) * 2u;
    const int steps = K / kStep;
    const int s_begin = split * steps / splits, s_end = (split + 1) * steps / splits;
    const int len = s_end - s_begin;

    // ---- per-lane copy offsets (relative to the step's first byte) ----
    // activations: copy i of this wave brings rows 4 * wave + 2i + (lane >> 5); lane stores
    // chunk position lane & 31, which holds source chunk position ^ (row & 15)
    uint32_t x_voff[kXCopiesPerWave];
#pragma unroll
    for (int i = 0; i < kXCopiesPerWave; ++i) {
        const int r = 4 * wave + 2 * i + (lane >> 5), pos = lane & 31;
        x_voff[i] = uint32_t(r) * uint32_t(K) * 2u + uint32_t(pos ^ (r & 15)) * 16u;
    }
    // packed words: column block cb, lane -> row l16, chunk q (16 bytes)
    const unsigned char* w_base = reinterpret_cast<const unsigned char*>(p.W) + size_t(n_wave) * row_bytes;
    const uint32_t w_bytes = uint32_t(NW * 16) * row_bytes;
    uint32_t w_voff[NW];
#pragma unroll
    for (int cb = 0; cb < NW; ++cb) w_voff[cb] = uint32_t(cb * 16 + l16) * row_bytes + uint32_t(q) * 16u;
    // scales: lane -> row lane / SDW of the wave's NW * 16 rows, dword lane % SDW; lanes past
    // the rows read past the resource (zero)
    const unsigned char* s_base = reinterpret_cast<const unsigned char*>(p.S) + size_t(n_wave) * s_row_bytes;
    const uint32_t s_bytes = uint32_t(NW * 16) * s_row_bytes;
    const uint32_t s_voff = lane < NW * 16 * C::SDW
                                ? uint32_t(lane / C::SDW) * s_row_bytes + uint32_t(lane % C::SDW) * 4u
                                : 0xFFFFFF00u;
    const unsigned char* x_base = reinterpret_cast<const unsigned char*>(p.X);
    const uint32_t x_bytes = uint32_t(M) * uint32_t(K) * 2u;

    // ---- per-lane read offsets ----
    int x_rd[8];  // operand (c, j) of lane (q, m = l16): logical chunk 8c + 2q + j of row m
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int j = 0; j < 2; ++j) x_rd[c * 2 + j] = l16 * kXRow + (((8 * c + 2 * q + j) ^ l16) << 4);
    const int w_rd = wave * C::W_WAVE + l16 * 16 + q * 4;  // + cb * 1024 + c * 256
    const int s_rd = wave * C::S_WAVE + l16 * C::SB;       // + cb * 16 * SB

    // Copies of one step into one stage.  Steps past the range go through empty resources:
    // every stage then issues the same number of copies, which the waits below count on.
    auto issue = [&](int t, unsigned char* xs, unsigned char* ws, unsigned char* ss) {
        const int s = s_begin + t;
        const bool live = t < len;
        const uint32_t xk = uint32_t(live ? s : 0) * kXRow;
        const __amdgpu_buffer_rsrc_t xr = make_rsrc(x_base + xk, live ? x_bytes - xk : 0u);
#pragma unroll
        for (int i = 0; i < kXCopiesPerWave; ++i) dma16(xr, xs + (wave * kXCopiesPerWave + i) * 1024, x_voff[i], 0);
        const uint32_t wk = uint32_t(live ? s : 0) * 64u;
        const __amdgpu_buffer_rsrc_t wr = make_rsrc(w_base + wk, live ? w_bytes - wk : 0u);
#pragma unroll
        for (int cb = 0; cb < NW; ++cb) dma16(wr, ws + wave * C::W_WAVE + cb * 1024, w_voff[cb], 0);
        const uint32_t sk = uint32_t(live ? s : 0) * uint32_t(C::SB);
        const __amdgpu_buffer_rsrc_t sr = make_rsrc(s_base + sk, live ? s_bytes - sk : 0u);
        dma4(sr, ss + wave * C::S_WAVE, s_voff);
    };

    f32x4_t acc[NW];
#pragma unroll
    for (int cb = 0; cb < NW; ++cb) acc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const unsigned char* xs, const unsigned char* ws, const unsigned char* ss) {
        float sc[NW][C::GPS];
        uint32_t wd[NW][4];
#pragma unroll
        for (int cb = 0; cb < NW; ++cb) {
#pragma unroll
            for (int c = 0; c < 4; ++c) wd[cb][c] = *reinterpret_cast<const uint32_t*>(ws + w_rd + cb * 1024 + c * 256);
#pragma unroll
            for (int gi = 0; gi < C::GPS; ++gi)
                sc[cb][gi] = half_bits_to_float(*reinterpret_cast<const uint16_t*>(ss + s_rd + cb * 16 * C::SB + 2 * gi)) *
                             0.5f;  // the operand holds 2c
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            bf16x8_t xa[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) xa[j] = *reinterpret_cast<const bf16x8_t*>(xs + x_rd[c * 2 + j]);
#pragma unroll
            for (int cb = 0; cb < NW; ++cb) {
                uint32_t d[8];
                expand_ternary_word(wd[cb][c], d);
                f32x4_t t = {0.f, 0.f, 0.f, 0.f};
                t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[0], __builtin_bit_cast(bf16x8_t, u32x4_t{d[0], d[1], d[2], d[3]}),
                                                            t, 0, 0, 0);
                t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[1], __builtin_bit_cast(bf16x8_t, u32x4_t{d[4], d[5], d[6], d[7]}),
                                                            t, 0, 0, 0);
                const float s = sc[cb][c * C::GPS / 4];
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[cb][i] = __builtin_fmaf(s, t[i], acc[cb][i]);
            }
        }
    };

    // One step: wait for this wave's copies of the stage, publish the stage to the workgroup
    // (and learn that every wave is done with the previous stage), refill that previous stage
    // three steps ahead, compute.
    auto step = [&](int t, unsigned char* xs, unsigned char* ws, unsigned char* ss, unsigned char* xn,
                    unsigned char* wn, unsigned char* sn) {
        wait_vmcnt<(kD - 2) * C::PER_STAGE>();
        lds_barrier();
        issue(t + kD - 1, xn, wn, sn);
        compute(xs, ws, ss);
    };

    issue(0, x0, w0, s0);
    issue(1, x1, w1, s1);
    issue(2, x2, w2, s2);
    int t = 0;
#pragma nounroll
    for (; t + 4 <= len; t += 4) {
        step(t, x0, w0, s0, x3, w3, s3);
        step(t + 1, x1, w1, s1, x0, w0, s0);
        step(t + 2, x2, w2, s2, x1, w1, s1);
        step(t + 3, x3, w3, s3, x2, w2, s2);
    }
    if (t < len) step(t, x0, w0, s0, x3, w3, s3);
    if (t + 1 < len) step(t + 1, x1, w1, s1, x0, w0, s0);
    if (t + 2 < len) step(t + 2, x2, w2, s2, x1, w1, s1);
    wait_vmcnt<0>();

    // ---- epilogue: lane (q, n) holds rows 4q + i of column n of each of its blocks ----
    if (splits == 1) {
#pragma unroll
        for (int cb = 0; cb < NW; ++cb) {
            const int col = n_wave + cb * 16 + l16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * q + i;
                if (m < M) p.Y[int64_t(m) * N + col] = float_to_bf16_bits(acc[cb][i]);
            }
        }
        return;
    }
    // Partial sums: ws[((tile * splits + split) * kWaves + wave) * NW + cb][lane][4] fp32.
    // They travel as agent-scope relaxed atomics, which go through to the device-coherent
    // level (the L2 of one XCD is not coherent with the others); a release / acquire fence
    // instead writes back and invalidates the whole L2 of the XCD for every workgroup.
    // Order: this workgroup's stores complete (counted wait) before its arrival is counted;
    // the last workgroup's loads start after it has seen every arrival.
    float* part = a.ws;
    const size_t tile_base = size_t(tile) * splits * kWaves * NW * 64;
#pragma unroll
    for (int cb = 0; cb < NW; ++cb) {
        float* dst = part + (tile_base + (size_t(split) * kWaves * NW + wave * NW + cb) * 64 + lane) * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) __hip_atomic_store(dst + i, acc[cb][i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    wait_vmcnt<0>();
    __syncthreads();
    if (threadIdx.x == 0)
        last_flag = __hip_atomic_fetch_add(&a.counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                    uint32_t(splits - 1);
    __syncthreads();
    if (!last_flag) return;
#pragma unroll
    for (int cb = 0; cb < NW; ++cb) {
        // Loads of four splits are issued before any of them is added (each is a memory round
        // trip); the additions stay in split order.
        f32x4_t v = {0.f, 0.f, 0.f, 0.f};
        const float* src = part + (tile_base + size_t(wave * NW + cb) * 64 + lane) * 4;
        const size_t split_stride = size_t(kWaves) * NW * 64 * 4;
        for (int s = 0; s < splits; s += 4) {
            float u[4][4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    u[j][i] = s + j < splits ? __hip_atomic_load(src + (s + j) * split_stride + i, __ATOMIC_RELAXED,
                                                                 __HIP_MEMORY_SCOPE_AGENT)
                                             : 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (s + j < splits) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] += u[j][i];
                }
        }
        const int col = n_wave + cb * 16 + l16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * q + i;
            if (m < M) p.Y[int64_t(m) * N + col] = float_to_bf16_bits(v[i]);
        }
    }
    if (threadIdx.x == 0) __hip_atomic_store(&a.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int G, int NW>
hipError_t launch_ring_cfg(const RingArgs& a, hipStream_t stream) {
    const int tiles = a.p.N / (kWaves * NW * 16);
    hipLaunchKernelGGL((gemm_ring_kernel<G, NW>), dim3(tiles * a.splits), dim3(64 * kWaves), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

bool ring_supported(int64_t M, int64_t N, int64_t K, int g, int bits) {
    return bits == 2 && (g == 64 || g == 128) && M >= 1 && M <= 16 && K % kStep == 0 && N % (kWaves * 16) == 0;
}

RingPlan plan_ring(int64_t N, int64_t K, int max_splits) {
    // Widest column tiles first; the fewest splits that give ~384+ workgroups with at least
    // three steps each (the ring is three steps deep).
    const int steps = int(K / kStep);
    RingPlan best{0, 0, 0};
    for (int nw = 2; nw >= 1; --nw) {
        if (N % (kWaves * nw * 16) != 0) continue;
        const int tiles = int(N / (kWaves * nw * 16));
        for (int s = 1; s <= max_splits && s <= steps; ++s) {
            if (s > 1 && steps / s < 3) break;
            const int wgs = tiles * s;
            if (wgs > best.tiles * best.splits) best = RingPlan{nw, s, tiles};
            if (wgs >= 384) return RingPlan{nw, s, tiles};
        }
    }
    return best;
}

size_t ring_workspace_bytes(const RingPlan& plan, int64_t N) {
    if (plan.splits <= 1) return 0;
    const size_t counters = (size_t(plan.tiles) * 4 + 255) / 256 * 256;
    return counters + size_t(plan.splits) * size_t(N) * 16 * 4;  // fp32 partials of 16 rows
}

hipError_t launch_gemm_ring(const GemmProblem& p, int g, const RingPlan& plan, void* workspace, hipStream_t stream) {
    RingArgs a{};
    a.p = p;
    a.splits = plan.splits;
    if (plan.splits > 1) {
        const size_t counters = (size_t(plan.tiles) * 4 + 255) / 256 * 256;
        a.counters = static_cast<uint32_t*>(workspace);
        a.ws = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + counters);
    }
    if (g == 64) return plan.nw == 2 ? launch_ring_cfg<64, 2>(a, stream) : launch_ring_cfg<64, 1>(a, stream);
    return plan.nw == 2 ? launch_ring_cfg<128, 2>(a, stream) : launch_ring_cfg<128, 1>(a, stream);
}

}  // namespace lowbit

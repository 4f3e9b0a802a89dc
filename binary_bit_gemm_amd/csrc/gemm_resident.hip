// Skinny-M ternary GEMM with the activations resident in LDS: Y[M,N] = X[M,K] . dequant(W)[N,K]^T
// for M <= 16, scale groups of 64 or 128 and K % 256 == 0, optionally split along K across
// workgroups through a caller-provided workspace.
//
// At M = 16 each packed weight byte meets only 16 activation rows, so the kernel streams the
// weights from HBM and what decides its speed is how many weight bytes every compute unit
// keeps in flight while it expands and multiplies.  The design gives that to the weights:
//   * a workgroup owns CB column blocks of 16 weight rows and one contiguous range of the K
//     steps (a step = 256 codes = 64 bytes of a row): the whole of K, or one of `splits`
//     ranges.  It first copies the activations of its K range (16 rows, rows at or past M
//     read as zero) and the scales of its rows and range into LDS, once;
//   * its waves own (column block, K slice) pairs: the CB blocks times KS contiguous slices
//     of the range;
//   * every wave loads the packed words of its steps (16 bytes per lane and step; at most 12
//     steps) straight into registers, two steps ahead of their use, and consumes them in
//     order.  No LDS write sits between these loads and the compute;
//   * the KS partial sums of a column block are added in LDS in slice order 0, 1, ...; with
//     splits > 1 the workgroup then stores its fp32 partial sums in the workspace and counts
//     itself in on its column group's counter; the workgroup that arrives last adds the
//     partials in split order 0, 1, ... (fixed order: the result does not depend on timing),
//     writes Y and resets the counter.
// The code expansion, the K order inside a step and the scale handling are those of the
// other 16x16x32 kernels: after a 4x4 lane-quarter transpose, register c of lane quarter q
// holds word q of the row's 16-byte piece c; each MFMA takes eight consecutive codes of that
// word, all inside one 64-code piece, and the piece's group scale multiplies the MFMA's
// partial sum in fp32 (w = scale_g * b, model card "Binary Weight Representation: 1-bit
// g128").  The operand holds 2c; the factor 1/2 is applied once to the final sum.
#include <atomic>
#include <cstdio>
#include <cstdlib>

#include "lowbit_device.h"
#include "lowbit_internal.h"

namespace lowbit {
namespace {

constexpr int kStepCodes = 256;   // ternary codes of one row per step (64 bytes)
constexpr int kMaxWaves = 16;
constexpr int kMaxLen = 12;       // steps per wave (4 registers each)
constexpr int kMaxLds = 160 * 1024;
constexpr int kTargetWorkgroups = 256;  // whole-K plans: one per compute unit
// Split plans: small workgroups (4..16 waves, little LDS), several per compute unit.  Measured
// on the M = 16 K-heavy shapes: 4..8 column blocks and 384..768 workgroups beat 12..16
// blocks and 256 workgroups by 15 - 20%.
constexpr int kSplitWorkgroups = 512;
// A split launch's workspace starts with a region of arrival counters of one fixed size,
// whatever the shape, and its fp32 partial sums follow it.  Launches of different shapes that
// share a workspace then find their counters at the same place: a counter region that grew
// with the tile count would let one launch read another's left-over partial sums as counters.
// Split plans have at most kSplitWorkgroups / 2 tiles (two splits or more each); forced plans
// with more tiles than counters are refused.
constexpr int kMaxCounterTiles = 1024;
constexpr size_t kCounterBytes = size_t(kMaxCounterTiles) * 4u;

// LDS layout of a workgroup whose K range has `tw` steps: activation row r at r * x_row,
// x_row = 512 * tw + 16 (the pad puts the same 16-byte chunk of the 16 rows into 16
// different bank groups, and keeps every operand address a lane base plus a constant); the
// scales of the CB * 16 weight rows for the range follow at the next 1 KB boundary (row-
// major, tw * groups-per-step fp16 each); then one int.
__host__ __device__ constexpr uint32_t x_row_bytes(int tw) { return 512u * uint32_t(tw) + 16u; }
__host__ __device__ constexpr uint32_t x_region_bytes(int tw) { return (16u * x_row_bytes(tw) + 1023u) & ~1023u; }
__host__ __device__ constexpr uint32_t s_row_lds(int tw, int g) { return uint32_t(tw) * uint32_t(kStepCodes / g) * 2u; }
__host__ __device__ constexpr uint32_t s_region_bytes(int tw, int g, int cb) {
    return (uint32_t(cb) * 16u * s_row_lds(tw, g) + 1023u) & ~1023u;
}
__host__ __device__ constexpr uint32_t lds_bytes(int tw, int g, int cb) {
    return x_region_bytes(tw) + s_region_bytes(tw, g, cb) + 16u;
}

struct ResidentArgs {
    ProblemGroup grp;     // tiles: groups of CB column blocks (tile_end counts them)
    int cb;               // column blocks per workgroup
    int ks;               // K slices per column block inside a workgroup
    int splits;           // workgroups per tile along K
    int tiles;            // tiles of the launch
    float* ws;            // [tiles][splits][cb][64][4] fp32 partial sums (splits > 1)
    uint32_t* counters;   // [tiles] arrival counters, zero between calls (splits > 1)
};

// 4-byte direct-to-LDS copy: lane i's 4 bytes land at lds_wave_base + 4 * i.
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t rs, void* lds_wave_base, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_wave_base, 4, voff, 0,
                                            0, 0);
}

// EPI = kEpiSwiglu: the problem's W and S hold 2N rows (gate rows [0, N), up rows [N, 2N)) and
// Y[M, N] = silu(X . Wgate^T) * (X . Wup^T).  A workgroup's CB (even) column blocks are then CB / 2
// gate blocks and the up blocks of the same output columns; after the K-slice reduction the up
// sums reach the gate blocks' waves through LDS.  EPI = kEpiResidual: Y = R + gate[n] * (X . W^T)
// (Y may be R: each element is read and written by the same lane).  Both: whole K only (one split).
template <int G, int LEN, int EPI = kEpiPlain>
__global__ __launch_bounds__(64 * kMaxWaves, 1) void gemm_resident_kernel(ResidentArgs a) {
    constexpr bool SWIGLU = EPI == kEpiSwiglu;
    constexpr int GPS = kStepCodes / G;  // scale groups per step: 4 or 2
    extern __shared__ __attribute__((aligned(1024))) unsigned char lds[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
    const int nwaves = int(blockDim.x >> 6);
    const int q = lane >> 4, n = lane & 15;
    const int split = int(blockIdx.x) / a.tiles;
    const int tile = int(blockIdx.x) - split * a.tiles;
    int pi = 0;
    while (pi + 1 < a.grp.count && tile >= a.grp.tile_end[pi]) ++pi;
    const GemmProblem p = a.grp.p[pi];
    const int group = tile - (pi > 0 ? a.grp.tile_end[pi - 1] : 0);
    const int M = p.M, N = p.N, K = p.K;
    const int CB = a.cb, KS = a.ks, S = a.splits;
    const int cbi = wave % CB, ks = wave / CB;
    // global weight block of local block c (SwiGLU: gate block j or up block N/16 + j of output
    // block j = group * CB/2 + c % (CB/2)), and whether it holds output columns
    const int HB = CB / 2;
    auto out_block = [&](int c) { return SWIGLU ? group * HB + c % HB : group * CB + c; };
    auto w_block = [&](int c) { return SWIGLU && c >= HB ? N / 16 + out_block(c) : out_block(c); };
    const int cb = w_block(cbi);
    const bool active = out_block(cbi) < N / 16;  // wave-uniform
    const int w_rows = SWIGLU ? 2 * N : N;
    const int T = K / kStepCodes;
    const int kb = split * T / S, tw = (split + 1) * T / S - kb;  // the workgroup's K range
    const int t_begin = ks * tw / KS;                             // relative to kb
    const int len = (ks + 1) * tw / KS - t_begin;                 // <= LEN (host)

    // ---- activations and scales of the range into LDS (direct-to-LDS copies).  Activation
    // slot (row r, position pos) holds 16-byte chunk pos of the range of row r; the pad slot
    // at the end of a row gets chunk 0 again.  Workgroups start at different copies so that
    // they do not all ask the same L2 channel for the same line at once.
    const uint32_t xrow = x_row_bytes(tw);
    const int row_slots = 32 * tw + 1;
    const int x_copies = (16 * row_slots + 63) / 64;
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.X, uint32_t(M) * uint32_t(K) * 2u);
    const uint32_t x_src = uint32_t(kb) * 512u;
    const int rot = int(blockIdx.x) % x_copies;
    for (int jj = wave; jj < x_copies; jj += nwaves) {
        const int j = jj + rot < x_copies ? jj + rot : jj + rot - x_copies;
        const int slot = 64 * j + lane;
        const int r = slot / row_slots, pos = slot - r * row_slots;
        const int chunk = pos < 32 * tw ? pos : 0;
        dma16(xr, lds + 1024 * j, uint32_t(r) * uint32_t(K) * 2u + x_src + uint32_t(chunk) * 16u, 0);
    }
    // scales: dword d of the region = dword d % dpr of row d / dpr's range
    const uint32_t s_row = uint32_t(K / G) * 2u;
    const uint32_t s_base = x_region_bytes(tw);
    const int dpr = int(s_row_lds(tw, G) / 4u);
    const int s_copies = (CB * 16 * dpr + 63) / 64;
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(p.S, uint32_t(w_rows) * s_row);
    const uint32_t s_src = uint32_t(group * CB * 16) * s_row + uint32_t(kb * GPS) * 2u;
    if (SWIGLU) {
        // row r of the region is row r % 16 of weight block w_block(r / 16); rows of blocks past
        // the output read past the end of S (zeros, never used)
        for (int j = wave; j < s_copies; j += nwaves) {
            const int d = 64 * j + lane;
            const int r = d / dpr, k = d - r * dpr;
            const uint32_t src = r < CB * 16 && out_block(r / 16) < N / 16
                                     ? uint32_t(w_block(r / 16) * 16 + (r & 15)) * s_row + uint32_t(kb * GPS) * 2u +
                                           uint32_t(k) * 4u
                                     : uint32_t(w_rows) * s_row;
            dma4(sr, lds + s_base + 256 * j, src);
        }
    } else if (tw == T) {
        // whole K: the workgroup's rows of scales are one contiguous block of CB * 16 * s_row
        // bytes (a multiple of 16, at a multiple of 16); 16-byte copies, a quarter of the
        // instructions of the row-by-row 4-byte copies below (the region is rounded up to
        // 1 KB, so the last copy fits; past the buffer's end it reads zeros)
        const int s16 = (CB * 16 * int(s_row) + 1023) / 1024;
        for (int j = wave; j < s16; j += nwaves) dma16(sr, lds + s_base + 1024 * j, s_src + 1024u * uint32_t(j) + 16u * uint32_t(lane), 0);
    } else {
        for (int j = wave; j < s_copies; j += nwaves) {
            const int d = 64 * j + lane;
            const int r = d / dpr, k = d - r * dpr;
            dma4(sr, lds + s_base + 256 * j, s_src + uint32_t(r) * s_row + uint32_t(k) * 4u);
        }
    }
    // the counted wait below relies on these copies preceding the weight loads
    asm volatile("" ::: "memory");

    // ---- packed words of all the wave's steps (steps past its slice, and waves past the
    // last column block, read through an empty resource: no memory traffic) ----
    const uint32_t w_row = uint32_t(K) / 4u;
    const uint32_t row = uint32_t(cb * 16 + n);
    const __amdgpu_buffer_rsrc_t w_rs = make_rsrc(p.W, active ? uint32_t(w_rows) * w_row : 0u);
    const __amdgpu_buffer_rsrc_t none = make_rsrc(p.W, 0u);
#ifndef LOWBIT_RESIDENT_AHEAD
#define LOWBIT_RESIDENT_AHEAD 2
#endif
    // The first AHEAD steps' loads are issued before the barrier, every later one AHEAD steps
    // ahead of the step being computed.  Issuing them all up front stalls each wave at issue
    // until the weight stream has drained far enough, and so holds the barrier -- and all
    // compute -- back until nearly the whole matrix has arrived (measured: the M = 16 denoise
    // step ran 10% faster with AHEAD = 2 than with all loads up front; 1, 3, 4 and 6 lie
    // between).
    constexpr int AHEAD = LEN < LOWBIT_RESIDENT_AHEAD ? LEN : LOWBIT_RESIDENT_AHEAD;
    u32x4_t wv[LEN];
    auto load_w = [&](int i) {
        wv[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                i < len ? w_rs : none,
                                                row * w_row + uint32_t(kb + t_begin + i) * 64u + 16u * uint32_t(q), 0, 0));
    };
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) load_w(i);
    wait_vmcnt<AHEAD>();
    lds_barrier();

    // Operand (step t, piece c, half h) of lane (q, m): activation chunk 32t + 8c + 2q + h of
    // row m -- the codes 64c + 16q + 8h .. +8 of the step, which lane (q, n) holds in word q
    // of piece c after the transpose.
    const unsigned char* xl = lds + n * xrow + 32 * q + 512 * t_begin;
    const unsigned char* sl = lds + s_base + (cbi * 16 + n) * s_row_lds(tw, G) + uint32_t(t_begin * GPS) * 2u;
    auto xop = [&](int i, int c, int h) { return *reinterpret_cast<const bf16x8_t*>(xl + 512 * i + 128 * c + 16 * h); };

    // Piece p = 4 * step + c computes with operand buffer p & 1 while the next piece's
    // operands are read into the other buffer.
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    bf16x8_t xb[2][2];
    xb[0][0] = xop(0, 0, 0);
    xb[0][1] = xop(0, 0, 1);
#pragma unroll
    for (int i = 0; i < LEN; ++i) {
        if (i + AHEAD < LEN) {
            load_w(i + AHEAD);
            __builtin_amdgcn_sched_barrier(0);  // keep the load here, AHEAD steps ahead of its use
        }
        if (i < len) {
            uint32_t sw[2];
            if constexpr (GPS == 4) {
                const auto v = *reinterpret_cast<const uint32_t __attribute__((ext_vector_type(2)))*>(sl + 8 * i);
                sw[0] = v[0];
                sw[1] = v[1];
            } else {
                sw[0] = *reinterpret_cast<const uint32_t*>(sl + 4 * i);
                sw[1] = 0;
            }
            u32x4_t w = wv[i];
            transpose_words(w);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int b = c & 1;  // (4 * i + c) & 1
                if (c < 3 || i + 1 < len) {
                    const int ni = c == 3 ? i + 1 : i, nc = c == 3 ? 0 : c + 1;
                    xb[b ^ 1][0] = xop(ni, nc, 0);
                    xb[b ^ 1][1] = xop(ni, nc, 1);
                }
                uint32_t d[8];
                expand_ternary_word(w[c], d);
                const int gi = c * GPS / 4;  // scale group of piece c within the step
                const uint32_t s2 = sw[gi >> 1];
                const float sc = half_bits_to_float(uint16_t((gi & 1) ? (s2 >> 16) : (s2 & 0xFFFFu)));
                f32x4_t t = {0.f, 0.f, 0.f, 0.f};
                t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    xb[b][0], __builtin_bit_cast(bf16x8_t, u32x4_t{d[0], d[1], d[2], d[3]}), t, 0, 0, 0);
                t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    xb[b][1], __builtin_bit_cast(bf16x8_t, u32x4_t{d[4], d[5], d[6], d[7]}), t, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(sc, t[e], acc[e]);
            }
        }
    }

    // ---- fixed-order reduction over the K slices of the workgroup ----
    // 16x16 MFMA result layout: lane l holds column l % 16, rows 4 * (l / 16) + e.
    if (KS > 1) {
        __syncthreads();  // every LDS read is done: the reduction reuses the LDS
        f32x4_t* red = reinterpret_cast<f32x4_t*>(lds);
        red[wave * 64 + lane] = acc;
        __syncthreads();
        if (ks == 0) {
            for (int k = 1; k < KS; ++k) {
                const f32x4_t u = red[(cbi + CB * k) * 64 + lane];
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] += u[e];
            }
        }
    }
    if constexpr (SWIGLU) {
        // up sums (blocks HB .. CB-1, slice 0) to the gate blocks' waves; silu(g) * u from the
        // fp32 sums (the operand holds 2c: both halved), rounded to bf16 once
        __syncthreads();  // the reduction's reads of the LDS are done
        f32x4_t* xch = reinterpret_cast<f32x4_t*>(lds);
        if (ks == 0 && cbi >= HB) xch[(cbi - HB) * 64 + lane] = acc;
        __syncthreads();
        if (ks == 0 && cbi < HB && active) {
            const f32x4_t u = xch[cbi * 64 + lane];
            const int col = out_block(cbi) * 16 + n;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = 4 * q + e;
                const float gt = 0.5f * acc[e];
                if (m < M) p.Y[int64_t(m) * N + col] = float_to_bf16_bits(gt * (0.5f * u[e]) / (1.0f + __expf(-gt)));
            }
        }
        return;
    }
    const int col = cb * 16 + n;
    if (S == 1) {
        if (ks == 0 && active) {
            const float gt = EPI == kEpiResidual ? static_cast<float>(__builtin_bit_cast(__bf16, p.gate[col])) : 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = 4 * q + e;
                if (m < M) {
                    float v = 0.5f * acc[e];  // operand holds 2c
                    if constexpr (EPI == kEpiResidual)
                        v = __builtin_fmaf(gt, v, static_cast<float>(__builtin_bit_cast(__bf16, p.R[int64_t(m) * N + col])));
                    p.Y[int64_t(m) * N + col] = float_to_bf16_bits(v);
                }
            }
        }
        return;
    }

    // ---- split K: partial sums through the workspace, the last workgroup adds them ----
    // They travel as 16-byte loads and stores with the sc1 cache policy (what agent-scope
    // relaxed atomics compile to here): through to the device-coherent level, since the L2
    // of one XCD is not coherent with the others.  A release / acquire fence instead writes
    // back and invalidates the whole L2 of the XCD for every workgroup.  Order: this
    // workgroup's stores complete (counted wait) before its arrival is counted; the last
    // workgroup's loads start after it has seen every arrival.
    constexpr int kSc1 = 16;  // cache policy bit sc1 of buffer loads and stores
    const uint32_t part_bytes = uint32_t(a.tiles) * uint32_t(S) * uint32_t(CB) * 1024u;
    const __amdgpu_buffer_rsrc_t ws_rs = make_rsrc(a.ws, part_bytes);
    const uint32_t tile_part = uint32_t(tile) * uint32_t(S) * uint32_t(CB) * 1024u;  // bytes
    if (ks == 0)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, acc), ws_rs,
                                               tile_part + (uint32_t(split * CB + cbi) * 64u + uint32_t(lane)) * 16u,
                                               0, kSc1);
    wait_vmcnt<0>();
    __syncthreads();
    int* last_flag = reinterpret_cast<int*>(lds + s_base + s_region_bytes(tw, G, CB));
    if (threadIdx.x == 0)
        *last_flag = __hip_atomic_fetch_add(&a.counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                     uint32_t(S - 1);
    __syncthreads();
    if (!*last_flag) return;
    if (ks == 0 && active) {
        // the loads of up to 16 splits are issued before any of them is added; the additions
        // stay in split order
        const uint32_t src = tile_part + (uint32_t(cbi) * 64u + uint32_t(lane)) * 16u;
        const uint32_t stride = uint32_t(CB) * 1024u;
        f32x4_t v = {0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0; s0 < S; s0 += 16) {
            u32x4_t u[16];
#pragma unroll
            for (int j = 0; j < 16; ++j)
                u[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                       s0 + j < S ? ws_rs : make_rsrc(a.ws, 0u),
                                                       src + uint32_t(s0 + j) * stride, 0, kSc1));
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (s0 + j < S) {
                    const f32x4_t f = __builtin_bit_cast(f32x4_t, u[j]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] += f[e];
                }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = 4 * q + e;
            if (m < M) p.Y[int64_t(m) * N + col] = float_to_bf16_bits(0.5f * v[e]);
        }
    }
    if (threadIdx.x == 0) __hip_atomic_store(&a.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int G, int LEN, int EPI = kEpiPlain>
hipError_t launch_cfg(const ResidentArgs& a, uint32_t lds, hipStream_t stream) {
    // allow the dynamic LDS of the largest plan, once per kernel and device (threads that get here
    // first at the same time may both set it; the value is the same)
    static std::atomic<int> attr_set[64];
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    if (attr_set[dev].load(std::memory_order_acquire) == 0) {
        err = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_resident_kernel<G, LEN, EPI>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
        if (err != hipSuccess) return err;
        attr_set[dev].store(1, std::memory_order_release);
    }
    hipLaunchKernelGGL((gemm_resident_kernel<G, LEN, EPI>), dim3(a.tiles * a.splits), dim3(64 * a.cb * a.ks), lds,
                       stream, a);
    const hipError_t e = hipGetLastError();
    if (e == hipSuccess && trace_enabled()) {
        char cfg[96];
        snprintf(cfg, sizeof cfg, "column_blocks=%d k_slices=%d steps=%d splits=%d tiles=%d epi=%s", a.cb, a.ks, LEN,
                 a.splits, a.tiles, EPI == kEpiSwiglu ? "swiglu" : EPI == kEpiResidual ? "residual" : "plain");
        trace_launch("resident", cfg, G, 2, a.grp.p, a.grp.count, unsigned(a.tiles * a.splits), 64u * a.cb * a.ks, lds);
    }
    return e;
}

template <int G, int EPI = kEpiPlain>
hipError_t launch_g(const ResidentArgs& a, uint32_t lds, int len, hipStream_t stream) {
    switch (len) {
        case 1: return launch_cfg<G, 1, EPI>(a, lds, stream);
        case 2: return launch_cfg<G, 2, EPI>(a, lds, stream);
        case 3: return launch_cfg<G, 3, EPI>(a, lds, stream);
        case 4: return launch_cfg<G, 4, EPI>(a, lds, stream);
        case 5: return launch_cfg<G, 5, EPI>(a, lds, stream);
        case 6: return launch_cfg<G, 6, EPI>(a, lds, stream);
        case 7: return launch_cfg<G, 7, EPI>(a, lds, stream);
        case 8: return launch_cfg<G, 8, EPI>(a, lds, stream);
        case 9: return launch_cfg<G, 9, EPI>(a, lds, stream);
        case 10: return launch_cfg<G, 10, EPI>(a, lds, stream);
        case 11: return launch_cfg<G, 11, EPI>(a, lds, stream);
        case 12: return launch_cfg<G, 12, EPI>(a, lds, stream);
        default: return hipErrorInvalidValue;
    }
}

int64_t column_blocks(const GemmProblem* probs, int count) {
    int64_t blocks = 0;
    for (int i = 0; i < count; ++i) blocks += probs[i].N / 16;
    return blocks;
}

int64_t tiles_of(const GemmProblem* probs, int count, int cb) {
    int64_t tiles = 0;
    for (int i = 0; i < count; ++i) tiles += (probs[i].N / 16 + cb - 1) / cb;
    return tiles;
}

// Whole-K plan: column blocks per workgroup enough that the blocks fill one round of
// workgroups over the compute units; K slices as many as the remaining waves allow.
ResidentPlan plan_whole(const GemmProblem* probs, int count, int g) {
    const int64_t blocks = column_blocks(probs, count);
    const int T = probs[0].K / kStepCodes;
    ResidentPlan pl{};
    pl.splits = 1;
    pl.cb = int((blocks + kTargetWorkgroups - 1) / kTargetWorkgroups);
    pl.cb = pl.cb < 1 ? 1 : (pl.cb > kMaxWaves ? kMaxWaves : pl.cb);
    pl.ks = kMaxWaves / pl.cb;
    pl.ks = pl.ks < T ? pl.ks : T;
    pl.len = (T + pl.ks - 1) / pl.ks;
    pl.tiles = int(tiles_of(probs, count, pl.cb));
    if (pl.len > kMaxLen || lds_bytes(T, g, pl.cb) > uint32_t(kMaxLds)) pl.len = 0;
    return pl;
}

// LOWBIT_RESIDENT_PLAN = "cb,splits" fixes the split plan (A/B runs); 0 when unset.
bool forced_split(int& cb, int& splits) {
    const char* v = std::getenv("LOWBIT_RESIDENT_PLAN");
    if (v == nullptr) return false;
    return std::sscanf(v, "%d,%d", &cb, &splits) == 2 && cb >= 1 && cb <= kMaxWaves && splits >= 2;
}

// Split-K plan: as many column blocks per workgroup as there are waves (one K slice each),
// and the splits that bring the workgroups closest to one round over the compute units.
ResidentPlan plan_split(const GemmProblem* probs, int count, int g) {
    const int64_t blocks = column_blocks(probs, count);
    const int T = probs[0].K / kStepCodes;
    int fcb = 0, fs = 0;
    if (forced_split(fcb, fs)) {
        fs = fs < T ? fs : T;
        const int len = (T + fs - 1) / fs;
        const int64_t tiles = tiles_of(probs, count, fcb);
        if (fs < 2 || len > kMaxLen || lds_bytes(len, g, fcb) > uint32_t(kMaxLds) || tiles > kMaxCounterTiles)
            return ResidentPlan{};
        return ResidentPlan{fcb, 1, len, fs, int(tiles)};
    }
    ResidentPlan best{};
    int64_t best_score = -1;
    for (int cb = 4; cb <= kMaxWaves; ++cb) {
        if (cb > blocks) break;
        const int64_t tiles = tiles_of(probs, count, cb);
        int s = int(kSplitWorkgroups / tiles);
        s = s < 1 ? 1 : (s > T ? T : s);
        const int len = (T + s - 1) / s;
        if (s < 2 || len > kMaxLen || lds_bytes(len, g, cb) > uint32_t(kMaxLds) || tiles > kMaxCounterTiles) continue;
        // prefer workgroups up to the target, then whole column blocks in every tile, then
        // even ranges, then (first found) fewer waves per workgroup
        const int64_t wgs = tiles * s;
        const int64_t score = (wgs < kSplitWorkgroups ? wgs : kSplitWorkgroups) * 4 + (blocks % cb == 0 ? 2 : 0) +
                              (T % s == 0 ? 1 : 0);
        if (score > best_score) {
            best_score = score;
            best = ResidentPlan{cb, 1, len, s, int(tiles)};
        }
    }
    return best;  // len 0: no split plan
}

}  // namespace

bool resident_supported(int64_t M, int64_t N, int64_t K, int g, int bits) {
    return bits == 2 && (g == 64 || g == 128) && M >= 1 && M <= 16 && N >= 16 && N % 16 == 0 &&
           K >= kStepCodes && K % kStepCodes == 0;
}

// With a workspace, problems whose K does not fit the whole-K plan (the activations of the
// whole K exceed the LDS, or a wave would need more than kMaxLen steps) are split along K;
// the rest run whole.  (Splitting problems that do fit, to give every compute unit a
// workgroup, measured no faster at M = 16.)
ResidentPlan plan_resident(const GemmProblem* probs, int count, int g, bool may_split) {
    const ResidentPlan whole = plan_whole(probs, count, g);
    if (!may_split) return whole;
    int fcb = 0, fs = 0;
    if (forced_split(fcb, fs)) {
        const ResidentPlan split = plan_split(probs, count, g);
        return split.len > 0 ? split : whole;
    }
    if (whole.len > 0) return whole;  // measured: splitting K only pays where the whole K does not fit
    return plan_split(probs, count, g);
}

// Where the planner uses the resident kernel: split plans (a workspace is there and the
// problems' column blocks do not fill the machine, or K is past the whole-K plan), and
// whole-K plans from kPreferBlocks column blocks up (below that the skinny kernel, which
// splits K inside a workgroup, is as fast).
bool resident_preferred(const GemmProblem* probs, int count, int g, bool may_split) {
    constexpr int64_t kPreferBlocks = 512;
    const ResidentPlan pl = plan_resident(probs, count, g, may_split);
    if (pl.len == 0) return false;
    return pl.splits > 1 || column_blocks(probs, count) >= kPreferBlocks;
}

size_t resident_workspace_bytes(const ResidentPlan& pl) {
    if (pl.len == 0 || pl.splits <= 1) return 0;
    return kCounterBytes + size_t(pl.tiles) * size_t(pl.splits) * size_t(pl.cb) * 1024u;
}

hipError_t launch_gemm_resident_group(const GemmProblem* probs, int count, int g, const ResidentPlan& pl,
                                      void* workspace, hipStream_t stream) {
    if (count < 1 || count > kMaxGroup || pl.len == 0) return hipErrorInvalidValue;
    for (int i = 1; i < count; ++i)
        if (probs[i].K != probs[0].K) return hipErrorInvalidValue;
    ResidentArgs a{};
    int total = 0;
    for (int i = 0; i < count; ++i) {
        a.grp.p[i] = probs[i];
        total += (probs[i].N / 16 + pl.cb - 1) / pl.cb;
        a.grp.tile_end[i] = total;
    }
    a.grp.count = count;
    a.cb = pl.cb;
    a.ks = pl.ks;
    a.splits = pl.splits;
    a.tiles = total;
    if (pl.splits > 1) {
        if (workspace == nullptr || total > kMaxCounterTiles) return hipErrorInvalidValue;
        a.counters = static_cast<uint32_t*>(workspace);
        a.ws = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + kCounterBytes);
    }
    const int T = probs[0].K / kStepCodes;
    uint32_t lds = lds_bytes((T + pl.splits - 1) / pl.splits, g, pl.cb);
    const uint32_t red = uint32_t(pl.cb * pl.ks) * 1024u;  // the K-slice reduction reuses the LDS
    lds = lds > red ? lds : red;
    return g == 64 ? launch_g<64>(a, lds, pl.len, stream) : launch_g<128>(a, lds, pl.len, stream);
}

// Fused epilogues, whole K only; hipErrorNotSupported where no plan fits (the caller then takes
// the tile kernel).  SwiGLU (gate rows [0, N), up rows [N, 2N) of W and S; Y is [M, N]): the
// workgroups hold an even number of column blocks -- half gate, half the up blocks of the same
// output columns -- enough that the pairs fill one round over the compute units.  Residual: the
// plain whole-K plan.
hipError_t launch_gemm_resident_epilogue(const GemmProblem& p, int g, int epi, hipStream_t stream) {
    const bool swiglu = epi == kEpiSwiglu;
    const int64_t w_rows = swiglu ? 2 * int64_t(p.N) : p.N;
    if (!resident_supported(p.M, w_rows, p.K, g, 2) || (epi != kEpiSwiglu && epi != kEpiResidual))
        return hipErrorNotSupported;
    const int T = p.K / kStepCodes;
    const int64_t out_blocks = p.N / 16;
    int cb = int((w_rows / 16 + kTargetWorkgroups - 1) / kTargetWorkgroups);
    cb = cb < 1 ? 1 : cb;
    if (swiglu) cb = cb < 2 ? 2 : cb + (cb & 1);
    if (cb > kMaxWaves) return hipErrorNotSupported;
    int ks = kMaxWaves / cb;
    ks = ks < T ? ks : T;
    const int len = (T + ks - 1) / ks;
    if (len > kMaxLen || lds_bytes(T, g, cb) > uint32_t(kMaxLds)) return hipErrorNotSupported;
    const int per_tile = swiglu ? cb / 2 : cb;  // output column blocks per workgroup
    ResidentArgs a{};
    a.grp.p[0] = p;
    a.grp.count = 1;
    a.tiles = int((out_blocks + per_tile - 1) / per_tile);
    a.grp.tile_end[0] = a.tiles;
    a.cb = cb;
    a.ks = ks;
    a.splits = 1;
    uint32_t lds = lds_bytes(T, g, cb);
    const uint32_t red = uint32_t(cb * ks) * 1024u;  // the K-slice reduction reuses the LDS
    lds = lds > red ? lds : red;
    if (swiglu) return g == 64 ? launch_g<64, kEpiSwiglu>(a, lds, len, stream) : launch_g<128, kEpiSwiglu>(a, lds, len, stream);
    return g == 64 ? launch_g<64, kEpiResidual>(a, lds, len, stream) : launch_g<128, kEpiResidual>(a, lds, len, stream);
}

}  // namespace lowbit

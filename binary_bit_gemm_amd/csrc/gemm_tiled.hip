// Packed low-bit GEMM on the gfx950 matrix cores: Y[M,N] = X[M,K] . dequant(W)[N,K]^T.
//
// Tiles of BM x BN outputs per workgroup; each wave owns WM x WN of them as 32x32 blocks
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation).  The K loop advances 64 elements per step.
//
// Data movement is organised around the vector-memory (texture address) path, whose
// per-request cost is what limits a kernel whose math is cheap per byte: a wave that finds
// that path's queue full cannot issue its next instruction, MFMAs included.  Everything
// therefore moves in large contiguous pieces through direct-to-LDS buffer loads:
//   * X[BM, 64] per step, double-buffered (rows past M read as zero);
//   * packed weights in blocks of 64 bytes per weight row (4 steps of ternary codes,
//     8 of binary), double-buffered;
//   * fp16 scales in blocks of 8 groups per weight row, double-buffered.
// All LDS tiles are XOR-swizzled in 16-byte chunks so that the operand reads are free of
// bank conflicts.
//
// Per step each wave expands, in registers, the codes of its own WN weight rows to bf16
// operands (lowbit_device.h; each code is expanded once per wave and reused by WM/32 MFMA
// blocks), runs for every scale group tmp = sum of g/16 (at most 4) MFMAs and folds the
// group scale in after the MFMA: acc += scale * tmp in fp32 -- the fp16 scale multiplies the
// exact partial sum and is never rounded to bf16 (w = scale_g * b, model card "Binary Weight
// Representation: 1-bit g128").  A group of 128 spans two steps and its scale is applied to
// each 64-element half.  Epilogue: fp32 -> bf16 round-to-nearest-even.
//
// The K positions a lane feeds to one MFMA are a free choice as long as the activation and
// weight operands agree: lane half h takes the h-th half of every scale group (or of every
// 64-element step), chunk j its codes 8j..8j+7, so consecutive codes meet consecutive
// activations and X needs no reordering.
#include "lowbit_device.h"
#include "lowbit_internal.h"

namespace lowbit {
namespace {

constexpr int KS = 64;                    // K elements per step
constexpr int kRowBytes = KS * 2;         // one bf16 row of an X tile
constexpr int kChunksPerRow = KS / 8;     // 16-byte chunks per X row

__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// 16-byte direct-to-LDS copy with the sc1 cache policy (device-coherent: data other workgroups
// stored the same way); lane i's 16 bytes land at lds_wave_base + 16 * i.
__device__ __forceinline__ void dma16_sc1(__amdgpu_buffer_rsrc_t rs, void* lds_wave_base, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_wave_base, 16, voff, 0,
                                            0, 16);
}

__device__ __forceinline__ int x_off(int row, int chunk) { return row * kRowBytes + ((chunk ^ lds_swizzle(row)) << 4); }

// Packed-weight block: WB (32 or 64) bytes per row = WB/16 chunks of 16 bytes; chunk c of row
// r is stored at position c ^ w_swz(r) so that 16 consecutive rows reading the same chunk
// hit 16 different bank groups.
template <int WB>
__device__ __forceinline__ int w_swz(int row) { return WB == 64 ? (row >> 2) & 3 : (row >> 3) & 1; }

template <int BITS, int G, int BM, int BN, int WAVES_M, int WAVES_N, int WB>
struct Cfg {
    static constexpr int WAVES = WAVES_M * WAVES_N;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    static constexpr int MB = WM / 32, NB = WN / 32;
    static constexpr int SUBG = G < KS ? G : KS;             // K elements per scale application
    static constexpr int GPS = KS / SUBG;                    // scale applications per step
    static constexpr int CHUNKS = SUBG / 16;                 // MFMAs per application per block
    static constexpr int X_TILE = BM * kRowBytes;
    static constexpr int X_LOADS = X_TILE / (16 * THREADS);  // 16-byte copies per thread per step
    static constexpr int W_STEP_BYTES = KS * BITS / 8;       // packed bytes of one row per step
    static constexpr int W_SPB = WB / W_STEP_BYTES;          // steps per WB-byte weight block
    static constexpr int W_CPR = WB / 16;                    // 16-byte chunks per row of a block
    static constexpr int W_BLOCK = BN * WB;
    static constexpr int W_LOADS = W_BLOCK / 16;             // 16-byte copies per weight block
    static constexpr int S_GPB = 8;                          // scale groups per scale block
    static constexpr int S_BLOCK = BN * 32;                  // two aligned 16-byte windows per row
    static constexpr int S_LOADS = S_BLOCK / 16;
    static_assert(MB >= 1 && NB >= 1, "wave tile too small");
    static_assert(X_TILE % (16 * THREADS) == 0, "X tile is not a whole number of copies");
    static_assert(W_LOADS % 64 == 0 && S_LOADS % 64 == 0, "blocks are whole waves of copies");
};

// Stream-K launch (SK = true, one problem): a grid of `nwg` workgroups, workgroup w owning the
// (tile, step) units [w U / nwg, (w + 1) U / nwg) of the U = tiles x steps units in tile-major
// order.  A tile whose steps span several workgroups is finished by one of them from fp32
// partial tiles in the workspace: `counters` (zero between calls, one per split tile, indexed
// by the workgroup that owns the tile's last step) and `parts` (two partial-tile slots per
// workgroup: the tile of its first unit, the tile of its last).
struct StreamK {
    uint32_t* counters;
    unsigned char* parts;
    int nwg;
};

template <int BITS, int G, int BM, int BN, int WAVES_M, int WAVES_N, int WB, bool SK = false>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, 1) void gemm_tiled_kernel(ProblemGroup grp, StreamK sk) {
    using C = Cfg<BITS, G, BM, BN, WAVES_M, WAVES_N, WB>;
    // Separate static buffers (not one array indexed by parity): the compiler can then see
    // that reads of one buffer do not depend on copies still landing in the other.
    __shared__ __attribute__((aligned(16))) unsigned char xa0[C::X_TILE];
    __shared__ __attribute__((aligned(16))) unsigned char xa1[C::X_TILE];
    __shared__ __attribute__((aligned(16))) unsigned char wk0[C::W_BLOCK];
    __shared__ __attribute__((aligned(16))) unsigned char wk1[C::W_BLOCK];
    __shared__ __attribute__((aligned(16))) unsigned char sk0[C::S_BLOCK];
    __shared__ __attribute__((aligned(16))) unsigned char sk1[C::S_BLOCK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int wave_m = wave % WAVES_M, wave_n = wave / WAVES_M;
    const int half = lane >> 5, col = lane & 31;
    f32x16_t acc[C::MB][C::NB];

    // Steps [kb, ke) of tile `tile` of problem p, summed into acc from zero.
    auto run = [&](const GemmProblem& p, int tile, int kb, int ke) __attribute__((always_inline)) {
    const int M = p.M, N = p.N, K = p.K;
    const int tiles_n = (N + BN - 1) / BN;
    const int tm = tile / tiles_n, tn = tile % tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;
    const int wm0 = wave_m * C::WM, wn0 = wave_n * C::WN;

    const int kgroups = K / G;
    const int ksub = K / C::SUBG;
    const int ksteps = (K + KS - 1) / KS;
    const uint32_t w_row_bytes = uint32_t(K) * BITS / 8;
    const uint32_t s_row_bytes = uint32_t(kgroups) * 2u;

    // ---- X: thread copies a fixed chunk column of rows r_first + i * rows_per_copy ----
    constexpr int kRowsPerCopy = C::THREADS / kChunksPerRow;
    const int r_first = tid / kChunksPerRow;
    const uint32_t x_voff = uint32_t(r_first) * uint32_t(K) * 2u +
                            uint32_t((tid % kChunksPerRow) ^ lds_swizzle(r_first)) * 16u;
    const uint32_t x_row_step = uint32_t(kRowsPerCopy) * uint32_t(K) * 2u;
    const unsigned char* x_tile = reinterpret_cast<const unsigned char*>(p.X) + size_t(m0) * size_t(K) * 2;
    const uint32_t x_tile_bytes = uint32_t(M - m0 < BM ? M - m0 : BM) * uint32_t(K) * 2u;
    auto issue_x = [&](int step, unsigned char* buf) {
        const uint32_t kb = uint32_t(step) * KS * 2u;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(x_tile + kb, x_tile_bytes - kb);
#pragma unroll
        for (int i = 0; i < C::X_LOADS; ++i)
            dma16(rs, buf + (i * C::THREADS + wave_u * 64) * 16, x_voff + uint32_t(i) * x_row_step, 0);
    };

    // ---- packed weights: block b holds steps [b*W_SPB, (b+1)*W_SPB) of the tile's BN rows.
    // Copy slot t (of W_LOADS) = row t/W_CPR, stored chunk t%W_CPR, which holds source chunk
    // (t%W_CPR) ^ w_swz(row).  Rows past N re-read row N-1.
    const __amdgpu_buffer_rsrc_t w_rs = make_rsrc(p.W, uint32_t(N) * w_row_bytes);
    auto issue_w = [&](int block, unsigned char* buf) {
#pragma unroll
        for (int i = 0; i < (C::W_LOADS + C::THREADS - 1) / C::THREADS; ++i) {
            const int slot0 = i * C::THREADS + wave_u * 64;  // first slot of this wave's copy
            if (slot0 < C::W_LOADS) {
                const int slot = slot0 + lane;
                const int r = slot / C::W_CPR;
                int n = n0 + r;
                n = n < N ? n : N - 1;
                const uint32_t voff = uint32_t(n) * w_row_bytes + uint32_t(((slot % C::W_CPR) ^ w_swz<WB>(r)) * 16);
                dma16(w_rs, buf + slot0 * 16, voff, __builtin_amdgcn_readfirstlane(block * WB));
            }
        }
    };

    // ---- scales: block b holds groups [8b, 8b+8) of the tile's BN rows as two aligned
    // 16-byte windows per row (32 bytes); the row's group 8b sits (row offset & 15) bytes in.
    const __amdgpu_buffer_rsrc_t s_rs = make_rsrc(p.S, uint32_t(N) * s_row_bytes);
    auto issue_s = [&](int block, unsigned char* buf) {
#pragma unroll
        for (int i = 0; i < (C::S_LOADS + C::THREADS - 1) / C::THREADS; ++i) {
            const int slot0 = i * C::THREADS + wave_u * 64;
            if (slot0 < C::S_LOADS) {
                const int slot = slot0 + lane;
                const int r = slot >> 1;
                int n = n0 + r;
                n = n < N ? n : N - 1;
                const uint32_t start = uint32_t(n) * s_row_bytes + uint32_t(block) * 16u;
                const uint32_t voff = (start & ~15u) + uint32_t(slot & 1) * 16u;
                dma16(s_rs, buf + slot0 * 16, voff, 0);
            }
        }
    };

    // Per-lane byte offset of its NB weight rows' group 8b within a scale block.
    int s_rd[C::NB];
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) {
        const int r = wn0 + nb * 32 + col;
        int n = n0 + r;
        n = n < N ? n : N - 1;
        s_rd[nb] = r * 32 + int((uint32_t(n) * s_row_bytes) & 15u);
    }

#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.0f;

    const float code_scale = BITS == 2 ? 0.5f : -0.5f;  // operand holds 2c (ternary), -2c (binary)

    // A step's packed words and scales are read from LDS into registers before any copy of
    // the step is issued: the compiler cannot tell which of the two weight / scale buffers a
    // step reads, and would otherwise wait for every copy in flight before these reads.
    typedef uint32_t u32x2_t __attribute__((__vector_size__(8)));
    constexpr int kWordsPerLane = (C::SUBG / 2) * BITS / 32 > 0 ? (C::SUBG / 2) * BITS / 32 : 1;
    struct Ops {
        uint32_t w[C::GPS][C::NB][kWordsPerLane];
        float sc[C::GPS][C::NB];
    };
    auto read_operands = [&](const unsigned char* wt, const unsigned char* st, int step, Ops& o) {
        const int wj = step % C::W_SPB;  // step within the weight block
#pragma unroll
        for (int q = 0; q < C::GPS; ++q) {
            const int grp = (step * KS + q * C::SUBG) / G;
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb) {
                const int r = wn0 + nb * 32 + col;
                o.sc[q][nb] = half_bits_to_float(*reinterpret_cast<const uint16_t*>(st + s_rd[nb] + (grp & 7) * 2)) *
                              code_scale;
                // this lane's codes: sub-group q of the step, half `half` -> SUBG/2 codes
                const int code0 = q * C::SUBG + half * (C::SUBG / 2);       // within the step
                const int byte0 = wj * C::W_STEP_BYTES + code0 * BITS / 8;  // within the block row
                const int chunk = byte0 >> 4, inb = byte0 & 15;
                const unsigned char* src = wt + r * WB + ((chunk ^ w_swz<WB>(r)) << 4) + inb;
                if constexpr (kWordsPerLane == 2) {
                    const u32x2_t v = *reinterpret_cast<const u32x2_t*>(src);
                    o.w[q][nb][0] = v[0];
                    o.w[q][nb][1] = v[1];
                } else if constexpr ((C::SUBG / 2) * BITS >= 32) {
                    o.w[q][nb][0] = *reinterpret_cast<const uint32_t*>(src);
                } else {  // binary g = 32: 16 codes = half of an aligned word
                    const uint32_t w = *reinterpret_cast<const uint32_t*>(src - (inb & 3));
                    o.w[q][nb][0] = w >> ((inb & 2) * 8);
                }
            }
        }
    };

    // `issue` runs once the first row block's MFMAs of the step are under way: the next step's
    // copies then do not go out in a burst with the step's first operand reads and expansion.
    auto compute = [&](const unsigned char* xt, const Ops& o, int step, auto&& issue) {
#pragma unroll
        for (int q = 0; q < C::GPS; ++q) {
            if (C::GPS > 1 && step * C::GPS + q >= ksub) break;  // K tail (g = 32, K % 64 == 32)
            u32x4_t bfr[C::NB][C::CHUNKS];
            float sc[C::NB];
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb) {
                sc[nb] = o.sc[q][nb];
                uint32_t d[C::CHUNKS * 4];
                if constexpr (BITS == 2) {
#pragma unroll
                    for (int w = 0; w < kWordsPerLane; ++w) expand_ternary_word(o.w[q][nb][w], d + 8 * w);
                } else if constexpr (C::SUBG == 64) {
                    expand_binary_word<16>(o.w[q][nb][0], d);
                } else {
                    expand_binary_word<8>(o.w[q][nb][0], d);
                }
#pragma unroll
                for (int j = 0; j < C::CHUNKS; ++j)
                    bfr[nb][j] = u32x4_t{d[4 * j], d[4 * j + 1], d[4 * j + 2], d[4 * j + 3]};
            }

            // Blocks b = mb*NB + nb in order; the MFMA chain of block b is issued before the
            // scale FMAs of block b-1, which use the other partial-sum registers.
            f32x16_t tmp[2];
            bf16x8_t afr[C::CHUNKS];
#pragma unroll
            for (int b = 0; b <= C::MB * C::NB; ++b) {
                if (q == 0 && b == (C::MB > 1 && C::GPS == 1 ? C::NB : 0)) issue();
                if (b < C::MB * C::NB) {
                    const int mb = b / C::NB, nb = b % C::NB;
                    if (nb == 0) {
                        const int row = wm0 + mb * 32 + col;
#pragma unroll
                        for (int j = 0; j < C::CHUNKS; ++j)
                            afr[j] = *reinterpret_cast<const bf16x8_t*>(
                                xt + x_off(row, (q * C::SUBG + half * (C::SUBG / 2)) / 8 + j));
                    }
                    f32x16_t t = {};
#pragma unroll
                    for (int j = 0; j < C::CHUNKS; ++j)
                        t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr[j], __builtin_bit_cast(bf16x8_t, bfr[nb][j]),
                                                                    t, 0, 0, 0);
                    tmp[b & 1] = t;
                }
                if (b > 0) {
                    const int pb = b - 1, mb = pb / C::NB, nb = pb % C::NB;
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        acc[mb][nb][i] = __builtin_fmaf(sc[nb], tmp[pb & 1][i], acc[mb][nb][i]);
                }
            }
        }
    };

    // Block bookkeeping: the weight block of step s is s / W_SPB, its scale block group / 8.
    auto w_buf = [&](int step) -> unsigned char* { return ((step / C::W_SPB) & 1) ? wk1 : wk0; };
    auto s_block = [&](int step) { return (step * KS / G) / C::S_GPB; };
    auto s_buf = [&](int step) -> unsigned char* { return (s_block(step) & 1) ? sk1 : sk0; };
    const int w_blocks = (ksteps + C::W_SPB - 1) / C::W_SPB;
    const int s_blocks = (kgroups + C::S_GPB - 1) / C::S_GPB;

    // During step s: X of step s+1, and -- on the first step of a weight or scale block, or the
    // range's first step, which can fall inside a block -- the next block into the other buffer
    // (after this step's operands were read), as long as the range still reaches it.
    // (The whole-K launch keeps the plain conditions, with kb = 0 and ke = ksteps.)
    auto prefetch_x = [&](int step, unsigned char* xbuf) {
        if (step + 1 < (SK ? ke : ksteps)) issue_x(step + 1, xbuf);
    };
    auto prefetch_blocks = [&](int step) {
        const int wb = step / C::W_SPB;
        const int sb = s_block(step);
        if constexpr (SK) {
            if ((step == kb || step % C::W_SPB == 0) && wb + 1 < w_blocks && (wb + 1) * C::W_SPB < ke)
                issue_w(wb + 1, ((wb + 1) & 1) ? wk1 : wk0);
            if ((step == kb || s_block(step - 1) != sb) && sb + 1 < s_blocks && s_block(ke - 1) > sb)
                issue_s(sb + 1, ((sb + 1) & 1) ? sk1 : sk0);
        } else {
            if (step % C::W_SPB == 0 && wb + 1 < w_blocks) issue_w(wb + 1, ((wb + 1) & 1) ? wk1 : wk0);
            if ((step == 0 || s_block(step - 1) != sb) && sb + 1 < s_blocks) issue_s(sb + 1, ((sb + 1) & 1) ? sk1 : sk0);
        }
    };

    issue_x(kb, xa0);
    issue_w(kb / C::W_SPB, w_buf(kb));
    issue_s(s_block(kb), s_buf(kb));
    wait_vmcnt0();
    __syncthreads();

    Ops ops;
    for (int step = kb; step < ke; step += 2) {
        read_operands(w_buf(step), s_buf(step), step, ops);
        compute(xa0, ops, step, [&]() {
            prefetch_x(step, xa1);
            prefetch_blocks(step);
        });
        wait_vmcnt0();
        __syncthreads();
        if (step + 1 >= ke) break;
        read_operands(w_buf(step + 1), s_buf(step + 1), step + 1, ops);
        compute(xa1, ops, step + 1, [&]() {
            prefetch_x(step + 1, xa0);
            prefetch_blocks(step + 1);
        });
        wait_vmcnt0();
        __syncthreads();
    }

    if constexpr (!SK) {
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
    };

    // The same epilogue for a stream-K tile (after the range's last segment of it).
    auto store_y = [&](const GemmProblem& p, int tile) __attribute__((always_inline)) {
        const int tiles_n = (p.N + BN - 1) / BN;
        const int m0 = (tile / tiles_n) * BM + wave_m * C::WM, n0 = (tile % tiles_n) * BN + wave_n * C::WN;
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) {
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb) {
                const int n = n0 + nb * 32 + col;
                if (n >= p.N) continue;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int m = m0 + mb * 32 + 8 * (i / 4) + 4 * half + (i % 4);
                    if (m < p.M) p.Y[int64_t(m) * p.N + n] = float_to_bf16_bits(acc[mb][nb][i]);
                }
            }
        }
    };

    if constexpr (!SK) {
        // Workgroup -> (problem, tile); the tiles one XCD runs are contiguous in the group's
        // tile order.
        const int t = xcd_remap(blockIdx.x, grp.tile_end[grp.count - 1]);
        int pi = 0;
        while (pi + 1 < grp.count && t >= grp.tile_end[pi]) ++pi;
        const GemmProblem p = grp.p[pi];
        const int tile = t - (pi > 0 ? grp.tile_end[pi - 1] : 0);
        run(p, tile, 0, (p.K + KS - 1) / KS);  // the whole K, Y written at its end
    } else {
        // The tiles of a workgroup's range run last to first: a tile's first steps are then
        // the end of one workgroup's range, computed first, and its last steps the start of the
        // next one's, computed last -- so the workgroup owning a tile's last step is nearly
        // always the last to finish it, and adds the others' partials to its own registers
        // without storing them.  Partial tiles travel as 16-byte loads and stores with the sc1
        // cache policy (through to the device-coherent level: the L2 of one XCD is not
        // coherent with the others); a workgroup's stores complete before its arrival is
        // counted.  Every tile's sum runs in one fixed order, last steps first, whichever
        // workgroup adds it, so results do not depend on timing.  No workgroup waits for
        // another.
        const GemmProblem p = grp.p[0];
        // uniform values in scalar registers (32-bit: the host keeps units * workgroups < 2^31)
        auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
        const int ksteps = uni((p.K + KS - 1) / KS);
        const int U = uni(((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN) * ksteps);
        const int nwg = sk.nwg;
        const int w = uni(xcd_remap(blockIdx.x, nwg));
        const int u0 = uni(w * U / nwg), u1 = uni((w + 1) * U / nwg);
        if (u0 >= u1) return;
        constexpr int kSc1 = 16;  // cache policy bit sc1 of buffer loads and stores
        constexpr uint32_t kSlot = uint32_t(BM) * BN * 4u;
        constexpr int kPairs = C::MB * C::NB * 4;  // (block, quarter) pairs of a lane's accumulators
        const __amdgpu_buffer_rsrc_t prs = make_rsrc(sk.parts, uint32_t(2 * nwg) * kSlot);
        __shared__ int sk_last;
        // A slot holds pair q of wave v's lanes at (q * WAVES + v) KB, lanes contiguous: each wave
        // moves only its own 1 KB pieces.
        auto piece = [&](int q) { return (uint32_t(q) * C::WAVES + uint32_t(wave_u)) * 1024u; };
        // A finisher's staging: two 4 KB buffers per wave in the X tiles, idle between segments.
        unsigned char* const stg0 = xa0 + wave_u * 4096;
        unsigned char* const stg1 = xa1 + wave_u * 4096;
        static_assert(C::X_TILE >= C::WAVES * 4096, "staging does not fit the X tiles");
        // Y = bf16(acc + the part in slot s), block by block: block b's four 1 KB pieces are
        // copied into one staging buffer while the previous block is added and stored (direct-
        // to-LDS copies need no registers while acc holds the tile).
        auto store_y_plus = [&](int tile, uint32_t s) __attribute__((always_inline)) {
            const uint32_t base = s * kSlot + uint32_t(lane) * 16u;
            auto fetch = [&](int b, unsigned char* buf) __attribute__((always_inline)) {
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) dma16_sc1(prs, buf + i4 * 1024, base + piece(4 * b + i4));
            };
            const int tiles_n = (p.N + BN - 1) / BN;
            const int m0 = (tile / tiles_n) * BM + wave_m * C::WM, n0 = (tile % tiles_n) * BN + wave_n * C::WN;
            fetch(0, stg0);
#pragma unroll
            for (int b = 0; b < C::MB * C::NB; ++b) {
                if (b + 1 < C::MB * C::NB) {
                    fetch(b + 1, (b & 1) ? stg0 : stg1);
                    wait_vmcnt<4>();
                } else {
                    wait_vmcnt<0>();
                }
                const unsigned char* buf = (b & 1) ? stg1 : stg0;
                const int mb = b / C::NB, nb = b % C::NB;
                const int n = n0 + nb * 32 + col;
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const f32x4_t f = *reinterpret_cast<const f32x4_t*>(buf + i4 * 1024 + lane * 16);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = 4 * i4 + e;
                        const int m = m0 + mb * 32 + 8 * (i / 4) + 4 * half + (i % 4);
                        if (n < p.N && m < p.M) p.Y[int64_t(m) * p.N + n] = float_to_bf16_bits(acc[mb][nb][i] + f[e]);
                    }
                }
            }
        };
        const int t_first = uni(u0 / ksteps);
        for (int tile = uni((u1 - 1) / ksteps); tile >= t_first; --tile) {
            const int tu = tile * ksteps;
            const int kb = (u0 > tu ? u0 : tu) - tu;
            const int ke = (u1 < tu + ksteps ? u1 : tu + ksteps) - tu;
            run(p, tile, kb, ke);
            if (kb == 0 && ke == ksteps) {
                store_y(p, tile);
                continue;
            }
            // the tile's workgroups wf .. wl (owners of its first and last unit)
            const int wf = uni(((tu + 1) * nwg - 1) / U);
            const int wl = uni(((tu + ksteps) * nwg - 1) / U);
            uint32_t* counter = sk.counters + wl;
            // slot of workgroup v's part of this tile: 2v for the tile of v's first unit, else 2v + 1
            auto slot = [&](int v) { return uint32_t(uni(2 * v + ((v * U / nwg) / ksteps == tile ? 0 : 1))); };
            if (tid == 0)
                sk_last = wl - wf == 1 && __hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                                         uint32_t(wl - wf);
            __syncthreads();
            if (!sk_last) {
                const uint32_t base = slot(w) * kSlot + uint32_t(lane) * 16u;
#pragma unroll
                for (int q = 0; q < kPairs; ++q) {
                    const int bb = q / 4, i4 = q % 4, mb = bb / C::NB, nb = bb % C::NB;
                    // whole-vector bit cast (a bit cast of one vector element read element 0 here)
                    const f32x4_t v = {acc[mb][nb][4 * i4], acc[mb][nb][4 * i4 + 1], acc[mb][nb][4 * i4 + 2],
                                       acc[mb][nb][4 * i4 + 3]};
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), prs, base + piece(q), 0,
                                                           kSc1);
                }
                wait_vmcnt0();
                __syncthreads();
                if (tid == 0)
                    sk_last = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                              uint32_t(wl - wf);
                __syncthreads();
                if (!sk_last) continue;
            }
            // Sum = ((P_wl + P_wl-1) + ...) + P_wf.  A two-part tile's finisher owns its last step
            // (the shortcut above, or the count) and adds the other part to its registers.
            if (wl - wf == 1) {
                store_y_plus(tile, slot(w == wl ? wf : wl));
            } else {
                // every part is in the workspace: from -0 (-0 + x == x for every x), in the same
                // order, four outputs at a time
                const int tiles_n = (p.N + BN - 1) / BN;
                const int m0 = (tile / tiles_n) * BM + wave_m * C::WM, n0 = (tile % tiles_n) * BN + wave_n * C::WN;
                for (int q = 0; q < kPairs; ++q) {
                    f32x4_t t = {-0.0f, -0.0f, -0.0f, -0.0f};
                    for (int v = wl; v >= wf; --v)
                        t += __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                             prs, slot(v) * kSlot + uint32_t(lane) * 16u + piece(q), 0,
                                                             kSc1));
                    const int bb = q / 4, i4 = q % 4, mb = bb / C::NB, nb = bb % C::NB;
                    const int n = n0 + nb * 32 + col;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = 4 * i4 + e;
                        const int m = m0 + mb * 32 + 8 * (i / 4) + 4 * half + (i % 4);
                        if (n < p.N && m < p.M) p.Y[int64_t(m) * p.N + n] = float_to_bf16_bits(t[e]);
                    }
                }
            }
            __syncthreads();  // the staging buffers are the next segment's X tiles
            if (tid == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <int BITS, int G, int BM, int BN, int WAVES_M, int WAVES_N, int WB>
hipError_t launch_cfg(const GemmProblem* probs, int count, hipStream_t stream) {
    ProblemGroup grp{};
    int total = 0;
    for (int i = 0; i < count; ++i) {
        grp.p[i] = probs[i];
        total += int(tiles_of(probs[i].M, BM) * tiles_of(probs[i].N, BN));
        grp.tile_end[i] = total;
    }
    grp.count = count;
    hipLaunchKernelGGL((gemm_tiled_kernel<BITS, G, BM, BN, WAVES_M, WAVES_N, WB>), dim3(total),
                       dim3(64 * WAVES_M * WAVES_N), 0, stream, grp, StreamK{});
    const hipError_t e = hipGetLastError();
    if (e == hipSuccess && trace_enabled()) {
        char cfg[64];
        snprintf(cfg, sizeof cfg, "%dx%d waves=%dx%d", BM, BN, WAVES_M, WAVES_N);
        trace_launch("tiled32", cfg, G, BITS, probs, count, unsigned(total), 64u * WAVES_M * WAVES_N, 0u);
    }
    return e;
}

// Stream-K on the 256 x 256 tile (8 waves of 128 x 64): one workgroup per compute unit.
constexpr int kSkBM = 256, kSkBN = 256;
constexpr size_t kSkCounterBytes = 4096;  // the workspace's counter region (as the resident kernel's)

int streamk_workgroups(const GemmProblem& p) {
    const int64_t units = tiles_of(p.M, kSkBM) * tiles_of(p.N, kSkBN) * tiles_of(p.K, 64);
    return int(units < kComputeUnits ? units : kComputeUnits);
}

template <int BITS, int G>
hipError_t launch_streamk_cfg(const GemmProblem& p, void* workspace, hipStream_t stream) {
    ProblemGroup grp{};
    grp.p[0] = p;
    grp.count = 1;
    grp.tile_end[0] = int(tiles_of(p.M, kSkBM) * tiles_of(p.N, kSkBN));
    StreamK sk{};
    sk.nwg = streamk_workgroups(p);
    sk.counters = static_cast<uint32_t*>(workspace);
    sk.parts = static_cast<unsigned char*>(workspace) + kSkCounterBytes;
    hipLaunchKernelGGL((gemm_tiled_kernel<BITS, G, kSkBM, kSkBN, 2, 4, 64, true>), dim3(sk.nwg), dim3(512), 0, stream,
                       grp, sk);
    const hipError_t e = hipGetLastError();
    if (e == hipSuccess && trace_enabled())
        trace_launch("tiled32", "256x256 waves=2x4 streamk", G, BITS, &p, 1, unsigned(sk.nwg), 512u, 0u);
    return e;
}

template <int BITS, int G>
hipError_t launch_bits_g(const GemmProblem* probs, int count, int variant, hipStream_t stream) {
    // LDS: 256x128 = 80 KB and 128x256 = 72 KB (two workgroups per CU); 256x256 = 112 KB.
    switch (variant) {
        case TILE_256x128: return launch_cfg<BITS, G, 256, 128, 2, 2, 32>(probs, count, stream);
        case TILE_256x256: return launch_cfg<BITS, G, 256, 256, 2, 4, 64>(probs, count, stream);
        case TILE_128x256: return launch_cfg<BITS, G, 128, 256, 1, 4, 32>(probs, count, stream);
        default:           return launch_cfg<BITS, G, 64, 256, 1, 4, 32>(probs, count, stream);
    }
}

}  // namespace

namespace {

struct TileShape {
    int variant, bm, bn, per_cu;  // workgroups resident per compute unit
    float eff, eff_binary;        // relative per-FLOP efficiency of the tile, ternary / binary
};

// Measured at M = 4608 on the denoise-step shapes: a 288 x 192 tile does ~0.87 (ternary) and
// ~0.82 (binary) of a 256 x 256 tile's work per unit time (smaller wave tiles: less operand
// reuse), which about cancels (ternary) or outweighs (binary) the 16% of units a 256 x 256
// grid leaves idle at N = 3072.  A 96 x 192 tile (four waves, one per SIMD) does ~0.54; it
// pays where nothing larger fills the chip (1536 x 3072: 256 tiles).  The same tile with K
// split between two groups of four waves does ~0.65 where the grid is a single round (one
// workgroup per compute unit: 1536 x 3072 at K = 3072 and 9216 measured 17% and 21% faster);
// over several rounds two plain 96 x 192 workgroups share a compute unit instead, and the
// split measured slower.
constexpr TileShape kTiles[] = {
    {TILE_256x256, 256, 256, 1, 1.00f, 1.00f},
    {TILE_288x192, 288, 192, 1, 0.87f, 0.82f},
    {TILE_256x192, 256, 192, 1, 0.87f, 0.82f},
    {TILE_128x256, 128, 256, 2, 0.92f, 0.92f},
    {TILE_64x256, 64, 256, 2, 0.75f, 0.75f},
    {TILE_96x192, 96, 192, 1, 0.54f, 0.51f},
    {TILE_96x192K2, 96, 192, 1, 0.65f, 0.62f},
    // 4-bit codes only (the one kernel they run on): fills the chip where 96 x 192 leaves most
    // compute units idle, e.g. the text encoder's 512 x 2560 down projection (160 vs 84 tiles)
    {TILE_64x128K2, 64, 128, 1, 0.40f, 0.40f},
};

}  // namespace

int pick_tile_variant(const GemmProblem* probs, int count, int g, int bits) {
    int best = bits == 4 ? TILE_288x192 : TILE_64x256;
    double best_cost = 0.0;
    for (const TileShape& t : kTiles) {
        if (is_tile16_variant(t.variant) && !tile16_supported(g, bits)) continue;
        if (bits == 4 && !is_tile16_variant(t.variant)) continue;  // 4-bit codes: the 16x16-block tile only
        if (t.variant == TILE_64x128K2) {
            bool skip = bits != 4;
            for (int i = 0; i < count; ++i) skip = skip || (probs[i].K / 64) % 2 != 0;
            if (skip) continue;
        }
        if ((t.variant == TILE_96x192 || t.variant == TILE_96x192K2) && bits != 4) {
            // measured at M = 1536; below M = 1024 they stay unused.  The K split needs an even
            // number of 64-element steps.
            bool skip = false;
            for (int i = 0; i < count; ++i)
                skip = skip || probs[i].M < 1024 || (t.variant == TILE_96x192K2 && (probs[i].K / 64) % 2 != 0);
            if (skip) continue;
        }
        int64_t tiles = 0;
        for (int i = 0; i < count; ++i)
            tiles += tiles_of(probs[i].M, t.bm) * tiles_of(probs[i].N, t.bn);
        const int64_t slots = int64_t(kComputeUnits) * t.per_cu;
        const int64_t rounds = (tiles + slots - 1) / slots;
        if (t.variant == TILE_96x192K2 && rounds > 1) continue;  // single rounds only (see above)
        const double cost = double(rounds) * t.per_cu * t.bm * t.bn / (bits == 1 ? t.eff_binary : t.eff);
        if (best_cost == 0.0 || cost < best_cost) {
            best = t.variant;
            best_cost = cost;
        }
    }
    return best;
}

int pick_tile_variant(int64_t M, int64_t N, int64_t K, int g, int bits) {
    const GemmProblem p{nullptr, nullptr, nullptr, nullptr, int(M), int(N), int(K)};
    return pick_tile_variant(&p, 1, g, bits);
}

const char* tile_variant_name(int variant) {
    switch (variant) {
        case TILE_256x128: return "tile256x128";
        case TILE_256x256: return "tile256x256";
        case TILE_128x256: return "tile128x256";
        case TILE_288x192: return "tile288x192";
        case TILE_96x192: return "tile96x192";
        case TILE_96x192K2: return "tile96x192k2";
        case TILE_64x128K2: return "tile64x128k2";
        case TILE_256x192: return "tile256x192";
        case TILE_256x256SK: return "tile256x256sk";
        default: return "tile64x256";
    }
}

hipError_t launch_gemm_tiled_group(const GemmProblem* probs, int count, int g, int bits, int variant,
                                   hipStream_t stream) {
    if (bits == 4 && !is_tile16_variant(variant)) variant = TILE_288x192;  // the only 4-bit kernel
    if (variant == TILE_256x256SK) variant = TILE_256x256;  // stream-K needs a workspace (the grouped launch)
    if (is_tile16_variant(variant)) {
        if (tile16_supported(g, bits)) return launch_gemm_tile16_group(probs, count, g, bits, variant, stream);
        variant = TILE_256x256;
    }
    if (bits == 2) {
        switch (g) {
            case 32: return launch_bits_g<2, 32>(probs, count, variant, stream);
            case 64: return launch_bits_g<2, 64>(probs, count, variant, stream);
            default: return launch_bits_g<2, 128>(probs, count, variant, stream);
        }
    }
    switch (g) {
        case 32: return launch_bits_g<1, 32>(probs, count, variant, stream);
        case 64: return launch_bits_g<1, 64>(probs, count, variant, stream);
        default: return launch_bits_g<1, 128>(probs, count, variant, stream);
    }
}

size_t streamk_workspace_bytes(const GemmProblem& p, int g, int bits) {
    (void)g;
    if ((bits != 1 && bits != 2) || p.M <= 0 || p.N <= 0 || p.K <= 0) return 0;
    // the kernel's partition arithmetic is 32-bit: units x workgroups < 2^31
    const int64_t units = tiles_of(p.M, kSkBM) * tiles_of(p.N, kSkBN) * tiles_of(p.K, 64);
    if (units * kComputeUnits >= (int64_t(1) << 31)) return 0;
    return kSkCounterBytes + 2 * size_t(streamk_workgroups(p)) * size_t(kSkBM) * kSkBN * 4u;
}

hipError_t launch_gemm_streamk(const GemmProblem& p, int g, int bits, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
    const size_t need = streamk_workspace_bytes(p, g, bits);
    if (need == 0 || workspace == nullptr || workspace_bytes < need) return hipErrorInvalidValue;
    if (bits == 2) {
        switch (g) {
            case 32: return launch_streamk_cfg<2, 32>(p, workspace, stream);
            case 64: return launch_streamk_cfg<2, 64>(p, workspace, stream);
            default: return launch_streamk_cfg<2, 128>(p, workspace, stream);
        }
    }
    switch (g) {
        case 32: return launch_streamk_cfg<1, 32>(p, workspace, stream);
        case 64: return launch_streamk_cfg<1, 64>(p, workspace, stream);
        default: return launch_streamk_cfg<1, 128>(p, workspace, stream);
    }
}

hipError_t launch_gemm_tiled(const GemmProblem& p, int g, int bits, int variant, hipStream_t stream) {
    return launch_gemm_tiled_group(&p, 1, g, bits, variant, stream);
}

}  // namespace lowbit

// Packed ternary, binary or 4-bit GEMM on 16x16x32 MFMA blocks: Y[M,N] = X[M,K] . dequant(W)[N,K]^T,
// for scale groups of 64 or 128.
//
// Why a second tile kernel: with 32x32 blocks a workgroup tile is a multiple of 32 in both
// directions and 8 waves want a multiple of 8 blocks, so 4608 x 3072 outputs come out as 216
// tiles of 256 x 256 on 256 compute units -- 16% of the chip idles.  16x16 blocks allow a
// 288 x 192 tile (12 waves of 144 x 32): 4608 x 3072 is then exactly 256 tiles, 4608 x 9216
// and 4608 x 18432 whole multiples of 256.  Per FLOP the 16x16x32 instruction needs the same
// operand bytes, the same code expansion and the same scale FMAs as the 32x32x16 one.  The
// same kernel with 4 waves makes a 96 x 192 tile: 1536 x 3072 is then exactly 256 tiles.  There
// one wave per SIMD leaves the SIMD idle whenever its wave waits, so that tile also comes with
// its K range split between KSPLIT groups of 4 waves: each group streams its own half of K
// through its own LDS buffers (the groups share the step barrier), and at the end the groups'
// fp32 sums are added in group order 0, 1 (a fixed order) before the epilogue.
//
// The 288 x 192 tile (108 KB of LDS, one workgroup per compute unit) launches persistent when a
// problem group has more tiles than compute units: 256 workgroups, each looping over the tiles
// of virtual ids b, b + 256, ...  Between two tiles a workgroup issues the next tile's first
// copies before its epilogue, and no new workgroup has to be launched on the compute unit.
//
// Data movement is that of the 32x32 kernel (direct-to-LDS copies of X per 64-element step,
// of packed weights in 64-byte row blocks, of scales in 8-group blocks; everything
// double-buffered and XOR-swizzled in 16-byte chunks).  A step is one scale group of 64 (or
// half of a group of 128, whose scale then multiplies each half: w = scale_g * b, model card
// "Binary Weight Representation: 1-bit g128").  A 64-byte weight block holds 4 ternary or 8
// binary steps of a row.
//
// K order inside a step, chosen for gfx950's LDS: a 16-byte read (ds_read_b128) runs at full
// rate only if lanes l and l + 16 read the same 32-byte block (equal 16-byte chunks, or chunks
// that differ in bit 0); chunks two or four apart cost a second pass (measured with the LDS
// bank-conflict counter).  So in MFMA j of a step, lane quarter q takes the eight codes of
// chunk phi(q, j) = 4 (q >> 1) + (q & 1) + 2 j of the step, and quarters 0/1 and 2/3 read
// neighbouring chunks of each activation row.  Its codes are then the low (q even) or high
// (q odd) halves of two consecutive ternary words (codes 32 (q >> 1) + 16 i + 8 (q & 1) ..),
// or bytes (q & 1) and (q & 1) + 2 of binary word q >> 1; one 8-byte read of the row's step
// words and one byte permute gather them.  4-bit codes (8 per word) make each chunk one word:
// the lane reads words phi(q, 0) and phi(q, 0) + 2 of the step (one two-dword LDS read).
#include "lowbit_device.h"
#include "lowbit_internal.h"

namespace lowbit {
namespace {

constexpr int KS = 64;                 // K elements per step
constexpr int kRowBytes = KS * 2;      // one bf16 row of an X tile per step
constexpr int kXChunks = kRowBytes / 16;
constexpr int kWB = 64;                // packed bytes per weight row and block
constexpr int kSGpb = 8;               // scale groups per scale block

__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ int x_off(int row, int chunk) { return row * kRowBytes + ((chunk ^ lds_swizzle(row)) << 4); }

// Chunk c of weight row r within a block sits at position c ^ ((r >> 2) & 3): the 16 rows one
// 8-byte operand read touches land in 16 different 16-byte bank groups.
__device__ __forceinline__ int w_pos(int row, int chunk) { return chunk ^ ((row >> 2) & 3); }

template <int G, int BITS, int BM, int BN, int WAVES_M, int WAVES_N>
struct Cfg16 {
    static constexpr int WAVES = WAVES_M * WAVES_N;  // of one K group
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    static constexpr int MB = WM / 16, NB = WN / 16;
    static constexpr int X_TILE = BM * kRowBytes;
    static constexpr int X_SLOTS = BM * kXChunks;            // 16-byte copies per step
    static constexpr int W_BLOCK = BN * kWB;
    static constexpr int W_SLOTS = BN * (kWB / 16);
    static constexpr int S_BLOCK = BN * 32;                  // two aligned 16-byte windows per row
    static constexpr int S_SLOTS = BN * 2;
    static_assert(WM % 16 == 0 && WN % 16 == 0 && MB >= 1 && NB >= 1, "wave tile");
    static_assert(THREADS % kXChunks == 0, "a thread copies one chunk column of X");
    static constexpr int W_STEP = KS * BITS / 8;             // packed bytes per row and step
    static constexpr int W_SPB = kWB / W_STEP;               // steps per weight block
    static_assert(G == 64 || G == 128, "scale groups of 64 or 128");
    static_assert(BITS == 1 || BITS == 2 || BITS == 4, "binary, ternary or 4-bit codes");
};

// EPI = kEpiSwiglu: the problem's W and S hold 2N rows, gate rows [0, N) then up rows [N, 2N), and
// Y[M, N] = silu(X . Wgate^T) * (X . Wup^T), both factors taken from the fp32 sums and rounded to
// bf16 once.  A wave's two 16-column blocks are then the gate and the up rows of the same 16
// output columns, so the epilogue combines them in registers; a BN-row weight tile makes BN / 2
// output columns.  EPI = kEpiResidual: Y = R + gate[n] * (X . W^T) in fp32, rounded once (Y may
// be R: every element is read and written by the same lane).
// AFFINE (4-bit codes only): the nibbles are unsigned levels q of affine groups, w = s * q + b with
// an fp16 scale S and an fp16 bias B per group (the 4-bit text encoder's bits = 4, group_size = 64
// quantisation of the mlx guide's component architecture).  Per group the output gains
// b * (sum of the group's activations); that row sum comes from one MFMA pair against an all-ones
// operand per row block (exact products, fp32 sums, in the accumulator layout), shared by the
// wave's column blocks, and enters with one more fp32 FMA per output and group.
// XSPLIT: K split across `sk.splits` workgroups per tile (workgroup b runs split b / tiles of tile
// b % tiles), for grids that leave compute units idle.  Each split's workgroup stores its fp32 sums
// in the caller's workspace and counts itself in on the tile's counter; the last to arrive adds the
// splits' sums in split order 0, 1, ... (a fixed order: the result does not depend on timing),
// resets the counter and runs the epilogue.
struct SplitK {
    float* ws;            // [tiles][splits][waves][MB * NB][64 lanes][4] fp32 sums
    uint32_t* counters;   // [tiles], zero between calls
    int splits;
};

template <int G, int BITS, int BM, int BN, int WAVES_M, int WAVES_N, int KSPLIT, int EPI = kEpiPlain,
          bool AFFINE = false, bool XSPLIT = false>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N * KSPLIT, 1) void gemm_tile16_kernel(ProblemGroup grp, SplitK sk) {
    constexpr bool SWIGLU = EPI == kEpiSwiglu;
    static_assert(!AFFINE || (BITS == 4 && EPI == kEpiPlain), "affine groups: 4-bit levels, plain epilogue");
    using C = Cfg16<G, BITS, BM, BN, WAVES_M, WAVES_N>;
    constexpr int kWSpb = C::W_SPB;
    static_assert(KSPLIT == 1 || (KSPLIT == 2 && C::WAVES == 4), "K groups of 4 waves, two of them");
    static_assert(!SWIGLU || (C::NB == 2 && KSPLIT == 1), "gate and up block per wave");
    constexpr int kOutBn = SWIGLU ? BN / 2 : BN;  // output columns per tile
    // One set of buffers per K group.  Separate static arrays per buffer role (not one array
    // indexed by parity): the compiler can then see that reads of one buffer do not depend on
    // copies still landing in the other.
    __shared__ __attribute__((aligned(16))) unsigned char xa0_[KSPLIT][C::X_TILE];
    __shared__ __attribute__((aligned(16))) unsigned char xa1_[KSPLIT][C::X_TILE];
    __shared__ __attribute__((aligned(16))) unsigned char wk0_[KSPLIT][C::W_BLOCK];
    __shared__ __attribute__((aligned(16))) unsigned char wk1_[KSPLIT][C::W_BLOCK];
    __shared__ __attribute__((aligned(16))) unsigned char sk0_[KSPLIT][C::S_BLOCK];
    __shared__ __attribute__((aligned(16))) unsigned char sk1_[KSPLIT][C::S_BLOCK];
    // affine groups: the bias blocks, laid out as the scale blocks
    constexpr int kBBlock = AFFINE ? C::S_BLOCK : 16;
    __shared__ __attribute__((aligned(16))) unsigned char bk0_[KSPLIT][kBBlock];
    __shared__ __attribute__((aligned(16))) unsigned char bk1_[KSPLIT][kBBlock];

    // K group kg (wave-uniform) and the thread's index inside it
    const int kg = KSPLIT == 1 ? 0 : __builtin_amdgcn_readfirstlane(int(threadIdx.x) / C::THREADS);
    unsigned char* const xa0 = xa0_[kg];
    unsigned char* const xa1 = xa1_[kg];
    unsigned char* const wk0 = wk0_[kg];
    unsigned char* const wk1 = wk1_[kg];
    unsigned char* const sk0 = sk0_[kg];
    unsigned char* const sk1 = sk1_[kg];
    unsigned char* const bk0 = bk0_[kg];
    unsigned char* const bk1 = bk1_[kg];
    const int tid = int(threadIdx.x) - kg * C::THREADS;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int wave_m = wave % WAVES_M, wave_n = wave / WAVES_M;
    const int q = lane >> 4, l16 = lane & 15;

    // ---- the tile of virtual workgroup id vt: its problem, origin, K range and copy sources ----
    struct TileCtx {
        GemmProblem p;
        int M, N, K, m0, n0, kbeg, kend;
        uint32_t w_row_bytes, s_row_bytes, x_voff, x_row_step, x_tile_bytes;
        const unsigned char* x_tile;
        __amdgpu_buffer_rsrc_t w_rs, s_rs, b_rs;
    };
    // X: thread copies chunk position tid % 8 of rows tid / 8 + i * (THREADS / 8)
    constexpr int kRowsPerRound = C::THREADS / kXChunks;
    const int r_first = tid / kXChunks;
    const int total_tiles = grp.tile_end[grp.count - 1];
    auto tile_ctx = [&](int vt) __attribute__((always_inline)) {
        TileCtx c;
        const int t = xcd_remap(vt, total_tiles);
        int pi = 0;
        while (pi + 1 < grp.count && t >= grp.tile_end[pi]) ++pi;
        c.p = grp.p[pi];
        const int tile = t - (pi > 0 ? grp.tile_end[pi - 1] : 0);
        c.M = c.p.M;
        c.N = c.p.N;
        c.K = c.p.K;
        const int tiles_n = (c.N + kOutBn - 1) / kOutBn;
        c.m0 = (tile / tiles_n) * BM;
        c.n0 = (tile % tiles_n) * kOutBn;
        // the group's steps [kbeg, kend); every group has the same count (the host sends
        // KSPLIT = 2 only for an even step count), so all run the same barriers
        const int ksteps = c.K / KS;
        if constexpr (XSPLIT) {
            const int sp = int(blockIdx.x) / total_tiles;
            c.kbeg = sp * ksteps / sk.splits;
            c.kend = (sp + 1) * ksteps / sk.splits;
        } else {
            c.kbeg = kg * (ksteps / KSPLIT);
            c.kend = c.kbeg + ksteps / KSPLIT;
        }
        c.w_row_bytes = uint32_t(c.K) * BITS / 8u;
        c.s_row_bytes = uint32_t(c.K / G) * 2u;
        c.x_voff = uint32_t(r_first) * uint32_t(c.K) * 2u + uint32_t((tid % kXChunks) ^ lds_swizzle(r_first)) * 16u;
        c.x_row_step = uint32_t(kRowsPerRound) * uint32_t(c.K) * 2u;
        c.x_tile = reinterpret_cast<const unsigned char*>(c.p.X) + size_t(c.m0) * size_t(c.K) * 2;
        c.x_tile_bytes = uint32_t(c.M - c.m0 < BM ? c.M - c.m0 : BM) * uint32_t(c.K) * 2u;
        const uint32_t w_rows = uint32_t(SWIGLU ? 2 * c.N : c.N);
        c.w_rs = make_rsrc(c.p.W, w_rows * c.w_row_bytes);
        c.s_rs = make_rsrc(c.p.S, w_rows * c.s_row_bytes);
        c.b_rs = make_rsrc(AFFINE ? c.p.B : c.p.S, w_rows * c.s_row_bytes);
        return c;
    };
    // Global weight row of the tile's weight row r (rows past the last output column re-read a
    // valid row; their results are not stored).  SwiGLU: row r = 32 w + 16 h + i is output
    // column n0 + 16 w + i, of the gate (h = 0) or the up (h = 1) half.
    auto wrow_of = [&](const TileCtx& c, int r) __attribute__((always_inline)) {
        if constexpr (SWIGLU) {
            const int col = c.n0 + 16 * (r >> 5) + (r & 15);
            return (col < c.N ? col : c.N - 1) + ((r >> 4) & 1) * c.N;
        } else {
            const int n = c.n0 + r;
            return n < c.N ? n : c.N - 1;
        }
    };
    auto issue_x_of = [&](const TileCtx& c, int step, unsigned char* buf) __attribute__((always_inline)) {
        const uint32_t kb = uint32_t(step) * KS * 2u;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(c.x_tile + kb, c.x_tile_bytes - kb);
#pragma unroll
        for (int i = 0; i < (C::X_SLOTS + C::THREADS - 1) / C::THREADS; ++i) {
            if (i * C::THREADS + wave_u * 64 < C::X_SLOTS)
                dma16(rs, buf + (i * C::THREADS + wave_u * 64) * 16, c.x_voff + uint32_t(i) * c.x_row_step, 0);
        }
    };
    // packed weights: block b = steps [b W_SPB, (b+1) W_SPB) of the tile's BN rows, 64 bytes per
    // row.  Copy slot s = row s / 4, stored position s % 4 (holding source chunk w_pos(row, s % 4)).
    auto issue_w_of = [&](const TileCtx& c, int block, unsigned char* buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < (C::W_SLOTS + C::THREADS - 1) / C::THREADS; ++i) {
            const int slot0 = i * C::THREADS + wave_u * 64;
            if (slot0 < C::W_SLOTS) {
                const int slot = slot0 + lane;
                const int r = slot >> 2;
                const int n = wrow_of(c, r);
                const uint32_t voff = uint32_t(n) * c.w_row_bytes + uint32_t(w_pos(r, slot & 3) * 16);
                dma16(c.w_rs, buf + slot0 * 16, voff, __builtin_amdgcn_readfirstlane(block * kWB));
            }
        }
    };
    // scales: block b = groups [8b, 8b+8) of the tile's BN rows, as two aligned 16-byte windows
    // per row; the row's group 8b sits (row offset & 15) bytes in.  Affine: the bias block alike
    // into `bbuf`.
    auto issue_s_of = [&](const TileCtx& c, int block, unsigned char* buf, unsigned char* bbuf)
                          __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < (C::S_SLOTS + C::THREADS - 1) / C::THREADS; ++i) {
            const int slot0 = i * C::THREADS + wave_u * 64;
            if (slot0 < C::S_SLOTS) {
                const int slot = slot0 + lane;
                const int r = slot >> 1;
                const int n = wrow_of(c, r);
                const uint32_t start = uint32_t(n) * c.s_row_bytes + uint32_t(block) * 16u;
                const uint32_t voff = (start & ~15u) + uint32_t(slot & 1) * 16u;
                dma16(c.s_rs, buf + slot0 * 16, voff, 0);
                if constexpr (AFFINE) dma16(c.b_rs, bbuf + slot0 * 16, voff, 0);
            }
        }
    };
    auto s_block = [&](int step) __attribute__((always_inline)) { return (step * KS / G) / kSGpb; };
    // the first step's X, weight and scale blocks of a tile
    auto issue_first = [&](const TileCtx& c) __attribute__((always_inline)) {
        const int wb = c.kbeg / kWSpb, sb = s_block(c.kbeg);
        issue_x_of(c, c.kbeg, xa0);
        issue_w_of(c, wb, (wb & 1) ? wk1 : wk0);
        issue_s_of(c, sb, (sb & 1) ? sk1 : sk0, (sb & 1) ? bk1 : bk0);
    };

    // Tiles: workgroup b runs the tiles of virtual ids b, b + grid, ...  A persistent launch
    // (grid below the tile count, a multiple of the 8 XCDs, so that every virtual id keeps its
    // workgroup's XCD and xcd_remap's tile order) saves the next workgroup's launch on the
    // compute unit, and the next tile's first copies go out before this tile's epilogue.
    static_assert(!XSPLIT || (KSPLIT == 1 && !SWIGLU), "K split across workgroups: one K group, plain epilogue");
    int vt = XSPLIT ? int(blockIdx.x) % total_tiles : int(blockIdx.x);
    TileCtx cur = tile_ctx(vt);
    issue_first(cur);
#pragma nounroll
    for (;;) {
        const GemmProblem p = cur.p;
        const int M = cur.M, N = cur.N, K = cur.K;
        const int m0 = cur.m0, n0 = cur.n0;
        auto wrow = [&](int r) __attribute__((always_inline)) { return wrow_of(cur, r); };
        const int wm0 = wave_m * C::WM, wn0 = wave_n * C::WN;

        const int kgroups = K / G;
        const int ksteps = K / KS;
        const int kbeg = cur.kbeg, kend = cur.kend;
        const uint32_t s_row_bytes = cur.s_row_bytes;
        auto issue_x = [&](int step, unsigned char* buf) __attribute__((always_inline)) { issue_x_of(cur, step, buf); };
        auto issue_w = [&](int block, unsigned char* buf) __attribute__((always_inline)) { issue_w_of(cur, block, buf); };
        auto issue_s = [&](int block, unsigned char* buf, unsigned char* bbuf) __attribute__((always_inline)) {
            issue_s_of(cur, block, buf, bbuf);
        };

        // Per-lane LDS offsets: weight row of each column block (ternary: the lane's word pair of
        // a step chunk; binary: the step's two words), its scale window.  The byte permute that
        // gathers the lane's 16 codes from the two words: ternary halves (q & 1) of both words,
        // binary bytes (q & 1) and (q & 1) + 2 of word q >> 1.
        const uint32_t gather_sel =
            BITS == 2 ? ((q & 1) ? 0x07060302u : 0x05040100u)
                      : 0x0C0C0000u | (uint32_t(4 * (q >> 1) + (q & 1) + 2) << 8) | uint32_t(4 * (q >> 1) + (q & 1));
        const uint32_t two_pair = opaque_two_pair();
        int w_rd[C::NB], s_rd[C::NB];
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
            const int r = wn0 + nb * 16 + l16;
            const int n = wrow(r);
            w_rd[nb] = r * kWB + (BITS == 2 ? 8 * (q >> 1) : 0);
            s_rd[nb] = r * 32 + int((uint32_t(n) * s_row_bytes) & 15u);
        }

        static_assert(C::WM % 16 == 0, "row blocks start at multiples of 16");
        int x_rd[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) x_rd[j] = x_off(wm0 + l16, 4 * (q >> 1) + (q & 1) + 2 * j);

        f32x4_t acc[C::MB][C::NB];
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        // A step's words and scales are read from LDS before any copy of the step is issued (the
        // compiler cannot tell which of the two buffers a step reads).
        struct Ops {
            u32x2_t w[C::NB];
            float sc[C::NB];
            float bs[AFFINE ? C::NB : 1];  // affine: the group's bias
        };
        auto read_operands = [&](const unsigned char* wt, const unsigned char* st, const unsigned char* bt, int step,
                                 Ops& o) __attribute__((always_inline)) {
            const int wj = step % kWSpb;
            const int grp_in_block = (step * KS / G) & (kSGpb - 1);
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb) {
                const int r = wn0 + nb * 16 + l16;
                if constexpr (BITS == 4) {
                    // words phi(q, 0) and phi(q, 1) = phi(q, 0) + 2 of the step: dwords q & 1 and
                    // (q & 1) + 2 of the step's 16-byte chunk q >> 1
                    const int byte0 = wj * C::W_STEP + 16 * (q >> 1);
                    const unsigned char* b = wt + w_rd[nb] + (w_pos(r, byte0 >> 4) << 4) + 4 * (q & 1);
                    o.w[nb] = u32x2_t{*reinterpret_cast<const uint32_t*>(b), *reinterpret_cast<const uint32_t*>(b + 8)};
                } else {
                    const int byte0 = wj * C::W_STEP;  // the step's bytes within the block row
                    o.w[nb] = *reinterpret_cast<const u32x2_t*>(wt + w_rd[nb] + (w_pos(r, byte0 >> 4) << 4) + (byte0 & 15));
                }
                // x 1/2 (ternary: the operand holds 2c), x -1/2 (binary: -2c) or x 1/16 (4-bit: 16c).  Also keeps the
                // conversion out of the FMA (an fp16 operand makes it v_fma_mix_f32, whose result
                // does not share the accumulator's register and doubles the accumulator registers
                // across the unrolled steps).
                o.sc[nb] = half_bits_to_float(*reinterpret_cast<const uint16_t*>(st + s_rd[nb] + grp_in_block * 2)) *
                           (BITS == 2 ? 0.5f : BITS == 4 ? 0.0625f : -0.5f);
                if constexpr (AFFINE)
                    o.bs[nb] = half_bits_to_float(*reinterpret_cast<const uint16_t*>(bt + s_rd[nb] + grp_in_block * 2));
            }
        };

        // `issue` runs after the first row block's MFMAs: the next step's copies go out once the
        // step's first operand reads, expansion and MFMAs are under way, not in a burst with them
        // right after the barrier (measured 3% faster on the 4608-row denoise shapes).
        auto compute = [&](const unsigned char* xt, const Ops& o, auto&& issue) __attribute__((always_inline)) {
            // Codes of column block nb are expanded just before its first MFMA pair (row block 0),
            // behind a scheduling fence: the expansion of block nb + 1 then runs while the matrix
            // core works on block nb, instead of every wave of a SIMD expanding all its codes
            // right after the step's barrier while the matrix core idles.
            u32x4_t bfr[C::NB][2];
            auto expand = [&](int nb) __attribute__((always_inline)) {
                uint32_t d[8];
                if constexpr (AFFINE) {
                    expand_u4_word(o.w[nb][0], d);
                    expand_u4_word(o.w[nb][1], d + 4);
                } else if constexpr (BITS == 4) {
                    expand_int4_word(o.w[nb][0], d);
                    expand_int4_word(o.w[nb][1], d + 4);
                } else {
                    const uint32_t codes = perm_b32(o.w[nb][1], o.w[nb][0], gather_sel);
                    if constexpr (BITS == 2)
                        expand_ternary_word(codes, d);
                    else
                        expand_binary_16(codes, two_pair, d);
                }
                bfr[nb][0] = u32x4_t{d[0], d[1], d[2], d[3]};
                bfr[nb][1] = u32x4_t{d[4], d[5], d[6], d[7]};
            };
            // Row blocks in order; within one, the MFMA pair of block (mb, nb) is issued before the
            // scale FMAs of the previous block, which use the other partial-sum registers.  The
            // activation operands of row block mb + 1 are read while row block mb computes.  Row
            // blocks start at multiples of 16, so the swizzle of row wm0 + 16 mb + l16 does not
            // depend on mb: one base address per chunk, the row block as an immediate offset.
            f32x4_t tmp[2];
            bf16x8_t afr[2][2];  // [row block parity][k half]
            // affine: the row block's activation sums over the step (rows 4q + i in lane (q, l16),
            // every column alike), from an MFMA pair against an all-ones operand
            f32x4_t rsum[2];
            const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
#pragma unroll
            for (int j = 0; j < 2; ++j) afr[0][j] = *reinterpret_cast<const bf16x8_t*>(xt + x_rd[j]);
            int pb = -1;  // previous block, its partial sum in tmp[pb & 1]
#pragma unroll
            for (int mb = 0; mb < C::MB; ++mb) {
                if (mb == (C::MB > 1 ? 1 : 0)) issue();
                if (mb + 1 < C::MB) {
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        afr[(mb + 1) & 1][j] = *reinterpret_cast<const bf16x8_t*>(xt + x_rd[j] + (mb + 1) * 16 * kRowBytes);
                }
                if constexpr (AFFINE) {
                    f32x4_t r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[mb & 1][j], ones, r, 0, 0, 0);
                    rsum[mb & 1] = r;
                }
#pragma unroll
                for (int nb = 0; nb < C::NB; ++nb) {
                    const int b = mb * C::NB + nb;
                    if (mb == 0) expand(nb);
                    f32x4_t v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        v = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[mb & 1][j],
                                                                    __builtin_bit_cast(bf16x8_t, bfr[nb][j]), v, 0,
                                                                    0, 0);
                    if (mb == 0) __builtin_amdgcn_sched_barrier(0);
                    tmp[b & 1] = v;
                    if (pb >= 0) {
                        const int pm = pb / C::NB, pn = pb % C::NB;
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            acc[pm][pn][i] = __builtin_fmaf(o.sc[pn], tmp[pb & 1][i], acc[pm][pn][i]);
                        if constexpr (AFFINE) {
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                acc[pm][pn][i] = __builtin_fmaf(o.bs[pn], rsum[pm & 1][i], acc[pm][pn][i]);
                        }
                    }
                    pb = b;
                }
            }
            {
                const int pm = pb / C::NB, pn = pb % C::NB;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[pm][pn][i] = __builtin_fmaf(o.sc[pn], tmp[pb & 1][i], acc[pm][pn][i]);
                if constexpr (AFFINE) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[pm][pn][i] = __builtin_fmaf(o.bs[pn], rsum[pm & 1][i], acc[pm][pn][i]);
                }
            }
            // An empty side-effecting use of every accumulator closes the step: otherwise the
            // compiler sinks this step's scale FMAs past the barrier into the next step's first
            // block, and all partial sums of the step stay live at once.
#pragma unroll
            for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < C::NB; ++nb) asm volatile("" ::"v"(acc[mb][nb]));
        };

        auto w_buf = [&](int step) __attribute__((always_inline)) -> unsigned char* {
            return ((step / kWSpb) & 1) ? wk1 : wk0;
        };
        auto s_buf = [&](int step) __attribute__((always_inline)) -> unsigned char* {
            return (s_block(step) & 1) ? sk1 : sk0;
        };
        auto b_buf = [&](int step) __attribute__((always_inline)) -> unsigned char* {
            return (s_block(step) & 1) ? bk1 : bk0;
        };
        const int w_blocks = (ksteps + kWSpb - 1) / kWSpb;
        const int s_blocks = (kgroups + kSGpb - 1) / kSGpb;

        auto prefetch_x = [&](int step, unsigned char* xbuf) __attribute__((always_inline)) {
            if (step + 1 < kend) issue_x(step + 1, xbuf);
        };
        // The next weight (scale) block is copied on the first step of a block and on the group's
        // first step, which can fall inside a block.
        auto prefetch_blocks = [&](int step) __attribute__((always_inline)) {
            const int wb = step / kWSpb;
            if ((step == kbeg || step % kWSpb == 0) && wb + 1 < w_blocks && (wb + 1) * kWSpb < kend)
                issue_w(wb + 1, ((wb + 1) & 1) ? wk1 : wk0);
            const int sb = s_block(step);
            if ((step == kbeg || s_block(step - 1) != sb) && sb + 1 < s_blocks && s_block(kend - 1) > sb) {
                if constexpr (AFFINE)
                    issue_s(sb + 1, ((sb + 1) & 1) ? sk1 : sk0, ((sb + 1) & 1) ? bk1 : bk0);
                else
                    issue_s(sb + 1, ((sb + 1) & 1) ? sk1 : sk0, nullptr);
            }
        };

        wait_vmcnt0();
        __syncthreads();

        // Steps in pairs (static LDS buffers, so the compiler's wait insertion stays exact) with a
        // single loop exit; an odd last step runs after the loop.  A break between the two steps
        // of an iteration made the register allocator give every accumulator a second register
        // and copy it back each iteration.
        Ops ops;
        int step = kbeg;
#pragma nounroll
        for (; step + 1 < kend; step += 2) {
            read_operands(w_buf(step), s_buf(step), AFFINE ? b_buf(step) : nullptr, step, ops);
            compute(xa0, ops, [&]() __attribute__((always_inline)) {
                prefetch_x(step, xa1);
                prefetch_blocks(step);
            });
            wait_vmcnt0();
            __syncthreads();
            read_operands(w_buf(step + 1), s_buf(step + 1), AFFINE ? b_buf(step + 1) : nullptr, step + 1, ops);
            compute(xa1, ops, [&]() __attribute__((always_inline)) {
                prefetch_x(step + 1, xa0);
                prefetch_blocks(step + 1);
            });
            wait_vmcnt0();
            __syncthreads();
        }
        if (step < kend) {
            read_operands(w_buf(step), s_buf(step), AFFINE ? b_buf(step) : nullptr, step, ops);
            compute(xa0, ops, []() {});
        }

        // ---- K groups: group 1's sums through LDS, added to group 0's (order 0, 1) ----
        if constexpr (KSPLIT == 2) {
            __syncthreads();  // every read of the last step is done: the buffers are free
            // A wave's sums (MB x NB blocks of 64 lanes x 16 bytes, 18 KB at 96 x 48) go to the
            // wave's buffer role (wave 0: X buffer 0, 1: X buffer 1, 2 and 3: weight buffers 0 and 1)
            // of both sets: blocks [0, kPer) into group 0's, the rest into group 1's.
            constexpr int kPer = C::X_TILE / 1024;
            static_assert(C::X_TILE == C::W_BLOCK && C::MB * C::NB <= 2 * kPer, "a wave's sums fit two buffers");
            unsigned char* const r0 = wave_u == 0 ? xa0_[0] : wave_u == 1 ? xa1_[0] : wave_u == 2 ? wk0_[0] : wk1_[0];
            unsigned char* const r1 = wave_u == 0 ? xa0_[1] : wave_u == 1 ? xa1_[1] : wave_u == 2 ? wk0_[1] : wk1_[1];
            auto slot = [&](int b) __attribute__((always_inline)) {
                return reinterpret_cast<f32x4_t*>(b < kPer ? r0 + 1024 * b : r1 + 1024 * (b - kPer)) + lane;
            };
            if (kg == 1) {
#pragma unroll
                for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
                    for (int nb = 0; nb < C::NB; ++nb) *slot(mb * C::NB + nb) = acc[mb][nb];
            }
            __syncthreads();
            if (kg == 1) return;
#pragma unroll
            for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < C::NB; ++nb) {
                    const f32x4_t u = *slot(mb * C::NB + nb);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[mb][nb][i] += u[i];
                }
        }

        // ---- the next tile's first copies, once every wave is done with this tile's buffers ----
        const int vn = vt + int(gridDim.x);
        const bool more = KSPLIT == 1 && !XSPLIT && vn < total_tiles;
        TileCtx nxt;
        if (more) {
            nxt = tile_ctx(vn);
            __syncthreads();
            issue_first(nxt);
        }

        // ---- K split across workgroups: this split's sums to the workspace, the last one adds ----
        // (16-byte loads and stores with the sc1 cache policy: through to the device-coherent
        // level, since the L2 of one XCD is not coherent with the others; the stores complete
        // before the arrival is counted)
        if constexpr (XSPLIT) {
            constexpr int kSc1 = 16;
            constexpr int kBlocks = C::MB * C::NB;
            const int t = xcd_remap(vt, total_tiles);
            const int sp = int(blockIdx.x) / total_tiles;
            const uint32_t wave_bytes = uint32_t(kBlocks) * 1024u;
            const uint32_t tile_bytes = uint32_t(sk.splits) * uint32_t(C::WAVES) * wave_bytes;
            const __amdgpu_buffer_rsrc_t ws_rs = make_rsrc(sk.ws, uint32_t(total_tiles) * tile_bytes);
            const uint32_t mine = uint32_t(t) * tile_bytes + (uint32_t(sp) * uint32_t(C::WAVES) + uint32_t(wave)) * wave_bytes +
                                  16u * uint32_t(lane);
#pragma unroll
            for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < C::NB; ++nb)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, acc[mb][nb]), ws_rs,
                                                           mine + uint32_t(mb * C::NB + nb) * 1024u, 0, kSc1);
            wait_vmcnt0();
            __syncthreads();
            __shared__ int last_split;
            if (threadIdx.x == 0)
                last_split = __hip_atomic_fetch_add(&sk.counters[t], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                             uint32_t(sk.splits - 1);
            __syncthreads();
            if (!last_split) return;
            // every split's sums, split by split, added in split order
            const uint32_t first = uint32_t(t) * tile_bytes + uint32_t(wave) * wave_bytes + 16u * uint32_t(lane);
#pragma unroll
            for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < C::NB; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            for (int s2 = 0; s2 < sk.splits; ++s2) {
                u32x4_t part[kBlocks];
                const uint32_t src = first + uint32_t(s2) * uint32_t(C::WAVES) * wave_bytes;
#pragma unroll
                for (int b = 0; b < kBlocks; ++b)
                    part[b] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ws_rs, src + uint32_t(b) * 1024u,
                                                                                              0, kSc1));
#pragma unroll
                for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
                    for (int nb = 0; nb < C::NB; ++nb) {
                        const f32x4_t f = __builtin_bit_cast(f32x4_t, part[mb * C::NB + nb]);
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[mb][nb][i] += f[i];
                    }
            }
            if (threadIdx.x == 0) __hip_atomic_store(&sk.counters[t], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }

        // ---- epilogue ----
        // 16x16 block layout: lane (q, l16) holds column l16, rows 4q + i.  A 4x4 transpose inside
        // each group of four lanes l16 = 4a + b (two DPP quad permutes and byte permutes of bf16
        // pairs) gives lane (q, 4a + b) row 4q + b, columns 4a .. 4a + 3: one 8-byte store instead
        // of four 2-byte ones.
        //   stage 1, lanes b <-> b ^ 2: lanes b < 2 keep rows (0, 1) of their column and take rows
        //            (0, 1) of column b + 2; lanes b >= 2 keep rows (2, 3) and take column b - 2's.
        //            E = column b & 1, F = column (b & 1) + 2, both for the lane's row pair.
        //   stage 2, lanes b <-> b ^ 1: even lanes keep the first row of the pair, odd lanes the
        //            second; each sends the partner the halves it needs.
        const int b4 = l16 & 3;
        const bool lower_pair = b4 < 2, odd = (b4 & 1) != 0;
        const uint32_t send_sel = odd ? 0x05040100u : 0x07060302u;   // (E.lo, F.lo) : (E.hi, F.hi)
        const uint32_t d0_sel = odd ? 0x03020504u : 0x05040100u;     // (R.lo, E.hi) : (E.lo, R.lo)
        const uint32_t d1_sel = odd ? 0x03020706u : 0x07060100u;     // (R.hi, F.hi) : (F.lo, R.hi)
        constexpr int kQuadSwap2 = 0x4E;  // quad_perm [2, 3, 0, 1]
        constexpr int kQuadSwap1 = 0xB1;  // quad_perm [1, 0, 3, 2]
        auto pack = [](float lo, float hi) __attribute__((always_inline)) {
            return uint32_t(float_to_bf16_bits(lo)) | (uint32_t(float_to_bf16_bits(hi)) << 16);
        };
        // one 16x16 block of fp32 results to bf16 at columns nblk .. nblk + 15 of row block mb
        auto store_block = [&](f32x4_t a, int nblk, int mb) __attribute__((always_inline)) {
            if (nblk >= N) return;  // N % 16 == 0: a block is in or out as a whole
            if constexpr (EPI == kEpiResidual) {
                // lane (q, l16) holds column nblk + l16 of rows 4q + i: the gated residual update
                const int col = nblk + l16;
                const float gt = static_cast<float>(__builtin_bit_cast(__bf16, p.gate[col]));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = m0 + wm0 + mb * 16 + 4 * q + i;
                    const float r = m < M ? static_cast<float>(__builtin_bit_cast(__bf16, p.R[int64_t(m) * N + col])) : 0.f;
                    a[i] = __builtin_fmaf(gt, a[i], r);
                }
            }
            const uint32_t P = pack(a[0], a[1]);  // rows 0, 1 of column b4
            const uint32_t Q = pack(a[2], a[3]);  // rows 2, 3
            const uint32_t own = lower_pair ? P : Q;
            const uint32_t got =
                uint32_t(__builtin_amdgcn_update_dpp(0, int(lower_pair ? Q : P), kQuadSwap2, 0xF, 0xF, true));
            const uint32_t E = lower_pair ? own : got, F = lower_pair ? got : own;
            const uint32_t R =
                uint32_t(__builtin_amdgcn_update_dpp(0, int(perm_b32(F, E, send_sel)), kQuadSwap1, 0xF, 0xF, true));
            const uint32_t d0 = perm_b32(R, E, d0_sel), d1 = perm_b32(R, F, d1_sel);
            const int m = m0 + wm0 + mb * 16 + 4 * q + b4;
            if (m < M) {
                *reinterpret_cast<u32x2_t*>(p.Y + int64_t(m) * N + nblk + (l16 & ~3)) = u32x2_t{d0, d1};
            }
        };
#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) {
            if constexpr (SWIGLU) {
                // silu(g) * u = g * u / (1 + exp(-g)); exp overflows to inf for very negative g and
                // the quotient goes to -0, the limit
                f32x4_t y;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float gt = acc[mb][0][i];
                    y[i] = gt * acc[mb][1][i] / (1.0f + __expf(-gt));
                }
                store_block(y, n0 + 16 * wave_n, mb);
            } else {
#pragma unroll
                for (int nb = 0; nb < C::NB; ++nb) store_block(acc[mb][nb], n0 + wn0 + nb * 16, mb);
            }
        }
        if (!more) break;
        cur = nxt;
        vt = vn;
    }
}

template <int G, int BITS, int BM, int BN, int WAVES_M, int WAVES_N, int KSPLIT = 1, int EPI = kEpiPlain,
          bool AFFINE = false, bool XSPLIT = false>
hipError_t launch_cfg16(const GemmProblem* probs, int count, hipStream_t stream, SplitK sk = SplitK{}) {
    ProblemGroup grp{};
    int total = 0;
    constexpr int kOutBn = EPI == kEpiSwiglu ? BN / 2 : BN;
    for (int i = 0; i < count; ++i) {
        grp.p[i] = probs[i];
        total += int(tiles_of(probs[i].M, BM) * tiles_of(probs[i].N, kOutBn));
        grp.tile_end[i] = total;
    }
    grp.count = count;
    // A tile whose LDS admits one workgroup per compute unit runs persistent: at most one
    // workgroup per compute unit, each looping over its tiles.
    using Cf = Cfg16<G, BITS, BM, BN, WAVES_M, WAVES_N>;
    constexpr int kLds = KSPLIT * 2 * (Cf::X_TILE + Cf::W_BLOCK + Cf::S_BLOCK + (AFFINE ? Cf::S_BLOCK : 16));
    constexpr bool kPersistent = KSPLIT == 1 && kLds > 80 * 1024;
    const int grid = XSPLIT ? total * sk.splits : kPersistent && total > kComputeUnits ? kComputeUnits : total;
    hipLaunchKernelGGL((gemm_tile16_kernel<G, BITS, BM, BN, WAVES_M, WAVES_N, KSPLIT, EPI, AFFINE, XSPLIT>), dim3(grid),
                       dim3(64 * WAVES_M * WAVES_N * KSPLIT), 0, stream, grp, sk);
    const hipError_t e = hipGetLastError();
    if (e == hipSuccess && trace_enabled()) {
        char cfg[96];
        snprintf(cfg, sizeof cfg, "%dx%d waves=%dx%dx%d epi=%s%s splits=%d", BM, BN, WAVES_M, WAVES_N, KSPLIT,
                 EPI == kEpiSwiglu ? "swiglu" : EPI == kEpiResidual ? "residual" : "plain", AFFINE ? " affine" : "",
                 XSPLIT ? sk.splits : 1);
        trace_launch("tile16", cfg, G, BITS, probs, count, unsigned(grid), 64u * WAVES_M * WAVES_N * KSPLIT, 0u);
    }
    return e;
}

}  // namespace

bool tile16_supported(int g, int bits) { return (bits == 1 || bits == 2 || bits == 4) && (g == 64 || g == 128); }

template <int G, int BITS, bool AFFINE = false>
hipError_t launch_variant16(const GemmProblem* probs, int count, int variant, hipStream_t stream) {
    // 288 x 192 in 12 waves of 144 x 32: LDS 72 KB (X) + 24 KB (W) + 12 KB (S).  The step is
    // bound by VALU issue (code expansion and scale FMAs next to the MFMAs); 144 x 32 wave tiles
    // expand each code for two waves instead of three (96 x 48), for 1.5x the activation reads:
    // measured 1.8% faster on the 4608-row denoise shapes.
    // 96 x 192 in 4 waves of 96 x 48 (LDS 60 KB): 1536 x 3072 outputs are exactly 256 tiles.
    // With K split between two groups of 4 waves (LDS 120 KB) where every problem has an even
    // number of 64-element steps.
    if constexpr (BITS == 4) {
        // 64 x 128 in two groups of 4 waves of 64 x 32 (LDS 80 KB), K split between the groups
        if (variant == TILE_64x128K2) {
            bool even = true;
            for (int i = 0; i < count; ++i) even = even && (probs[i].K / KS) % 2 == 0;
            if (even) return launch_cfg16<G, BITS, 64, 128, 1, 4, 2, kEpiPlain, AFFINE>(probs, count, stream);
            return launch_cfg16<G, BITS, 64, 128, 1, 4, 1, kEpiPlain, AFFINE>(probs, count, stream);
        }
    }
    if (variant == TILE_96x192K2) {
        bool even = true;
        for (int i = 0; i < count; ++i) even = even && (probs[i].K / KS) % 2 == 0;
        if (even) return launch_cfg16<G, BITS, 96, 192, 1, 4, 2, kEpiPlain, AFFINE>(probs, count, stream);
        return launch_cfg16<G, BITS, 96, 192, 1, 4, 1, kEpiPlain, AFFINE>(probs, count, stream);
    }
    if (variant == TILE_96x192) return launch_cfg16<G, BITS, 96, 192, 1, 4, 1, kEpiPlain, AFFINE>(probs, count, stream);
    if (variant == TILE_256x192) return launch_cfg16<G, BITS, 256, 192, 2, 6, 1, kEpiPlain, AFFINE>(probs, count, stream);
    return launch_cfg16<G, BITS, 288, 192, 2, 6, 1, kEpiPlain, AFFINE>(probs, count, stream);
}

template <int G, int BITS, int EPI>
hipError_t launch_epi16(const GemmProblem* probs, int count, hipStream_t stream) {
    return launch_cfg16<G, BITS, 288, 192, 2, 6, 1, EPI>(probs, count, stream);
}

template <int EPI>
hipError_t launch_epi16_gb(const GemmProblem* probs, int count, int g, int bits, hipStream_t stream) {
    if (bits == 2)
        return g == 64 ? launch_epi16<64, 2, EPI>(probs, count, stream) : launch_epi16<128, 2, EPI>(probs, count, stream);
    if (bits == 4)
        return g == 64 ? launch_epi16<64, 4, EPI>(probs, count, stream) : launch_epi16<128, 4, EPI>(probs, count, stream);
    return g == 64 ? launch_epi16<64, 1, EPI>(probs, count, stream) : launch_epi16<128, 1, EPI>(probs, count, stream);
}

hipError_t launch_gemm_tile16_epilogue(const GemmProblem* probs, int count, int g, int bits, int epi,
                                       hipStream_t stream) {
    if (count < 1 || count > kMaxGroup || !tile16_supported(g, bits)) return hipErrorInvalidValue;
    if (epi == kEpiSwiglu) return launch_epi16_gb<kEpiSwiglu>(probs, count, g, bits, stream);
    if (epi == kEpiResidual) return launch_epi16_gb<kEpiResidual>(probs, count, g, bits, stream);
    return hipErrorInvalidValue;
}

// Affine 4-bit GEMMs whose 64 x 128 tile grid leaves a quarter of the compute units or more idle
// (the text encoder's 512 x 2560 down projection: 160 tiles) split K three ways across workgroups
// through a caller workspace: three 4-wave workgroups of 48 KB LDS share a compute unit, so the
// 480 workgroups run in one round.  0 where no split applies.
constexpr int kAffineSplits = 3;
constexpr size_t kAffineCounterBytes = 4096;  // 1024 tile counters, at the workspace's start
size_t affine_split_bytes(const GemmProblem& p, int g) {
    if (!tile16_supported(g, 4) || pick_tile_variant(&p, 1, g, 4) != TILE_64x128K2) return 0;
    const int64_t tiles = tiles_of(p.M, 64) * tiles_of(p.N, 128);
    if (tiles * 4 > int64_t(kComputeUnits) * 3 || tiles > 1024 || p.K / KS < 8 * kAffineSplits) return 0;
    using Cf = Cfg16<64, 4, 64, 128, 1, 4>;
    return kAffineCounterBytes + size_t(tiles) * kAffineSplits * Cf::WAVES * Cf::MB * Cf::NB * 1024u;
}

size_t affine_workspace_bytes(const GemmProblem& p, int g) { return affine_split_bytes(p, g); }

hipError_t launch_gemm_tile16_affine_ex(const GemmProblem& p, int g, void* workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
    const size_t need = affine_split_bytes(p, g);
    if (need == 0 || workspace == nullptr || workspace_bytes < need) return hipErrorNotSupported;
    SplitK sk{reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + kAffineCounterBytes),
              static_cast<uint32_t*>(workspace), kAffineSplits};
    return g == 64 ? launch_cfg16<64, 4, 64, 128, 1, 4, 1, kEpiPlain, true, true>(&p, 1, stream, sk)
                   : launch_cfg16<128, 4, 64, 128, 1, 4, 1, kEpiPlain, true, true>(&p, 1, stream, sk);
}

hipError_t launch_gemm_tile16_affine(const GemmProblem* probs, int count, int g, int variant, hipStream_t stream) {
    if (count < 1 || count > kMaxGroup || !tile16_supported(g, 4)) return hipErrorInvalidValue;
    if (!is_tile16_variant(variant)) variant = TILE_288x192;
    return g == 64 ? launch_variant16<64, 4, true>(probs, count, variant, stream)
                   : launch_variant16<128, 4, true>(probs, count, variant, stream);
}

hipError_t launch_gemm_tile16_group(const GemmProblem* probs, int count, int g, int bits, int variant,
                                    hipStream_t stream) {
    if (bits == 2)
        return g == 64 ? launch_variant16<64, 2>(probs, count, variant, stream)
                       : launch_variant16<128, 2>(probs, count, variant, stream);
    if (bits == 4)
        return g == 64 ? launch_variant16<64, 4>(probs, count, variant, stream)
                       : launch_variant16<128, 4>(probs, count, variant, stream);
    return g == 64 ? launch_variant16<64, 1>(probs, count, variant, stream)
                   : launch_variant16<128, 1>(probs, count, variant, stream);
}

}  // namespace lowbit

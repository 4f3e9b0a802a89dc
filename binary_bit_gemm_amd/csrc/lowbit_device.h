// Device-side building blocks of the low-bit GEMM kernels (gfx950 only).
//
// Weight codes are expanded in registers into bf16 MFMA operand dwords.  Each dword holds
// two consecutive codes k, k+1 as a bf16 pair (lo half = code k).  The value of a code c is
// written as 2*c (ternary) or -2*c (binary): +-2.0 has a zero low byte (0x4000 / 0xC000),
// so only the high byte of every bf16 has to be produced, and the factor +-1/2 is folded
// exactly into the fp32 group scale that multiplies each group's partial sum after the MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lowbit {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4_t __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2_t __attribute__((__vector_size__(2 * sizeof(uint32_t))));

// v_perm_b32: byte i of the result is byte sel.byte[i] of the 8-byte value {hi:lo}
// (0..3 -> lo, 4..7 -> hi); selector 0x0C yields 0x00.
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// Selector that builds the bf16 pair [0x00, lo.byte[b], 0x00, hi.byte[b]].
__device__ __forceinline__ constexpr uint32_t pair_sel(int b) {
    return 0x0Cu | (uint32_t(b) << 8) | (0x0Cu << 16) | (uint32_t(4 + b) << 24);
}

// Ternary word (16 codes, 2-bit fields 00 -> 0, 01 -> +1, 10 -> -1, 11 -> 0) to 8 operand
// dwords; out[d] = bf16 pair (2*c[2d], 2*c[2d+1]).
//   e_r  = fields r, r+4, r+8, r+12 moved to the low bits of bytes 0..3
//   l_r  = table lookup of each byte: 0 -> 0x00, 1 -> 0x40, 2 -> 0xC0, 3 -> 0x00
//   out  = byte gathers from l_r (codes 4b+r sit in byte b of l_r)
// 8 signed 4-bit codes (two's complement, code i at bits 4i .. 4i+3) -> 8 bf16 of 16 * code;
// out[j] holds codes 2j (low half) and 2j + 1 (high half).  Each code moves to the top nibble
// of a byte, whose signed value is 16 * code; its fp32 conversion is exact, and so is the bf16
// taken as the upper half of that fp32 (16 * code has at most 4 significant bits).
__device__ __forceinline__ void expand_int4_word(uint32_t w, uint32_t out[4]) {
    const uint32_t ev = (w << 4) & 0xF0F0F0F0u;  // codes 0, 2, 4, 6
    const uint32_t od = w & 0xF0F0F0F0u;         // codes 1, 3, 5, 7
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float fe = static_cast<float>(static_cast<int8_t>(ev >> (8 * j)));
        const float fo = static_cast<float>(static_cast<int8_t>(od >> (8 * j)));
        out[j] = perm_b32(__float_as_uint(fo), __float_as_uint(fe), 0x07060302u);
    }
}

// 8 unsigned 4-bit levels (level i at bits 4i .. 4i+3) -> 8 bf16 of 16 * level, paired as in
// expand_int4_word.  Each level moves to the top nibble of a byte, whose unsigned value is
// 16 * level (0 .. 240); its fp32 conversion is exact, and so is the bf16 taken as the upper half
// of that fp32 (at most 4 significant bits).
__device__ __forceinline__ void expand_u4_word(uint32_t w, uint32_t out[4]) {
    const uint32_t ev = (w << 4) & 0xF0F0F0F0u;  // levels 0, 2, 4, 6
    const uint32_t od = w & 0xF0F0F0F0u;         // levels 1, 3, 5, 7
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float fe = static_cast<float>(static_cast<uint8_t>(ev >> (8 * j)));
        const float fo = static_cast<float>(static_cast<uint8_t>(od >> (8 * j)));
        out[j] = perm_b32(__float_as_uint(fo), __float_as_uint(fe), 0x07060302u);
    }
}

__device__ __forceinline__ void expand_ternary_word(uint32_t w, uint32_t out[8]) {
    constexpr uint32_t kHighByte = 0x00C04000u;
    const uint32_t e0 = w & 0x03030303u;
    const uint32_t e1 = (w >> 2) & 0x03030303u;
    const uint32_t e2 = (w >> 4) & 0x03030303u;
    const uint32_t e3 = (w >> 6) & 0x03030303u;
    const uint32_t l0 = perm_b32(kHighByte, kHighByte, e0);
    const uint32_t l1 = perm_b32(kHighByte, kHighByte, e1);
    const uint32_t l2 = perm_b32(kHighByte, kHighByte, e2);
    const uint32_t l3 = perm_b32(kHighByte, kHighByte, e3);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        out[2 * b] = perm_b32(l1, l0, pair_sel(b));
        out[2 * b + 1] = perm_b32(l3, l2, pair_sel(b));
    }
}

// Binary word (32 codes, bit 1 -> +1, bit 0 -> -1) to 16 operand dwords;
// out[d] = bf16 pair (-2*c[2d], -2*c[2d+1]).  NOUT < 16 expands only the low 2*NOUT codes.
//   e_j = byte b holds 0x40 | bit(8b+j) << 7, i.e. +2.0 for bit 0 and -2.0 for bit 1
template <int NOUT = 16>
__device__ __forceinline__ void expand_binary_word(uint32_t w, uint32_t out[NOUT]) {
    uint32_t e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = ((w << (7 - j)) & 0x80808080u) | 0x40404040u;
#pragma unroll
    for (int d = 0; d < NOUT; ++d) {
        const int b = d >> 2, j = 2 * (d & 3);
        out[d] = perm_b32(e[j + 1], e[j], pair_sel(b));
    }
}

// 0x40004000 (a pair of bf16 2.0) in a register whose value the compiler does not see, so that
// (x << s | it) & mask stays two instructions (v_lshl_or_b32 + v_and_b32) instead of being
// rewritten as a shift, an and and an or (a three-operand instruction takes no literal here).
__device__ __forceinline__ uint32_t opaque_two_pair() {
    uint32_t c;
    asm("s_mov_b32 %0, 0x40004000" : "=s"(c));
    return c;
}

// Sixteen binary codes, the low 16 bits of h (the high bits zero), to 8 operand dwords,
// out[d] = bf16 pair (-2*c[2d], -2*c[2d+1]), in 17 instructions:
//   v = h | h << 15, so bit 2d of v is code 2d and bit 16 + 2d is code 2d + 1;
//   out[d] = ((v << (15 - 2d)) | 0x40004000) & 0xC000C000 puts them on the two sign bits.
// `two_pair` is opaque_two_pair().
__device__ __forceinline__ void expand_binary_16(uint32_t h, uint32_t two_pair, uint32_t out[8]) {
    const uint32_t v = h | (h << 15);
#pragma unroll
    for (int d = 0; d < 8; ++d) out[d] = ((v << (15 - 2 * d)) | two_pair) & 0xC000C000u;
}

// LDS tiles are stored as rows of 128-byte (or 256-byte) lines of 16-byte chunks; chunk c of
// row r lives at chunk position c ^ lds_swizzle(r).  gfx950's LDS serves a 128-bit read for
// 16 lanes per cycle across 64 four-byte banks, i.e. 16 distinct 16-byte bank groups.  The
// MFMA operand reads have 16 lanes on 16 consecutive rows at the same logical chunk; a
// 128-byte row covers half the banks, so even and odd rows already differ in the upper
// half and the XOR only has to separate the 8 rows of each parity: (r >> 1) & 7.
__device__ __forceinline__ int lds_swizzle(int row) { return (row >> 1) & 7; }

// fp16 bits -> fp32 (exact).
__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// fp32 -> bf16 bits, round to nearest even (finite and infinite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Hardware workgroup id -> tile id, so that the tiles one XCD runs are contiguous in tile
// order.  Workgroups are dealt to the 8 XCDs round-robin (id % 8); XCD x gets the tile
// range [start(x), start(x) + count(x)).
__device__ __forceinline__ int xcd_remap(int pid, int total) {
    constexpr int kXcd = 8;
    const int x = pid % kXcd, slot = pid / kXcd;
    const int base = total / kXcd, extra = total % kXcd;
    return x * base + (x < extra ? x : extra) + slot;
}

// Raw buffer resource (gfx9 family flags) with its fields forced into scalar registers.  Loads
// through it at offsets at or past `bytes` return zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(a));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(a >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((uint64_t(hi) << 32) | lo), 0, int(n),
                                             0x00020000);
}

// 4x4 transpose of (lane quarter, register) blocks: lane quarter q (lanes 16q .. 16q+15)
// holds words w[0..3] of its 16-byte piece q; afterwards register c of lane quarter q holds
// word q of piece c.  Four lane-row swaps (v_permlane32_swap, v_permlane16_swap).
__device__ __forceinline__ void transpose_words(u32x4_t& w) {
    uint32_t r0 = w[0], r1 = w[1], r2 = w[2], r3 = w[3];
    auto a = __builtin_amdgcn_permlane32_swap(r0, r2, false, false);
    auto b = __builtin_amdgcn_permlane32_swap(r1, r3, false, false);
    r0 = a[0]; r2 = a[1]; r1 = b[0]; r3 = b[1];
    auto c = __builtin_amdgcn_permlane16_swap(r0, r1, false, false);
    auto d = __builtin_amdgcn_permlane16_swap(r2, r3, false, false);
    w = u32x4_t{c[0], c[1], d[0], d[1]};
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left alone).  Vector-memory operations complete
// in issue order, so vmcnt(N) means "all but the last N issued are done".
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    // encoding: vmcnt in bits [3:0] and [15:14], expcnt 7, lgkmcnt 15
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS that keeps loads in flight.  __syncthreads() releases at
// workgroup scope, which on gfx9 waits for every outstanding vector-memory operation --
// prefetches included.  Where each wave has already waited (counted waits) for its own
// copies into LDS, a bare s_barrier is enough; the empty asm statements keep the compiler
// from moving memory operations across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// 16-byte direct-to-LDS copy: lane i's 16 bytes (at voff + soff in the buffer) land at
// lds_wave_base + 16 * i.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, void* lds_wave_base, uint32_t voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_wave_base, 16, voff,
                                            soff, 0, 0);
}

}  // namespace lowbit

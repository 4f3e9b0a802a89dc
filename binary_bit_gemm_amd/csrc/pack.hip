// Packing and unpacking of weight codes (offline / load-time steps).
//
// One thread per output uint32 word.  Ternary: 16 int8 codes -> 2-bit fields
// (00 -> 0, 01 -> +1, 10 -> -1), binary: 32 codes -> bits (1 -> +1, 0 -> -1), 4-bit: 8 codes
// in [-8, 7] -> two's complement nibbles, affine 4-bit: 8 unsigned levels 0 .. 15 -> nibbles;
// least significant field first along K.  Invalid codes pack as 0 bits and are counted.
#include "lowbit_internal.h"

namespace lowbit {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t ternary_field(int c, int& bad) {
    bad += (c < -1 || c > 1);
    return c == 1 ? 1u : (c == -1 ? 2u : 0u);
}

__device__ __forceinline__ uint32_t bytes_to_u32(const int8_t* p4) {
    return *reinterpret_cast<const uint32_t*>(p4);
}

template <int BITS>
__global__ __launch_bounds__(kThreads) void pack_kernel(const int8_t* __restrict__ codes,
                                                        uint32_t* __restrict__ W, int64_t nwords,
                                                        int32_t* __restrict__ bad_count) {
    constexpr int kPer = 32 / BITS;
    const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    int bad = 0;
    if (BITS == 4 && i < nwords) {
        const uint2 v = *reinterpret_cast<const uint2*>(codes + i * kPer);
        uint32_t word = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int c = int(int8_t((k < 4 ? v.x : v.y) >> (8 * (k & 3))));
            const bool ok = c >= -8 && c <= 7;
            bad += !ok;
            word |= (ok ? uint32_t(c) & 0xFu : 0u) << (4 * k);
        }
        W[i] = word;
    } else if (i < nwords) {
        // Codes of word i are contiguous: [i*kPer, (i+1)*kPer) of the row-major [N, K] array.
        const uint4* src = reinterpret_cast<const uint4*>(codes + i * kPer);
        uint32_t word = 0;
#pragma unroll
        for (int v = 0; v < kPer / 16; ++v) {
            const uint4 q = src[v];
            const uint32_t parts[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int p = 0; p < 4; ++p) {
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int c = int(int8_t(parts[p] >> (8 * b)));
                    const int k = v * 16 + p * 4 + b;
                    if (BITS == 2) {
                        word |= ternary_field(c, bad) << (2 * k);
                    } else {
                        bad += (c != 1 && c != -1);
                        word |= uint32_t(c == 1) << k;
                    }
                }
            }
        }
        W[i] = word;
    }
    if (bad_count != nullptr) {
        // Integer counts: one atomic per wave that saw an invalid code.
        const unsigned long long mask = __ballot(bad != 0);
        if (mask != 0) {
            int total = bad;
            for (int off = 32; off > 0; off >>= 1) total += __shfl_xor(total, off);
            if ((threadIdx.x & 63) == 0) atomicAdd(bad_count, total);
        }
    }
}

// Unsigned 4-bit levels of affine groups: 8 levels 0 .. 15 -> nibbles, least significant first.
__global__ __launch_bounds__(kThreads) void pack_u4_kernel(const uint8_t* __restrict__ levels,
                                                           uint32_t* __restrict__ W, int64_t nwords,
                                                           int32_t* __restrict__ bad_count) {
    const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    int bad = 0;
    if (i < nwords) {
        const uint2 v = *reinterpret_cast<const uint2*>(levels + i * 8);
        uint32_t word = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t q = ((k < 4 ? v.x : v.y) >> (8 * (k & 3))) & 0xFFu;
            bad += q > 15u;
            word |= (q <= 15u ? q : 0u) << (4 * k);
        }
        W[i] = word;
    }
    if (bad_count != nullptr) {
        const unsigned long long mask = __ballot(bad != 0);
        if (mask != 0) {
            int total = bad;
            for (int off = 32; off > 0; off >>= 1) total += __shfl_xor(total, off);
            if ((threadIdx.x & 63) == 0) atomicAdd(bad_count, total);
        }
    }
}

template <int BITS>
__global__ __launch_bounds__(kThreads) void unpack_kernel(const uint32_t* __restrict__ W,
                                                          int8_t* __restrict__ codes, int64_t nwords) {
    constexpr int kPer = 32 / BITS;
    const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (i >= nwords) return;
    const uint32_t w = W[i];
    if constexpr (BITS == 4) {
        uint32_t parts[2] = {0u, 0u};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int c = int(w << (28 - 4 * k)) >> 28;  // sign-extended nibble k
            parts[k >> 2] |= (uint32_t(c) & 0xFFu) << (8 * (k & 3));
        }
        *reinterpret_cast<uint2*>(codes + i * kPer) = make_uint2(parts[0], parts[1]);
        return;
    }
    uint4* dst = reinterpret_cast<uint4*>(codes + i * kPer);
#pragma unroll
    for (int v = 0; v < kPer / 16; ++v) {
        uint32_t parts[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            uint32_t out = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int k = v * 16 + p * 4 + b;
                int c;
                if (BITS == 2) {
                    const uint32_t f = (w >> (2 * k)) & 3u;
                    c = int(f & 1u) - int((f >> 1) & 1u);
                } else {
                    c = 2 * int((w >> k) & 1u) - 1;
                }
                out |= (uint32_t(c) & 0xFFu) << (8 * b);
            }
            parts[p] = out;
        }
        dst[v] = make_uint4(parts[0], parts[1], parts[2], parts[3]);
    }
}

}  // namespace

hipError_t launch_pack(const int8_t* codes, uint32_t* W, int64_t N, int64_t K, int bits,
                       int32_t* bad_count, hipStream_t stream) {
    const int64_t nwords = N * K * bits / 32;
    if (nwords == 0) return hipSuccess;
    const dim3 grid(unsigned((nwords + kThreads - 1) / kThreads));
    if (bits == 4)
        hipLaunchKernelGGL(pack_kernel<4>, grid, dim3(kThreads), 0, stream, codes, W, nwords, bad_count);
    else if (bits == 2)
        hipLaunchKernelGGL(pack_kernel<2>, grid, dim3(kThreads), 0, stream, codes, W, nwords, bad_count);
    else
        hipLaunchKernelGGL(pack_kernel<1>, grid, dim3(kThreads), 0, stream, codes, W, nwords, bad_count);
    return hipGetLastError();
}

hipError_t launch_pack_u4(const uint8_t* levels, uint32_t* W, int64_t N, int64_t K, int32_t* bad_count,
                          hipStream_t stream) {
    const int64_t nwords = N * K / 8;
    if (nwords == 0) return hipSuccess;
    const dim3 grid(unsigned((nwords + kThreads - 1) / kThreads));
    hipLaunchKernelGGL(pack_u4_kernel, grid, dim3(kThreads), 0, stream, levels, W, nwords, bad_count);
    return hipGetLastError();
}

hipError_t launch_unpack(const uint32_t* W, int8_t* codes, int64_t N, int64_t K, int bits,
                         hipStream_t stream) {
    const int64_t nwords = N * K * bits / 32;
    if (nwords == 0) return hipSuccess;
    const dim3 grid(unsigned((nwords + kThreads - 1) / kThreads));
    if (bits == 4)
        hipLaunchKernelGGL(unpack_kernel<4>, grid, dim3(kThreads), 0, stream, W, codes, nwords);
    else if (bits == 2)
        hipLaunchKernelGGL(unpack_kernel<2>, grid, dim3(kThreads), 0, stream, W, codes, nwords);
    else
        hipLaunchKernelGGL(unpack_kernel<1>, grid, dim3(kThreads), 0, stream, W, codes, nwords);
    return hipGetLastError();
}

}  // namespace lowbit

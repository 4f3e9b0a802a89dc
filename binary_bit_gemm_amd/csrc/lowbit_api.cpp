// C-ABI of liblowbit: host-side validation, device check, variant choice and launch.
//
// Argument checks run before any HIP call, so a bad call returns a status without
// touching the device (and can be exercised on a machine without a GPU).  The library
// allocates no device memory.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>

#include "../../include/lowbit.h"
#include "lowbit_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
    g_last_hip_error = int(e);
    return LOWBIT_E_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
// Limits of the kernels' addressing: packed weights (and the smaller scales) are read
// through 32-bit buffer ranges, an X tile of up to 288 rows likewise, and tile counts are
// 32-bit.  M and X/Y offsets are 64-bit.
constexpr int64_t kMaxK = int64_t(1) << 22;
constexpr int64_t kMaxWeightBytes = (int64_t(1) << 32) - 1;
constexpr int64_t kMaxOutputs = int64_t(1) << 37;
constexpr int64_t kMaxCodes = int64_t(1) << 40;

int check_pack_args(const void* codes, const void* W, int64_t N, int64_t K, int bits) {
    if (bits != 1 && bits != 2) return LOWBIT_E_UNSUPPORTED;
    if (N < 0 || K < 0 || N > kMaxDim || K > kMaxDim) return LOWBIT_E_INVALID;
    if (K % (32 / bits) != 0) return LOWBIT_E_INVALID;
    if (N * K > kMaxCodes) return LOWBIT_E_UNSUPPORTED;
    if (N * K == 0) return LOWBIT_OK;
    if (codes == nullptr || W == nullptr) return LOWBIT_E_INVALID;
    if (!aligned16(codes) || !aligned16(W)) return LOWBIT_E_ALIGN;
    return LOWBIT_OK;
}

// Cached gfx950 check per device ordinal: -1 unknown, 0 no, 1 yes.
int g_dev_ok[64];
bool g_dev_init = false;

int device_check() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    const int r = lowbit_device_supported(dev);
    if (r < 0) return LOWBIT_E_HIP;
    return r == 1 ? LOWBIT_OK : LOWBIT_E_UNSUPPORTED;
}

// Variant override for A/B runs and tests: LOWBIT_VARIANT = auto | skinny | tile256 | tile256w | tile128 | tile64 |
// tile288 (the last falls back to tile256w where the 16x16 kernel does not apply)
int forced_variant() {
    const char* v = std::getenv("LOWBIT_VARIANT");
    if (v == nullptr || std::strcmp(v, "auto") == 0 || v[0] == 0) return -1;
    if (std::strcmp(v, "skinny") == 0) return 100;
    if (std::strcmp(v, "tile256") == 0) return lowbit::TILE_256x128;
    if (std::strcmp(v, "tile256w") == 0) return lowbit::TILE_256x256;
    if (std::strcmp(v, "tile128") == 0) return lowbit::TILE_128x256;
    if (std::strcmp(v, "tile64") == 0) return lowbit::TILE_64x256;
    if (std::strcmp(v, "tile288") == 0) return lowbit::TILE_288x192;
    if (std::strcmp(v, "ring") == 0) return 101;
    return -1;
}

// Largest K split of the ring kernel (LOWBIT_RING_MAX_SPLITS, for A/B runs and tests).
int ring_max_splits() {
    const char* v = std::getenv("LOWBIT_RING_MAX_SPLITS");
    const int n = v != nullptr ? std::atoi(v) : 0;
    return n >= 1 && n <= 64 ? n : 16;
}

// Ring kernel without a workspace: only when it fills the machine without splitting K.
bool ring_without_workspace(int64_t M, int64_t N, int64_t K, int g, int bits) {
    if (!lowbit::ring_supported(M, N, K, g, bits)) return false;
    const lowbit::RingPlan plan = lowbit::plan_ring(N, K, 1);
    return plan.tiles * plan.splits >= 384;
}

int choose_variant(int64_t M, int64_t N, int64_t K, int g, int bits) {
    const int f = forced_variant();
    if (f == 101 && lowbit::ring_supported(M, N, K, g, bits)) return 101;
    if (f == 100 && lowbit::use_skinny(M, N, K, g, bits)) return 100;
    if (f >= 0 && f != 100 && f != 101) return f;
    if (ring_without_workspace(M, N, K, g, bits)) return 101;
    if (lowbit::use_skinny(M, N, K, g, bits)) return 100;
    return lowbit::pick_tile_variant(M, N, K, g, bits);
}

__global__ void zero_fill_kernel(uint16_t* y, int64_t n) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) y[i] = 0;
}

int launch_one(const lowbit::GemmProblem& p, int g, int bits, hipStream_t stream) {
    if (p.M == 0 || p.N == 0) return LOWBIT_OK;
    hipError_t e;
    if (p.K == 0) {
        const int64_t n = int64_t(p.M) * p.N;
        hipLaunchKernelGGL(zero_fill_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream, p.Y, n);
        e = hipGetLastError();
    } else {
        const int v = choose_variant(p.M, p.N, p.K, g, bits);
        if (v == 101) {
            e = lowbit::launch_gemm_ring(p, g, lowbit::plan_ring(p.N, p.K, 1), nullptr, stream);
        } else {
            e = v == 100 ? lowbit::launch_gemm_skinny(p, g, bits, stream)
                         : lowbit::launch_gemm_tiled(p, g, bits, v, stream);
        }
    }
    return e == hipSuccess ? LOWBIT_OK : hip_fail(e);
}

}  // namespace

extern "C" {

int lowbit_version(void) { return LOWBIT_VERSION; }

const char* lowbit_status_string(int status) {
    switch (status) {
        case LOWBIT_OK: return "ok";
        case LOWBIT_E_INVALID: return "invalid argument (null pointer, bad size, N % 16 or K % g != 0)";
        case LOWBIT_E_UNSUPPORTED: return "unsupported (bits must be 1 or 2, g one of 32/64/128, device gfx950)";
        case LOWBIT_E_ALIGN: return "tensor pointer not 16-byte aligned";
        case LOWBIT_E_HIP: return "HIP runtime error (see lowbit_last_hip_error)";
        case LOWBIT_E_TOO_MANY: return "too many problems in one batched call";
        default: return "unknown status";
    }
}

int lowbit_last_hip_error(void) { return g_last_hip_error; }

int lowbit_device_supported(int device) {
    if (!g_dev_init) {
        for (int& v : g_dev_ok) v = -1;
        g_dev_init = true;
    }
    if (device < 0 || device >= 64) return 0;
    if (g_dev_ok[device] >= 0) return g_dev_ok[device];
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, device);
    if (e != hipSuccess) {
        g_last_hip_error = int(e);
        return -LOWBIT_E_HIP;
    }
    g_dev_ok[device] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
    return g_dev_ok[device];
}

int lowbit_check_gemm_args(const void* X, const uint32_t* W, const void* S, const void* Y,
                           int64_t M, int64_t N, int64_t K, int g, int bits) {
    if (bits != 1 && bits != 2) return LOWBIT_E_UNSUPPORTED;
    if (g != 32 && g != 64 && g != 128) return LOWBIT_E_UNSUPPORTED;
    if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return LOWBIT_E_INVALID;
    if (K % g != 0 || N % 16 != 0) return LOWBIT_E_INVALID;
    if (K > kMaxK || N * K / 8 * bits > kMaxWeightBytes || M * N > kMaxOutputs) return LOWBIT_E_UNSUPPORTED;
    if (M * N == 0) return LOWBIT_OK;
    if (Y == nullptr) return LOWBIT_E_INVALID;
    if (K > 0 && (X == nullptr || W == nullptr || S == nullptr)) return LOWBIT_E_INVALID;
    if (!aligned16(Y)) return LOWBIT_E_ALIGN;
    if (K > 0 && (!aligned16(X) || !aligned16(W) || !aligned16(S))) return LOWBIT_E_ALIGN;
    return LOWBIT_OK;
}

const char* lowbit_gemm_variant(int64_t M, int64_t N, int64_t K, int g, int bits) {
    int v = choose_variant(M, N, K, g, bits);
    if (v == 100) return "skinny";
    if (v == 101) return "ring";
    if (v == lowbit::TILE_288x192 && !lowbit::tile16_supported(g, bits)) v = lowbit::TILE_256x256;
    return lowbit::tile_variant_name(v);
}

int lowbit_pack(const int8_t* codes, uint32_t* W, int64_t N, int64_t K, int bits,
                int32_t* bad_count, void* stream) {
    int st = check_pack_args(codes, W, N, K, bits);
    if (st != LOWBIT_OK || N * K == 0) return st;
    st = device_check();
    if (st != LOWBIT_OK) return st;
    hipError_t e = lowbit::launch_pack(codes, W, N, K, bits, bad_count, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LOWBIT_OK : hip_fail(e);
}

int lowbit_unpack(const uint32_t* W, int8_t* codes, int64_t N, int64_t K, int bits, void* stream) {
    int st = check_pack_args(codes, W, N, K, bits);
    if (st != LOWBIT_OK || N * K == 0) return st;
    st = device_check();
    if (st != LOWBIT_OK) return st;
    hipError_t e = lowbit::launch_unpack(W, codes, N, K, bits, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LOWBIT_OK : hip_fail(e);
}

int lowbit_gemm(const void* X, const uint32_t* W, const void* S, void* Y,
                int64_t M, int64_t N, int64_t K, int g, int bits, void* stream) {
    int st = lowbit_check_gemm_args(X, W, S, Y, M, N, K, g, bits);
    if (st != LOWBIT_OK || M * N == 0) return st;
    st = device_check();
    if (st != LOWBIT_OK) return st;
    lowbit::GemmProblem p{static_cast<const uint16_t*>(X), W, static_cast<const uint16_t*>(S),
                          static_cast<uint16_t*>(Y), int(M), int(N), int(K)};
    return launch_one(p, g, bits, static_cast<hipStream_t>(stream));
}

size_t lowbit_workspace_size(int64_t M, int64_t N, int64_t K, int g, int bits) {
    if (lowbit_check_gemm_args(nullptr, nullptr, nullptr, nullptr, 0, N, K, g, bits) != LOWBIT_OK) return 0;
    if (!lowbit::ring_supported(M, N, K, g, bits)) return 0;
    return lowbit::ring_workspace_bytes(lowbit::plan_ring(N, K, ring_max_splits()), N);
}

int lowbit_gemm_ex(const void* X, const uint32_t* W, const void* S, void* Y, int64_t M, int64_t N, int64_t K,
                   int g, int bits, void* workspace, size_t workspace_bytes, void* stream) {
    int st = lowbit_check_gemm_args(X, W, S, Y, M, N, K, g, bits);
    if (st != LOWBIT_OK || M * N == 0) return st;
    if (workspace != nullptr && !aligned16(workspace)) return LOWBIT_E_ALIGN;
    if (K == 0 || !lowbit::ring_supported(M, N, K, g, bits) || forced_variant() >= 0)
        return lowbit_gemm(X, W, S, Y, M, N, K, g, bits, stream);
    const lowbit::RingPlan plan = lowbit::plan_ring(N, K, ring_max_splits());
    if (plan.splits > 1 && (workspace == nullptr || workspace_bytes < lowbit::ring_workspace_bytes(plan, N)))
        return lowbit_gemm(X, W, S, Y, M, N, K, g, bits, stream);
    st = device_check();
    if (st != LOWBIT_OK) return st;
    lowbit::GemmProblem p{static_cast<const uint16_t*>(X), W, static_cast<const uint16_t*>(S),
                          static_cast<uint16_t*>(Y), int(M), int(N), int(K)};
    const hipError_t e = lowbit::launch_gemm_ring(p, g, plan, workspace, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LOWBIT_OK : hip_fail(e);
}

int lowbit_gemm_batched(const lowbit_problem* problems, int count, void* stream) {
    if (count < 0 || (count > 0 && problems == nullptr)) return LOWBIT_E_INVALID;
    if (count > LOWBIT_MAX_BATCH) return LOWBIT_E_TOO_MANY;
    for (int i = 0; i < count; ++i) {
        const lowbit_problem& q = problems[i];
        const int st = lowbit_check_gemm_args(q.X, q.W, q.S, q.Y, q.M, q.N, q.K, q.g, q.bits);
        if (st != LOWBIT_OK) return st;
    }
    if (count == 0) return LOWBIT_OK;
    int st = device_check();
    if (st != LOWBIT_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);

    // Problems of one (g, bits) class with K > 0 go into one grouped launch.
    static const int kClasses[6][2] = {{64, 2}, {64, 1}, {128, 2}, {128, 1}, {32, 2}, {32, 1}};
    lowbit::GemmProblem grp[LOWBIT_MAX_BATCH];
    for (const auto& cls : kClasses) {
        int n = 0;
        for (int i = 0; i < count; ++i) {
            const lowbit_problem& q = problems[i];
            if (q.g != cls[0] || q.bits != cls[1] || q.M * q.N == 0) continue;
            lowbit::GemmProblem p{static_cast<const uint16_t*>(q.X), q.W, static_cast<const uint16_t*>(q.S),
                                  static_cast<uint16_t*>(q.Y), int(q.M), int(q.N), int(q.K)};
            if (q.K == 0) {
                st = launch_one(p, q.g, q.bits, s);
                if (st != LOWBIT_OK) return st;
                continue;
            }
            grp[n++] = p;
        }
        if (n == 0) continue;
        hipError_t e = lowbit::launch_gemm_grouped(grp, n, cls[0], cls[1], s);
        if (e != hipSuccess) return hip_fail(e);
    }
    return LOWBIT_OK;
}

}  // extern "C"

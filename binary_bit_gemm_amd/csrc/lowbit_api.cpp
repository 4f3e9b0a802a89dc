// C-ABI of liblowbit: host-side validation, device check, variant choice and launch.
//
// Argument checks run before any HIP call, so a bad call returns a status without
// touching the device (and can be exercised on a machine without a GPU).  The library
// allocates no device memory.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/lowbit.h"
#include "lowbit_internal.h"

namespace lowbit {

// The affine GEMM with K split across workgroups through a caller workspace (gemm_tile16.hip;
// hipErrorNotSupported where the shape takes no split or the workspace is too small), and the
// workspace it needs.
hipError_t launch_gemm_tile16_affine_ex(const GemmProblem& p, int g, void* workspace, size_t workspace_bytes,
                                        hipStream_t stream);
size_t affine_workspace_bytes(const GemmProblem& p, int g);

bool trace_enabled() {
    const char* v = std::getenv("LOWBIT_TRACE");
    return v != nullptr && v[0] != 0 && std::strcmp(v, "0") != 0;
}

void trace_launch(const char* family, const char* config, int g, int bits, const GemmProblem* probs, int count,
                  unsigned grid, unsigned block, unsigned lds) {
    char line[1024];
    int n = snprintf(line, sizeof line, "lowbit: %s %s g=%d bits=%d grid=%u block=%u lds=%u problems=", family, config,
                     g, bits, grid, block, lds);
    for (int i = 0; i < count && n > 0 && n < int(sizeof line) - 48; ++i)
        n += snprintf(line + n, sizeof line - size_t(n), "%s%dx%dx%d", i ? "," : "", probs[i].M, probs[i].N, probs[i].K);
    std::fprintf(stderr, "%s\n", line);
}

}  // namespace lowbit

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
    if (bits != 1 && bits != 2 && bits != 4) return LOWBIT_E_UNSUPPORTED;
    if (N < 0 || K < 0 || N > kMaxDim || K > kMaxDim) return LOWBIT_E_INVALID;
    if (K % (32 / bits) != 0) return LOWBIT_E_INVALID;
    if (N * K > kMaxCodes) return LOWBIT_E_UNSUPPORTED;
    if (N * K == 0) return LOWBIT_OK;
    if (codes == nullptr || W == nullptr) return LOWBIT_E_INVALID;
    if (!aligned16(codes) || !aligned16(W)) return LOWBIT_E_ALIGN;
    return LOWBIT_OK;
}

// Cached gfx950 check per device ordinal: 0 not yet probed, 1 no, 2 yes.  Threads that make
// their first call at the same time may both probe; they store the same value.
std::atomic<int> g_dev_ok[64];

int device_check() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    const int r = lowbit_device_supported(dev);
    if (r < 0) return LOWBIT_E_HIP;
    return r == 1 ? LOWBIT_OK : LOWBIT_E_UNSUPPORTED;
}

// Variant override for A/B runs and tests: LOWBIT_VARIANT = auto | skinny | resident | tile256 | tile256w |
// tile128 | tile64 | tile288 | tile256n (256 x 192) | tile96 | tile96k2 | tile64k2 (the 16x16-block tiles,
// tile288 onwards, fall back to tile256w where that kernel does not apply) | tile256sk (stream-K on
// 256 x 256 in the calls that pass a workspace large enough, tile256w in the others)
int forced_variant() {
    const char* v = std::getenv("LOWBIT_VARIANT");
    if (v == nullptr || std::strcmp(v, "auto") == 0 || v[0] == 0) return -1;
    if (std::strcmp(v, "skinny") == 0) return 100;
    if (std::strcmp(v, "tile256") == 0) return lowbit::TILE_256x128;
    if (std::strcmp(v, "tile256w") == 0) return lowbit::TILE_256x256;
    if (std::strcmp(v, "tile128") == 0) return lowbit::TILE_128x256;
    if (std::strcmp(v, "tile64") == 0) return lowbit::TILE_64x256;
    if (std::strcmp(v, "tile288") == 0) return lowbit::TILE_288x192;
    if (std::strcmp(v, "tile96") == 0) return lowbit::TILE_96x192;
    if (std::strcmp(v, "tile96k2") == 0) return lowbit::TILE_96x192K2;
    if (std::strcmp(v, "tile256n") == 0) return lowbit::TILE_256x192;
    if (std::strcmp(v, "tile64k2") == 0) return lowbit::TILE_64x128K2;
    if (std::strcmp(v, "tile256sk") == 0) return lowbit::TILE_256x256SK;
    if (std::strcmp(v, "resident") == 0) return 102;
    return -1;
}

// Resident plan of one problem (len 0: not covered).  `may_split`: a workspace is available.
lowbit::ResidentPlan resident_plan(int64_t M, int64_t N, int64_t K, int g, int bits, bool may_split) {
    if (!lowbit::resident_supported(M, N, K, g, bits)) return lowbit::ResidentPlan{};
    const lowbit::GemmProblem p{nullptr, nullptr, nullptr, nullptr, int(M), int(N), int(K)};
    return lowbit::plan_resident(&p, 1, g, may_split);
}

int choose_variant(int64_t M, int64_t N, int64_t K, int g, int bits) {
    const int f = forced_variant();
    if (f == 102 && resident_plan(M, N, K, g, bits, false).len > 0) return 102;
    if (f == 100 && lowbit::use_skinny(M, N, K, g, bits)) return 100;
    if (f >= 0 && f < 100) return f;
    if (f < 0 && lowbit::resident_supported(M, N, K, g, bits)) {
        const lowbit::GemmProblem p{nullptr, nullptr, nullptr, nullptr, int(M), int(N), int(K)};
        if (lowbit::resident_preferred(&p, 1, g, false)) return 102;
    }
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
        if (v == 102) {
            e = lowbit::launch_gemm_resident_group(&p, 1, g, lowbit::plan_resident(&p, 1, g, false), nullptr, stream);
        } else {
            e = v == 100 ? lowbit::launch_gemm_skinny(p, g, bits, stream)
                         : lowbit::launch_gemm_tiled(p, g, bits, v, stream);
        }
    }
    return e == hipSuccess ? LOWBIT_OK : hip_fail(e);
}

// Calls f(group, n, g, bits) for the problems of each (g, bits) class with M, N, K > 0.
template <class F>
int for_each_class(const lowbit_problem* problems, int count, F&& f) {
    static const int kClasses[8][2] = {{64, 2}, {64, 1}, {128, 2}, {128, 1}, {32, 2}, {32, 1}, {64, 4}, {128, 4}};
    lowbit::GemmProblem grp[LOWBIT_MAX_BATCH];
    for (const auto& cls : kClasses) {
        int n = 0;
        for (int i = 0; i < count; ++i) {
            const lowbit_problem& q = problems[i];
            if (q.g != cls[0] || q.bits != cls[1] || q.M * q.N == 0 || q.K == 0) continue;
            grp[n++] = lowbit::GemmProblem{static_cast<const uint16_t*>(q.X), q.W, static_cast<const uint16_t*>(q.S),
                                           static_cast<uint16_t*>(q.Y), int(q.M), int(q.N), int(q.K)};
        }
        if (n == 0) continue;
        const int st = f(grp, n, cls[0], cls[1]);
        if (st != LOWBIT_OK) return st;
    }
    return LOWBIT_OK;
}

int batched(const lowbit_problem* problems, int count, void* workspace, size_t workspace_bytes, void* stream) {
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
    // K == 0: Y = 0
    for (int i = 0; i < count; ++i) {
        const lowbit_problem& q = problems[i];
        if (q.M * q.N == 0 || q.K != 0) continue;
        lowbit::GemmProblem p{static_cast<const uint16_t*>(q.X), q.W, static_cast<const uint16_t*>(q.S),
                              static_cast<uint16_t*>(q.Y), int(q.M), int(q.N), int(q.K)};
        st = launch_one(p, q.g, q.bits, s);
        if (st != LOWBIT_OK) return st;
    }
    // each (g, bits) class: one grouped launch per kernel family
    return for_each_class(problems, count, [&](const lowbit::GemmProblem* grp, int n, int g, int bits) {
        const hipError_t e = lowbit::launch_gemm_grouped(grp, n, g, bits, workspace, workspace_bytes, s);
        return e == hipSuccess ? LOWBIT_OK : hip_fail(e);
    });
}

// ---- static scratch of lowbit_gemm_noalloc ----
// The split-K workspace of the resident kernel, for callers that cannot allocate: one array
// per device, held from the library's load until the process ends.  Its size is the largest
// workspace an automatic split plan asks for (the 4 KiB counter region plus at most
// 512 workgroups x 16 column blocks x 1 KiB of fp32 partial sums).  In host code `scratch`
// names a host-side stand-in, not device memory: only the address hipGetSymbolAddress returns
// for the current device (kept per device below) is passed to kernels.
static_assert(LOWBIT_NOALLOC_SCRATCH_BYTES == 4096 + 512 * 16 * 1024, "scratch size");
static __device__ __align__(256) unsigned char scratch[LOWBIT_NOALLOC_SCRATCH_BYTES];
std::atomic<void*> g_scratch_dev[64];
constexpr int kCounterWords = 1024;  // the workspace's counter region (first 4 KiB)

__global__ void zero_u32_kernel(uint32_t* p, int n) {
    const int i = int(blockIdx.x) * int(blockDim.x) + int(threadIdx.x);
    if (i < n) p[i] = 0u;
}

// The current device's scratch address, looked up once per device (the device must be current).
int scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= 64) return LOWBIT_E_UNSUPPORTED;
    void* ptr = g_scratch_dev[dev].load(std::memory_order_acquire);
    if (ptr == nullptr) {
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e);
        if (ptr == nullptr) return LOWBIT_E_HIP;
        g_scratch_dev[dev].store(ptr, std::memory_order_release);
    }
    *out = ptr;
    return LOWBIT_OK;
}

}  // namespace

extern "C" {

int lowbit_version(void) { return LOWBIT_VERSION; }

const char* lowbit_status_string(int status) {
    switch (status) {
        case LOWBIT_OK: return "ok";
        case LOWBIT_E_INVALID: return "invalid argument (null pointer, bad size, N % 16 or K % g != 0)";
        case LOWBIT_E_UNSUPPORTED: return "unsupported (bits must be 1, 2 or 4, g one of 32/64/128 (4-bit: 64/128), device gfx950)";
        case LOWBIT_E_ALIGN: return "tensor pointer not 16-byte aligned";
        case LOWBIT_E_HIP: return "HIP runtime error (see lowbit_last_hip_error)";
        case LOWBIT_E_TOO_MANY: return "too many problems in one batched call";
        case LOWBIT_E_SCRATCH: return "the shape needs more workspace than the static scratch of lowbit_gemm_noalloc holds";
        default: return "unknown status";
    }
}

int lowbit_last_hip_error(void) { return g_last_hip_error; }

int lowbit_device_supported(int device) {
    if (device < 0 || device >= 64) return 0;
    const int known = g_dev_ok[device].load(std::memory_order_relaxed);
    if (known != 0) return known - 1;
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, device);
    if (e != hipSuccess) {
        g_last_hip_error = int(e);
        return -LOWBIT_E_HIP;
    }
    const int ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
    g_dev_ok[device].store(ok + 1, std::memory_order_relaxed);
    return ok;
}

int lowbit_check_gemm_args(const void* X, const uint32_t* W, const void* S, const void* Y,
                           int64_t M, int64_t N, int64_t K, int g, int bits) {
    if (bits != 1 && bits != 2 && bits != 4) return LOWBIT_E_UNSUPPORTED;
    if (g != 32 && g != 64 && g != 128) return LOWBIT_E_UNSUPPORTED;
    if (bits == 4 && g == 32) return LOWBIT_E_UNSUPPORTED;  // 4-bit codes run on the 16x16-block tile only
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
    if (v == 102) return "resident";
    if (bits == 4 && !lowbit::is_tile16_variant(v)) v = lowbit::TILE_288x192;  // as launch_gemm_tiled_group
    if (lowbit::is_tile16_variant(v) && !lowbit::tile16_supported(g, bits)) v = lowbit::TILE_256x256;
    if (v == lowbit::TILE_256x256SK) v = lowbit::TILE_256x256;  // stream-K runs only with a workspace
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

int lowbit_pack_u4(const uint8_t* levels, uint32_t* W, int64_t N, int64_t K, int32_t* bad_count, void* stream) {
    int st = check_pack_args(levels, W, N, K, 4);
    if (st != LOWBIT_OK || N * K == 0) return st;
    st = device_check();
    if (st != LOWBIT_OK) return st;
    hipError_t e = lowbit::launch_pack_u4(levels, W, N, K, bad_count, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LOWBIT_OK : hip_fail(e);
}

size_t lowbit_affine_workspace_size(int64_t M, int64_t N, int64_t K, int g) {
    if (lowbit_check_gemm_args(reinterpret_cast<const void*>(256), reinterpret_cast<const uint32_t*>(256),
                               reinterpret_cast<const void*>(256), reinterpret_cast<const void*>(256), M, N, K, g,
                               4) != LOWBIT_OK ||
        M * N * K == 0)
        return 0;
    const lowbit::GemmProblem p{nullptr, nullptr, nullptr, nullptr, int(M), int(N), int(K)};
    return lowbit::affine_workspace_bytes(p, g);
}

int lowbit_gemm_affine_ex(const void* X, const uint32_t* W, const void* S, const void* B, void* Y, int64_t M,
                          int64_t N, int64_t K, int g, void* workspace, size_t workspace_bytes, void* stream) {
    int st = lowbit_check_gemm_args(X, W, S, Y, M, N, K, g, 4);
    if (st != LOWBIT_OK || M * N == 0) return st;
    if (K > 0 && B == nullptr) return LOWBIT_E_INVALID;
    if (K > 0 && !aligned16(B)) return LOWBIT_E_ALIGN;
    if (workspace != nullptr && !aligned16(workspace)) return LOWBIT_E_ALIGN;
    const size_t need = lowbit_affine_workspace_size(M, N, K, g);
    if (need == 0 || workspace == nullptr || workspace_bytes < need || forced_variant() >= 0)
        return lowbit_gemm_affine(X, W, S, B, Y, M, N, K, g, stream);
    st = device_check();
    if (st != LOWBIT_OK) return st;
    lowbit::GemmProblem p{static_cast<const uint16_t*>(X), W, static_cast<const uint16_t*>(S),
                          static_cast<uint16_t*>(Y), int(M), int(N), int(K)};
    p.B = static_cast<const uint16_t*>(B);
    const hipError_t e = lowbit::launch_gemm_tile16_affine_ex(p, g, workspace, workspace_bytes,
                                                              static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LOWBIT_OK : hip_fail(e);
}

int lowbit_gemm_affine(const void* X, const uint32_t* W, const void* S, const void* B, void* Y, int64_t M,
                       int64_t N, int64_t K, int g, void* stream) {
    int st = lowbit_check_gemm_args(X, W, S, Y, M, N, K, g, 4);
    if (st != LOWBIT_OK || M * N == 0) return st;
    if (K > 0 && B == nullptr) return LOWBIT_E_INVALID;
    if (K > 0 && !aligned16(B)) return LOWBIT_E_ALIGN;
    st = device_check();
    if (st != LOWBIT_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    lowbit::GemmProblem p{static_cast<const uint16_t*>(X), W, static_cast<const uint16_t*>(S),
                          static_cast<uint16_t*>(Y), int(M), int(N), int(K)};
    p.B = static_cast<const uint16_t*>(B);
    hipError_t e;
    if (K == 0) {  // an empty sum
        const int64_t n = M * N;
        hipLaunchKernelGGL(zero_fill_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, p.Y, n);
        e = hipGetLastError();
    } else {
        const int f = forced_variant();
        const int v = f >= 0 && f < 100 ? f : lowbit::pick_tile_variant(M, N, K, g, 4);
        e = lowbit::launch_gemm_tile16_affine(&p, 1, g, v, s);
    }
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

int lowbit_import_ternary(const void* src, int layout, int zero, uint32_t* W, int64_t N, int64_t K,
                          int32_t* bad_count, void* stream) {
    static_assert(lowbit::kLayoutGemliteU8T == LOWBIT_LAYOUT_GEMLITE_U8T && lowbit::kLayoutMlxU32 == LOWBIT_LAYOUT_MLX_U32,
                  "layout values");
    if (layout != LOWBIT_LAYOUT_GEMLITE_U8T && layout != LOWBIT_LAYOUT_MLX_U32) return LOWBIT_E_INVALID;
    if (zero < 0 || zero > 3) return LOWBIT_E_INVALID;
    if (N < 0 || K < 0 || N % 16 != 0 || K % 16 != 0) return LOWBIT_E_INVALID;
    if (N > kMaxDim || K > kMaxK || N * K > kMaxCodes) return LOWBIT_E_UNSUPPORTED;
    if (N * K == 0) return LOWBIT_OK;
    if (src == nullptr || W == nullptr) return LOWBIT_E_INVALID;
    if (!aligned16(src) || !aligned16(W)) return LOWBIT_E_ALIGN;
    int st = device_check();
    if (st != LOWBIT_OK) return st;
    hipError_t e = lowbit::launch_import(src, layout, zero, W, N, K, bad_count, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LOWBIT_OK : hip_fail(e);
}

int lowbit_import_binary_gemlite(const uint8_t* src, uint32_t* W, int64_t N, int64_t K, void* stream) {
    if (N < 0 || K < 0 || N % 16 != 0 || K % 32 != 0) return LOWBIT_E_INVALID;
    if (N > kMaxDim || K > kMaxK || N * K > kMaxCodes) return LOWBIT_E_UNSUPPORTED;
    if (N * K == 0) return LOWBIT_OK;
    if (src == nullptr || W == nullptr) return LOWBIT_E_INVALID;
    if (!aligned16(src) || !aligned16(W)) return LOWBIT_E_ALIGN;
    int st = device_check();
    if (st != LOWBIT_OK) return st;
    hipError_t e = lowbit::launch_import_binary_gemlite(src, W, N, K, static_cast<hipStream_t>(stream));
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

int lowbit_gemm_swiglu(const void* X, const uint32_t* W, const void* S, void* Y, int64_t M, int64_t N, int64_t K,
                       int g, int bits, void* stream) {
    if (N < 0 || N > kMaxDim / 2) return LOWBIT_E_INVALID;
    // the weight side has 2N rows; Y has N columns (checked against 2N outputs: stricter)
    int st = lowbit_check_gemm_args(X, W, S, Y, M, 2 * N, K, g, bits);
    if (st != LOWBIT_OK || M * N == 0) return st;
    if (!lowbit::tile16_supported(g, bits)) return LOWBIT_E_UNSUPPORTED;
    st = device_check();
    if (st != LOWBIT_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    lowbit::GemmProblem p{static_cast<const uint16_t*>(X), W, static_cast<const uint16_t*>(S),
                          static_cast<uint16_t*>(Y), int(M), int(N), int(K)};
    hipError_t e;
    if (K == 0) {  // silu(0) * 0
        const int64_t n = M * N;
        hipLaunchKernelGGL(zero_fill_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, p.Y, n);
        e = hipGetLastError();
    } else {
        // skinny ternary M on the resident kernel where a whole-K plan fits, else the tile kernel
        e = hipErrorNotSupported;
        if (bits == 2 && M <= 16) e = lowbit::launch_gemm_resident_epilogue(p, g, lowbit::kEpiSwiglu, s);
        if (e == hipErrorNotSupported) e = lowbit::launch_gemm_tile16_epilogue(&p, 1, g, bits, lowbit::kEpiSwiglu, s);
    }
    return e == hipSuccess ? LOWBIT_OK : hip_fail(e);
}

int lowbit_gemm_residual(const void* X, const uint32_t* W, const void* S, const void* R, const void* gate, void* Y,
                         int64_t M, int64_t N, int64_t K, int g, int bits, void* stream) {
    int st = lowbit_check_gemm_args(X, W, S, Y, M, N, K, g, bits);
    if (st != LOWBIT_OK || M * N == 0) return st;
    if (R == nullptr || gate == nullptr) return LOWBIT_E_INVALID;
    if (!aligned16(R) || !aligned16(gate)) return LOWBIT_E_ALIGN;
    if (!lowbit::tile16_supported(g, bits)) return LOWBIT_E_UNSUPPORTED;
    st = device_check();
    if (st != LOWBIT_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (K == 0) {  // Y = R + gate * 0
        e = R == Y ? hipSuccess
                   : hipMemcpyAsync(Y, R, size_t(M) * size_t(N) * 2u, hipMemcpyDeviceToDevice, s);
    } else {
        lowbit::GemmProblem p{static_cast<const uint16_t*>(X), W, static_cast<const uint16_t*>(S),
                              static_cast<uint16_t*>(Y), int(M), int(N), int(K),
                              static_cast<const uint16_t*>(R), static_cast<const uint16_t*>(gate)};
        e = hipErrorNotSupported;
        if (bits == 2 && M <= 16) e = lowbit::launch_gemm_resident_epilogue(p, g, lowbit::kEpiResidual, s);
        if (e == hipErrorNotSupported) e = lowbit::launch_gemm_tile16_epilogue(&p, 1, g, bits, lowbit::kEpiResidual, s);
    }
    return e == hipSuccess ? LOWBIT_OK : hip_fail(e);
}

size_t lowbit_workspace_size(int64_t M, int64_t N, int64_t K, int g, int bits) {
    if (lowbit_check_gemm_args(nullptr, nullptr, nullptr, nullptr, 0, N, K, g, bits) != LOWBIT_OK) return 0;
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    const lowbit::GemmProblem p{nullptr, nullptr, nullptr, nullptr, int(M), int(N), int(K)};
    return lowbit::grouped_workspace_bytes(&p, 1, g, bits);
}

int lowbit_gemm_ex(const void* X, const uint32_t* W, const void* S, void* Y, int64_t M, int64_t N, int64_t K,
                   int g, int bits, void* workspace, size_t workspace_bytes, void* stream) {
    int st = lowbit_check_gemm_args(X, W, S, Y, M, N, K, g, bits);
    if (st != LOWBIT_OK || M * N == 0) return st;
    if (workspace != nullptr && !aligned16(workspace)) return LOWBIT_E_ALIGN;
    const size_t need = lowbit_workspace_size(M, N, K, g, bits);
    const int f = forced_variant();
    if (need == 0 || workspace == nullptr || workspace_bytes < need || (f >= 0 && f != lowbit::TILE_256x256SK))
        return lowbit_gemm(X, W, S, Y, M, N, K, g, bits, stream);
    st = device_check();
    if (st != LOWBIT_OK) return st;
    lowbit::GemmProblem p{static_cast<const uint16_t*>(X), W, static_cast<const uint16_t*>(S),
                          static_cast<uint16_t*>(Y), int(M), int(N), int(K)};
    const hipError_t e = lowbit::launch_gemm_grouped(&p, 1, g, bits, workspace, workspace_bytes,
                                                     static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LOWBIT_OK : hip_fail(e);
}

int lowbit_gemm_noalloc(const void* X, const uint32_t* W, const void* S, void* Y, int64_t M, int64_t N, int64_t K,
                        int g, int bits, void* stream) {
    int st = lowbit_check_gemm_args(X, W, S, Y, M, N, K, g, bits);
    if (st != LOWBIT_OK || M * N == 0) return st;
    // a forced variant (LOWBIT_VARIANT) runs as lowbit_gemm, whatever workspace it would take
    if (forced_variant() >= 0) return lowbit_gemm(X, W, S, Y, M, N, K, g, bits, stream);
    const size_t need = lowbit_workspace_size(M, N, K, g, bits);
    if (need > LOWBIT_NOALLOC_SCRATCH_BYTES) return LOWBIT_E_SCRATCH;
    if (need == 0) return lowbit_gemm(X, W, S, Y, M, N, K, g, bits, stream);
    st = device_check();
    if (st != LOWBIT_OK) return st;
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st != LOWBIT_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    // the arrival counters must start at zero: every call leaves them so, and a fill kernel
    // (not a memset, which a captured graph must not hold) clears them again first
    hipLaunchKernelGGL(zero_u32_kernel, dim3(kCounterWords / 256), dim3(256), 0, s, static_cast<uint32_t*>(ws),
                       kCounterWords);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e);
    lowbit::GemmProblem p{static_cast<const uint16_t*>(X), W, static_cast<const uint16_t*>(S),
                          static_cast<uint16_t*>(Y), int(M), int(N), int(K)};
    e = lowbit::launch_gemm_grouped(&p, 1, g, bits, ws, LOWBIT_NOALLOC_SCRATCH_BYTES, s);
    return e == hipSuccess ? LOWBIT_OK : hip_fail(e);
}

size_t lowbit_batched_workspace_size(const lowbit_problem* problems, int count) {
    if (count <= 0 || count > LOWBIT_MAX_BATCH || problems == nullptr) return 0;
    size_t need = 0;
    for_each_class(problems, count, [&](const lowbit::GemmProblem* grp, int n, int g, int bits) {
        const size_t b = lowbit::grouped_workspace_bytes(grp, n, g, bits);
        need = b > need ? b : need;
        return LOWBIT_OK;
    });
    return need;
}

int lowbit_gemm_batched_ex(const lowbit_problem* problems, int count, void* workspace, size_t workspace_bytes,
                           void* stream) {
    if (workspace != nullptr && !aligned16(workspace)) return LOWBIT_E_ALIGN;
    const int f = forced_variant();
    return batched(problems, count, f >= 0 && f != lowbit::TILE_256x256SK ? nullptr : workspace, workspace_bytes,
                   stream);
}

int lowbit_gemm_batched(const lowbit_problem* problems, int count, void* stream) {
    return batched(problems, count, nullptr, 0, stream);
}

}  // extern "C"

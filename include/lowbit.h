/*
 * lowbit.h -- packed low-bit weight GEMM for AMD Instinct MI355X (gfx950).
 *
 * The library computes, for bf16 activations X and packed ternary or binary weights W
 * with fp16 group scales S,
 *
 *     Y[m, n] = sum_k  X[m, k] * c[n, k] * S[n, k / g]              (Y in bf16)
 *
 * which is the linear layer of the Bonsai-quantised FLUX.2 Klein 4B diffusion
 * transformer:
 *   - binary weights w = scale_g * b, b in {-1, +1}, one fp16 scale per group of g
 *     consecutive weights ("bonsai-image-binary-4B-gemlite-1bit" model card, section
 *     "Binary Weight Representation: 1-bit g128"; the same card's "Model Overview" lists
 *     the binary values + FP16 group-wise scales weight format);
 *   - ternary weights {-1, 0, +1} in 2 bits, multiplied by a 2-bit quantised matmul
 *     (mlx-vlm Prism Bonsai ternary 2-bit guide, section 运行前提 / prerequisites);
 *   - weights kept as packed uint32 words plus scales ("backend/ -- FastAPI Mac backend",
 *     section "Checkpoint layout").
 *
 * ---------------------------------------------------------------------------------
 * Packed weight format (the pages leave the bit layout open; this is the library's):
 *   ternary (bits = 2): 16 codes per uint32, along K, least significant field first:
 *       code k of row n is the 2-bit field at bits 2*(k%16) .. 2*(k%16)+1 of
 *       W[n * (K/16) + k/16];  field 00 -> 0, 01 -> +1, 10 -> -1.  The field 11 is never
 *       written; readers decode it as 0.
 *   binary  (bits = 1): 32 codes per uint32, along K: code k of row n is bit k%32 of
 *       W[n * (K/32) + k/32];  1 -> +1, 0 -> -1.
 *   4-bit   (bits = 4): 8 codes per uint32, along K: code k of row n is the two's complement
 *       nibble at bits 4*(k%8) .. 4*(k%8)+3 of W[n * (K/8) + k/8], values -8 .. 7, symmetric
 *       w = s * c (the 4-bit text encoder of the binary model card's "Model Overview" table).
 *       The affine form of the same encoder (unsigned levels with a scale and a bias per
 *       group) has its own entry points: lowbit_pack_u4 and lowbit_gemm_affine.
 *   scales: fp16 (IEEE binary16) S[n * (K/g) + k/g], symmetric (no zero point).
 * Activations X[M, K] and outputs Y[M, N] are bf16, row-major, contiguous.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller, 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Work is enqueued
 *     asynchronously; nothing synchronises the host.  Device-side faults surface at the
 *     caller's next synchronisation.
 *   - Arguments are validated on the host before anything is enqueued; a non-zero
 *     return means nothing was launched.
 *   - Supported: bits in {1, 2, 4} (4: g in {64, 128} only); g in {32, 64, 128}; K % g == 0; N % 16 == 0; M >= 0
 *     (M == 0 or N == 0 is a no-op); M, N < 2^31; K <= 2^22; packed weights under 4 GiB
 *     (N*K*bits/8 < 2^32); M*N <= 2^37; the current device is gfx950.  lowbit_pack and
 *     lowbit_unpack take N*K <= 2^40 codes.  Shapes past these limits return
 *     LOWBIT_E_UNSUPPORTED.
 *   - The library allocates no device memory and uses no hidden workspace; the only
 *     workspace is the one a caller passes to lowbit_gemm_ex.
 *   - Results are deterministic: the same inputs give bitwise the same Y on every run.
 */
#ifndef LOWBIT_H
#define LOWBIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LOWBIT_VERSION 100 /* 1.0.0 */

/* Status codes returned by every entry point. */
enum {
    LOWBIT_OK = 0,
    LOWBIT_E_INVALID = 1,     /* null pointer, negative size, N % 16 or K % g != 0 ...     */
    LOWBIT_E_UNSUPPORTED = 2, /* bits / g or a size outside the supported set, or device not gfx950 */
    LOWBIT_E_ALIGN = 3,       /* a tensor pointer is not 16-byte aligned                   */
    LOWBIT_E_HIP = 4,         /* a HIP runtime call failed; see lowbit_last_hip_error()    */
    LOWBIT_E_TOO_MANY = 5,    /* batched call: more problems than one call accepts         */
    LOWBIT_E_SCRATCH = 6      /* lowbit_gemm_noalloc: the shape needs more than its scratch */
};

/*
 * lowbit_pack -- int8 codes [N, K] -> packed words [N, K*bits/32] in the format above.
 *   codes       device, N*K int8, row-major.  Ternary expects {-1,0,1}, binary {-1,1},
 *               4-bit -8 .. 7.
 *   W           device, N*K*bits/32 uint32, written.
 *   bad_count   device int32 or NULL.  When given, the number of codes outside the
 *               valid set is ADDED to *bad_count (the caller zeroes it); such codes are
 *               packed as 0 bits (ternary 0, binary -1, 4-bit 0).
 *   Requires K % (32/bits) == 0.  This is the offline, load-time step.
 */
int lowbit_pack(const int8_t* codes, uint32_t* W, int64_t N, int64_t K, int bits,
                int32_t* bad_count, void* stream);

/*
 * lowbit_pack_u4 -- unsigned 4-bit levels [N, K] -> packed words [N, K/8] for affine groups
 * (lowbit_gemm_affine): level k of row n is the nibble at bits 4*(k%8) .. 4*(k%8)+3 of
 * W[n * (K/8) + k/8] (least significant nibble first, the same positions as the signed 4-bit
 * format).
 *   levels     device, N*K uint8 in 0 .. 15, row-major.
 *   W          device, N*K/8 uint32, written.
 *   bad_count  device int32 or NULL: levels above 15 pack as 0 and their number is ADDED to
 *              *bad_count (the caller zeroes it).
 *   Requires K % 8 == 0; errors as lowbit_pack.  Offline, load-time step.
 */
int lowbit_pack_u4(const uint8_t* levels, uint32_t* W, int64_t N, int64_t K, int32_t* bad_count, void* stream);

/*
 * lowbit_unpack -- packed words -> int8 codes [N, K] (ternary field 11 -> 0).
 */
int lowbit_unpack(const uint32_t* W, int8_t* codes, int64_t N, int64_t K, int bits, void* stream);

/*
 * lowbit_import_ternary -- ternary weights packed by another runtime -> packed words [N, K/16]
 * in the format above (an offline, load-time step like lowbit_pack).
 *   Both source layouts hold unsigned 2-bit levels q in {0, 1, 2, 3}, least significant field
 *   first along K; the code is c = q - zero.  The pages name the layouts but not the level
 *   coding: zero = 1 is the symmetric ternary form (q = 0, 1, 2 -> -1, 0, +1).
 *   layout  LOWBIT_LAYOUT_GEMLITE_U8T: src is uint8 [K/4, N], transposed: byte (j, n) holds
 *             codes k = 4j .. 4j+3 of output row n at bits 2(k%4) .. 2(k%4)+1 (GemLite's
 *             int2 weights, packed over K with a transpose, shape (in_features / 4,
 *             out_features): comment thread of the Bonsai-Image-Demo pull request "CPU
 *             bring-up").  The shape, not a guess from the buffer, fixes the orientation: a
 *             square weight is read as (K/4, N) like any other.
 *           LOWBIT_LAYOUT_MLX_U32: src is uint32 [N, K/16], row-major by output feature:
 *             word (n, j) holds codes k = 16j .. 16j+15 at bits 2(k%16) .. 2(k%16)+1 (packed
 *             uint32 weights of the MLX checkpoint: "backend/ -- FastAPI Mac backend",
 *             section "Checkpoint layout").  With MLX's affine groups w = s*q + b this
 *             is exact when b = -zero*s; the library's scale is then s.
 *   zero    0 .. 3.
 *   W       device, N*K/16 uint32, written.
 *   bad_count  device int32 or NULL: codes outside {-1, 0, +1} are packed as 0 and their
 *           number is ADDED to *bad_count (the caller zeroes it).
 *   Requires N % 16 == 0, K % 16 == 0, K <= 2^22, 16-byte aligned src and W.  Scales are not
 *   touched: the library's fp16 [N, K/g] scales are the caller's.
 */
#define LOWBIT_LAYOUT_GEMLITE_U8T 1
#define LOWBIT_LAYOUT_MLX_U32 2
int lowbit_import_ternary(const void* src, int layout, int zero, uint32_t* W, int64_t N, int64_t K,
                          int32_t* bad_count, void* stream);

/*
 * lowbit_import_binary_gemlite -- binary weights in GemLite's transposed 1-bit pack -> packed
 * words [N, K/32] in the format above (offline, like lowbit_pack).
 *   src  device uint8 [K/8, N]: bit i of byte (j, n) is code k = 8j + i of output row n, 1 -> +1,
 *        0 -> -1.  The binary model card ("bonsai-image-binary-4B-gemlite-1bit", "Binary Weight
 *        Representation: 1-bit g128") gives w = scale_g * b with b in {-1, +1} and a GemLite
 *        1-bit pack; the byte orientation is the one the Bonsai-Image-Demo pull request's "CPU
 *        bring-up" comment gives for GemLite's int2 weights, (in_features / bytes-per-code,
 *        out_features).  Every bit pattern is a valid code.
 *   W    device, N*K/32 uint32, written.
 *   Requires N % 16 == 0, K % 32 == 0, K <= 2^22, 16-byte aligned src and W.  Scales are the
 *   caller's (the card's per-group fp16 scale_g is the library's scale).
 *   The byte layout is a reading, not a published format: the card names the GemLite 1-bit
 *   pack without describing its bits, so this importer's parity against real GemLite files is
 *   unpinned (none is available); only its self-consistency with lowbit_pack is tested.
 */
int lowbit_import_binary_gemlite(const uint8_t* src, uint32_t* W, int64_t N, int64_t K, void* stream);

/*
 * lowbit_gemm -- Y[M, N] = X[M, K] . dequant(W)[N, K]^T, bf16 out (round to nearest even).
 *   X  device bf16 [M, K];  W  device packed words [N, K*bits/32];
 *   S  device fp16 [N, K/g];  Y  device bf16 [M, N], fully overwritten.
 * The weight codes are expanded to bf16 in registers and multiplied on the bf16 matrix
 * cores with fp32 accumulation; each group's partial sum is multiplied by its fp32 scale
 * after the matrix multiply (the scale is not rounded to bf16).  The kernel is chosen
 * from M (skinny M uses split-K inside a workgroup, reduced in a fixed order).
 */
int lowbit_gemm(const void* X, const uint32_t* W, const void* S, void* Y,
                int64_t M, int64_t N, int64_t K, int g, int bits, void* stream);

/* One problem of a batched call: the same meaning as the lowbit_gemm arguments. */
typedef struct lowbit_problem {
    const void* X;
    const uint32_t* W;
    const void* S;
    void* Y;
    int64_t M, N, K;
    int32_t g, bits;
} lowbit_problem;

#define LOWBIT_MAX_BATCH 64

/*
 * lowbit_gemm_batched -- `count` independent GEMMs in one launch per (bits, g) class.
 *   problems  HOST array of `count` problems (read before return; may be freed after).
 * Intended for the independent linears of one transformer block (e.g. the image and text
 * streams' QKV of a double-stream block), so that small-M and small-N problems share the
 * machine.  Problems must not write overlapping Y.  count <= LOWBIT_MAX_BATCH.
 * Every problem is validated as in lowbit_gemm before anything is launched.
 */
int lowbit_gemm_batched(const lowbit_problem* problems, int count, void* stream);

/*
 * lowbit_workspace_size -- bytes of caller-provided device workspace with which
 * lowbit_gemm_ex can split K across workgroups for this shape (0: it never needs one).
 * The split applies to skinny ternary problems (M <= 16, g = 64 or 128, K % 256 == 0)
 * whose K is too long for the activations of the whole K to stay in one workgroup's LDS
 * (K above about 4.5K).  The fp32
 * partial sums of the K ranges are added in a fixed order, so the result is deterministic
 * (it can differ in the last bits from lowbit_gemm's, which splits K differently).
 * Returns 0 for invalid arguments.
 */
size_t lowbit_workspace_size(int64_t M, int64_t N, int64_t K, int g, int bits);

/*
 * lowbit_gemm_ex -- lowbit_gemm with a caller-provided workspace.
 *   workspace        device memory of at least lowbit_workspace_size(...) bytes, 16-byte
 *                    aligned, ZERO-FILLED before its first use.  Its first 4096 bytes hold
 *                    arrival counters at the same place for every shape; every call leaves
 *                    them at zero again, so one workspace serves calls of any shapes in
 *                    turn as is (the rest holds partial sums, which need no clearing).
 *                    Calls that share a workspace must not run concurrently.
 *   workspace_bytes  its size.  With a NULL or too small workspace (or for shapes that need
 *                    none) the call is exactly lowbit_gemm.
 */
int lowbit_gemm_ex(const void* X, const uint32_t* W, const void* S, void* Y,
                   int64_t M, int64_t N, int64_t K, int g, int bits,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * lowbit_gemm_noalloc -- lowbit_gemm_ex without a caller workspace and without any allocation,
 * for callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, kernels and results as
 * lowbit_gemm_ex given a large enough workspace.
 *   The workspace is a static device array of LOWBIT_NOALLOC_SCRATCH_BYTES per GPU, held from
 *   the library's load until the process ends; it covers every automatic split plan.  A shape
 *   whose lowbit_workspace_size exceeds it returns LOWBIT_E_SCRATCH and launches nothing
 *   (only a forced split plan can).  Shapes that need no workspace run as lowbit_gemm.
 *   Every call on one GPU shares that GPU's array: calls that overlap on one GPU (other
 *   streams, other host threads) race and must be serialised by the caller.  Each call first
 *   clears the array's counter region with a fill kernel on `stream` (no memset).
 *   The call allocates nothing: no hipMalloc, hipFree or allocating library routine.
 */
#define LOWBIT_NOALLOC_SCRATCH_BYTES (4096u + 512u * 16u * 1024u)
int lowbit_gemm_noalloc(const void* X, const uint32_t* W, const void* S, void* Y,
                        int64_t M, int64_t N, int64_t K, int g, int bits, void* stream);

/*
 * lowbit_batched_workspace_size / lowbit_gemm_batched_ex -- lowbit_gemm_batched with a
 * caller-provided workspace, under the same rules as lowbit_gemm_ex: the launches of one
 * call use the workspace one after the other on `stream`; size from
 * lowbit_batched_workspace_size (0 for invalid arguments or when no launch needs one).
 */
size_t lowbit_batched_workspace_size(const lowbit_problem* problems, int count);
int lowbit_gemm_batched_ex(const lowbit_problem* problems, int count, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * lowbit_gemm_swiglu -- the MLP-in linear with its SwiGLU gate fused into the epilogue:
 *   Y[M, N] = silu(X . dequant(Wg)^T) * (X . dequant(Wu)^T),  silu(a) = a / (1 + exp(-a)),
 * where W / S hold 2N rows: gate rows Wg = rows [0, N), up rows Wu = rows [N, 2N) (the
 * MMDiT's MLP-in linear of 2 x 9216 outputs in the mlx page's component architecture; which
 * half gates is not stated there -- gate first is this library's reading).
 *   X  device bf16 [M, K];  W  device packed words [2N, K*bits/32];
 *   S  device fp16 [2N, K/g];  Y  device bf16 [M, N], fully overwritten.
 * Both factors are the fp32 sums of lowbit_gemm's arithmetic; the product is rounded to
 * bf16 once.  Supports g = 64 or 128 (all bit widths); g = 32 returns LOWBIT_E_UNSUPPORTED.
 * Ternary problems with M <= 16 whose whole K fits one workgroup run on the skinny resident
 * kernel; every other shape runs on the 16x16-block tile kernel.  Argument checks and errors
 * as lowbit_gemm, with 2N weight rows.
 */
int lowbit_gemm_swiglu(const void* X, const uint32_t* W, const void* S, void* Y,
                       int64_t M, int64_t N, int64_t K, int g, int bits, void* stream);

/*
 * lowbit_gemm_residual -- a block's output linear with its gated residual update fused:
 *   Y[m, n] = R[m, n] + gate[n] * (X . dequant(W)^T)[m, n]
 * (the modulation gate of an MMDiT block applied to the proj / MLP-out linear, added to the
 * residual stream; the mlx page's component architecture names the modulated blocks, the exact
 * form is this library's reading).
 *   X, W, S, M, N, K, g, bits  as lowbit_gemm;
 *   R     device bf16 [M, N], the residual; may be the same memory as Y (in-place update);
 *   gate  device bf16 [N], one factor per output feature;
 *   Y     device bf16 [M, N], fully overwritten.
 * The product, the gate multiply and the add are done in fp32 and rounded to bf16 once.
 * g = 64 or 128 (g = 32 returns LOWBIT_E_UNSUPPORTED); a null R or gate returns
 * LOWBIT_E_INVALID, an unaligned one LOWBIT_E_ALIGN.  K = 0 gives Y = R.
 */
int lowbit_gemm_residual(const void* X, const uint32_t* W, const void* S, const void* R, const void* gate,
                         void* Y, int64_t M, int64_t N, int64_t K, int g, int bits, void* stream);

/*
 * lowbit_gemm_affine -- Y[M, N] = X[M, K] . W[N, K]^T for 4-bit weights in affine groups,
 *     W[n, k] = S[n, k/g] * q[n, k] + B[n, k/g],   q in 0 .. 15 unsigned,
 * the form of the text encoder that the mlx guide's component architecture loads quantised at
 * bits = 4, group_size = 64 (MLX's affine 4-bit groups; an HQQ zero point z is B = -z * S).
 *   X  device bf16 [M, K];  W  device packed levels [N, K/8] (lowbit_pack_u4);
 *   S, B  device fp16 [N, K/g] scales and biases;  Y  device bf16 [M, N], fully overwritten.
 * The levels are expanded to bf16 (exact) and multiplied on the bf16 matrix cores with fp32
 * sums; per group the fp32 sum times S, plus B times the group's fp32 activation sum (from the
 * matrix cores against an all-ones operand), is added in fp32; Y is rounded to bf16 once.
 * g = 64 or 128 (g = 32 returns LOWBIT_E_UNSUPPORTED).  A null or unaligned B with K > 0 returns
 * LOWBIT_E_INVALID / LOWBIT_E_ALIGN; other checks as lowbit_gemm with bits = 4.  K = 0 gives
 * Y = 0.  Runs on the 16x16-block tile kernel at every M.
 */
int lowbit_gemm_affine(const void* X, const uint32_t* W, const void* S, const void* B, void* Y,
                       int64_t M, int64_t N, int64_t K, int g, void* stream);

/*
 * lowbit_affine_workspace_size / lowbit_gemm_affine_ex -- lowbit_gemm_affine with a caller-provided
 * workspace, with which the call splits K across workgroups where the output tile grid leaves a
 * quarter of the compute units or more idle (the text encoder's 512 x 2560 down projection at
 * K = 9728, a shape of the mlx guide's component architecture): three workgroups per output tile,
 * whose fp32 sums are added in a fixed split order (deterministic; the last bits can differ from
 * lowbit_gemm_affine's, which runs K in one workgroup).
 *   workspace        device memory of at least lowbit_affine_workspace_size(...) bytes, 16-byte
 *                    aligned, ZERO-FILLED before its first use; its first 4096 bytes hold arrival
 *                    counters that every call leaves at zero again, so one workspace serves calls
 *                    of any shapes in turn.  Calls that share a workspace must not run concurrently.
 *   workspace_bytes  its size.  With a NULL or too small workspace, or for shapes that take no
 *                    split (size 0), the call is exactly lowbit_gemm_affine.
 * lowbit_affine_workspace_size returns 0 for invalid arguments and for shapes that take no split.
 */
size_t lowbit_affine_workspace_size(int64_t M, int64_t N, int64_t K, int g);
int lowbit_gemm_affine_ex(const void* X, const uint32_t* W, const void* S, const void* B, void* Y,
                          int64_t M, int64_t N, int64_t K, int g, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Host-only argument check of lowbit_gemm (no HIP call): returns the status lowbit_gemm
 * would return before touching the device. */
int lowbit_check_gemm_args(const void* X, const uint32_t* W, const void* S, const void* Y,
                           int64_t M, int64_t N, int64_t K, int g, int bits);

/* Name of the kernel variant lowbit_gemm picks for a shape (for logs and tests).
 *
 * Launch log: with the environment variable LOWBIT_TRACE set (to anything but "" or "0", read at
 * every launch), each GEMM kernel launch of every entry point writes one line to stderr:
 *   lowbit: <family> <configuration> g=<g> bits=<bits> grid=<workgroups> block=<threads>
 *           lds=<dynamic LDS bytes> problems=<M>x<N>x<K>[,<M>x<N>x<K>...]
 * (one line; family resident, skinny, tile16 or tiled32; the configuration names the tile and
 * wave layout, or the resident plan's column blocks, K slices, steps, splits and tiles). */
const char* lowbit_gemm_variant(int64_t M, int64_t N, int64_t K, int g, int bits);

/* Human-readable text for a status code. */
const char* lowbit_status_string(int status);

/* hipError_t of the last failed HIP call in this thread (0 if none). */
int lowbit_last_hip_error(void);

/* 1 if `device` is a gfx950 GPU the library can run on, 0 if not, -LOWBIT_E_HIP on error. */
int lowbit_device_supported(int device);

/* LOWBIT_VERSION of the built library. */
int lowbit_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LOWBIT_H */

/*
 * vqv.h - C ABI of libvqv: the block-verification projection of DFlash-style
 * speculative decoding on AMD Instinct MI355X (gfx950).
 *
 * Two core operations, each an asynchronous launch on the caller's HIP stream:
 *
 *   vqv_qgemm   y[M,N] = x[M,K] . W^T, W[N,K] 4-bit group-quantized (affine,
 *               group 32, 64 or 128 along K), fp32 output. This is the quantized linear
 *               that a target model runs over the M rows of a verify block
 *               ("perf: tune DFlash2 M=8 verification for M1 and M2", PR
 *               description: tuned M=8 verification QMM with BF16/FP16
 *               activations and a W4A32 draft/vocabulary path).
 *   vqv_verify  per-row greedy argmax of fp32 logits[B*T, N], then per
 *               sequence the number of leading drafts that the target
 *               confirms ("perf(speculative): commit per-row accepts in
 *               batched DFlash", commit message: each row commits its own
 *               walk count; "dspark: fold first-token forward into verify +
 *               bit-exact M5 Metal decode wins", first commit: the committed
 *               token is verified as row 0 of the block).
 *
 * Around them: vqv_qgemm_verify fuses the two, vqv_verify_ex and
 * vqv_qgemm_verify_ex add per-sequence draft lengths and top-1/top-2 margins,
 * and vqv_qgemm_swiglu is the projection of a stacked gate/up weight with its
 * silu-gated activation.
 *
 * Memory and ownership
 *   Every pointer is DEVICE memory owned by the caller; the library never
 *   allocates, frees or keeps a pointer after the call returns. Tensors are
 *   dense and row-major. `hip_stream` is a hipStream_t (NULL = the default
 *   stream). Calls only enqueue work: results are valid once the stream has
 *   been synchronized. Asynchronous faults surface at that synchronization.
 *   Calls are thread-safe and deterministic: the same inputs give the same
 *   output bits on every call.
 *
 * Errors
 *   Arguments are checked on the host before anything is launched, and so
 *   is the choice of kernel (a problem no kernel's LDS image takes returns
 *   VQV_ERR_UNSUPPORTED). A call that returns VQV_ERR_ARG,
 *   VQV_ERR_UNSUPPORTED, VQV_ERR_ALIGN or VQV_ERR_WORKSPACE has launched
 *   nothing and written nothing. VQV_ERR_HIP means the HIP runtime refused a
 *   launch (hipGetLastError); in the calls that launch two kernels it can
 *   come after the first was enqueued, which may then write its outputs and
 *   scratch. Each call clears the calling thread's HIP error state
 *   (hipGetLastError) before its first launch.
 */
#ifndef VQV_H
#define VQV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VQV_ABI_VERSION 6

typedef enum {
  VQV_BF16 = 0, /* bfloat16 activations                                  */
  VQV_FP16 = 1, /* IEEE half activations                                 */
  VQV_FP32 = 2  /* IEEE single activations (the W4A32 draft projection)  */
} vqv_dtype;

typedef enum {
  VQV_OK = 0,
  VQV_ERR_ARG = 1,         /* NULL pointer, size out of range, or aliasing   */
  VQV_ERR_UNSUPPORTED = 2, /* valid request the library does not handle  */
  VQV_ERR_ALIGN = 3,       /* a pointer breaks its alignment requirement    */
  VQV_ERR_WORKSPACE = 4,   /* workspace missing or smaller than queried     */
  VQV_ERR_HIP = 5          /* the HIP runtime refused the launch            */
} vqv_status;

/* VQV_ABI_VERSION of the loaded library. */
int vqv_abi_version(void);

/* Static English text for a status code (never NULL). */
const char* vqv_status_string(vqv_status s);

/*
 * Weight format (the affine 4-bit layout shared by the tuned kernels and the
 * stock QMM path they fall back to, "perf: tune DFlash2 M=8 verification for
 * M1 and M2", PR description; the pages do not spell out the bits, the
 * reading used here is):
 *   wq      uint8  [N, K/2]  row n holds column n's K codes, K-contiguous
 *                            ("K-major"); byte j packs k=2j in bits 0-3 and
 *                            k=2j+1 in bits 4-7. Codes q are 0..15.
 *   scales  fp16   [N, K/group]  s[n,g]
 *   biases  fp16   [N, K/group]  b[n,g]
 *   w[n,k] = s[n, k/group] * q[n,k] + b[n, k/group]
 *   y[m,n] = sum_k x[m,k] * w[n,k]      (accumulated in fp32)
 *
 * Arguments
 *   x          [M, K] in act_dtype. 16-byte aligned.
 *   wq         [N, K/2] uint8. 16-byte aligned.
 *   scales     [N, K/group] fp16 bit patterns. 2-byte aligned.
 *   biases     [N, K/group] fp16 bit patterns. 2-byte aligned.
 *   y          [M, N] fp32, written. 4-byte aligned. Must not overlap any
 *              input (VQV_ERR_ARG).
 *   M          1..64 verify rows (a block of 8 or 16, up to 64 batched).
 *   K          multiple of the group, 64 <= K <= 16384 (larger K returns
 *              VQV_ERR_UNSUPPORTED; K not a multiple of the group returns
 *              VQV_ERR_ARG); with group 32 also K % 64 == 0 and K <= 8192
 *              (else VQV_ERR_UNSUPPORTED); M*K*sizeof(act) < 2^31.
 *   N          >= 1 output columns; any N (tails are masked).
 *   group      32, 64 or 128 contiguous k per scale and bias (else
 *              VQV_ERR_UNSUPPORTED). The pages name no group size; 64 is the
 *              layout of the tuned kernels, 32 and 128 the other common W4
 *              layouts. All three run on the same kernels; group 32 keeps
 *              twice the partial sums per step and reads twice the scale
 *              and bias entries, so it runs somewhat slower.
 *   act_dtype  a vqv_dtype (else VQV_ERR_ARG).
 *   workspace  device scratch of at least vqv_qgemm_workspace_bytes(...)
 *              bytes; may be NULL when that is 0.
 *
 * Numerics: products of x and the 4-bit codes are exact; sums are fp32; the
 * scale and bias are applied in fp32 after each 64-value partial sum (a
 * 128-group's scale and bias apply to each of its two halves), or after each
 * 32-value partial sum with group 32. NaN/Inf in x, scales or biases
 * propagate by IEEE rules.
 */
size_t vqv_qgemm_workspace_bytes(int M, int K, int N, int group, vqv_dtype act_dtype);

/*
 * The projection kernel that vqv_qgemm (and the fused calls) run for these
 * sizes on the current device: a static string such as "qgemm_w4_m8q", the
 * name a kernel trace shows, or NULL for arguments vqv_qgemm rejects. For
 * profiling, the environment variable VQV_FORCE_VARIANT (read at each call)
 * pins the one- and two-row and 8-row choice: "m8" the half-line
 * MFMA kernel, "m8q" the whole-line one, "v" the vector-ALU kernel where it
 * applies ("perf: tune DFlash2 M=8 verification for M1 and M2", PR
 * description: the single-variant mode for tracing).
 */
const char* vqv_qgemm_kernel(int M, int K, int N, int group, vqv_dtype act_dtype);

vqv_status vqv_qgemm(const void* x, const uint8_t* wq, const uint16_t* scales,
                     const uint16_t* biases, float* y, int M, int K, int N, int group,
                     vqv_dtype act_dtype, void* workspace, size_t workspace_bytes,
                     void* hip_stream);

/*
 * Greedy verify over one verify block per sequence.
 *   logits      [B*T, N] fp32, row b*T+i is sequence b's row i. Row 0 is the
 *               committed token, rows 1..T-1 the drafts. 16-byte aligned.
 *   draft       [B, T-1] int32: draft[b,i] is the token fed at row i+1.
 *               May be NULL only when T == 1. 4-byte aligned.
 *   argmax      [B*T] int32, written: lowest index of the row maximum; -0
 *               and +0 are equal; a row holding NaN gives its first NaN.
 *   accept_len  [B] int32, written: the largest L in 0..T-1 such that
 *               argmax[b*T+i] == draft[b,i] for every i < L. The bonus token
 *               argmax[b*T+L] is implied; tokens committed = L + 1.
 *   B >= 1, 1 <= T <= 64, N >= 1, B*T*N < 2^31.
 *   workspace   at least vqv_verify_workspace_bytes(B, T, N) bytes, 16-byte
 *               aligned; its contents on entry do not matter.
 * Draft ids are compared as plain int32: ids outside [0, N) never match.
 * No output may overlap an input, another output or the workspace
 * (VQV_ERR_ARG).
 */
size_t vqv_verify_workspace_bytes(int B, int T, int N);

vqv_status vqv_verify(const float* logits, const int32_t* draft, int B, int T, int N,
                      int32_t* argmax, int32_t* accept_len, void* workspace,
                      size_t workspace_bytes, void* hip_stream);

/*
 * vqv_verify with two optional extras (either may be NULL; with both NULL
 * the call is vqv_verify):
 *   draft_len   [B] int32 input: sequence b holds draft_len[b] valid drafts,
 *               clamped to 0..T-1, and its walk stops there, so accept_len[b]
 *               <= clamp(draft_len[b]). In a batched round loop the live
 *               sequences carry blocks of different valid lengths, and a
 *               block may end in a partial tail ("perf(speculative): commit
 *               per-row accepts in batched DFlash", commit message: each row
 *               commits its own count; "perf: tune DFlash2 M=8 verification
 *               for M1 and M2", Validation: the partial-tail case). Drafts
 *               past the valid length do not affect the result, but draft
 *               must still hold all B*(T-1) entries. 4-byte aligned.
 *   margin      [B*T] fp32 output: top-1 minus top-2 of each row, where top-2
 *               is the largest value at any index other than the argmax; the
 *               value a margin gate compares with its bar ("dspark: fold
 *               first-token forward into verify + bit-exact M5 Metal decode
 *               wins", first commit: the top-1/top-2 margin gate). A tied
 *               maximum gives 0 (-0 and +0 tie, as do two infinities of one
 *               sign), a row holding NaN gives NaN, a row of one value (N == 1)
 *               gives +inf; otherwise it is the fp32 difference, rounded to
 *               nearest. 4-byte aligned.
 * argmax and accept_len are as in vqv_verify; the workspace is the same.
 */
vqv_status vqv_verify_ex(const float* logits, const int32_t* draft, const int32_t* draft_len,
                         int B, int T, int N, int32_t* argmax, int32_t* accept_len,
                         float* margin, void* workspace, size_t workspace_bytes,
                         void* hip_stream);

/*
 * Projection and greedy verify in one call: y = x . W^T as vqv_qgemm, then
 * argmax and accept_len of y as vqv_verify with B*T == M. The argmax is
 * fused into the projection's epilogue (every row count 1..64, activation
 * type and group size): each work-group of the projection keeps the two
 * best values of each row over its columns, and one small kernel per
 * sequence reduces them and walks the drafts, so the logits are never read
 * back ("dspark: fold first-token forward into verify + bit-exact M5 Metal
 * decode wins", first commit: the fused argmax of the CUDA path and the
 * single accept loop; "perf(speculative): commit per-row accepts in batched
 * DFlash", commit message: the batched verify of B = 4 blocks of 16).
 *
 * Arguments
 *   x, wq, scales, biases, M, K, N, group, act_dtype
 *              as vqv_qgemm.
 *   y          [M, N] fp32 logits, written; may be NULL when they are not
 *              needed. 16-byte aligned.
 *   draft, B, T, argmax, accept_len
 *              as vqv_verify, with B*T == M (else VQV_ERR_ARG).
 *   workspace  at least vqv_qgemm_verify_workspace_bytes(M, K, N, group,
 *              act_dtype) bytes, 256-byte aligned: 256 bytes and one 16-byte
 *              partial per row and projection work-group (at most 64 x 256
 *              partials on the vocabulary kernels, N/16 to N/80 per row on
 *              the others); 0 for arguments the call rejects. Its contents
 *              on entry do not matter. Calls that share a workspace must not
 *              overlap in time (same stream, or synchronized).
 * The results are bit-identical to vqv_qgemm followed by vqv_verify on the
 * same inputs.
 */
size_t vqv_qgemm_verify_workspace_bytes(int M, int K, int N, int group, vqv_dtype act_dtype);

vqv_status vqv_qgemm_verify(const void* x, const uint8_t* wq, const uint16_t* scales,
                            const uint16_t* biases, float* y, int M, int K, int N, int group,
                            vqv_dtype act_dtype, const int32_t* draft, int B, int T,
                            int32_t* argmax, int32_t* accept_len, void* workspace,
                            size_t workspace_bytes, void* hip_stream);

/*
 * vqv_qgemm_verify with vqv_verify_ex's two optional extras: draft_len [B]
 * (the valid drafts of each sequence) and margin [B*T] (top-1 minus top-2 of
 * each logits row). On the fused path the projection's epilogue keeps each
 * row's two best keys, so the margin costs no extra read of the logits. The
 * results are bit-identical to vqv_qgemm followed by vqv_verify_ex.
 */
vqv_status vqv_qgemm_verify_ex(const void* x, const uint8_t* wq, const uint16_t* scales,
                               const uint16_t* biases, float* y, int M, int K, int N, int group,
                               vqv_dtype act_dtype, const int32_t* draft,
                               const int32_t* draft_len, int B, int T, int32_t* argmax,
                               int32_t* accept_len, float* margin, void* workspace,
                               size_t workspace_bytes, void* hip_stream);

/*
 * vqv_qgemm_verify_ex for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. It takes no workspace: its scratch (the projection's per-row
 * partials, vqv_qgemm_verify_workspace_bytes of them) lives in a static
 * device array of VQV_NOALLOC_SCRATCH_BYTES bytes that the library holds on
 * each GPU it runs on until the process ends. The arguments and results are
 * those of vqv_qgemm_verify_ex.
 *   A problem whose scratch exceeds VQV_NOALLOC_SCRATCH_BYTES returns
 *   VQV_ERR_WORKSPACE with nothing launched (on 80-column work-groups, M <= 8
 *   with 16-bit activations, that is N above roughly 650,000; on 64-column
 *   work-groups at M = 64, N above about 65,000 where the vocabulary kernels
 *   do not apply).
 *   The first call on a device looks the array up (hipGetSymbolAddress);
 *   VQV_ERR_HIP if that fails. No call allocates or frees anything.
 *   All calls on one GPU share that GPU's array: calls that overlap in time
 *   on one GPU (different streams, or different host threads without
 *   synchronization) race on it and their results are undefined. Nothing in
 *   it needs to start at zero, and each call overwrites what it uses.
 */
#define VQV_NOALLOC_SCRATCH_BYTES (1u << 20)

vqv_status vqv_qgemm_verify_ex_noalloc(const void* x, const uint8_t* wq, const uint16_t* scales,
                                       const uint16_t* biases, float* y, int M, int K, int N,
                                       int group, vqv_dtype act_dtype, const int32_t* draft,
                                       const int32_t* draft_len, int B, int T, int32_t* argmax,
                                       int32_t* accept_len, float* margin, void* hip_stream);

/*
 * Gate/up projection with its SwiGLU activation: y = x . W^T as vqv_qgemm over
 * a stacked weight W [N, K] whose rows 0..N/2-1 are the gate projection and
 * rows N/2..N-1 the up projection, then
 *     h[m, j] = silu(y[m, j]) * y[m, N/2 + j],   silu(g) = g / (1 + exp(-g)),
 * written as h [M, N/2] fp32; y itself is not written. This is the fused
 * gate/up block of the M=16 verify pass ("perf: tune DFlash2 M=8 verification
 * for M1 and M2", Validation: the M=16 gate/up block and its 1e-3 bound; the
 * pages name no activation, and a silu-gated MLP is the reading taken for the
 * Qwen 3.5 targets of "perf(speculative): commit per-row accepts in batched
 * DFlash").
 *
 * Arguments
 *   x, wq, scales, biases, M, K, group, act_dtype   as vqv_qgemm, with N the
 *              row count of the stacked weight: N even, N >= 2.
 *   h          [M, N/2] fp32, written. 4-byte aligned. Must not overlap an
 *              input or the workspace.
 *   workspace  at least vqv_qgemm_swiglu_workspace_bytes(...) bytes,
 *              256-byte aligned; may be NULL when that is 0. It is 0 where
 *              the activation is fused into the projection (bf16/fp16
 *              activations, K <= 2560); elsewhere the projection's output
 *              goes there first (M*N fp32).
 *
 * Numerics: the gate and up sums are those of vqv_qgemm (fp32); silu uses
 * the fp32 exponential and an IEEE division.
 */
size_t vqv_qgemm_swiglu_workspace_bytes(int M, int K, int N, int group, vqv_dtype act_dtype);

vqv_status vqv_qgemm_swiglu(const void* x, const uint8_t* wq, const uint16_t* scales,
                            const uint16_t* biases, float* h, int M, int K, int N, int group,
                            vqv_dtype act_dtype, void* workspace, size_t workspace_bytes,
                            void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* VQV_H */

// Internal launch interface between the C-ABI entry points (vqv_api.hip) and
// the kernels (qgemm.hip, verify.hip). Arguments here are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vqv {

enum ActKind { ACT_BF16 = 0, ACT_FP16 = 1, ACT_FP32 = 2 };

// Largest K: a work-group keeps its columns' scale/bias rows in LDS (twice
// as many entries per row for group 32).
constexpr int kMaxK = 16384;
constexpr int kMaxK32 = 8192;

// The greedy verify's arguments. With argmax set, a projection launch is the
// fused verify's first half: each work-group reduces its columns to one
// top-two partial (argmax.h) per row it covers, written to
// partials[row * pgroups + g] (g: the work-group's index among the
// work-groups that cover the row). verify_stage2 (verify.hip) then reduces
// each row's pgroups partials, writes argmax, the margins (when asked) and
// the accept lengths. With argmax NULL a launch is the plain projection.
struct VerifyArgs {
  const int32_t* draft;      // [B, T-1]
  const int32_t* draft_len;  // [B] valid drafts per sequence, or NULL for T-1
  int B, T;
  int32_t* argmax;           // [B*T]
  int32_t* accept_len;       // [B]
  float* margin;             // [B*T] or NULL
  uint4* partials;           // [B*T][pgroups]: (k1, i1, k2, -)
  int pgroups;               // partials per row
};

// y[M,N] = x[M,K] . W^T for 1 <= M <= 64, 64 <= K <= kMaxK, K % 64 == 0.
// Every launcher takes the group shift gs: scales and biases hold one entry
// per group of a row, 64 << gs values for gs = 0 (group 64) and gs = 1
// (group 128, K % 128 == 0), 32 values for gs = -1 (group 32, K <= kMaxK32;
// the whole-tile kernel takes it only where K/128 is a multiple of 4).
// With va.argmax set (va.pgroups = qgemm_verify_groups) the launch also
// writes the fused verify's partials; y may then be NULL (not written).
hipError_t launch_qgemm(const void* x, const uint8_t* wq, const uint16_t* scales,
                        const uint16_t* biases, float* y, int M, int K, int N, int act, int gs,
                        const VerifyArgs& va, hipStream_t stream);

// Whether some kernel takes the problem (its LDS image fits); checked before
// anything is launched. The name of that kernel, or NULL.
bool qgemm_supported(int M, int K, int N, int act, int gs);
const char* qgemm_kernel_name(int M, int K, int N, int act, int gs);

// Partials per row of the fused verify (the work-groups that cover a row of
// the kernel launch_qgemm picks), or 0 when no kernel takes the problem.
int qgemm_verify_groups(int M, int K, int N, int act, int gs);

// The fused verify: the projection with the top-two epilogue, then
// verify_stage2 over its partials (va.partials holds M * qgemm_verify_groups
// 16-byte slots; va.pgroups is set here).
hipError_t launch_qgemm_verify(const void* x, const uint8_t* wq, const uint16_t* scales,
                               const uint16_t* biases, float* y, int M, int K, int N, int act,
                               int gs, const VerifyArgs& va, hipStream_t stream);

// verify_stage2 over va.partials ([B*T][va.pgroups]).
hipError_t launch_verify_finish(const VerifyArgs& va, hipStream_t stream);

// M <= 8 with 16-bit activations, group 64 or 128 (gs 0 or 1), K % 256 == 0:
// qgemm_w4_m8q (qgemm_m8.hip), codes read in whole 128-byte lines. With
// va.argmax it is the fused verify's projection (one partial per row and
// work-group, qgemm_m8q_cols(N) columns per work-group).
bool qgemm_m8q_fits(int M, int K, int act, int gs);
int qgemm_m8q_cols(int N);
hipError_t launch_qgemm_m8q(const void* x, const uint8_t* wq, const uint16_t* scales,
                            const uint16_t* biases, float* y, int M, int K, int N, int act,
                            int gs, const VerifyArgs& va, hipStream_t stream);

// One or two rows of 16-bit activations on the vector ALUs (qgemm_v.hip):
// qgemm_w4_v, a K-major dot2 matvec, qgemm_v_groups(N) work-groups (one
// partial per row and work-group with va.argmax).
bool qgemm_v_fits(int M, int K, int N, int act, int gs);
int qgemm_v_groups(int N);
hipError_t launch_qgemm_v(const void* x, const uint8_t* wq, const uint16_t* scales,
                          const uint16_t* biases, float* y, int M, int K, int N, int act, int gs,
                          const VerifyArgs& va, hipStream_t stream);

// The kernel family a bench or profiler run pins through the environment
// variable VQV_FORCE_VARIANT (read at each plan): "m8" the half-line
// 8-row kernel, "m8q" the whole-line one, "v" the vector-ALU kernel where it
// fits; kVariantAuto when it is unset or names no family. Only the M <= 8
// projection honours it.
enum Variant { kVariantAuto = 0, kVariantM8 = 1, kVariantM8Q = 2, kVariantV = 3 };
Variant forced_variant();

// 9..64 rows in row sets of 16 (bf16/fp16, K within the kernel's LDS
// budget): qgemm_w4_m16 (qgemm_m16.hip). Whether it takes the problem, its
// workers per row set (the fused verify's partials per row), and the launch.
bool qgemm_m16_fits(int M, int K, int act, int gs);
int qgemm_m16_workers(int M, int N);
hipError_t launch_qgemm_m16(const void* x, const uint8_t* wq, const uint16_t* scales,
                            const uint16_t* biases, float* y, int M, int K, int N, int act,
                            int gs, const VerifyArgs& va, hipStream_t stream);

// 17..64 rows at vocabulary widths: one weight stream for every row set
// (qgemm_w4_rows, qgemm_m16.hip); one work-group covers all rows of its
// columns (qgemm_rows_groups(N) work-groups).
bool qgemm_rows_fits(int M, int K, int N, int act);
int qgemm_rows_groups(int N);
hipError_t launch_qgemm_rows(const void* x, const uint8_t* wq, const uint16_t* scales,
                             const uint16_t* biases, float* y, int M, int K, int N, int act,
                             int gs, const VerifyArgs& va, hipStream_t stream);

// Wide outputs (at least two column tiles per wave of one work-group per
// CU): qgemm_w4_wide (qgemm_m16.hip), waves own whole tiles over all of K;
// each row set has qgemm_wide_workers(M) work-groups.
bool qgemm_wide_fits(int M, int K, int N, int act, int gs);
int qgemm_wide_workers(int M);
hipError_t launch_qgemm_wide(const void* x, const uint8_t* wq, const uint16_t* scales,
                             const uint16_t* biases, float* y, int M, int K, int N, int act,
                             int gs, const VerifyArgs& va, hipStream_t stream);

// h[M, N/2] = silu(y[:, :N/2]) * y[:, N/2:] of y = x . W^T, W the stacked
// gate/up weight [N, K]. Fused into the 16-row kernel when
// qgemm_swiglu_fused(); otherwise the projection writes `scratch_y` [M, N]
// and an elementwise kernel forms h.
bool qgemm_swiglu_fused(int M, int K, int N, int act, int gs);
hipError_t launch_qgemm_swiglu(const void* x, const uint8_t* wq, const uint16_t* scales,
                               const uint16_t* biases, float* h, int M, int K, int N, int act,
                               int gs, float* scratch_y, hipStream_t stream);

// Logits per verify work-group (one row, one chunk of columns).
constexpr int kVerifyChunk = 4096;

inline int verify_chunks(int N) { return (N + kVerifyChunk - 1) / kVerifyChunk; }

// Two-stage greedy verify over fp32 logits [B*T, N]; `va.partials` holds
// B*T*verify_chunks(N) 16-byte slots (va.pgroups is not used).
hipError_t launch_verify(const float* logits, int N, const VerifyArgs& va, hipStream_t stream);

}  // namespace vqv

// Internal launch interface between the C-ABI entry points (vqv_api.hip) and
// the kernels (qgemm.hip, verify.hip). Arguments here are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vqv {

enum ActKind { ACT_BF16 = 0, ACT_FP16 = 1, ACT_FP32 = 2 };

// Largest K: a work-group keeps its columns' scale/bias rows in LDS.
constexpr int kMaxK = 16384;

// y[M,N] = x[M,K] . W^T for 1 <= M <= 64, 64 <= K <= kMaxK, K % 64 == 0, group 64.
hipError_t launch_qgemm(const void* x, const uint8_t* wq, const uint16_t* scales,
                        const uint16_t* biases, float* y, int M, int K, int N, int act,
                        hipStream_t stream);

// Logits per verify work-group (one row, one chunk of columns).
constexpr int kVerifyChunk = 4096;

inline int verify_chunks(int N) { return (N + kVerifyChunk - 1) / kVerifyChunk; }

// Two-stage greedy verify; `partials` holds B*T*verify_chunks(N) 8-byte slots.
hipError_t launch_verify(const float* logits, const int32_t* draft, int B, int T, int N,
                         int32_t* argmax, int32_t* accept_len, void* partials,
                         hipStream_t stream);

}  // namespace vqv

// Device helpers of the greedy verify, shared by the standalone verify kernels
// (verify.hip) and the projection kernel's fused epilogue (qgemm.hip).
//
// The target's choice at a verify row is the lowest index of the row maximum
// ("perf: tune DFlash2 M=8 verification for M1 and M2", PR description: the
// greedy verifier compares the target's argmax with each draft). The key
// orders floats as unsigned ints with every NaN above +inf and -0 folded onto
// +0; among equal keys the lower index wins. The pair (key, index) is then
// unique for every row, so any reduction order gives the same result.
#pragma once

#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

namespace vqv {

__device__ __forceinline__ unsigned order_key(float v) {
  unsigned u = __float_as_uint(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0xFFFFFFFFu;  // any NaN: above all
  if (u == 0x80000000u) u = 0u;                              // -0 ties with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Real values map to keys >= 0x007FFFFF, so (0, INT_MAX) is "no candidate".
__device__ __forceinline__ void take_better(unsigned& k, int& i, unsigned k2, int i2) {
  if (k2 > k || (k2 == k && i2 < i)) { k = k2; i = i2; }
}

// (key, index) of the best candidate across the 64 lanes of a wave, in every lane.
__device__ __forceinline__ void wave_best(unsigned& k, int& i) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const unsigned k2 = __shfl_xor(k, off);
    const int i2 = __shfl_xor(i, off);
    take_better(k, i, k2, i2);
  }
}

// (key, index) of the best candidate across each group of 16 lanes, in every
// lane of the group (DPP: swap neighbours, swap pairs, mirror 8, mirror 16).
__device__ __forceinline__ void best16(unsigned& k, int& i) {
#define VQV_BEST16_STEP(ctrl)                                                          \
  {                                                                                    \
    const unsigned k2 = __builtin_amdgcn_update_dpp(0u, k, ctrl, 0xF, 0xF, false);     \
    const int i2 = __builtin_amdgcn_update_dpp(0, i, ctrl, 0xF, 0xF, false);           \
    take_better(k, i, k2, i2);                                                         \
  }
  VQV_BEST16_STEP(0xB1)
  VQV_BEST16_STEP(0x4E)
  VQV_BEST16_STEP(0x141)
  VQV_BEST16_STEP(0x140)
#undef VQV_BEST16_STEP
}

// (key, index) of the best candidate across the 64 lanes of a wave, uniform.
__device__ __forceinline__ void best64(unsigned& k, int& i) {
  best16(k, i);
  unsigned kb = __builtin_amdgcn_readlane(k, 0);
  int ib = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
  for (int r = 16; r < 64; r += 16)
    take_better(kb, ib, __builtin_amdgcn_readlane(k, r), __builtin_amdgcn_readlane(i, r));
  k = kb;
  i = ib;
}

// Accept lengths of the sequences whose rows lanes 0..B*T-1 hold (lane r is
// row r = b*T + i with argmax a and, for i < T-1, draft d fed at row i+1).
// Called by one whole wave, B*T <= 64: the length is the number of leading
// rows whose argmax equals their draft (row T-1 never matches, so it ends
// every sequence's run). Returns, in lane b < B, the accept length of
// sequence b.
__device__ __forceinline__ int accept_lengths_of(int a, int d, int B, int T) {
  const int lane = threadIdx.x & 63;
  const int i = lane % T;
  const bool hit = lane < B * T && i < T - 1 && a == d;
  const unsigned long long hits = __ballot(hit);
  const int first = (lane < B ? lane : 0) * T;
  return __builtin_ctzll(~(hits >> first));
}

// The draft fed after row `lane` (lane = b*T + i, i < T-1), else -1.
__device__ __forceinline__ int draft_of_row(const int32_t* __restrict__ draft, int B, int T) {
  const int lane = threadIdx.x & 63;
  const int b = lane / T, i = lane - b * T;
  return lane < B * T && i < T - 1 ? draft[(size_t)b * (T - 1) + i] : -1;
}

// Same, loading the drafts itself.
__device__ __forceinline__ int accept_lengths(int a, int B, int T,
                                              const int32_t* __restrict__ draft) {
  return accept_lengths_of(a, draft_of_row(draft, B, T), B, T);
}

}  // namespace vqv

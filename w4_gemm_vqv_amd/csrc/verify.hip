// Greedy verify of a DFlash block on gfx950: per-row argmax of fp32 logits,
// then the accept walk of each sequence against its drafts.
//
// Row b*T+i of the logits is sequence b's row i; row 0 is the committed token
// and rows 1..T-1 the drafts ("dspark: fold first-token forward into verify +
// bit-exact M5 Metal decode wins", first commit). Each sequence keeps its own
// accept count ("perf(speculative): commit per-row accepts in batched
// DFlash", commit message).
//
// Stage 1: one 256-thread work-group per (row, chunk of kVerifyChunk logits)
// scans with 16-byte loads and reduces (key, index) pairs (argmax.h) by wave
// shuffles, then across the four waves in LDS.
// Stage 2: one wave per sequence. Lane i reduces row i's chunk partials in
// order, writes argmax, compares with draft i, and a ballot's count of
// trailing ones is the accept length.

#include <limits.h>

#include "argmax.h"
#include "vqv_internal.h"

namespace vqv {
namespace {

template <bool VEC4>
__global__ __launch_bounds__(256) void verify_stage1(const float* __restrict__ logits, int N,
                                                     int nchunks, uint2* __restrict__ part) {
  const int row = blockIdx.x / nchunks;
  const int chunk = blockIdx.x - row * nchunks;
  const float* rp = logits + (size_t)row * N;
  const int beg = chunk * kVerifyChunk;
  const int end = min(N, beg + kVerifyChunk);

  unsigned bk = 0u;
  int bi = INT_MAX;
  if constexpr (VEC4) {
    const float4* rp4 = reinterpret_cast<const float4*>(rp);
    for (int q = (beg >> 2) + threadIdx.x; q < (end >> 2); q += 256) {
      const float4 v = rp4[q];
      take_better(bk, bi, order_key(v.x), 4 * q);
      take_better(bk, bi, order_key(v.y), 4 * q + 1);
      take_better(bk, bi, order_key(v.z), 4 * q + 2);
      take_better(bk, bi, order_key(v.w), 4 * q + 3);
    }
  } else {
    for (int c = beg + threadIdx.x; c < end; c += 256) take_better(bk, bi, order_key(rp[c]), c);
  }

  wave_best(bk, bi);
  __shared__ unsigned sk[4];
  __shared__ int si[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) { sk[wave] = bk; si[wave] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) take_better(bk, bi, sk[w], si[w]);
    part[(size_t)row * nchunks + chunk] = make_uint2(bk, (unsigned)bi);
  }
}

__global__ __launch_bounds__(64) void verify_stage2(const uint2* __restrict__ part, int nchunks,
                                                    const int32_t* __restrict__ draft, int T,
                                                    int32_t* __restrict__ argmax,
                                                    int32_t* __restrict__ accept_len) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  int a = -1;
  if (lane < T) {
    const size_t row = (size_t)b * T + lane;
    const uint2* pr = part + row * nchunks;
    unsigned bk = 0u;
    int bi = INT_MAX;
    for (int c = 0; c < nchunks; ++c) {
      const uint2 v = pr[c];
      take_better(bk, bi, v.x, (int)v.y);
    }
    a = bi;
    argmax[row] = a;
  }
  const bool hit = (lane < T - 1) && (a == draft[(size_t)b * (T - 1) + lane]);
  const unsigned long long miss = ~__ballot(hit);  // lane T-1 never hits, so miss != 0
  if (lane == 0) accept_len[b] = __builtin_ctzll(miss);
}

// The fused projection's second half: wave m reduces row m's per-group
// partials (lanes stride over the groups, then a fixed-order lane tree), and
// wave 0 walks every sequence.
__global__ __launch_bounds__(512) void verify_finish(const uint2* __restrict__ part, int groups,
                                                     const int32_t* __restrict__ draft, int B,
                                                     int T, int32_t* __restrict__ argmax,
                                                     int32_t* __restrict__ accept_len) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rows = B * T;
  const int d = wave == 0 ? draft_of_row(draft, B, T) : -1;
  __shared__ int best[8];
  if (wave < rows) {
    unsigned k = 0u;
    int ix = INT_MAX;
    for (int g = lane; g < groups; g += 64) {
      const uint2 v = part[(size_t)g * 8 + wave];
      take_better(k, ix, v.x, (int)v.y);
    }
    best64(k, ix);
    if (lane == 0) {
      argmax[wave] = ix;
      best[wave] = ix;
    }
  }
  __syncthreads();
  if (wave == 0) {
    const int len = accept_lengths_of(lane < rows ? best[lane] : -1, d, B, T);
    if (lane < B) accept_len[lane] = len;
  }
}

}  // namespace

hipError_t launch_verify_finish(const uint2* partials, int groups, const int32_t* draft, int B,
                                int T, int32_t* argmax, int32_t* accept_len, hipStream_t stream) {
  hipLaunchKernelGGL(verify_finish, dim3(1), dim3(512), 0, stream, partials, groups, draft, B, T,
                     argmax, accept_len);
  return hipGetLastError();
}

hipError_t launch_verify(const float* logits, const int32_t* draft, int B, int T, int N,
                         int32_t* argmax, int32_t* accept_len, void* partials,
                         hipStream_t stream) {
  const int nchunks = verify_chunks(N);
  const dim3 g1(nchunks * B * T);  // B*T*N < 2^31 keeps this below 2^31 / kVerifyChunk
  uint2* part = static_cast<uint2*>(partials);
  if ((N & 3) == 0)
    hipLaunchKernelGGL(verify_stage1<true>, g1, dim3(256), 0, stream, logits, N, nchunks, part);
  else
    hipLaunchKernelGGL(verify_stage1<false>, g1, dim3(256), 0, stream, logits, N, nchunks, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(verify_stage2, dim3(B), dim3(64), 0, stream, part, nchunks, draft, T,
                     argmax, accept_len);
  return hipGetLastError();
}

}  // namespace vqv

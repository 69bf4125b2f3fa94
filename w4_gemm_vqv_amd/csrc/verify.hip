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
// scans with 16-byte loads and reduces top-two partials (argmax.h: best key,
// its lowest index, best other key) across lanes by DPP and across the four
// waves in LDS.
// Stage 2: one work-group per sequence. A wave reduces one row's partials at
// a time (lanes over partials, all loads in flight), writes argmax (and the
// top-1 minus top-2 margin when asked); then wave 0 compares each row's
// argmax with its draft, and a ballot's count of trailing ones is the accept
// length. A sequence with fewer valid drafts (draft_len) stops its walk
// there. The fused projection (qgemm*.hip) writes its per-work-group
// partials in the same [rows][partials per row] layout, and this kernel
// finishes that path too.

#include <limits.h>

#include "argmax.h"
#include "vqv_internal.h"

namespace vqv {
namespace {

template <bool VEC4>
__global__ __launch_bounds__(256) void verify_stage1(const float* __restrict__ logits, int N,
                                                     int nchunks, uint4* __restrict__ part) {
  const int row = blockIdx.x / nchunks;
  const int chunk = blockIdx.x - row * nchunks;
  const float* rp = logits + (size_t)row * N;
  const int beg = chunk * kVerifyChunk;
  const int end = min(N, beg + kVerifyChunk);

  // Every load of the chunk goes out before the first compare.
  Top2 t = top2_none();
  if constexpr (VEC4) {
    constexpr int kPer = kVerifyChunk / (4 * 256);
    const float4* rp4 = reinterpret_cast<const float4*>(rp);
    float4 v[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int q = (beg >> 2) + threadIdx.x + 256 * j;
      const float ninf = -__builtin_inff();
      v[j] = q < (end >> 2) ? rp4[q] : make_float4(ninf, ninf, ninf, ninf);
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int q = (beg >> 2) + threadIdx.x + 256 * j;
      if (q < (end >> 2)) {
        top2_add(t, v[j].x, 4 * q);
        top2_add(t, v[j].y, 4 * q + 1);
        top2_add(t, v[j].z, 4 * q + 2);
        top2_add(t, v[j].w, 4 * q + 3);
      }
    }
  } else {
    constexpr int kPer = kVerifyChunk / 256;
    float v[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int c = beg + threadIdx.x + 256 * j;
      v[j] = c < end ? rp[c] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int c = beg + threadIdx.x + 256 * j;
      if (c < end) top2_add(t, v[j], c);
    }
  }

  t = top2_best64(t);
  __shared__ uint4 sw[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) sw[wave] = top2_pack(t);
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) top2_merge(t, sw[w]);
    part[(size_t)row * nchunks + chunk] = top2_pack(t);
  }
}

// One work-group per sequence: wave w reduces the partials of rows w, w+16,
// ... (lanes over partials), then wave 0 walks the sequence.
constexpr int kStage2Waves = 16;

__global__ __launch_bounds__(64 * kStage2Waves) void verify_stage2(const uint4* __restrict__ part,
                                                                   int nparts, VerifyArgs va) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int T = va.T;
  int d = -1, limit = T - 1;  // limit: raw valid-draft count, clamped at the walk
  if (wave == 0) {
    d = draft_of_row(va.draft + (size_t)b * (T - 1), 1, T);
    limit = draft_len_of_row(va.draft_len ? va.draft_len + b : nullptr, 1, T);
  }
  __shared__ int best[64];
  for (int i = wave; i < T; i += kStage2Waves) {
    const size_t row = (size_t)b * T + i;
    const Top2 t = top2_reduce_strided(part + row * nparts, nparts, 1);
    if (lane == 0) {
      va.argmax[row] = t.i1;
      if (va.margin) va.margin[row] = top2_margin(t);
      best[i] = t.i1;
    }
  }
  __syncthreads();
  if (wave == 0) {
    const int len =
        accept_lengths_of(lane < T ? best[lane] : -1, d, clamp_limit(limit, T), 1, T);
    if (lane == 0) va.accept_len[b] = len;
  }
}

}  // namespace

hipError_t launch_verify_finish(const VerifyArgs& va, hipStream_t stream) {
  hipLaunchKernelGGL(verify_stage2, dim3(va.B), dim3(64 * kStage2Waves), 0, stream, va.partials,
                     va.pgroups, va);
  return hipGetLastError();
}

hipError_t launch_verify(const float* logits, int N, const VerifyArgs& va, hipStream_t stream) {
  const int nchunks = verify_chunks(N);
  const dim3 g1(nchunks * va.B * va.T);  // B*T*N < 2^31 keeps this below 2^31 / kVerifyChunk
  if ((N & 3) == 0)
    hipLaunchKernelGGL(verify_stage1<true>, g1, dim3(256), 0, stream, logits, N, nchunks,
                       va.partials);
  else
    hipLaunchKernelGGL(verify_stage1<false>, g1, dim3(256), 0, stream, logits, N, nchunks,
                       va.partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(verify_stage2, dim3(va.B), dim3(64 * kStage2Waves), 0, stream, va.partials,
                     nchunks, va);
  return hipGetLastError();
}

}  // namespace vqv

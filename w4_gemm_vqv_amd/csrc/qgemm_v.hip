// W4 dequant matvec on the vector ALUs for one or two activation rows: the
// K-major scalar kernel of "perf: tune DFlash2 M=8 verification for M1 and
// M2" (PR description: the scalar kernel beside the matrix-unit ones), set
// beside the MFMA kernels so that a trace can tell which serves a row count.
//
// y[m,n] = sum_g ( s[n,g] * sum_{k in g} x[m,k]*q[n,k] + b[n,g] * sum_{k in g} x[m,k] )
//
// Work split. A wave takes one column at a time; its 64 lanes split the
// column's K/2 code bytes into 16-byte chunks (lane l, round c: bytes
// 16*(64c + l) .. +16, i.e. 32 codes, half of a 64-group). The lane's
// activations for those codes are loaded once per wave and kept in registers
// in the unpack order, with their sums; columns then stream through a ring
// of D columns' codes, scales and biases. Waves take columns round robin, so
// neighbouring waves read neighbouring weight rows.
//
// Per chunk: the codes become the 16-bit floats (c0 + q) by OR-ing them into
// the mantissa of c0 (exact), v_dot2 forms sum x*(c0+q) in fp32, and
//     part = s*acc + (b - c0*s)*xs
// is the chunk's contribution (xs the sum of its 32 activations). Each lane
// adds its chunks in order, the wave adds its lanes by a fixed DPP tree, and
// lane 0 stores y: the results do not depend on timing.
//
// With va.argmax set each wave also keeps the top two of the columns it
// stored (in increasing order), the work-group merges its waves in LDS, and
// thread 0 writes one top-two partial per row and work-group.

#include "argmax.h"
#include "qgemm_common.h"
#include "vqv_internal.h"

namespace vqv {
namespace {

constexpr int kVWaves = 4;                            // waves per work-group

// Sum over the 64 lanes of a wave, in every lane (fixed order: DPP within
// rows of 16, then the four row sums through readlane).
__device__ __forceinline__ float wave_sum(float s) {
  s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                     0, __builtin_bit_cast(int, s), 0xB1, 0xF, 0xF, false));
  s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                     0, __builtin_bit_cast(int, s), 0x4E, 0xF, 0xF, false));
  s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                     0, __builtin_bit_cast(int, s), 0x141, 0xF, 0xF, false));
  s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                     0, __builtin_bit_cast(int, s), 0x140, 0xF, 0xF, false));
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), 48));
  return (r0 + r1) + (r2 + r3);
}

template <int ACT>
__device__ __forceinline__ float dot2(unsigned a, unsigned b, float c) {
  if constexpr (ACT == ACT_FP16)
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c,
                                  false);
  else
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
}

// MR rows (1 or 2), C chunk rounds (ceil(K/2 / 1024)), D columns in flight,
// GS the group shift (0: group 64, 1: group 128).
template <int ACT, int MR, int C, int D, int GS>
__global__ __launch_bounds__(64 * kVWaves) void qgemm_w4_v(
    const void* __restrict__ x, const uint8_t* __restrict__ wq,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases,
    float* __restrict__ y, int M, int K, int N, VerifyArgs va) {
  using TR = ActTraits<ACT>;
  static_assert(TR::parts == 1, "16-bit activations only");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gw = blockIdx.x * kVWaves + wave;          // this wave's index in the grid
  const int W = gridDim.x * kVWaves;
  const unsigned rowbytes = (unsigned)K >> 1;
  const unsigned ME = (unsigned)(K >> 6) >> GS;        // scale entries per row
  const bool fused = va.argmax != nullptr;             // uniform

  unsigned magic;
  asm volatile("v_mov_b32 %0, %1" : "=v"(magic) : "i"(TR::magic));

  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(wq), (short)0, (unsigned)N * rowbytes, kBufferFlags);
  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(scales), (short)0, (unsigned)N * ME * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(biases), (short)0, (unsigned)N * ME * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(x), (short)0, (unsigned)(M * K * 2), kBufferFlags);

  // This lane's chunks: code bytes boff[c] of a row (out of range past the
  // row: zero codes, zero activations, zero scale and bias, adding nothing).
  unsigned woff[C], soff[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const unsigned o = 16u * (64u * c + lane);
    const bool in = o < rowbytes;
    woff[c] = in ? o : kOutOfRange;
    soff[c] = in ? 2u * ((o >> 5) >> GS) : kOutOfRange;  // 32 code bytes per 64-group
  }

  // Activations in the unpack order, and their sums per chunk.
  u32x4 xa[MR][C][4];
  float xs[MR][C];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const bool row = m < M;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const unsigned off = woff[c] == kOutOfRange || !row
                                 ? kOutOfRange
                                 : (unsigned)(m * K * 2) + 4u * woff[c] + 16u * t;
        xa[m][c][t] = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
      }
    }
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int c = 0; c < C; ++c) {
      float s = 0.0f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        s += block_sum<ACT>(xa[m][c][t]);
        xa[m][c][t] = permute_pairs(xa[m][c][t]);
      }
      xs[m][c] = s;
    }

  // The ring: codes and the 16-bit scale and bias of each chunk.
  struct Col {
    u32x4 w[C];
    unsigned s[C], b[C];
  };
  Col ring[D];
  auto load = [&](int n, Col& col) {
    const bool in = n < N;                               // uniform
    const unsigned wso = in ? (unsigned)n * rowbytes : 0x7FF00000u;
    const unsigned sso = in ? (unsigned)n * ME * 2u : 0x7FF00000u;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      col.w[c] = __builtin_amdgcn_raw_buffer_load_b128(wr, woff[c], wso, 2);
      col.s[c] = __builtin_amdgcn_raw_buffer_load_b16(sr, soff[c], sso, 0);
      col.b[c] = __builtin_amdgcn_raw_buffer_load_b16(br, soff[c], sso, 0);
    }
  };
  const int ncols = gw < N ? (N - 1 - gw) / W + 1 : 0;   // columns gw, gw + W, ...
#pragma unroll
  for (int d = 0; d < D; ++d) load(gw + d * W, ring[d]);

  Top2Scan best[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) best[m] = top2_scan_none();

  auto compute = [&](int n, const Col& col) {
    float part[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) part[m] = 0.0f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const float s = half_lo(col.s[c]);
      const float bb = fmaf(-TR::c0, s, half_lo(col.b[c]));
      float acc[MR];
#pragma unroll
      for (int m = 0; m < MR; ++m) acc[m] = 0.0f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const u32x4 q = unpack_codes(col.w[c][t], magic);
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          acc[m] = dot2<ACT>(q.x, xa[m][c][t].x, acc[m]);
          acc[m] = dot2<ACT>(q.y, xa[m][c][t].y, acc[m]);
          acc[m] = dot2<ACT>(q.z, xa[m][c][t].z, acc[m]);
          acc[m] = dot2<ACT>(q.w, xa[m][c][t].w, acc[m]);
        }
      }
#pragma unroll
      for (int m = 0; m < MR; ++m) part[m] = fmaf(s, acc[m], fmaf(bb, xs[m][c], part[m]));
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const float v = wave_sum(part[m]);
      if (m < M) {
        if (lane == 0 && (!fused || y)) y[(size_t)m * N + n] = v;
        if (fused) top2_scan(best[m], v, n, v == v);
      }
    }
  };

  int i = 0;
  for (; i + D <= ncols; i += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      compute(gw + (i + d) * W, ring[d]);
      load(gw + (i + d + D) * W, ring[d]);
    }
  }
#pragma unroll
  for (int d = 0; d < D - 1; ++d)
    if (i + d < ncols) compute(gw + (i + d) * W, ring[d]);

  if (!fused) return;
  // ---- fused greedy verify, first half: each wave's top two per row (the
  // same in every lane), merged over the work-group's waves in wave order.
  __shared__ unsigned cand[kVWaves][MR][3];
  if (lane == 0) {
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const Top2 t = top2_of_scan(best[m]);
      cand[wave][m][0] = t.k1;
      cand[wave][m][1] = (unsigned)t.i1;
      cand[wave][m][2] = t.k2;
    }
  }
  __syncthreads();
  if (threadIdx.x < (unsigned)M) {
    const int m = threadIdx.x;
    Top2 r = top2_none();
#pragma unroll
    for (int w = 0; w < kVWaves; ++w) top2_merge(r, cand[w][m][0], (int)cand[w][m][1], cand[w][m][2]);
    va.partials[(size_t)m * va.pgroups + blockIdx.x] = top2_pack(r);
  }
}

template <int ACT, int MR, int C, int GS>
hipError_t launch_v(const void* x, const uint8_t* wq, const uint16_t* scales,
                    const uint16_t* biases, float* y, int M, int K, int N, const VerifyArgs& va,
                    hipStream_t stream) {
  constexpr int D = MR == 1 ? 4 : 2;
  hipLaunchKernelGGL((qgemm_w4_v<ACT, MR, C, D, GS>), dim3(qgemm_v_groups(N)),
                     dim3(64 * kVWaves), 0, stream, x, wq, scales, biases, y, M, K, N, va);
  return hipGetLastError();
}

template <int ACT, int MR, int GS>
hipError_t launch_v_chunks(const void* x, const uint8_t* wq, const uint16_t* scales,
                           const uint16_t* biases, float* y, int M, int K, int N,
                           const VerifyArgs& va, hipStream_t s) {
  const int chunks = (K / 2 + 1023) / 1024;
  switch (chunks) {
    case 1: return launch_v<ACT, MR, 1, GS>(x, wq, scales, biases, y, M, K, N, va, s);
    case 2: return launch_v<ACT, MR, 2, GS>(x, wq, scales, biases, y, M, K, N, va, s);
    case 3: return launch_v<ACT, MR, 3, GS>(x, wq, scales, biases, y, M, K, N, va, s);
    case 4: return launch_v<ACT, MR, 4, GS>(x, wq, scales, biases, y, M, K, N, va, s);
    default: return hipErrorInvalidValue;              // never launched (qgemm_v_fits)
  }
}

}  // namespace

bool qgemm_v_fits(int M, int K, int N, int act, int gs) {
  // One or two rows of 16-bit activations, group 64 or 128, at most four
  // chunk rounds (K <= 8192) and 32-bit offsets.
  return M <= 2 && act != ACT_FP32 && (gs == 0 || gs == 1) && K % (64 << gs) == 0 &&
         K <= 8192 && (size_t)N * (size_t)(K / 2) < 0x7F000000u;
}

int qgemm_v_groups(int N) {
  // Two work-groups of four waves per CU, fewer when there are fewer columns.
  const int cus = device_cus();
  const int per = (N + kVWaves - 1) / kVWaves;
  return per < 2 * cus ? per : 2 * cus;
}

hipError_t launch_qgemm_v(const void* x, const uint8_t* wq, const uint16_t* scales,
                          const uint16_t* biases, float* y, int M, int K, int N, int act, int gs,
                          const VerifyArgs& va, hipStream_t s) {
  if (act == ACT_BF16) {
    if (M == 1)
      return gs ? launch_v_chunks<ACT_BF16, 1, 1>(x, wq, scales, biases, y, M, K, N, va, s)
                : launch_v_chunks<ACT_BF16, 1, 0>(x, wq, scales, biases, y, M, K, N, va, s);
    return gs ? launch_v_chunks<ACT_BF16, 2, 1>(x, wq, scales, biases, y, M, K, N, va, s)
              : launch_v_chunks<ACT_BF16, 2, 0>(x, wq, scales, biases, y, M, K, N, va, s);
  }
  if (act == ACT_FP16) {
    if (M == 1)
      return gs ? launch_v_chunks<ACT_FP16, 1, 1>(x, wq, scales, biases, y, M, K, N, va, s)
                : launch_v_chunks<ACT_FP16, 1, 0>(x, wq, scales, biases, y, M, K, N, va, s);
    return gs ? launch_v_chunks<ACT_FP16, 2, 1>(x, wq, scales, biases, y, M, K, N, va, s)
              : launch_v_chunks<ACT_FP16, 2, 0>(x, wq, scales, biases, y, M, K, N, va, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace vqv

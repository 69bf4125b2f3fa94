// W4 group-64 dequant GEMM for small M on gfx950 (CDNA4), on MFMA.
//
// y[m,n] = sum_g ( s[n,g] * sum_{k in g} x[m,k]*q[n,k] + b[n,g] * sum_{k in g} x[m,k] )
//
// This is the quantized verify projection of a DFlash block ("perf: tune
// DFlash2 M=8 verification for M1 and M2", PR description). Every packed
// weight byte is read from HBM once for all M rows, as the row-tiled matvec of
// "dspark: fold first-token forward into verify + bit-exact M5 Metal decode
// wins" (first commit, mv_ext row tiles) does for dense weights.
//
// Exactness. A 4-bit code q is turned into the 16-bit float (c0 + q) by
// OR-ing it into the mantissa of c0 (bf16: c0 = 128, fp16: c0 = 1024); that
// value is exact, and so is its product with a bf16 or fp16 activation in the
// fp32 MFMA accumulator. Rounding the dequantized weight s*q + b to 16 bits
// instead would cost far more than the 1e-3 contract. Per group the kernel
// forms acc' = sum x*(c0+q) and xs = sum x (an MFMA against ones) and applies
//     y += s*acc' + (b - c0*s)*xs
// in fp32, which equals s*sum(x*q) + b*sum(x) up to fp32 rounding. fp32
// activations (the W4A32 draft path) are split exactly into three bf16
// terms, hi + mid + lo, each multiplied separately.
//
// Row-split MFMA layout (8 activation rows per row set). v_mfma_f32_16x16x32
// has 16 A rows; rows 0-7 carry the 8 activation rows against group g0 = 2p
// and rows 8-15 the same 8 rows against group g1 = 2p+1, so no output lane is
// padding. A lanes (row i = lane%16, k slot h = lane/16) are non-zero only
// when (i < 8) == (h < 2). Lane (column j = lane%16, slot h) of B reads 16
// contiguous bytes of its column, bytes [16h, 16h+16) of the 64-byte group
// pair p, i.e. 32 codes of group 2p + h/2; dword t of that load feeds MFMA t.
// Unpacking a dword yields the element order (k0,k4),(k1,k5),(k2,k6),(k3,k7);
// the activation operand is permuted to match with v_perm_b32.
//
// Work split. A work-group of WK waves owns 16*TILES columns over all of K;
// wave w takes a contiguous range of group pairs and keeps fp32 partials in
// registers. The partials of the two row-split halves are added across lanes
// and those of the WK waves in LDS in a fixed order, so results are
// deterministic. Weights, scales and biases stream through a two-stage
// register ring (the next pair's loads are in flight while the current pair
// is computed). All loads are buffer loads: a per-lane offset fixed for the
// whole kernel plus a scalar offset per pair. Activations come from L2; A
// lanes that must supply zeros use an out-of-range offset, which the buffer
// unit returns as 0.

#include "vqv_internal.h"

namespace vqv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr unsigned kOutOfRange = 0x80000000u;   // buffer offset that reads as zero
constexpr int kBufferFlags = 0x00020000;        // raw buffer, 32-bit data format

template <int ACT> struct ActTraits;
template <> struct ActTraits<ACT_BF16> {
  static constexpr unsigned magic = 0x43004300u;  // bf16 pair (128, 128)
  static constexpr float c0 = 128.0f;
  static constexpr unsigned ones = 0x3F803F80u;   // bf16 pair (1, 1)
  static constexpr int esz = 2, parts = 1;
  static constexpr bool f16 = false;
};
template <> struct ActTraits<ACT_FP16> {
  static constexpr unsigned magic = 0x64006400u;  // fp16 pair (1024, 1024)
  static constexpr float c0 = 1024.0f;
  static constexpr unsigned ones = 0x3C003C00u;   // fp16 pair (1, 1)
  static constexpr int esz = 2, parts = 1;
  static constexpr bool f16 = true;
};
template <> struct ActTraits<ACT_FP32> {           // three bf16 terms per value
  static constexpr unsigned magic = 0x43004300u;
  static constexpr float c0 = 128.0f;
  static constexpr unsigned ones = 0x3F803F80u;
  static constexpr int esz = 4, parts = 3;
  static constexpr bool f16 = false;
};

template <bool F16>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 8 codes of one dword -> four 16-bit float pairs (c0+q): (n0,n4) (n1,n5) (n2,n6) (n3,n7).
__device__ __forceinline__ u32x4 unpack_codes(unsigned d, unsigned magic) {
  u32x4 q;
  q.x = (d & 0x000F000Fu) | magic;
  q.y = ((d >> 4) & 0x000F000Fu) | magic;
  q.z = ((d >> 8) & 0x000F000Fu) | magic;
  q.w = ((d >> 12) & 0x000F000Fu) | magic;
  return q;
}

// Natural-order 16-bit values (k0,k1)(k2,k3)(k4,k5)(k6,k7) -> unpack order.
__device__ __forceinline__ u32x4 permute_pairs(u32x4 r) {
  u32x4 a;
  a.x = __builtin_amdgcn_perm(r.z, r.x, 0x05040100u);
  a.y = __builtin_amdgcn_perm(r.z, r.x, 0x07060302u);
  a.z = __builtin_amdgcn_perm(r.w, r.y, 0x05040100u);
  a.w = __builtin_amdgcn_perm(r.w, r.y, 0x07060302u);
  return a;
}

// Upper 16 bits of eight fp32 words (k0..k3 in lo4, k4..k7 in hi4), unpack order.
__device__ __forceinline__ u32x4 high_halves(u32x4 lo4, u32x4 hi4) {
  u32x4 a;
  a.x = __builtin_amdgcn_perm(hi4.x, lo4.x, 0x07060302u);  // (k0, k4)
  a.y = __builtin_amdgcn_perm(hi4.y, lo4.y, 0x07060302u);  // (k1, k5)
  a.z = __builtin_amdgcn_perm(hi4.z, lo4.z, 0x07060302u);  // (k2, k6)
  a.w = __builtin_amdgcn_perm(hi4.w, lo4.w, 0x07060302u);  // (k3, k7)
  return a;
}

// Exact split f = hi + mid + lo, each a bf16: truncation leaves a remainder
// that the next term holds exactly. A non-finite f keeps only hi.
__device__ __forceinline__ void split3(unsigned f, unsigned& hi, unsigned& mid, unsigned& lo) {
  hi = f & 0xFFFF0000u;
  if ((f & 0x7F800000u) == 0x7F800000u) { mid = 0; lo = 0; return; }
  const float r1 = __uint_as_float(f) - __uint_as_float(hi);
  mid = __float_as_uint(r1) & 0xFFFF0000u;
  lo = __float_as_uint(r1 - __uint_as_float(mid)) & 0xFFFF0000u;
}

__device__ __forceinline__ float half_bits_to_float(unsigned v) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(v & 0xFFFFu));
}

// Weights, scale and bias of one group pair for every tile of the wave.
template <int TILES>
struct Stage {
  u32x4 w[TILES];
  unsigned s[TILES], b[TILES];
};

// ODDG: K/64 is odd, so the last pair has no second group and the scale and
// bias rows are not dword aligned; that path reads them 16 bits at a time.
template <int ACT, int R, int TILES, int WK, bool ODDG>
__global__ __launch_bounds__(64 * WK) void qgemm_rowsplit(
    const void* __restrict__ x, const uint8_t* __restrict__ wq,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases,
    float* __restrict__ y, int M, int K, int N) {
  using TR = ActTraits<ACT>;
  constexpr int P = TR::parts;
  constexpr int COLS = 16 * TILES;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 15;       // B/C column, A row
  const int h = lane >> 4;       // k slot
  const int half = h >> 1;       // 0: group 2p, 1: group 2p+1
  const int G = K >> 6;
  const int GP = (G + 1) >> 1;
  const int p0 = (wave * GP) / WK;
  const int p1 = ((wave + 1) * GP) / WK;
  const int col0 = blockIdx.x * COLS;
  const int ncols = min(COLS, N - col0);
  const unsigned rowbytes = (unsigned)K >> 1;

  // The code-to-float magic lives in a VGPR so that unpack_codes maps onto
  // v_and_or_b32 (gfx9 VOP3 takes no literal and one scalar operand).
  unsigned magic;
  asm volatile("v_mov_b32 %0, %1" : "=v"(magic) : "i"(TR::magic));
  u32x4 ones;
  ones.x = ones.y = ones.z = ones.w = TR::ones;

  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(wq) + (size_t)col0 * rowbytes, (short)0, ncols * rowbytes, kBufferFlags);
  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(scales) + (size_t)col0 * G, (short)0, ncols * G * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(biases) + (size_t)col0 * G, (short)0, ncols * G * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(x), (short)0, M * K * TR::esz, kBufferFlags);

  // Per-lane offsets, constant over the K loop. Tail columns re-read the last
  // valid column and are never stored.
  unsigned woff[TILES], soff[TILES];
#pragma unroll
  for (int t = 0; t < TILES; ++t) {
    const unsigned n = (unsigned)min(16 * t + j, ncols - 1);
    woff[t] = n * rowbytes + 16u * h;
    soff[t] = ODDG ? (n * G + half) * 2u : n * G * 2u;
  }
  const bool a_lane = ((j < 8) == (h < 2));   // A row j pairs with this lane's group
  unsigned xoff[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int m = 8 * r + (j & 7);
    xoff[r] = (a_lane && m < M) ? (unsigned)((m * K + 64 * half + 32 * (h & 1)) * TR::esz)
                                : kOutOfRange;
  }
  const unsigned sshift = ODDG ? 0u : 16u * half;   // which fp16 of the pair's dword

  float acc[R][TILES][4];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < TILES; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[r][t][e] = 0.0f;

  auto load = [&](int p, Stage<TILES>& st) {
    const bool full = !ODDG || (2 * p + 1 < G);   // uniform
    // A missing second group re-reads the first (its products are discarded).
    const unsigned wshift = full ? 0u : 32u * half;
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      st.w[t] = __builtin_amdgcn_raw_buffer_load_b128(wr, woff[t] - wshift, 64 * p, 0);
      if constexpr (ODDG) {
        const unsigned so = soff[t] - (full ? 0u : 2u * half);
        st.s[t] = __builtin_amdgcn_raw_buffer_load_b16(sr, so, 4 * p, 0);
        st.b[t] = __builtin_amdgcn_raw_buffer_load_b16(br, so, 4 * p, 0);
      } else {
        st.s[t] = __builtin_amdgcn_raw_buffer_load_b32(sr, soff[t], 4 * p, 0);
        st.b[t] = __builtin_amdgcn_raw_buffer_load_b32(br, soff[t], 4 * p, 0);
      }
    }
  };

  auto compute = [&](int p, const Stage<TILES>& st) {
    const bool full = !ODDG || (2 * p + 1 < G);   // uniform
    const bool g_ok = full || half == 0;
    u32x4 bq[4][TILES];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int tt = 0; tt < TILES; ++tt) bq[t][tt] = unpack_codes(st.w[tt][t], magic);
    float sv[TILES], bb[TILES];
#pragma unroll
    for (int tt = 0; tt < TILES; ++tt) {
      sv[tt] = half_bits_to_float(st.s[tt] >> sshift);
      bb[tt] = fmaf(-TR::c0, sv[tt], half_bits_to_float(st.b[tt] >> sshift));
      if (!g_ok) { sv[tt] = 0.0f; bb[tt] = 0.0f; }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const unsigned xo = g_ok ? xoff[r] : kOutOfRange;
      const int xs = 128 * TR::esz * p;
      u32x4 A[4][P];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if constexpr (P == 1) {
          A[t][0] = permute_pairs(__builtin_amdgcn_raw_buffer_load_b128(xr, xo + 16 * t, xs, 0));
        } else {
          const u32x4 f0 = __builtin_amdgcn_raw_buffer_load_b128(xr, xo + 32 * t, xs, 0);
          const u32x4 f1 = __builtin_amdgcn_raw_buffer_load_b128(xr, xo + 32 * t + 16, xs, 0);
          u32x4 hi0, mi0, lo0, hi1, mi1, lo1;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            unsigned a, b, c;
            split3(f0[e], a, b, c);
            hi0[e] = a; mi0[e] = b; lo0[e] = c;
            split3(f1[e], a, b, c);
            hi1[e] = a; mi1[e] = b; lo1[e] = c;
          }
          A[t][0] = high_halves(hi0, hi1);
          A[t][1] = high_halves(mi0, mi1);
          A[t][2] = high_halves(lo0, lo1);
        }
      }
      f32x4 C[TILES], O;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int q = 0; q < P; ++q) {
          const bool first = (t == 0) && (q == 0);
          const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
          O = mfma16x16x32<TR::f16>(A[t][q], ones, first ? zero : O);
#pragma unroll
          for (int tt = 0; tt < TILES; ++tt)
            C[tt] = mfma16x16x32<TR::f16>(A[t][q], bq[t][tt], first ? zero : C[tt]);
        }
      // Group epilogue in fp32: acc += s*C + (b - c0*s)*O.
#pragma unroll
      for (int tt = 0; tt < TILES; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[r][tt][e] = fmaf(sv[tt], C[tt][e], fmaf(bb[tt], O[e], acc[r][tt][e]));
    }
  };

  // Two-stage ring: pair q+1 loads while pair q is computed.
  Stage<TILES> s0, s1;
  const int np = p1 - p0;
  if (np > 0) load(p0, s0);
  for (int q = 0; q < np; q += 2) {
    if (q + 1 < np) load(p0 + q + 1, s1);
    compute(p0 + q, s0);
    if (q + 1 < np) {
      if (q + 2 < np) load(p0 + q + 2, s0);
      compute(p0 + q + 1, s1);
    }
  }

  // Reduce: the two row-split halves (lanes l and l^32), then the WK waves.
  __shared__ float red[WK][R][TILES][8][16];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int tt = 0; tt < TILES; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = acc[r][tt][e] + __shfl_xor(acc[r][tt][e], 32);
        if (lane < 32) red[wave][r][tt][4 * (lane >> 4) + e][j] = v;
      }
  __syncthreads();
  for (int idx = threadIdx.x; idx < R * 8 * COLS; idx += 64 * WK) {
    const int r = idx / (8 * COLS);
    const int rem = idx - r * 8 * COLS;
    const int m = rem / COLS;
    const int c = rem - m * COLS;
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < WK; ++w) s += red[w][r][c >> 4][m][c & 15];
    const int mg = 8 * r + m;
    if (mg < M && c < ncols) y[(size_t)mg * N + col0 + c] = s;
  }
}

template <int ACT, int R, int TILES, int WK>
hipError_t launch_rowsplit(const void* x, const uint8_t* wq, const uint16_t* scales,
                           const uint16_t* biases, float* y, int M, int K, int N,
                           hipStream_t stream) {
  const int cols = 16 * TILES;
  const dim3 grid((N + cols - 1) / cols);
  if ((K >> 6) & 1)
    hipLaunchKernelGGL((qgemm_rowsplit<ACT, R, TILES, WK, true>), grid, dim3(64 * WK), 0, stream,
                       x, wq, scales, biases, y, M, K, N);
  else
    hipLaunchKernelGGL((qgemm_rowsplit<ACT, R, TILES, WK, false>), grid, dim3(64 * WK), 0,
                       stream, x, wq, scales, biases, y, M, K, N);
  return hipGetLastError();
}

template <int ACT>
hipError_t dispatch_rows(const void* x, const uint8_t* wq, const uint16_t* scales,
                         const uint16_t* biases, float* y, int M, int K, int N,
                         hipStream_t s) {
  // fp32 activations carry three operand terms, so they get fewer tiles.
  constexpr int T4 = ACT == ACT_FP32 ? 2 : 4;
  constexpr int T2 = ACT == ACT_FP32 ? 1 : 2;
  if (M <= 8) return launch_rowsplit<ACT, 1, 4, 8>(x, wq, scales, biases, y, M, K, N, s);
  if (M <= 16) return launch_rowsplit<ACT, 2, T4, 8>(x, wq, scales, biases, y, M, K, N, s);
  if (M <= 32) return launch_rowsplit<ACT, 4, T2, 8>(x, wq, scales, biases, y, M, K, N, s);
  return launch_rowsplit<ACT, 8, T2, 8>(x, wq, scales, biases, y, M, K, N, s);
}

}  // namespace

hipError_t launch_qgemm(const void* x, const uint8_t* wq, const uint16_t* scales,
                        const uint16_t* biases, float* y, int M, int K, int N, int act,
                        hipStream_t stream) {
  switch (act) {
    case ACT_BF16: return dispatch_rows<ACT_BF16>(x, wq, scales, biases, y, M, K, N, stream);
    case ACT_FP16: return dispatch_rows<ACT_FP16>(x, wq, scales, biases, y, M, K, N, stream);
    case ACT_FP32: return dispatch_rows<ACT_FP32>(x, wq, scales, biases, y, M, K, N, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vqv

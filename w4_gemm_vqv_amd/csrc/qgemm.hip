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
// forms acc' = sum x*(c0+q) on MFMA and applies, in fp32,
//     y += s*acc' + (b - c0*s)*xs,    xs = sum_{k in g} x,
// which equals s*sum(x*q) + b*sum(x) up to fp32 rounding. fp32 activations
// (the W4A32 draft path) are split exactly into three bf16 terms hi+mid+lo.
//
// Row-split MFMA layout (8 activation rows per row set). v_mfma_f32_16x16x32
// has 16 A rows; rows 0-7 carry the 8 activation rows against group g0 = 2p
// and rows 8-15 the same 8 rows against group g1 = 2p+1, so no output lane is
// padding. A lanes (row i = lane%16, k slot h = lane/16) are non-zero only
// when (i < 8) == (h < 2). Lane (column j = lane%16, slot h) of B reads 16
// contiguous bytes of its column, bytes [16h, 16h+16) of the 64-byte group
// pair p, i.e. 32 codes of group 2p + h/2; dword t of that load feeds MFMA t.
// Unpacking a dword yields the element order (k0,k4),(k1,k5),(k2,k6),(k3,k7).
//
// Work split. A work-group has WN x WK waves and owns `cols` <= 16*TILES*WN
// columns over all of K (the host sizes `cols` so that narrow problems give
// every CU the same share). Wave (wn, wk) owns TILES column tiles and the
// wk-th of WK contiguous ranges of S = ceil(GP/WK) group pairs ("steps"). The
// two row-split halves are added across lanes and the WK partial sums of an
// output in LDS in a fixed order, so results are deterministic.
//
// Memory. Only the weight codes stream from HBM in the K loop, through a
// register ring D steps deep, issued with buffer loads (per-lane offset fixed,
// pair offset scalar). The loop body has no data-dependent branches and, with
// XALL, no barriers: steps past the end read zeros (an out-of-range weight
// offset, a zero activation image, a zero scale/bias pad entry) and add
// exactly nothing. The work-group's scale and bias rows (one contiguous block
// each) are loaded once at the start and kept in LDS as (s, b) fp16 pairs.
// Activations are staged into LDS permuted into the unpack order, with a zero
// slot that the idle A lanes read and the per-group sums xs computed on the
// way: with XALL the whole K range of the work-group once before the loop,
// otherwise KC steps at a time, double buffered, each chunk's loads issued
// with the weights of its first step so that storing it never drains the
// ring.

#include <stdlib.h>
#include <string.h>

#include "argmax.h"
#include "qgemm_common.h"
#include "vqv_internal.h"

namespace vqv {
namespace {

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


template <int ACT>
__device__ __forceinline__ float act16_to_float(unsigned bits16) {
  if constexpr (ACT == ACT_FP16) return half_lo(bits16);
  else return __uint_as_float(bits16 << 16);
}

// LDS image of the activations for one step, row set and term: four t-rows
// (one per MFMA step) of 32 A slots of 16 bytes plus one zero slot.
constexpr int kSlotBytes = 16;
constexpr int kTRowBytes = 33 * kSlotBytes;
constexpr int kPairBytes = 4 * kTRowBytes;

// Dynamic LDS of one work-group. XALL: one activation image per (range, step,
// row set, term) plus one zero image; otherwise two chunk buffers of KC
// steps. Then the row sums (likewise, 16 floats per image group) and the
// (s, b) table, G + 4 dwords per column (the 4 pad entries are zero).
struct LdsLayout {
  int xl, xs, sb, total, sbs, zimg, zxs;
};

// HV (group 32): row sums and table entries per 32-k half, twice as many.
template <int R, int P, int WK, int KC, int WGC, bool XALL, bool HV>
__host__ __device__ inline LdsLayout lds_layout(int G) {
  LdsLayout L{};
  const int GP = (G + 1) >> 1;
  const int S = (GP + WK - 1) / WK;
  const int nimg = XALL ? WK * S * R * P + 1 : 2 * WK * KC * R * P;
  const int nxs = XALL ? WK * S * R + 1 : 2 * WK * KC * R;
  L.xl = 0;
  L.zimg = XALL ? WK * S * R * P : 0;      // index of the zero image (XALL)
  L.xs = nimg * kPairBytes;
  L.zxs = XALL ? WK * S * R : 0;           // index of the zero row-sum group (XALL)
  L.sb = L.xs + nxs * (HV ? 32 : 16) * 4;
  L.sbs = (HV ? 2 * G : G) + 4;
  L.total = L.sb + WGC * L.sbs * 4;
  return L;
}

template <int ACT, int R, int TILES, int WN, int WK, int D, int KC, bool XALL, int GS>
__global__ __launch_bounds__(64 * WN * WK) void qgemm_w4(
    const void* __restrict__ x, const uint8_t* __restrict__ wq,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases,
    float* __restrict__ y, int M, int K, int N, int cols, VerifyArgs va) {
  using TR = ActTraits<ACT>;
  // GS: group 64 << GS for GS >= 0; GS = -1 is group 32, a scale and bias
  // per 32-k half: each step's MFMAs run once per half (the other half's
  // A slots masked to zero) and each half gets its own epilogue.
  constexpr int gs = GS > 0 ? GS : 0;               // table shift of group 128
  constexpr bool HV = GS < 0;
  constexpr int XSF = HV ? 32 : 16;                 // row sums per image group
  constexpr int P = TR::parts;
  constexpr int NT = 64 * WN * WK;                  // threads
  constexpr int WCOLS = 16 * TILES;                 // columns per wave
  constexpr int WGC = WN * WCOLS;                   // column slots per work-group
  constexpr int NS = XALL ? 1 : D / KC;             // staging register sets in flight
  constexpr int XBLK = WK * R * 8 * KC * 16;        // activation blocks per chunk
  constexpr int BPT = XALL ? 4 : (XBLK + NT - 1) / NT;
  constexpr int VPB = TR::esz == 4 ? 2 : 1;         // 16-byte loads per block
  constexpr int SBU = 4;                            // scale/bias units per thread per round
  static_assert(XALL || D % KC == 0, "ring depth must hold whole chunks");

  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % WN;                          // column slice of this wave
  const int wk = wave / WN;                          // K range of this wave
  const int j = lane & 15;       // B/C column, A row
  const int h = lane >> 4;       // k slot
  const int half = h >> 1;       // 0: group 2p, 1: group 2p+1
  const int G = K >> 6;
  const int GP = (G + 1) >> 1;
  const int S = (GP + WK - 1) / WK;                  // steps per K range
  const bool oddg = (G & 1) != 0;
  const unsigned rowbytes = (unsigned)K >> 1;
  const LdsLayout L = lds_layout<R, P, WK, KC, WGC, XALL, HV>(G);
  const int TG = HV ? 2 * G : G;                     // LDS table entries per column
  const int ME = HV ? 2 * G : (G >> gs);             // table entries per column in memory
  unsigned char* xl = lds + L.xl;
  float* xsl = reinterpret_cast<float*>(lds + L.xs);
  unsigned* sbl = reinterpret_cast<unsigned*>(lds + L.sb);

  // Columns: the work-group owns [wg0, wg0 + wgcols). Buffer descriptors
  // depend on the work-group only (they must be scalar). Tail lanes re-read
  // the group's last column and never store.
  const int wg0 = blockIdx.x * cols;
  const int wgcols = min(cols, N - wg0);
  const int wcol = wn * WCOLS;                       // first column of this wave in the group

  unsigned magic;  // in a VGPR so that unpack_codes maps onto v_and_or_b32
  asm volatile("v_mov_b32 %0, %1" : "=v"(magic) : "i"(TR::magic));

  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(wq) + (size_t)wg0 * rowbytes, (short)0, wgcols * rowbytes,
      kBufferFlags);
  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(scales) + (size_t)wg0 * ME, (short)0, wgcols * ME * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(biases) + (size_t)wg0 * ME, (short)0, wgcols * ME * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(x), (short)0, M * K * TR::esz, kBufferFlags);

  unsigned woff[TILES];
#pragma unroll
  for (int t = 0; t < TILES; ++t) {
    const unsigned n = (unsigned)min(wcol + 16 * t + j, wgcols - 1);
    woff[t] = n * rowbytes + 16u * h;
  }
  const bool a_lane = ((j < 8) == (h < 2));          // A row j meets this lane's group
  const int aslot = a_lane ? (h * 8 + (j & 7)) : 32; // the zero slot for idle lanes

  // ---- scale/bias table: issued first, written to LDS after the prologue.
  // Vector path (LDS entries per column a multiple of 8, 16-byte aligned
  // bases): 16-byte units of the work-group's contiguous block; otherwise
  // 16-bit loads.
  const bool sb_vec = (TG % 8) == 0 && ((reinterpret_cast<uintptr_t>(scales) |
                                         reinterpret_cast<uintptr_t>(biases)) & 15) == 0;
  const int sb_units = sb_vec ? wgcols * TG / 8 : wgcols * TG;
  u32x4 sbs[SBU], sbb[SBU];
  auto sb_load = [&](int round) {
#pragma unroll
    for (int u = 0; u < SBU; ++u) {
      const int i = (round * SBU + u) * NT + tid;
      if (sb_vec) {
        const unsigned off = i < sb_units ? (16u * i) >> gs : kOutOfRange;
        sbs[u] = sb_unit_load<GS>(sr, off);
        sbb[u] = sb_unit_load<GS>(br, off);
      } else {
        const unsigned off = i < sb_units ? 2u * ((unsigned)i >> gs) : kOutOfRange;
        sbs[u].x = __builtin_amdgcn_raw_buffer_load_b16(sr, off, 0, 0);
        sbb[u].x = __builtin_amdgcn_raw_buffer_load_b16(br, off, 0, 0);
      }
    }
  };
  auto sb_store = [&](int round) {
#pragma unroll
    for (int u = 0; u < SBU; ++u) {
      const int i = (round * SBU + u) * NT + tid;
      if (i < sb_units) {
        if (sb_vec) {
          const int e0 = 8 * i;                       // first element of the unit
          const int n = e0 / TG, g = e0 - n * TG;
          u32x4 lo, hi;                               // (s_g | b_g << 16) for g .. g+7
          sb_pairs<GS>(sbs[u], sbb[u], lo, hi);
          *reinterpret_cast<u32x4*>(&sbl[n * L.sbs + g]) = lo;
          *reinterpret_cast<u32x4*>(&sbl[n * L.sbs + g + 4]) = hi;
        } else {
          const int n = i / TG, g = i - n * TG;
          sbl[n * L.sbs + g] = (sbs[u].x & 0xFFFFu) | (sbb[u].x << 16);
        }
      }
    }
  };

  // ---- activation staging. A block is 8 consecutive k of one row. With
  // XALL a "chunk" is the whole range (steps 0..S-1 of all WK ranges);
  // otherwise chunk c holds steps [c*KC, c*KC + KC).
  const int csteps = XALL ? S : KC;                  // steps per chunk
  const int cblocks = WK * R * 8 * csteps * 16;       // blocks per chunk
  u32x4 sreg[NS][BPT][VPB];
  auto block_coords = [&](int bi, int& ks, int& mm, int& kb) {
    ks = bi / (R * 8 * csteps * 16);                  // K range
    const int rem = bi - ks * (R * 8 * csteps * 16);
    mm = rem / (16 * csteps);                         // activation row 0..8R-1
    kb = rem - mm * 16 * csteps;                      // 8-value block within the chunk
  };
  auto stage_load = [&](int c, int set, int base) {
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      const int bi = base + tid + i * NT;
      int ks, mm, kb;
      block_coords(bi, ks, mm, kb);
      const int q = c * csteps + (kb >> 4);           // step within the range
      const int p = ks * S + q;                       // group pair
      const int k = 128 * p + 8 * (kb & 15);
      const bool ok = bi < cblocks && mm < M && q < S && k < K;
      const unsigned off = ok ? (unsigned)((mm * K + k) * TR::esz) : kOutOfRange;
#pragma unroll
      for (int v = 0; v < VPB; ++v)
        sreg[set][i][v] = __builtin_amdgcn_raw_buffer_load_b128(xr, off + 16 * v, 0, 0);
    }
  };
  auto stage_store = [&](int set, int buf, int base) {
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      const int bi = base + tid + i * NT;
      int ks, mm, kb;
      block_coords(bi, ks, mm, kb);
      const int pp = kb >> 4;                         // step within the chunk
      const int r128 = 8 * (kb & 15);                 // offset within the pair's 128 k
      const int hf = r128 >> 6, hh = (r128 >> 5) & 1, t = (r128 >> 3) & 3;
      const int r = mm >> 3;
      const int slot = (hf * 2 + hh) * 8 + (mm & 7);
      // Sum of the block; the 8 blocks of one (row, group) are 8 adjacent lanes.
      float s8 = 0.0f;
      if constexpr (P == 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s8 += act16_to_float<ACT>(sreg[set][i][0][e] & 0xFFFFu);
          s8 += act16_to_float<ACT>(sreg[set][i][0][e] >> 16);
        }
      } else {
#pragma unroll
        for (int v = 0; v < 2; ++v)
#pragma unroll
          for (int e = 0; e < 4; ++e) s8 += __uint_as_float(sreg[set][i][v][e]);
      }
      s8 += __shfl_xor(s8, 1);
      s8 += __shfl_xor(s8, 2);                        // a 32-k half: 4 lanes
      if constexpr (!HV) s8 += __shfl_xor(s8, 4);     // a 64-group: 8 lanes
      if (bi < cblocks) {
        const int grp = ((buf * WK + ks) * csteps + pp) * R + r;   // (image group)
        unsigned char* dst = xl + grp * P * kPairBytes + t * kTRowBytes + slot * kSlotBytes;
        if constexpr (P == 1) {
          *reinterpret_cast<u32x4*>(dst) = permute_pairs(sreg[set][i][0]);
        } else {
          u32x4 hi0, mi0, lo0, hi1, mi1, lo1;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            unsigned a, b, cc;
            split3(sreg[set][i][0][e], a, b, cc);
            hi0[e] = a; mi0[e] = b; lo0[e] = cc;
            split3(sreg[set][i][1][e], a, b, cc);
            hi1[e] = a; mi1[e] = b; lo1[e] = cc;
          }
          *reinterpret_cast<u32x4*>(dst) = high_halves(hi0, hi1);
          *reinterpret_cast<u32x4*>(dst + kPairBytes) = high_halves(mi0, mi1);
          *reinterpret_cast<u32x4*>(dst + 2 * kPairBytes) = high_halves(lo0, lo1);
        }
        if constexpr (HV) {
          if ((bi & 3) == 0) xsl[((grp * 2 + hf) * 2 + hh) * 8 + (mm & 7)] = s8;
        } else {
          if ((bi & 7) == 0) xsl[(grp * 2 + hf) * 8 + (mm & 7)] = s8;
        }
      }
    }
  };

  // ---- weight ring: step q of this wave is pair wk*S + q; out-of-range steps
  // (past this range or past GP) read zeros.
  u32x4 st[D][TILES];
  auto load = [&](int q, u32x4 (&w)[TILES]) {
    const int p = wk * S + q;
    const bool in = q < S && p < GP;                 // uniform
    const bool full = !oddg || (2 * p + 1 < G);
    const unsigned wshift = full ? 0u : 32u * half;  // a missing g1 re-reads g0
#pragma unroll
    for (int t = 0; t < TILES; ++t)
      w[t] = __builtin_amdgcn_raw_buffer_load_b128(wr, in ? woff[t] - wshift : kOutOfRange,
                                                   64 * (in ? p : 0), 0);
  };

  float acc[R][TILES][4];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < TILES; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[r][t][e] = 0.0f;

  // One step: A and xs from this step's image group (the zero group past the
  // range), (s, b) of this lane's group (the zero pad entry past the range),
  // four MFMAs per tile and row set, then acc += s*C + (b - c0*s)*xs.
  auto compute = [&](int q, const u32x4 (&w)[TILES], int buf) {
    const int p = wk * S + q;
    const bool in = q < S;                            // uniform
    const int grp0 = XALL ? (in ? (wk * S + q) * R : L.zxs) : ((buf * WK + wk) * KC + q % KC) * R;
    const int sbi = in ? min(2 * p + half, G) : G;
    u32x4 bq[4][TILES];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int tt = 0; tt < TILES; ++tt) bq[t][tt] = unpack_codes(w[tt][t], magic);
    // (s, b) of the lane's group, or of its two halves (HV; sbi = G is the
    // zero pad either way).
    constexpr int NH = HV ? 2 : 1;
    float sv[NH][TILES], bb[NH][TILES];
#pragma unroll
    for (int hv = 0; hv < NH; ++hv)
#pragma unroll
      for (int tt = 0; tt < TILES; ++tt) {
        const unsigned v = sbl[(wcol + 16 * tt + j) * L.sbs + NH * sbi + hv];
        sv[hv][tt] = half_lo(v);
        bb[hv][tt] = fmaf(-TR::c0, sv[hv][tt], half_hi(v));
      }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int grp = XALL && !in ? L.zxs : grp0 + r;
      const int img = XALL && !in ? L.zimg : (grp0 + r) * P;
      const unsigned char* ab = xl + img * kPairBytes + aslot * kSlotBytes;
      f32x4 xs[NH];
#pragma unroll
      for (int hv = 0; hv < NH; ++hv)
        xs[hv] = *reinterpret_cast<const f32x4*>(
            &xsl[((grp * 2 + half) * NH + hv) * 8 + 4 * (h & 1)]);
      f32x4 C[NH][TILES];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int u = 0; u < P; ++u) {
          const unsigned char* ap = XALL && !in ? ab : ab + u * kPairBytes;
          const u32x4 A = *reinterpret_cast<const u32x4*>(ap + t * kTRowBytes);
          const bool first = (t == 0) && (u == 0);
          const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int hv = 0; hv < NH; ++hv) {
            // HV: lanes of k slot h hold the 32-k half h & 1 of their group.
            const u32x4 zA = {0u, 0u, 0u, 0u};
            const u32x4 Ah = !HV || (h & 1) == hv ? A : zA;
#pragma unroll
            for (int tt = 0; tt < TILES; ++tt)
              C[hv][tt] = mfma16x16x32<TR::f16>(Ah, bq[t][tt], first ? zero : C[hv][tt]);
          }
        }
#pragma unroll
      for (int hv = 0; hv < NH; ++hv)
#pragma unroll
        for (int tt = 0; tt < TILES; ++tt)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[r][tt][e] = fmaf(sv[hv][tt], C[hv][tt][e],
                                 fmaf(bb[hv][tt], xs[hv][e], acc[r][tt][e]));
    }
  };

  // ---- prologue: zero slots, zero image and pads, the scale/bias table, the
  // first D steps of weights, the activations.
  {
    const int nimg = XALL ? L.zimg : 2 * WK * KC * R * P;
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int i = tid; i < nimg * 4; i += NT)
      *reinterpret_cast<u32x4*>(xl + (i >> 2) * kPairBytes + (i & 3) * kTRowBytes +
                                32 * kSlotBytes) = z;
    if constexpr (XALL) {
      for (int i = tid; i < kPairBytes / 16; i += NT)
        *reinterpret_cast<u32x4*>(xl + L.zimg * kPairBytes + 16 * i) = z;
      if (tid < XSF) xsl[L.zxs * XSF + tid] = 0.0f;
    }
    for (int i = tid; i < WGC * 4; i += NT) sbl[(i >> 2) * L.sbs + TG + (i & 3)] = 0u;
  }
  sb_load(0);
#pragma unroll
  for (int d = 0; d < D; ++d) {
    if constexpr (!XALL)
      if (d % KC == 0) stage_load(d / KC, d / KC, 0);
    load(d, st[d]);
  }
  if constexpr (XALL) {
    for (int base = 0; base < cblocks; base += BPT * NT) {
      stage_load(0, 0, base);
      stage_store(0, 0, base);
    }
  }
  sb_store(0);
  for (int round = 1; round * SBU * NT < sb_units; ++round) {  // only for very wide tables
    sb_load(round);
    sb_store(round);
  }
  if constexpr (!XALL) stage_store(0, 0, 0);
  __syncthreads();

  // ---- main loop: straight-line body, D steps per iteration.
  const int steps = (S + D - 1) / D * D;
  for (int qb = 0; qb < steps; qb += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int q = qb + d;
      compute(q, st[d], XALL ? 0 : (q / KC) & 1);
      load(q + D, st[d]);
      if constexpr (!XALL) {
        if (d % KC == 0) stage_load((q + D) / KC, d / KC, 0);
        if (d % KC == KC - 1) {
          stage_store(((d + 1) / KC) % NS, ((q + 1) / KC) & 1, 0);
          __syncthreads();
        }
      }
    }
  }

  // ---- reduce: the two row-split halves (lanes l and l^32), then the WK
  // ranges in order, through LDS (reused once every wave is past the loop).
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds);        // [WK][WN][R][TILES][8][16]
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int tt = 0; tt < TILES; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = acc[r][tt][e] + __shfl_xor(acc[r][tt][e], 32);
        if (lane < 32)
          red[((((wk * WN + wn) * R + r) * TILES + tt) * 8 + 4 * (lane >> 4) + e) * 16 + j] = v;
      }
  __syncthreads();
  // With the fused verify, the 16 outputs idx .. idx + 15 (one row, 16
  // columns, held by 16 adjacent lanes) reduce to one top-two candidate in
  // slot idx / 16 after the partial sums.
  const bool fused = va.argmax != nullptr;           // uniform
  constexpr int OUTS = WN * R * TILES * 128;
  unsigned* cand = reinterpret_cast<unsigned*>(red + WK * OUTS);  // [OUTS / 16] x (k1, i1, k2)
  for (int idx = tid; idx < OUTS; idx += NT) {
    float s = 0.0f;
#pragma unroll
    for (int k2 = 0; k2 < WK; ++k2) s += red[k2 * OUTS + idx];
    const int jj = idx & 15;
    const int m8 = (idx >> 4) & 7;
    const int rest = idx >> 7;                       // (wn * R + r) * TILES + tt
    const int tt = rest % TILES;
    const int r = (rest / TILES) % R;
    const int wn2 = rest / (TILES * R);
    const int m = 8 * r + m8;
    const int c = wn2 * WCOLS + 16 * tt + jj;
    const bool out = m < M && c < wgcols;
    if (out && (!fused || y)) y[(size_t)m * N + wg0 + c] = s;
    if (fused) {                                     // uniform per 16 lanes
      Top2 t = top2_none();
      if (out) top2_add(t, s, wg0 + c);
      top2_best16(t);
      if (jj == 0) {
        unsigned* q = cand + (idx >> 4) * 3;
        q[0] = t.k1;
        q[1] = (unsigned)t.i1;
        q[2] = t.k2;
      }
    }
  }
  if (!fused) return;

  // ---- fused greedy verify, first half: thread m < M merges row m's
  // candidates, slots ((wn * R + m / 8) * TILES + tt) * 8 + m % 8, and writes
  // the work-group's partial for that row.
  __syncthreads();
  if (tid < M) {
    const int r = tid >> 3, m8 = tid & 7;
    Top2 b = top2_none();
#pragma unroll
    for (int wn2 = 0; wn2 < WN; ++wn2)
#pragma unroll
      for (int tt = 0; tt < TILES; ++tt) {
        const unsigned* q = cand + (((wn2 * R + r) * TILES + tt) * 8 + m8) * 3;
        top2_merge(b, q[0], (int)q[1], q[2]);
      }
    va.partials[(size_t)tid * va.pgroups + blockIdx.x] = top2_pack(b);
  }
}


// Group 32 in qgemm_w4_m8: lane l and lane l ^ 16 hold the two 32-k halves
// of one group (k slots 2g and 2g + 1), dwords t = the 8-value blocks t of
// the half. After the exchange, dword t of every lane holds block
// 2 (t % 2) + (h % 2) of half t / 2, so MFMAs 0-1 of a step see only the
// first halves and MFMAs 2-3 only the second.
__device__ __forceinline__ u32x4 pair_halves(const u32x4& w) {
  const auto a = __builtin_amdgcn_permlane16_swap(w.x, w.y, false, false);
  const auto b = __builtin_amdgcn_permlane16_swap(w.z, w.w, false, false);
  return u32x4{a[0], b[0], a[1], b[1]};
}

// LDS of qgemm_w4_m8: GP activation images and one zero image (more when the
// staging rounds are padded), the row sums (16 floats per image), the (s, b)
// table (G + 4 dwords per column), the partial-sum slots (two 8x16 tiles per
// wave), then each run's first and last tile.
struct M8Layout {
  int xs, sb, sbs, red, runs, total;
};

// HV (group 32): row sums and table entries per 32-k half, twice as many.
__host__ __device__ inline M8Layout m8_layout(int G, int WGC, int NW, int XB, bool HV) {
  const int GP = (G + 1) >> 1;
  const int rounds = (2 * GP + NW - 1) / NW;             // staging rounds per wave
  const int padded = (rounds + XB - 1) / XB * XB * NW;   // groups the staging writes
  const int nimg = GP + 1 > padded / 2 ? GP + 1 : padded / 2;
  M8Layout L{};
  L.xs = nimg * kPairBytes;
  L.sb = L.xs + nimg * (HV ? 32 : 16) * 4;
  L.sbs = (HV ? 2 * G : G) + 4;
  L.red = L.sb + WGC * L.sbs * 4;
  L.runs = L.red + NW * 2 * 128 * 4;
  L.total = L.runs + NW * 2 * 4;
  return L;
}

// ---------------------------------------------------------------------------
// One row set (M <= 8), 16-bit activations, the work-group's whole K range in
// LDS. With FUSED the greedy verify runs in the epilogue (VerifyArgs). Same per-step arithmetic as qgemm_w4 with R = 1; the work split and
// the schedule differ:
//  * Work is cut into blocks of DB consecutive group pairs of one column
//    tile; the work-group's blocks, tile-major, are dealt to its NW waves as
//    contiguous runs of equal length (+-1), so every SIMD carries the same
//    load whatever the tile count. Addresses are set once per block; the
//    steps of a block use immediate offsets. A run spans at most two tiles:
//    a wave flushes its partial sums to LDS when its tile changes, and the
//    final reduction adds the flushed tiles in wave order (a fixed order:
//    results are deterministic).
//  * The weight ring holds RB blocks (D = RB*DB steps). The activation and
//    scale/bias loads go out first with D0 ring steps; the other ring steps
//    are issued one per staging round. Loads retire in order, so staging
//    waits for the activations only; a full ring issued up front would queue
//    ahead of the activation and table reads in the memory system, and a
//    wave that issues more loads than the memory queue holds stalls until
//    they drain, which would hold up its staging.
//  * Staging needs no division: lane (e = lane%8, row = lane/8) of wave w
//    moves the 8 values k = 64g + 8e.. of group g = w + NW*i; the row sums
//    come from dot products with ones and three DPP adds.
//  * In the loop the LDS operands of step q+1 are read while step q runs,
//    and step q's epilogue waits until step q+1's MFMAs are issued.
//  * A missing odd last group reads whatever codes follow (or zeros past
//    the buffer): its activations, row sum, scale and bias are all zero, so
//    it adds exactly nothing. Columns past the work-group's read zeros and
//    are never stored.
template <int ACT, int NW, int TW, int DB, int RB, int D0, int XB, bool FUSED, int GS>
__global__ __launch_bounds__(64 * NW) void qgemm_w4_m8(
    const void* __restrict__ x, const uint8_t* __restrict__ wq,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases,
    float* __restrict__ y, int M, int K, int N, int cols, VerifyArgs va) {
  using TR = ActTraits<ACT>;
  // GS: group 64 << GS for GS >= 0. GS = -1 is group 32: the codes of a
  // lane pair (lanes l and l + 16) are exchanged so that MFMAs 0-1 of a step
  // cover the first 32-k half of each group and MFMAs 2-3 the second; each
  // half accumulates apart and takes its own scale, bias and row sum.
  constexpr int gs = GS > 0 ? GS : 0;               // table shift of group 128
  constexpr bool HV = GS < 0;
  constexpr int NH = HV ? 2 : 1;                    // scaled partial sums per group
  constexpr int XSF = HV ? 32 : 16;                 // row sums per activation image
  static_assert(TR::parts == 1, "16-bit activations only");
  static_assert(TW <= NW, "a run must span at most two tiles");
  static_assert(NW >= 8, "the partial-sum slots double as an 8 KB write sink");
  constexpr int D = DB * RB;
  static_assert(D0 >= 0 && D0 <= D, "prologue ring depth");
  constexpr int NT = 64 * NW;
  constexpr int WGC = 16 * TW;
  constexpr int SBU = 2;                            // table units per thread per round
  constexpr unsigned kSkip = 0x7FF00000u;           // scalar offset that reads as zero

  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15;
  const int h = lane >> 4;
  const int half = h >> 1;
  const int G = K >> 6;
  const int GP = (G + 1) >> 1;                       // a multiple of DB (host)
  const int bpt = GP / DB;                           // blocks per tile
  const unsigned rowbytes = (unsigned)K >> 1;
  const M8Layout L = m8_layout(G, WGC, NW, XB, HV);
  const int TG = HV ? 2 * G : G;                     // LDS table entries per column
  const int ME = HV ? 2 * G : (G >> gs);             // table entries per column in memory
  unsigned char* xl = lds;
  float* xsl = reinterpret_cast<float*>(lds + L.xs);
  unsigned* sbl = reinterpret_cast<unsigned*>(lds + L.sb);
  float* red = reinterpret_cast<float*>(lds + L.red);
  int* run_tiles = reinterpret_cast<int*>(lds + L.runs);

  const int wg0 = blockIdx.x * cols;
  const int wgcols = min(cols, N - wg0);
  const int tiles = (wgcols + 15) >> 4;
  const int nblk = tiles * bpt;
  const int b0 = (wave * nblk) / NW;
  const int nb = ((wave + 1) * nblk) / NW - b0;
  const int tfirst = b0 / bpt;

  unsigned magic;
  asm volatile("v_mov_b32 %0, %1" : "=v"(magic) : "i"(TR::magic));

  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(wq) + (size_t)wg0 * rowbytes, (short)0, wgcols * rowbytes,
      kBufferFlags);
  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(scales) + (size_t)wg0 * ME, (short)0, wgcols * ME * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(biases) + (size_t)wg0 * ME, (short)0, wgcols * ME * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(x), (short)0, M * K * 2, kBufferFlags);

  const unsigned woff = (unsigned)j * rowbytes + 16u * h;
  const bool a_lane = ((j < 8) == (h < 2));
  const int aslot = a_lane ? (h * 8 + (j & 7)) : 32;

  // ---- activation staging, batch by batch (one batch up to K = 64*NW*XB).
  const int ngrp = 2 * GP;                           // groups incl. a missing odd one
  const int rounds = (ngrp + NW - 1) / NW;
  const int e8 = lane & 7;                           // 8-value block within the group
  const int mm = lane >> 3;                          // activation row
  u32x4 xv[XB];
  auto x_load = [&](int bb) {
#pragma unroll
    for (int i = 0; i < XB; ++i) {
      const int g = wave + NW * (bb + i);
      const int k = 64 * g + 8 * e8;
      const bool ok = mm < M && k < K;
      xv[i] = __builtin_amdgcn_raw_buffer_load_b128(
          xr, ok ? (unsigned)((mm * K + k) * 2) : kOutOfRange, 0, 0);
    }
  };
  // Block e8 feeds MFMA t from k slot h (high bit: the group in the pair):
  // t = e8 % 4 and h low bit = e8 / 4, or with HV t = 2 (e8 / 4) + (e8 % 4) / 2
  // and h low bit = e8 % 2 (the order the exchanged codes arrive in).
  const unsigned xl_lane =
      HV ? (2 * (e8 >> 2) + ((e8 & 3) >> 1)) * kTRowBytes + ((e8 & 1) * 8 + mm) * kSlotBytes
         : (e8 & 3) * kTRowBytes + ((e8 >> 2) * 8 + mm) * kSlotBytes;
  // The image area is padded (m8_layout) so that every round of every batch
  // has a slot: rounds past the last group stage zeros (their loads read
  // past K) into images that are never read, or into the zero image.
  auto x_store_round = [&](int bb, int i) {
    const int g = wave + NW * (bb + i);               // uniform
    // Sum of the row's 64 values (the eight lanes of (row, group) all hold
    // it), or with HV of a half's 32 values (the four lanes of (row, group,
    // half)).
    const float s8 = HV ? sum4_lanes(block_sum<ACT>(xv[i])) : sum8_lanes(block_sum<ACT>(xv[i]));
    *reinterpret_cast<u32x4*>(xl + (g >> 1) * kPairBytes + (g & 1) * 16 * kSlotBytes +
                              xl_lane) = permute_pairs(xv[i]);
    xsl[HV ? (g * 2 + (e8 >> 2)) * 8 + mm : g * 8 + mm] = s8;
  };
  auto x_store = [&](int bb) {
#pragma unroll
    for (int i = 0; i < XB; ++i) x_store_round(bb, i);
  };

  // ---- scale/bias table (as in qgemm_w4).
  const bool sb_vec = (TG % 8) == 0 && ((reinterpret_cast<uintptr_t>(scales) |
                                         reinterpret_cast<uintptr_t>(biases)) & 15) == 0;
  const int sb_units = sb_vec ? wgcols * TG / 8 : wgcols * TG;
  u32x4 sbs[SBU], sbb[SBU];
  auto sb_load = [&](int round) {
#pragma unroll
    for (int u = 0; u < SBU; ++u) {
      const int i = (round * SBU + u) * NT + tid;
      if (sb_vec) {
        const unsigned off = i < sb_units ? (16u * i) >> gs : kOutOfRange;
        sbs[u] = sb_unit_load<GS>(sr, off);
        sbb[u] = sb_unit_load<GS>(br, off);
      } else {
        const unsigned off = i < sb_units ? 2u * ((unsigned)i >> gs) : kOutOfRange;
        sbs[u].x = __builtin_amdgcn_raw_buffer_load_b16(sr, off, 0, 0);
        sbb[u].x = __builtin_amdgcn_raw_buffer_load_b16(br, off, 0, 0);
      }
    }
  };
  // n = e / TG as a high product with ceil(2^32 / TG) (exact for
  // e < 2^32 / TG); TG = 1 has no 32-bit reciprocal and is handled directly.
  const unsigned g_recip = 0xFFFFFFFFu / (unsigned)TG + 1u;
  auto div_g = [&](unsigned e) { return TG == 1 ? e : __umulhi(e, g_recip); };
  auto sb_store = [&](int round) {
#pragma unroll
    for (int u = 0; u < SBU; ++u) {
      const int i = (round * SBU + u) * NT + tid;
      const bool ok = i < sb_units;
      if (sb_vec) {
        const unsigned e0 = 8u * (unsigned)i;         // first element of the unit
        const unsigned n = div_g(e0), g = e0 - n * (unsigned)TG;
        u32x4 lo, hi;                                 // (s_g | b_g << 16) for g .. g+7
        sb_pairs<GS>(sbs[u], sbb[u], lo, hi);
        // Units past the table write into the partial-sum slots (8 KB, not
        // read before the end of the loop).
        const unsigned o = ok ? (unsigned)L.sb + 4u * (n * (unsigned)L.sbs + g)
                              : (unsigned)L.red + 32u * ((unsigned)tid & 255u);
        *reinterpret_cast<u32x4*>(lds + o) = lo;
        *reinterpret_cast<u32x4*>(lds + o + 16) = hi;
      } else if (ok) {
        const unsigned n = div_g((unsigned)i), g = (unsigned)i - n * (unsigned)TG;
        sbl[n * L.sbs + g] = (sbs[u].x & 0xFFFFu) | (sbb[u].x << 16);
      }
    }
  };

  // ---- blocks of the run. Block i of this wave (0 <= i < nb) is block
  // b0 + i of the work-group: tile t, pairs p .. p + DB - 1. Blocks are
  // walked incrementally (no division in the loop).
  struct Blk {
    int t, p, left;                                  // left: blocks of the run from here on
  };
  const Blk kfirst = {tfirst, (b0 - tfirst * bpt) * DB, nb};
  auto next = [&](Blk k) {
    k.p += DB;
    k.t += k.p == GP;
    k.p = k.p == GP ? 0 : k.p;
    k.left -= 1;
    return k;
  };
  u32x4 st[D];
  // Scalar offset of block k's codes (past the run: an offset that reads zeros).
  auto codes_at = [&](const Blk& k) {
    return k.left > 0 ? (unsigned)k.t * 16u * rowbytes + 64u * (unsigned)k.p : kSkip;
  };
  // Step d of the block at scalar offset `so` into a ring slot.
  auto load = [&](unsigned so, int d, u32x4& w) {
    w = __builtin_amdgcn_raw_buffer_load_b128(wr, woff + 64u * d, so, 0);
  };

  // ---- prologue.
  Blk kl = kfirst;                                    // the next block to load
  auto ring_load = [&](int d) {                       // ring slot d, in slot order
    load(codes_at(kl), d % DB, st[d]);
    if (d % DB == DB - 1) kl = next(kl);
  };
  x_load(0);
  sb_load(0);
#pragma unroll
  for (int d = 0; d < D0; ++d) ring_load(d);
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int i = tid; i < GP * 4; i += NT)
      *reinterpret_cast<u32x4*>(xl + (i >> 2) * kPairBytes + (i & 3) * kTRowBytes +
                                32 * kSlotBytes) = z;
    for (int i = tid; i < kPairBytes / 16; i += NT)
      *reinterpret_cast<u32x4*>(xl + GP * kPairBytes + 16 * i) = z;
    if (tid < XSF) xsl[GP * XSF + tid] = 0.0f;
    for (int i = tid; i < WGC * 4; i += NT) sbl[(i >> 2) * L.sbs + TG + (i & 3)] = 0u;
  }
  // The first batch is staged round by round, one more ring slot issued
  // before each round, so the weight stream starts while staging runs.
#pragma unroll
  for (int i = 0; i < XB; ++i) {
    if (D0 + i < D) ring_load(D0 + i);
    x_store_round(0, i);
  }
  sb_store(0);
  for (int bb = XB; bb < rounds; bb += XB) {          // K above 64*NW*XB only
    x_load(bb);
    x_store(bb);
  }
  for (int round = 1; round * SBU * NT < sb_units; ++round) {
    sb_load(round);
    sb_store(round);
  }
#pragma unroll
  for (int d = D0 + XB; d < D; ++d) ring_load(d);
  if (lane == 0) {                                    // this run's tiles, for the reduction
    run_tiles[2 * wave] = nb > 0 ? tfirst : 1 << 30;
    run_tiles[2 * wave + 1] = nb > 0 ? (b0 + nb - 1) / bpt : -1;
  }
  __syncthreads();

  // ---- main loop.
  const unsigned char* abase = xl + aslot * kSlotBytes;
  const float* xsbase = xsl + half * (XSF / 2) + 4 * (h & 1);
  const unsigned* sbbase = sbl + j * L.sbs + NH * half;
  struct Ops { u32x4 A[4]; f32x4 xs[NH]; unsigned sb[NH]; };
  // LDS bases of block k (the zero image and pad past the run); step d of a
  // block reads at immediate offsets from them.
  struct Base {
    const unsigned char* a;
    const float* xs;
    const unsigned* sb;
  };
  auto base_of = [&](const Blk& k) {
    const bool in = k.left > 0;                      // uniform
    const int img = in ? k.p : GP;
    Base b;
    b.a = abase + img * kPairBytes;
    b.xs = xsbase + img * XSF;
    b.sb = sbbase + (in ? k.t * 16 * L.sbs + 2 * NH * k.p : (HV ? TG : G + 2));
    return b;
  };
  auto fetch = [&](const Base& b, int d, Ops& o) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
      o.A[t] = *reinterpret_cast<const u32x4*>(b.a + d * kPairBytes + t * kTRowBytes);
#pragma unroll
    for (int hv = 0; hv < NH; ++hv) {
      o.xs[hv] = *reinterpret_cast<const f32x4*>(b.xs + d * XSF + 8 * hv);
      o.sb[hv] = b.sb[2 * NH * d + hv];
    }
  };
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  int acc_tile = tfirst;
  auto flush = [&](int seg) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = acc[e] + __shfl_xor(acc[e], 32);
      if (lane < 32) red[((wave * 2 + seg) * 8 + 4 * (lane >> 4) + e) * 16 + j] = v;
      acc[e] = 0.0f;
    }
  };
  struct Acc { f32x4 c[NH]; };                      // a step's partial sums
  auto epilogue = [&](const Acc& C, const Ops& o) {
#pragma unroll
    for (int hv = 0; hv < NH; ++hv) {
      const float sv = half_lo(o.sb[hv]);
      const float bb = fmaf(-TR::c0, sv, half_hi(o.sb[hv]));
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = fmaf(sv, C.c[hv][e], fmaf(bb, o.xs[hv][e], acc[e]));
    }
  };

  Ops cur, prev;
  const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
  Acc Cprev;
#pragma unroll
  for (int hv = 0; hv < NH; ++hv) {
    Cprev.c[hv] = zero4;
    prev.sb[hv] = 0u;                                 // step -1 adds exactly nothing
    prev.xs[hv] = zero4;
  }
  int prev_tile = tfirst;
  Blk kc = kfirst;                                    // the block being computed
  Base bc = base_of(kc);
  fetch(bc, 0, cur);
  // One block: its DB steps from ring slots r*DB.., loading block kl into
  // them when `reload`.
  auto run_block = [&](int r, bool reload) {
    const Blk kn = next(kc);                          // the next block (LDS prefetch)
    const Base bn = base_of(kn);
    const unsigned so = codes_at(kl);
#pragma unroll
    for (int d = 0; d < DB; ++d) {
      u32x4 bq[4];
      Acc C;
      if constexpr (HV) {
        const u32x4 w = pair_halves(st[r * DB + d]);
#pragma unroll
        for (int t = 0; t < 4; ++t) bq[t] = unpack_codes(w[t], magic);
        C.c[0] = mfma16x16x32<TR::f16>(cur.A[0], bq[0], zero4);
        C.c[0] = mfma16x16x32<TR::f16>(cur.A[1], bq[1], C.c[0]);
        C.c[1] = mfma16x16x32<TR::f16>(cur.A[2], bq[2], zero4);
        C.c[1] = mfma16x16x32<TR::f16>(cur.A[3], bq[3], C.c[1]);
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) bq[t] = unpack_codes(st[r * DB + d][t], magic);
        C.c[0] = zero4;
#pragma unroll
        for (int t = 0; t < 4; ++t) C.c[0] = mfma16x16x32<TR::f16>(cur.A[t], bq[t], C.c[0]);
      }
      Ops nxt;
      if (d + 1 < DB) fetch(bc, d + 1, nxt);
      else fetch(bn, 0, nxt);
      if (d == 0 && kc.t != prev_tile) {              // uniform: the last step ended a tile
        epilogue(Cprev, prev);
        flush(0);
        acc_tile = kc.t;
        prev_tile = kc.t;
      } else {
        epilogue(Cprev, prev);
      }
      if (reload) load(so, d, st[r * DB + d]);
      Cprev = C;
      prev = cur;
      cur = nxt;
    }
    if (reload) kl = next(kl);
    kc = kn;
    bc = bn;
  };
  int i = 0;
  for (; i + RB <= nb; i += RB) {
#pragma unroll
    for (int r = 0; r < RB; ++r) run_block(r, true);
  }
#pragma unroll
  for (int r = 0; r < RB - 1; ++r)                    // the last nb % RB blocks
    if (i + r < nb) run_block(r, false);
  epilogue(Cprev, prev);
  flush(acc_tile > tfirst ? 1 : 0);

  // ---- reduce: each output tile adds the flushed partials of the runs that
  // cover it, in wave order. With the fused verify each thread also keeps the
  // top two keys (and the best's index) of the row its outputs belong to:
  // output idx is row (idx >> 4) & 7, and NT is a multiple of 128, so that row
  // is fixed per thread, (tid >> 4) & 7.
  __syncthreads();
  // Every wave's slot is read unconditionally (a run's first or last tile
  // slot, whichever is nearer) and the covering runs are selected afterwards,
  // so the reads of one output go out together instead of one after another.
  int tb[NW], te[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    tb[w] = run_tiles[2 * w];
    te[w] = run_tiles[2 * w + 1];
  }
  Top2 best = top2_none();
  for (int idx = tid; idx < tiles * 128; idx += NT) {
    const int t = idx >> 7;
    const int within = idx & 127;                     // row * 16 + column
    float v[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int seg = min(max(t - tb[w], 0), 1);
      v[w] = red[((w * 2 + seg) * 128) + within];
    }
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) s = (t >= tb[w] && t <= te[w]) ? s + v[w] : s;
    const int m = within >> 4;
    const int c = t * 16 + (within & 15);
    if (m < M && c < wgcols) {
      if (!FUSED || y) y[(size_t)m * N + wg0 + c] = s;
      if (FUSED) top2_add(best, s, wg0 + c);
    }
  }
  if constexpr (!FUSED) return;

  // ---- fused greedy verify, first half. The 16 lanes of one row in a wave
  // reduce their top two; a work-group's row result combines its waves in
  // wave order and is written as this group's partial for the finishing
  // kernel. The candidates overlay the activation image, which the reduction
  // above no longer reads.
  static_assert(NT % 128 == 0 && NW % 2 == 0, "one row per thread in the epilogue");
  top2_best16(best);
  unsigned* cand = reinterpret_cast<unsigned*>(lds);  // [NW][4] x (k1, i1, k2)
  if ((lane & 15) == 0) {
    unsigned* p = cand + (wave * 4 + (lane >> 4)) * 3;
    p[0] = best.k1;
    p[1] = (unsigned)best.i1;
    p[2] = best.k2;
  }
  __syncthreads();
  // Lane m < M of wave 0: row m is held by the waves of parity m / 4, in
  // their quarter m % 4.
  if (wave == 0 && lane < M) {
    Top2 r = top2_none();
    for (int w = lane >> 2; w < NW; w += 2) {
      const unsigned* p = cand + (w * 4 + (lane & 3)) * 3;
      top2_merge(r, p[0], (int)p[1], p[2]);
    }
    va.partials[(size_t)lane * va.pgroups + blockIdx.x] = top2_pack(r);
  }
}

template <int ACT, int R, int TILES, int WN, int WK, int D, int KC, bool XALL>
int lds_bytes_for(int K, int gs) {
  constexpr int WGC = 16 * TILES * WN;
  constexpr int P = ActTraits<ACT>::parts;
  const LdsLayout L = gs < 0 ? lds_layout<R, P, WK, KC, WGC, XALL, true>(K >> 6)
                             : lds_layout<R, P, WK, KC, WGC, XALL, false>(K >> 6);
  // The partial sums of the reduction, then the fused verify's candidates.
  const int red_bytes = WK * WN * R * TILES * 128 * 4 + WN * R * TILES * 8 * 12;
  return L.total > red_bytes ? L.total : red_bytes;
}

template <int ACT, int R, int TILES, int WN, int WK, int D, int KC, bool XALL>
hipError_t launch_w4(const void* x, const uint8_t* wq, const uint16_t* scales,
                     const uint16_t* biases, float* y, int M, int K, int N, int cols, int gs,
                     const VerifyArgs& va, hipStream_t stream) {
  const int lds_bytes = lds_bytes_for<ACT, R, TILES, WN, WK, D, KC, XALL>(K, gs);
  if (lds_bytes > kLdsLimit) return hipErrorInvalidValue;  // never launched
  auto kern = qgemm_w4<ACT, R, TILES, WN, WK, D, KC, XALL, 0>;
  if (gs > 0) kern = qgemm_w4<ACT, R, TILES, WN, WK, D, KC, XALL, 1>;
  if (gs < 0) kern = qgemm_w4<ACT, R, TILES, WN, WK, D, KC, XALL, -1>;
  if (lds_bytes > 65536) {
    const hipError_t e = allow_lds(reinterpret_cast<const void*>(kern));
    if (e != hipSuccess) return e;
  }
  const dim3 grid((N + cols - 1) / cols);
  hipLaunchKernelGGL(kern, grid, dim3(64 * WN * WK), lds_bytes, stream, x, wq, scales, biases,
                     y, M, K, N, cols, va);
  return hipGetLastError();
}

template <int ACT, int NW, int DB, int RB, int XB, int D0 = 2>
hipError_t launch_m8(const void* x, const uint8_t* wq, const uint16_t* scales,
                     const uint16_t* biases, float* y, int M, int K, int N, int cols, int gs,
                     const VerifyArgs& va, hipStream_t stream) {
  constexpr int TW = 5;
  const M8Layout L = m8_layout(K >> 6, 16 * TW, NW, XB, gs < 0);
  if (L.total > kLdsLimit) return hipErrorInvalidValue;  // never launched
  auto kern = qgemm_w4_m8<ACT, NW, TW, DB, RB, D0, XB, false, 0>;
  if (va.argmax) {
    kern = qgemm_w4_m8<ACT, NW, TW, DB, RB, D0, XB, true, 0>;
    if (gs > 0) kern = qgemm_w4_m8<ACT, NW, TW, DB, RB, D0, XB, true, 1>;
    if (gs < 0) kern = qgemm_w4_m8<ACT, NW, TW, DB, RB, D0, XB, true, -1>;
  } else {
    if (gs > 0) kern = qgemm_w4_m8<ACT, NW, TW, DB, RB, D0, XB, false, 1>;
    if (gs < 0) kern = qgemm_w4_m8<ACT, NW, TW, DB, RB, D0, XB, false, -1>;
  }
  if (L.total > 65536) {
    const hipError_t e = allow_lds(reinterpret_cast<const void*>(kern));
    if (e != hipSuccess) return e;
  }
  const dim3 grid((N + cols - 1) / cols);
  hipLaunchKernelGGL(kern, grid, dim3(64 * NW), L.total, stream, x, wq, scales, biases, y, M,
                     K, N, cols, va);
  return hipGetLastError();
}

// Staging rounds per batch: 5 up to K = 2560, else 10 (8 waves; one batch up
// to K = 5120).
constexpr int m8_xb(int K) { return K <= 2560 ? 5 : 10; }

// Block length of qgemm_w4_m8: the largest of 5, 4, 2, 1 that divides the
// group-pair count; the ring holds one block of 5, two of 4, four of 2 or
// eight of 1 (deeper rings delay the staging reads, measured at K = 5120).
template <int ACT, int XB>
hipError_t launch_m8_blocks(const void* x, const uint8_t* wq, const uint16_t* scales,
                            const uint16_t* biases, float* y, int M, int K, int N, int cols,
                            int gs, const VerifyArgs& va, hipStream_t s) {
  const int GP = ((K >> 6) + 1) >> 1;
  if (GP % 5 == 0)
    return launch_m8<ACT, 8, 5, 1, XB>(x, wq, scales, biases, y, M, K, N, cols, gs, va, s);
  if (GP % 4 == 0)
    return launch_m8<ACT, 8, 4, 2, XB>(x, wq, scales, biases, y, M, K, N, cols, gs, va, s);
  if (GP % 2 == 0)
    return launch_m8<ACT, 8, 2, 4, XB>(x, wq, scales, biases, y, M, K, N, cols, gs, va, s);
  return launch_m8<ACT, 8, 1, 8, XB>(x, wq, scales, biases, y, M, K, N, cols, gs, va, s);
}

// Columns per work-group of qgemm_w4_m8 (an equal share of the CUs, at most
// five tiles) and whether its LDS image fits.
int m8_cols(int N) {
  const int cus = device_cus();
  const int share = ((N + cus - 1) / cus + 3) / 4 * 4;
  return share < 80 ? share : 80;
}
bool m8_fits(int K, int gs) {
  return m8_layout(K >> 6, 80, 8, m8_xb(K), gs < 0).total <= kLdsLimit;
}

template <int ACT>
hipError_t launch_m8_any(const void* x, const uint8_t* wq, const uint16_t* scales,
                         const uint16_t* biases, float* y, int M, int K, int N, int gs,
                         const VerifyArgs& va, hipStream_t s) {
  const int cols = m8_cols(N);
  if (m8_xb(K) == 5)
    return launch_m8_blocks<ACT, 5>(x, wq, scales, biases, y, M, K, N, cols, gs, va, s);
  return launch_m8_blocks<ACT, 10>(x, wq, scales, biases, y, M, K, N, cols, gs, va, s);
}

// The whole-line kernel for one row set, unless a profiling run pins the
// half-line one.
bool use_m8q(int M, int K, int act, int gs) {
  return forced_variant() != kVariantM8 && qgemm_m8q_fits(M, K, act, gs);
}

// ---------------------------------------------------------------------------
// Kernel choice. plan_for picks the kernel of a problem (for qgemm_w4 also
// its configuration and columns per work-group) before anything is
// launched, and checks that its LDS image fits. The plain projection and the
// fused verify take the same plan, so their outputs agree bit for bit.
enum class Path { None, Rows, Wide, V, M8Q, M8, M16, W4 };
struct Plan {
  Path path;
  int cfg;   // qgemm_w4 configuration (W4)
  int cols;  // columns per work-group (M8Q, M8, W4)
};

// qgemm_w4 configurations (R, TILES, WN, WK, D, KC, XALL), by index.
#define VQV_W4_CONFIGS(X)             \
  X(0, 1, 1, 5, 2, 8, 1, true)        \
  X(1, 1, 1, 1, 8, 1, 1, false)       \
  X(2, 1, 1, 4, 2, 8, 1, true)        \
  X(3, 1, 1, 4, 2, 4, 2, false)       \
  X(4, 2, 1, 4, 2, 4, 2, false)       \
  X(5, 2, 1, 2, 1, 2, 1, false)       \
  X(6, 4, 1, 4, 1, 4, 1, false)       \
  X(7, 4, 1, 2, 1, 2, 1, false)       \
  X(8, 8, 1, 4, 1, 2, 1, false)       \
  X(9, 8, 1, 2, 1, 2, 1, false)

template <int ACT>
bool w4_fits(int cfg, int K, int gs) {
  switch (cfg) {
#define VQV_W4_FITS(i, R, T, WN, WK, D, KC, XA) \
  case i: return lds_bytes_for<ACT, R, T, WN, WK, D, KC, XA>(K, gs) <= kLdsLimit;
    VQV_W4_CONFIGS(VQV_W4_FITS)
#undef VQV_W4_FITS
  }
  return false;
}

template <int ACT>
hipError_t launch_w4_cfg(int cfg, const void* x, const uint8_t* wq, const uint16_t* scales,
                         const uint16_t* biases, float* y, int M, int K, int N, int cols, int gs,
                         const VerifyArgs& va, hipStream_t s) {
  switch (cfg) {
#define VQV_W4_LAUNCH(i, R, T, WN, WK, D, KC, XA) \
  case i:                                         \
    return launch_w4<ACT, R, T, WN, WK, D, KC, XA>(x, wq, scales, biases, y, M, K, N, cols, gs, va, s);
    VQV_W4_CONFIGS(VQV_W4_LAUNCH)
#undef VQV_W4_LAUNCH
  }
  return hipErrorInvalidValue;
}

// One row of 16-bit activations (group 64 or 128, K <= 8192) below
// vocabulary widths takes the vector-ALU kernel. M <= 8 (one row set) takes,
// in order: the whole-line
// kernel, the half-line kernel, then qgemm_w4 (narrow N split into exactly one work-group per CU,
// columns rounded up to 4; the W4A32 draft's narrow outputs one 16-column
// tile per work-group with K split over 8 waves, measured fastest at
// K = 5120, N = 1024: 11.1 us against 15.5 us for 64-column groups; wide N in
// 64-column groups). 17..64 rows at vocabulary widths share one weight
// stream (qgemm_w4_rows); vocabulary widths with K <= 2560 otherwise take
// whole-tile waves (qgemm_w4_wide), 9..64 rows with K <= 2560 the 16-row
// kernel; the rest qgemm_w4 with row sets of 8 and chunked staging (the
// smaller fallback, 32 columns with one K range, keeps fp32 at large K
// within LDS).
template <int ACT>
Plan plan_act(int M, int K, int N, int gs) {
  constexpr bool h16 = ACT != ACT_FP32;
  if (h16 && qgemm_rows_fits(M, K, N, ACT)) return {Path::Rows, 0, 0};
  // One row: the vector-ALU kernel, measured faster than the 8-row MFMA
  // kernels at M = 1 and slower from M = 2, and slower than the whole-tile
  // kernel at vocabulary widths; a profiling run may pin either.
  const Variant fv = forced_variant();
  const bool vfit = h16 && qgemm_v_fits(M, K, N, ACT, gs);
  if (vfit && fv == kVariantV) return {Path::V, 0, 0};
  if (qgemm_wide_fits(M, K, N, ACT, gs)) return {Path::Wide, 0, 0};
  if (vfit && fv == kVariantAuto && M == 1) return {Path::V, 0, 0};
  if (h16 && M <= 8 && use_m8q(M, K, ACT, gs)) return {Path::M8Q, 0, qgemm_m8q_cols(N)};
  if (h16 && M <= 8 && m8_fits(K, gs)) return {Path::M8, 0, m8_cols(N)};
  if (M > 8 && qgemm_m16_fits(M, K, ACT, gs)) return {Path::M16, 0, 0};
  if (M <= 8) {
    const int cus = device_cus();
    const int share = ((N + cus - 1) / cus + 3) / 4 * 4;
    if (share > 48 && share <= 80 && w4_fits<ACT>(0, K, gs)) return {Path::W4, 0, share};
    if ((N + 63) / 64 < cus && w4_fits<ACT>(1, K, gs)) return {Path::W4, 1, 16};
    if (w4_fits<ACT>(2, K, gs)) return {Path::W4, 2, 64};
    if (w4_fits<ACT>(3, K, gs)) return {Path::W4, 3, 64};
    return {Path::None, 0, 0};
  }
  const int cfg = M <= 16 ? 4 : M <= 32 ? 6 : 8;
  if (w4_fits<ACT>(cfg, K, gs)) return {Path::W4, cfg, 64};
  if (w4_fits<ACT>(cfg + 1, K, gs)) return {Path::W4, cfg + 1, 32};
  return {Path::None, 0, 0};
}

Plan plan_for(int M, int K, int N, int act, int gs) {
  switch (act) {
    case ACT_BF16: return plan_act<ACT_BF16>(M, K, N, gs);
    case ACT_FP16: return plan_act<ACT_FP16>(M, K, N, gs);
    case ACT_FP32: return plan_act<ACT_FP32>(M, K, N, gs);
    default: return {Path::None, 0, 0};
  }
}

template <int ACT>
hipError_t launch_plan(const Plan& p, const void* x, const uint8_t* wq, const uint16_t* scales,
                       const uint16_t* biases, float* y, int M, int K, int N, int gs,
                       const VerifyArgs& va, hipStream_t s) {
  switch (p.path) {
    case Path::Rows: return launch_qgemm_rows(x, wq, scales, biases, y, M, K, N, ACT, gs, va, s);
    case Path::Wide: return launch_qgemm_wide(x, wq, scales, biases, y, M, K, N, ACT, gs, va, s);
    case Path::V: return launch_qgemm_v(x, wq, scales, biases, y, M, K, N, ACT, gs, va, s);
    case Path::M8Q: return launch_qgemm_m8q(x, wq, scales, biases, y, M, K, N, ACT, gs, va, s);
    case Path::M8:
      if constexpr (ACT != ACT_FP32)
        return launch_m8_any<ACT>(x, wq, scales, biases, y, M, K, N, gs, va, s);
      break;
    case Path::M16: return launch_qgemm_m16(x, wq, scales, biases, y, M, K, N, ACT, gs, va, s);
    case Path::W4:
      return launch_w4_cfg<ACT>(p.cfg, x, wq, scales, biases, y, M, K, N, p.cols, gs, va, s);
    case Path::None: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool qgemm_supported(int M, int K, int N, int act, int gs) {
  return plan_for(M, K, N, act, gs).path != Path::None;
}

const char* qgemm_kernel_name(int M, int K, int N, int act, int gs) {
  switch (plan_for(M, K, N, act, gs).path) {
    case Path::Rows: return "qgemm_w4_rows";
    case Path::Wide: return "qgemm_w4_wide";
    case Path::V: return "qgemm_w4_v";
    case Path::M8Q: return "qgemm_w4_m8q";
    case Path::M8: return "qgemm_w4_m8";
    case Path::M16: return "qgemm_w4_m16";
    case Path::W4: return "qgemm_w4";
    case Path::None: break;
  }
  return nullptr;
}

hipError_t launch_qgemm(const void* x, const uint8_t* wq, const uint16_t* scales,
                        const uint16_t* biases, float* y, int M, int K, int N, int act, int gs,
                        const VerifyArgs& va, hipStream_t stream) {
  const Plan p = plan_for(M, K, N, act, gs);
  switch (act) {
    case ACT_BF16:
      return launch_plan<ACT_BF16>(p, x, wq, scales, biases, y, M, K, N, gs, va, stream);
    case ACT_FP16:
      return launch_plan<ACT_FP16>(p, x, wq, scales, biases, y, M, K, N, gs, va, stream);
    case ACT_FP32:
      return launch_plan<ACT_FP32>(p, x, wq, scales, biases, y, M, K, N, gs, va, stream);
    default: return hipErrorInvalidValue;
  }
}

int qgemm_verify_groups(int M, int K, int N, int act, int gs) {
  // Partials per row: one per work-group that covers the row. The
  // persistent kernels (qgemm_w4_wide, qgemm_w4_m16) give each row set
  // `workers` work-groups of its own.
  const Plan p = plan_for(M, K, N, act, gs);
  switch (p.path) {
    case Path::Rows: return qgemm_rows_groups(N);
    case Path::Wide: return qgemm_wide_workers(M);
    case Path::V: return qgemm_v_groups(N);
    case Path::M16: return qgemm_m16_workers(M, N);
    case Path::M8Q:
    case Path::M8:
    case Path::W4: return (N + p.cols - 1) / p.cols;
    case Path::None: break;
  }
  return 0;
}

hipError_t launch_qgemm_verify(const void* x, const uint8_t* wq, const uint16_t* scales,
                               const uint16_t* biases, float* y, int M, int K, int N, int act,
                               int gs, const VerifyArgs& va, hipStream_t stream) {
  VerifyArgs v = va;
  v.pgroups = qgemm_verify_groups(M, K, N, act, gs);
  if (v.pgroups <= 0) return hipErrorInvalidValue;
  const hipError_t e = launch_qgemm(x, wq, scales, biases, y, M, K, N, act, gs, v, stream);
  if (e != hipSuccess) return e;
  return launch_verify_finish(v, stream);
}

Variant forced_variant() {
  // Read on every plan (a short scan of the environment), so that a process
  // can switch variants between calls.
  const char* e = getenv("VQV_FORCE_VARIANT");
  if (!e) return kVariantAuto;
  if (!strcmp(e, "m8")) return kVariantM8;
  if (!strcmp(e, "m8q")) return kVariantM8Q;
  if (!strcmp(e, "v")) return kVariantV;
  return kVariantAuto;
}

}  // namespace vqv

// W4 group-64 dequant GEMM for 9..64 activation rows on gfx950 (row sets of
// 16), and the same kernel with a SwiGLU epilogue over a stacked gate/up
// weight.
//
// y[m,n] = sum_k x[m,k] * (s[n,k/64]*q[n,k] + b[n,k/64]), as the projection of
// qgemm.hip, for one row set of up to 16 rows: the verify block of 16 and the
// M=16 gate/up block ("perf: tune DFlash2 M=8 verification for M1 and M2",
// Validation). With SWIGLU the weight holds Nh gate rows then Nh up rows
// (N = 2*Nh) and the kernel writes h[m,j] = silu(y[m,j]) * y[m,Nh+j] only,
// [M, Nh] fp32, never the gate and up outputs themselves.
//
// MFMA layout. v_mfma_f32_16x16x32 with all 16 A rows real: A row i is
// activation row i. Lane (column j = lane%16, k slot h = lane/16) of B loads
// the 16 contiguous bytes [16h, 16h+16) of its column's 64-byte group pair
// (one 16-byte load per lane: full 64-byte runs of each weight row, which the
// memory system streams much faster than 32-byte pieces). Two lane-half swaps
// (split_groups) then give each lane 8 bytes of group 2p in dwords 0-1 and
// the same 8 bytes of group 2p+1 in dwords 2-3, so MFMAs 0-1 sum within group
// 2p, MFMAs 2-3 within 2p+1, and each group epilogue applies that group's
// scale and bias:
//     y += s*acc' + (b - c0*s)*xs,  acc' = sum x*(c0+q),  xs = sum x.
// The per-step work, the exact unpack and the weight ring follow
// qgemm_w4_m8; the activation image holds 16 rows per group pair.
//
// Persistent work-groups. One work-group per CU stages its row set's
// activations once and then takes column groups in turn (worker w: groups w,
// w + workers, ...), with the table, the weight ring and the reduction per
// group. With more than 16 rows, row set r (rows 16r .. 16r+15) has workers
// of its own, and the grid is laid out so that the row sets of one worker are
// consecutive on one XCD (work-groups are dealt to the 8 XCDs in turn): they
// walk the same column groups together, so the XCD reads those weights from
// HBM once and serves the other row sets from its L2.
//
// SwiGLU columns. The work-group's logical columns interleave the two halves:
// logical column 2u reads gate row u and 2u+1 reads up row Nh+u, so the
// gate and up values of one hidden unit land in adjacent output columns of
// the same tile and the final reduction pairs them.

#include <type_traits>

#include "argmax.h"
#include "qgemm_common.h"
#include "vqv_internal.h"

namespace vqv {
namespace {

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Activation image of one group pair: four t-rows (MFMA t) of 64 slots of 16
// bytes, slot h*16 + row. No zero slot: every A lane is a real row (rows past
// M are staged as zeros).
constexpr int kSlot16 = 16;
constexpr int kTRow16 = 64 * kSlot16;
constexpr int kPair16 = 4 * kTRow16;

struct M16Layout {
  int xs, sb, sbs, red, runs, total;
};

// The staging writes whole batches of XB rounds of NW groups, so the image
// area is padded to that many pairs; image GP (the last, or a padding image
// that the loads fill with zeros) is the zero image of steps past a run.
// HV (group 32): row sums and table entries per 32-k half, twice as many;
// table rows a multiple of 4 entries for 16-byte reads.
__host__ __device__ inline M16Layout m16_layout(int G, int WGC, int NW, int XB, bool HV = false) {
  const int GP = (G + 1) >> 1;
  const int rounds = (2 * GP + NW - 1) / NW;
  const int padded = (rounds + XB - 1) / XB * XB * NW;
  const int nimg = GP + 1 > padded / 2 ? GP + 1 : padded / 2;
  M16Layout L{};
  L.xs = nimg * kPair16;
  L.sb = L.xs + nimg * (HV ? 64 : 32) * 4;              // 2 groups (x 2 halves) x 16 rows
  L.sbs = HV ? (2 * G + 7) & ~3 : (G + 5) & ~1;          // >= entries + 4; 16- or 8-byte reads
  L.red = L.sb + WGC * L.sbs * 4;
  L.runs = L.red + NW * 2 * 256 * 4;
  L.total = L.runs + NW * 2 * 4;
  return L;
}

// silu(g) * u in fp32 with the library's exp and an IEEE division.
__device__ __forceinline__ float swiglu(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// Lane (j, h) loads bytes [16h, 16h+16) of its column's 64-byte group pair:
// group 2p for h < 2, group 2p+1 for h >= 2. Two swaps between the lane
// halves (lane L < 32 with lane L + 32) leave every lane 8 bytes of each
// group: dwords 0-1 hold bytes [8s, 8s+8) of group 2p and dwords 2-3 the same
// bytes of group 2p+1, with s = sigma(h) = (0, 2, 1, 3)[h] (h's two bits
// swapped), so that MFMAs 0-1 sum within group 2p and MFMAs 2-3 within 2p+1.
__device__ __forceinline__ int sigma_slot(int h) { return ((h & 1) << 1) | (h >> 1); }

__device__ __forceinline__ u32x4 split_groups(const u32x4& w) {
  const auto a = __builtin_amdgcn_permlane32_swap(w.x, w.z, false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(w.y, w.w, false, false);
  return u32x4{a[0], b[0], a[1], b[1]};
}

// One group pair for 16 rows: A[t] holds the activations whose codes sit in
// dword t after split_groups (all 16 rows real). C0 collects group 2p, C1
// group 2p+1.
// Group 32: after split_groups one more swap, between lanes l and l + 16
// (k slots 2i and 2i + 1), leaves every MFMA a single 32-k half of one group,
// with k slot h holding k = 32 hh + 8h .. of half hh. A[t] holds the
// activations of half t % 2 of group 2p + t / 2; C[t] collects them.
template <bool F16>
__device__ __forceinline__ void pair_step_halves(const u32x4 (&A)[4], const u32x4& w,
                                                 unsigned magic, f32x4 (&C)[4]) {
  const u32x4 v = split_groups(w);
  const auto a = __builtin_amdgcn_permlane16_swap(v.x, v.y, false, false);
  const auto b = __builtin_amdgcn_permlane16_swap(v.z, v.w, false, false);
  const u32x4 bq0 = unpack_codes(a[0], magic), bq1 = unpack_codes(a[1], magic);
  const u32x4 bq2 = unpack_codes(b[0], magic), bq3 = unpack_codes(b[1], magic);
  C[0] = mfma16x16x32<F16>(A[0], bq0, C[0]);
  C[2] = mfma16x16x32<F16>(A[2], bq2, C[2]);
  C[1] = mfma16x16x32<F16>(A[1], bq1, C[1]);
  C[3] = mfma16x16x32<F16>(A[3], bq3, C[3]);
}

template <bool F16>
__device__ __forceinline__ void pair_step(const u32x4 (&A)[4], const u32x4& w, unsigned magic,
                                          f32x4& C0, f32x4& C1) {
  const u32x4 v = split_groups(w);
  u32x4 bq[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) bq[t] = unpack_codes(v[t], magic);
  C0 = mfma16x16x32<F16>(A[0], bq[0], C0);
  C1 = mfma16x16x32<F16>(A[2], bq[2], C1);
  C0 = mfma16x16x32<F16>(A[1], bq[1], C0);
  C1 = mfma16x16x32<F16>(A[3], bq[3], C1);
}

template <int ACT, int NW, int TW, int DB, int RB, int D0, int XB, bool SWIGLU, bool SBV,
          int GS>
__global__ __launch_bounds__(64 * NW) void qgemm_w4_m16(
    const void* __restrict__ x, const uint8_t* __restrict__ wq,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases,
    float* __restrict__ y, int M, int K, int N, int cols, int rsets, int workers,
    VerifyArgs va) {
  using TR = ActTraits<ACT>;
  // GS: group 64 << GS for GS >= 0; GS = -1 is group 32 (pair_step_halves:
  // four partial sums per group pair, each with its own scale, bias and
  // row sum).
  constexpr int gs = GS > 0 ? GS : 0;               // table shift of group 128
  constexpr bool HV = GS < 0;
  constexpr int XSF = HV ? 64 : 32;                 // row sums per activation image
  static_assert(TR::parts == 1, "16-bit activations only");
  static_assert(TW <= NW, "a run must span at most two tiles");
  static_assert(NW >= 8, "the partial-sum slots double as a write sink");
  constexpr int D = DB * RB;
  static_assert(D0 >= 0 && D0 <= D, "prologue ring depth");
  constexpr int NT = 64 * NW;
  constexpr int WGC = 16 * TW;
  constexpr int SBU = 2;
  constexpr unsigned kSkip = 0x7FF00000u;             // scalar offset that reads as zero

  // Work-group -> (row set, worker). Worker w takes the column groups w,
  // w + workers, ...; the row sets of one worker are consecutive on one XCD.
  const int ngroups = (N + cols - 1) / cols;
  int wk = blockIdx.x, rs = 0;
  if (rsets > 1) {
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    rs = local % rsets;
    wk = (local / rsets) * 8 + xcd;
  }
  const bool fused = !SWIGLU && va.argmax != nullptr;  // uniform
  const int rows = min(16, M - 16 * rs);            // rows of this row set
  if (wk >= workers || wk >= ngroups) {              // the whole group leaves
    if (fused && (int)threadIdx.x < rows)            // with empty partials
      va.partials[(size_t)(16 * rs + threadIdx.x) * va.pgroups + wk] = top2_pack(top2_none());
    return;
  }
  x = static_cast<const uint16_t*>(x) + (size_t)rs * 16 * K;
  if (y) y += (size_t)rs * 16 * (SWIGLU ? N / 2 : N);
  M = rows;

  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15;
  const int h = lane >> 4;
  const int G = K >> 6;
  const int GP = (G + 1) >> 1;
  const int bpt = GP / DB;
  const unsigned rowbytes = (unsigned)K >> 1;
  const int Nh = N >> 1;
  const M16Layout L = m16_layout(G, WGC, NW, XB, HV);
  const int TG = HV ? 2 * G : G;                     // LDS table entries per column
  const int ME = HV ? 2 * G : (G >> gs);             // table entries per row in memory
  unsigned char* xl = lds;
  float* xsl = reinterpret_cast<float*>(lds + L.xs);
  unsigned* sbl = reinterpret_cast<unsigned*>(lds + L.sb);
  float* red = reinterpret_cast<float*>(lds + L.red);
  int* run_tiles = reinterpret_cast<int*>(lds + L.runs);

  unsigned magic;
  asm volatile("v_mov_b32 %0, %1" : "=v"(magic) : "i"(TR::magic));
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(x), (short)0, M * K * 2, kBufferFlags);

  // ---- activation staging, once per work-group: lane (e8, mm) moves
  // x[mm + 8r, 64g + 8e8 .. +8]; one batch of XB rounds covers the 2*GP
  // groups (host: K <= 64 * NW * XB).
  const int e8 = lane & 7;
  const int mm = lane >> 3;
  u32x4 xv[XB][2];
  auto x_load = [&](int bb) {
#pragma unroll
    for (int i = 0; i < XB; ++i) {
      const int g = wave + NW * (bb + i);
      const int k = 64 * g + 8 * e8;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int row = mm + 8 * r;
        const bool ok = row < M && k < K;
        xv[i][r] = __builtin_amdgcn_raw_buffer_load_b128(
            xr, ok ? (unsigned)((row * K + k) * 2) : kOutOfRange, 0, 0);
      }
    }
  };
  // Values k = 8e8.. of group g feed MFMA t = 2(g&1) + e8%2 in the k slot h
  // whose lanes hold those codes after split_groups: sigma(h) = e8/2.
  // With HV (pair_step_halves) they feed MFMA 2(g&1) + e8/4 from k slot e8%4.
  const unsigned xl_lane =
      HV ? (e8 >> 2) * kTRow16 + ((e8 & 3) * 16 + mm) * kSlot16
         : (e8 & 1) * kTRow16 + (sigma_slot(e8 >> 1) * 16 + mm) * kSlot16;
  auto x_store_round = [&](int bb, int i) {
    const int g = wave + NW * (bb + i);               // uniform
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      // Row sum over the group (8 lanes) or, with HV, over its half (4 lanes).
      const float s8 = HV ? sum4_lanes(block_sum<ACT>(xv[i][r]))
                          : sum8_lanes(block_sum<ACT>(xv[i][r]));
      *reinterpret_cast<u32x4*>(xl + (g >> 1) * kPair16 + (g & 1) * 2 * kTRow16 + xl_lane +
                                r * 8 * kSlot16) = permute_pairs(xv[i][r]);
      xsl[HV ? (g * 2 + (e8 >> 2)) * 16 + mm + 8 * r : g * 16 + mm + 8 * r] = s8;
    }
  };
  // SBV (host): K/64 a multiple of 8 and 16-byte aligned scale and bias
  // arrays, so the table moves in 16-byte units. A template flag rather than
  // a runtime branch: loads on either side of a branch make the compiler wait
  // for every load in flight, the staging loads included.
  constexpr bool sb_vec = SBV;
  const unsigned g_recip = 0xFFFFFFFFu / (unsigned)TG + 1u;
  auto div_g = [&](unsigned e) { return TG == 1 ? e : __umulhi(e, g_recip); };
  const unsigned char* abase = xl + (h * 16 + j) * kSlot16;
  const float* xsbase = xsl + 4 * h;
  const unsigned* sbbase = sbl + j * L.sbs;
  // Past a run: the zero image's row sums double as zero (s, b) entries
  // (16-byte aligned whatever G is).
  const unsigned* sbzero = reinterpret_cast<const unsigned*>(xsl + GP * XSF);
  auto rel_row = [&](int c) { return SWIGLU ? (c & 1) * Nh + (c >> 1) : c; };
  // Lane j of tile t reads logical column 16t + j: weight row rel_row(j) plus
  // the tile's rows (16 per tile, or 8 gate and 8 up rows with SWIGLU).
  const unsigned woff = (unsigned)rel_row(j) * rowbytes + 16u * h;
  constexpr unsigned kTileRows = SWIGLU ? 8u : 16u;

  // The activation loads go out now (one batch: K <= 64*NW*XB, host). With a
  // one-block ring (RB == 1) they are staged inside the first column group,
  // once that group's table and ring are in flight too, so the weight stream
  // starts while the staging waits; deeper rings stage here (registers).
  constexpr bool kLateStaging = RB == 1;
  x_load(0);
  if constexpr (!kLateStaging) {
#pragma unroll
    for (int i = 0; i < XB; ++i) x_store_round(0, i);
  }
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int i = tid; i < kPair16 / 16; i += NT)      // the zero image
      *reinterpret_cast<u32x4*>(xl + GP * kPair16 + 16 * i) = z;
    if (tid < XSF) xsl[GP * XSF + tid] = 0.0f;
    if constexpr (HV) {
      for (int i = tid; i < WGC * 4; i += NT) sbl[(i >> 2) * L.sbs + TG + (i & 3)] = 0u;
    } else {
      for (int i = tid; i < WGC * 2; i += NT) sbl[(i >> 1) * L.sbs + G + (i & 1)] = 0u;
    }
  }

  // With the fused verify each thread keeps the top two of its outputs, all
  // of row (tid >> 4) & 15 (the reduction's output order, NT a multiple of 256).
  Top2 best = top2_none();
  for (int cg = wk; cg < ngroups; cg += workers) {
    const int wg0 = cg * cols;                        // first logical column
    const int wgcols = min(cols, N - wg0);
    const int tiles = (wgcols + 15) >> 4;
    const int nblk = tiles * bpt;
    // SIMD s = wave % 4 takes the s-th quarter of the blocks. Its two waves
    // share the SIMD's issue slots and the older one (waves 0-3 are
    // dispatched first) wins the arbitration, so it takes 9/16 of them,
    // rounded up.
    const int sq0 = ((wave & 3) * nblk) >> 2, sq1 = (((wave & 3) + 1) * nblk) >> 2;
    const int smid = sq0 + (((sq1 - sq0) * 9 + 15) >> 4);
    const int b0 = NW == 8 ? (wave < 4 ? sq0 : smid) : (wave * nblk) / NW;
    const int nb = NW == 8 ? (wave < 4 ? smid : sq1) - b0 : ((wave + 1) * nblk) / NW - b0;
    const int tfirst = b0 / bpt;
    // Weight row of logical column c of this group, relative to `row0`.
    const int row0 = SWIGLU ? (wg0 >> 1) : wg0;
    const int nrows = SWIGLU ? N - row0 : wgcols;     // rows the buffers may touch
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(wq) + (size_t)row0 * rowbytes, (short)0, nrows * rowbytes,
        kBufferFlags);
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(scales) + (size_t)row0 * ME, (short)0, nrows * ME * 2,
        kBufferFlags);
    const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(biases) + (size_t)row0 * ME, (short)0, nrows * ME * 2,
        kBufferFlags);

    // ---- scale/bias table: row n of the table is logical column n.
    const int sb_units = sb_vec ? wgcols * TG / 8 : wgcols * TG;
    u32x4 sbs[SBU], sbb[SBU];
    auto sb_load = [&](int round) {
#pragma unroll
      for (int u = 0; u < SBU; ++u) {
        const int i = (round * SBU + u) * NT + tid;
        if constexpr (sb_vec) {
          const unsigned e0 = 8u * (unsigned)i;
          const unsigned n = div_g(e0), g = e0 - n * (unsigned)TG;
          const unsigned off =
              i < sb_units ? 2u * (((unsigned)rel_row((int)n) * (unsigned)TG + g) >> gs)
                           : kOutOfRange;
          sbs[u] = sb_unit_load<GS>(sr, off);
          sbb[u] = sb_unit_load<GS>(br, off);
        } else {
          const unsigned n = div_g((unsigned)i), g = (unsigned)i - n * (unsigned)TG;
          const unsigned off =
              i < sb_units ? 2u * (((unsigned)rel_row((int)n) * (unsigned)TG + g) >> gs)
                           : kOutOfRange;
          sbs[u].x = __builtin_amdgcn_raw_buffer_load_b16(sr, off, 0, 0);
          sbb[u].x = __builtin_amdgcn_raw_buffer_load_b16(br, off, 0, 0);
        }
      }
    };
    auto sb_store = [&](int round) {
#pragma unroll
      for (int u = 0; u < SBU; ++u) {
        const int i = (round * SBU + u) * NT + tid;
        const bool ok = i < sb_units;
        if constexpr (sb_vec) {
          const unsigned e0 = 8u * (unsigned)i;
          const unsigned n = div_g(e0), g = e0 - n * (unsigned)TG;
          u32x4 lo, hi;                               // (s_g | b_g << 16) for g .. g+7
          sb_pairs<GS>(sbs[u], sbb[u], lo, hi);
          // Units past the table write into the partial-sum slots (16 KB,
          // not read until this group's loop has ended).
          const unsigned o = ok ? (unsigned)L.sb + 4u * (n * (unsigned)L.sbs + g)
                                : (unsigned)L.red + 32u * ((unsigned)tid & 511u);
          *reinterpret_cast<u32x4*>(lds + o) = lo;
          *reinterpret_cast<u32x4*>(lds + o + 16) = hi;
        } else if (ok) {
          const unsigned n = div_g((unsigned)i), g = (unsigned)i - n * (unsigned)TG;
          sbl[n * L.sbs + g] = (sbs[u].x & 0xFFFFu) | (sbb[u].x << 16);
        }
      }
    };

    // ---- blocks of the run (as qgemm_w4_m8).
    struct Blk {
      int t, p, left;
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
    auto codes_at = [&](const Blk& k) {
      return k.left > 0 ? (unsigned)k.t * kTileRows * rowbytes + 64u * (unsigned)k.p : kSkip;
    };
    // Step d of the block at scalar offset `so`: 8 bytes of each group.
    auto load = [&](unsigned so, int d, u32x4& w) {
      w = __builtin_amdgcn_raw_buffer_load_b128(wr, woff + 64u * d, so, 0);
    };

    // ---- table, then the weight ring; run bounds for the reduction.
    Blk kl = kfirst;
    sb_load(0);
#pragma unroll
    for (int d = 0; d < D0; ++d) {
      load(codes_at(kl), d % DB, st[d]);
      if (d % DB == DB - 1) kl = next(kl);
    }
    asm volatile("" ::: "memory");                   // the loads above go out first
    if (kLateStaging && cg == wk) {                   // uniform: the first group stages
      // The empty asm keeps the staging arithmetic here, after the loads
      // above: hoisted out of the loop it would wait for the activations first.
#pragma unroll
      for (int i = 0; i < XB; ++i) {
        asm volatile("" : "+v"(xv[i][0]), "+v"(xv[i][1]));
        x_store_round(0, i);
      }
    }
#pragma unroll
    for (int d = D0; d < D; ++d) {
      load(codes_at(kl), d % DB, st[d]);
      if (d % DB == DB - 1) kl = next(kl);
    }
    sb_store(0);
    for (int round = 1; round * SBU * NT < sb_units; ++round) {
      sb_load(round);
      sb_store(round);
    }
    if (lane == 0) {
      run_tiles[2 * wave] = nb > 0 ? tfirst : 1 << 30;
      run_tiles[2 * wave + 1] = nb > 0 ? (b0 + nb - 1) / bpt : -1;
    }
    __syncthreads();

    // ---- main loop.
    // Row sums and (s, b) words of the step: of groups 2p, 2p+1, or with HV
    // of their four halves.
    constexpr int NQ = HV ? 4 : 2;
    struct Ops {
      u32x4 A[4];
      f32x4 xs[NQ];
      unsigned sb[NQ];
    };
    struct Base {
      const unsigned char* a;
      const float* xs;
      const unsigned* sb;
    };
    auto base_of = [&](const Blk& k) {
      const bool in = k.left > 0;                     // uniform
      const int img = in ? k.p : GP;
      Base bs;
      bs.a = abase + img * kPair16;
      bs.xs = xsbase + img * XSF;
      bs.sb = in ? sbbase + k.t * 16 * L.sbs + NQ * k.p : sbzero;
      return bs;
    };
    auto fetch = [&](const Base& bs, int d, Ops& o) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        o.A[t] = *reinterpret_cast<const u32x4*>(bs.a + d * kPair16 + t * kTRow16);
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        o.xs[q] = *reinterpret_cast<const f32x4*>(bs.xs + d * XSF + 16 * q);
      if constexpr (HV) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(bs.sb + 4 * d);
#pragma unroll
        for (int q = 0; q < NQ; ++q) o.sb[q] = v[q];
      } else {
        const u32x2 v = *reinterpret_cast<const u32x2*>(bs.sb + 2 * d);
        o.sb[0] = v.x;
        o.sb[1] = v.y;
      }
    };
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    int acc_tile = tfirst;
    auto flush = [&](int seg) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        red[((wave * 2 + seg) * 16 + 4 * h + e) * 16 + j] = acc[e];
        acc[e] = 0.0f;
      }
    };
    struct Acc { f32x4 c[NQ]; };                    // a step's partial sums
    auto epilogue = [&](const Acc& C, const Ops& o) {
      float s[NQ], c[NQ];
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        s[q] = half_lo(o.sb[q]);
        c[q] = fmaf(-TR::c0, s[q], half_hi(o.sb[q]));
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int q = 0; q < NQ; ++q) acc[e] = fmaf(s[q], C.c[q][e], fmaf(c[q], o.xs[q][e], acc[e]));
    };

    Ops cur, prev;
    const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
    Acc P;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      P.c[q] = zero4;
      prev.sb[q] = 0u;                                // step -1 adds exactly nothing
      prev.xs[q] = zero4;
    }
    int prev_tile = tfirst;
    Blk kc = kfirst;
    Base bc = base_of(kc);
    fetch(bc, 0, cur);
    auto run_block = [&](int r, bool reload) {
      const Blk kn = next(kc);
      const Base bn = base_of(kn);
      const unsigned so = codes_at(kl);
#pragma unroll
      for (int d = 0; d < DB; ++d) {
        Acc C;
#pragma unroll
        for (int q = 0; q < NQ; ++q) C.c[q] = zero4;
        if constexpr (HV)
          pair_step_halves<TR::f16>(cur.A, st[r * DB + d], magic, C.c);
        else
          pair_step<TR::f16>(cur.A, st[r * DB + d], magic, C.c[0], C.c[1]);
        Ops nxt;
        if (d + 1 < DB) fetch(bc, d + 1, nxt);
        else fetch(bn, 0, nxt);
        if (d == 0 && kc.t != prev_tile) {            // uniform: the last step ended a tile
          epilogue(P, prev);
          flush(0);
          acc_tile = kc.t;
          prev_tile = kc.t;
        } else {
          epilogue(P, prev);
        }
        if (reload) load(so, d, st[r * DB + d]);
        P = C;
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
    for (int r = 0; r < RB - 1; ++r)
      if (i + r < nb) run_block(r, false);
    epilogue(P, prev);
    flush(acc_tile > tfirst ? 1 : 0);

    // ---- reduce: each output tile adds the flushed partials of the runs
    // that cover it, in wave order; SWIGLU takes the (gate, up) column pairs.
    __syncthreads();
    // All waves' slots are read unconditionally (nearest valid slot) and the
    // covering runs selected afterwards: the reads go out together.
    int tb[NW], te[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      tb[w] = run_tiles[2 * w];
      te[w] = run_tiles[2 * w + 1];
    }
    auto tile_sum = [&](int t, int within) {
      float v[NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int seg = min(max(t - tb[w], 0), 1);
        v[w] = red[((w * 2 + seg) * 256) + within];
      }
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) sum = (t >= tb[w] && t <= te[w]) ? sum + v[w] : sum;
      return sum;
    };
    if constexpr (SWIGLU) {
      for (int idx = tid; idx < tiles * 128; idx += NT) {
        const int t = idx >> 7;
        const int m = (idx >> 3) & 15;
        const int c = t * 16 + 2 * (idx & 7);         // gate column; c + 1 is its up
        if (m < M && c < wgcols) {
          const float g = tile_sum(t, m * 16 + (c & 15));
          const float u = tile_sum(t, m * 16 + (c & 15) + 1);
          y[(size_t)m * Nh + ((wg0 + c) >> 1)] = swiglu(g, u);
        }
      }
    } else {
      for (int idx = tid; idx < tiles * 256; idx += NT) {
        const int t = idx >> 8;
        const int m = (idx >> 4) & 15;
        const int c = t * 16 + (idx & 15);
        if (m < M && c < wgcols) {
          const float v = tile_sum(t, idx & 255);
          if (!fused || y) y[(size_t)m * N + wg0 + c] = v;
          if (fused) top2_add(best, v, wg0 + c);
        }
      }
    }
    __syncthreads();                                  // the table, runs and partials are reused
  }
  if (!fused) return;

  // ---- fused greedy verify, first half: the 16 lanes of a row in a wave
  // reduce, then lane m of wave 0 merges row m's two holders (waves m/4 and
  // m/4 + 4, quarter m % 4) and writes the row set's partial for this worker.
  static_assert(NW == 8, "two waves per row in the epilogue");
  top2_best16(best);
  unsigned* cand = reinterpret_cast<unsigned*>(lds);  // [NW][4] x (k1, i1, k2)
  if (j == 0) {
    unsigned* p = cand + (wave * 4 + h) * 3;
    p[0] = best.k1;
    p[1] = (unsigned)best.i1;
    p[2] = best.k2;
  }
  __syncthreads();
  if (wave == 0 && lane < M) {
    Top2 r = top2_none();
    for (int w = lane >> 2; w < NW; w += 4) {
      const unsigned* p = cand + (w * 4 + (lane & 3)) * 3;
      top2_merge(r, p[0], (int)p[1], p[2]);
    }
    va.partials[(size_t)(16 * rs + lane) * va.pgroups + wk] = top2_pack(r);
  }
}

// ---------------------------------------------------------------------------
// Wide outputs (vocabulary projections, N/16 tiles far above the wave count).
// The per-step arithmetic and the 16-row MFMA layout are those of
// qgemm_w4_m16; the split is by whole column tiles: persistent work-groups
// stage their row set's activations once (one barrier), then each wave
// streams its own tiles over all of K (tiles tbeg + w, tbeg + w + 8, ... of
// its worker's range), with a weight ring that runs on across tiles, a
// private (s, b) table in LDS rebuilt per tile from loads issued a tile
// ahead, and each finished tile stored straight to y. No barrier, partial
// sum or reduction follows the staging. Row sets and the XCD layout are as
// in qgemm_w4_m16. With va.argmax set each lane also keeps the top two of
// its rows over all its columns, and the work-group writes one top-two
// partial per row of its row set (the greedy verify's first half, as in
// qgemm_w4_m8's fused epilogue).
template <int ACT, int DB, int RB, int GS>
__global__ __launch_bounds__(512) void qgemm_w4_wide(
    const void* __restrict__ x, const uint8_t* __restrict__ wq,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases,
    float* __restrict__ y, int M, int K, int N, int rsets, int workers, int tpw,
    VerifyArgs va) {
  using TR = ActTraits<ACT>;
  // GS: group 64 << GS for GS >= 0; GS = -1 is group 32 (as in
  // qgemm_w4_m16: pair_step_halves, four partial sums per group pair).
  constexpr int gs = GS > 0 ? GS : 0;               // table shift of group 128
  constexpr bool HV = GS < 0;
  constexpr int NQ = HV ? 4 : 2;                    // scaled partial sums per pair
  constexpr int XSF = 16 * NQ;                      // row sums per activation image
  constexpr int NTR = HV ? 3 : 2;                   // table load rounds (K <= 2560, host)
  static_assert(TR::parts == 1, "16-bit activations only");
  constexpr int NW = 8, NT = 512, XB = 5;
  const bool fused = va.argmax != nullptr;           // uniform
  constexpr int D = DB * RB;
  constexpr unsigned kSkip = 0x7FF00000u;

  const int T = (N + 15) >> 4;                        // column tiles
  int wk = blockIdx.x, rs = 0;
  if (rsets > 1) {
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    rs = local % rsets;
    wk = (local / rsets) * 8 + xcd;
  }
  const int tbeg = wk * tpw, tend = min(T, tbeg + tpw);
  const int rows = min(16, M - 16 * rs);            // rows of this row set
  if (wk >= workers || tbeg >= T) {                  // the whole group leaves
    if (fused && (int)threadIdx.x < rows)            // with empty partials
      va.partials[(size_t)(16 * rs + threadIdx.x) * va.pgroups + wk] = top2_pack(top2_none());
    return;
  }
  x = static_cast<const uint16_t*>(x) + (size_t)rs * 16 * K;
  if (y) y += (size_t)rs * 16 * N;
  M = rows;

  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15;
  const int h = lane >> 4;
  const int G = K >> 6;                               // even, a multiple of 8 (host)
  const int GP = G >> 1;
  const int bpt = GP / DB;
  const unsigned rowbytes = (unsigned)K >> 1;
  const M16Layout L = m16_layout(G, 16, NW, XB, HV);
  const int TG = HV ? 2 * G : G;                      // table entries per column
  unsigned char* xl = lds;
  float* xsl = reinterpret_cast<float*>(lds + L.xs);
  // Per-wave table: [16 columns][TG] of (s | b << 16), after the row sums.
  unsigned* tab = reinterpret_cast<unsigned*>(lds + L.sb) + wave * 16 * TG;

  unsigned magic;
  asm volatile("v_mov_b32 %0, %1" : "=v"(magic) : "i"(TR::magic));
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(x), (short)0, M * K * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(wq), (short)0, (unsigned)N * rowbytes, kBufferFlags);
  const unsigned ME = HV ? 2u * (unsigned)G : (unsigned)(G >> gs);  // table entries per row
  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(scales), (short)0, (unsigned)N * ME * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(biases), (short)0, (unsigned)N * ME * 2, kBufferFlags);

  // ---- this wave's tiles and blocks: tile ordinal k is column tile
  // tbeg + wave + 8k; block (k, p) covers pairs p .. p + DB - 1.
  const int ntile = tend > tbeg + wave ? (tend - tbeg - wave + NW - 1) / NW : 0;
  const int nb = ntile * bpt;
  struct Blk {
    int k, p, left;
  };
  auto next = [&](Blk b) {
    b.p += DB;
    b.k += b.p == GP;
    b.p = b.p == GP ? 0 : b.p;
    b.left -= 1;
    return b;
  };
  auto col0 = [&](int k) { return (tbeg + wave + NW * k) * 16; };
  const unsigned woff = (unsigned)j * rowbytes + 16u * h;
  auto codes_at = [&](const Blk& b) {
    return b.left > 0 ? (unsigned)col0(b.k) * rowbytes + 64u * (unsigned)b.p : kSkip;
  };
  u32x4 st[D];
  auto load = [&](unsigned so, int d, u32x4& w) {
    w = __builtin_amdgcn_raw_buffer_load_b128(wr, woff + 64u * d, so, 0);
  };
  // A tile's table: 16 columns x TG entries, contiguous in memory; unit u
  // (16 bytes, entries 8(u % (TG/8)) ..) of each array per lane and round.
  const int tunits = 2 * TG;                          // 16 * TG / 8
  u32x4 ts[NTR], tb[NTR];
  auto tab_load = [&](int k) {                        // k may be past the run: zeros
#pragma unroll
    for (int r = 0; r < NTR; ++r) {
      const int u = r * 64 + lane;
      const int c = col0(k) + (8 * u) / TG;
      const bool ok = k < ntile && u < tunits && c < N;
      const unsigned off =
          ok ? 2u * (((unsigned)col0(k) * (unsigned)TG + 8u * (unsigned)u) >> gs) : kOutOfRange;
      ts[r] = sb_unit_load<GS>(sr, off);
      tb[r] = sb_unit_load<GS>(br, off);
    }
  };
  auto tab_store = [&]() {
#pragma unroll
    for (int r = 0; r < NTR; ++r) {
      const int u = r * 64 + lane;
      if (u < tunits) {
        u32x4 lo, hi;
        sb_pairs<GS>(ts[r], tb[r], lo, hi);
        *reinterpret_cast<u32x4*>(tab + 8 * u) = lo;
        *reinterpret_cast<u32x4*>(tab + 8 * u + 4) = hi;
      }
    }
  };

  // ---- prologue: the activation loads first, then tile 0's table and the
  // weight ring; staging; tile 0's table to LDS and tile 1's loads.
  const int ngrp = 2 * GP;
  const int rounds = (ngrp + NW - 1) / NW;            // <= XB (host: K <= 64 * NW * XB)
  const int e8 = lane & 7;
  const int mm = lane >> 3;
  u32x4 xv[XB][2];
#pragma unroll
  for (int i = 0; i < XB; ++i) {
    const int g = wave + NW * i;
    const int kk = 64 * g + 8 * e8;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = mm + 8 * r;
      const bool ok = row < M && kk < K;
      xv[i][r] = __builtin_amdgcn_raw_buffer_load_b128(
          xr, ok ? (unsigned)((row * K + kk) * 2) : kOutOfRange, 0, 0);
    }
  }
  tab_load(0);
  const Blk kfirst = {0, 0, nb};
  Blk kl = kfirst;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    load(codes_at(kl), d % DB, st[d]);
    if (d % DB == DB - 1) kl = next(kl);
  }
  (void)rounds;
  const unsigned xl_lane =
      HV ? (e8 >> 2) * kTRow16 + ((e8 & 3) * 16 + mm) * kSlot16
         : (e8 & 1) * kTRow16 + (sigma_slot(e8 >> 1) * 16 + mm) * kSlot16;
#pragma unroll
  for (int i = 0; i < XB; ++i) {
    const int g = wave + NW * i;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const float s8 = HV ? sum4_lanes(block_sum<ACT>(xv[i][r]))
                          : sum8_lanes(block_sum<ACT>(xv[i][r]));
      *reinterpret_cast<u32x4*>(xl + (g >> 1) * kPair16 + (g & 1) * 2 * kTRow16 + xl_lane +
                                r * 8 * kSlot16) = permute_pairs(xv[i][r]);
      xsl[HV ? (g * 2 + (e8 >> 2)) * 16 + mm + 8 * r : g * 16 + mm + 8 * r] = s8;
    }
  }
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int i = tid; i < kPair16 / 16; i += NT)      // the zero image
      *reinterpret_cast<u32x4*>(xl + GP * kPair16 + 16 * i) = z;
    if (tid < XSF) xsl[GP * XSF + tid] = 0.0f;
  }
  tab_store();
  tab_load(1);
  __syncthreads();                                    // the activation image is complete

  // ---- main loop (the step, ring and deferred epilogue of qgemm_w4_m16).
  const unsigned char* abase = xl + (h * 16 + j) * kSlot16;
  const float* xsbase = xsl + 4 * h;
  const unsigned* tbase = tab + j * TG;
  const unsigned* sbzero = reinterpret_cast<const unsigned*>(xsl + GP * XSF);
  // The step's operands: of groups 2p and 2p+1, or (HV) of their halves.
  struct OpsG {
    u32x4 A[4];
    f32x4 xs0, xs1;
    u32x2 sb;
  };
  struct OpsH {
    u32x4 A[4];
    f32x4 xs[4];
    u32x4 sb;
  };
  using Ops = std::conditional_t<HV, OpsH, OpsG>;
  struct Base {
    const unsigned char* a;
    const float* xs;
    const unsigned* sb;
  };
  auto base_of = [&](const Blk& b) {
    const bool in = b.left > 0;                       // uniform
    const int img = in ? b.p : GP;
    Base bs;
    bs.a = abase + img * kPair16;
    bs.xs = xsbase + img * XSF;
    bs.sb = in ? tbase + NQ * b.p : sbzero;
    return bs;
  };
  auto fetch = [&](const Base& bs, int d, Ops& o) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
      o.A[t] = *reinterpret_cast<const u32x4*>(bs.a + d * kPair16 + t * kTRow16);
    if constexpr (HV) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o.xs[q] = *reinterpret_cast<const f32x4*>(bs.xs + d * XSF + 16 * q);
      o.sb = *reinterpret_cast<const u32x4*>(bs.sb + 4 * d);
    } else {
      o.xs0 = *reinterpret_cast<const f32x4*>(bs.xs + d * 32);
      o.xs1 = *reinterpret_cast<const f32x4*>(bs.xs + d * 32 + 16);
      o.sb = *reinterpret_cast<const u32x2*>(bs.sb + 2 * d);
    }
  };
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  Top2Scan best[4] = {top2_scan_none(), top2_scan_none(), top2_scan_none(), top2_scan_none()};
  // A finished tile goes straight to y: lane (j, h) holds rows 4h .. 4h+3 of
  // column j (a lane's tiles come in increasing column order, as top2_scan
  // needs). The stores are non-temporal: nothing here reads y again, and at
  // the vocabulary width (4.9 MB of logits) the projection ran 46.8 against
  // 47.7 us with ordinary stores.
  auto store_tile = [&](int k) {
    const int c = col0(k) + j;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 4 * h + e;
      if (m < M && c < N) {
        if (!fused || y) __builtin_nontemporal_store(acc[e], &y[(size_t)m * N + c]);
        if (fused) top2_scan(best[e], acc[e], c, acc[e] == acc[e]);
      }
      acc[e] = 0.0f;
    }
  };
  struct Acc { f32x4 c[NQ]; };                      // a step's partial sums
  auto epilogue = [&](const Acc& C, const Ops& o) {
    if constexpr (HV) {
      float s[4], c[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        s[q] = half_lo(o.sb[q]);
        c[q] = fmaf(-TR::c0, s[q], half_hi(o.sb[q]));
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[e] = fmaf(s[q], C.c[q][e], fmaf(c[q], o.xs[q][e], acc[e]));
    } else {
      const float s0 = half_lo(o.sb.x), s1 = half_lo(o.sb.y);
      const float c0 = fmaf(-TR::c0, s0, half_hi(o.sb.x));
      const float c1 = fmaf(-TR::c0, s1, half_hi(o.sb.y));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] = fmaf(s0, C.c[0][e], fmaf(c0, o.xs0[e], acc[e]));
        acc[e] = fmaf(s1, C.c[1][e], fmaf(c1, o.xs1[e], acc[e]));
      }
    }
  };

  Ops cur, prev;
  const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
  Acc P;
#pragma unroll
  for (int q = 0; q < NQ; ++q) P.c[q] = zero4;
  if constexpr (HV) {                                // step -1 adds exactly nothing
    prev.sb = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < 4; ++q) prev.xs[q] = zero4;
  } else {
    prev.sb = u32x2{0u, 0u};
    prev.xs0 = zero4;
    prev.xs1 = zero4;
  }
  Blk kc = kfirst;
  Base bc = base_of(kc);
  fetch(bc, 0, cur);
  auto run_block = [&](int r, bool reload) {
    const Blk kn = next(kc);
    const unsigned so = codes_at(kl);
#pragma unroll
    for (int d = 0; d < DB; ++d) {
      Acc C;
#pragma unroll
      for (int q = 0; q < NQ; ++q) C.c[q] = zero4;
      if constexpr (HV)
        pair_step_halves<TR::f16>(cur.A, st[r * DB + d], magic, C.c);
      else
        pair_step<TR::f16>(cur.A, st[r * DB + d], magic, C.c[0], C.c[1]);
      Ops nxt;
      if (d + 1 < DB) {
        fetch(bc, d + 1, nxt);
      } else {
        // The next block starts a new tile: its table (loaded during this
        // tile) replaces this tile's, whose remaining entries are already in
        // registers, and the loads for the tile after it go out.
        if (kn.p == 0 && kn.left > 0) {
          tab_store();
          tab_load(kn.k + 1);
        }
        fetch(base_of(kn), 0, nxt);
      }
      epilogue(P, prev);
      if (d == 0 && kc.p == 0 && kc.k > 0) store_tile(kc.k - 1);  // uniform
      if (reload) load(so, d, st[r * DB + d]);
      P = C;
      prev = cur;
      cur = nxt;
    }
    if (reload) kl = next(kl);
    kc = kn;
    bc = base_of(kc);
  };
  int i = 0;
  for (; i + RB <= nb; i += RB) {
#pragma unroll
    for (int r = 0; r < RB; ++r) run_block(r, true);
  }
#pragma unroll
  for (int r = 0; r < RB - 1; ++r)
    if (i + r < nb) run_block(r, false);
  epilogue(P, prev);
  if (ntile > 0) store_tile(ntile - 1);

  if (fused) {
    // The 16 lanes of a (row, h) group reduce; the waves' results combine in
    // LDS (the activation image is no longer read once every wave is past
    // its loop); lane m of wave 0 writes the partial of the row set's row m.
    __syncthreads();
    unsigned* cand = reinterpret_cast<unsigned*>(lds);  // [NW][16 rows] x (k1, i1, k2)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      Top2 t = top2_of_scan(best[e]);
      top2_best16(t);
      if (j == 0) {
        unsigned* q = cand + (wave * 16 + 4 * h + e) * 3;
        q[0] = t.k1;
        q[1] = (unsigned)t.i1;
        q[2] = t.k2;
      }
    }
    __syncthreads();
    if (wave == 0 && lane < M) {
      Top2 r = top2_none();
      for (int w = 0; w < NW; ++w) {
        const unsigned* q = cand + (w * 16 + lane) * 3;
        top2_merge(r, q[0], (int)q[1], q[2]);
      }
      va.partials[(size_t)(16 * rs + lane) * va.pgroups + wk] = top2_pack(r);
    }
  }
}

// Elementwise SwiGLU of a [M, 2*Nh] projection output (the fallback path).
__global__ __launch_bounds__(256) void swiglu_rows(const float* __restrict__ yg,
                                                   float* __restrict__ hout, int M, int Nh) {
  const long long total = (long long)M * Nh;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (long long)gridDim.x * 256) {
    const long long m = i / Nh, jj = i - m * Nh;
    const float* row = yg + m * 2 * Nh;
    hout[i] = swiglu(row[jj], row[Nh + jj]);
  }
}

constexpr int kM16Waves = 8;
constexpr int kM16Tiles = 5;
constexpr int kM16XB = 5;

// Columns per column group of qgemm_w4_m16: an equal share of the CUs,
// rounded up to 4, at most kM16Tiles tiles.
int m16_cols(int N) {
  const int cus = device_cus();
  const int share = ((N + cus - 1) / cus + 3) / 4 * 4;
  return share < 16 * kM16Tiles ? share : 16 * kM16Tiles;
}

// Workers per row set of qgemm_w4_m16: one work-group per CU, rsets row
// sets of `workers` each (a multiple of 8 when there are several row sets,
// for the XCD layout); one row set takes no more workers than groups.
int m16_workers(int M, int N) {
  const int rsets = (M + 15) / 16;
  const int cols = m16_cols(N);
  const int groups = (N + cols - 1) / cols;
  const int cus = device_cus();
  int workers = rsets > 1 ? (cus / rsets) / 8 * 8 : cus;
  if (workers < 8) workers = 8;
  if (rsets == 1 && workers > groups) workers = groups;
  return workers;
}

template <int ACT, int DB, int RB, bool SWIGLU>
hipError_t launch_m16(const void* x, const uint8_t* wq, const uint16_t* scales,
                      const uint16_t* biases, float* y, int M, int K, int N, int cols,
                      int gs, const VerifyArgs& va, hipStream_t stream) {
  const int rsets = (M + 15) / 16;
  const int workers = m16_workers(M, N);
  const M16Layout L = m16_layout(K >> 6, 16 * kM16Tiles, kM16Waves, kM16XB, gs < 0);
  if (L.total > kLdsLimit) return hipErrorInvalidValue;  // never launched
  constexpr int D0 = DB;                                // one block ahead of the staging
  const int tg = gs < 0 ? 2 * (K >> 6) : (K >> 6);      // table entries per column
  const bool sbv = tg % 8 == 0 &&
                   ((reinterpret_cast<uintptr_t>(scales) | reinterpret_cast<uintptr_t>(biases)) &
                    15) == 0;
  constexpr int W = kM16Waves, T = kM16Tiles, X = kM16XB;
  auto kern = qgemm_w4_m16<ACT, W, T, DB, RB, D0, X, SWIGLU, false, 0>;
  if (sbv) {
    kern = qgemm_w4_m16<ACT, W, T, DB, RB, D0, X, SWIGLU, true, 0>;
    if (gs > 0) kern = qgemm_w4_m16<ACT, W, T, DB, RB, D0, X, SWIGLU, true, 1>;
    if (gs < 0) kern = qgemm_w4_m16<ACT, W, T, DB, RB, D0, X, SWIGLU, true, -1>;
  } else {
    if (gs > 0) kern = qgemm_w4_m16<ACT, W, T, DB, RB, D0, X, SWIGLU, false, 1>;
    if (gs < 0) kern = qgemm_w4_m16<ACT, W, T, DB, RB, D0, X, SWIGLU, false, -1>;
  }
  if (L.total > 65536) {
    const hipError_t e = allow_lds(reinterpret_cast<const void*>(kern));
    if (e != hipSuccess) return e;
  }
  const dim3 grid(workers * rsets);
  hipLaunchKernelGGL(kern, grid, dim3(64 * kM16Waves), L.total, stream, x, wq, scales, biases,
                     y, M, K, N, cols, rsets, workers, va);
  return hipGetLastError();
}

template <int ACT, bool SWIGLU>
hipError_t launch_m16_blocks(const void* x, const uint8_t* wq, const uint16_t* scales,
                             const uint16_t* biases, float* y, int M, int K, int N,
                             int gs, const VerifyArgs& va, hipStream_t s) {
  const int cols = m16_cols(N);
  const int GP = ((K >> 6) + 1) >> 1;
  if (GP % 5 == 0)
    return launch_m16<ACT, 5, 1, SWIGLU>(x, wq, scales, biases, y, M, K, N, cols, gs, va, s);
  if (GP % 4 == 0)
    return launch_m16<ACT, 4, 2, SWIGLU>(x, wq, scales, biases, y, M, K, N, cols, gs, va, s);
  if (GP % 2 == 0)
    return launch_m16<ACT, 2, 4, SWIGLU>(x, wq, scales, biases, y, M, K, N, cols, gs, va, s);
  return launch_m16<ACT, 1, 8, SWIGLU>(x, wq, scales, biases, y, M, K, N, cols, gs, va, s);
}

template <int ACT, int DB, int RB>
hipError_t launch_wide(const void* x, const uint8_t* wq, const uint16_t* scales,
                       const uint16_t* biases, float* y, int M, int K, int N, int rsets,
                       int workers, int gs, const VerifyArgs& va, hipStream_t stream) {
  const int G = K >> 6;
  const M16Layout L = m16_layout(G, 16, 8, 5, gs < 0);
  const int lds_bytes = L.sb + 8 * 16 * (gs < 0 ? 2 * G : G) * 4;
  if (lds_bytes > kLdsLimit) return hipErrorInvalidValue;  // never launched
  auto kern = qgemm_w4_wide<ACT, DB, RB, 0>;
  if (gs > 0) kern = qgemm_w4_wide<ACT, DB, RB, 1>;
  if constexpr (DB == 4 && RB == 1) {
    if (gs < 0) kern = qgemm_w4_wide<ACT, DB, RB, -1>;
  } else {
    if (gs < 0) return hipErrorInvalidValue;         // never launched
  }
  if (lds_bytes > 65536) {
    const hipError_t e = allow_lds(reinterpret_cast<const void*>(kern));
    if (e != hipSuccess) return e;
  }
  const int T = (N + 15) / 16;
  const int tpw = (T + workers - 1) / workers;
  hipLaunchKernelGGL(kern, dim3(workers * rsets), dim3(512), lds_bytes, stream, x, wq, scales,
                     biases, y, M, K, N, rsets, workers, tpw, va);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Wide outputs with 17..64 rows: every row set on one weight stream.
// qgemm_w4_wide gives each row set work-groups of their own, so each weight
// byte is unpacked once per row set and crosses the CU-L2 link once per row
// set. Here one work-group per CU owns a contiguous range of column tiles for
// all RS row sets, and K is cut into chunks of KCP group pairs: the chunk's
// activations of all rows (RS images per pair, the 16-row layout above) and
// the waves' (s, b) tables are staged, then each wave runs its tiles over
// the chunk's pairs with one unpack per code and RS x 4 MFMAs per step,
// accumulating in registers across chunks (KT tiles x RS row sets).
// * Step order: the wave's tiles in blocks of two; within a block the pairs
//   in order, and at each pair both tiles' codes are unpacked once for all
//   row sets, then each row set's A operands are read once from LDS for
//   both tiles. (Pair-major order over all tiles, holding some A operands in
//   registers, was about 4 % slower than one tile at a time; two tiles per
//   A read is 2 % faster than one.)
// * Weight ring: whole-line units (qgemm_common.h: a tile times 128 bytes of
//   each column, two loads of eight whole lines each, rearranged into the
//   two steps' operands by exchange()), kRowsRing units ahead, running on
//   across chunk boundaries, so the next chunk's first weights are in flight
//   during its staging. Loading each line in two 64-byte halves, one step
//   apart, read a third of the lines twice (1.32x the weight bytes; 1.04x
//   whole). Non-temporal: the codes are read once. Units past a wave's tiles
//   or past K read zeros.
// * The work-group's tiles: [tbeg, tbeg + tpw); wave w takes tbeg + w + 8k.
// Every sum runs in a fixed order, so results are deterministic. With
// va.argmax set the work-group also writes one top-two partial per row over
// its columns (the greedy verify's first half, as in qgemm_w4_wide).
// LDS of qgemm_w4_rows: the chunk's activation images and row sums and each
// wave's (s, b) table during the loop; the fused verify's candidates after
// it (one line per wave and column, then one entry per wave and row).
template <int RS, int KT, int KCP, bool HV>
constexpr int rows_lds_bytes() {
  const int loop = KCP * RS * (kPair16 + (HV ? 256 : 128)) + 8 * KT * 16 * (HV ? 4 : 2) * KCP * 4;
  const int cand = 8 * 16 * (3 * 16 * RS + 1) * 4 + 8 * 16 * RS * 12;
  return loop > cand ? loop : cand;
}

// Whole-line units of weights in flight per wave in qgemm_w4_rows (two steps
// each; 2 and 3 measured about 1 % slower), and their cache policy bits
// (non-temporal: without them the kernel read 319 against 227 MB per launch
// at K = 2560, N = 151936, and ran 6 % slower).
constexpr int kRowsRing = 4;
constexpr int kRowsAux = 2;

template <int ACT, int RS, int KT, int KCP, int GS>
__global__ __launch_bounds__(512) void qgemm_w4_rows(
    const void* __restrict__ x, const uint8_t* __restrict__ wq,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases,
    float* __restrict__ y, int M, int K, int N, int tpw, VerifyArgs va) {
  using TR = ActTraits<ACT>;
  // GS: group 64 << GS for GS >= 0; GS = -1 is group 32 (as in
  // qgemm_w4_m16: four partial sums per pair and row set, one per group
  // half, each with its own scale, bias and row sum).
  constexpr int gs = GS > 0 ? GS : 0;               // table shift of group 128
  constexpr bool HV = GS < 0;
  constexpr int NQ = HV ? 4 : 2;                    // scaled partial sums per pair
  constexpr int XSF = 16 * NQ;                      // row sums per image
  static_assert(TR::parts == 1, "16-bit activations only");
  constexpr int NW = 8;
  constexpr int GC = 2 * KCP;                        // groups per chunk
  constexpr int ITEMS = GC * 2 * RS;                 // (group, row octet) staging items
  constexpr int XR = (ITEMS + NW - 1) / NW;          // staging loads per lane
  constexpr int TABD = KT * 16 * KCP;                // table dwords per array and wave
  constexpr int TABL = (TABD + 63) / 64;             // table loads per array and lane
  constexpr unsigned kSkip = 0x7FF00000u;

  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  unsigned char* ximg = lds;                                        // [KCP][RS] images
  float* xsl = reinterpret_cast<float*>(lds + KCP * RS * kPair16);  // [KCP][RS][NQ][16]
  unsigned* tab_all = reinterpret_cast<unsigned*>(lds + KCP * RS * (kPair16 + 4 * XSF));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15;
  const int h = lane >> 4;
  const int G = K >> 6;                              // even (host)
  const int GP = G >> 1;
  const int nch = (GP + KCP - 1) / KCP;
  const unsigned rowbytes = (unsigned)K >> 1;
  const int T = (N + 15) >> 4;
  const int tbeg = blockIdx.x * tpw;
  const int tend = min(T, tbeg + tpw);
  // [KT][16 columns][NQ * KCP] of (s | b << 16)
  unsigned* tab = tab_all + wave * KT * 16 * NQ * KCP;

  unsigned magic;
  asm volatile("v_mov_b32 %0, %1" : "=v"(magic) : "i"(TR::magic));
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(x), (short)0, M * K * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(wq), (short)0, (unsigned)N * rowbytes, kBufferFlags);
  const unsigned ME = HV ? 2u * (unsigned)G : (unsigned)(G >> gs);  // table entries per row
  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(scales), (short)0, (unsigned)N * ME * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(biases), (short)0, (unsigned)N * ME * 2, kBufferFlags);

  // This wave's tiles (uniform): tile k is tbeg + wave + 8k while below tend.
  int tile[KT];
  bool tin[KT];
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    tile[k] = tbeg + wave + NW * k;
    tin[k] = tile[k] < tend;
  }
  // Whole-line units (qgemm_common.h): tile k times the 128 bytes of group
  // pairs 2q and 2q+1 of the chunk, two loads (columns 0-7 and 8-15).
  static_assert(KCP % 2 == 0, "chunks of whole 128-byte lines");
  constexpr int QC = KCP / 2;                        // units per tile and chunk
  const unsigned voff_a = (unsigned)(j & 7) * rowbytes + 64u * (unsigned)(j >> 3) + 16u * h;
  const unsigned voff_b = voff_a + 8u * rowbytes;
  auto codes_at = [&](int c, int q, int k) {        // unit (chunk, pair pair, tile)
    const int pg = c * KCP + 2 * q;
    return tin[k] && c < nch && pg < GP
               ? (unsigned)tile[k] * 16u * rowbytes + 64u * (unsigned)pg
               : kSkip;
  };
  // The units in flight: ring[i] holds unit u + i's codes when unit u is
  // next, the units running tile-major through each chunk and on into the
  // next (unit u of a chunk: tile u / QC, pairs 2(u % QC) and 2(u % QC) + 1).
  constexpr int RU = kRowsRing;
  static_assert(RU <= KT * QC, "the ring reaches at most one chunk ahead");
  struct Unit {
    u32x4 a, b;
  };
  // Unit u of a chunk in consumption order: tiles in blocks of two (the
  // last block of one when KT is odd), and within a block the quads in
  // order, the block's two tiles alternating.
  auto unit_load = [&](int c, int u) {
    constexpr int F = (KT / 2) * 2 * QC;             // units in two-tile blocks
    const int dc = u / (KT * QC), w = u % (KT * QC);
    const int k = w < F ? 2 * (w / (2 * QC)) + (w % 2) : KT - 1;
    const int q = w < F ? (w % (2 * QC)) / 2 : w - F;
    const unsigned so = codes_at(c + dc, q, k);
    Unit r;
    r.a = __builtin_amdgcn_raw_buffer_load_b128(wr, voff_a, so, kRowsAux);
    r.b = __builtin_amdgcn_raw_buffer_load_b128(wr, voff_b, so, kRowsAux);
    return r;
  };
  Unit ring[RU];
#pragma unroll
  for (int i = 0; i < RU; ++i) ring[i] = unit_load(0, i);

  f32x4 acc[KT][RS];
#pragma unroll
  for (int k = 0; k < KT; ++k)
#pragma unroll
    for (int r = 0; r < RS; ++r) acc[k][r] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int e8 = lane & 7;
  const int mm = lane >> 3;
  const unsigned xl_lane =
      HV ? (e8 >> 2) * kTRow16 + ((e8 & 3) * 16 + mm) * kSlot16
         : (e8 & 1) * kTRow16 + (sigma_slot(e8 >> 1) * 16 + mm) * kSlot16;

  // ---- activations of all rows for groups cc*GC .. cc*GC + GC-1; items
  // (group gl, row octet ro) are dealt to the waves. Chunk 0's are loaded
  // here, each later chunk's during the previous chunk's last block of
  // tiles, so that its staging finds them in registers (chunks past K load
  // nothing).
  u32x4 xv[XR];
  auto x_load = [&](int cc) {
#pragma unroll
    for (int i = 0; i < XR; ++i) {
      const int it = wave + NW * i;
      const int gl = it / (2 * RS), ro = it % (2 * RS);
      const int row = 8 * ro + mm;
      const int kk = 64 * (cc * GC + gl) + 8 * e8;
      const bool ok = it < ITEMS && row < M && kk < K;
      xv[i] = __builtin_amdgcn_raw_buffer_load_b128(
          xr, ok ? (unsigned)((row * K + kk) * 2) : kOutOfRange, 0, 0);
    }
  };
  x_load(0);

  for (int c = 0; c < nch; ++c) {
    if (c > 0) __syncthreads();                      // chunk c-1's image and tables are read
    // ---- this wave's table for the chunk, and the activations' image.
    // One dword per entry pair, two with HV (four entries).
    using TabWord = std::conditional_t<HV, u32x2, unsigned>;
    TabWord ts[TABL], tb[TABL];
#pragma unroll
    for (int n = 0; n < TABL; ++n) {
      const int e = 64 * n + lane;
      const int k = e / (16 * KCP), jj = (e / KCP) % 16, d = e % KCP;
      const int col = (tbeg + wave + NW * k) * 16 + jj;
      const bool ok = e < TABD && tbeg + wave + NW * k < tend && col < N && c * KCP + d < GP;
      // Entries of groups 2d and 2d+1 of the chunk: one 32-bit load, the one
      // entry of their 128-group twice, or (HV) the four entries of their
      // halves in one 64-bit load.
      if constexpr (HV) {
        const unsigned e0 = (unsigned)col * ME + 4u * (unsigned)(c * KCP + d);
        const unsigned off = ok ? 2u * e0 : kOutOfRange;
        ts[n] = __builtin_amdgcn_raw_buffer_load_b64(sr, off, 0, 0);
        tb[n] = __builtin_amdgcn_raw_buffer_load_b64(br, off, 0, 0);
      } else {
        const unsigned e0 = ((unsigned)col * (unsigned)G + (unsigned)(c * GC + 2 * d)) >> gs;
        const unsigned off = ok ? 2u * e0 : kOutOfRange;
        if constexpr (GS == 0) {
          ts[n] = __builtin_amdgcn_raw_buffer_load_b32(sr, off, 0, 0);
          tb[n] = __builtin_amdgcn_raw_buffer_load_b32(br, off, 0, 0);
        } else {
          ts[n] = 0x10001u * (unsigned)__builtin_amdgcn_raw_buffer_load_b16(sr, off, 0, 0);
          tb[n] = 0x10001u * (unsigned)__builtin_amdgcn_raw_buffer_load_b16(br, off, 0, 0);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < XR; ++i) {
      const int it = wave + NW * i;
      if (it >= ITEMS) continue;                     // uniform: the last round is partial
      const int gl = it / (2 * RS), ro = it % (2 * RS);
      const int r = ro >> 1, r8 = ro & 1;
      const float s8 = HV ? sum4_lanes(block_sum<ACT>(xv[i])) : sum8_lanes(block_sum<ACT>(xv[i]));
      *reinterpret_cast<u32x4*>(ximg + ((gl >> 1) * RS + r) * kPair16 + (gl & 1) * 2 * kTRow16 +
                                xl_lane + r8 * 8 * kSlot16) = permute_pairs(xv[i]);
      const int q = HV ? (gl & 1) * 2 + (e8 >> 2) : (gl & 1);  // partial sum of the values
      xsl[((gl >> 1) * RS + r) * XSF + q * 16 + mm + 8 * r8] = s8;
    }
#pragma unroll
    for (int n = 0; n < TABL; ++n) {
      const int e = 64 * n + lane;
      if (e < TABD) {
        const int k = e / (16 * KCP), jj = (e / KCP) % 16, d = e % KCP;
        unsigned* q = tab + (k * 16 + jj) * (NQ * KCP) + NQ * d;
        if constexpr (HV) {
          q[0] = __builtin_amdgcn_perm(tb[n].x, ts[n].x, 0x05040100u);
          q[1] = __builtin_amdgcn_perm(tb[n].x, ts[n].x, 0x07060302u);
          q[2] = __builtin_amdgcn_perm(tb[n].y, ts[n].y, 0x05040100u);
          q[3] = __builtin_amdgcn_perm(tb[n].y, ts[n].y, 0x07060302u);
        } else {
          q[0] = __builtin_amdgcn_perm(tb[n], ts[n], 0x05040100u);
          q[1] = __builtin_amdgcn_perm(tb[n], ts[n], 0x07060302u);
        }
      }
    }
    __syncthreads();

    // ---- the chunk's steps in blocks of two tiles (the last block of an odd
    // KT has one): for each pair p the codes of the block's tiles are
    // unpacked, then each row set's A operands are read once from LDS and
    // meet both tiles. An even pair takes the next unit of each tile: the
    // exchange gives the unit's two steps' operands, the ring shifts
    // (register renaming in the unrolled chunk) and loads the unit RU ahead;
    // the odd pair uses the second operands.
    u32x4 w_odd[2];
    int u = 0;                                       // this chunk's next unit (compile-time)
#pragma unroll
    for (int kb = 0; kb < (KT + 1) / 2; ++kb) {
      const int nk = 2 * kb + 1 < KT ? 2 : 1;
#pragma unroll
      for (int p = 0; p < KCP; ++p) {
        // Per-step LDS offsets behind an empty asm: the steps' reads must not
        // be hoisted out of the loops (registers).
        unsigned a_step = (unsigned)(h * 16 + j) * kSlot16, x_step = 4u * (unsigned)h;
        asm volatile("" : "+v"(a_step), "+v"(x_step));
        if (kb == (KT - 1) / 2 && p == 0) x_load(c + 1);  // the next chunk's activations
        u32x4 bq[2][4];
        float sq[2][NQ], cq[2][NQ];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          if (kk >= nk) continue;
          const int k = 2 * kb + kk;
          u32x4 w;
          if (p % 2 == 0) {
            exchange(ring[0].a, ring[0].b, w, w_odd[kk]);
            // Both operands are complete before the refill is issued, so the
            // slot's registers are free for it.
            asm volatile("" : "+v"(w), "+v"(w_odd[kk]) :: "memory");
#pragma unroll
            for (int i = 0; i + 1 < RU; ++i) ring[i] = ring[i + 1];
            ring[RU - 1] = unit_load(c, u + RU);
            ++u;
          } else {
            w = w_odd[kk];
          }
          const u32x4 v = split_groups(w);
          if constexpr (HV) {
            // One more swap per group: MFMA q sees half q % 2 of group 2p + q / 2.
            const auto a = __builtin_amdgcn_permlane16_swap(v.x, v.y, false, false);
            const auto b = __builtin_amdgcn_permlane16_swap(v.z, v.w, false, false);
            bq[kk][0] = unpack_codes(a[0], magic);
            bq[kk][1] = unpack_codes(a[1], magic);
            bq[kk][2] = unpack_codes(b[0], magic);
            bq[kk][3] = unpack_codes(b[1], magic);
            const u32x4 sb =
                *reinterpret_cast<const u32x4*>(tab + (k * 16 + j) * (NQ * KCP) + NQ * p);
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
              sq[kk][q] = half_lo(sb[q]);
              cq[kk][q] = fmaf(-TR::c0, sq[kk][q], half_hi(sb[q]));
            }
          } else {
            // The bias term is added per chunk (below): only the scales here.
#pragma unroll
            for (int t = 0; t < 4; ++t) bq[kk][t] = unpack_codes(v[t], magic);
            const u32x2 sb = *reinterpret_cast<const u32x2*>(tab + (k * 16 + j) * GC + 2 * p);
            sq[kk][0] = half_lo(sb.x);
            sq[kk][1] = half_lo(sb.y);
          }
        }
#pragma unroll
        for (int r = 0; r < RS; ++r) {
          const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
          u32x4 Ar[4];
#pragma unroll
          for (int t = 0; t < 4; ++t)
            Ar[t] = *reinterpret_cast<const u32x4*>(ximg + a_step + (p * RS + r) * kPair16 +
                                                    t * kTRow16);
          const float* xs = xsl + (p * RS + r) * XSF + x_step;
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            if (kk >= nk) continue;
            const int k = 2 * kb + kk;
            if constexpr (HV) {
              f32x4 C[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) C[q] = mfma16x16x32<TR::f16>(Ar[q], bq[kk][q], zero4);
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const f32x4 xq = *reinterpret_cast<const f32x4*>(xs + 16 * q);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  acc[k][r][e] =
                      fmaf(sq[kk][q], C[q][e], fmaf(cq[kk][q], xq[e], acc[k][r][e]));
              }
            } else {
              (void)xs;
              f32x4 C0 = mfma16x16x32<TR::f16>(Ar[0], bq[kk][0], zero4);
              f32x4 C1 = mfma16x16x32<TR::f16>(Ar[2], bq[kk][2], zero4);
              C0 = mfma16x16x32<TR::f16>(Ar[1], bq[kk][1], C0);
              C1 = mfma16x16x32<TR::f16>(Ar[3], bq[kk][3], C1);
#pragma unroll
              for (int e = 0; e < 4; ++e)
                acc[k][r][e] = fmaf(sq[kk][1], C1[e], fmaf(sq[kk][0], C0[e], acc[k][r][e]));
            }
            // The tile's sums are not read again before the chunk's bias
            // term: without this the compiler defers every step's update to
            // there and keeps all the steps' products live.
            asm volatile("" : "+v"(acc[k][r]));
          }
        }
      }
    }

    if constexpr (!HV) {
      // ---- the chunk's bias term, sum_g (b - c0*s)[n, g] * xs[m, g] over its
      // 2*KCP groups: a [16 rows x groups] x [groups x 16 columns] contraction
      // on the fp32 MFMA, four groups at a time, added into the accumulators
      // (same output layout). Lane (i, h) brings xs of row i, group 4u + h;
      // lane (j, h) brings b - c0*s of column j, the same group; groups past
      // the chunk bring zeros.
      constexpr int NU = (GC + 3) / 4;
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int gl = 4 * u + h;
        const bool gin = gl < GC;
        float xa[RS], bb[KT];
#pragma unroll
        for (int r = 0; r < RS; ++r)
          xa[r] = gin ? xsl[((gl >> 1) * RS + r) * XSF + (gl & 1) * 16 + j] : 0.0f;
#pragma unroll
        for (int k = 0; k < KT; ++k) {
          const unsigned sb = gin ? tab[(k * 16 + j) * GC + gl] : 0u;
          bb[k] = fmaf(-TR::c0, half_lo(sb), half_hi(sb));
        }
#pragma unroll
        for (int k = 0; k < KT; ++k)
#pragma unroll
          for (int r = 0; r < RS; ++r)
            acc[k][r] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[r], bb[k], acc[k][r], 0, 0, 0);
      }
    }
  }

  const bool fused = va.argmax != nullptr;           // uniform
  if (fused) {
    // ---- fused greedy verify, first half. Each lane takes the top two of its
    // tiles in each of its rows into LDS, [wave][lane column j][row]; lane m of
    // each wave then merges row m's 16 columns, and lane m of wave 0 the 8
    // waves. The lanes scan in fp32 (top2_scan); a wave with a NaN among its
    // outputs scans again with order keys. Rows m >= M are scanned too (their
    // accumulators hold finite sums of zero activations) and never read.
    constexpr int R16 = 16 * RS;
    constexpr int JS = 3 * R16 + 1;                    // dwords per (wave, j) line
    static_assert(NW * 16 * JS * 4 + NW * R16 * 12 <= rows_lds_bytes<RS, KT, KCP, HV>(),
                  "the candidates fit in the kernel's LDS");
    __syncthreads();                                   // every wave is past its last LDS read
    unsigned* cand = reinterpret_cast<unsigned*>(lds);
    unsigned* cand2 = cand + NW * 16 * JS;             // [NW][R16] x (k1, i1, k2)
    unsigned* line = cand + (wave * 16 + j) * JS;
    auto put = [&](int m, const Top2& t) {
      line[3 * m] = t.k1;
      line[3 * m + 1] = (unsigned)t.i1;
      line[3 * m + 2] = t.k2;
    };
    // Tile-major, so that each tile's range test is made once (uniform).
    float chk[4] = {0.0f, 0.0f, 0.0f, 0.0f};           // NaN if some output is NaN (or inf - inf)
    Top2Scan sc[RS][4];
#pragma unroll
    for (int r = 0; r < RS; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) sc[r][e] = top2_scan_none();
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      const int col = tile[k] * 16 + j;
      if (tin[k] && tile[k] * 16 + 16 <= N) {         // uniform: a whole tile
#pragma unroll
        for (int r = 0; r < RS; ++r)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            chk[e] += acc[k][r][e];
            top2_scan(sc[r][e], acc[k][r][e], col);
          }
      } else if (tin[k] && col < N) {                 // the last, partial tile
#pragma unroll
        for (int r = 0; r < RS; ++r)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            chk[e] += acc[k][r][e];
            top2_scan(sc[r][e], acc[k][r][e], col);
          }
      }
    }
#pragma unroll
    for (int r = 0; r < RS; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) put(16 * r + 4 * h + e, top2_of_scan(sc[r][e]));
    const float chk_all = (chk[0] + chk[1]) + (chk[2] + chk[3]);
    if (__ballot(chk_all != chk_all) != 0) {           // uniform
#pragma unroll
      for (int r = 0; r < RS; ++r)
#pragma unroll 1
        for (int e = 0; e < 4; ++e) {
          Top2 t = top2_none();
#pragma unroll
          for (int k = 0; k < KT; ++k) {
            const int col = tile[k] * 16 + j;
            if (tin[k] && col < N) top2_add(t, acc[k][r][e], col);
          }
          put(16 * r + 4 * h + e, t);
        }
    }
    __syncthreads();
    if (lane < R16) {
      const unsigned* q = cand + wave * 16 * JS + 3 * lane;
      unsigned k1 = q[0], k2 = q[2];
      int i1 = (int)q[1];
#pragma unroll
      for (int jj = 1; jj < 16; ++jj)
        top2_merge_ranked(k1, i1, k2, q[jj * JS], (int)q[jj * JS + 1], q[jj * JS + 2]);
      unsigned* o = cand2 + (wave * R16 + lane) * 3;
      o[0] = k1;
      o[1] = (unsigned)i1;
      o[2] = k2;
    }
    __syncthreads();
    if (wave == 0 && lane < M) {
      const unsigned* q = cand2 + lane * 3;
      unsigned k1 = q[0], k2 = q[2];
      int i1 = (int)q[1];
#pragma unroll
      for (int w = 1; w < NW; ++w)
        top2_merge_ranked(k1, i1, k2, q[w * R16 * 3], (int)q[w * R16 * 3 + 1], q[w * R16 * 3 + 2]);
      va.partials[(size_t)lane * va.pgroups + blockIdx.x] = make_uint4(k1, (unsigned)i1, k2, 0u);
    }
  }

  // ---- results: lane (j, h) holds rows 4h .. 4h+3 of column j of each row set.
  // With the fused verify the logits are stored last, after its barriers,
  // which would otherwise wait for every store to complete.
  if (!fused || y) {
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      const int col = tile[k] * 16 + j;
      if (!tin[k] || col >= N) continue;
#pragma unroll
      for (int r = 0; r < RS; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = 16 * r + 4 * h + e;
          if (m < M) y[(size_t)m * N + col] = acc[k][r][e];
        }
    }
  }
}


constexpr int kRowsKT = 5;
// Group pairs per chunk: even, so that no 128-byte line of a column's codes
// is split between two chunks (with 5, the lines of pairs 4-5 and 14-15 were
// read twice: 305 against 288.5 MB per launch at K = 2560).
constexpr int kRowsKCP = 4;

// Column tiles per work-group of qgemm_w4_rows: an equal share of the CUs.
int rows_tiles_per_group(int N) {
  const int cus = device_cus();
  const int T = (N + 15) / 16;
  return (T + cus - 1) / cus;
}

template <int ACT, int RS>
hipError_t launch_rows(const void* x, const uint8_t* wq, const uint16_t* scales,
                       const uint16_t* biases, float* y, int M, int K, int N, int gs,
                       const VerifyArgs& va, hipStream_t stream) {
  const int lds_bytes = gs < 0 ? rows_lds_bytes<RS, kRowsKT, kRowsKCP, true>()
                              : rows_lds_bytes<RS, kRowsKT, kRowsKCP, false>();
  static_assert(rows_lds_bytes<4, kRowsKT, kRowsKCP, true>() <= kLdsLimit, "LDS budget");
  auto kern = qgemm_w4_rows<ACT, RS, kRowsKT, kRowsKCP, 0>;
  if (gs > 0) kern = qgemm_w4_rows<ACT, RS, kRowsKT, kRowsKCP, 1>;
  if (gs < 0) kern = qgemm_w4_rows<ACT, RS, kRowsKT, kRowsKCP, -1>;
  const hipError_t e = allow_lds(reinterpret_cast<const void*>(kern));
  if (e != hipSuccess) return e;
  const int T = (N + 15) / 16;
  const int tpw = rows_tiles_per_group(N);
  hipLaunchKernelGGL(kern, dim3((T + tpw - 1) / tpw), dim3(512), lds_bytes, stream, x, wq,
                     scales, biases, y, M, K, N, tpw, va);
  return hipGetLastError();
}

// Workers per row set: one work-group per CU (a multiple of 8 with several
// row sets, for the XCD layout).
int wide_workers(int rsets) {
  const int cus = device_cus();
  int w = rsets > 1 ? (cus / rsets) / 8 * 8 : cus;
  return w < 8 ? 8 : w;
}

template <int ACT>
hipError_t launch_wide_any(const void* x, const uint8_t* wq, const uint16_t* scales,
                           const uint16_t* biases, float* y, int M, int K, int N, int gs,
                           const VerifyArgs& va, hipStream_t s) {
  const int rsets = (M + 15) / 16;
  const int workers = wide_workers(rsets);
  const int GP = (K >> 6) >> 1;
  // Group 32 keeps four partial sums per step: only the 4-pair block with a
  // one-block ring stays within 256 registers (qgemm_wide_fits).
  if (gs < 0)
    return launch_wide<ACT, 4, 1>(x, wq, scales, biases, y, M, K, N, rsets, workers, gs, va, s);
  if (GP % 5 == 0)
    return launch_wide<ACT, 5, 1>(x, wq, scales, biases, y, M, K, N, rsets, workers, gs, va, s);
  if (GP % 4 == 0)
    return launch_wide<ACT, 4, 1>(x, wq, scales, biases, y, M, K, N, rsets, workers, gs, va, s);
  if (GP % 2 == 0)
    return launch_wide<ACT, 2, 4>(x, wq, scales, biases, y, M, K, N, rsets, workers, gs, va, s);
  return launch_wide<ACT, 1, 8>(x, wq, scales, biases, y, M, K, N, rsets, workers, gs, va, s);
}

}  // namespace

bool qgemm_rows_fits(int M, int K, int N, int act) {
  // 17..64 rows of 16-bit activations, whole group pairs, 32-bit offsets,
  // and at most kRowsKT tiles per wave with every wave busy.
  if (M <= 16 || M > 64 || act == ACT_FP32 || K % 128 != 0) return false;
  if ((size_t)N * (size_t)(K / 2) >= 0x7F000000u) return false;
  const int tpw = rows_tiles_per_group(N);
  return tpw >= 8 && tpw <= 8 * kRowsKT;
}

int qgemm_rows_groups(int N) {
  const int T = (N + 15) / 16;
  const int tpw = rows_tiles_per_group(N);
  return (T + tpw - 1) / tpw;
}

hipError_t launch_qgemm_rows(const void* x, const uint8_t* wq, const uint16_t* scales,
                             const uint16_t* biases, float* y, int M, int K, int N, int act,
                             int gs, const VerifyArgs& va, hipStream_t s) {
  const int rs = (M + 15) / 16;
  if (act == ACT_BF16) {
    if (rs == 2) return launch_rows<ACT_BF16, 2>(x, wq, scales, biases, y, M, K, N, gs, va, s);
    if (rs == 3) return launch_rows<ACT_BF16, 3>(x, wq, scales, biases, y, M, K, N, gs, va, s);
    return launch_rows<ACT_BF16, 4>(x, wq, scales, biases, y, M, K, N, gs, va, s);
  }
  if (act == ACT_FP16) {
    if (rs == 2) return launch_rows<ACT_FP16, 2>(x, wq, scales, biases, y, M, K, N, gs, va, s);
    if (rs == 3) return launch_rows<ACT_FP16, 3>(x, wq, scales, biases, y, M, K, N, gs, va, s);
    return launch_rows<ACT_FP16, 4>(x, wq, scales, biases, y, M, K, N, gs, va, s);
  }
  return hipErrorInvalidValue;
}

bool qgemm_wide_fits(int M, int K, int N, int act, int gs) {
  // Whole tiles per wave need many of them: at least two per wave.
  const int G = K >> 6;
  const int T = (N + 15) / 16;
  const int rsets = (M + 15) / 16;
  // Group 32 runs the 4-pair block only (launch_wide_any): K/128 a multiple of 4.
  return M <= 64 && act != ACT_FP32 && K <= 64 * 8 * 5 && G % 8 == 0 &&
         (gs >= 0 || (G / 2) % 4 == 0) &&
         (size_t)N * (size_t)(K / 2) < 0x7F000000u && T >= 16 * wide_workers(rsets) &&
         m16_layout(G, 16, 8, 5, gs < 0).sb + 8 * 16 * (gs < 0 ? 2 * G : G) * 4 <= kLdsLimit;
}

int qgemm_wide_workers(int M) { return wide_workers((M + 15) / 16); }

hipError_t launch_qgemm_wide(const void* x, const uint8_t* wq, const uint16_t* scales,
                             const uint16_t* biases, float* y, int M, int K, int N, int act,
                             int gs, const VerifyArgs& va, hipStream_t stream) {
  if (act == ACT_BF16)
    return launch_wide_any<ACT_BF16>(x, wq, scales, biases, y, M, K, N, gs, va, stream);
  if (act == ACT_FP16)
    return launch_wide_any<ACT_FP16>(x, wq, scales, biases, y, M, K, N, gs, va, stream);
  return hipErrorInvalidValue;
}

bool qgemm_m16_fits(int M, int K, int act, int gs) {
  // One batch of staging (K <= 64 * waves * XB) keeps the padded image small.
  return M <= 64 && act != ACT_FP32 && K <= 64 * kM16Waves * kM16XB &&
         m16_layout(K >> 6, 16 * kM16Tiles, kM16Waves, kM16XB, gs < 0).total <= kLdsLimit;
}

bool qgemm_swiglu_fused(int M, int K, int N, int act, int gs) {
  // The fused kernel's weight buffer spans the whole stacked weight from the
  // work-group's first gate row; it must stay below the scalar offset that
  // reads as zero.
  return qgemm_m16_fits(M, K, act, gs) && (size_t)N * (size_t)(K / 2) < 0x7F000000u;
}

int qgemm_m16_workers(int M, int N) { return m16_workers(M, N); }

hipError_t launch_qgemm_m16(const void* x, const uint8_t* wq, const uint16_t* scales,
                            const uint16_t* biases, float* y, int M, int K, int N, int act,
                            int gs, const VerifyArgs& va, hipStream_t stream) {
  if (act == ACT_BF16)
    return launch_m16_blocks<ACT_BF16, false>(x, wq, scales, biases, y, M, K, N, gs, va, stream);
  if (act == ACT_FP16)
    return launch_m16_blocks<ACT_FP16, false>(x, wq, scales, biases, y, M, K, N, gs, va, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_qgemm_swiglu(const void* x, const uint8_t* wq, const uint16_t* scales,
                               const uint16_t* biases, float* h, int M, int K, int N, int act,
                               int gs, float* scratch_y, hipStream_t stream) {
  const VerifyArgs none{};
  if (qgemm_swiglu_fused(M, K, N, act, gs)) {
    if (act == ACT_BF16)
      return launch_m16_blocks<ACT_BF16, true>(x, wq, scales, biases, h, M, K, N, gs, none, stream);
    return launch_m16_blocks<ACT_FP16, true>(x, wq, scales, biases, h, M, K, N, gs, none, stream);
  }
  hipError_t e = launch_qgemm(x, wq, scales, biases, scratch_y, M, K, N, act, gs, none, stream);
  if (e != hipSuccess) return e;
  const long long total = (long long)M * (N / 2);
  const int blocks = (int)((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
  hipLaunchKernelGGL(swiglu_rows, dim3(blocks), dim3(256), 0, stream, scratch_y, h, M, N / 2);
  return hipGetLastError();
}

}  // namespace vqv

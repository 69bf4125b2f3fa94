// The verify projection for one row set (M <= 8) on gfx950: W4 group-64
// codes streamed in whole 128-byte lines.
//
// y[m,n] = sum_g ( s[n,g] * sum_{k in g} x[m,k]*q[n,k] + b[n,g] * sum_{k in g} x[m,k] )
//
// This is the quantized verify projection of a DFlash block ("perf: tune
// DFlash2 M=8 verification for M1 and M2", PR description), each weight byte
// read once for all rows as the row tiles of "dspark: fold first-token
// forward into verify + bit-exact M5 Metal decode wins" (first commit) do.
//
// Arithmetic (exact unpack into the mantissa of c0, the row-split
// v_mfma_f32_16x16x32 layout, the group epilogue y += s*C + (b - c0*s)*xs, the
// fixed-order reductions) is that of qgemm_w4_m8 in qgemm.hip. What differs is
// how the codes reach the MFMA:
//
//  * A unit is one 16-column tile times 128 bytes of each column (a quad: two
//    group pairs, 256 k). It is read by two load instructions, columns 0-7 and
//    8-15 of the tile, eight lanes per column, so every instruction covers
//    eight whole 128-byte lines. Loads that cover half lines (16 columns x 64
//    bytes, the layout the MFMA consumes directly) stream the same bytes
//    markedly slower on this part.
//  * The lane that loads a 16-byte chunk is chosen so that the MFMA operands
//    of the unit's two steps come out of one row shift by eight lanes each:
//    lane (j = lane%16, h = lane/16) of the first load holds column j%8,
//    chunk 4*(j/8) + h, and the second load the same for columns 8-15. Step 0
//    needs column j, chunk h, step 1 column j, chunk 4 + h; so
//      step0 = j < 8 ? first[lane] : second[lane - 8]
//      step1 = j < 8 ? first[lane + 8] : second[lane]
//    which are two DPP moves (row_shr:8 / row_shl:8 with bank masks) per
//    dword.
//  * Weight loads are non-temporal: the stream is read once, and keeping it
//    out of the caches' normal replacement also shortens the boundary to the
//    kernel that follows.
//  * A work-group's units (tile-major) are dealt to its 8 waves as runs of
//    equal length; a run spans at most two tiles, whose partial sums the
//    reduction adds in wave order.
//
// Requirements (the launcher checks them): M <= 8, bf16 or fp16 activations,
// group 64, K a multiple of 256 (whole quads: no unit reads past a row), the
// work-group's activation image within LDS.

#include "argmax.h"
#include "qgemm_common.h"
#include "vqv_internal.h"

namespace vqv {
namespace {

constexpr int kSlotBytes = 16;
constexpr int kTRowBytes = 33 * kSlotBytes;
constexpr int kPairBytes = 4 * kTRowBytes;

// LDS: GP activation images and one zero image (more when the staging rounds
// are padded), the row sums (16 floats per image), the (s, b) table (G + 4
// dwords per column), the partial-sum slots (two 8x16 tiles per wave), then
// each run's first and last tile.
struct Q8Layout {
  int xs, sb, sbs, red, runs, total;
};

__host__ __device__ inline Q8Layout q8_layout(int G, int WGC, int NW, int XB) {
  const int GP = G >> 1;
  const int rounds = (2 * GP + NW - 1) / NW;             // staging rounds per wave
  const int padded = (rounds + XB - 1) / XB * XB * NW;   // groups the staging writes
  const int nimg = GP + 1 > padded / 2 ? GP + 1 : padded / 2;
  Q8Layout L{};
  L.xs = nimg * kPairBytes;
  L.sb = L.xs + nimg * 16 * 4;
  L.sbs = G + 4;
  L.red = L.sb + WGC * L.sbs * 4;
  L.runs = L.red + NW * 2 * 128 * 4;
  L.total = L.runs + NW * 2 * 4;
  return L;
}

template <int ACT, int D, int XB, int AUX, bool FUSED, int GS>
__global__ __launch_bounds__(512) void qgemm_w4_m8q(
    const void* __restrict__ x, const uint8_t* __restrict__ wq,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases,
    float* __restrict__ y, int M, int K, int N, int cols, VerifyArgs va) {
  using TR = ActTraits<ACT>;
  constexpr int NW = 8, NT = 64 * NW, TW = 5, WGC = 16 * TW;
  constexpr int XSF = 16;                           // row sums per activation image
  constexpr int SBU = 2;                            // table units per thread per round
  static_assert(D >= 1, "ring depth");

  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15;
  const int h = lane >> 4;
  const int half = h >> 1;
  const int G = K >> 6;                              // a multiple of 4
  const int GP = G >> 1;
  const int Q = GP >> 1;                             // quads per column
  const unsigned rowbytes = (unsigned)K >> 1;
  const Q8Layout L = q8_layout(G, WGC, NW, XB);
  unsigned char* xl = lds;
  float* xsl = reinterpret_cast<float*>(lds + L.xs);
  unsigned* sbl = reinterpret_cast<unsigned*>(lds + L.sb);
  float* red = reinterpret_cast<float*>(lds + L.red);
  int* run_tiles = reinterpret_cast<int*>(lds + L.runs);

  const int wg0 = blockIdx.x * cols;
  const int wgcols = min(cols, N - wg0);
  const int tiles = (wgcols + 15) >> 4;
  const int units = tiles * Q;
  // SIMD s = wave % 4 takes units [sU/4, (s+1)U/4). Its two waves share
  // the SIMD's issue slots, and the older one (waves 0-3 are dispatched
  // first) wins the arbitration, so it takes 9/16 of them: both then end at
  // about the same time (with equal halves the younger wave ran about 2 us
  // longer at the target shape, with only half the loads in flight).
  const int sq0 = ((wave & 3) * units) >> 2, sq1 = (((wave & 3) + 1) * units) >> 2;
  const int smid = sq0 + (((sq1 - sq0) * 9) >> 4);
  const int u0 = wave < 4 ? sq0 : smid;
  const int nu = (wave < 4 ? smid : sq1) - u0;        // this wave's run
  const int tfirst = u0 / Q;
  const int qfirst = u0 - tfirst * Q;

  unsigned magic;
  asm volatile("v_mov_b32 %0, %1" : "=v"(magic) : "i"(TR::magic));

  // Weights are read through a descriptor per tile: its base is the tile's
  // first column and its size the tile's valid columns (none for loads past
  // a run), so lanes past the columns read zeros by their vector offset
  // alone; the buffer offset carries the quad.
  uint8_t* const wq_wg = const_cast<uint8_t*>(wq) + (size_t)wg0 * rowbytes;
  const int tlast = tiles - 1;
  const unsigned rec_full = 16u * rowbytes;
  const unsigned rec_last = (unsigned)(wgcols - 16 * tlast) * rowbytes;
  // GS = 1 (group 128): one scale and bias per 128-group in memory; the LDS
  // table keeps one entry per 64-group, each 128-group entry in both of its
  // halves, and the per-64-group row sums give b * (xs0 + xs1) = b * xs.
  const int ME = G >> GS;                            // table entries per column in memory
  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(scales) + (size_t)wg0 * ME, (short)0, wgcols * ME * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(biases) + (size_t)wg0 * ME, (short)0, wgcols * ME * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(x), (short)0, M * K * 2, kBufferFlags);

  // Load lanes: column j%8 (+8 for the second load) of the tile, chunk
  // 4*(j/8) + h of the quad. Columns past the work-group's read zeros through
  // an out-of-range vector offset.
  const int lcol = j & 7;
  const unsigned lchunk = 64u * (unsigned)(j >> 3) + 16u * (unsigned)h;
  const unsigned voff_a = (unsigned)lcol * rowbytes + lchunk;
  const unsigned voff_b = voff_a + 8u * rowbytes;
  const bool a_lane = ((j < 8) == (h < 2));
  const int aslot = a_lane ? (h * 8 + (j & 7)) : 32;

  // ---- activation staging (as qgemm_w4_m8): lane (e = lane%8, row =
  // lane/8) of wave w moves the 8 values k = 64g + 8e.. of group g = w + NW*i.
  const int ngrp = 2 * GP;
  const int rounds = (ngrp + NW - 1) / NW;
  const int e8 = lane & 7;
  const int mm = lane >> 3;
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
  const unsigned xl_lane = (e8 & 3) * kTRowBytes + ((e8 >> 2) * 8 + mm) * kSlotBytes;
  auto x_store_round = [&](int bb, int i) {
    const int g = wave + NW * (bb + i);
    const float s8 = sum8_lanes(block_sum<ACT>(xv[i]));
    *reinterpret_cast<u32x4*>(xl + (g >> 1) * kPairBytes + (g & 1) * 16 * kSlotBytes +
                              xl_lane) = permute_pairs(xv[i]);
    xsl[g * 8 + mm] = s8;
  };

  // ---- scale/bias table: units of 8 LDS entries from the work-group's
  // contiguous block (16 bytes of memory, 8 for group 128), or single
  // entries when the arrays are not 16-byte aligned or G % 8 != 0.
  const bool sb_vec = (G % 8) == 0 && ((reinterpret_cast<uintptr_t>(scales) |
                                        reinterpret_cast<uintptr_t>(biases)) & 15) == 0;
  const int sb_units = sb_vec ? wgcols * G / 8 : wgcols * G;
  u32x4 sbs[SBU], sbb[SBU];
  auto sb_load = [&](int round) {
#pragma unroll
    for (int u = 0; u < SBU; ++u) {
      const int i = (round * SBU + u) * NT + tid;
      if (sb_vec) {
        const unsigned off = i < sb_units ? (16u * i) >> GS : kOutOfRange;
        sbs[u] = sb_unit_load<GS>(sr, off);
        sbb[u] = sb_unit_load<GS>(br, off);
      } else {
        const unsigned off = i < sb_units ? 2u * ((unsigned)i >> GS) : kOutOfRange;
        sbs[u].x = __builtin_amdgcn_raw_buffer_load_b16(sr, off, 0, 0);
        sbb[u].x = __builtin_amdgcn_raw_buffer_load_b16(br, off, 0, 0);
      }
    }
  };
  const unsigned g_recip = 0xFFFFFFFFu / (unsigned)G + 1u;
  auto div_g = [&](unsigned e) { return __umulhi(e, g_recip); };
  auto sb_store = [&](int round) {
#pragma unroll
    for (int u = 0; u < SBU; ++u) {
      const int i = (round * SBU + u) * NT + tid;
      const bool ok = i < sb_units;
      if (sb_vec) {
        const unsigned e0 = 8u * (unsigned)i;
        const unsigned n = div_g(e0), g = e0 - n * (unsigned)G;
        u32x4 lo, hi;
        sb_pairs<GS>(sbs[u], sbb[u], lo, hi);
        // Units past the table write into the partial-sum slots (8 KB, not
        // read before the end of the loop).
        const unsigned o = ok ? (unsigned)L.sb + 4u * (n * (unsigned)L.sbs + g)
                              : (unsigned)L.red + 32u * ((unsigned)tid & 255u);
        *reinterpret_cast<u32x4*>(lds + o) = lo;
        *reinterpret_cast<u32x4*>(lds + o + 16) = hi;
      } else if (ok) {
        const unsigned n = div_g((unsigned)i), g = (unsigned)i - n * (unsigned)G;
        sbl[n * L.sbs + g] = (sbs[u].x & 0xFFFFu) | (sbb[u].x << 16);
      }
    }
  };

  // ---- the run's units: unit i of the run (0 <= i < nu) is unit u0 + i of
  // the work-group, tile (u0 + i) / Q, quad (u0 + i) % Q. The loads run D
  // units ahead of the arithmetic; both walk the run with scalar offsets
  // that advance by one quad and jump at a tile's end.
  struct Ring {
    u32x4 a, b;
  };
  Ring ring[D];
  unsigned ld_so = 128u * (unsigned)qfirst;          // quad offset within the tile
  unsigned ld_tile = (unsigned)tfirst * 16u * rowbytes; // tile offset (whole tiles)
  int ld_q = qfirst, ld_t = tfirst, ld_left = nu;
  // The next unit's two loads, then advance.
  auto ring_load = [&](Ring& r) {
    const unsigned rec = ld_left <= 0 ? 0u : ld_t == tlast ? rec_last : rec_full;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(wq_wg + ld_tile, (short)0, rec, kBufferFlags);
    r.a = __builtin_amdgcn_raw_buffer_load_b128(rs, voff_a, ld_so, AUX);
    r.b = __builtin_amdgcn_raw_buffer_load_b128(rs, voff_b, ld_so, AUX);
    const bool wrap = ld_q + 1 == Q;
    ld_so = wrap ? 0u : ld_so + 128u;
    ld_q = wrap ? 0 : ld_q + 1;
    ld_tile = wrap ? ld_tile + 16u * rowbytes : ld_tile;
    ld_t = wrap ? ld_t + 1 : ld_t;
    ld_left -= 1;
  };

  // ---- prologue: the activations and the first table round go out first,
  // then the ring; staging waits on the activations only.
  x_load(0);
  sb_load(0);
#pragma unroll
  for (int d = 0; d < D; ++d) ring_load(ring[d]);
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int i = tid; i < GP * 4; i += NT)
      *reinterpret_cast<u32x4*>(xl + (i >> 2) * kPairBytes + (i & 3) * kTRowBytes +
                                32 * kSlotBytes) = z;
    for (int i = tid; i < kPairBytes / 16; i += NT)
      *reinterpret_cast<u32x4*>(xl + GP * kPairBytes + 16 * i) = z;
    if (tid < XSF) xsl[GP * XSF + tid] = 0.0f;
    for (int i = tid; i < WGC * 4; i += NT) sbl[(i >> 2) * L.sbs + G + (i & 3)] = 0u;
  }
#pragma unroll
  for (int i = 0; i < XB; ++i) x_store_round(0, i);
  sb_store(0);
  for (int bb = XB; bb < rounds; bb += XB) {          // K above 64*NW*XB only
    x_load(bb);
#pragma unroll
    for (int i = 0; i < XB; ++i) x_store_round(bb, i);
  }
  for (int round = 1; round * SBU * NT < sb_units; ++round) {
    sb_load(round);
    sb_store(round);
  }
  if (lane == 0) {
    run_tiles[2 * wave] = nu > 0 ? tfirst : 1 << 30;
    run_tiles[2 * wave + 1] = nu > 0 ? (u0 + nu - 1) / Q : -1;
  }
  __syncthreads();

  // ---- main loop.
  const unsigned char* abase = xl + aslot * kSlotBytes;
  const unsigned* sbbase = sbl + j * L.sbs + half;
  struct Ops { u32x4 A[4]; unsigned sb; };
  // LDS operands of image (group pair) img with the table of the tile at
  // dword offset sbo. Past the run the reads land on images and table rows
  // that exist but are never used.
  auto fetch = [&](int img, int sbo, Ops& o) {
    const unsigned char* a = abase + img * kPairBytes;
#pragma unroll
    for (int t = 0; t < 4; ++t) o.A[t] = *reinterpret_cast<const u32x4*>(a + t * kTRowBytes);
    o.sb = sbbase[sbo + 2 * img];
  };
  // The bias term sum_g (b - c0*s)[n,g] * xs[m,g] of a unit's four groups
  // is one fp32 MFMA (16 x 16 x 4): A = the row sums (rows 8-15 zero), B =
  // (b - c0*s) of the tile's columns; it accumulates per tile in D.
  // A lane (i = lane%16, k = lane/16) reads xs[row i][group 4q + k], a B lane
  // (j, k) the table entry of column j, group 4q + k.
  const float* bxs = xsl + (j < 8 ? 8 * h + j : 16 * GP);  // GP*16: the zero row sums
  const int bxs_step = j < 8 ? 32 : 0;
  const unsigned* bsb = sbl + j * L.sbs + h;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  f32x4 dbias = {0.0f, 0.0f, 0.0f, 0.0f};             // the tile's bias term so far
  int acc_seg = 0;
  // A finished tile's partial sums (the row-split halves added: lane l and
  // lane l + 32 hold the same outputs for the two groups of a pair).
  auto flush = [&](int seg) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[e]),
                                                       __float_as_uint(acc[e]), false, false);
      const float v = acc[e] + __uint_as_float(sw[1]) + dbias[e];
      if (lane < 32) red[((wave * 2 + seg) * 8 + 4 * (lane >> 4) + e) * 16 + j] = v;
      acc[e] = 0.0f;
      dbias[e] = 0.0f;
    }
  };
  auto epilogue = [&](const f32x4& C, const Ops& o) {
    const float sv = half_lo(o.sb);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = fmaf(sv, C[e], acc[e]);
  };
  auto bias = [&](int q, int sbo) {
    const float xa = bxs[bxs_step * q];
    const unsigned e = bsb[sbo + 4 * q];
    const float bb = fmaf(-TR::c0, half_lo(e), half_hi(e));
    dbias = __builtin_amdgcn_mfma_f32_16x16x4f32(xa, bb, dbias, 0, 0, 0);
  };
  auto step = [&](const u32x4& w, const Ops& o) {
    f32x4 C = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < 4; ++t) C = mfma16x16x32<TR::f16>(o.A[t], unpack_codes(w[t], magic), C);
    return C;
  };

  Ops cur, prev;
  f32x4 Cprev = {0.0f, 0.0f, 0.0f, 0.0f};
  prev.sb = 0u;                                       // step -1 adds exactly nothing
  int c_img = 2 * qfirst;                             // image of the unit's first step
  const int sbo_first = tfirst * 16 * L.sbs;
  int c_sbo = sbo_first;                              // table offset of the unit's tile
  fetch(c_img, c_sbo, cur);
  auto run_unit = [&](int r) {
    u32x4 w0, w1;
    exchange(ring[r].a, ring[r].b, w0, w1);
    // Both operands are complete before the refill is issued, so the slot's
    // old values are dead there and the refill can take their registers
    // (otherwise the loop carries a copy that waits for the ring to drain).
    asm volatile("" : "+v"(w0), "+v"(w1) :: "memory");
    ring_load(ring[r]);                               // refill as soon as the slot is read
    const bool wrap = c_img + 2 == 2 * Q;             // the next unit starts a tile
    const int n_img = wrap ? 0 : c_img + 2;
    const int n_sbo = wrap ? c_sbo + 16 * L.sbs : c_sbo;
    // step 0
    f32x4 C = step(w0, cur);
    Ops nxt;
    fetch(c_img + 1, c_sbo, nxt);
    epilogue(Cprev, prev);
    if (c_img == 0 && c_sbo != sbo_first) {           // uniform: the last step ended a tile
      flush(0);
      acc_seg = 1;
    }
    Cprev = C;
    prev = cur;
    cur = nxt;
    // step 1
    C = step(w1, cur);
    bias(c_img >> 1, c_sbo);
    fetch(n_img, n_sbo, nxt);
    epilogue(Cprev, prev);
    Cprev = C;
    prev = cur;
    cur = nxt;
    c_img = n_img;
    c_sbo = n_sbo;
  };
  int i = 0;
  for (; i + D <= nu; i += D) {
#pragma unroll
    for (int r = 0; r < D; ++r) run_unit(r);
  }
#pragma unroll
  for (int r = 0; r < D - 1; ++r)                     // the last nu % D units
    if (i + r < nu) run_unit(r);
  epilogue(Cprev, prev);
  flush(acc_seg);

  // ---- reduce (as qgemm_w4_m8): each output tile adds the flushed partials
  // of the runs that cover it, in wave order.
  __syncthreads();
  int tb[NW], te[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    tb[w] = run_tiles[2 * w];
    te[w] = run_tiles[2 * w + 1];
  }
  Top2 best = top2_none();
  for (int idx = tid; idx < tiles * 128; idx += NT) {
    const int t = idx >> 7;
    const int within = idx & 127;
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

  // ---- fused greedy verify, first half (as qgemm_w4_m8).
  static_assert(NT % 128 == 0 && NW % 2 == 0, "one row per thread in the epilogue");
  top2_best16(best);
  unsigned* cand = reinterpret_cast<unsigned*>(lds);
  if ((lane & 15) == 0) {
    unsigned* p = cand + (wave * 4 + (lane >> 4)) * 3;
    p[0] = best.k1;
    p[1] = (unsigned)best.i1;
    p[2] = best.k2;
  }
  __syncthreads();
  if (wave == 0 && lane < M) {
    Top2 r = top2_none();
    for (int w = lane >> 2; w < NW; w += 2) {
      const unsigned* p = cand + (w * 4 + (lane & 3)) * 3;
      top2_merge(r, p[0], (int)p[1], p[2]);
    }
    va.partials[(size_t)lane * va.pgroups + blockIdx.x] = top2_pack(r);
  }
}

constexpr int kQ8D = 2;       // units in flight per wave
constexpr int kQ8Aux = 2;     // non-temporal weight loads

constexpr int q8_xb(int K) { return K <= 2560 ? 5 : 10; }

template <int ACT, int XB>
hipError_t launch_q8(const void* x, const uint8_t* wq, const uint16_t* scales,
                     const uint16_t* biases, float* y, int M, int K, int N, int cols, int gs,
                     const VerifyArgs& va, hipStream_t stream) {
  const Q8Layout L = q8_layout(K >> 6, 80, 8, XB);
  if (L.total > kLdsLimit) return hipErrorInvalidValue;  // never launched
  auto kern = va.argmax ? qgemm_w4_m8q<ACT, kQ8D, XB, kQ8Aux, true, 0>
                        : qgemm_w4_m8q<ACT, kQ8D, XB, kQ8Aux, false, 0>;
  if (gs == 1)
    kern = va.argmax ? qgemm_w4_m8q<ACT, kQ8D, XB, kQ8Aux, true, 1>
                     : qgemm_w4_m8q<ACT, kQ8D, XB, kQ8Aux, false, 1>;
  if (L.total > 65536) {
    const hipError_t e = allow_lds(reinterpret_cast<const void*>(kern));
    if (e != hipSuccess) return e;
  }
  const dim3 grid((N + cols - 1) / cols);
  hipLaunchKernelGGL(kern, grid, dim3(512), L.total, stream, x, wq, scales, biases, y, M, K, N,
                     cols, va);
  return hipGetLastError();
}

}  // namespace

bool qgemm_m8q_fits(int M, int K, int act, int gs) {
  if (M > 8 || act == ACT_FP32 || (gs != 0 && gs != 1) || K % 256 != 0) return false;
  return q8_layout(K >> 6, 80, 8, q8_xb(K)).total <= kLdsLimit;
}

int qgemm_m8q_cols(int N) {
  const int cus = device_cus();
  const int share = ((N + cus - 1) / cus + 3) / 4 * 4;
  return share < 80 ? share : 80;
}

hipError_t launch_qgemm_m8q(const void* x, const uint8_t* wq, const uint16_t* scales,
                            const uint16_t* biases, float* y, int M, int K, int N, int act,
                            int gs, const VerifyArgs& va, hipStream_t stream) {
  const int cols = qgemm_m8q_cols(N);
  if (act == ACT_BF16) {
    if (q8_xb(K) == 5)
      return launch_q8<ACT_BF16, 5>(x, wq, scales, biases, y, M, K, N, cols, gs, va, stream);
    return launch_q8<ACT_BF16, 10>(x, wq, scales, biases, y, M, K, N, cols, gs, va, stream);
  }
  if (q8_xb(K) == 5)
    return launch_q8<ACT_FP16, 5>(x, wq, scales, biases, y, M, K, N, cols, gs, va, stream);
  return launch_q8<ACT_FP16, 10>(x, wq, scales, biases, y, M, K, N, cols, gs, va, stream);
}

}  // namespace vqv

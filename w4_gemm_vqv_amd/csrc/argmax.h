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

// The float a key stands for (-0 comes back as +0, every NaN as one NaN).
__device__ __forceinline__ float key_value(unsigned k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Real values map to keys >= 0x007FFFFF, so (0, INT_MAX) is "no candidate".
__device__ __forceinline__ void take_better(unsigned& k, int& i, unsigned k2, int i2) {
  if (k2 > k || (k2 == k && i2 < i)) { k = k2; i = i2; }
}

// The best candidate (key k1, lowest index i1) and the best key among all
// other candidates (k2; 0 when there is none). Two tied maxima leave k2 ==
// k1, so the margin is 0.
struct Top2 {
  unsigned k1;
  int i1;
  unsigned k2;
};

__device__ __forceinline__ Top2 top2_none() { return Top2{0u, INT_MAX, 0u}; }

__device__ __forceinline__ void top2_merge(Top2& a, unsigned k1, int i1, unsigned k2) {
  if (k1 > a.k1 || (k1 == a.k1 && i1 < a.i1)) {
    a.k2 = a.k1 > k2 ? a.k1 : k2;
    a.k1 = k1;
    a.i1 = i1;
  } else {
    const unsigned o = k1 > k2 ? k1 : k2;
    a.k2 = a.k2 > o ? a.k2 : o;
  }
}

__device__ __forceinline__ void top2_add(Top2& a, float v, int i) {
  top2_merge(a, order_key(v), i, 0u);
}

// Top-1 minus top-2 in fp32: NaN when the row holds a NaN, +inf with no
// second value, 0 for tied maxima (also two infinities).
__device__ __forceinline__ float top2_margin(const Top2& t) {
  if (t.k1 == 0xFFFFFFFFu) return __uint_as_float(0x7FC00000u);
  if (t.k2 == 0u) return __uint_as_float(0x7F800000u);
  if (t.k1 == t.k2) return 0.0f;
  return key_value(t.k1) - key_value(t.k2);
}

// The Top2 of each group of 16 lanes, in every lane of the group (DPP: swap
// neighbours, swap pairs, mirror 8, mirror 16).
__device__ __forceinline__ void top2_best16(Top2& t) {
#define VQV_TOP2_STEP(ctrl)                                                              \
  {                                                                                      \
    const unsigned k1 = __builtin_amdgcn_update_dpp(0u, t.k1, ctrl, 0xF, 0xF, false);    \
    const int i1 = __builtin_amdgcn_update_dpp(0, t.i1, ctrl, 0xF, 0xF, false);          \
    const unsigned k2 = __builtin_amdgcn_update_dpp(0u, t.k2, ctrl, 0xF, 0xF, false);    \
    top2_merge(t, k1, i1, k2);                                                           \
  }
  VQV_TOP2_STEP(0xB1)
  VQV_TOP2_STEP(0x4E)
  VQV_TOP2_STEP(0x141)
  VQV_TOP2_STEP(0x140)
#undef VQV_TOP2_STEP
}

// The Top2 of the 64 lanes of a wave, uniform.
__device__ __forceinline__ Top2 top2_best64(Top2 t) {
  top2_best16(t);
  Top2 r{(unsigned)__builtin_amdgcn_readlane(t.k1, 0), __builtin_amdgcn_readlane(t.i1, 0),
         (unsigned)__builtin_amdgcn_readlane(t.k2, 0)};
#pragma unroll
  for (int l = 16; l < 64; l += 16)
    top2_merge(r, (unsigned)__builtin_amdgcn_readlane(t.k1, l),
               __builtin_amdgcn_readlane(t.i1, l), (unsigned)__builtin_amdgcn_readlane(t.k2, l));
  return r;
}

// A lane's running top two over values offered in increasing index order,
// compared as fp32 (ties keep the earlier index, -0 ties +0, denormals
// compare exactly: the kernels keep fp32 denormals). b1 is the best number
// and i1 its index (b1 NaN and i1 INT_MAX while no number has been offered),
// b2 the best of the other numbers (NaN while there is none), inan the index
// of the first NaN offered (INT_MAX: none). About half the instructions of
// top2_add per value.
struct Top2Scan {
  float b1, b2;
  int i1, inan;
};

__device__ __forceinline__ Top2Scan top2_scan_none() {
  const float none = __uint_as_float(0x7FC00000u);
  return Top2Scan{none, none, INT_MAX, INT_MAX};
}

// Offer v at index i. `num` says v is not NaN; a caller that knows it passes
// true and leaves inan alone. A NaN value (num false) is not a candidate, but
// it may leave b2 NaN: a row with a NaN has the NaN margin whatever b2 is.
__device__ __forceinline__ void top2_scan(Top2Scan& s, float v, int i, bool num = true) {
  const bool take = num && !(v <= s.b1);       // the first number: b1 is NaN
  const float other = take ? s.b1 : v;
  s.b2 = !(other <= s.b2) ? other : s.b2;      // b2 NaN: none yet
  s.b1 = take ? v : s.b1;
  s.i1 = take ? i : s.i1;
  if (!num) s.inan = min(s.inan, i);
}

// The scan as a Top2. With a NaN the first NaN is the best (key 0xFFFFFFFF)
// and k2 is the best number's key: the exact k2 would be the NaN key when a
// second NaN was offered, but a row holding a NaN has the NaN margin and its
// first NaN as argmax either way.
__device__ __forceinline__ Top2 top2_of_scan(const Top2Scan& s) {
  const unsigned kb = s.i1 == INT_MAX ? 0u : order_key(s.b1);
  if (s.inan != INT_MAX) return Top2{0xFFFFFFFFu, s.inan, kb};
  return Top2{kb, s.i1, s.b2 != s.b2 ? 0u : order_key(s.b2)};
}

// A candidate packed for merging by 64-bit compares: (k1 << 32 | ~i1) puts
// the higher key first and, among equal keys, the lower index.
__device__ __forceinline__ unsigned long long top2_rank(unsigned k1, int i1) {
  return (unsigned long long)k1 << 32 | (unsigned)~i1;
}

// top2_merge of a candidate (k1, i1, k2) into (ak1, ai1, ak2), on ranks.
__device__ __forceinline__ void top2_merge_ranked(unsigned& ak1, int& ai1, unsigned& ak2,
                                                  unsigned k1, int i1, unsigned k2) {
  const bool win = top2_rank(k1, i1) > top2_rank(ak1, ai1);
  const unsigned lose = win ? ak1 : k1;
  ak2 = max(max(ak2, k2), lose);
  ak1 = win ? k1 : ak1;
  ai1 = win ? i1 : ai1;
}

// A partial as stored in a workspace: (k1, i1, k2, unused).
__device__ __forceinline__ uint4 top2_pack(const Top2& t) {
  return make_uint4(t.k1, (unsigned)t.i1, t.k2, 0u);
}
__device__ __forceinline__ void top2_merge(Top2& a, const uint4& p) {
  top2_merge(a, p.x, (int)p.y, p.z);
}

// Accept lengths of the sequences whose rows lanes 0..B*T-1 hold (lane r is
// row r = b*T + i with argmax a and, for i < T-1, draft d fed at row i+1;
// `limit` is the count of valid drafts of the lane's sequence, already
// clamped to 0..T-1). Called by one whole wave, B*T <= 64: the length is the
// number of leading rows whose argmax equals their draft (row `limit` never
// counts, so it ends every sequence's run). Returns, in lane b < B, the
// accept length of sequence b.
__device__ __forceinline__ int accept_lengths_of(int a, int d, int limit, int B, int T) {
  const int lane = threadIdx.x & 63;
  const int i = lane % T;
  const bool hit = lane < B * T && i < limit && a == d;
  const unsigned long long hits = __ballot(hit);
  const int first = (lane < B ? lane : 0) * T;
  return __builtin_ctzll(~(hits >> first));
}

// The draft fed after row `lane` (lane = b*T + i, i < T-1), else -1. Loaded
// whatever the sequence's valid length, so that this load and the length's
// go out together; the walk ignores drafts past the length.
__device__ __forceinline__ int draft_of_row(const int32_t* __restrict__ draft, int B, int T) {
  const int lane = threadIdx.x & 63;
  const int b = lane / T, i = lane - b * T;
  return lane < B * T && i < T - 1 ? draft[(size_t)b * (T - 1) + i] : -1;
}

// Top2 over count partials p[0], p[stride], ... spread over the lanes of a
// wave (lane l takes l, l+64, ...), eight loads in flight per lane. Returns
// the wave-uniform result.
__device__ __forceinline__ Top2 top2_reduce_strided(const uint4* __restrict__ p, int count,
                                                    size_t stride) {
  const int lane = threadIdx.x & 63;
  Top2 t = top2_none();
  for (int c0 = 0; c0 < count; c0 += 64 * 8) {
    uint4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = c0 + lane + 64 * j;
      v[j] = c < count ? p[(size_t)c * stride] : make_uint4(0u, (unsigned)INT_MAX, 0u, 0u);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) top2_merge(t, v[j]);
  }
  return top2_best64(t);
}

// The raw valid-draft count of the sequence of row `lane` (T-1 when
// draft_len is NULL); clamp it with clamp_limit where it is used, so that the
// wait for this load does not stall the loads issued after it.
__device__ __forceinline__ int draft_len_of_row(const int32_t* __restrict__ draft_len, int B,
                                                int T) {
  const int lane = threadIdx.x & 63;
  if (!draft_len || lane >= B * T) return T - 1;
  return draft_len[lane / T];
}

__device__ __forceinline__ int clamp_limit(int v, int T) {
  return v < 0 ? 0 : (v > T - 1 ? T - 1 : v);
}

}  // namespace vqv

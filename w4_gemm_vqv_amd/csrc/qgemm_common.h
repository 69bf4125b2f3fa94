// Helpers shared by the projection kernels (qgemm.hip, qgemm_m16.hip): the
// 16-bit MFMA wrapper, the exact code unpack and the activation permutation
// that matches it, activation sums, and launch sizing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
#include <unordered_map>

#include "vqv_internal.h"

namespace vqv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr unsigned kOutOfRange = 0x80000000u;   // buffer offset that reads as zero
constexpr int kBufferFlags = 0x00020000;        // raw buffer, 32-bit data format

template <int ACT> struct ActTraits;
template <> struct ActTraits<ACT_BF16> {
  static constexpr unsigned magic = 0x43004300u;  // bf16 pair (128, 128)
  static constexpr float c0 = 128.0f;
  static constexpr int esz = 2, parts = 1;
  static constexpr bool f16 = false;
};
template <> struct ActTraits<ACT_FP16> {
  static constexpr unsigned magic = 0x64006400u;  // fp16 pair (1024, 1024)
  static constexpr float c0 = 1024.0f;
  static constexpr int esz = 2, parts = 1;
  static constexpr bool f16 = true;
};
template <> struct ActTraits<ACT_FP32> {           // three bf16 terms per value
  static constexpr unsigned magic = 0x43004300u;
  static constexpr float c0 = 128.0f;
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

__device__ __forceinline__ float half_lo(unsigned v) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(v & 0xFFFFu));
}
__device__ __forceinline__ float half_hi(unsigned v) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(v >> 16));
}

// Sum of the eight 16-bit activations held in one 16-byte block.
template <int ACT>
__device__ __forceinline__ float block_sum(const u32x4& v) {
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const unsigned w = v[e];  // a scalar copy: bit_cast must not see the vector element
    if constexpr (ACT == ACT_FP16)
      s = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w),
                                 __builtin_bit_cast(f16x2, 0x3C003C00u), s, false);
    else
      s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                          __builtin_bit_cast(bf16x2, 0x3F803F80u), s, false);
  }
  return s;
}

// Sum over the four lanes 4i..4i+3 (DPP: swap neighbours, then swap pairs).
__device__ __forceinline__ float sum4_lanes(float s) {
  s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                     0, __builtin_bit_cast(int, s), 0xB1, 0xF, 0xF, false));
  s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                     0, __builtin_bit_cast(int, s), 0x4E, 0xF, 0xF, false));
  return s;
}

// Sum over the eight lanes 8i..8i+7 (DPP: swap neighbours, swap pairs, then
// mirror within the half row).
__device__ __forceinline__ float sum8_lanes(float s) {
  s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                     0, __builtin_bit_cast(int, s), 0xB1, 0xF, 0xF, false));
  s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                     0, __builtin_bit_cast(int, s), 0x4E, 0xF, 0xF, false));
  s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                     0, __builtin_bit_cast(int, s), 0x141, 0xF, 0xF, false));
  return s;
}

// Scales and biases hold one 16-bit entry per group of 64 << GS values
// (GS = 0: group 64, GS = 1: group 128; a template parameter of the kernels).
// The kernels' tables are per 64-group: a 128-group's entry serves both of
// its 64-groups, and the per-64-group row sums make the bias term
// b * (xs0 + xs1) come out as b * xs of the 128-group. GS = -1 (group 32)
// keeps one LDS entry per 32-group, twice the entries per column, takes the
// group-64 forms below, and the kernels apply each entry to its own 32-k
// half of a 64-k step.
// A table unit covers 8 consecutive 64-groups of one column (K/64 a multiple
// of 8). sb_unit_load reads one unit's entries from byte offset `off` of an
// array: 16 bytes for group 64, or the 4 entries of group 128 (8 bytes,
// 8-byte aligned) in .x and .y. sb_pairs then forms the unit's 8 LDS words
// (s_g | b_g << 16) for g = 0..3 (lo) and 4..7 (hi), each 128-group entry
// serving two consecutive words. The shuffles sit where the words are
// stored, so the loads need not complete before later loads are issued.
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
template <int GS>
__device__ __forceinline__ u32x4 sb_unit_load(__amdgpu_buffer_rsrc_t r, unsigned off) {
  if constexpr (GS <= 0) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  } else {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    return u32x4{v.x, v.y, 0u, 0u};
  }
}

template <int GS>
__device__ __forceinline__ void sb_pairs(const u32x4& s, const u32x4& b, u32x4& lo, u32x4& hi) {
  if constexpr (GS <= 0) {
    lo.x = __builtin_amdgcn_perm(b.x, s.x, 0x05040100u);
    lo.y = __builtin_amdgcn_perm(b.x, s.x, 0x07060302u);
    lo.z = __builtin_amdgcn_perm(b.y, s.y, 0x05040100u);
    lo.w = __builtin_amdgcn_perm(b.y, s.y, 0x07060302u);
    hi.x = __builtin_amdgcn_perm(b.z, s.z, 0x05040100u);
    hi.y = __builtin_amdgcn_perm(b.z, s.z, 0x07060302u);
    hi.z = __builtin_amdgcn_perm(b.w, s.w, 0x05040100u);
    hi.w = __builtin_amdgcn_perm(b.w, s.w, 0x07060302u);
  } else {
    lo.x = lo.y = __builtin_amdgcn_perm(b.x, s.x, 0x05040100u);
    lo.z = lo.w = __builtin_amdgcn_perm(b.x, s.x, 0x07060302u);
    hi.x = hi.y = __builtin_amdgcn_perm(b.y, s.y, 0x05040100u);
    hi.z = hi.w = __builtin_amdgcn_perm(b.y, s.y, 0x07060302u);
  }
}

constexpr int kLdsLimit = 160 * 1024;
constexpr int kMaxDevices = 64;

// The launchers' two per-device facts, looked up once per device (or per
// kernel and device) and kept for the life of the process: the CU count that
// sizes the grids, and the dynamic LDS limit a kernel may launch with.
inline int current_device() {
  int dev = 0;
  return hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices ? dev : -1;
}

inline int device_cus() {
  static std::atomic<int> known[kMaxDevices];
  const int dev = current_device();
  if (dev < 0) return 256;
  int cus = known[dev].load(std::memory_order_relaxed);
  if (cus > 0) return cus;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return 256;
  known[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Lets `kern` launch with up to kLdsLimit bytes of dynamic LDS on the current
// device (hipFuncSetAttribute once per kernel and device).
inline hipError_t allow_lds(const void* kern) {
  static std::mutex mu;
  static std::unordered_map<const void*, unsigned long long> done;  // device bits
  const int dev = current_device();
  const unsigned long long bit = 1ull << (dev < 0 ? kMaxDevices - 1 : dev);
  {
    std::lock_guard<std::mutex> lock(mu);
    const auto it = done.find(kern);
    if (dev >= 0 && it != done.end() && (it->second & bit)) return hipSuccess;
  }
  const hipError_t e =
      hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsLimit);
  if (e == hipSuccess && dev >= 0) {
    std::lock_guard<std::mutex> lock(mu);
    done[kern] |= bit;
  }
  return e;
}

// Whole-line weight units. A unit is one 16-column tile times 128 bytes of
// each column (two group pairs), read by two 16-byte loads per lane: load a
// covers columns 0-7, load b columns 8-15, lane (j = lane%16, h = lane/16)
// of each taking column j%8 (+8 for b), chunk 4*(j/8) + h of the 128 bytes,
// so every load instruction covers eight whole 128-byte lines. exchange()
// turns the pair into the MFMA operands of the unit's two steps: lane (j, h)
// of s0 holds column j, 16-byte chunk h of the first group pair, and of s1
// the same of the second:
//   s0 = j < 8 ? a[lane] : b[lane - 8],  s1 = j < 8 ? a[lane + 8] : b[lane],
// one v_cndmask_b32 with a row-shifted DPP source per dword (VCC holds the
// lanes that keep their own value). The row shifts write every lane, so no
// result is tied to a load register, which can be refilled as soon as this
// has run. The leading s_nop covers a VALU write of a or b just before (two
// wait states before a DPP read).
__device__ __forceinline__ void exchange(const u32x4& a, const u32x4& b, u32x4& s0, u32x4& s1) {
  asm volatile(
      "s_nop 1\n\t"
      "s_mov_b32 vcc_lo, 0x00ff00ff\n\t"
      "s_mov_b32 vcc_hi, 0x00ff00ff\n\t"
      "v_cndmask_b32_dpp %0, %8, %12, vcc row_shr:8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_cndmask_b32_dpp %1, %9, %13, vcc row_shr:8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_cndmask_b32_dpp %2, %10, %14, vcc row_shr:8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_cndmask_b32_dpp %3, %11, %15, vcc row_shr:8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "s_mov_b32 vcc_lo, 0xff00ff00\n\t"
      "s_mov_b32 vcc_hi, 0xff00ff00\n\t"
      "v_cndmask_b32_dpp %4, %12, %8, vcc row_shl:8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_cndmask_b32_dpp %5, %13, %9, vcc row_shl:8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_cndmask_b32_dpp %6, %14, %10, vcc row_shl:8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_cndmask_b32_dpp %7, %15, %11, vcc row_shl:8 row_mask:0xf bank_mask:0xf bound_ctrl:1"
      : "=&v"(s0.x), "=&v"(s0.y), "=&v"(s0.z), "=&v"(s0.w), "=&v"(s1.x), "=&v"(s1.y),
        "=&v"(s1.z), "=&v"(s1.w)
      : "v"(b.x), "v"(b.y), "v"(b.z), "v"(b.w), "v"(a.x), "v"(a.y), "v"(a.z), "v"(a.w)
      : "vcc");
}

}  // namespace vqv

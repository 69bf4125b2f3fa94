// C-ABI entry points of libvqv: argument checks on the host, then one launch
// sequence on the caller's stream. Nothing is allocated or kept between calls.

#include <stdint.h>

#include <atomic>

#include "../../include/vqv.h"
#include "vqv_internal.h"

namespace {

constexpr int kGroup = 64;
constexpr int kMaxRows = 64;
constexpr int kMaxBlock = 64;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return na && nb && a0 < b0 + nb && b0 < a0 + na;
}

int act_size(vqv_dtype a) { return a == VQV_FP32 ? 4 : 2; }

// Group shift of a supported group size: 0 for 64, 1 for 128 (64 << gs values
// per scale), -1 for 32; kNoGroup for any other size.
constexpr int kNoGroup = 99;
int group_shift(int group) {
  return group == 64 ? 0 : group == 128 ? 1 : group == 32 ? -1 : kNoGroup;
}

}  // namespace

extern "C" {

int vqv_abi_version(void) { return VQV_ABI_VERSION; }

const char* vqv_status_string(vqv_status s) {
  switch (s) {
    case VQV_OK: return "ok";
    case VQV_ERR_ARG: return "invalid argument (null pointer, size out of range or aliasing)";
    case VQV_ERR_UNSUPPORTED: return "unsupported request (e.g. group size other than 32, 64 or 128)";
    case VQV_ERR_ALIGN: return "pointer alignment requirement not met";
    case VQV_ERR_WORKSPACE: return "workspace missing or too small";
    case VQV_ERR_HIP: return "HIP runtime error at launch";
  }
  return "unknown status";
}

const char* vqv_qgemm_kernel(int M, int K, int N, int group, vqv_dtype act_dtype) {
  const int gs = group_shift(group);
  if (M < 1 || M > kMaxRows || N < 1 || K < kGroup || gs == kNoGroup || K % group ||
      K % kGroup || K > (gs < 0 ? vqv::kMaxK32 : vqv::kMaxK))
    return nullptr;
  if (act_dtype != VQV_BF16 && act_dtype != VQV_FP16 && act_dtype != VQV_FP32) return nullptr;
  return vqv::qgemm_kernel_name(M, K, N, (int)act_dtype, gs);
}

size_t vqv_qgemm_workspace_bytes(int M, int K, int N, int group, vqv_dtype act_dtype) {
  (void)M; (void)K; (void)N; (void)group; (void)act_dtype;
  return 0;  // partial sums are reduced on chip
}

vqv_status vqv_qgemm(const void* x, const uint8_t* wq, const uint16_t* scales,
                     const uint16_t* biases, float* y, int M, int K, int N, int group,
                     vqv_dtype act_dtype, void* workspace, size_t workspace_bytes,
                     void* hip_stream) {
  (void)workspace;
  if (!x || !wq || !scales || !biases || !y) return VQV_ERR_ARG;
  if (act_dtype != VQV_BF16 && act_dtype != VQV_FP16 && act_dtype != VQV_FP32)
    return VQV_ERR_ARG;
  if (M < 1 || M > kMaxRows || N < 1 || K < kGroup) return VQV_ERR_ARG;
  const int gs = group_shift(group);
  if (gs == kNoGroup) return VQV_ERR_UNSUPPORTED;
  if (K % group) return VQV_ERR_ARG;
  if (K % kGroup) return VQV_ERR_UNSUPPORTED;  // group 32 with an odd count of 32-groups
  if (K > (gs < 0 ? vqv::kMaxK32 : vqv::kMaxK)) return VQV_ERR_UNSUPPORTED;
  const size_t esz = (size_t)act_size(act_dtype);
  const size_t xbytes = (size_t)M * K * esz;
  const size_t wbytes = (size_t)N * (K / 2);
  const size_t sbytes = (size_t)N * (K / group) * 2;
  const size_t ybytes = (size_t)M * N * 4;
  if (xbytes >= (1ull << 31) || wbytes >= (1ull << 32) || (size_t)N * (K / kGroup) >= (1ull << 31))
    return VQV_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(wq, 16) || !aligned(scales, 2) || !aligned(biases, 2) ||
      !aligned(y, 4))
    return VQV_ERR_ALIGN;
  if (overlaps(y, ybytes, x, xbytes) || overlaps(y, ybytes, wq, wbytes) ||
      overlaps(y, ybytes, scales, sbytes) || overlaps(y, ybytes, biases, sbytes))
    return VQV_ERR_ARG;
  if (workspace_bytes < vqv_qgemm_workspace_bytes(M, K, N, group, act_dtype))
    return VQV_ERR_WORKSPACE;
  if (!vqv::qgemm_supported(M, K, N, (int)act_dtype, gs)) return VQV_ERR_UNSUPPORTED;
  (void)hipGetLastError();  // start from a clean error state
  const vqv::VerifyArgs plain{};
  const hipError_t e = vqv::launch_qgemm(x, wq, scales, biases, y, M, K, N, (int)act_dtype, gs,
                                         plain, static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? VQV_OK : VQV_ERR_HIP;
}

// Fused projection + verify: a 256-byte head (unused), then the projection's
// per-row partials, [M][groups] 16-byte slots.
constexpr size_t kHead = 256;

static size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

size_t vqv_qgemm_verify_workspace_bytes(int M, int K, int N, int group, vqv_dtype act_dtype) {
  const int gs = group_shift(group);
  if (M < 1 || M > kMaxRows || N < 1 || K < kGroup || gs == kNoGroup) return 0;
  if (act_dtype != VQV_BF16 && act_dtype != VQV_FP16 && act_dtype != VQV_FP32) return 0;
  const int groups = vqv::qgemm_verify_groups(M, K, N, (int)act_dtype, gs);
  return groups > 0 ? kHead + (size_t)M * groups * 16 : 0;
}

vqv_status vqv_qgemm_verify(const void* x, const uint8_t* wq, const uint16_t* scales,
                            const uint16_t* biases, float* y, int M, int K, int N, int group,
                            vqv_dtype act_dtype, const int32_t* draft, int B, int T,
                            int32_t* argmax, int32_t* accept_len, void* workspace,
                            size_t workspace_bytes, void* hip_stream) {
  return vqv_qgemm_verify_ex(x, wq, scales, biases, y, M, K, N, group, act_dtype, draft,
                             nullptr, B, T, argmax, accept_len, nullptr, workspace,
                             workspace_bytes, hip_stream);
}

}  // extern "C"

namespace {

// Everything vqv_qgemm_verify_ex checks except the workspace; fills the sizes
// the workspace and overlap checks use.
struct FusedSizes {
  size_t xbytes, wbytes, sbytes, ybytes;
  int gs;
};

vqv_status check_qgemm_verify(const void* x, const uint8_t* wq, const uint16_t* scales,
                              const uint16_t* biases, const float* y, int M, int K, int N,
                              int group, vqv_dtype act_dtype, const int32_t* draft,
                              const int32_t* draft_len, int B, int T, const int32_t* argmax,
                              const int32_t* accept_len, const float* margin, FusedSizes* fs) {
  if (!x || !wq || !scales || !biases || !argmax || !accept_len) return VQV_ERR_ARG;
  if (act_dtype != VQV_BF16 && act_dtype != VQV_FP16 && act_dtype != VQV_FP32)
    return VQV_ERR_ARG;
  if (M < 1 || M > kMaxRows || N < 1 || K < kGroup) return VQV_ERR_ARG;
  if (B < 1 || T < 1 || T > kMaxBlock || (long long)B * T != M) return VQV_ERR_ARG;
  if (T > 1 && !draft) return VQV_ERR_ARG;
  const int gs = group_shift(group);
  if (gs == kNoGroup) return VQV_ERR_UNSUPPORTED;
  if (K % group) return VQV_ERR_ARG;
  if (K % kGroup) return VQV_ERR_UNSUPPORTED;  // group 32 with an odd count of 32-groups
  if (K > (gs < 0 ? vqv::kMaxK32 : vqv::kMaxK)) return VQV_ERR_UNSUPPORTED;
  const size_t esz = (size_t)act_size(act_dtype);
  fs->xbytes = (size_t)M * K * esz;
  fs->wbytes = (size_t)N * (K / 2);
  fs->sbytes = (size_t)N * (K / group) * 2;
  fs->ybytes = (size_t)M * N * 4;
  fs->gs = gs;
  if (fs->xbytes >= (1ull << 31) || fs->wbytes >= (1ull << 32) ||
      (size_t)N * (K / kGroup) >= (1ull << 31) || fs->ybytes >= (1ull << 31))
    return VQV_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(wq, 16) || !aligned(scales, 2) || !aligned(biases, 2) ||
      (y && !aligned(y, 16)) || !aligned(argmax, 4) || !aligned(accept_len, 4) ||
      (draft && !aligned(draft, 4)) || (draft_len && !aligned(draft_len, 4)) ||
      (margin && !aligned(margin, 4)))
    return VQV_ERR_ALIGN;
  const void* ins[6] = {x, wq, scales, biases, draft, draft_len};
  const size_t insz[6] = {fs->xbytes, fs->wbytes, fs->sbytes, fs->sbytes,
                          draft ? (size_t)B * (T - 1) * 4 : 0, draft_len ? (size_t)B * 4 : 0};
  const void* outs[4] = {y, argmax, accept_len, margin};
  const size_t outsz[4] = {y ? fs->ybytes : 0, (size_t)M * 4, (size_t)B * 4,
                           margin ? (size_t)M * 4 : 0};
  for (int o = 0; o < 4; ++o) {
    for (int i = 0; i < 6; ++i)
      if (overlaps(outs[o], outsz[o], ins[i], insz[i])) return VQV_ERR_ARG;
    for (int o2 = o + 1; o2 < 4; ++o2)
      if (overlaps(outs[o], outsz[o], outs[o2], outsz[o2])) return VQV_ERR_ARG;
  }
  return VQV_OK;
}

// The launch sequence of a checked call whose scratch (the partials, at
// ws + kHead) holds M * groups slots.
vqv_status launch_qgemm_verify_at(const void* x, const uint8_t* wq, const uint16_t* scales,
                                  const uint16_t* biases, float* y, int M, int K, int N, int gs,
                                  vqv_dtype act_dtype, const int32_t* draft,
                                  const int32_t* draft_len, int B, int T, int32_t* argmax,
                                  int32_t* accept_len, float* margin, unsigned char* ws,
                                  hipStream_t st) {
  (void)hipGetLastError();
  const vqv::VerifyArgs va{draft, draft_len, B, T, argmax, accept_len, margin,
                           reinterpret_cast<uint4*>(ws + kHead), 0};
  const hipError_t e =
      vqv::launch_qgemm_verify(x, wq, scales, biases, y, M, K, N, (int)act_dtype, gs, va, st);
  return e == hipSuccess ? VQV_OK : VQV_ERR_HIP;
}

// The scratch of vqv_qgemm_verify_ex_noalloc: one array per GPU, held until
// the process ends. Host code uses it only through the address
// hipGetSymbolAddress returns for the current device, kept per device.
constexpr int kMaxDevices = 64;
std::atomic<unsigned char*> g_scratch[kMaxDevices];

}  // namespace

static __device__ __align__(256) unsigned char scratch[VQV_NOALLOC_SCRATCH_BYTES];

namespace {

// The address of `scratch` on the current device, looked up on the first call
// on that device (concurrent first calls look it up twice, harmlessly).
hipError_t scratch_of_current_device(unsigned char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  unsigned char* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    void* q = nullptr;
    e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    p = static_cast<unsigned char*>(q);
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" {

vqv_status vqv_qgemm_verify_ex(const void* x, const uint8_t* wq, const uint16_t* scales,
                               const uint16_t* biases, float* y, int M, int K, int N, int group,
                               vqv_dtype act_dtype, const int32_t* draft,
                               const int32_t* draft_len, int B, int T, int32_t* argmax,
                               int32_t* accept_len, float* margin, void* workspace,
                               size_t workspace_bytes, void* hip_stream) {
  FusedSizes fs;
  const vqv_status st = check_qgemm_verify(x, wq, scales, biases, y, M, K, N, group, act_dtype,
                                           draft, draft_len, B, T, argmax, accept_len, margin, &fs);
  if (st != VQV_OK) return st;
  const size_t need = vqv_qgemm_verify_workspace_bytes(M, K, N, group, act_dtype);
  if (need == 0) return VQV_ERR_UNSUPPORTED;  // no kernel takes the problem
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return VQV_ERR_WORKSPACE;
  const void* ins[6] = {x, wq, scales, biases, draft, draft_len};
  const size_t insz[6] = {fs.xbytes, fs.wbytes, fs.sbytes, fs.sbytes,
                          draft ? (size_t)B * (T - 1) * 4 : 0, draft_len ? (size_t)B * 4 : 0};
  const void* outs[4] = {y, argmax, accept_len, margin};
  const size_t outsz[4] = {y ? fs.ybytes : 0, (size_t)M * 4, (size_t)B * 4,
                           margin ? (size_t)M * 4 : 0};
  for (int i = 0; i < 6; ++i)
    if (overlaps(workspace, need, ins[i], insz[i])) return VQV_ERR_ARG;
  for (int o = 0; o < 4; ++o)
    if (overlaps(workspace, need, outs[o], outsz[o])) return VQV_ERR_ARG;
  return launch_qgemm_verify_at(x, wq, scales, biases, y, M, K, N, fs.gs, act_dtype, draft,
                                draft_len, B, T, argmax, accept_len, margin,
                                static_cast<unsigned char*>(workspace),
                                static_cast<hipStream_t>(hip_stream));
}

vqv_status vqv_qgemm_verify_ex_noalloc(const void* x, const uint8_t* wq, const uint16_t* scales,
                                       const uint16_t* biases, float* y, int M, int K, int N,
                                       int group, vqv_dtype act_dtype, const int32_t* draft,
                                       const int32_t* draft_len, int B, int T, int32_t* argmax,
                                       int32_t* accept_len, float* margin, void* hip_stream) {
  FusedSizes fs;
  const vqv_status st = check_qgemm_verify(x, wq, scales, biases, y, M, K, N, group, act_dtype,
                                           draft, draft_len, B, T, argmax, accept_len, margin, &fs);
  if (st != VQV_OK) return st;
  const size_t need = vqv_qgemm_verify_workspace_bytes(M, K, N, group, act_dtype);
  if (need == 0) return VQV_ERR_UNSUPPORTED;  // no kernel takes the problem
  if (need > VQV_NOALLOC_SCRATCH_BYTES) return VQV_ERR_WORKSPACE;
  unsigned char* ws = nullptr;
  if (scratch_of_current_device(&ws) != hipSuccess) return VQV_ERR_HIP;
  return launch_qgemm_verify_at(x, wq, scales, biases, y, M, K, N, fs.gs, act_dtype, draft,
                                draft_len, B, T, argmax, accept_len, margin, ws,
                                static_cast<hipStream_t>(hip_stream));
}

size_t vqv_qgemm_swiglu_workspace_bytes(int M, int K, int N, int group, vqv_dtype act_dtype) {
  const int gs = group_shift(group);
  if (M < 1 || M > kMaxRows || N < 2 || (N & 1) || K < kGroup || gs == kNoGroup) return 0;
  if (vqv::qgemm_swiglu_fused(M, K, N, (int)act_dtype, gs)) return 0;
  return align256((size_t)M * N * 4);  // the stacked gate/up output
}

vqv_status vqv_qgemm_swiglu(const void* x, const uint8_t* wq, const uint16_t* scales,
                            const uint16_t* biases, float* h, int M, int K, int N, int group,
                            vqv_dtype act_dtype, void* workspace, size_t workspace_bytes,
                            void* hip_stream) {
  if (!x || !wq || !scales || !biases || !h) return VQV_ERR_ARG;
  if (act_dtype != VQV_BF16 && act_dtype != VQV_FP16 && act_dtype != VQV_FP32)
    return VQV_ERR_ARG;
  if (M < 1 || M > kMaxRows || N < 2 || (N & 1) || K < kGroup) return VQV_ERR_ARG;
  const int gs = group_shift(group);
  if (gs == kNoGroup) return VQV_ERR_UNSUPPORTED;
  if (K % group) return VQV_ERR_ARG;
  if (K % kGroup) return VQV_ERR_UNSUPPORTED;  // group 32 with an odd count of 32-groups
  if (K > (gs < 0 ? vqv::kMaxK32 : vqv::kMaxK)) return VQV_ERR_UNSUPPORTED;
  const size_t esz = (size_t)act_size(act_dtype);
  const size_t xbytes = (size_t)M * K * esz;
  const size_t wbytes = (size_t)N * (K / 2);
  const size_t sbytes = (size_t)N * (K / group) * 2;
  const size_t hbytes = (size_t)M * (N / 2) * 4;
  if (xbytes >= (1ull << 31) || wbytes >= (1ull << 32) || (size_t)N * (K / kGroup) >= (1ull << 31) ||
      (size_t)M * N * 4 >= (1ull << 31))
    return VQV_ERR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(wq, 16) || !aligned(scales, 2) || !aligned(biases, 2) ||
      !aligned(h, 4))
    return VQV_ERR_ALIGN;
  const size_t need = vqv_qgemm_swiglu_workspace_bytes(M, K, N, group, act_dtype);
  if (need && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
    return VQV_ERR_WORKSPACE;
  const void* ins[4] = {x, wq, scales, biases};
  const size_t insz[4] = {xbytes, wbytes, sbytes, sbytes};
  for (int i = 0; i < 4; ++i) {
    if (overlaps(h, hbytes, ins[i], insz[i])) return VQV_ERR_ARG;
    if (need && overlaps(workspace, need, ins[i], insz[i])) return VQV_ERR_ARG;
  }
  if (need && overlaps(h, hbytes, workspace, need)) return VQV_ERR_ARG;
  if (!vqv::qgemm_swiglu_fused(M, K, N, (int)act_dtype, gs) &&
      !vqv::qgemm_supported(M, K, N, (int)act_dtype, gs))
    return VQV_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  const hipError_t e = vqv::launch_qgemm_swiglu(x, wq, scales, biases, h, M, K, N,
                                                (int)act_dtype, gs, static_cast<float*>(workspace),
                                                static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? VQV_OK : VQV_ERR_HIP;
}

size_t vqv_verify_workspace_bytes(int B, int T, int N) {
  if (B < 1 || T < 1 || N < 1) return 0;
  return (size_t)B * T * vqv::verify_chunks(N) * 16;
}

vqv_status vqv_verify(const float* logits, const int32_t* draft, int B, int T, int N,
                      int32_t* argmax, int32_t* accept_len, void* workspace,
                      size_t workspace_bytes, void* hip_stream) {
  return vqv_verify_ex(logits, draft, nullptr, B, T, N, argmax, accept_len, nullptr, workspace,
                       workspace_bytes, hip_stream);
}

vqv_status vqv_verify_ex(const float* logits, const int32_t* draft, const int32_t* draft_len,
                         int B, int T, int N, int32_t* argmax, int32_t* accept_len,
                         float* margin, void* workspace, size_t workspace_bytes,
                         void* hip_stream) {
  if (!logits || !argmax || !accept_len) return VQV_ERR_ARG;
  if (B < 1 || T < 1 || T > kMaxBlock || N < 1) return VQV_ERR_ARG;
  if (T > 1 && !draft) return VQV_ERR_ARG;
  const size_t rows = (size_t)B * T;
  if (rows * (size_t)N >= (1ull << 31)) return VQV_ERR_ARG;
  if (!aligned(logits, 16) || !aligned(argmax, 4) || !aligned(accept_len, 4) ||
      (draft && !aligned(draft, 4)) || (draft_len && !aligned(draft_len, 4)) ||
      (margin && !aligned(margin, 4)))
    return VQV_ERR_ALIGN;
  const size_t need = vqv_verify_workspace_bytes(B, T, N);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return VQV_ERR_WORKSPACE;
  const void* ins[3] = {logits, draft, draft_len};
  const size_t insz[3] = {rows * N * 4, draft ? (size_t)B * (T - 1) * 4 : 0,
                          draft_len ? (size_t)B * 4 : 0};
  void* outs[4] = {argmax, accept_len, margin, workspace};
  const size_t outsz[4] = {rows * 4, (size_t)B * 4, margin ? rows * 4 : 0, need};
  for (int o = 0; o < 4; ++o) {
    for (int i = 0; i < 3; ++i)
      if (overlaps(outs[o], outsz[o], ins[i], insz[i])) return VQV_ERR_ARG;
    for (int o2 = o + 1; o2 < 4; ++o2)
      if (overlaps(outs[o], outsz[o], outs[o2], outsz[o2])) return VQV_ERR_ARG;
  }
  (void)hipGetLastError();
  const vqv::VerifyArgs va{draft, draft_len, B, T, argmax, accept_len, margin,
                           static_cast<uint4*>(workspace)};
  const hipError_t e = vqv::launch_verify(logits, N, va, static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? VQV_OK : VQV_ERR_HIP;
}

}  // extern "C"

// ssd_verify_noalloc: ssd_verify for callers that cannot allocate device
// memory (code under graph capture, tight serving loops, hosts that forbid
// hipMalloc). Its workspace is a file-scope device array of fixed size,
// one copy per GPU, held until the process ends; the kernels are those of
// ssd_verify.
//
// On the host the array's name is not a device address: its address on the
// current device is looked up once per device (hipGetSymbolAddress) and only
// that pointer is ever handed to kernels. Every call first clears the part
// of the array the call uses with a fill kernel (no memset, so a captured
// graph holds only kernels), so the contents a previous call left behind,
// at any shape, never matter. Calls that overlap on one GPU share the array
// and race.
#include <algorithm>
#include <cstdio>
#include <mutex>

#include "ssd_internal.hpp"

namespace {

constexpr size_t kScratchBytes = size_t(SSD_NOALLOC_SCRATCH_BYTES);
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

void* g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mu;

// Address of this device's copy of the array (looked up once per device,
// with that device current).
hipError_t scratch_on_device(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

// Zero n16 16-byte words at p (grid-stride).
__global__ __launch_bounds__(256) void k_zero16(uint4* p, size_t n16) {
  for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < n16; i += size_t(gridDim.x) * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

extern "C" {

// Defined in ssd_api.cpp: the status message setter shared by every entry point.
int ssd_internal_fail(int code, const char* msg);

SSD_API size_t ssd_noalloc_scratch_bytes(void) { return kScratchBytes; }

SSD_API int ssd_verify_noalloc(const void* target_logits, int64_t target_bstride,
                               const void* draft_logits, int64_t draft_bstride, int dtype,
                               int32_t B, int32_t K, int32_t V, float tau,
                               const int32_t* draft_tokens, const float* u_acc, const float* u_res,
                               const ssd_sigma* sigma,
                               int32_t* accepted, int32_t* out_tokens, float* probs,
                               float* resid_mass, float* row_lse, void* hip_stream) {
  const size_t need = ssd_verify_workspace_size(B, K, V, dtype);
  if (need == 0) {
    // invalid shape or dtype: let ssd_verify report it precisely
    return ssd_verify(target_logits, target_bstride, draft_logits, draft_bstride, dtype, B, K, V, tau,
                      draft_tokens, u_acc, u_res, sigma, accepted, out_tokens, probs, resid_mass, row_lse,
                      nullptr, 0, hip_stream);
  }
  if (need > kScratchBytes) {
    char msg[192];
    snprintf(msg, sizeof(msg), "ssd_verify_noalloc: B=%d K=%d V=%d needs %zu bytes of workspace, above its %zu",
             B, K, V, need, kScratchBytes);
    return ssd_internal_fail(SSD_EINVAL, msg);
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return ssd_internal_fail(SSD_EHIP, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return ssd_internal_fail(SSD_EHIP, "device ordinal out of range");
  void* ws = nullptr;
  if ((e = scratch_on_device(dev, &ws)) != hipSuccess) return ssd_internal_fail(SSD_EHIP, hipGetErrorString(e));
  hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  const size_t n16 = (need + 15) / 16;
  const unsigned grid = unsigned(std::min<size_t>((n16 + 255) / 256, 1024));
  hipLaunchKernelGGL(k_zero16, dim3(grid), dim3(256), 0, st, static_cast<uint4*>(ws), n16);
  if ((e = hipGetLastError()) != hipSuccess) return ssd_internal_fail(SSD_EHIP, hipGetErrorString(e));
  return ssd_verify(target_logits, target_bstride, draft_logits, draft_bstride, dtype, B, K, V, tau, draft_tokens,
                    u_acc, u_res, sigma, accepted, out_tokens, probs, resid_mass, row_lse, ws, kScratchBytes,
                    hip_stream);
}

}  // extern "C"

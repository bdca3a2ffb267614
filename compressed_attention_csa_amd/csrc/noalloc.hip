// csa_attend_noalloc: csa_attend on scratch the library holds itself, for
// callers that cannot allocate (code under graph capture, tight serving loops).
//
// The scratch is one file-scope device array per GPU (static, so every GPU
// that loads the library holds its own copy until the process ends).  Its
// device address is looked up once per device with hipGetSymbolAddress and
// kept; kernels only ever see that address.  The first 2 MiB hold the control
// words (arrival counters) that csa_attend's kernels expect at zero; they are
// cleared by a fill kernel when the device is first set up, and every call
// returns them to zero.  The rest is written before it is read.
#include <hip/hip_runtime.h>

#include <mutex>

#include "csa.h"
#include "kernels.h"

namespace {

constexpr size_t kScratchBytes = size_t(CSA_NOALLOC_SCRATCH_BYTES);
static_assert(kScratchBytes >= csa::kHeaderBytes, "the scratch holds the control header");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device (nullptr: not set up)

__global__ __launch_bounds__(256) void zero_fill(uint4* p, size_t n16) {
  for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < n16; i += size_t(gridDim.x) * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The scratch address of the current device, set up on first use.
csa_status_t device_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return csa::set_error(CSA_E_HIP, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return csa::set_error(CSA_E_UNSUPPORTED, "device index beyond 64");
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return csa::set_error(CSA_E_HIP, e != hipSuccess ? hipGetErrorString(e) : "scratch has no device address");
    // Control words start at zero (a fill kernel, not a memset node).
    const size_t n16 = csa::kHeaderBytes / 16;
    hipLaunchKernelGGL(zero_fill, dim3(512), dim3(256), 0, stream, static_cast<uint4*>(ptr), n16);
    e = hipGetLastError();
    if (e != hipSuccess) return csa::set_error(CSA_E_HIP, hipGetErrorString(e));
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return CSA_OK;
}

}  // namespace

extern "C" csa_status_t csa_attend_noalloc(const void* q, csa_dtype_t dt, const void* k_cmp, const void* v_cmp,
                                           csa_dtype_t kv_dt, const float* k_scale, const float* v_scale,
                                           int64_t N_alloc, int m, const int32_t* idx, int top_k,
                                           const void* k_raw, const void* v_raw, int64_t raw_base, int64_t n_raw,
                                           int B, int64_t T, int H, int d, int64_t t0, int window, float scale,
                                           void* out, csa_dtype_t out_dt, float* lse, csa_stream_t stream) {
  const size_t need = csa_attend_workspace(B, T, H, d, top_k, window);
  if (need > kScratchBytes) {
    char msg[160];
    snprintf(msg, sizeof msg, "this shape needs %zu bytes of scratch; the library's scratch holds %zu", need,
             kScratchBytes);
    return csa::set_error(CSA_E_WORKSPACE, msg);
  }
  // Validate every argument before any HIP call (a placeholder workspace
  // address stands in for the scratch, which is looked up only afterwards).
  void* const placeholder = reinterpret_cast<void*>(uintptr_t(256));
  csa_status_t st = csa::csa_attend_checked(q, dt, k_cmp, v_cmp, kv_dt, k_scale, v_scale, N_alloc, m, idx, top_k,
                                            k_raw, v_raw, raw_base, n_raw, B, T, H, d, t0, window, scale, out,
                                            out_dt, lse, placeholder, kScratchBytes, stream, false);
  if (st != CSA_OK) return st;
  void* ws = nullptr;
  st = device_scratch(reinterpret_cast<hipStream_t>(stream), &ws);
  if (st != CSA_OK) return st;
  return csa::csa_attend_checked(q, dt, k_cmp, v_cmp, kv_dt, k_scale, v_scale, N_alloc, m, idx, top_k, k_raw,
                                 v_raw, raw_base, n_raw, B, T, H, d, t0, window, scale, out, out_dt, lse, ws,
                                 kScratchBytes, stream, true);
}

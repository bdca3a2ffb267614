// Per-kernel timing hook (diagnostics).  While enabled on a thread, each kernel
// that thread enqueues through the library is bracketed by two HIP events on
// the kernel's stream.  csa_profile_report() waits for the events and returns,
// per kernel name, the number of launches and their total time.  Nothing is
// skipped or changed in the work itself; recording costs two event records per
// kernel, so timing runs should not be captured into graphs.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <string>
#include <vector>

#include "csa.h"
#include "kernels.h"

namespace {

struct Rec {
  const char* name;
  hipEvent_t a, b;
};

struct ProfState {
  bool on = false;
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};

thread_local ProfState g_prof;

}  // namespace

namespace csa {

ProfScope::ProfScope(const char* name, hipStream_t s) : name_(name), stream_(s), start_(nullptr) {
  if (!g_prof.on) return;
  hipEvent_t e = g_prof.get();
  if (!e) return;
  if (hipEventRecord(e, stream_) != hipSuccess) {  // not timed; the event goes back
    g_prof.pool.push_back(e);
    return;
  }
  start_ = e;
}

ProfScope::~ProfScope() {
  if (!start_) return;
  hipEvent_t a = reinterpret_cast<hipEvent_t>(start_);
  hipEvent_t stop = g_prof.get();
  if (!stop || hipEventRecord(stop, stream_) != hipSuccess) {  // this launch goes untimed
    g_prof.pool.push_back(a);
    if (stop) g_prof.pool.push_back(stop);
    return;
  }
  g_prof.recs.push_back(Rec{name_, a, stop});
}

}  // namespace csa

namespace {

// Plain streaming read of a buffer (the HBM read ceiling): every workgroup reads
// one contiguous chunk with 16-byte loads, 8 in flight per thread.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ p, size_t n16, uint32_t* sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t lo = size_t(blockIdx.x) * per;
  const size_t hi = lo + per < n16 ? lo + per : n16;
  uint32_t acc = 0;
  size_t i = lo + threadIdx.x;
  for (; i + 7 * 256 < hi; i += 8 * 256) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[i + u * 256];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < hi; i += 256) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;  // keeps the loads; almost never taken
}

// Row gather (the decode attention's access pattern): workgroup g reads rows
// idx[g * per_group + s] of k and v, 256 bytes each, 16 lanes per row, four
// rows of each per 16 lanes in flight.  Indices are staged in LDS first, as
// the attention stages its selection list, and clamped into [0, n_rows).
constexpr int kGatherThreads = 512;
constexpr int kGatherMaxPerGroup = 4096;
__global__ __launch_bounds__(kGatherThreads) void gather_read_kernel(const uint4* __restrict__ k,
                                                                     const uint4* __restrict__ v, int32_t n_rows,
                                                                     const int32_t* __restrict__ idx, int per_group,
                                                                     uint32_t* sink) {
  __shared__ int32_t src[kGatherMaxPerGroup];
  const int tid = threadIdx.x;
  const int32_t* id = idx + int64_t(blockIdx.x) * per_group;
  for (int s = tid; s < per_group; s += kGatherThreads) {
    const int32_t j = id[s];
    src[s] = j < 0 ? 0 : (j >= n_rows ? n_rows - 1 : j);
  }
  __syncthreads();
  constexpr int kSlots = kGatherThreads / 16;  // rows per round of loads
  uint32_t acc = 0;
  for (int s0 = 0; s0 < per_group; s0 += 4 * kSlots) {
    uint4 kv[4], vv[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      int s = s0 + d * kSlots + tid / 16;
      s = s < per_group ? s : per_group - 1;
      const int64_t j = src[s];
      kv[d] = k[j * 16 + (tid & 15)];
      vv[d] = v[j * 16 + (tid & 15)];
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) acc ^= kv[d].x ^ kv[d].w ^ vv[d].y ^ vv[d].z;
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;  // keeps the loads; almost never taken
}

// Fills n16 16-byte words with all-ones (debug builds only).
__global__ __launch_bounds__(256) void poison_kernel(uint4* p, size_t n16) {
  for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < n16; i += size_t(gridDim.x) * 256)
    p[i] = make_uint4(~0u, ~0u, ~0u, ~0u);
}

}  // namespace

namespace csa {

bool log_enabled() {
  static const bool on = [] {
    const char* e = getenv("CSA_LOG");
    return e != nullptr && e[0] != '\0' && e[0] != '0';
  }();
  return on;
}

void log_dispatch(const char* fmt, ...) {
  if (!log_enabled()) return;
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  fprintf(stderr, "[csa] %s\n", buf);
}

hipError_t debug_poison(void* p, size_t n, hipStream_t s) {
  if (!kDebug || p == nullptr || n < 16) return hipSuccess;
  const size_t n16 = n / 16;
  const size_t blocks = n16 / 256 + 1 < 4096 ? n16 / 256 + 1 : 4096;
  hipLaunchKernelGGL(poison_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, static_cast<uint4*>(p), n16);
  return hipGetLastError();
}

void debug_check_failed(const char* cond, const char* file, int line) {
  fprintf(stderr, "[csa] debug check failed: %s (%s:%d)\n", cond, file, line);
}

}  // namespace csa

extern "C" {

int csa_profile_enable(int on) {
  int was = g_prof.on ? 1 : 0;
  g_prof.on = on != 0;
  return was;
}

csa_status_t csa_diag_stream_read(const void* buf, size_t bytes, uint32_t* sink, csa_stream_t stream) {
  if (bytes == 0) return CSA_OK;
  if (buf == nullptr || sink == nullptr) return csa::set_error(CSA_E_NULL, "buf / sink is NULL");
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0 || bytes % 16 != 0)
    return csa::set_error(CSA_E_ALIGN, "buf must be 16-byte aligned and bytes a multiple of 16");
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  csa::ProfScope prof("stream_read", s);
  hipLaunchKernelGGL(stream_read_kernel, dim3(8192), dim3(256), 0, s, static_cast<const uint4*>(buf), bytes / 16,
                     sink);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? CSA_OK : csa::set_error(CSA_E_HIP, hipGetErrorString(e));
}

csa_status_t csa_diag_gather_read(const void* k, const void* v, int64_t n_rows, const int32_t* idx,
                                  int64_t groups, int64_t per_group, uint32_t* sink, csa_stream_t stream) {
  if (k == nullptr || v == nullptr || idx == nullptr || sink == nullptr)
    return csa::set_error(CSA_E_NULL, "k / v / idx / sink is NULL");
  if ((reinterpret_cast<uintptr_t>(k) & 15u) != 0 || (reinterpret_cast<uintptr_t>(v) & 15u) != 0)
    return csa::set_error(CSA_E_ALIGN, "k and v must be 16-byte aligned");
  if (groups < 1 || groups > 65536 || per_group < 1 || per_group > kGatherMaxPerGroup || n_rows < 1 ||
      n_rows >= (int64_t(1) << 31))
    return csa::set_error(CSA_E_SHAPE, "need 1 <= groups <= 65536, 1 <= per_group <= 4096, 1 <= n_rows < 2^31");
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  csa::ProfScope prof("gather_read", s);
  hipLaunchKernelGGL(gather_read_kernel, dim3(unsigned(groups)), dim3(kGatherThreads), 0, s,
                     static_cast<const uint4*>(k), static_cast<const uint4*>(v), int32_t(n_rows), idx,
                     int(per_group), sink);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? CSA_OK : csa::set_error(CSA_E_HIP, hipGetErrorString(e));
}

int csa_profile_report(char* buf, size_t n) {
  std::map<std::string, std::pair<long, double>> agg;
  int status = CSA_OK;
  for (const Rec& r : g_prof.recs) {
    float ms = 0.0f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
      status = CSA_E_HIP;
    auto& v = agg[r.name];
    v.first += 1;
    v.second += ms;
    g_prof.pool.push_back(r.a);
    g_prof.pool.push_back(r.b);
  }
  g_prof.recs.clear();
  std::string out = "{";
  bool first = true;
  for (auto& kv : agg) {
    char item[256];
    snprintf(item, sizeof item, "%s\"%s\": {\"launches\": %ld, \"total_ms\": %.6f}", first ? "" : ", ",
             kv.first.c_str(), kv.second.first, kv.second.second);
    out += item;
    first = false;
  }
  out += "}";
  if (buf && n) snprintf(buf, n, "%s", out.c_str());
  return status == CSA_OK ? int(out.size()) : -1;
}

}  // extern "C"

// Per-kernel timing hook (diagnostics).  While enabled on a thread, each kernel
// that thread enqueues through the library is bracketed by two HIP events on
// the kernel's stream.  csa_profile_report() waits for the events and returns,
// per kernel name, the number of launches and their total time.  Nothing is
// skipped or changed in the work itself; recording costs two event records per
// kernel, so timing runs should not be captured into graphs.
#include <hip/hip_runtime.h>

#include <cstdio>
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

extern "C" {

int csa_profile_enable(int on) {
  int was = g_prof.on ? 1 : 0;
  g_prof.on = on != 0;
  return was;
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

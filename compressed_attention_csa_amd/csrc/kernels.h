// Internal interface between the validated C ABI (api.cpp) and the gfx950 kernels.
// Argument structs carry already-validated values; launchers only enqueue work.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "csa.h"

namespace csa {

// csa_attend's validation and dispatch (api.cpp); with launch = false it only
// validates.  Used by the entry point that brings its own scratch.
csa_status_t csa_attend_checked(const void* q, csa_dtype_t dt, const void* k_cmp, const void* v_cmp,
                                csa_dtype_t kv_dt, const float* k_scale, const float* v_scale,
                                int64_t N_alloc, int m, const int32_t* idx, int top_k, const void* k_raw,
                                const void* v_raw, int64_t raw_base, int64_t n_raw, int B, int64_t T,
                                int H, int d, int64_t t0, int window, float scale, void* out,
                                csa_dtype_t out_dt, float* lse, void* workspace, size_t workspace_bytes,
                                csa_stream_t stream, bool launch);
// Records the thread-local error text of a status (csa_last_error) and returns it.
csa_status_t set_error(csa_status_t s, const char* msg);

// ------------------------------------------------------------------ diagnostics
//
// CSA_LOG=1 in the environment: every launch decision (path, plan, grid) is
// printed to stderr.  Builds with CSA_DEBUG defined (libcsa_debug.so) also fill
// the scratch part of every workspace, and every kernel's LDS, with all-ones
// words (NaN as fp32 and as bf16) before use, so that a read of memory nothing
// wrote shows up in the results, and check the launch plans' invariants on the
// host before every launch (a failed check is reported as CSA_E_HIP with
// hipErrorInvalidValue and launches nothing).
#ifdef CSA_DEBUG
constexpr bool kDebug = true;
#else
constexpr bool kDebug = false;
#endif
bool log_enabled();
void log_dispatch(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
// Debug builds: bytes [0, n) at p set to 0xff, by a fill kernel on s.
hipError_t debug_poison(void* p, size_t n, hipStream_t s);
void debug_check_failed(const char* cond, const char* file, int line);
#define CSA_HOST_CHECK(cond)                                  \
  do {                                                        \
    if (::csa::kDebug && !(cond)) {                           \
      ::csa::debug_check_failed(#cond, __FILE__, __LINE__);   \
      return hipErrorInvalidValue;                            \
    }                                                         \
  } while (0)

// Brackets one kernel launch with HIP events when per-kernel timing is enabled
// (csa_profile_enable); otherwise does nothing.
class ProfScope {
 public:
  ProfScope(const char* name, hipStream_t s);
  ~ProfScope();

 private:
  const char* name_;
  hipStream_t stream_;
  void* start_;
};

struct CompressArgs {
  const void* x;
  bool x_bf16;
  int B;
  int64_t n_raw;
  int d;
  int64_t raw_base;
  const float* logits;  // m + overlap slot logits
  int m;
  int overlap;          // rows of the previous block folded into each entry (0: none)
  int64_t entry_begin, entry_end, N_alloc;
  void* out;
  int out_kind;  // 0 fp32, 1 bf16, 2 e4m3 + scale
  float* out_scale;
  hipStream_t stream;
};
hipError_t launch_compress(const CompressArgs& a);

// State-cache append in one launch: the rows x_new [B, T_new, d] of positions
// t0 .. t0 + T_new - 1 go to rows p % R and p % R + R of the ring a.x
// [B, 2R, d], and entries [a.entry_begin, a.entry_end) are compressed (from
// the ring with a.raw_base / a.n_raw = 2R, or from x_new for positions >= t0).
hipError_t launch_append(const CompressArgs& a, const void* x_new, int64_t t0, int T_new, int64_t R);

// ------------------------------------------------------------------ indexer + top-k

// kKeyE4M3Q8: e4m3 keys and a bf16 query quantised to e4m3 in the kernel (one
// scale per (token, head) row), so the dot products are fp8 x fp8.
enum KeyKind { kKeyF32 = 0, kKeyBF16 = 1, kKeyE4M3 = 2, kKeyE4M3Q8 = 3 };
constexpr bool key_is_e4m3(int kk) { return kk == kKeyE4M3 || kk == kKeyE4M3Q8; }

struct IndexArgs {
  const void* q_idx;  // [B, T, H_I, d_I]
  const float* w;     // [B, T, H_I] or null
  const void* k_idx;  // [B, N_alloc, d_I]
  const float* k_scale;
  int key_kind;
  int B;
  int64_t T;
  int H_I, d_I;
  int64_t N_alloc, t0;
  int m, top_k;
  int32_t* out_idx;
  float* out_score;
  void* ws;
  hipStream_t stream;
  bool bf16_scores;  // rank scores rounded to bf16 (the approximate selector)
};

// Workspace layout shared by every call.  The first kHeaderBytes hold control
// words only (arrival counters, row histograms) at fixed offsets that do not
// depend on the call's shape; every call returns them to zero.  Data regions
// (keys, staging, partial results) start after the header and are always
// written before they are read, so any sequence of calls of any shapes may
// share one workspace that was zero-filled once.
constexpr size_t kHeaderBytes = size_t(2) << 20;
constexpr size_t kAttendCtrlOff = 0;          // 1024 (row, head group) units x 16 B
constexpr int64_t kAttendCtrlUnits = 1024;
constexpr size_t kIndexCtrlOff = 16384;       // 64 rows x 16 B
constexpr int64_t kIndexChunkRows = 64;       // rows per multi-slice launch

// Slicing plan of the general (rows x slices) indexer path; shared by the
// workspace-size query and the launcher so both agree.
// Prefill path (many query rows per sequence): one workgroup per 32 queries.
constexpr int kPrefillQPW = 4;                        // queries per wave
constexpr int kPrefillWaves = 8;                      // waves per workgroup
constexpr int kPrefillQPB = kPrefillWaves * kPrefillQPW;  // queries per workgroup
constexpr int kPrefillStage = 304 * kPrefillQPW;          // LDS staging slots per wave
constexpr int64_t kPrefillMinT = 64;                  // rows per sequence to use it

struct IndexPlan {
  bool prefill;        // streaming top-k path (query-tiled)
  int64_t cap;         // prefill: candidate buffer entries per query
  int64_t rows;        // B * T
  int64_t c_max;       // largest visible-entry count over the rows
  int64_t slice;       // entries per slice (multiple of 256, <= kMaxSlice)
  int64_t slices;      // slices of the longest row
  int64_t chunk_rows;  // rows per launch pair when rows have several slices
  size_t ws_bytes;     // workspace bytes
  // data offsets (after the header); indexed by the row's position in its chunk
  size_t off_cand, off_tau, off_over;
  int64_t cand_row;    // candidate slots per row (rows x slices path)
};
constexpr int64_t kMaxSlice = 4096;
IndexPlan plan_index(int B, int64_t T, int H_I, int d_I, int64_t N_alloc, int top_k, int key_kind);
hipError_t launch_index_topk(const IndexArgs& a, const IndexPlan& p);
bool prefill_path(int64_t T, int H_I, int key_kind);
hipError_t launch_index_prefill(const IndexArgs& a, const IndexPlan& p);

// ------------------------------------------------------------------ attention

struct AttendArgs {
  bool hca;        // dense over heavy entries (no idx)
  bool bf16;       // q / K / V dtype (else fp32)
  const void* q;   // [B, T, H, d]
  const void* k_cmp;
  const void* v_cmp;  // [B, N_alloc, d]
  bool kv8;           // k_cmp / v_cmp hold e4m3 codes with per-entry scales
  const float* k_scale;
  const float* v_scale;  // [B, N_alloc] (kv8 only)
  int64_t N_alloc;
  int m;  // block size for visibility (CSA m or HCA m_heavy)
  const int32_t* idx;
  int top_k;
  const void* k_raw;
  const void* v_raw;  // [B, n_raw, d]
  int64_t raw_base, n_raw;
  int B;
  int64_t T;
  int H, d;
  int64_t t0;
  int window;
  float scale;
  void* out;
  bool out_bf16;
  float* lse;
  void* ws;
  hipStream_t stream;
};

struct AttendPlan {
  int64_t rows;      // B * T
  int64_t groups;    // head groups (bf16: 1, all heads; fp32: groups of 64 heads)
  int64_t slots;     // longest slot list (entries + window)
  int64_t per_split; // slots per split (multiple of the tile)
  int64_t splits;    // splits of the longest row
  int64_t group_stride;  // block ids per head group (rows * splits rounded up to 8)
  size_t ws_bytes;
  size_t off_part, off_ml;  // data offsets (after the header)
};
constexpr int kAttendGroupHeads = 64;
// max_entries: top_k for CSA, N_alloc for HCA.  The bf16 and fp32 kernels split
// the work differently; the workspace query takes the larger of the two.
AttendPlan plan_attend(bool bf16, int B, int64_t T, int H, int d, int64_t max_entries, int window);
int64_t attend_grid(const AttendPlan& p, bool bf16);
hipError_t launch_attend(const AttendArgs& a, const AttendPlan& p);

}  // namespace csa

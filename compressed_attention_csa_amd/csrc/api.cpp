// C ABI of libcsa: argument validation, workspace sizing and kernel dispatch.
// Every check runs before any HIP call, so a rejected call enqueues nothing.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "csa.h"

#include <algorithm>
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

csa_status_t fail(csa_status_t s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

csa_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return CSA_OK;
  return fail(CSA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE(cond, status, ...) \
  do {                             \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

#define REQUIRE_PTR(p) REQUIRE((p) != nullptr, CSA_E_NULL, "%s is NULL", #p)
// A pointer to an array with no elements may be NULL.
#define REQUIRE_PTR_IF(p, nonempty) REQUIRE((p) != nullptr || !(nonempty), CSA_E_NULL, "%s is NULL", #p)
#define REQUIRE_ALIGN(p) REQUIRE(aligned16(p), CSA_E_ALIGN, "%s is not 16-byte aligned", #p)

constexpr int64_t kMaxEntries = int64_t(1) << 22;  // indexer entries per sequence
constexpr int64_t kMaxGrid = (int64_t(1) << 31) - 1;

csa_status_t check_attend_common(const void* q, csa_dtype_t dt, const void* k_cmp,
                                 const void* v_cmp, int64_t N_alloc, int m, const void* k_raw,
                                 const void* v_raw, int64_t raw_base, int64_t n_raw, int B,
                                 int64_t T, int H, int d, int64_t t0, int window, void* out,
                                 csa_dtype_t out_dt, const float* lse) {
  REQUIRE_PTR_IF(q, T > 0);
  REQUIRE_PTR_IF(k_cmp, N_alloc > 0);
  REQUIRE_PTR_IF(v_cmp, N_alloc > 0);
  REQUIRE_PTR_IF(k_raw, n_raw > 0);
  REQUIRE_PTR_IF(v_raw, n_raw > 0);
  REQUIRE_PTR_IF(out, T > 0);
  REQUIRE(dt == CSA_F32 || dt == CSA_BF16, CSA_E_DTYPE, "dt must be CSA_F32 or CSA_BF16");
  REQUIRE(out_dt == CSA_F32 || out_dt == CSA_BF16, CSA_E_DTYPE, "out_dt must be CSA_F32 or CSA_BF16");
  REQUIRE(B >= 1 && B <= 65535, CSA_E_SHAPE, "B=%d out of range [1, 65535]", B);
  REQUIRE(T >= 0, CSA_E_SHAPE, "T=%lld < 0", (long long)T);
  REQUIRE(t0 >= 0, CSA_E_SHAPE, "t0=%lld < 0", (long long)t0);
  REQUIRE(m >= 1, CSA_E_SHAPE, "block size %d < 1", m);
  REQUIRE(N_alloc >= 0, CSA_E_SHAPE, "N_alloc < 0");
  REQUIRE(window >= 0 && window <= 1024, CSA_E_SHAPE, "window=%d out of range [0, 1024]", window);
  REQUIRE(raw_base >= 0 && n_raw >= 0, CSA_E_SHAPE, "raw_base / n_raw must be >= 0");
  if (dt == CSA_BF16) {
    REQUIRE(d == 64 || d == 128, CSA_E_UNSUPPORTED, "bf16 attention needs d in {64, 128}, got %d", d);
    REQUIRE(H >= 16 && H <= 128 && H % 16 == 0, CSA_E_UNSUPPORTED,
            "bf16 attention needs H a multiple of 16 in [16, 128], got %d", H);
  } else {
    REQUIRE(d == 32 || d == 64 || d == 128, CSA_E_UNSUPPORTED, "fp32 attention needs d in {32, 64, 128}, got %d", d);
    REQUIRE(H >= 1 && H <= 32, CSA_E_UNSUPPORTED, "fp32 attention needs 1 <= H <= 32, got %d", H);
  }
  if (window > 0 && T > 0) {
    const int64_t first = t0 - window + 1 > 0 ? t0 - window + 1 : 0;
    const int64_t last = t0 + T - 1;
    REQUIRE(first >= raw_base && last < raw_base + n_raw, CSA_E_SHAPE,
            "window positions [%lld, %lld] not inside raw rows [%lld, %lld)", (long long)first,
            (long long)last, (long long)raw_base, (long long)(raw_base + n_raw));
  }
  REQUIRE_ALIGN(q);
  REQUIRE_ALIGN(k_cmp);
  REQUIRE_ALIGN(v_cmp);
  REQUIRE_ALIGN(k_raw);
  REQUIRE_ALIGN(v_raw);
  REQUIRE_ALIGN(out);
  REQUIRE(lse == nullptr || aligned16(lse), CSA_E_ALIGN, "lse is not 16-byte aligned");
  return CSA_OK;
}

}  // namespace

extern "C" {

int csa_abi_version(void) { return CSA_ABI_VERSION; }

const char* csa_status_string(int s) {
  switch (s) {
    case CSA_OK: return "CSA_OK";
    case CSA_E_NULL: return "CSA_E_NULL";
    case CSA_E_SHAPE: return "CSA_E_SHAPE";
    case CSA_E_DTYPE: return "CSA_E_DTYPE";
    case CSA_E_ALIGN: return "CSA_E_ALIGN";
    case CSA_E_WORKSPACE: return "CSA_E_WORKSPACE";
    case CSA_E_UNSUPPORTED: return "CSA_E_UNSUPPORTED";
    case CSA_E_HIP: return "CSA_E_HIP";
    default: return "CSA_E_UNKNOWN";
  }
}

const char* csa_last_error(void) { return g_last_error.c_str(); }

csa_status_t csa_compress(const void* x, csa_dtype_t x_dt, int B, int64_t n_raw, int d,
                          int64_t raw_base, const float* logits, int m, int overlap,
                          int64_t entry_begin, int64_t entry_end, int64_t N_alloc, void* out,
                          csa_dtype_t out_dt, float* out_scale, csa_stream_t stream) {
  REQUIRE_PTR_IF(x, n_raw > 0);
  REQUIRE_PTR(logits);
  REQUIRE_PTR_IF(out, N_alloc > 0);
  REQUIRE(x_dt == CSA_F32 || x_dt == CSA_BF16, CSA_E_DTYPE, "x_dt must be CSA_F32 or CSA_BF16");
  REQUIRE(out_dt == CSA_F32 || out_dt == CSA_BF16 || out_dt == CSA_FP8_E4M3, CSA_E_DTYPE,
          "unknown out_dt %d", int(out_dt));
  if (out_dt == CSA_FP8_E4M3) REQUIRE_PTR_IF(out_scale, N_alloc > 0);
  else REQUIRE(out_scale == nullptr, CSA_E_DTYPE, "out_scale must be NULL unless out_dt is CSA_FP8_E4M3");
  REQUIRE(B >= 1 && B <= 65535, CSA_E_SHAPE, "B=%d out of range [1, 65535]", B);
  REQUIRE(d >= 8 && d <= 512 && d % 8 == 0, CSA_E_SHAPE, "d=%d must be a multiple of 8 in [8, 512]", d);
  REQUIRE(out_dt != CSA_FP8_E4M3 || (d >= 16 && (d & (d - 1)) == 0), CSA_E_SHAPE,
          "fp8 output needs d a power of two >= 16, got %d", d);
  REQUIRE(m >= 1 && m <= 128, CSA_E_SHAPE, "m=%d out of range [1, 128]", m);
  REQUIRE(overlap >= 0 && m + overlap <= 128, CSA_E_SHAPE, "overlap=%d: need 0 <= overlap and m + overlap <= 128",
          overlap);
  REQUIRE(n_raw >= 0 && raw_base >= 0, CSA_E_SHAPE, "n_raw / raw_base must be >= 0");
  REQUIRE(0 <= entry_begin && entry_begin <= entry_end && entry_end <= N_alloc, CSA_E_SHAPE,
          "need 0 <= entry_begin <= entry_end <= N_alloc");
  if (entry_end > entry_begin) {
    const int64_t first = entry_begin * m - overlap > 0 ? entry_begin * m - overlap : 0;
    REQUIRE(first >= raw_base && entry_end * m <= raw_base + n_raw, CSA_E_SHAPE,
            "the rows of blocks [%lld, %lld) (positions %lld .. %lld) are not inside the raw rows [%lld, %lld)",
            (long long)entry_begin, (long long)entry_end, (long long)first, (long long)(entry_end * m - 1),
            (long long)raw_base, (long long)(raw_base + n_raw));
    REQUIRE((entry_end - entry_begin) / (256 / (d / 8)) < kMaxGrid, CSA_E_SHAPE, "too many entries");
  }
  REQUIRE_ALIGN(x);
  REQUIRE_ALIGN(logits);
  REQUIRE_ALIGN(out);
  REQUIRE(out_scale == nullptr || aligned16(out_scale), CSA_E_ALIGN, "out_scale is not 16-byte aligned");
  csa::CompressArgs a{x,     x_dt == CSA_BF16, B,         n_raw,    d,
                      raw_base, logits, m, overlap, entry_begin, entry_end, N_alloc,
                      out,   out_dt == CSA_F32 ? 0 : (out_dt == CSA_BF16 ? 1 : 2), out_scale,
                      reinterpret_cast<hipStream_t>(stream)};
  return hip_status(csa::launch_compress(a), "compress launch");
}

csa_status_t csa_append(const void* x_new, csa_dtype_t dt, int B, int T_new, int d, int64_t t0,
                        void* ring, int64_t R, const float* logits, int m, int overlap, int64_t N_alloc,
                        void* out, csa_dtype_t out_dt, float* out_scale, csa_stream_t stream) {
  REQUIRE_PTR_IF(x_new, T_new > 0);
  REQUIRE_PTR(ring);
  REQUIRE_PTR(logits);
  REQUIRE_PTR_IF(out, N_alloc > 0);
  REQUIRE(dt == CSA_F32 || dt == CSA_BF16, CSA_E_DTYPE, "dt must be CSA_F32 or CSA_BF16");
  REQUIRE(out_dt == CSA_F32 || out_dt == CSA_BF16 || out_dt == CSA_FP8_E4M3, CSA_E_DTYPE,
          "unknown out_dt %d", int(out_dt));
  if (out_dt == CSA_FP8_E4M3) REQUIRE_PTR_IF(out_scale, N_alloc > 0);
  else REQUIRE(out_scale == nullptr, CSA_E_DTYPE, "out_scale must be NULL unless out_dt is CSA_FP8_E4M3");
  REQUIRE(B >= 1 && B <= 65535, CSA_E_SHAPE, "B=%d out of range [1, 65535]", B);
  REQUIRE(d >= 8 && d <= 512 && d % 8 == 0, CSA_E_SHAPE, "d=%d must be a multiple of 8 in [8, 512]", d);
  REQUIRE(out_dt != CSA_FP8_E4M3 || (d >= 16 && (d & (d - 1)) == 0), CSA_E_SHAPE,
          "fp8 output needs d a power of two >= 16, got %d", d);
  REQUIRE(m >= 1 && m <= 128, CSA_E_SHAPE, "m=%d out of range [1, 128]", m);
  REQUIRE(overlap >= 0 && m + overlap <= 128, CSA_E_SHAPE, "overlap=%d: need 0 <= overlap and m + overlap <= 128",
          overlap);
  REQUIRE(T_new >= 0 && T_new <= 4096, CSA_E_SHAPE, "T_new=%d out of range [0, 4096]", T_new);
  REQUIRE(t0 >= 0 && N_alloc >= 0, CSA_E_SHAPE, "t0 / N_alloc must be >= 0");
  REQUIRE(R >= 1 && R <= (int64_t(1) << 24), CSA_E_SHAPE, "R=%lld out of range [1, 2^24]", (long long)R);
  REQUIRE(R >= int64_t(m) + overlap + T_new - 1, CSA_E_SHAPE,
          "R=%lld must hold a block and the new rows: R >= m + overlap + T_new - 1 = %d", (long long)R,
          m + overlap + T_new - 1);
  REQUIRE_ALIGN(x_new);
  REQUIRE_ALIGN(ring);
  REQUIRE_ALIGN(logits);
  REQUIRE_ALIGN(out);
  REQUIRE(out_scale == nullptr || aligned16(out_scale), CSA_E_ALIGN, "out_scale is not 16-byte aligned");
  if (T_new == 0) return CSA_OK;
  // Blocks completed by the new rows: (j + 1) m - 1 in [t0, t0 + T_new - 1].
  const int64_t j_lo = t0 / m;
  int64_t j_hi = (t0 + T_new) / m;
  if (j_hi > N_alloc) j_hi = N_alloc;
  if (j_hi < j_lo) j_hi = j_lo;
  // Their rows (positions j_lo m - overlap .. , those >= 0) are consecutive
  // ring rows from p_lo % R on.
  const int64_t p_lo = j_lo * m - overlap > 0 ? j_lo * m - overlap : 0;
  csa::CompressArgs a{ring, dt == CSA_BF16, B, 2 * R, d, p_lo - p_lo % R, logits, m, overlap, j_lo, j_hi, N_alloc,
                      out, out_dt == CSA_F32 ? 0 : (out_dt == CSA_BF16 ? 1 : 2), out_scale,
                      reinterpret_cast<hipStream_t>(stream)};
  return hip_status(csa::launch_append(a, x_new, t0, T_new, R), "append launch");
}

size_t csa_index_topk_workspace(int B, int64_t T, int H_I, int d_I, int64_t N_alloc, int top_k,
                                csa_dtype_t k_dt) {
  if (B < 1 || T < 0 || N_alloc < 0) return 0;
  const int kind = k_dt == CSA_F32 ? csa::kKeyF32 : (k_dt == CSA_BF16 ? csa::kKeyBF16 : csa::kKeyE4M3);
  return csa::plan_index(B, T, H_I, d_I, N_alloc, top_k, kind).ws_bytes;
}

static csa_status_t index_topk(const void* q_idx, csa_dtype_t q_dt, const float* w, const void* k_idx,
                               csa_dtype_t k_dt, const float* k_scale, int B, int64_t T, int H_I,
                               int d_I, int64_t N_alloc, int64_t t0, int m, int top_k,
                               int32_t* out_idx, float* out_score, void* workspace,
                               size_t workspace_bytes, csa_stream_t stream, bool bf16_scores,
                               bool fp8_query = false) {
  REQUIRE_PTR_IF(q_idx, T > 0);
  REQUIRE_PTR_IF(k_idx, N_alloc > 0);
  REQUIRE_PTR_IF(out_idx, T > 0 && top_k > 0);
  const bool ok_dt = (q_dt == CSA_F32 && k_dt == CSA_F32) || (q_dt == CSA_BF16 && k_dt == CSA_BF16) ||
                     (q_dt == CSA_BF16 && k_dt == CSA_FP8_E4M3);
  REQUIRE(ok_dt, CSA_E_DTYPE, "unsupported (q_dt, k_dt) = (%d, %d)", int(q_dt), int(k_dt));
  REQUIRE(!fp8_query || (q_dt == CSA_BF16 && k_dt == CSA_FP8_E4M3), CSA_E_DTYPE,
          "the fp8 x fp8 indexer takes (q_dt, k_dt) = (CSA_BF16, CSA_FP8_E4M3)");
  if (k_dt == CSA_FP8_E4M3) REQUIRE_PTR_IF(k_scale, N_alloc > 0);
  else REQUIRE(k_scale == nullptr, CSA_E_DTYPE, "k_scale must be NULL unless k_dt is CSA_FP8_E4M3");
  REQUIRE(B >= 1 && B <= 65535, CSA_E_SHAPE, "B=%d out of range [1, 65535]", B);
  REQUIRE(T >= 0, CSA_E_SHAPE, "T < 0");
  REQUIRE(H_I >= 1 && H_I <= 16, CSA_E_SHAPE, "H_I=%d out of range [1, 16]", H_I);
  REQUIRE(d_I == 32 || d_I == 64, CSA_E_SHAPE, "d_I=%d must be 32 or 64", d_I);
  REQUIRE(N_alloc >= 0 && N_alloc <= kMaxEntries, CSA_E_SHAPE, "N_alloc=%lld out of range [0, 2^22]",
          (long long)N_alloc);
  REQUIRE(t0 >= 0, CSA_E_SHAPE, "t0 < 0");
  REQUIRE(m >= 1, CSA_E_SHAPE, "m < 1");
  REQUIRE(top_k >= 1 && top_k <= 2048, CSA_E_SHAPE, "top_k=%d out of range [1, 2048]", top_k);
  const int kind = k_dt == CSA_F32    ? csa::kKeyF32
                   : k_dt == CSA_BF16 ? csa::kKeyBF16
                   : fp8_query        ? csa::kKeyE4M3Q8
                                      : csa::kKeyE4M3;
  const csa::IndexPlan p = csa::plan_index(B, T, H_I, d_I, N_alloc, top_k, kind);
  REQUIRE(p.prefill ? (T + csa::kPrefillQPB - 1) / csa::kPrefillQPB <= kMaxGrid
                    : p.rows * p.slices <= kMaxGrid, CSA_E_SHAPE, "too many query rows");
  REQUIRE(p.ws_bytes == 0 || workspace != nullptr, CSA_E_WORKSPACE, "workspace is NULL");
  REQUIRE(workspace_bytes >= p.ws_bytes, CSA_E_WORKSPACE, "workspace has %zu bytes, needs %zu",
          workspace_bytes, p.ws_bytes);
  REQUIRE_ALIGN(q_idx);
  REQUIRE_ALIGN(k_idx);
  REQUIRE_ALIGN(out_idx);
  REQUIRE(w == nullptr || aligned16(w), CSA_E_ALIGN, "w is not 16-byte aligned");
  REQUIRE(k_scale == nullptr || aligned16(k_scale), CSA_E_ALIGN, "k_scale is not 16-byte aligned");
  REQUIRE(out_score == nullptr || aligned16(out_score), CSA_E_ALIGN, "out_score is not 16-byte aligned");
  REQUIRE(workspace == nullptr || aligned16(workspace), CSA_E_ALIGN, "workspace is not 16-byte aligned");
  csa::IndexArgs a{q_idx, w, k_idx, k_scale, kind, B, T, H_I, d_I, N_alloc, t0, m, top_k, out_idx, out_score, workspace,
                   reinterpret_cast<hipStream_t>(stream), bf16_scores};
  return hip_status(csa::launch_index_topk(a, p), "index_topk launch");
}

csa_status_t csa_index_topk(const void* q_idx, csa_dtype_t q_dt, const float* w, const void* k_idx,
                            csa_dtype_t k_dt, const float* k_scale, int B, int64_t T, int H_I,
                            int d_I, int64_t N_alloc, int64_t t0, int m, int top_k,
                            int32_t* out_idx, float* out_score, void* workspace,
                            size_t workspace_bytes, csa_stream_t stream) {
  return index_topk(q_idx, q_dt, w, k_idx, k_dt, k_scale, B, T, H_I, d_I, N_alloc, t0, m, top_k,
                    out_idx, out_score, workspace, workspace_bytes, stream, false);
}

csa_status_t csa_index_topk_bf16(const void* q_idx, csa_dtype_t q_dt, const float* w,
                                 const void* k_idx, csa_dtype_t k_dt, const float* k_scale, int B,
                                 int64_t T, int H_I, int d_I, int64_t N_alloc, int64_t t0, int m,
                                 int top_k, int32_t* out_idx, float* out_score, void* workspace,
                                 size_t workspace_bytes, csa_stream_t stream) {
  return index_topk(q_idx, q_dt, w, k_idx, k_dt, k_scale, B, T, H_I, d_I, N_alloc, t0, m, top_k,
                    out_idx, out_score, workspace, workspace_bytes, stream, true);
}

csa_status_t csa_index_topk_fp8(const void* q_idx, const float* w, const void* k_idx, const float* k_scale,
                                int B, int64_t T, int H_I, int d_I, int64_t N_alloc, int64_t t0, int m,
                                int top_k, int32_t* out_idx, float* out_score, void* workspace,
                                size_t workspace_bytes, csa_stream_t stream) {
  return index_topk(q_idx, CSA_BF16, w, k_idx, CSA_FP8_E4M3, k_scale, B, T, H_I, d_I, N_alloc, t0, m, top_k,
                    out_idx, out_score, workspace, workspace_bytes, stream, false, true);
}

size_t csa_attend_workspace(int B, int64_t T, int H, int d, int top_k, int window) {
  if (B < 1 || T < 0 || H < 1 || d < 1 || top_k < 0 || window < 0) return 0;
  return std::max(csa::plan_attend(true, B, T, H, d, top_k, window).ws_bytes,
                  csa::plan_attend(false, B, T, H, d, top_k, window).ws_bytes);
}

size_t hca_attend_workspace(int B, int64_t T, int H, int d, int64_t N_alloc, int m_heavy, int window) {
  (void)m_heavy;
  if (B < 1 || T < 0 || H < 1 || d < 1 || N_alloc < 0 || window < 0) return 0;
  return std::max(csa::plan_attend(true, B, T, H, d, N_alloc, window).ws_bytes,
                  csa::plan_attend(false, B, T, H, d, N_alloc, window).ws_bytes);
}

static csa_status_t attend_impl(bool hca, const void* q, csa_dtype_t dt, const void* k_cmp,
                                const void* v_cmp, csa_dtype_t kv_dt, const float* k_scale,
                                const float* v_scale, int64_t N_alloc, int m, const int32_t* idx,
                                int top_k, const void* k_raw, const void* v_raw, int64_t raw_base,
                                int64_t n_raw, int B, int64_t T, int H, int d, int64_t t0,
                                int window, float scale, void* out, csa_dtype_t out_dt, float* lse,
                                void* workspace, size_t workspace_bytes, csa_stream_t stream,
                                bool launch = true) {
  csa_status_t st = check_attend_common(q, dt, k_cmp, v_cmp, N_alloc, m, k_raw, v_raw, raw_base,
                                        n_raw, B, T, H, d, t0, window, out, out_dt, lse);
  if (st != CSA_OK) return st;
  const bool kv8 = kv_dt == CSA_FP8_E4M3;
  REQUIRE(kv_dt == dt || (kv8 && dt == CSA_BF16), CSA_E_DTYPE,
          "kv_dt must equal dt, or be CSA_FP8_E4M3 with dt == CSA_BF16");
  if (kv8) {
    REQUIRE_PTR_IF(k_scale, N_alloc > 0);
    REQUIRE_PTR_IF(v_scale, N_alloc > 0);
    REQUIRE(aligned16(k_scale) && aligned16(v_scale), CSA_E_ALIGN, "k_scale / v_scale are not 16-byte aligned");
  } else {
    REQUIRE(k_scale == nullptr && v_scale == nullptr, CSA_E_DTYPE,
            "k_scale / v_scale must be NULL unless kv_dt is CSA_FP8_E4M3");
  }
  if (!hca) {
    REQUIRE(top_k >= 0 && top_k <= 2048, CSA_E_SHAPE, "top_k=%d out of range [0, 2048]", top_k);
    REQUIRE(top_k == 0 || T == 0 || idx != nullptr, CSA_E_NULL, "idx is NULL");
    REQUIRE(idx == nullptr || aligned16(idx), CSA_E_ALIGN, "idx is not 16-byte aligned");
  }
  const csa::AttendPlan p =
      csa::plan_attend(dt == CSA_BF16, B, T, H, d, hca ? N_alloc : int64_t(top_k), window);
  REQUIRE(csa::attend_grid(p, dt == CSA_BF16) <= kMaxGrid, CSA_E_SHAPE, "too many query rows");
  REQUIRE(p.ws_bytes == 0 || workspace != nullptr, CSA_E_WORKSPACE, "workspace is NULL");
  REQUIRE(workspace_bytes >= p.ws_bytes, CSA_E_WORKSPACE, "workspace has %zu bytes, needs %zu",
          workspace_bytes, p.ws_bytes);
  REQUIRE(workspace == nullptr || aligned16(workspace), CSA_E_ALIGN, "workspace is not 16-byte aligned");
  if (!launch) return CSA_OK;
  csa::AttendArgs a{hca, dt == CSA_BF16, q, k_cmp, v_cmp, kv8, k_scale, v_scale, N_alloc, m, hca ? nullptr : idx,
                    hca ? 0 : top_k, k_raw, v_raw, raw_base, n_raw, B, T, H, d, t0, window, scale,
                    out, out_dt == CSA_BF16, lse, workspace, reinterpret_cast<hipStream_t>(stream)};
  return hip_status(csa::launch_attend(a, p), hca ? "hca_attend launch" : "csa_attend launch");
}

}  // extern "C"

namespace csa {

csa_status_t csa_attend_checked(const void* q, csa_dtype_t dt, const void* k_cmp, const void* v_cmp,
                                csa_dtype_t kv_dt, const float* k_scale, const float* v_scale,
                                int64_t N_alloc, int m, const int32_t* idx, int top_k, const void* k_raw,
                                const void* v_raw, int64_t raw_base, int64_t n_raw, int B, int64_t T,
                                int H, int d, int64_t t0, int window, float scale, void* out,
                                csa_dtype_t out_dt, float* lse, void* workspace, size_t workspace_bytes,
                                csa_stream_t stream, bool launch) {
  return attend_impl(false, q, dt, k_cmp, v_cmp, kv_dt, k_scale, v_scale, N_alloc, m, idx, top_k, k_raw, v_raw,
                     raw_base, n_raw, B, T, H, d, t0, window, scale, out, out_dt, lse, workspace,
                     workspace_bytes, stream, launch);
}

csa_status_t set_error(csa_status_t s, const char* msg) { return fail(s, "%s", msg); }

}  // namespace csa

extern "C" {

csa_status_t csa_attend(const void* q, csa_dtype_t dt, const void* k_cmp, const void* v_cmp,
                        csa_dtype_t kv_dt, const float* k_scale, const float* v_scale,
                        int64_t N_alloc, int m, const int32_t* idx, int top_k, const void* k_raw,
                        const void* v_raw, int64_t raw_base, int64_t n_raw, int B, int64_t T,
                        int H, int d, int64_t t0, int window, float scale, void* out,
                        csa_dtype_t out_dt, float* lse, void* workspace, size_t workspace_bytes,
                        csa_stream_t stream) {
  return attend_impl(false, q, dt, k_cmp, v_cmp, kv_dt, k_scale, v_scale, N_alloc, m, idx, top_k, k_raw, v_raw, raw_base,
                     n_raw, B, T, H, d, t0, window, scale, out, out_dt, lse, workspace,
                     workspace_bytes, stream);
}

csa_status_t hca_attend(const void* q, csa_dtype_t dt, const void* k_cmp, const void* v_cmp,
                        csa_dtype_t kv_dt, const float* k_scale, const float* v_scale,
                        int64_t N_alloc, int m_heavy, const void* k_raw, const void* v_raw,
                        int64_t raw_base, int64_t n_raw, int B, int64_t T, int H, int d,
                        int64_t t0, int window, float scale, void* out, csa_dtype_t out_dt,
                        float* lse, void* workspace, size_t workspace_bytes, csa_stream_t stream) {
  return attend_impl(true, q, dt, k_cmp, v_cmp, kv_dt, k_scale, v_scale, N_alloc, m_heavy, nullptr, 0, k_raw, v_raw,
                     raw_base, n_raw, B, T, H, d, t0, window, scale, out, out_dt, lse, workspace,
                     workspace_bytes, stream);
}

}  // extern "C"

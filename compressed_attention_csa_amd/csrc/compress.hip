// Block KV compressor (CSA m = 4, HCA m' = 128) for gfx950.
//
// Entry j of a sequence is sum_s alpha_s * x[j*m + s] with alpha = softmax of the
// compressor's per-slot logits (V4 report digest, section 三; "Evolution map",
// section 4).  The m rows of one block are contiguous in memory, so each
// thread streams the same 8-column slice of the m rows of one entry with
// 16-byte (bf16) or 32-byte (fp32) loads: consecutive threads read consecutive
// 16 B of a row, a wave covers whole rows, and every byte is read once.
// Sums are accumulated in fp64 and rounded once to the output type.
// Long blocks (HCA, m' = 128) are also split over slots: P groups of threads
// each sum about 8 of the entry's slots and the P partial sums are added in
// group order through LDS, so a thread has all of its loads in flight at once
// instead of streaming 128 rows one after another (the same order for every
// call, so appends still reproduce the whole-history compression bit for bit).
#include "common.hpp"
#include "kernels.h"

namespace csa {
namespace {

constexpr int kThreads = 256;

template <typename TIn>
struct Row8;  // 8 consecutive elements converted to double

template <>
struct Row8<float> {
  static __device__ __forceinline__ void load(const float* p, double (&v)[8]) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};
template <>
struct Row8<bf16_t> {
  static __device__ __forceinline__ void load(const bf16_t* p, double (&v)[8]) {
    uint4 a = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = u32_as_f32(w[i] << 16);
      v[2 * i + 1] = u32_as_f32(w[i] & 0xffff0000u);
    }
  }
};

// The 16 or 32 bytes of 8 consecutive elements, loaded ahead of their use.
template <typename TIn>
struct Raw8;
template <>
struct Raw8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void to_double(double (&v)[8]) const {
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};
template <>
struct Raw8<bf16_t> {
  uint4 a;
  __device__ __forceinline__ void load(const bf16_t* p) { a = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void to_double(double (&v)[8]) const {
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = u32_as_f32(w[i] << 16);
      v[2 * i + 1] = u32_as_f32(w[i] & 0xffff0000u);
    }
  }
};

// The new rows of an append (state-cache ring, see csa_append): workgroups
// past the compression ones copy them into both ring rows of their position,
// and the compression reads positions >= t0 from them instead of the ring, so
// that one launch does both without ordering the two.
struct AppendTail {
  const void* x_new;  // [B, T_new, d]
  int64_t t0;
  int T_new;
  int64_t R;
  int cmp_blocks;     // workgroups (per sequence) that compress
};

// OUT: 0 = fp32, 1 = bf16, 2 = e4m3 + per-entry fp32 scale.
// Overlap o > 0 (a method variant): entry j folds the m + o rows of positions
// j*m - o .. j*m + m - 1 with the softmax of m + o logits; the first entries,
// whose leading slots fall before position 0, renormalise over the rest.
// Slot groups of an entry: about 8 slots each, as many as the threads allow.
__host__ __device__ __forceinline__ int slot_parts(int ms, int tpe) {
  int parts = (ms + 7) / 8;
  const int most = kThreads / tpe;
  return parts < most ? parts : most;
}

// SPLIT: the entry's slots are split over several thread groups (P > 1).
template <typename TIn, int OUT, bool APPEND, bool SPLIT>
__global__ __launch_bounds__(kThreads) void compress_kernel(
    const TIn* __restrict__ x, int64_t n_raw, int d, int64_t raw_base,
    const float* __restrict__ logits, int m, int o, int64_t entry_begin, int64_t n_ent, int64_t N_alloc,
    void* __restrict__ out, float* __restrict__ out_scale, AppendTail at) {
  __shared__ double alpha[128];
  __shared__ float zmax_s;
  __shared__ double partial[SPLIT ? kThreads : 1][8];  // slot-group sums
  debug_poison_lds(alpha);
  debug_poison_lds(zmax_s);
  debug_poison_lds(partial);
  const int tid = threadIdx.x;
  const int b = blockIdx.y;
  const TIn* xn = reinterpret_cast<const TIn*>(at.x_new) + int64_t(b) * at.T_new * d;
  if (APPEND && int(blockIdx.x) >= at.cmp_blocks) {
    // Copy: one thread per 16-byte chunk of a new row, written to rows
    // p % R and p % R + R of the (writable) ring x.
    constexpr int EPC = 16 / sizeof(TIn);  // elements per chunk
    const int cpr = d / EPC;
    const int64_t gi = int64_t(int(blockIdx.x) - at.cmp_blocks) * kThreads + tid;
    if (gi >= int64_t(at.T_new) * cpr) return;
    const int i = int(gi / cpr), c = int(gi - int64_t(i) * cpr);
    const int64_t slot = (at.t0 + i) % at.R;
    TIn* ring = const_cast<TIn*>(x) + int64_t(b) * n_raw * d + c * EPC;
    const uint4 v = *reinterpret_cast<const uint4*>(xn + int64_t(i) * d + c * EPC);
    *reinterpret_cast<uint4*>(ring + slot * d) = v;
    *reinterpret_cast<uint4*>(ring + (slot + at.R) * d) = v;
    return;
  }

  const int ms = m + o;  // slots per entry
  const int tpe = d >> 3;  // threads per entry and slot group, 8 columns each
  const int P = SPLIT ? slot_parts(ms, tpe) : 1;
  const int sper = (ms + P - 1) / P;  // slots per group
  const int epb = kThreads / (tpe * P);
  const int part = (tid / tpe) % P;
  const int64_t e_local = int64_t(blockIdx.x) * epb + tid / (tpe * P);
  const int seg = tid % tpe;
  const bool valid = tid < epb * tpe * P && e_local < n_ent;
  const int64_t j = entry_begin + e_local;
  const int64_t p0 = j * m - o;  // position of slot 0
  const TIn* xb = x + int64_t(b) * n_raw * d + seg * 8;
  const int s_begin = part * sper;
  const int s_end = (part + 1) * sper < ms ? (part + 1) * sper : ms;
  auto row_of = [&](int s) __attribute__((always_inline)) {
    const int64_t pos = p0 + s;
    if (APPEND && pos >= at.t0) return xn + (pos - at.t0) * d + seg * 8;
    return xb + (pos - raw_base) * d;
  };
  // The group's first kAhead rows are loaded before the weights are formed, so
  // that their latency overlaps the softmax (a decode step's append is one
  // chain of such latencies).
  constexpr int kAhead = sizeof(TIn) == 4 ? 4 : 8;  // fp32 rows take twice the registers
  Raw8<TIn> ahead[kAhead];
  if (valid) {
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      const int s = s_begin + u;
      if (s < s_end && p0 + s >= 0) ahead[u].load(row_of(s));
    }
  }

  // Slot weights: softmax of the logits, in fp64.
  if (tid < kWave) {
    float v = -INFINITY;
    for (int s = tid; s < ms; s += kWave) v = fmaxf(v, logits[s]);
    v = wave_max(v);
    if (tid == 0) zmax_s = v;
  }
  __syncthreads();
  for (int s = tid; s < ms; s += kThreads) alpha[s] = exp(double(logits[s]) - double(zmax_s));
  __syncthreads();
  double total = 0.0;
  for (int s = 0; s < ms; ++s) total += alpha[s];
  __syncthreads();
  for (int s = tid; s < ms; s += kThreads) alpha[s] = alpha[s] / total;
  __syncthreads();

  double acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0;
  if (valid) {
    // Slot order throughout: the rows loaded ahead, then the rest.
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      const int s = s_begin + u;
      if (s < s_end && p0 + s >= 0) {
        double v[8];
        ahead[u].to_double(v);
        const double a = alpha[s];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fma(a, v[i], acc[i]);
      }
    }
#pragma unroll 8
    for (int s = s_begin + kAhead; s < s_end; ++s) {
      if (p0 + s < 0) continue;
      double v[8];
      Row8<TIn>::load(row_of(s), v);
      const double a = alpha[s];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fma(a, v[i], acc[i]);
    }
  }
  if (SPLIT) {  // group 0 adds the other groups' sums, in group order
    if (valid && part > 0)
#pragma unroll
      for (int i = 0; i < 8; ++i) partial[tid][i] = acc[i];
    __syncthreads();
    if (valid && part == 0)
      for (int q = 1; q < P; ++q)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += partial[tid + q * tpe][i];
  }
  if (valid && p0 < 0) {
    double wsum = 0.0;  // weight of the slots at positions >= 0
    for (int s = 0; s < ms; ++s) wsum += (p0 + s >= 0) ? alpha[s] : 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] /= wsum;
  }

  const bool writer = valid && part == 0;  // the first slot group holds the sum
  const int64_t orow = int64_t(b) * N_alloc + j;
  if (OUT == 0) {
    if (writer) {
      float* o = reinterpret_cast<float*>(out) + orow * d + seg * 8;
      *reinterpret_cast<float4*>(o) = make_float4(float(acc[0]), float(acc[1]), float(acc[2]), float(acc[3]));
      *reinterpret_cast<float4*>(o + 4) = make_float4(float(acc[4]), float(acc[5]), float(acc[6]), float(acc[7]));
    }
  } else if (OUT == 1) {
    if (writer) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = uint32_t(f64_to_bf16(acc[2 * i])) | (uint32_t(f64_to_bf16(acc[2 * i + 1])) << 16);
      bf16_t* o = reinterpret_cast<bf16_t*>(out) + orow * d + seg * 8;
      *reinterpret_cast<uint4*>(o) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  } else {
    // e4m3: binary32 image of the sum, per-entry absmax / 448 scale.
    float r[8];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      r[i] = float(acc[i]);
      amax = fmaxf(amax, fabsf(r[i]));
    }
    for (int o = tpe >> 1; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    // fmaxf leaves NaN elements out of amax.  A quotient of 0 (an all-zero row,
    // or a largest magnitude below 448 * 2^-150, which underflows) takes scale 1.
    float scale = amax / 448.0f;
    if (scale == 0.0f) scale = 1.0f;
    if (writer) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo |= uint32_t(f32_to_e4m3(r[i] / scale)) << (8 * i);
        hi |= uint32_t(f32_to_e4m3(r[i + 4] / scale)) << (8 * i);
      }
      uint8_t* o = reinterpret_cast<uint8_t*>(out) + orow * d + seg * 8;
      *reinterpret_cast<uint2*>(o) = make_uint2(lo, hi);
      if (seg == 0) out_scale[orow] = scale;
    }
  }
}

template <typename TIn, int OUT, bool APPEND>
hipError_t launch(const CompressArgs& a, const AppendTail& at) {
  const int tpe = a.d / 8;
  const int parts = slot_parts(a.m + a.overlap, tpe);
  const int epb = kThreads / (tpe * parts);
  const int64_t n_ent = a.entry_end - a.entry_begin;
  AppendTail t = at;
  t.cmp_blocks = int((n_ent + epb - 1) / epb);
  int64_t blocks = t.cmp_blocks;
  if (APPEND) blocks += (int64_t(t.T_new) * (a.d * int64_t(sizeof(TIn)) / 16) + kThreads - 1) / kThreads;
  dim3 grid(unsigned(blocks), unsigned(a.B));
  CSA_HOST_CHECK(blocks >= 1 && a.m >= 1 && a.m + a.overlap <= 128);
  log_dispatch("%s: B=%d d=%d m=%d overlap=%d entries [%lld, %lld) -> grid %lld x %d, %d slot group(s)",
               APPEND ? "append" : "compress", a.B, a.d, a.m, a.overlap, (long long)a.entry_begin,
               (long long)a.entry_end, (long long)blocks, a.B, parts);
  ProfScope prof(APPEND ? "append" : "compress", a.stream);
  auto kernel = parts > 1 ? compress_kernel<TIn, OUT, APPEND, true> : compress_kernel<TIn, OUT, APPEND, false>;
  hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, a.stream,
                     reinterpret_cast<const TIn*>(a.x), a.n_raw, a.d, a.raw_base, a.logits, a.m, a.overlap,
                     a.entry_begin, n_ent, a.N_alloc, a.out, a.out_scale, t);
  return hipGetLastError();
}

template <bool APPEND>
hipError_t dispatch(const CompressArgs& a, const AppendTail& t) {
  if (a.x_bf16) {
    if (a.out_kind == 0) return launch<bf16_t, 0, APPEND>(a, t);
    if (a.out_kind == 1) return launch<bf16_t, 1, APPEND>(a, t);
    return launch<bf16_t, 2, APPEND>(a, t);
  }
  if (a.out_kind == 0) return launch<float, 0, APPEND>(a, t);
  if (a.out_kind == 1) return launch<float, 1, APPEND>(a, t);
  return launch<float, 2, APPEND>(a, t);
}

}  // namespace

hipError_t launch_compress(const CompressArgs& a) {
  if (a.entry_end <= a.entry_begin) return hipSuccess;
  return dispatch<false>(a, AppendTail{a.x, 0, 0, 1, 0});
}

hipError_t launch_append(const CompressArgs& a, const void* x_new, int64_t t0, int T_new, int64_t R) {
  if (T_new <= 0) return hipSuccess;
  return dispatch<true>(a, AppendTail{x_new, t0, T_new, R, 0});
}

}  // namespace csa

// Device-side helpers shared by the gfx950 kernels of libcsa.
//
// Number formats: bf16 is kept as raw uint16 bits (upper half of a binary32);
// fp8 is the OCP e4m3fn byte format.  Every conversion here is exact or
// round-to-nearest-even, so that stored values are reproducible bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

typedef uint16_t bf16_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;

constexpr int kWave = 64;

__device__ __forceinline__ float u32_as_f32(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t f32_as_u32(float f) { return __float_as_uint(f); }

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return u32_as_f32(uint32_t(h) << 16); }

// Round a binary32 to bf16, nearest-even (NaN stays NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = f32_as_u32(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return bf16_t((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return bf16_t(u >> 16);
}

// Round a binary64 to bf16 with a single nearest-even rounding.  The value is
// first narrowed to binary32 with round-to-odd (truncate, then set the last bit
// if anything was dropped): binary32 keeps 16 more bits than bf16 in every
// range, so the second, nearest-even, rounding then equals one direct rounding.
__device__ __forceinline__ bf16_t f64_to_bf16(double x) {
  float f = float(x);  // nearest-even
  double back = double(f);
  if (back != x && x == x) {
    uint32_t u = f32_as_u32(f);
    if (fabs(back) > fabs(x)) u -= 1u;  // rounded away from zero: step back (truncation)
    u |= 1u;                            // sticky bit
    f = u32_as_f32(u);
  }
  return f32_to_bf16(f);
}

// Two binary32 values to packed bf16 bits (element 0 in the low half), with the
// gfx950 conversion instruction (round to nearest even).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_bits(f32x2_t v) {
  const bf16x2_t h = __builtin_convertvector(v, bf16x2_t);
  uint32_t u;
  __builtin_memcpy(&u, &h, 4);
  return u;
}

// Two binary32 values to packed IEEE binary16 bits (element 0 in the low
// half), round to nearest even; magnitudes past the binary16 range give inf.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f16x2_bits(f32x2_t v) {
  const f16x2_t h = __builtin_convertvector(v, f16x2_t);
  uint32_t u;
  __builtin_memcpy(&u, &h, 4);
  return u;
}
// Two packed bf16 values to packed binary16: exact when both magnitudes are 0
// or lie in [2^-14, 65280] (the binary16 normal range holds every bf16 there).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  const f32x2_t f = {__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u)};
  return f16x2_bits(f);
}

// ---------------------------------------------------------------- fp8 e4m3fn

// Encode a binary32 as e4m3fn, nearest-even.  Magnitudes up to 464 round to at
// most 448 (464 ties to the even code 448); larger magnitudes and NaN give NaN.
__device__ __forceinline__ uint8_t f32_to_e4m3(float v) {
  uint32_t u = f32_as_u32(v);
  uint32_t sign = (u >> 24) & 0x80u;
  float a = fabsf(v);
  if (!(a == a)) return uint8_t(sign | 0x7fu);
  uint32_t code;
  if (a < 0.015625f) {  // below 2^-6: subnormal grid m * 2^-9 (m = 8 is the first normal)
    code = uint32_t(rintf(a * 512.0f));
  } else {
    uint32_t ua = f32_as_u32(a);
    uint32_t r = (ua + 0x7ffffu + ((ua >> 20) & 1u)) & 0xfff00000u;  // keep 3 mantissa bits
    int e = int(r >> 23) - 127;
    uint32_t mant = (r >> 20) & 7u;
    if (e > 8 || (e == 8 && mant == 7u)) return uint8_t(sign | 0x7fu);
    code = (uint32_t(e + 7) << 3) | mant;
  }
  return uint8_t(sign | code);
}

// Decode four e4m3fn bytes (packed little-endian in a uint32) into bf16 bit
// patterns (exact: every e4m3 value is a bf16 value).  Uses the gfx950 packed
// fp8 -> fp32 converter, whose OCP e4m3fn decoding is exact.
__device__ __forceinline__ void e4m3x4_to_bf16x4(uint32_t packed, uint32_t& lo, uint32_t& hi) {
  f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8(int(packed), false);
  f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8(int(packed), true);
  lo = (f32_as_u32(a[0]) >> 16) | (f32_as_u32(a[1]) & 0xffff0000u);
  hi = (f32_as_u32(b[0]) >> 16) | (f32_as_u32(b[1]) & 0xffff0000u);
}

// Two e4m3fn codes (the low or the high 16 bits of packed) widened exactly to
// a bf16 pair: every e4m3 value is a bf16 value, and a scale of 1 leaves it be.
template <bool HIGH>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t packed) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(packed, 1.0f, HIGH));
}

// ---------------------------------------------------------------- ordering keys

// A binary32 rounded to the nearest bf16 value (ties to even), as binary32.
__device__ __forceinline__ float round_bf16(float s) {
  const f32x2_t v = {s, 0.0f};
  return u32_as_f32(bf16x2_bits(v) << 16);
}

// Order-preserving image of a binary32 score: a > b  <=>  key(a) > key(b).
// -0 is folded onto +0 first so that equal scores get equal keys.  Every NaN,
// of either sign, maps to the largest key: a NaN score ranks above every
// number (+inf included), and key_score gives it back as a NaN.
__device__ __forceinline__ uint32_t score_key(float s) {
  const uint32_t u = f32_as_u32(s + 0.0f);
  const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (s != s) ? 0xffffffffu : k;
}
__device__ __forceinline__ float key_score(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return u32_as_f32(u);
}
// Total order used by the selection: higher score first, then lower index.
__device__ __forceinline__ uint64_t rank_key(uint32_t key, uint32_t idx) {
  return (uint64_t(key) << 32) | uint64_t(0xffffffffu - idx);
}
__device__ __forceinline__ uint32_t rank_key_idx(uint64_t rk) {
  return 0xffffffffu - uint32_t(rk & 0xffffffffu);
}

// The indexer's rectifier max(0, x), propagating NaN of either sign (IEEE
// 754-2019 maximum; one v_maximum3_f32 on gfx950).  +-0 give +0.
__device__ __forceinline__ float relu_nan(float x) { return __builtin_elementwise_maximum(x, 0.0f); }

// ---------------------------------------------------------------- MFMA

// D = A(16x32) * B(32x16) + C.  Lane l holds A row l%16 / B column l%16, k-slots
// 8*(l/16) .. 8*(l/16)+7; C/D lane l holds column l%16, rows 4*(l/16) .. +3.
__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
// The same product with binary16 operands.
__device__ __forceinline__ f32x4_t mfma16x16x32_f16(f16x8_t a, f16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16x8_t u32x4_as_f16x8(uint4 v) {
  f16x8_t r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

template <typename T>
__device__ __forceinline__ T as(const void* p) {
  return *reinterpret_cast<const T*>(p);
}

__device__ __forceinline__ bf16x8_t u32x4_as_bf16x8(uint4 v) {
  bf16x8_t r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// The same product with OCP e4m3fn operands: a lane's 8 k-slots are 8 codes
// packed little-endian in 64 bits (slot 8*(l/16) in the lowest byte).  Every
// e4m3 x e4m3 product is exact in binary32.
__device__ __forceinline__ f32x4_t mfma16x16x32_fp8(uint64_t a, uint64_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(static_cast<long>(a), static_cast<long>(b), c, 0, 0, 0);
}

// ---------------------------------------------------------------- e4m3 query rows
//
// A bf16 row held 8 values per lane by lanes l, l^16, l^32, l^48 (the A
// operand layout above) quantised to e4m3 with one binary32 scale per row, the
// rule of the key cache: scale = absmax / 448 (NaN elements ignored), 1 where
// that quotient is 0; code = e4m3 nearest-even of the binary32 quotient x / scale.

// Largest magnitude of the 8 bf16 values of v that are not NaN.
__device__ __forceinline__ float bf16x8_absmax(uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = fmaxf(m, fabsf(u32_as_f32(w[i] << 16)));          // fmaxf returns the non-NaN operand
    m = fmaxf(m, fabsf(u32_as_f32(w[i] & 0xffff0000u)));
  }
  return m;
}
// Row scale from this lane's part of the absmax (reduced over the 4 lanes of the row).
__device__ __forceinline__ float e4m3_row_scale(float part) {
  float m = fmaxf(part, __shfl_xor(part, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  const float s = m / 448.0f;
  return s == 0.0f ? 1.0f : s;
}
// e4m3 codes of the 8 bf16 values of v divided by scale.
__device__ __forceinline__ uint64_t bf16x8_to_e4m3x8(uint4 v, float scale) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint64_t r = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r |= uint64_t(f32_to_e4m3(u32_as_f32(w[i] << 16) / scale)) << (16 * i);
    r |= uint64_t(f32_to_e4m3(u32_as_f32(w[i] & 0xffff0000u) / scale)) << (16 * i + 8);
  }
  return r;
}

// ---------------------------------------------------------------- debug builds

// Builds with CSA_DEBUG: fill a kernel's LDS object with all-ones words (NaN as
// fp32 and bf16) and wait for every thread, before the kernel uses it.  Called
// first thing in a kernel, where every thread of the workgroup reaches it.
template <typename T>
__device__ __forceinline__ void debug_poison_lds(T& obj) {
#ifdef CSA_DEBUG
  uint32_t* p = reinterpret_cast<uint32_t*>(&obj);
  for (uint32_t i = threadIdx.x; i < uint32_t(sizeof(T) / 4); i += blockDim.x) p[i] = 0xffffffffu;
  __syncthreads();
#else
  (void)obj;
#endif
}

// ---------------------------------------------------------------- cross-workgroup handoff
//
// Data that one workgroup hands to another inside the same kernel is written
// with device-scope stores (they complete at the device coherence point, past
// the per-XCD L2) and read with device-scope loads.  The writer then waits for
// its stores to complete before it increments the arrival counter, so no
// L2 write-back / invalidate fence is needed.

template <typename T>
__device__ __forceinline__ void store_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T load_dev(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory operation this thread issued has completed.
__device__ __forceinline__ void wait_mem() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// All threads: after each thread's device-scope stores, count this workgroup in
// *counter; returns true in every thread of the workgroup that arrives last.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t expected, uint32_t* s_flag) {
  wait_mem();
  __syncthreads();
  if (threadIdx.x == 0)
    s_flag[0] = (__hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 expected - 1u) ? 1u : 0u;
  __syncthreads();
  return s_flag[0] != 0;
}

// ---------------------------------------------------------------- DPP wave scans
//
// Inclusive scans over the 64 lanes of a wave with DPP row shifts (within rows
// of 16 lanes) and the two row broadcasts, which need no LDS round trip.  Lanes
// without a source keep the identity.

template <typename Op>
__device__ __forceinline__ uint32_t wave_scan_dpp(uint32_t v, uint32_t identity, Op op) {
  const int e = int(identity);
  v = op(v, uint32_t(__builtin_amdgcn_update_dpp(e, int(v), 0x111, 0xf, 0xf, false)));  // row_shr:1
  v = op(v, uint32_t(__builtin_amdgcn_update_dpp(e, int(v), 0x112, 0xf, 0xf, false)));  // row_shr:2
  v = op(v, uint32_t(__builtin_amdgcn_update_dpp(e, int(v), 0x114, 0xf, 0xf, false)));  // row_shr:4
  v = op(v, uint32_t(__builtin_amdgcn_update_dpp(e, int(v), 0x118, 0xf, 0xf, false)));  // row_shr:8
  v = op(v, uint32_t(__builtin_amdgcn_update_dpp(e, int(v), 0x142, 0xa, 0xf, false)));  // row_bcast:15
  v = op(v, uint32_t(__builtin_amdgcn_update_dpp(e, int(v), 0x143, 0xc, 0xf, false)));  // row_bcast:31
  return v;
}
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v) {
  return wave_scan_dpp(v, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}
// Reductions: the last lane of the inclusive scan, broadcast.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return uint32_t(__builtin_amdgcn_readlane(
      int(wave_scan_dpp(v, 0xffffffffu, [](uint32_t a, uint32_t b) { return a < b ? a : b; })), 63));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return uint32_t(__builtin_amdgcn_readlane(
      int(wave_scan_dpp(v, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; })), 63));
}

// ---------------------------------------------------------------- integer division

// a / b and a % b for non-negative a and positive b; takes the 32-bit path when
// both fit (a full 64-bit division is a long instruction sequence on the GPU).
__device__ __forceinline__ int64_t div64(int64_t a, int64_t b) {
  if (((uint64_t(a) | uint64_t(b)) >> 32) == 0) return int64_t(uint32_t(a) / uint32_t(b));
  return a / b;
}
__device__ __forceinline__ int64_t mod64(int64_t a, int64_t b) { return a - div64(a, b) * b; }

// ---------------------------------------------------------------- reductions

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
// wave_max by DPP row shifts and row broadcasts (no LDS traffic): a lane with
// no source keeps its own value, so the result follows fmaxf over the 64
// values (NaN only if all are NaN), broadcast from lane 63.
__device__ __forceinline__ float dpp_max_step(float v, int moved) { return fmaxf(v, __builtin_bit_cast(float, moved)); }
__device__ __forceinline__ float wave_max_dpp(float v) {
#define CSA_DPP_MAX(ctrl, rows) \
  v = dpp_max_step(v, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v), ctrl, rows, 0xf, false))
  CSA_DPP_MAX(0x111, 0xf);  // row_shr:1
  CSA_DPP_MAX(0x112, 0xf);  // row_shr:2
  CSA_DPP_MAX(0x114, 0xf);  // row_shr:4
  CSA_DPP_MAX(0x118, 0xf);  // row_shr:8
  CSA_DPP_MAX(0x142, 0xa);  // row_bcast:15
  CSA_DPP_MAX(0x143, 0xc);  // row_bcast:31
#undef CSA_DPP_MAX
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

}  // namespace csa

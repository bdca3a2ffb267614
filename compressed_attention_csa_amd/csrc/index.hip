// Lightning-Indexer scoring and exact per-query top-k for gfx950 (rows x slices path).
//
// V4 report digest, section 三: an indexer scores the compressed entries and only
// the top-k enter the core attention; section 七: the indexer keys are cached in
// low precision.  Score of entry j for query row r (position t):
//     I(r, j) = sum_h w[r,h] * max(0, q[r,h] . k[j]),  j < c(t) = min(N, (t+1)/m)
// The selection is the min(k, c(t)) best entries by (score desc, index asc).
//
// Design (one kernel).  A row's visible entries are cut into slices; one
// workgroup scores one slice, keeping the fp32 scores as order-preserving
// uint32 keys in LDS, and ranks entries by the 64-bit key (score, ~index) so
// that all ranks are distinct.
//   * A row with a single slice is finished by its WG: an LDS radix select
//     finds the threshold of the kk best and the winners are written.
//   * A longer row: every WG writes its exact local top-K_loc in decreasing
//     order (K_loc: the slice's expected share of the row's winners plus four
//     standard deviations, and enough for the slices together to hold kk when
//     the last one is short) plus a certificate, the key below which it
//     dropped entries.  The last WG of the row to arrive loads every list and
//     certificate in one batch and radix-selects the row's kk best.  A slice
//     whose certificate lies above that threshold may have dropped a winner;
//     the last WG then rescores exactly those slices and adds the dropped
//     entries above the threshold before selecting again, so the result is
//     exact for any input; on typical inputs no slice needs it.
// Output order is deterministic (a fixed order of the candidates).
// bf16 / e4m3 keys are scored with 16x16x32 bf16 MFMA (query heads as rows,
// entries as columns; e4m3 codes are widened exactly to bf16 in registers),
// with 8 groups of 16 keys in flight per wave; fp32 keys use fp32 FMA with one
// entry per lane.
#include "common.hpp"
#include "kernels.h"

namespace csa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kUnroll = 8;  // 16-key groups in flight per wave

struct RowCtrl {
  uint32_t arrive, pad0, pad1, pad2;
};

struct RowInfo {
  int64_t r, b, i, t, c, kk, S, lo, hi, kloc;
};

__device__ __forceinline__ RowInfo row_info(const IndexArgs& a, const IndexPlan& p, int64_t r,
                                            int64_t s) {
  RowInfo ri;
  ri.r = r;
  ri.b = div64(r, a.T);
  ri.i = r - ri.b * a.T;
  ri.t = a.t0 + ri.i;
  int64_t c = div64(ri.t + 1, a.m);
  ri.c = c < a.N_alloc ? c : a.N_alloc;
  ri.kk = ri.c < a.top_k ? ri.c : a.top_k;
  int64_t S = div64(ri.c + p.slice - 1, p.slice);
  ri.S = S < 1 ? 1 : S;
  ri.lo = s * p.slice;
  int64_t hi = ri.lo + p.slice;
  ri.hi = hi < ri.c ? hi : ri.c;
  if (ri.hi < ri.lo) ri.hi = ri.lo;
  // Local candidates per slice: the slice's expected share of winners plus
  // four standard deviations of that count (about sqrt(share)) and a margin,
  // rounded up to 8.  A slice holding more winners is caught by its
  // certificate and rescored.
  const int64_t share = div64(ri.kk + ri.S - 1, ri.S);
  int64_t sd = 1;
  while (sd * sd < share) ++sd;
  int64_t kl = share + 4 * sd + 4;
  // Every slice lists at least min(kl, its size) entries; together they must
  // reach kk even when the last slice is short.
  if (ri.S > 1) {
    const int64_t last_n = ri.c - (ri.S - 1) * p.slice;
    const int64_t need = div64(ri.kk - (last_n < ri.kk ? last_n : ri.kk) + ri.S - 2, ri.S - 1);
    if (kl < need) kl = need;
  }
  kl = ((kl + 7) / 8) * 8;
  if (kl < 16) kl = 16;
  if (kl > p.slice) kl = p.slice;
  ri.kloc = kl;
  return ri;
}

// Exclusive position of this thread among the flagged threads of the block (thread
// order) and the block total.  All threads must call it.
__device__ __forceinline__ int block_rank(bool flag, int* s_wave, int& total) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  uint64_t bal = __ballot(flag);
  int in_wave = __popcll(bal & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
  if (lane == 0) s_wave[wid] = __popcll(bal);
  __syncthreads();
  int off = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    int v = s_wave[w];
    off += (w < wid) ? v : 0;
    total += v;
  }
  __syncthreads();
  return off + in_wave;
}

// Inclusive block-wide prefix sum of one uint32 per thread (thread order).
__device__ __forceinline__ uint32_t block_inclusive_sum(uint32_t v, uint32_t* s_scan) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  v = wave_incl_sum(v);
  if (lane == kWave - 1) s_scan[wid] = v;
  __syncthreads();
  uint32_t pre = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) pre += (w < wid) ? s_scan[w] : 0u;
  __syncthreads();
  return v + pre;
}

// ---------------------------------------------------------------- scoring

// Sum of x over the four 16-lane rows of the wave, in every lane (two lane
// swaps; no LDS round trip).
__device__ __forceinline__ float sum_rows4(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(f32_as_u32(x), f32_as_u32(x), false, false);
  const float y = u32_as_f32(a[0]) + u32_as_f32(a[1]);  // x[l] + x[l ^ 32]
  const auto b = __builtin_amdgcn_permlane16_swap(f32_as_u32(y), f32_as_u32(y), false, false);
  return u32_as_f32(b[0]) + u32_as_f32(b[1]);            // y[l] + y[l ^ 16]
}

// bf16 / e4m3 keys on 16x16x32 MFMA: query heads are the rows of A (zero past
// H_I), 16 keys are the columns of B, so lane (g, col) ends with heads
// 4g..4g+3 of key col.  Each wave takes groups of 16 keys; the loads of one
// round (8 groups, 4 for 64-dim bf16 keys) are in flight while the previous
// round is scored.
// Loads are unconditional (groups past the slice re-read its last key), so
// the compiler's wait counts stay exact.
// KK == kKeyE4M3Q8: the query rows are quantised to e4m3 and the products are
// fp8 x fp8 MFMAs on the raw key codes; each head's query scale moves into its
// weight (relu(s * x) = s * relu(x) for s > 0).
template <int KK, int DI, bool PEEL>
__device__ __forceinline__ void score_slice_mfma(const IndexArgs& a, const RowInfo& ri, uint32_t* keys,
                                                 int64_t qrow) {
  constexpr int CW = KK == kKeyBF16 ? 2 * DI / 16 : DI / 16;  // dwords of key per lane
  constexpr int U = CW > 4 ? kUnroll / 2 : kUnroll;             // groups per round and wave
  typedef uint32_t kregs_t __attribute__((ext_vector_type(U * CW)));
  typedef float sregs_t __attribute__((ext_vector_type(U)));
  struct Round {
    kregs_t k;
    sregs_t sc;
  };
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, g = lane >> 4, col = lane & 15;
  const int64_t n = ri.hi - ri.lo;
  const int H_I = a.H_I;
  const bf16_t* q = reinterpret_cast<const bf16_t*>(a.q_idx) + qrow * DI;
  // A operands: row = head col (zero past H_I), k-slots 8g..8g+7.  For 64 dims
  // the k-slots of the two products map to dims 16g..16g+7 and 16g+8..16g+15,
  // so a lane reads 16 contiguous dims of its key.
  constexpr bool Q8 = KK == kKeyE4M3Q8;
  bf16x8_t qa0, qa1;
  uint64_t q80 = 0, q81 = 0;  // the same k-slots as e4m3 codes (Q8)
  float qscale = 1.0f;        // scale of query head col (Q8)
  {
    uint4 v0 = make_uint4(0, 0, 0, 0), v1 = make_uint4(0, 0, 0, 0);
    if (col < H_I) {
      if (DI == 64) {
        v0 = *reinterpret_cast<const uint4*>(q + col * 64 + 16 * g);
        v1 = *reinterpret_cast<const uint4*>(q + col * 64 + 16 * g + 8);
      } else {
        v0 = *reinterpret_cast<const uint4*>(q + col * 32 + 8 * g);
      }
    }
    qa0 = u32x4_as_bf16x8(v0);
    qa1 = u32x4_as_bf16x8(v1);
    if (Q8) {
      qscale = e4m3_row_scale(fmaxf(bf16x8_absmax(v0), bf16x8_absmax(v1)));
      q80 = bf16x8_to_e4m3x8(v0, qscale);
      q81 = bf16x8_to_e4m3x8(v1, qscale);
    }
  }
  // Rows past H_I hold zeros; they are left out of the head sum rather than
  // weighted by 0, since their product with an infinite key element is NaN.
  float wr[4];
  bool hv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = 4 * g + j;
    hv[j] = h < H_I;
    wr[j] = hv[j] ? (a.w ? a.w[qrow + h] : 1.0f) : 0.0f;
    if (Q8) wr[j] *= __shfl(qscale, h);  // A row h is lane h
  }
  const int64_t kb = ri.b * a.N_alloc + ri.lo;
  const int64_t ngroups = (n + 15) / 16;
  constexpr int RS = kWaves * U;  // groups per round
  const int nr = int((ngroups + RS - 1) / RS);
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k_idx) + kb * DI * (KK == kKeyBF16 ? 2 : 1);
  const float* sbase = key_is_e4m3(KK) ? a.k_scale + kb : nullptr;
  const uint32_t last = uint32_t(n - 1);
  auto load = [&](Round& R, int rr) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t e = uint32_t((int64_t(rr) * RS + u * kWaves + wid) * 16 + col);
      const uint32_t ec = e < last ? e : last;
      if (KK == kKeyBF16) {
        const uint8_t* kp = kbase + ec * (DI * 2);
        const uint4 x0 = *reinterpret_cast<const uint4*>(kp + (DI == 64 ? 32 : 16) * g);
        R.k[CW * u] = x0.x; R.k[CW * u + 1] = x0.y; R.k[CW * u + 2] = x0.z; R.k[CW * u + 3] = x0.w;
        if (DI == 64) {
          const uint4 x1 = *reinterpret_cast<const uint4*>(kp + 32 * g + 16);
          R.k[CW * u + 4] = x1.x; R.k[CW * u + 5] = x1.y; R.k[CW * u + 6] = x1.z; R.k[CW * u + 7] = x1.w;
        }
      } else {
        const uint8_t* kp = kbase + ec * DI;
        if (DI == 64) {
          const uint4 x0 = *reinterpret_cast<const uint4*>(kp + 16 * g);
          R.k[CW * u] = x0.x; R.k[CW * u + 1] = x0.y; R.k[CW * u + 2] = x0.z; R.k[CW * u + 3] = x0.w;
        } else {
          const uint2 x0 = *reinterpret_cast<const uint2*>(kp + 8 * g);
          R.k[CW * u] = x0.x; R.k[CW * u + 1] = x0.y;
        }
        R.sc[u] = sbase[ec];
      }
    }
  };
  auto score = [&](const Round& R, int rr) __attribute__((always_inline)) {
    f32x4_t acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (Q8) {
        // Raw codes: dims 16g..16g+15 (DI = 64) or 8g..8g+7 (DI = 32).
        f32x4_t c = {0.0f, 0.0f, 0.0f, 0.0f};
        c = mfma16x16x32_fp8(q80, (uint64_t(R.k[CW * u + 1]) << 32) | R.k[CW * u], c);
        if (DI == 64) c = mfma16x16x32_fp8(q81, (uint64_t(R.k[CW * u + 3]) << 32) | R.k[CW * u + 2], c);
        acc[u] = c;
        continue;
      }
      uint4 b0, b1 = make_uint4(0, 0, 0, 0);
      if (KK == kKeyBF16) {
        b0 = make_uint4(R.k[CW * u], R.k[CW * u + 1], R.k[CW * u + 2], R.k[CW * u + 3]);
        if (DI == 64) b1 = make_uint4(R.k[CW * u + 4], R.k[CW * u + 5], R.k[CW * u + 6], R.k[CW * u + 7]);
      } else {
        // e4m3 codes widen exactly to bf16 (scale 1).
        b0.x = e4m3x2_to_bf16x2<false>(R.k[CW * u]);
        b0.y = e4m3x2_to_bf16x2<true>(R.k[CW * u]);
        b0.z = e4m3x2_to_bf16x2<false>(R.k[CW * u + 1]);
        b0.w = e4m3x2_to_bf16x2<true>(R.k[CW * u + 1]);
        if (DI == 64) {
          b1.x = e4m3x2_to_bf16x2<false>(R.k[CW * u + 2]);
          b1.y = e4m3x2_to_bf16x2<true>(R.k[CW * u + 2]);
          b1.z = e4m3x2_to_bf16x2<false>(R.k[CW * u + 3]);
          b1.w = e4m3x2_to_bf16x2<true>(R.k[CW * u + 3]);
        }
      }
      f32x4_t c = {0.0f, 0.0f, 0.0f, 0.0f};
      c = mfma16x16x32(qa0, u32x4_as_bf16x8(b0), c);
      if (DI == 64) c = mfma16x16x32(qa1, u32x4_as_bf16x8(b1), c);
      acc[u] = c;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float part = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        part = hv[j] ? fmaf(wr[j], relu_nan(acc[u][j]), part) : part;
      }
      part = sum_rows4(part);
      if (key_is_e4m3(KK)) part *= R.sc[u];
      if (a.bf16_scores) part = round_bf16(part);
      const int64_t e = (int64_t(rr) * RS + u * kWaves + wid) * 16 + col;
      if (g == 0 && e < n) keys[e] = score_key(part);
    }
  };
  // Two rounds alternate.  PEEL: the last one or two are peeled off so that
  // no load past the final round is issued (its wait would otherwise come due
  // before the selection that follows: 2% of a 1M-entry decode call).  The
  // variants with 16 slice keys per thread keep the plain loop, which needs
  // fewer registers.
  if (nr > 0) {
    Round R0, R1;
    load(R0, 0);
    if (PEEL) {
      int rr = 0;
      for (; rr + 2 < nr; rr += 2) {
        load(R1, rr + 1);
        score(R0, rr);
        load(R0, rr + 2);
        score(R1, rr + 1);
      }
      if (rr + 1 < nr) {
        load(R1, rr + 1);
        score(R0, rr);
        score(R1, rr + 1);
      } else {
        score(R0, rr);
      }
    } else {
      for (int rr = 0; rr < nr; rr += 2) {
        load(R1, rr + 1);
        score(R0, rr);
        if (rr + 1 >= nr) break;
        load(R0, rr + 2);
        score(R1, rr + 1);
      }
    }
  }
  __syncthreads();
}

// Scores of entries [lo, hi) of row ri into keys[0 .. hi-lo).
// Inlined at both call sites (a call would pass the arguments through scratch
// memory).
template <int KK, bool PEEL = true>
__device__ __forceinline__ void score_slice(const IndexArgs& a, const RowInfo& ri, uint32_t* keys, float* s_q) {
  const int tid = threadIdx.x;
  const int64_t n = ri.hi - ri.lo;
  const int H_I = a.H_I, d_I = a.d_I;
  const int64_t qrow = (ri.b * a.T + ri.i) * H_I;
  if (KK == kKeyF32) {
    const float* q = reinterpret_cast<const float*>(a.q_idx) + qrow * d_I;
    for (int x = tid; x < H_I * d_I; x += kThreads) s_q[x] = q[x];
    if (tid < 16) s_q[16 * 64 + tid] = (tid < H_I) ? (a.w ? a.w[qrow + tid] : 1.0f) : 0.0f;
    __syncthreads();
    const float* kbase = reinterpret_cast<const float*>(a.k_idx) + (ri.b * a.N_alloc + ri.lo) * d_I;
    if (d_I == 32) {
      // The key row is loaded once (8 x 16 bytes).  Each head's dot product
      // runs four partial sums: one sequential chain of fused multiply-adds per
      // entry and head made this loop latency-bound (0.18 -> 0.07 ms for 4096
      // rows of up to 1024 entries, 4 heads x 32 dims).
      for (int64_t e = tid; e < n; e += kThreads) {
        const float4* kp = reinterpret_cast<const float4*>(kbase + e * 32);
        float4 kr[8];
#pragma unroll
        for (int v = 0; v < 8; ++v) kr[v] = kp[v];
        float score = 0.0f;
        for (int h = 0; h < H_I; ++h) {
          const float* qh = s_q + h * 32;
          float d0 = 0.0f, d1 = 0.0f, d2 = 0.0f, d3 = 0.0f;
#pragma unroll
          for (int v = 0; v < 8; ++v) {
            d0 = fmaf(qh[4 * v], kr[v].x, d0);
            d1 = fmaf(qh[4 * v + 1], kr[v].y, d1);
            d2 = fmaf(qh[4 * v + 2], kr[v].z, d2);
            d3 = fmaf(qh[4 * v + 3], kr[v].w, d3);
          }
          score = fmaf(s_q[16 * 64 + h], relu_nan((d0 + d1) + (d2 + d3)), score);
        }
        keys[e] = score_key(a.bf16_scores ? round_bf16(score) : score);
      }
    } else {
      for (int64_t e = tid; e < n; e += kThreads) {
        const float4* kp = reinterpret_cast<const float4*>(kbase + e * d_I);
        float score = 0.0f;
        for (int h = 0; h < H_I; ++h) {
          const float* qh = s_q + h * d_I;
          float d0 = 0.0f, d1 = 0.0f, d2 = 0.0f, d3 = 0.0f;
          for (int v = 0; v < d_I / 4; ++v) {
            const float4 x = kp[v];
            d0 = fmaf(qh[4 * v], x.x, d0);
            d1 = fmaf(qh[4 * v + 1], x.y, d1);
            d2 = fmaf(qh[4 * v + 2], x.z, d2);
            d3 = fmaf(qh[4 * v + 3], x.w, d3);
          }
          score = fmaf(s_q[16 * 64 + h], relu_nan((d0 + d1) + (d2 + d3)), score);
        }
        keys[e] = score_key(a.bf16_scores ? round_bf16(score) : score);
      }
    }
    __syncthreads();
    return;
  } else if (d_I == 64) {
    score_slice_mfma<KK, 64, PEEL>(a, ri, keys, qrow);
  } else {
    score_slice_mfma<KK, 32, PEEL>(a, ri, keys, qrow);
  }
}

// ---------------------------------------------------------------- radix selection
//
// Thresholds are found by MSB-first radix selection on 12-bit digits of the
// 64-bit rank keys (counting in a 4096-bin LDS histogram).  Rank keys of real
// entries are never 0, so 0 marks an empty register slot.

constexpr int kDigitBits = 12;
constexpr int kBins = 1 << kDigitBits;
constexpr int kRelBins = 1024;  // bins of the range-relative first pass

struct SelLds {
  uint32_t scan[kWaves];
  uint32_t misc[4];
  uint32_t lo[kWaves], hi[kWaves];
  uint64_t wb[kWaves];
  uint64_t res;
  uint64_t list[kThreads];  // keys of one histogram bin, ranked exactly
};

// After the histogram of the current digit is complete: pick the digit that
// holds the need-th largest key.  Returns (digit, keys above it, keys in it).
__device__ __forceinline__ void pick_digit(const uint32_t* hist, uint32_t nb, int64_t need, SelLds& S,
                                           uint32_t& dstar, uint32_t& above, uint32_t& in_digit) {
  const int tid = threadIdx.x;
  const uint32_t bpt = nb >= kThreads ? nb / kThreads : 1u;  // bins per thread
  const uint32_t nthr = nb / bpt;
  uint32_t local = 0;
  if (uint32_t(tid) < nthr)
    for (uint32_t j = 0; j < bpt; ++j) local += hist[nb - 1 - (tid * bpt + j)];
  const uint32_t inc = block_inclusive_sum(local, S.scan);
  const uint32_t ex = inc - local;
  if (uint32_t(tid) < nthr && int64_t(ex) < need && int64_t(inc) >= need) {
    uint32_t cum = ex;
    for (uint32_t j = 0; j < bpt; ++j) {
      const uint32_t dd = nb - 1 - (tid * bpt + j);
      const uint32_t h = hist[dd];
      if (int64_t(cum + h) >= need) {
        S.misc[0] = dd;
        S.misc[1] = cum;
        S.misc[2] = h;
        break;
      }
      cum += h;
    }
  }
  __syncthreads();
  dstar = S.misc[0];
  above = S.misc[1];
  in_digit = S.misc[2];
  __syncthreads();
}

// Threshold T with exactly `need` keys >= T among the non-zero keys (1 <= need <=
// their count; keys distinct).  Keys live in registers: KPT per thread.
template <int KPT>
__device__ __forceinline__ uint64_t select_regs(const uint64_t (&v)[KPT], int64_t need, uint32_t* hist, SelLds& S,
                                uint64_t prefix = 0, int hi_bit = 64) {
  const int tid = threadIdx.x;
  while (hi_bit > 0) {
    const int width = hi_bit >= kDigitBits ? kDigitBits : hi_bit;
    const int shift = hi_bit - width;
    const uint32_t nb = 1u << width;
    for (int x = tid; x < kBins; x += kThreads) hist[x] = 0;
    __syncthreads();
    const uint64_t hi_mask = (hi_bit >= 64) ? 0ull : (~0ull << hi_bit);
#pragma unroll
    for (int u = 0; u < KPT; ++u)
      if (v[u] != 0 && (v[u] & hi_mask) == prefix)
        atomicAdd(&hist[uint32_t(v[u] >> shift) & (nb - 1u)], 1u);
    __syncthreads();
    uint32_t dstar, above, in_digit;
    pick_digit(hist, nb, need, S, dstar, above, in_digit);
    prefix |= uint64_t(dstar) << shift;
    need -= int64_t(above);
    hi_bit = shift;
    if (int64_t(in_digit) == need) break;  // every key in this digit is selected
  }
  return prefix;  // remaining low bits zero
}

// The same threshold with a first pass whose 1024 bins span only the occupied
// range of the keys' upper halves (min .. max), which usually leaves a handful
// of keys in the bin of the need-th key.  Those are then ranked exactly against
// each other in LDS; finer radix passes follow only if the bin is crowded.
template <int KPT>
__device__ __forceinline__ uint64_t select_rel(const uint64_t (&v)[KPT], int64_t need, uint32_t* hist, SelLds& S) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
  for (int u = 0; u < KPT; ++u)
    if (v[u] != 0) {
      const uint32_t h = uint32_t(v[u] >> 32);
      lo = h < lo ? h : lo;
      hi = h > hi ? h : hi;
    }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (lane == 0) {
    S.lo[wid] = lo;
    S.hi[wid] = hi;
  }
  for (int x = tid; x < kRelBins; x += kThreads) hist[x] = 0;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    lo = min(lo, S.lo[w]);
    hi = max(hi, S.hi[w]);
  }
  int sh = 0;
  while ((hi >> sh) - (lo >> sh) >= uint32_t(kRelBins)) ++sh;
  const uint32_t base = lo >> sh;
#pragma unroll
  for (int u = 0; u < KPT; ++u)
    if (v[u] != 0) atomicAdd(&hist[((uint32_t(v[u] >> 32) >> sh) - base) & (kRelBins - 1)], 1u);
  __syncthreads();
  uint32_t dstar, above, in_digit;
  pick_digit(hist, kRelBins, need, S, dstar, above, in_digit);
  const int hi_bit = 32 + sh;
  const uint64_t top = uint64_t(base + dstar);
  const uint64_t prefix = top << hi_bit;
  need -= int64_t(above);
  if (int64_t(in_digit) == need) return prefix;
  if (in_digit > uint32_t(kThreads)) return select_regs(v, need, hist, S, prefix, hi_bit);
  int cnt = 0;
#pragma unroll
  for (int u = 0; u < KPT; ++u) cnt += (v[u] != 0 && (v[u] >> hi_bit) == top) ? 1 : 0;
  uint32_t pos = block_inclusive_sum(uint32_t(cnt), S.scan) - uint32_t(cnt);
#pragma unroll
  for (int u = 0; u < KPT; ++u)
    if (v[u] != 0 && (v[u] >> hi_bit) == top) S.list[pos++] = v[u];
  __syncthreads();
  if (uint32_t(tid) < in_digit) {
    const uint64_t key = S.list[tid];
    int64_t gt = 0;
#pragma unroll 8
    for (uint32_t j = 0; j < in_digit; ++j) gt += S.list[j] > key;
    if (gt == need - 1) S.res = key;
  }
  __syncthreads();
  const uint64_t T = S.res;
  __syncthreads();
  return T;
}

// The same selection over n keys produced by get(i) (used for long candidate lists).
template <typename Get>
__device__ __forceinline__ uint64_t select_get(int64_t n, int64_t need, Get get, uint32_t* hist, SelLds& S) {
  const int tid = threadIdx.x;
  uint64_t prefix = 0;
  int hi_bit = 64;
  while (hi_bit > 0) {
    const int width = hi_bit >= kDigitBits ? kDigitBits : hi_bit;
    const int shift = hi_bit - width;
    const uint32_t nb = 1u << width;
    for (int x = tid; x < kBins; x += kThreads) hist[x] = 0;
    __syncthreads();
    const uint64_t hi_mask = (hi_bit >= 64) ? 0ull : (~0ull << hi_bit);
    for (int64_t i = tid; i < n; i += kThreads) {
      const uint64_t v = get(i);
      if ((v & hi_mask) == prefix) atomicAdd(&hist[uint32_t(v >> shift) & (nb - 1u)], 1u);
    }
    __syncthreads();
    uint32_t dstar, above, in_digit;
    pick_digit(hist, nb, need, S, dstar, above, in_digit);
    prefix |= uint64_t(dstar) << shift;
    need -= int64_t(above);
    hi_bit = shift;
    if (int64_t(in_digit) == need) break;
  }
  return prefix;
}

// A lower bound of the need-th largest key, found without ranking the keys:
// in every wave, the ceil(need/4)-th largest of the lanes' maxima (the 64
// maxima ranked against each other in LDS); the smallest of the four is the
// bound (need distinct threads hold a key at or above it).  Returns 0 (no
// bound) when a wave has fewer non-empty lanes than its share, or when need
// exceeds 4 * 64.  scratch: kThreads uint64 of LDS, free on entry.
template <int KPT>
__device__ __forceinline__ uint64_t lane_max_bound(const uint64_t (&v)[KPT], int64_t need, uint64_t* scratch,
                                                   SelLds& S) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int jw = int((need + kWaves - 1) / kWaves);  // share of each wave
  if (jw > kWave) return 0ull;
  uint64_t* tmax = scratch;
  uint64_t mx = 0;
#pragma unroll
  for (int u = 0; u < KPT; ++u) mx = v[u] > mx ? v[u] : mx;
  tmax[tid] = mx;
  if (lane == 0) S.wb[wid] = 0ull;  // fewer than jw non-empty lanes: no bound
  __builtin_amdgcn_wave_barrier();
  if (mx != 0) {
    const uint64_t* wt = tmax + wid * kWave;
    int above = 0;
#pragma unroll
    for (int t = 0; t < kWave; t += 2) {
      const uint4 w = *reinterpret_cast<const uint4*>(&wt[t]);
      above += ((uint64_t(w.y) << 32 | w.x) > mx) + ((uint64_t(w.w) << 32 | w.z) > mx);
    }
    if (above == jw - 1) S.wb[wid] = mx;
  }
  __syncthreads();
  uint64_t B = S.wb[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) B = S.wb[w] < B ? S.wb[w] : B;
  __syncthreads();
  return B;
}

__device__ __forceinline__ void write_out(const IndexArgs& a, int64_t r, int64_t slot, uint64_t v) {
  a.out_idx[r * a.top_k + slot] = int32_t(rank_key_idx(v));
  if (a.out_score) a.out_score[r * a.top_k + slot] = key_score(uint32_t(v >> 32));
}

__device__ __forceinline__ void write_pads(const IndexArgs& a, int64_t r, int64_t from) {
  for (int64_t x = from + threadIdx.x; x < a.top_k; x += kThreads) {
    a.out_idx[r * a.top_k + x] = -1;
    if (a.out_score) a.out_score[r * a.top_k + x] = -INFINITY;
  }
}

// Emit the register keys >= T in thread order (all of thread 0's, then thread
// 1's, ...); dst(pos, v) stores one.
template <int KPT, typename Dst>
__device__ __forceinline__ void emit_regs(const uint64_t (&v)[KPT], uint64_t T, int64_t from, Dst dst, uint32_t* s_scan) {
  int cnt = 0;
#pragma unroll
  for (int u = 0; u < KPT; ++u) cnt += (v[u] != 0 && v[u] >= T) ? 1 : 0;
  int64_t pos = from + int64_t(block_inclusive_sum(uint32_t(cnt), s_scan)) - cnt;
#pragma unroll
  for (int u = 0; u < KPT; ++u)
    if (v[u] != 0 && v[u] >= T) dst(pos++, v[u]);
}

// Exact top-kl of a slice's keys (kl < number of keys), written to
// dst[0 .. kl) in decreasing order with device-scope stores; returns the
// kl-th key: every key not written ranks below it.  The keys at or above
// lane_max_bound (usually a few more than kl) are ranked exactly against each
// other in LDS, and each writes itself at its rank; when more than kThreads
// keys reach the bound, a radix select finds the threshold instead and the
// winners are written in thread order.
template <int KPT>
__device__ __forceinline__ uint64_t local_topk(const uint64_t (&v)[KPT], int kl, uint64_t* dst, uint64_t* scratch, uint32_t* hist,
                               SelLds& S) {
  const int tid = threadIdx.x;
  const uint64_t B = lane_max_bound(v, kl, scratch, S);
  int cnt = 0;
#pragma unroll
  for (int u = 0; u < KPT; ++u) cnt += (v[u] != 0 && v[u] >= B) ? 1 : 0;
  const uint32_t inc = block_inclusive_sum(uint32_t(cnt), S.scan);
  if (tid == kThreads - 1) S.misc[3] = inc;
  __syncthreads();
  const uint32_t m = S.misc[3];
  if (m > uint32_t(kThreads)) {
    const uint64_t T = select_rel(v, kl, hist, S);
    emit_regs(v, T, 0, [&](int64_t pos, uint64_t val) { store_dev(&dst[pos], val); }, S.scan);
    return T;
  }
  uint32_t pos = inc - uint32_t(cnt);
#pragma unroll
  for (int u = 0; u < KPT; ++u)
    if (v[u] != 0 && v[u] >= B) S.list[pos++] = v[u];
  __syncthreads();
  if (uint32_t(tid) < m) {
    const uint64_t key = S.list[tid];
    int rank = 0;
#pragma unroll 8
    for (uint32_t j = 0; j < m; ++j) rank += S.list[j] > key;
    if (rank < kl) store_dev(&dst[rank], key);
    if (rank == kl - 1) S.res = key;
  }
  __syncthreads();
  const uint64_t T = S.res;
  __syncthreads();
  return T;
}

template <typename Get, typename Dst>
__device__ __forceinline__ int64_t emit_get(int64_t n, uint64_t T, Get get, int64_t from, Dst dst, int* s_wave) {
  int64_t done = from;
  for (int64_t x0 = 0; x0 < n; x0 += kThreads) {
    const int64_t x = x0 + threadIdx.x;
    const uint64_t v = x < n ? get(x) : 0ull;
    const bool win = x < n && v >= T;
    int total;
    const int pos = block_rank(win, s_wave, total);
    if (win) dst(done + pos, v);
    done += total;
  }
  return done - from;
}

constexpr int kCandPerThread = 16;                    // last-WG register capacity

struct LdsIdx {
  uint32_t keys[kMaxSlice];  // slice keys, then the radix histogram (kBins == kMaxSlice)
  float q[16 * 64 + 16];
  SelLds sel;
  int wave[kWaves];
  uint32_t flag[4];
};
static_assert(kBins == kMaxSlice, "the key buffer doubles as the histogram");

// KPT: slice keys per thread (slice <= KPT * kThreads).
// (At most 256 registers, so that two workgroups share a CU.)
template <int KK, int KPT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void idx_topk_kernel(
    IndexArgs a, IndexPlan p, int64_t row0) {
  __shared__ LdsIdx L;
  debug_poison_lds(L);
  const int64_t lr = div64(blockIdx.x, p.slices);  // row within this launch
  const int64_t r = row0 + lr;
  const int64_t s = blockIdx.x - lr * p.slices;
  const RowInfo ri = row_info(a, p, r, s);
  if (s >= ri.S) return;
  const int tid = threadIdx.x;
  const int64_t n = ri.hi - ri.lo;

  score_slice<KK, (KPT <= 8)>(a, ri, L.keys, L.q);
  const uint32_t base = uint32_t(ri.lo);
  uint64_t v[KPT];  // thread tid: slice elements tid + 256 u
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    const int64_t x = tid + int64_t(u) * kThreads;
    v[u] = x < n ? rank_key(L.keys[x], base + uint32_t(x)) : 0ull;
  }
  __syncthreads();  // L.keys is the histogram (or selection scratch) from here on
  auto out_dst = [&](int64_t pos, uint64_t val) { write_out(a, r, pos, val); };

  if (ri.S == 1) {  // the whole row is in this WG
    if (ri.kk > 0) {
      const uint64_t T = (ri.kk < n) ? select_rel(v, ri.kk, L.keys, L.sel) : 1ull;
      emit_regs(v, T, 0, out_dst, L.sel.scan);
    }
    write_pads(a, r, ri.kk);
    return;
  }

  // ---- several slices.  Each hands over its exact local top-kloc, in
  // decreasing order, and a certificate: every entry of the slice left off
  // the list ranks below the certificate.  Lists are dense (kloc slots per
  // slice; a short slice pads with zeros) and written with device-scope
  // stores.
  uint8_t* ws = reinterpret_cast<uint8_t*>(a.ws);
  RowCtrl* ctrl = reinterpret_cast<RowCtrl*>(ws + kIndexCtrlOff) + lr;
  uint64_t* cand = reinterpret_cast<uint64_t*>(ws + p.off_cand) + lr * p.cand_row;
  uint64_t* tau = reinterpret_cast<uint64_t*>(ws + p.off_tau) + lr * p.slices;
  uint64_t* over = reinterpret_cast<uint64_t*>(ws + p.off_over) + lr * a.N_alloc;
  const int kl = int(ri.kloc);
  uint64_t* my_cand = cand + s * kl;
  uint64_t cert = 0;  // 0: the whole slice is listed
  if (n > kl) {
    cert = local_topk(v, kl, my_cand, reinterpret_cast<uint64_t*>(L.keys), L.keys, L.sel);
  } else {
    emit_regs(v, 1ull, 0, [&](int64_t pos, uint64_t val) { store_dev(&my_cand[pos], val); }, L.sel.scan);
    for (int64_t x = n + tid; x < kl; x += kThreads) store_dev(&my_cand[x], uint64_t(0));
  }
  if (tid == 0) store_dev(&tau[s], cert);
  if (!arrive_last(&ctrl->arrive, uint32_t(ri.S), L.flag)) return;

  // ---- last WG of the row: the lists of every slice (S * kloc slots in
  // element order, zeros for the padding of a short slice) and the
  // certificates, loaded in one batch, then the exact selection of the kk best.
  const int64_t total = ri.S * int64_t(kl);
  auto get_c = [&](int64_t g) { return load_dev(&cand[g]); };
  const bool in_regs = total <= int64_t(kCandPerThread) * kThreads;
  uint64_t c[kCandPerThread];
  uint64_t tmax_cert = 0;  // largest certificate (its slice may hold more winners iff it is above T)
  uint64_t T;
  if (in_regs) {
#pragma unroll
    for (int u = 0; u < kCandPerThread; ++u) {
      const int64_t g = int64_t(u) * kThreads + tid;  // element order: coalesced loads
      c[u] = g < total ? get_c(g) : 0ull;
    }
    for (int64_t x = tid; x < ri.S; x += kThreads) {
      const uint64_t tx = load_dev(&tau[x]);
      tmax_cert = tx > tmax_cert ? tx : tmax_cert;
    }
    T = select_rel(c, ri.kk, L.keys, L.sel);
  } else {
    for (int64_t x = tid; x < ri.S; x += kThreads) {
      const uint64_t tx = load_dev(&tau[x]);
      tmax_cert = tx > tmax_cert ? tx : tmax_cert;
    }
    T = select_get(total, ri.kk, get_c, L.keys, L.sel);
  }
  if (!__syncthreads_or(tmax_cert > T)) {
    if (in_regs) emit_regs(c, T, 0, out_dst, L.sel.scan);
    else emit_get(total, T, get_c, 0, out_dst, L.wave);
    write_pads(a, r, ri.kk);
    if (tid == 0) ctrl->arrive = 0;
    return;
  }
  // Rare path: rescore every slice whose certificate is above T and add the
  // entries it dropped that reach T, then select again over everything.
  int64_t n_over = 0;
  for (int64_t x = 0; x < ri.S; ++x) {
    const uint64_t tx = load_dev(&tau[x]);
    if (tx <= T) continue;
    RowInfo rx = row_info(a, p, r, x);
    score_slice<KK, (KPT <= 8)>(a, rx, L.keys, L.q);
    const uint32_t bx = uint32_t(rx.lo);
    const int64_t nx = rx.hi - rx.lo;
    for (int64_t y0 = 0; y0 < nx; y0 += kThreads) {
      const int64_t y = y0 + tid;
      const uint64_t val = y < nx ? rank_key(L.keys[y], bx + uint32_t(y)) : 0ull;
      const bool add = y < nx && val >= T && val < tx;
      int cnt;
      const int pos = block_rank(add, L.wave, cnt);
      if (add) over[n_over + pos] = val;
      n_over += cnt;
    }
    __syncthreads();
  }
  auto get_all = [&](int64_t g) { return g < total ? get_c(g) : over[g - total]; };
  T = select_get(total + n_over, ri.kk, get_all, L.keys, L.sel);
  emit_get(total + n_over, T, get_all, 0, out_dst, L.wave);
  write_pads(a, r, ri.kk);
  if (tid == 0) ctrl->arrive = 0;
}

}  // namespace

IndexPlan plan_index(int B, int64_t T, int H_I, int d_I, int64_t N_alloc, int top_k, int key_kind) {
  IndexPlan p{};
  p.rows = int64_t(B) * T;
  if (prefill_path(T, H_I, key_kind) && N_alloc > 0) {
    p.prefill = true;
    // Room for a full LDS staging area (the 1216 pairs of one wave, all of
    // which may belong to one query) above the 5k/4 keys a compaction may keep:
    // 5k/4 + 1216 <= max(4096, 2k + 512) for every k <= 2048.
    static_assert(5 * 2048 / 4 + kPrefillStage <= 2 * 2048 + 512, "staging room at k = 2048");
    static_assert(5 * 1792 / 4 + kPrefillStage <= 4096, "staging room at 2k + 512 = 4096");
    p.cap = 4096;
    if (p.cap < 2 * int64_t(top_k) + 512) p.cap = 2 * int64_t(top_k) + 512;
    p.off_cand = kHeaderBytes;
    p.ws_bytes = kHeaderBytes + size_t(p.rows) * size_t(p.cap) * 8;
    return p;
  }
  p.c_max = N_alloc;
  // At most about 512 workgroups over the chip (256 CUs), and slices of at
  // least 128 KB of keys: a workgroup streaming less spends more on its share
  // of the selection tail than on the stream (measured: the Flash-like decode,
  // 33.5 MB of bf16 keys, takes 18.9 us in 512 slices, 17.2 us in 256 and
  // 20.5 us in 128).  Slices hold 256..4096 entries.
  const int64_t dk = d_I > 0 ? d_I : 1;
  const int64_t entry_bytes = key_kind == kKeyF32 ? 4 * dk : key_kind == kKeyBF16 ? 2 * dk : dk + 4;
  int64_t want = (p.rows > 0) ? (p.c_max * p.rows + 511) / 512 : 1;
  if (want < (int64_t(128) << 10) / entry_bytes) want = (int64_t(128) << 10) / entry_bytes;
  int64_t slice = ((want + 255) / 256) * 256;
  if (slice < 256) slice = 256;
  if (slice > kMaxSlice) slice = kMaxSlice;
  // No longer than the longest row needs: the registers per thread follow the
  // slice, and keys past the row's end are dead weight in every selection pass.
  const int64_t c_round = ((p.c_max + 255) / 256) * 256;
  if (slice > c_round && c_round >= 256) slice = c_round;
  p.slice = slice;
  p.slices = (p.c_max + slice - 1) / slice;
  if (p.slices < 1) p.slices = 1;
  const bool multi = p.slices > 1;
  p.chunk_rows = multi ? (p.rows < kIndexChunkRows ? p.rows : kIndexChunkRows) : p.rows;
  size_t off = kHeaderBytes;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (bytes + 255) & ~size_t(255);
    return o;
  };
  const size_t R = size_t(p.chunk_rows);
  // Candidate slots of a row: kloc per slice, and S * kloc <= c + slice.
  p.cand_row = N_alloc + p.slice;
  p.off_cand = take(R * size_t(p.cand_row) * 8);
  p.off_tau = take(R * size_t(p.slices) * 8);
  p.off_over = take(R * size_t(N_alloc) * 8);
  p.ws_bytes = multi ? off : 0;
  return p;
}

// Registers sized to the slice: 2, 4, 8 or 16 keys per thread.
template <int KK>
static void launch_kpt(const IndexArgs& a, const IndexPlan& p, int64_t row0, dim3 grid, dim3 block) {
  const int64_t kpt = (p.slice + kThreads - 1) / kThreads;
  if (kpt <= 2) hipLaunchKernelGGL((idx_topk_kernel<KK, 2>), grid, block, 0, a.stream, a, p, row0);
  else if (kpt <= 4) hipLaunchKernelGGL((idx_topk_kernel<KK, 4>), grid, block, 0, a.stream, a, p, row0);
  else if (kpt <= 8) hipLaunchKernelGGL((idx_topk_kernel<KK, 8>), grid, block, 0, a.stream, a, p, row0);
  else hipLaunchKernelGGL((idx_topk_kernel<KK, 16>), grid, block, 0, a.stream, a, p, row0);
}

hipError_t launch_index_topk(const IndexArgs& a, const IndexPlan& p) {
  if (p.rows == 0) return hipSuccess;
  static const char* const kKinds[] = {"f32", "bf16", "e4m3", "e4m3 (fp8 query)"};
  log_dispatch("index_topk: B=%d T=%lld H_I=%d d_I=%d N=%lld k=%d keys=%s%s -> %s path, ws %zu B", a.B,
               (long long)a.T, a.H_I, a.d_I, (long long)a.N_alloc, a.top_k, kKinds[a.key_kind & 3],
               a.bf16_scores ? " bf16 scores" : "", p.prefill ? "prefill" : "rows x slices", p.ws_bytes);
  CSA_HOST_CHECK(p.ws_bytes == 0 || a.ws != nullptr);
  if (kDebug && p.ws_bytes > kHeaderBytes) {
    const hipError_t e = debug_poison(static_cast<uint8_t*>(a.ws) + kHeaderBytes, p.ws_bytes - kHeaderBytes, a.stream);
    if (e != hipSuccess) return e;
  }
  if (p.prefill) return launch_index_prefill(a, p);
  CSA_HOST_CHECK(p.slice >= 256 && p.slice <= kMaxSlice && p.slice % 256 == 0);
  CSA_HOST_CHECK(p.slices >= 1 && p.slices * p.slice >= p.c_max);
  CSA_HOST_CHECK(p.slices == 1 || (p.off_over + size_t(p.chunk_rows) * size_t(a.N_alloc) * 8 <= p.ws_bytes &&
                                   p.off_cand >= kHeaderBytes && p.chunk_rows <= kIndexChunkRows));
  log_dispatch("index_topk: %lld rows, %lld slices of %lld entries, %lld rows per launch", (long long)p.rows,
               (long long)p.slices, (long long)p.slice, (long long)p.chunk_rows);
  const dim3 block(kThreads);
  for (int64_t row0 = 0; row0 < p.rows; row0 += p.chunk_rows) {
    const int64_t nr = (p.rows - row0) < p.chunk_rows ? (p.rows - row0) : p.chunk_rows;
    const dim3 grid(unsigned(nr * p.slices));
    ProfScope prof("index_topk", a.stream);
    if (a.key_kind == kKeyF32) launch_kpt<kKeyF32>(a, p, row0, grid, block);
    else if (a.key_kind == kKeyBF16) launch_kpt<kKeyBF16>(a, p, row0, grid, block);
    else if (a.key_kind == kKeyE4M3) launch_kpt<kKeyE4M3>(a, p, row0, grid, block);
    else launch_kpt<kKeyE4M3Q8>(a, p, row0, grid, block);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace csa

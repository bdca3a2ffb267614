// CSA / HCA attention with the raw sliding window under one softmax, for gfx950.
//
// V4 report digest, section 三: CSA attends to the top-k compressed entries, HCA
// to every heavy entry, and both add the newest window tokens uncompressed.  For
// query row r (position t) the slot list is
//     CSA: idx[r, 0..k)          (skipped unless 0 <= j < min(N, (t+1)/m))
//     HCA: heavy entries 0 .. min(N, (t+1)/m')
//     then raw positions max(0, t-W+1) .. t
// and every head h computes o = softmax(scale * q_h . K) V over all slots.
//
// One workgroup handles a contiguous range of slots ("split") of one row for
// all heads: all query heads share the one KV head, so a K/V row fetched once
// feeds every head.  bf16 path: 32-slot tiles are gathered into LDS (K
// row-major, V transposed); S^T = K Q^T on 16x16x32 MFMA puts one head per
// lane column and 8 slots per lane, which is exactly the B-operand layout of
// O^T = V^T P^T, so the softmax weights never move between lanes.  P enters
// the MFMA as a bf16 hi + lo pair (16 significant bits).  fp32 path: fp32 FMA,
// one slot per lane.  With several splits, each writes (O, max, sum) partials
// and the last split of the row to finish merges them (log-sum-exp).
#include "common.hpp"
#include "kernels.h"

namespace csa {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 32;           // bf16 slots per tile
constexpr int kTileF32 = 64;        // fp32 slots per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct RowSlots {
  int64_t r, b, t, c, wstart, wn, L, lo, hi, S;
};

__device__ __forceinline__ RowSlots row_slots(const AttendArgs& a, const AttendPlan& p, int64_t r,
                                              int64_t s) {
  RowSlots x;
  x.r = r;
  x.b = r / a.T;
  x.t = a.t0 + r % a.T;
  int64_t c = (x.t + 1) / a.m;
  x.c = c < a.N_alloc ? c : a.N_alloc;
  int64_t ws = x.t - a.window + 1;
  x.wstart = ws > 0 ? ws : 0;
  x.wn = x.t - x.wstart + 1;
  if (a.window == 0) x.wn = 0;
  x.L = (a.hca ? x.c : int64_t(a.top_k)) + x.wn;
  int64_t S = (x.L + p.per_split - 1) / p.per_split;
  x.S = S < 1 ? 1 : S;
  x.lo = s * p.per_split;
  int64_t hi = x.lo + p.per_split;
  x.hi = hi < x.L ? hi : x.L;
  if (x.hi < x.lo) x.hi = x.lo;
  return x;
}

// Source row of slot `slot`, or null when the slot is skipped.
template <typename T>
__device__ __forceinline__ const T* slot_row(const AttendArgs& a, const RowSlots& x, int64_t slot,
                                             bool value) {
  const T* cmp = reinterpret_cast<const T*>(value ? a.v_cmp : a.k_cmp);
  const T* raw = reinterpret_cast<const T*>(value ? a.v_raw : a.k_raw);
  const int64_t nsel = a.hca ? x.c : int64_t(a.top_k);
  if (slot < nsel) {
    int64_t j = slot;
    if (!a.hca) {
      j = a.idx[x.r * a.top_k + slot];
      if (j < 0 || j >= x.c) return nullptr;
    }
    return cmp + (x.b * a.N_alloc + j) * a.d;
  }
  const int64_t pos = x.wstart + (slot - nsel);
  return raw + (x.b * a.n_raw + (pos - a.raw_base)) * a.d;
}

struct SplitCtrl {
  uint32_t arrive;
  uint32_t pad[3];
};

// Merge the S partials of row r (all heads) and write out / lse.
// part: [S][H][d] un-normalised O; ml: [S][H][2] (max in log2 units, sum).
__device__ void merge_row(const AttendArgs& a, const float* part, const float* ml, int64_t S,
                          int64_t r) {
  const int H = a.H, d = a.d;
  for (int x = threadIdx.x; x < H * d; x += kThreads) {
    const int h = x / d;
    float M = -INFINITY;
    for (int64_t s = 0; s < S; ++s) M = fmaxf(M, ml[(s * H + h) * 2]);
    float Lsum = 0.0f, O = 0.0f;
    if (M != -INFINITY) {
      for (int64_t s = 0; s < S; ++s) {
        const float ms = ml[(s * H + h) * 2];
        const float f = exp2f(ms - M);  // 0 for empty splits (ms = -inf)
        Lsum = fmaf(f, ml[(s * H + h) * 2 + 1], Lsum);
        O = fmaf(f, part[(s * H + h) * int64_t(d) + (x - h * d)], O);
      }
    }
    const float o = (Lsum > 0.0f) ? O / Lsum : 0.0f;
    const int64_t oi = (r * H + h) * int64_t(d) + (x - h * d);
    if (a.out_bf16) reinterpret_cast<bf16_t*>(a.out)[oi] = f32_to_bf16(o);
    else reinterpret_cast<float*>(a.out)[oi] = o;
    if (a.lse && x - h * d == 0) a.lse[r * H + h] = (Lsum > 0.0f) ? (M + log2f(Lsum)) * kLn2 : -INFINITY;
  }
}

// Publish this split's partials; the last split of the row merges.  Returns
// after the merge (or immediately for non-last splits).
__device__ void finish_split(const AttendArgs& a, const AttendPlan& p, const RowSlots& x, int64_t s,
                             uint32_t* s_flag) {
  uint8_t* ws = reinterpret_cast<uint8_t*>(a.ws);
  SplitCtrl* ctrl = reinterpret_cast<SplitCtrl*>(ws + kAttendCtrlOff) + x.r;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_flag[0] = (atomicAdd(&ctrl->arrive, 1u) == uint32_t(x.S - 1)) ? 1u : 0u;
  __syncthreads();
  if (!s_flag[0]) return;
  __threadfence();
  const float* part = reinterpret_cast<const float*>(ws + p.off_part) + x.r * p.splits * a.H * a.d;
  const float* ml = reinterpret_cast<const float*>(ws + p.off_ml) + x.r * p.splits * a.H * 2;
  merge_row(a, part, ml, x.S, x.r);
  if (threadIdx.x == 0) ctrl->arrive = 0;
}

// ---------------------------------------------------------------- bf16 MFMA kernel

template <int D>
struct LdsBF16 {
  bf16_t k[kTile][D + 8];   // row-major K tile (padded rows)
  bf16_t vt[D][kTile + 8];  // transposed V tile
  uint32_t flag[4];
};

template <int D>
__global__ __launch_bounds__(kThreads) void attend_bf16_kernel(AttendArgs a, AttendPlan p) {
  __shared__ LdsBF16<D> L;
  const int64_t r = blockIdx.x / p.splits;
  const int64_t s = blockIdx.x % p.splits;
  const RowSlots x = row_slots(a, p, r, s);
  if (s >= x.S) return;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, g = lane >> 4, col = lane & 15;
  const int H = a.H;
  const int NG = H / 16;  // head groups of 16
  constexpr int KS = D / 32;   // k-steps of the QK product
  constexpr int DVT = D / 16;  // 16-column tiles of the output
  // This wave's head groups: wid and wid + 4.
  const int hg0 = wid, hg1 = wid + 4;
  const bool has0 = hg0 < NG, has1 = hg1 < NG;

  bf16x8_t qb[2][KS];
  const bf16_t* qrow = reinterpret_cast<const bf16_t*>(a.q) + r * int64_t(H) * D;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int hg = u == 0 ? hg0 : hg1;
    const bool has = u == 0 ? has0 : has1;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (has) v = *reinterpret_cast<const uint4*>(qrow + (hg * 16 + col) * D + 32 * kk + 8 * g);
      qb[u][kk] = u32x4_as_bf16x8(v);
    }
  }
  const float sl2 = a.scale * kLog2e;
  f32x4_t o[2][DVT];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < DVT; ++v) o[u][v] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float mrun[2] = {-INFINITY, -INFINITY};
  float lpart[2] = {0.0f, 0.0f};

  constexpr int CPR = D / 8;  // 16-byte chunks per row
  for (int64_t t0 = x.lo; t0 < x.hi; t0 += kTile) {
    // Gather the K / V rows of 32 slots into LDS.
    for (int c = tid; c < kTile * CPR; c += kThreads) {
      const int sl = c / CPR, ch = c % CPR;
      const int64_t slot = t0 + sl;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (slot < x.hi) {
        const bf16_t* kr = slot_row<bf16_t>(a, x, slot, false);
        if (kr) {
          const bf16_t* vr = slot_row<bf16_t>(a, x, slot, true);
          kv = *reinterpret_cast<const uint4*>(kr + ch * 8);
          vv = *reinterpret_cast<const uint4*>(vr + ch * 8);
        }
      }
      *reinterpret_cast<uint4*>(&L.k[sl][ch * 8]) = kv;
      const uint32_t w4[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        L.vt[ch * 8 + 2 * i][sl] = bf16_t(w4[i] & 0xffffu);
        L.vt[ch * 8 + 2 * i + 1][sl] = bf16_t(w4[i] >> 16);
      }
    }
    __syncthreads();
    // Which of this tile's slots are live (lane-independent per slot index).
    bool live[2][4];
#pragma unroll
    for (int cg = 0; cg < 2; ++cg)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t slot = t0 + cg * 16 + 4 * g + j;
        live[cg][j] = slot < x.hi && slot_row<bf16_t>(a, x, slot, false) != nullptr;
      }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (!(u == 0 ? has0 : has1)) continue;
      f32x4_t sc[2];
#pragma unroll
      for (int cg = 0; cg < 2; ++cg) {
        f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          const uint4 kv = *reinterpret_cast<const uint4*>(&L.k[cg * 16 + col][32 * kk + 8 * g]);
          acc = mfma16x16x32(u32x4_as_bf16x8(kv), qb[u][kk], acc);
        }
        sc[cg] = acc;
      }
      // Online softmax in log2 units; lane holds head (16*hg + col), 8 slots.
      float tmax = -INFINITY;
#pragma unroll
      for (int cg = 0; cg < 2; ++cg)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float v = live[cg][j] ? sc[cg][j] * sl2 : -INFINITY;
          sc[cg][j] = v;
          tmax = fmaxf(tmax, v);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float mnew = fmaxf(mrun[u], tmax);
      const float corr = (mnew == -INFINITY) ? 1.0f : exp2f(mrun[u] - mnew);
      mrun[u] = mnew;
      float psum = 0.0f;
      uint32_t phi[4], plo[4];
#pragma unroll
      for (int cg = 0; cg < 2; ++cg)
#pragma unroll
        for (int j = 0; j < 4; j += 2) {
          float p0 = (mnew == -INFINITY) ? 0.0f : exp2f(sc[cg][j] - mnew);
          float p1 = (mnew == -INFINITY) ? 0.0f : exp2f(sc[cg][j + 1] - mnew);
          psum += p0 + p1;
          const bf16_t h0 = f32_to_bf16(p0), h1 = f32_to_bf16(p1);
          const bf16_t l0 = f32_to_bf16(p0 - bf16_to_f32(h0));
          const bf16_t l1 = f32_to_bf16(p1 - bf16_to_f32(h1));
          phi[cg * 2 + j / 2] = uint32_t(h0) | (uint32_t(h1) << 16);
          plo[cg * 2 + j / 2] = uint32_t(l0) | (uint32_t(l1) << 16);
        }
      lpart[u] = lpart[u] * corr + psum;
      const bf16x8_t pb_hi = u32x4_as_bf16x8(make_uint4(phi[0], phi[1], phi[2], phi[3]));
      const bf16x8_t pb_lo = u32x4_as_bf16x8(make_uint4(plo[0], plo[1], plo[2], plo[3]));
#pragma unroll
      for (int v = 0; v < DVT; ++v) {
        f32x4_t acc = o[u][v];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] *= corr;
        const uint2 a0 = *reinterpret_cast<const uint2*>(&L.vt[v * 16 + col][4 * g]);
        const uint2 a1 = *reinterpret_cast<const uint2*>(&L.vt[v * 16 + col][16 + 4 * g]);
        const bf16x8_t va = u32x4_as_bf16x8(make_uint4(a0.x, a0.y, a1.x, a1.y));
        acc = mfma16x16x32(va, pb_hi, acc);
        acc = mfma16x16x32(va, pb_lo, acc);
        o[u][v] = acc;
      }
    }
    __syncthreads();
  }

  // Per-head totals; lane (g, col) holds head 16*hg+col, dv = 16v + 4g + j.
  float lt[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    float v = lpart[u];
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    lt[u] = v;
  }
  if (x.S == 1) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (!(u == 0 ? has0 : has1)) continue;
      const int h = (u == 0 ? hg0 : hg1) * 16 + col;
      const float inv = lt[u] > 0.0f ? 1.0f / lt[u] : 0.0f;
#pragma unroll
      for (int v = 0; v < DVT; ++v) {
        const int64_t oi = (r * H + h) * int64_t(D) + v * 16 + 4 * g;
        if (a.out_bf16) {
          uint32_t w0 = uint32_t(f32_to_bf16(o[u][v][0] * inv)) | (uint32_t(f32_to_bf16(o[u][v][1] * inv)) << 16);
          uint32_t w1 = uint32_t(f32_to_bf16(o[u][v][2] * inv)) | (uint32_t(f32_to_bf16(o[u][v][3] * inv)) << 16);
          *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(a.out) + oi) = make_uint2(w0, w1);
        } else {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + oi) =
              make_float4(o[u][v][0] * inv, o[u][v][1] * inv, o[u][v][2] * inv, o[u][v][3] * inv);
        }
      }
      if (a.lse && g == 0)
        a.lse[r * H + h] = lt[u] > 0.0f ? (mrun[u] + log2f(lt[u])) * kLn2 : -INFINITY;
    }
    return;
  }
  uint8_t* ws = reinterpret_cast<uint8_t*>(a.ws);
  float* part = reinterpret_cast<float*>(ws + p.off_part) + (r * p.splits + s) * int64_t(H) * D;
  float* ml = reinterpret_cast<float*>(ws + p.off_ml) + (r * p.splits + s) * int64_t(H) * 2;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if (!(u == 0 ? has0 : has1)) continue;
    const int h = (u == 0 ? hg0 : hg1) * 16 + col;
#pragma unroll
    for (int v = 0; v < DVT; ++v)
      *reinterpret_cast<float4*>(part + int64_t(h) * D + v * 16 + 4 * g) =
          make_float4(o[u][v][0], o[u][v][1], o[u][v][2], o[u][v][3]);
    if (g == 0) {
      ml[h * 2] = mrun[u];
      ml[h * 2 + 1] = lt[u];
    }
  }
  finish_split(a, p, x, s, L.flag);
}

// ---------------------------------------------------------------- fp32 kernel

template <int D>
struct LdsF32 {
  float k[kTileF32][D + 1];
  float v[kTileF32][D];
  float q[32][D];
  float pr[32][kTileF32];
  uint32_t flag[4];
};

template <int D>
__global__ __launch_bounds__(kThreads) void attend_f32_kernel(AttendArgs a, AttendPlan p) {
  __shared__ LdsF32<D> L;
  const int64_t r = blockIdx.x / p.splits;
  const int64_t s = blockIdx.x % p.splits;
  const RowSlots x = row_slots(a, p, r, s);
  if (s >= x.S) return;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int H = a.H;
  constexpr int DPL = (D + 63) / 64;  // output columns per lane
  const float* qrow = reinterpret_cast<const float*>(a.q) + r * int64_t(H) * D;
  for (int i = tid; i < H * D; i += kThreads) L.q[i / D][i % D] = qrow[i];
  const float sl2 = a.scale * kLog2e;
  float o[8][DPL];
  float mrun[8], lpart[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    mrun[u] = -INFINITY;
    lpart[u] = 0.0f;
#pragma unroll
    for (int c = 0; c < DPL; ++c) o[u][c] = 0.0f;
  }
  for (int64_t t0 = x.lo; t0 < x.hi; t0 += kTileF32) {
    __syncthreads();
    for (int i = tid; i < kTileF32 * (D / 4); i += kThreads) {
      const int sl = i / (D / 4), ch = i % (D / 4);
      const int64_t slot = t0 + sl;
      float4 kv = make_float4(0, 0, 0, 0), vv = make_float4(0, 0, 0, 0);
      if (slot < x.hi) {
        const float* kr = slot_row<float>(a, x, slot, false);
        if (kr) {
          kv = *reinterpret_cast<const float4*>(kr + ch * 4);
          vv = *reinterpret_cast<const float4*>(slot_row<float>(a, x, slot, true) + ch * 4);
        }
      }
      L.k[sl][ch * 4] = kv.x; L.k[sl][ch * 4 + 1] = kv.y; L.k[sl][ch * 4 + 2] = kv.z; L.k[sl][ch * 4 + 3] = kv.w;
      *reinterpret_cast<float4*>(&L.v[sl][ch * 4]) = vv;
    }
    __syncthreads();
    const int64_t slot = t0 + lane;
    const bool live = slot < x.hi && slot_row<float>(a, x, slot, false) != nullptr;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int h = wid + 4 * u;
      if (h >= H) break;
      float dot = 0.0f;
      for (int dd = 0; dd < D; ++dd) dot = fmaf(L.q[h][dd], L.k[lane][dd], dot);
      const float sv = live ? dot * sl2 : -INFINITY;
      const float mnew = fmaxf(mrun[u], wave_max(sv));
      const float corr = (mnew == -INFINITY) ? 1.0f : exp2f(mrun[u] - mnew);
      const float pv = (mnew == -INFINITY) ? 0.0f : exp2f(sv - mnew);
      mrun[u] = mnew;
      lpart[u] = lpart[u] * corr + pv;
      L.pr[h][lane] = pv;
#pragma unroll
      for (int c = 0; c < DPL; ++c) o[u][c] *= corr;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int h = wid + 4 * u;
      if (h >= H) break;
#pragma unroll
      for (int c = 0; c < DPL; ++c) {
        const int dv = lane + 64 * c;
        if (dv >= D) continue;
        float acc = o[u][c];
        for (int e = 0; e < kTileF32; ++e) acc = fmaf(L.pr[h][e], L.v[e][dv], acc);
        o[u][c] = acc;
      }
    }
  }
  float lt[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) lt[u] = wave_sum(lpart[u]);
  if (x.S == 1) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int h = wid + 4 * u;
      if (h >= H) break;
      const float inv = lt[u] > 0.0f ? 1.0f / lt[u] : 0.0f;
#pragma unroll
      for (int c = 0; c < DPL; ++c) {
        const int dv = lane + 64 * c;
        if (dv >= D) continue;
        const int64_t oi = (r * H + h) * int64_t(D) + dv;
        if (a.out_bf16) reinterpret_cast<bf16_t*>(a.out)[oi] = f32_to_bf16(o[u][c] * inv);
        else reinterpret_cast<float*>(a.out)[oi] = o[u][c] * inv;
      }
      if (a.lse && lane == 0)
        a.lse[r * H + h] = lt[u] > 0.0f ? (mrun[u] + log2f(lt[u])) * kLn2 : -INFINITY;
    }
    return;
  }
  uint8_t* ws = reinterpret_cast<uint8_t*>(a.ws);
  float* part = reinterpret_cast<float*>(ws + p.off_part) + (r * p.splits + s) * int64_t(H) * D;
  float* ml = reinterpret_cast<float*>(ws + p.off_ml) + (r * p.splits + s) * int64_t(H) * 2;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int h = wid + 4 * u;
    if (h >= H) break;
#pragma unroll
    for (int c = 0; c < DPL; ++c) {
      const int dv = lane + 64 * c;
      if (dv < D) part[int64_t(h) * D + dv] = o[u][c];
    }
    if (lane == 0) {
      ml[h * 2] = mrun[u];
      ml[h * 2 + 1] = lt[u];
    }
  }
  finish_split(a, p, x, s, L.flag);
}

}  // namespace

AttendPlan plan_attend(bool hca, int B, int64_t T, int H, int d, int64_t max_entries, int window) {
  (void)hca;
  AttendPlan p{};
  p.rows = int64_t(B) * T;
  p.slots = max_entries + window;
  const int64_t tile = 64;  // multiple of both tile sizes
  // Split rows until there are about 256 workgroups, keeping >= 4 tiles per split.
  int64_t splits = 1;
  if (p.rows > 0 && p.rows < kAttendCtrlRows) {
    splits = (256 + p.rows - 1) / p.rows;
    const int64_t max_splits = (p.slots + 4 * tile - 1) / (4 * tile);
    if (splits > max_splits) splits = max_splits;
    if (splits < 1) splits = 1;
  }
  int64_t per = (p.slots + splits - 1) / splits;
  per = ((per + tile - 1) / tile) * tile;
  if (per < tile) per = tile;
  p.per_split = per;
  p.splits = (p.slots + per - 1) / per;
  if (p.splits < 1) p.splits = 1;
  size_t off = kHeaderBytes;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (bytes + 255) & ~size_t(255);
    return o;
  };
  const bool multi = p.splits > 1;
  const size_t R = size_t(p.rows);
  p.off_part = take(R * size_t(p.splits) * H * d * 4);
  p.off_ml = take(R * size_t(p.splits) * H * 2 * 4);
  p.ws_bytes = multi ? off : 0;
  return p;
}

hipError_t launch_attend(const AttendArgs& a, const AttendPlan& p) {
  if (p.rows == 0) return hipSuccess;
  dim3 grid(unsigned(p.rows * p.splits)), block(kThreads);
  if (a.bf16) {
    if (a.d == 128) hipLaunchKernelGGL(attend_bf16_kernel<128>, grid, block, 0, a.stream, a, p);
    else hipLaunchKernelGGL(attend_bf16_kernel<64>, grid, block, 0, a.stream, a, p);
  } else {
    if (a.d == 128) hipLaunchKernelGGL(attend_f32_kernel<128>, grid, block, 0, a.stream, a, p);
    else if (a.d == 64) hipLaunchKernelGGL(attend_f32_kernel<64>, grid, block, 0, a.stream, a, p);
    else hipLaunchKernelGGL(attend_f32_kernel<32>, grid, block, 0, a.stream, a, p);
  }
  return hipGetLastError();
}

}  // namespace csa

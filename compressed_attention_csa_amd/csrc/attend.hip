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
// Work split.  A workgroup handles one row, one group of up to 64 heads and one
// contiguous range of slots ("split").  All query heads share the one KV head,
// so a K/V row fetched once feeds every head of the group; the head groups of
// one (row, split) get block ids that are equal modulo 8, which places them on
// the same XCD so that the second group finds the rows in that XCD's L2.
//
// bf16 path: 32-slot tiles are gathered into LDS (K row-major, V transposed)
// while the next tile's rows are already being loaded into registers.
// S^T = K Q^T on 16x16x32 MFMA puts one head per lane column and 8 slots per
// lane, which is exactly the B-operand layout of O^T = V^T P^T, so the softmax
// weights never move between lanes.  P enters the MFMA as a bf16 hi + lo pair
// (16 significant bits).  fp32 path: fp32 FMA with one slot per lane.
// With several splits, each writes (O, max, sum) partials and the last split of
// the (row, head group) to finish merges them (log-sum-exp).
#include "common.hpp"
#include "kernels.h"

namespace csa {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 32;      // bf16 slots per tile
constexpr int kTileF32 = 64;   // fp32 slots per tile
constexpr int kMaxSplits = 64;
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

// Element offset of the source row of `slot` in the compressed (cmp=true) or raw
// tensors, or -1 when the slot is skipped.
__device__ __forceinline__ int64_t slot_offset(const AttendArgs& a, const RowSlots& x, int64_t slot,
                                               bool& cmp) {
  const int64_t nsel = a.hca ? x.c : int64_t(a.top_k);
  if (slot < nsel) {
    cmp = true;
    int64_t j = slot;
    if (!a.hca) {
      j = a.idx[x.r * a.top_k + slot];
      if (j < 0 || j >= x.c) return -1;
    }
    return (x.b * a.N_alloc + j) * a.d;
  }
  cmp = false;
  const int64_t pos = x.wstart + (slot - nsel);
  return (x.b * a.n_raw + (pos - a.raw_base)) * a.d;
}

struct SplitCtrl {
  uint32_t arrive;
  uint32_t pad[3];
};

__device__ __forceinline__ float4 load_dev4(const float* p) {
  return make_float4(load_dev(p), load_dev(p + 1), load_dev(p + 2), load_dev(p + 3));
}

struct MergeLds {
  float f[kMaxSplits][kAttendGroupHeads];  // per-split weight exp2(m_s - M) / L
  float lse[kAttendGroupHeads];
};

// Merge the S partials of one (row, head group) and write out / lse.
// part: [S][nhs][d] un-normalised O; ml: [S][nhs][2] (max in log2 units, sum);
// nhs is the per-group stride, nh <= nhs the group's heads.
__device__ void merge_group(const AttendArgs& a, const float* part, const float* ml, int64_t S,
                            int64_t r, int h_begin, int nh, int nhs, MergeLds& M) {
  const int d = a.d, tid = threadIdx.x;
  for (int h = tid; h < nh; h += kThreads) {
    float mx = -INFINITY;
    for (int64_t s = 0; s < S; ++s) mx = fmaxf(mx, load_dev(&ml[(s * nhs + h) * 2]));
    float Lsum = 0.0f;
    if (mx != -INFINITY)
      for (int64_t s = 0; s < S; ++s)
        Lsum = fmaf(exp2f(load_dev(&ml[(s * nhs + h) * 2]) - mx), load_dev(&ml[(s * nhs + h) * 2 + 1]), Lsum);
    const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
    for (int64_t s = 0; s < S; ++s)
      M.f[s][h] = (mx == -INFINITY) ? 0.0f : exp2f(load_dev(&ml[(s * nhs + h) * 2]) - mx) * inv;
    M.lse[h] = Lsum > 0.0f ? (mx + log2f(Lsum)) * kLn2 : -INFINITY;
  }
  __syncthreads();
  const int cpr = d / 4;  // float4 chunks per head
  for (int c = tid; c < nh * cpr; c += kThreads) {
    const int h = c / cpr, col = (c % cpr) * 4;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    int64_t s = 0;
    for (; s + 4 <= S; s += 4) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = load_dev4(part + ((s + u) * nhs + h) * int64_t(d) + col);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float f = M.f[s + u][h];
        acc.x = fmaf(f, v[u].x, acc.x); acc.y = fmaf(f, v[u].y, acc.y);
        acc.z = fmaf(f, v[u].z, acc.z); acc.w = fmaf(f, v[u].w, acc.w);
      }
    }
    for (; s < S; ++s) {
      const float4 v = load_dev4(part + (s * nhs + h) * int64_t(d) + col);
      const float f = M.f[s][h];
      acc.x = fmaf(f, v.x, acc.x); acc.y = fmaf(f, v.y, acc.y);
      acc.z = fmaf(f, v.z, acc.z); acc.w = fmaf(f, v.w, acc.w);
    }
    const int64_t oi = (r * a.H + h_begin + h) * int64_t(d) + col;
    if (a.out_bf16) {
      const uint32_t w0 = uint32_t(f32_to_bf16(acc.x)) | (uint32_t(f32_to_bf16(acc.y)) << 16);
      const uint32_t w1 = uint32_t(f32_to_bf16(acc.z)) | (uint32_t(f32_to_bf16(acc.w)) << 16);
      *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(a.out) + oi) = make_uint2(w0, w1);
    } else {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + oi) = acc;
    }
  }
  if (a.lse)
    for (int h = tid; h < nh; h += kThreads) a.lse[r * a.H + h_begin + h] = M.lse[h];
}

// Publish this split's partials; the last split of the (row, group) merges.
__device__ void finish_split(const AttendArgs& a, const AttendPlan& p, const RowSlots& x,
                             int64_t unit, int h_begin, int nh, int nhs, uint32_t* s_flag,
                             MergeLds& M) {
  uint8_t* ws = reinterpret_cast<uint8_t*>(a.ws);
  SplitCtrl* ctrl = reinterpret_cast<SplitCtrl*>(ws + kAttendCtrlOff) + unit;
  if (!arrive_last(&ctrl->arrive, uint32_t(x.S), s_flag)) return;
  const float* part = reinterpret_cast<const float*>(ws + p.off_part) + unit * p.splits * nhs * a.d;
  const float* ml = reinterpret_cast<const float*>(ws + p.off_ml) + unit * p.splits * nhs * 2;
  merge_group(a, part, ml, x.S, x.r, h_begin, nh, nhs, M);
  if (threadIdx.x == 0) ctrl->arrive = 0;
}

// Block id -> (head group, row, split).  Each group spans group_stride ids (a
// multiple of 8), so the groups of one (row, split) share id mod 8 and hence
// an XCD.  Returns false for the padding ids.
__device__ __forceinline__ bool decode_block(const AttendPlan& p, int64_t& hg, int64_t& r, int64_t& s) {
  hg = blockIdx.x / p.group_stride;
  const int64_t rem = blockIdx.x % p.group_stride;
  if (rem >= p.rows * p.splits) return false;
  r = rem / p.splits;
  s = rem % p.splits;
  return true;
}

// ---------------------------------------------------------------- bf16 MFMA kernel

template <int D>
struct LdsBF16 {
  bf16_t k[kTile][D + 8];   // row-major K tile (padded rows)
  bf16_t vt[D][kTile + 8];  // transposed V tile
  uint32_t live[kTile];
  uint32_t flag[4];
  MergeLds merge;
};

template <int D>
__global__ __launch_bounds__(kThreads) void attend_bf16_kernel(AttendArgs a, AttendPlan p) {
  __shared__ LdsBF16<D> L;
  int64_t hg, r, s;
  if (!decode_block(p, hg, r, s)) return;
  const RowSlots x = row_slots(a, p, r, s);
  if (s >= x.S) return;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, g = lane >> 4, col = lane & 15;
  const int H = a.H;
  const int h_begin = int(hg) * kAttendGroupHeads;
  const int nh = (H - h_begin) < kAttendGroupHeads ? (H - h_begin) : kAttendGroupHeads;
  const int h0 = h_begin + wid * 16;  // this wave's 16 heads
  const bool has = wid * 16 < nh;
  constexpr int KS = D / 32;   // k-steps of the QK product
  constexpr int DVT = D / 16;  // 16-column tiles of the output
  constexpr int CPR = D / 8;   // 16-byte chunks per row
  constexpr int NCH = kTile * CPR / kThreads;  // chunks per thread per tensor

  bf16x8_t qb[KS];
  const bf16_t* qrow = reinterpret_cast<const bf16_t*>(a.q) + r * int64_t(H) * D;
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (has) v = *reinterpret_cast<const uint4*>(qrow + (h0 + col) * D + 32 * kk + 8 * g);
    qb[kk] = u32x4_as_bf16x8(v);
  }
  const float sl2 = a.scale * kLog2e;
  f32x4_t o[DVT];
#pragma unroll
  for (int v = 0; v < DVT; ++v) o[v] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float mrun = -INFINITY, lpart = 0.0f;

  const bf16_t* kc = reinterpret_cast<const bf16_t*>(a.k_cmp);
  const bf16_t* vc = reinterpret_cast<const bf16_t*>(a.v_cmp);
  const bf16_t* kr = reinterpret_cast<const bf16_t*>(a.k_raw);
  const bf16_t* vr = reinterpret_cast<const bf16_t*>(a.v_raw);
  uint4 pk[NCH], pv[NCH];
  bool plive[NCH];
  auto fetch = [&](int64_t t0) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int id = tid + c * kThreads, sl = id / CPR, ch = id % CPR;
      const int64_t slot = t0 + sl;
      pk[c] = make_uint4(0, 0, 0, 0);
      pv[c] = make_uint4(0, 0, 0, 0);
      plive[c] = false;
      if (slot < x.hi) {
        bool cmp;
        const int64_t off = slot_offset(a, x, slot, cmp);
        if (off >= 0) {
          plive[c] = true;
          pk[c] = *reinterpret_cast<const uint4*>((cmp ? kc : kr) + off + ch * 8);
          pv[c] = *reinterpret_cast<const uint4*>((cmp ? vc : vr) + off + ch * 8);
        }
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int id = tid + c * kThreads, sl = id / CPR, ch = id % CPR;
      *reinterpret_cast<uint4*>(&L.k[sl][ch * 8]) = pk[c];
      const uint32_t w4[4] = {pv[c].x, pv[c].y, pv[c].z, pv[c].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        L.vt[ch * 8 + 2 * i][sl] = bf16_t(w4[i] & 0xffffu);
        L.vt[ch * 8 + 2 * i + 1][sl] = bf16_t(w4[i] >> 16);
      }
      if (ch == 0) L.live[sl] = plive[c] ? 1u : 0u;
    }
  };

  if (x.lo < x.hi) fetch(x.lo);
  for (int64_t t0 = x.lo; t0 < x.hi; t0 += kTile) {
    stash();
    __syncthreads();
    if (t0 + kTile < x.hi) fetch(t0 + kTile);  // next tile in flight during the math
    if (has) {
      f32x4_t sc[2];
#pragma unroll
      for (int cg = 0; cg < 2; ++cg) {
        f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          const uint4 kv = *reinterpret_cast<const uint4*>(&L.k[cg * 16 + col][32 * kk + 8 * g]);
          acc = mfma16x16x32(u32x4_as_bf16x8(kv), qb[kk], acc);
        }
        sc[cg] = acc;
      }
      // Online softmax in log2 units; lane holds head h0 + col and 8 slots.
      float tmax = -INFINITY;
#pragma unroll
      for (int cg = 0; cg < 2; ++cg)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float v = L.live[cg * 16 + 4 * g + j] ? sc[cg][j] * sl2 : -INFINITY;
          sc[cg][j] = v;
          tmax = fmaxf(tmax, v);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float mnew = fmaxf(mrun, tmax);
      const float corr = (mnew == -INFINITY) ? 1.0f : exp2f(mrun - mnew);
      mrun = mnew;
      float psum = 0.0f;
      uint32_t phi[4], plo[4];
#pragma unroll
      for (int cg = 0; cg < 2; ++cg)
#pragma unroll
        for (int j = 0; j < 4; j += 2) {
          const float p0 = (mnew == -INFINITY) ? 0.0f : exp2f(sc[cg][j] - mnew);
          const float p1 = (mnew == -INFINITY) ? 0.0f : exp2f(sc[cg][j + 1] - mnew);
          psum += p0 + p1;
          const bf16_t h0b = f32_to_bf16(p0), h1b = f32_to_bf16(p1);
          const bf16_t l0 = f32_to_bf16(p0 - bf16_to_f32(h0b));
          const bf16_t l1 = f32_to_bf16(p1 - bf16_to_f32(h1b));
          phi[cg * 2 + j / 2] = uint32_t(h0b) | (uint32_t(h1b) << 16);
          plo[cg * 2 + j / 2] = uint32_t(l0) | (uint32_t(l1) << 16);
        }
      lpart = lpart * corr + psum;
      const bf16x8_t pb_hi = u32x4_as_bf16x8(make_uint4(phi[0], phi[1], phi[2], phi[3]));
      const bf16x8_t pb_lo = u32x4_as_bf16x8(make_uint4(plo[0], plo[1], plo[2], plo[3]));
#pragma unroll
      for (int v = 0; v < DVT; ++v) {
        f32x4_t acc = o[v];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] *= corr;
        const uint2 a0 = *reinterpret_cast<const uint2*>(&L.vt[v * 16 + col][4 * g]);
        const uint2 a1 = *reinterpret_cast<const uint2*>(&L.vt[v * 16 + col][16 + 4 * g]);
        const bf16x8_t va = u32x4_as_bf16x8(make_uint4(a0.x, a0.y, a1.x, a1.y));
        acc = mfma16x16x32(va, pb_hi, acc);
        acc = mfma16x16x32(va, pb_lo, acc);
        o[v] = acc;
      }
    }
    __syncthreads();
  }

  // Per-head totals; lane (g, col) holds head h0 + col, columns 16v + 4g + j.
  float lt = lpart;
  lt += __shfl_xor(lt, 16);
  lt += __shfl_xor(lt, 32);
  const int h = h0 + col;
  if (x.S == 1) {
    if (has) {
      const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
#pragma unroll
      for (int v = 0; v < DVT; ++v) {
        const int64_t oi = (r * H + h) * int64_t(D) + v * 16 + 4 * g;
        if (a.out_bf16) {
          uint32_t w0 = uint32_t(f32_to_bf16(o[v][0] * inv)) | (uint32_t(f32_to_bf16(o[v][1] * inv)) << 16);
          uint32_t w1 = uint32_t(f32_to_bf16(o[v][2] * inv)) | (uint32_t(f32_to_bf16(o[v][3] * inv)) << 16);
          *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(a.out) + oi) = make_uint2(w0, w1);
        } else {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + oi) =
              make_float4(o[v][0] * inv, o[v][1] * inv, o[v][2] * inv, o[v][3] * inv);
        }
      }
      if (a.lse && g == 0) a.lse[r * H + h] = lt > 0.0f ? (mrun + log2f(lt)) * kLn2 : -INFINITY;
    }
    return;
  }
  const int64_t unit = hg * p.rows + r;
  const int nhs = H < kAttendGroupHeads ? H : kAttendGroupHeads;  // partial stride per group
  uint8_t* ws = reinterpret_cast<uint8_t*>(a.ws);
  float* part = reinterpret_cast<float*>(ws + p.off_part) + (unit * p.splits + s) * int64_t(nhs) * D;
  float* ml = reinterpret_cast<float*>(ws + p.off_ml) + (unit * p.splits + s) * int64_t(nhs) * 2;
  if (has) {
    const int hl = wid * 16 + col;
#pragma unroll
    for (int v = 0; v < DVT; ++v)
#pragma unroll
      for (int j = 0; j < 4; ++j) store_dev(part + int64_t(hl) * D + v * 16 + 4 * g + j, o[v][j]);
    if (g == 0) {
      store_dev(&ml[hl * 2], mrun);
      store_dev(&ml[hl * 2 + 1], lt);
    }
  }
  finish_split(a, p, x, unit, h_begin, nh, nhs, L.flag, L.merge);
}

// ---------------------------------------------------------------- fp32 kernel

template <int D>
struct LdsF32 {
  float k[kTileF32][D + 1];
  float v[kTileF32][D];
  float q[32][D];
  float pr[32][kTileF32];
  uint32_t flag[4];
  MergeLds merge;
};

template <int D>
__global__ __launch_bounds__(kThreads) void attend_f32_kernel(AttendArgs a, AttendPlan p) {
  __shared__ LdsF32<D> L;
  int64_t hg, r, s;
  if (!decode_block(p, hg, r, s)) return;
  const RowSlots x = row_slots(a, p, r, s);
  if (s >= x.S) return;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int H = a.H;  // <= 32: one head group
  constexpr int DPL = (D + 63) / 64;  // output columns per lane
  const float* qrow = reinterpret_cast<const float*>(a.q) + r * int64_t(H) * D;
  for (int i = tid; i < H * D; i += kThreads) L.q[i / D][i % D] = qrow[i];
  const float sl2 = a.scale * kLog2e;
  const float* kc = reinterpret_cast<const float*>(a.k_cmp);
  const float* vc = reinterpret_cast<const float*>(a.v_cmp);
  const float* kr = reinterpret_cast<const float*>(a.k_raw);
  const float* vr = reinterpret_cast<const float*>(a.v_raw);
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
        bool cmp;
        const int64_t off = slot_offset(a, x, slot, cmp);
        if (off >= 0) {
          kv = *reinterpret_cast<const float4*>((cmp ? kc : kr) + off + ch * 4);
          vv = *reinterpret_cast<const float4*>((cmp ? vc : vr) + off + ch * 4);
        }
      }
      L.k[sl][ch * 4] = kv.x; L.k[sl][ch * 4 + 1] = kv.y; L.k[sl][ch * 4 + 2] = kv.z; L.k[sl][ch * 4 + 3] = kv.w;
      *reinterpret_cast<float4*>(&L.v[sl][ch * 4]) = vv;
    }
    __syncthreads();
    const int64_t slot = t0 + lane;
    bool cmp;
    const bool live = slot < x.hi && slot_offset(a, x, slot, cmp) >= 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int h = wid + 4 * u;
      if (h < H) {
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
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int h = wid + 4 * u;
      if (h < H) {
#pragma unroll
        for (int c = 0; c < DPL; ++c) {
          const int dv = lane + 64 * c;
          if (dv < D) {
            float acc = o[u][c];
            for (int e = 0; e < kTileF32; ++e) acc = fmaf(L.pr[h][e], L.v[e][dv], acc);
            o[u][c] = acc;
          }
        }
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
      if (h < H) {
        const float inv = lt[u] > 0.0f ? 1.0f / lt[u] : 0.0f;
#pragma unroll
        for (int c = 0; c < DPL; ++c) {
          const int dv = lane + 64 * c;
          if (dv < D) {
            const int64_t oi = (r * H + h) * int64_t(D) + dv;
            if (a.out_bf16) reinterpret_cast<bf16_t*>(a.out)[oi] = f32_to_bf16(o[u][c] * inv);
            else reinterpret_cast<float*>(a.out)[oi] = o[u][c] * inv;
          }
        }
        if (a.lse && lane == 0)
          a.lse[r * H + h] = lt[u] > 0.0f ? (mrun[u] + log2f(lt[u])) * kLn2 : -INFINITY;
      }
    }
    return;
  }
  const int64_t unit = r;  // one head group
  uint8_t* ws = reinterpret_cast<uint8_t*>(a.ws);
  float* part = reinterpret_cast<float*>(ws + p.off_part) + (unit * p.splits + s) * int64_t(H) * D;
  float* ml = reinterpret_cast<float*>(ws + p.off_ml) + (unit * p.splits + s) * int64_t(H) * 2;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int h = wid + 4 * u;
    if (h < H) {
#pragma unroll
      for (int c = 0; c < DPL; ++c) {
        const int dv = lane + 64 * c;
        if (dv < D) store_dev(&part[int64_t(h) * D + dv], o[u][c]);
      }
      if (lane == 0) {
        store_dev(&ml[h * 2], mrun[u]);
        store_dev(&ml[h * 2 + 1], lt[u]);
      }
    }
  }
  finish_split(a, p, x, unit, 0, H, H, L.flag, L.merge);
}

}  // namespace

AttendPlan plan_attend(bool hca, int B, int64_t T, int H, int d, int64_t max_entries, int window) {
  (void)hca;
  AttendPlan p{};
  p.rows = int64_t(B) * T;
  p.groups = (H + kAttendGroupHeads - 1) / kAttendGroupHeads;
  p.slots = max_entries + window;
  const int64_t tile = 64;  // multiple of both tile sizes
  // Split rows until there are about 256 workgroups, keeping >= 2 tiles of 64 per split.
  const int64_t units = p.rows * p.groups;
  int64_t splits = 1;
  if (units > 0 && units <= kAttendCtrlUnits) {
    splits = (256 + units - 1) / units;
    const int64_t max_splits = (p.slots + 2 * tile - 1) / (2 * tile);
    if (splits > max_splits) splits = max_splits;
    if (splits > kMaxSplits) splits = kMaxSplits;
    if (splits < 1) splits = 1;
  }
  int64_t per = (p.slots + splits - 1) / splits;
  per = ((per + tile - 1) / tile) * tile;
  if (per < tile) per = tile;
  p.per_split = per;
  p.splits = (p.slots + per - 1) / per;
  if (p.splits < 1) p.splits = 1;
  p.group_stride = ((p.rows * p.splits + 7) / 8) * 8;
  size_t off = kHeaderBytes;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (bytes + 255) & ~size_t(255);
    return o;
  };
  const bool multi = p.splits > 1;
  const size_t U = size_t(units);
  const size_t nh = size_t(H < kAttendGroupHeads ? H : kAttendGroupHeads);
  p.off_part = take(U * size_t(p.splits) * nh * d * 4);
  p.off_ml = take(U * size_t(p.splits) * nh * 2 * 4);
  p.ws_bytes = multi ? off : 0;
  return p;
}

hipError_t launch_attend(const AttendArgs& a, const AttendPlan& p) {
  if (p.rows == 0) return hipSuccess;
  dim3 grid(unsigned(p.groups * p.group_stride)), block(kThreads);
  ProfScope prof(a.hca ? "hca_attend" : "csa_attend", a.stream);
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

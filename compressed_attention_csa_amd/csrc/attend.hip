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
// Work split.  All query heads share the one KV head, so a K/V row fetched
// once feeds every head that a workgroup holds.
//
// bf16 path: a workgroup handles one row, every head of it (wave w owns heads
// 16w .. 16w+15; split rows with few workgroups split the heads into two
// groups instead, and split rows of at most four head waves have two wave sets
// that take the two tiles of each staged pair) and one contiguous range of
// slots ("split").  32-slot tiles
// are gathered into LDS (K row-major, V transposed) while the next tiles' rows
// are already being loaded into registers.  S^T = K Q^T on 16x16x32 MFMA puts
// one head per lane column and 8 slots per lane, which is exactly the
// B-operand layout of O^T = V^T P^T, so the softmax weights never move between
// lanes.  P enters the MFMA as a bf16 hi + lo pair (16 significant bits).  With
// several splits, each writes (O, max, sum) partials to the workspace and a
// separate merge kernel (one thread per row, head and 16-byte column chunk)
// combines them by log-sum-exp.  HCA over many consecutive query tokens uses
// the multi-token kernel below instead (no splits).
//
// fp32 path: fp32 FMA, scores with one slot per lane and outputs with one
// column per lane; a workgroup handles one row (up to 32 heads) and one split,
// and the last split of a row to finish merges the partials (log-sum-exp).
#include <type_traits>

#include "common.hpp"
#include "kernels.h"

namespace csa {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 32;      // bf16 slots per tile
constexpr int kTileF32 = 64;   // fp32 slots per tile
constexpr int kMaxSplits = 64;
// bf16 decode with fewer than 128 (row, split) workgroups: the heads are split
// into this many groups, each a workgroup of its own (twice the workgroups, each
// with half the products; the K / V rows of a split are gathered once per group,
// the second time mostly from the XCD's L2).
constexpr int kFewSplitHeadGroups = 2;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct RowSlots {
  int64_t r, b, t, c, wstart, wn, L, lo, hi, S;
};

__device__ __forceinline__ RowSlots row_slots(const AttendArgs& a, const AttendPlan& p, int64_t r,
                                              int64_t s) {
  RowSlots x;
  x.r = r;
  x.b = div64(r, a.T);
  x.t = a.t0 + (r - x.b * a.T);
  int64_t c = div64(x.t + 1, a.m);
  x.c = c < a.N_alloc ? c : a.N_alloc;
  int64_t ws = x.t - a.window + 1;
  x.wstart = ws > 0 ? ws : 0;
  x.wn = x.t - x.wstart + 1;
  if (a.window == 0) x.wn = 0;
  x.L = (a.hca ? x.c : int64_t(a.top_k)) + x.wn;
  int64_t S = div64(x.L + p.per_split - 1, p.per_split);
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

// Block id -> (head group, row, split).  With several groups, each spans
// group_stride ids (a multiple of 8), so the groups of one (row, split) share
// id mod 8 and hence an XCD.  Returns false for the padding ids.
__device__ __forceinline__ bool decode_block(const AttendPlan& p, int64_t& hg, int64_t& r, int64_t& s) {
  hg = blockIdx.x / p.group_stride;
  const int64_t rem = blockIdx.x % p.group_stride;
  if (rem >= p.rows * p.splits) return false;
  r = rem / p.splits;
  s = rem % p.splits;
  return true;
}

// ---------------------------------------------------------------- bf16 MFMA kernel
//
// One workgroup = one (row, split) and every head of the row (or of one head
// group, for split rows with few workgroups): wave w owns heads 16w .. 16w+15
// of its group, so each K/V row is read from memory once per split and group.  Tiles of
// 32 slots go through two LDS buffers; SETS further tiles are always in flight
// in registers (about 64 KB per workgroup; 32 KB for unsplit 64-head rows, which
// run three workgroups per CU), enough to cover memory latency in decode, where
// a split is a few tiles long.  A CU gathers only about 50 GB/s of scattered
// 256-byte rows however many loads it has in flight, so a decode row is split
// over many workgroups (csa_diag_gather_read, the Pro-like step's 4 rows of 1152
// slots: 32 workgroups, one per row and 16-head group, each gathering a whole
// row take 12.7 us; 72 workgroups of 128 slots, the split plan, 4.0 us), and the
// splits are merged afterwards.  Loads are issued unconditionally
// (dead slots read the query row instead), so the compiler's wait counts stay
// exact and no wait drains the prefetch.

constexpr int kTB = 32;           // slots per tile
constexpr int kMaxTable = 3072;   // selected-entry slots of one CSA split (top_k + window bound)

template <int D, int NB>
struct LdsB {
  uint4 k[NB][kTB * D / 8];  // K rows, 16-byte chunks swizzled for row-wise reads
  uint4 v[NB][kTB * D / 8];  // V rows, swizzled for transposing reads
  uint32_t live[NB][kTB];    // all ones for a live slot, 0 for a skipped one
  float ksc[NB][kTB];        // fp8 caches: per-slot score factor (K scale * scale * log2 e)
  float vsc[NB][kTB];        // fp8 caches: per-slot V scale
  int32_t src[kMaxTable];    // selected compressed entry of each CSA slot of the split, -1 if skipped
};

// K chunk position: 16 lanes reading one chunk of 16 consecutive rows, and 16
// lanes writing one row, hit distinct 16-byte bank groups.
template <int CPR>
__device__ __forceinline__ int k_pos(int sl, int ch) {
  if (CPR == 16) return sl * 16 + (ch ^ (sl & 15));
  return sl * 8 + (ch ^ ((sl & 7) ^ ((sl >> 3) & 1)));
}
// V chunk position: the transposing read of 4 consecutive rows x 2 adjacent
// chunks by 16 lanes hits distinct 8-byte bank pairs, and the next 16 lanes
// (the next 4 rows) the other half of the banks.
template <int CPR>
__device__ __forceinline__ int v_pos(int sl, int ch) {
  if (CPR == 16) return sl * 16 + (ch ^ (2 * (sl & 3)) ^ (8 * ((sl >> 2) & 1)));
  return sl * CPR + (ch ^ (2 * ((sl & 3) ^ ((sl >> 2) & 1))));
}

typedef short v4s_t __attribute__((ext_vector_type(4)));

// x where mask is all ones, -inf where it is 0 (one bitfield select).
__device__ __forceinline__ float mask_or_neg_inf(float x, uint32_t mask) {
  return __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, x) & mask) | (~mask & 0xff800000u));
}

// KV8: the compressed caches hold e4m3 codes with one fp32 scale per entry
// (K and V each).  The codes are widened exactly to bf16 when a tile is
// staged; the K scale joins the per-slot score factor and the V scale the
// slot's weight in O^T += V^T P^T (not in the softmax sum).
// Registers are capped at 256 per lane (two waves per SIMD) for bf16 caches: a
// workgroup of fewer than 8 waves could otherwise take 512 (one wave per SIMD);
// the cap measured faster (CSA prefill attention 0.79 -> 0.72 ms, the Pro-like
// decode 1.7%).  The fp8-cache variants keep the default, since the cap would
// make them spill.  The unsplit CSA rows of 64 heads (prefill) go further: 168
// registers, three waves per SIMD (three workgroups per CU, which their LDS
// allows), with two tiles in flight instead of four so that nothing spills
// (CSA prefill attention at 1M 0.72 -> 0.63 ms: more gathers in flight per CU
// from more waves, each with fewer).
// TH = 2 (split rows with at most 4 waves of heads): two sets of NW waves share
// the heads, and of each staged tile pair the first set computes one tile and
// the second set the other; the two online softmax states are combined in LDS
// at the end.  With one wave per SIMD the product / softmax chain of a tile is
// latency-bound, so two tiles at once on different waves halve the chain.
template <int D, int NW, bool HCA, int PAIR, bool KV8, int TH = 1>
__global__ __launch_bounds__(NW * TH * 64) __attribute__((amdgpu_waves_per_eu(KV8 ? 1 : (PAIR == 1 && NW == 4 && !HCA ? 3 : 2)))) void attend_bf16_kernel(AttendArgs a, AttendPlan p) {
  static_assert(TH == 1 || PAIR == 2, "tile halves take the two tiles of a pair");
  constexpr int kT = NW * TH * 64;
  constexpr int CPR = D / 8;                     // 16-byte chunks per row
  constexpr int CT = kTB * CPR;                  // chunks per tensor per tile
  constexpr int CPT = CT >= kT ? CT / kT : 1;    // chunks per thread per tensor per tile
  constexpr int SETS = CPT >= 4 ? 2 : (PAIR == 1 && NW == 4 && !HCA ? 2 : 4);  // tiles in flight in registers
  constexpr int KS = D / 32;                     // k-steps of the QK product
  constexpr int DVT = D / 16;                    // 16-column tiles of the output
  constexpr int NB = 2 * PAIR;                   // LDS tile buffers
  __shared__ LdsB<D, NB> L;
  debug_poison_lds(L);
  int64_t hg, r, s;
  if (!decode_block(p, hg, r, s)) return;
  const RowSlots x = row_slots(a, p, r, s);
  if (s >= x.S) return;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, g = lane >> 4, col = lane & 15;
  const int H = a.H;
  const int hw = wid % NW, half = wid / NW;        // head wave, tile half (TH = 2)
  const int h0 = int(hg) * (NW * 16) + hw * 16;   // this wave's 16 heads
  const bool has = h0 < H;
  const int64_t nsel = HCA ? x.c : int64_t(a.top_k);

  // Selected entries of this split (CSA), checked against visibility once.
  if (!HCA) {
    const int64_t e_end = x.hi < nsel ? x.hi : nsel;
    for (int64_t sl = x.lo + tid; sl < e_end; sl += kT) {
      const int32_t j = a.idx[x.r * a.top_k + sl];
      L.src[sl - x.lo] = (j >= 0 && j < x.c) ? j : -1;
    }
  }

  const bf16_t* qrow = reinterpret_cast<const bf16_t*>(a.q) + r * int64_t(H) * D;
  bf16x8_t qb[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (has) v = *reinterpret_cast<const uint4*>(qrow + (h0 + col) * D + 32 * kk + 8 * g);
    qb[kk] = u32x4_as_bf16x8(v);
  }
  __syncthreads();

  const bf16_t* kc = reinterpret_cast<const bf16_t*>(a.k_cmp) + x.b * a.N_alloc * D;
  const bf16_t* vc = reinterpret_cast<const bf16_t*>(a.v_cmp) + x.b * a.N_alloc * D;
  const uint8_t* kc8 = reinterpret_cast<const uint8_t*>(a.k_cmp) + x.b * a.N_alloc * D;
  const uint8_t* vc8 = reinterpret_cast<const uint8_t*>(a.v_cmp) + x.b * a.N_alloc * D;
  const float* ksp = a.k_scale + x.b * a.N_alloc;
  const float* vsp = a.v_scale + x.b * a.N_alloc;
  const bf16_t* kr = reinterpret_cast<const bf16_t*>(a.k_raw) + (x.b * a.n_raw - a.raw_base) * D;
  const bf16_t* vr = reinterpret_cast<const bf16_t*>(a.v_raw) + (x.b * a.n_raw - a.raw_base) * D;
  const float sl2 = a.scale * kLog2e;
  // Registers of one tile in flight (vectors rather than arrays, so that they
  // stay in registers).  With KV8, a chunk of a compressed row holds 8 codes
  // in its first two words (bit c of f8) until it is staged.
  typedef uint32_t chunks_t __attribute__((ext_vector_type(4 * CPT)));
  struct Pre {
    chunks_t k, v;
    uint32_t lv, f8;
    float ks, vs;  // KV8: scales of slot tid of the tile (threads tid < kTB)
  };
  // Loads tile t of the split (slots beyond the split or skipped read the query row).
  const int64_t cmp_end = x.hi < nsel ? x.hi : nsel;  // end of the compressed slots of the split
  auto fetch = [&](Pre& P, int t) __attribute__((always_inline)) {
    const int64_t t0 = x.lo + int64_t(t) * kTB;
    // HCA tile of consecutive live compressed rows (all but the split's last
    // tiles): one base address for the workgroup.
    if (HCA && t0 + kTB <= cmp_end) {
      const bf16_t* kb = kc + t0 * D;
      const bf16_t* vb = vc + t0 * D;
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int id = (tid + c * kT) % CT;
        if (KV8) {
          const uint2 kw = *reinterpret_cast<const uint2*>(kc8 + t0 * D + id * 8);
          const uint2 vw = *reinterpret_cast<const uint2*>(vc8 + t0 * D + id * 8);
          P.k[4 * c] = kw.x; P.k[4 * c + 1] = kw.y;
          P.v[4 * c] = vw.x; P.v[4 * c + 1] = vw.y;
        } else {
          const uint4 kw = *reinterpret_cast<const uint4*>(kb + id * 8);
          const uint4 vw = *reinterpret_cast<const uint4*>(vb + id * 8);
          P.k[4 * c] = kw.x; P.k[4 * c + 1] = kw.y; P.k[4 * c + 2] = kw.z; P.k[4 * c + 3] = kw.w;
          P.v[4 * c] = vw.x; P.v[4 * c + 1] = vw.y; P.v[4 * c + 2] = vw.z; P.v[4 * c + 3] = vw.w;
        }
      }
      P.lv = (1u << CPT) - 1;
      P.f8 = KV8 ? (1u << CPT) - 1 : 0u;
      if (KV8 && tid < kTB) {
        P.ks = ksp[t0 + tid];
        P.vs = vsp[t0 + tid];
      }
      return;
    }
    uint32_t lv = 0, f8 = 0;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int id = (tid + c * kT) % CT, sl = id / CPR, ch = id % CPR;
      const int64_t slot = t0 + sl;
      const bf16_t* kp = qrow;
      const bf16_t* vp = qrow;
      bool live = false, cmp8 = false;
      int64_t j = 0;
      if (slot < x.hi) {
        if (slot < nsel) {
          j = slot;
          if (!HCA) j = L.src[slot - x.lo];
          if (j >= 0) {
            kp = kc + j * D;
            vp = vc + j * D;
            live = true;
            cmp8 = KV8;
          }
        } else {
          const int64_t pos = x.wstart + (slot - nsel);
          kp = kr + pos * D;
          vp = vr + pos * D;
          live = true;
        }
      }
      if (KV8 && cmp8) {
        const uint2 kw = *reinterpret_cast<const uint2*>(kc8 + j * D + ch * 8);
        const uint2 vw = *reinterpret_cast<const uint2*>(vc8 + j * D + ch * 8);
        P.k[4 * c] = kw.x; P.k[4 * c + 1] = kw.y;
        P.v[4 * c] = vw.x; P.v[4 * c + 1] = vw.y;
      } else {
        const uint4 kw = *reinterpret_cast<const uint4*>(kp + ch * 8);
        const uint4 vw = *reinterpret_cast<const uint4*>(vp + ch * 8);
        P.k[4 * c] = kw.x; P.k[4 * c + 1] = kw.y; P.k[4 * c + 2] = kw.z; P.k[4 * c + 3] = kw.w;
        P.v[4 * c] = vw.x; P.v[4 * c + 1] = vw.y; P.v[4 * c + 2] = vw.z; P.v[4 * c + 3] = vw.w;
      }
      lv |= uint32_t(live) << c;
      f8 |= uint32_t(cmp8) << c;
    }
    P.lv = lv;
    P.f8 = f8;
    if (KV8 && tid < kTB) {  // the scales of slot t0 + tid (1 for window and skipped slots)
      const int64_t slot = t0 + tid;
      int64_t j = -1;
      if (slot < x.hi && slot < nsel) j = HCA ? slot : int64_t(L.src[slot - x.lo]);
      P.ks = j >= 0 ? ksp[j] : 1.0f;
      P.vs = j >= 0 ? vsp[j] : 1.0f;
    }
  };
  auto stage = [&](const Pre& P, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int id = tid + c * kT, sl = (id % CT) / CPR, ch = id % CPR;
      if (id < CT) {
        uint4 kw = make_uint4(P.k[4 * c], P.k[4 * c + 1], P.k[4 * c + 2], P.k[4 * c + 3]);
        uint4 vw = make_uint4(P.v[4 * c], P.v[4 * c + 1], P.v[4 * c + 2], P.v[4 * c + 3]);
        if (KV8 && ((P.f8 >> c) & 1u)) {
          kw = make_uint4(e4m3x2_to_bf16x2<false>(P.k[4 * c]), e4m3x2_to_bf16x2<true>(P.k[4 * c]),
                          e4m3x2_to_bf16x2<false>(P.k[4 * c + 1]), e4m3x2_to_bf16x2<true>(P.k[4 * c + 1]));
          vw = make_uint4(e4m3x2_to_bf16x2<false>(P.v[4 * c]), e4m3x2_to_bf16x2<true>(P.v[4 * c]),
                          e4m3x2_to_bf16x2<false>(P.v[4 * c + 1]), e4m3x2_to_bf16x2<true>(P.v[4 * c + 1]));
        }
        // A skipped slot holds zeros, not the query row it was loaded from: its
        // weight is 0, and 0 times a NaN or an infinity there would be NaN.
        if (!((P.lv >> c) & 1u)) kw = vw = make_uint4(0u, 0u, 0u, 0u);
        L.k[buf][k_pos<CPR>(sl, ch)] = kw;
        L.v[buf][v_pos<CPR>(sl, ch)] = vw;
        if (ch == 0) L.live[buf][sl] = ((P.lv >> c) & 1u) ? 0xffffffffu : 0u;
      }
    }
    if (KV8 && tid < kTB) {
      L.ksc[buf][tid] = P.ks * sl2;
      L.vsc[buf][tid] = P.vs;
    }
  };

  f32x4_t o[DVT];
#pragma unroll
  for (int v = 0; v < DVT; ++v) o[v] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  // Softmax reference of this lane's head (log2 units; equal in the 4 lanes of
  // a head): the running maximum as of the last rescale.  Weights are formed
  // against it as long as no score exceeds it by more than kSlack, so most tiles
  // need neither a cross-lane reduction nor a rescale of O.
  constexpr float kSlack = 8.0f;
  float mref = -INFINITY, lpart = 0.0f;

  // S^T = K Q^T (lane: head h0 + col, slots 16cg + 4g + j), weights in log2
  // units, then O^T += V^T P^T with P as a bf16 hi + lo pair.
  auto qk = [&](int buf, f32x4_t (&sc)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int cg = 0; cg < 2; ++cg) {
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const uint4 kv = L.k[buf][k_pos<CPR>(cg * 16 + col, 4 * kk + g)];
        acc = mfma16x16x32(u32x4_as_bf16x8(kv), qb[kk], acc);
      }
      sc[cg] = acc;
    }
  };
  // A operand of V^T for output columns 16v..16v+15: lane (g, col) needs
  // V[slot][16v + col] for the slots 4g..4g+3 and 16+4g..16+4g+3; a
  // transposing read of 4 rows returns them.
  auto vfrag = [&](int buf, int v) __attribute__((always_inline)) {
    const int vr0 = 4 * g + col / 4, half = col & 1;
    const int ch = 2 * v + (col & 3) / 2;
    const short* b0 = reinterpret_cast<const short*>(&L.v[buf][v_pos<CPR>(vr0, ch)]) + 4 * half;
    const short* b1 = reinterpret_cast<const short*>(&L.v[buf][v_pos<CPR>(vr0 + 16, ch)]) + 4 * half;
    const v4s_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)(b0));
    const v4s_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)(b1));
    uint4 w;
    __builtin_memcpy(&w.x, &t0, 8);
    __builtin_memcpy(&w.z, &t1, 8);
    return u32x4_as_bf16x8(w);
  };
  // One group of PAIR staged tiles (buffers b0, b0+1): the scores of all of
  // them, one reference check for the group, then weights and O^T updates.
  // A tile past the split was staged with every slot skipped, so it adds
  // nothing and needs no branch.
  constexpr int CP = TH == 2 ? 1 : PAIR;  // tiles one wave computes per staged group
  auto compute = [&](int b0) __attribute__((always_inline)) {
    f32x4_t sc[CP][2];
#pragma unroll
    for (int i = 0; i < CP; ++i) qk(b0 + i, sc[i]);
    // Paired tiles read the first tile's V^T operands while the products run;
    // single tiles read them just before use (fewer registers, for occupancy).
    bf16x8_t va[DVT];
    if (CP == 2) {
#pragma unroll
      for (int v = 0; v < DVT; ++v) va[v] = vfrag(b0, v);
    }
    // u = score - reference (log2 units); skipped slots get -inf (a bit
    // select with the slot's mask, which also holds while the reference is
    // -inf).
    float u[CP][2][4];
    float umax = -INFINITY;
    const float nref = -mref;
#pragma unroll
    for (int i = 0; i < CP; ++i)
#pragma unroll
      for (int cg = 0; cg < 2; ++cg) {
        const uint4 lm = *reinterpret_cast<const uint4*>(&L.live[b0 + i][cg * 16 + 4 * g]);
        const uint32_t lmv[4] = {lm.x, lm.y, lm.z, lm.w};
        float4 kf = make_float4(sl2, sl2, sl2, sl2);
        if (KV8) kf = *reinterpret_cast<const float4*>(&L.ksc[b0 + i][cg * 16 + 4 * g]);
        const float kfv[4] = {kf.x, kf.y, kf.z, kf.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u[i][cg][j] = mask_or_neg_inf(fmaf(sc[i][cg][j], kfv[j], nref), lmv[j]);
          umax = fmaxf(umax, u[i][cg][j]);
        }
      }
    // A live score above reference + kSlack (or a live slot while there is no
    // reference yet: u = +inf) moves the reference to the running maximum (a
    // wave-uniform branch).
    if (__builtin_expect(__ballot(umax > kSlack) != 0, 0)) {
      float tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < CP; ++i)
#pragma unroll
        for (int cg = 0; cg < 2; ++cg) {
          const uint4 lm = *reinterpret_cast<const uint4*>(&L.live[b0 + i][cg * 16 + 4 * g]);
          const uint32_t lmv[4] = {lm.x, lm.y, lm.z, lm.w};
          float4 kf = make_float4(sl2, sl2, sl2, sl2);
          if (KV8) kf = *reinterpret_cast<const float4*>(&L.ksc[b0 + i][cg * 16 + 4 * g]);
          const float kfv[4] = {kf.x, kf.y, kf.z, kf.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            u[i][cg][j] = mask_or_neg_inf(sc[i][cg][j] * kfv[j], lmv[j]);
            tmax = fmaxf(tmax, u[i][cg][j]);
          }
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float mnew = fmaxf(mref, tmax);
      // With no live slot yet everything is zero: subtract 0 instead of -inf.
      const float msafe = (mnew == -INFINITY) ? 0.0f : mnew;
      const float corr = exp2f(mref - msafe);
      mref = mnew;
      lpart *= corr;
#pragma unroll
      for (int v = 0; v < DVT; ++v)
#pragma unroll
        for (int j = 0; j < 4; ++j) o[v][j] *= corr;
#pragma unroll
      for (int i = 0; i < CP; ++i)
#pragma unroll
        for (int cg = 0; cg < 2; ++cg)
#pragma unroll
          for (int j = 0; j < 4; ++j) u[i][cg][j] -= msafe;
    }
#pragma unroll
    for (int i = 0; i < CP; ++i) {
      f32x2_t ps = {0.0f, 0.0f};
      uint32_t phi[4], plo[4];
#pragma unroll
      for (int cg = 0; cg < 2; ++cg) {
        float4 vf = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
        if (KV8) vf = *reinterpret_cast<const float4*>(&L.vsc[b0 + i][cg * 16 + 4 * g]);
        const float vfv[4] = {vf.x, vf.y, vf.z, vf.w};
#pragma unroll
        for (int j = 0; j < 4; j += 2) {
          // hardware 2^x (results below the normal range flush to 0, far below
          // what a weight within 2^8 of the reference can matter)
          f32x2_t pp = {__builtin_amdgcn_exp2f(u[i][cg][j]), __builtin_amdgcn_exp2f(u[i][cg][j + 1])};
          ps = (cg == 0 && j == 0) ? pp : ps + pp;
          if (KV8) pp = f32x2_t{pp[0] * vfv[j], pp[1] * vfv[j + 1]};  // the slot's V scale
          // P = hi + lo, both bf16 (hardware round-to-nearest-even conversions).
          const uint32_t hi = bf16x2_bits(pp);
          const f32x2_t back = {u32_as_f32(hi << 16), u32_as_f32(hi & 0xffff0000u)};
          phi[cg * 2 + j / 2] = hi;
          plo[cg * 2 + j / 2] = bf16x2_bits(pp - back);
        }
      }
      lpart += ps[0] + ps[1];
      const bf16x8_t pb_hi = u32x4_as_bf16x8(make_uint4(phi[0], phi[1], phi[2], phi[3]));
      const bf16x8_t pb_lo = u32x4_as_bf16x8(make_uint4(plo[0], plo[1], plo[2], plo[3]));
      if (CP == 1 || i == 1) {
#pragma unroll
        for (int v = 0; v < DVT; ++v) va[v] = vfrag(b0 + i, v);
      }
      // Eight independent accumulators: the hi pass, then the lo pass.
#pragma unroll
      for (int v = 0; v < DVT; ++v) o[v] = mfma16x16x32(va[v], pb_hi, o[v]);
#pragma unroll
      for (int v = 0; v < DVT; ++v) o[v] = mfma16x16x32(va[v], pb_lo, o[v]);
    }
  };

  const int nt = int((x.hi - x.lo + kTB - 1) / kTB);
  // PAIR tiles are staged per barrier, into buffers PAIR * (group & 1) + i;
  // a buffer is last read for the group two before: every wave passed the
  // barrier of the group in between only after finishing that.  Tiles past
  // the split are staged and fetched like the others (from the query row) so
  // that every thread issues the same loads; only their math is skipped.
  auto step = [&](Pre& P0, Pre& P1, int t) __attribute__((always_inline)) {
    const int b0 = PAIR * ((t / PAIR) & 1);
    stage(P0, b0);
    if (PAIR == 2) stage(P1, b0 + 1);
    __syncthreads();
    fetch(P0, t + SETS);
    if (PAIR == 2) fetch(P1, t + 1 + SETS);
    if (TH == 2) {
      if (has && t + half < nt) compute(b0 + half);
    } else if (has && t < nt) {
      compute(b0);
    }
  };
  Pre P[SETS];
#pragma unroll
  for (int i = 0; i < SETS; ++i) fetch(P[i], i);
  for (int t0 = 0; t0 < nt; t0 += SETS) {
#pragma unroll
    for (int i = 0; i < SETS; i += PAIR) step(P[i], P[i + PAIR - 1], t0 + i);
  }

  if constexpr (TH == 2) {
    // The second set's state (O, reference, partial sums) through LDS (the
    // tile buffers, free once every wave is past its last tile); the first
    // set combines it with its own under the larger reference.
    static_assert(sizeof(L.k) + sizeof(L.v) >= size_t(NW) * (DVT * 4 + 2) * 64 * 4, "exchange fits");
    float* xo = reinterpret_cast<float*>(&L.k[0][0]) + hw * ((DVT * 4 + 2) * 64);
    __syncthreads();
    if (half == 1) {
#pragma unroll
      for (int v = 0; v < DVT; ++v)
#pragma unroll
        for (int j = 0; j < 4; ++j) xo[(v * 4 + j) * 64 + lane] = o[v][j];
      xo[(DVT * 4) * 64 + lane] = mref;
      xo[(DVT * 4 + 1) * 64 + lane] = lpart;
    }
    __syncthreads();
    if (half == 1) return;
    const float m1 = xo[(DVT * 4) * 64 + lane], l1 = xo[(DVT * 4 + 1) * 64 + lane];
    const float mn = fmaxf(mref, m1);
    // A reference of -inf means no live slot so far: its state is all zero.
    const float s0 = mref == -INFINITY ? 0.0f : exp2f(mref - mn);
    const float s1 = m1 == -INFINITY ? 0.0f : exp2f(m1 - mn);
#pragma unroll
    for (int v = 0; v < DVT; ++v)
#pragma unroll
      for (int j = 0; j < 4; ++j) o[v][j] = o[v][j] * s0 + xo[(v * 4 + j) * 64 + lane] * s1;
    lpart = lpart * s0 + l1 * s1;
    mref = mn;
  }
  // Per-head totals; lane (g, col) holds head h0 + col, columns 16v + 4g + j.
  float lt = lpart;
  lt += __shfl_xor(lt, 16);
  lt += __shfl_xor(lt, 32);
  if (!has) return;
  const int h = h0 + col;
  if (x.S == 1) {
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
    if (a.lse && g == 0) a.lse[r * H + h] = lt > 0.0f ? (mref + log2f(lt)) * kLn2 : -INFINITY;
    return;
  }
  // Partials for the merge kernel: un-normalised O, running max (log2 units), sum.
  uint8_t* ws = reinterpret_cast<uint8_t*>(a.ws);
  float* part = reinterpret_cast<float*>(ws + p.off_part) + ((r * p.splits + s) * H + h) * int64_t(D);
  float* ml = reinterpret_cast<float*>(ws + p.off_ml) + ((r * p.splits + s) * H + h) * 2;
#pragma unroll
  for (int v = 0; v < DVT; ++v)
    *reinterpret_cast<float4*>(part + v * 16 + 4 * g) = make_float4(o[v][0], o[v][1], o[v][2], o[v][3]);
  if (g == 0) *reinterpret_cast<float2*>(ml) = make_float2(mref, lt);
}

// ---------------------------------------------------------------- HCA prefill kernel
//
// Consecutive query tokens of one sequence see the same heavy entries except
// at most the newest one (a heavy block completes every m' positions) and
// windows that overlap in all but a few positions.  A workgroup therefore takes
// QT consecutive tokens and every head: wave w owns 16 heads and RB of the
// tokens, so each K/V tile staged in LDS, and each MFMA operand read from it,
// serves RB query rows.  The slots are the heavy entries visible to the last
// token of the workgroup, then the union of the windows of its tokens.  Only
// the last heavy tile and the window tiles need a per-token visibility test: a
// range test on the slot's coordinate (entry index or position).

// Rows are padded by two 16-byte chunks instead of swizzled: the LDS counters
// show no bank conflicts for the row reads of K, the transposing reads of V
// and the staging writes (a one-chunk K pad conflicted on a quarter of the LDS
// cycles), and every read address of a lane is one base plus a constant, so
// the compiler folds the offsets into the instructions.
template <int D>
struct LdsM {
  static constexpr int KS = D / 8 + 2;  // K row stride in chunks
  static constexpr int VS = D / 8 + 2;  // V row stride in chunks
  uint4 k[2][kTB * KS];
  uint4 v[2][kTB * VS];
  uint4 vh[2][kTB * VS];  // bf16 caches: the V tile as binary16
  alignas(8) uint8_t vflag[2][8];  // per wave, staged |V|: bit 0, one != 0; bit 1, one >= 2^-10; bit 2, one > 65280
  float ksc[2][kTB];      // fp8 caches: per-slot score factor (K scale * scale * log2 e)
  float vsc[2][kTB];      // fp8 caches: per-slot V scale
};

// KV8 as in attend_bf16_kernel: heavy tiles hold e4m3 codes (widened when
// staged) with per-entry K and V scales; window tiles are bf16.
//
// Binary16 weights (bf16 caches).  Every bf16 value of magnitude 0 or in
// [2^-14, 65280] is a binary16 value, so a V tile in that range is staged a
// second time as binary16, exactly.  Such a tile enters O^T += V^T P^T with P
// rounded once to binary16 (11 significant bits, relative error at most
// 2^-11 per weight): one product per operand pair instead of the bf16 hi + lo
// pair.  A tile whose largest |V| exceeds 65280 (it would overflow), or is
// nonzero and below 2^-10 (so that values losing bits as binary16 subnormals,
// by at most 2^-25 each, could matter next to the output), ends the binary16
// run: it and every later tile of the workgroup take the hi + lo path.  Every
// staged chunk counts, rows a token does not see too: their weight is 0, and 0
// times an overflowed binary16 value would be NaN.  (Slots outside every
// range are staged as zeros.)  A NaN or infinity in a K or V row therefore
// also reaches the tokens of the workgroup that share its tile without seeing
// it (in the newest heavy tile and the window tiles): 0 times NaN is NaN.
template <int D, int NW, int RB, bool KV8>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW == 8 ? 2 : 1))) void hca_multi_kernel(AttendArgs a, int64_t groups_per_seq) {
  constexpr int kT = NW * 64;
  constexpr int CPR = D / 8;
  constexpr int CT = kTB * CPR;
  constexpr int CPT = CT >= kT ? CT / kT : 1;
  constexpr int KS = D / 32;
  constexpr int DVT = D / 16;
  constexpr bool F16 = !KV8;  // binary16 path available
  static_assert(NW <= 8, "one V range flag per wave");
  __shared__ LdsM<D> L;
  debug_poison_lds(L);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, col = lane & 15;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = a.H, HW = H / 16;
  const int QT = RB * (NW / HW);
  const int64_t T = a.T;
  const int64_t b = blockIdx.x / groups_per_seq;
  const int64_t i0 = (blockIdx.x - b * groups_per_seq) * QT;  // first token of the workgroup
  const int64_t ilast = (i0 + QT < T ? i0 + QT : T) - 1;
  const int h0 = (wid % HW) * 16;
  const int64_t iw = i0 + (wid / HW) * RB;  // first token of this wave

  // Visibility of the wave's tokens: heavy entries [0, c), positions [wl, t].
  int64_t tr[RB], cr[RB], wlr[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int64_t i = iw + rb < ilast ? iw + rb : ilast;
    tr[rb] = a.t0 + i;
    const int64_t c = div64(tr[rb] + 1, a.m);
    cr[rb] = c < a.N_alloc ? c : a.N_alloc;
    const int64_t ws = tr[rb] - a.window + 1;
    wlr[rb] = a.window == 0 ? tr[rb] + 1 : (ws > 0 ? ws : 0);
  }
  // Slots of the workgroup: heavy tiles, then the windows' union.
  const int64_t t_first = a.t0 + i0, t_last = a.t0 + ilast;
  const int64_t cl = div64(t_last + 1, a.m);
  const int64_t c_max = cl < a.N_alloc ? cl : a.N_alloc;
  const int64_t wlo0 = t_first - a.window + 1;
  const int64_t wlo = wlo0 > 0 ? wlo0 : 0;
  const int64_t whi = a.window == 0 ? wlo : t_last + 1;
  const int nht = int((c_max + kTB - 1) / kTB);
  const int nt = nht + int((whi - wlo + kTB - 1) / kTB);
  const int64_t wdelta = wlo - int64_t(nht) * kTB;  // window tile t starts at position t * kTB + wdelta

  const bf16_t* qbase = reinterpret_cast<const bf16_t*>(a.q) + (b * T) * int64_t(H) * D;
  const bf16_t* qrow = qbase + i0 * int64_t(H) * D;  // a safe address for skipped slots
  bf16x8_t qb[RB][KS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int64_t i = iw + rb < ilast ? iw + rb : ilast;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
      qb[rb][kk] = u32x4_as_bf16x8(
          *reinterpret_cast<const uint4*>(qbase + (i * H + h0 + col) * int64_t(D) + 32 * kk + 8 * g));
  }

  const bf16_t* kc = reinterpret_cast<const bf16_t*>(a.k_cmp) + b * a.N_alloc * D;
  const bf16_t* vc = reinterpret_cast<const bf16_t*>(a.v_cmp) + b * a.N_alloc * D;
  const bf16_t* kr = reinterpret_cast<const bf16_t*>(a.k_raw) + (b * a.n_raw - a.raw_base) * D;
  const bf16_t* vr = reinterpret_cast<const bf16_t*>(a.v_raw) + (b * a.n_raw - a.raw_base) * D;
  const uint8_t* kc8 = reinterpret_cast<const uint8_t*>(a.k_cmp) + b * a.N_alloc * D;
  const uint8_t* vc8 = reinterpret_cast<const uint8_t*>(a.v_cmp) + b * a.N_alloc * D;
  const float* ksp = a.k_scale + b * a.N_alloc;
  const float* vsp = a.v_scale + b * a.N_alloc;
  const float sl2 = a.scale * kLog2e;
  typedef uint32_t chunks_t __attribute__((ext_vector_type(4 * CPT)));
  struct Pre {
    chunks_t k, v;
    uint32_t lv;    // bit c: chunk c holds a row of the slot range (else zeros are staged)
    bool f8;        // a heavy tile of e4m3 codes (two words per chunk)
    float ks, vs;   // its scales of slot tid (threads tid < kTB)
  };
  // Loads tile t (tiles past the end, and slots past the heavy or window
  // range, read the query row; their math is masked or skipped).  Written
  // without branches, so that the tile loop body stays one basic block.
  auto fetch = [&](Pre& P, int t) __attribute__((always_inline)) {
    P.f8 = KV8 && t < nht;
    if (KV8 && t < nht) {
      const int64_t r0 = int64_t(t) * kTB;
      uint32_t lv = 0;
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int id = (tid + c * kT) % CT, sl = id / CPR, ch = id % CPR;
        lv |= uint32_t(r0 + sl < c_max) << c;
        const int64_t row = r0 + sl < c_max ? r0 + sl : c_max - 1;  // past the end: re-read the last entry
        const uint2 kw = *reinterpret_cast<const uint2*>(kc8 + row * D + ch * 8);
        const uint2 vw = *reinterpret_cast<const uint2*>(vc8 + row * D + ch * 8);
        P.k[4 * c] = kw.x; P.k[4 * c + 1] = kw.y;
        P.v[4 * c] = vw.x; P.v[4 * c + 1] = vw.y;
      }
      if (tid < kTB) {
        const int64_t row = r0 + tid < c_max ? r0 + tid : c_max - 1;
        P.ks = ksp[row];
        P.vs = vsp[row];
      }
      P.lv = lv;
      return;
    }
    // Wave-uniform choices as masks rather than branches.
    const int64_t win = -int64_t(t >= nht);  // all ones for a window tile
    const int64_t past = -int64_t(t >= nt);
    const bf16_t* kb = reinterpret_cast<const bf16_t*>((reinterpret_cast<intptr_t>(kc) & ~win) |
                                                       (reinterpret_cast<intptr_t>(kr) & win));
    const bf16_t* vb = reinterpret_cast<const bf16_t*>((reinterpret_cast<intptr_t>(vc) & ~win) |
                                                       (reinterpret_cast<intptr_t>(vr) & win));
    const int64_t r0 = int64_t(t) * kTB + (wdelta & win);
    const int64_t lim = ((c_max & ~win) | (whi & win)) & ~past;
    uint32_t lv = 0;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int id = (tid + c * kT) % CT, sl = id / CPR, ch = id % CPR;
      const int64_t row = r0 + sl;
      const bool ok = row < lim;
      lv |= uint32_t(ok) << c;
      const bf16_t* kp = ok ? kb + row * D : qrow;
      const bf16_t* vp = ok ? vb + row * D : qrow;
      const uint4 kw = *reinterpret_cast<const uint4*>(kp + ch * 8);
      const uint4 vw = *reinterpret_cast<const uint4*>(vp + ch * 8);
      P.k[4 * c] = kw.x; P.k[4 * c + 1] = kw.y; P.k[4 * c + 2] = kw.z; P.k[4 * c + 3] = kw.w;
      P.v[4 * c] = vw.x; P.v[4 * c + 1] = vw.y; P.v[4 * c + 2] = vw.z; P.v[4 * c + 3] = vw.w;
    }
    P.lv = lv;
    if (KV8) {
      P.ks = 1.0f;
      P.vs = 1.0f;
    }
  };
  typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
  auto stage = [&](const Pre& P, int buf, auto w16_c) __attribute__((always_inline)) {
    constexpr bool W16 = F16 && decltype(w16_c)::value;
    u16x2_t vmax = {0, 0};  // largest |V| bit patterns of the staged chunks
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int id = tid + c * kT, sl = (id % CT) / CPR, ch = id % CPR;
      if (CT >= kT || id < CT) {
        uint4 kw = make_uint4(P.k[4 * c], P.k[4 * c + 1], P.k[4 * c + 2], P.k[4 * c + 3]);
        uint4 vw = make_uint4(P.v[4 * c], P.v[4 * c + 1], P.v[4 * c + 2], P.v[4 * c + 3]);
        if (KV8 && P.f8) {
          kw = make_uint4(e4m3x2_to_bf16x2<false>(P.k[4 * c]), e4m3x2_to_bf16x2<true>(P.k[4 * c]),
                          e4m3x2_to_bf16x2<false>(P.k[4 * c + 1]), e4m3x2_to_bf16x2<true>(P.k[4 * c + 1]));
          vw = make_uint4(e4m3x2_to_bf16x2<false>(P.v[4 * c]), e4m3x2_to_bf16x2<true>(P.v[4 * c]),
                          e4m3x2_to_bf16x2<false>(P.v[4 * c + 1]), e4m3x2_to_bf16x2<true>(P.v[4 * c + 1]));
        }
        // Slots outside the heavy and window ranges hold zeros, not the row
        // they were loaded from (0 times a NaN there would be NaN).
        if (!((P.lv >> c) & 1u)) kw = vw = make_uint4(0u, 0u, 0u, 0u);
        L.k[buf][sl * LdsM<D>::KS + ch] = kw;
        L.v[buf][sl * LdsM<D>::VS + ch] = vw;
        if (W16) {
          L.vh[buf][sl * LdsM<D>::VS + ch] = make_uint4(bf16x2_to_f16x2(vw.x), bf16x2_to_f16x2(vw.y),
                                                        bf16x2_to_f16x2(vw.z), bf16x2_to_f16x2(vw.w));
          auto mag = [](uint32_t w) {
            const uint32_t m = w & 0x7fff7fffu;
            u16x2_t r;
            __builtin_memcpy(&r, &m, 4);
            return r;
          };
          vmax = __builtin_elementwise_max(vmax, __builtin_elementwise_max(mag(vw.x), mag(vw.y)));
          vmax = __builtin_elementwise_max(vmax, __builtin_elementwise_max(mag(vw.z), mag(vw.w)));
        }
      }
    }
    if (W16) {
      const uint32_t mx = vmax[0] > vmax[1] ? vmax[0] : vmax[1];
      const bool big = __ballot(mx >= 0x3A80u) != 0;  // 2^-10
      const bool ovf = __ballot(mx > 0x477Fu) != 0;   // 65280
      const bool nz = __ballot(mx != 0u) != 0;
      if (lane == 0) L.vflag[buf][wid] = uint8_t((ovf ? 4u : 0u) | (big ? 2u : 0u) | (nz ? 1u : 0u));
    }
    if (KV8 && tid < kTB) {
      L.ksc[buf][tid] = P.ks * sl2;
      L.vsc[buf][tid] = P.vs;
    }
  };

  f32x4_t o[RB][DVT];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int v = 0; v < DVT; ++v) o[rb][v] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  // Per-row softmax reference (log2 units) and partial sum, as in the kernel
  // above: the reference moves only when a score exceeds it by kSlack.
  constexpr float kSlack = 8.0f;
  float mref[RB], lpart[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    mref[rb] = -INFINITY;
    lpart[rb] = 0.0f;
  }

  // V^T operand v of a 16-bit V tile (bf16 or binary16 bits).
  auto vfrag_bits = [&](const uint4* vt, int v) __attribute__((always_inline)) {
    const int vr0 = 4 * g + col / 4, half = col & 1;
    const int ch = 2 * v + (col & 3) / 2;
    const short* b0 = reinterpret_cast<const short*>(&vt[vr0 * LdsM<D>::VS + ch]) + 4 * half;
    const short* b1 = reinterpret_cast<const short*>(&vt[(vr0 + 16) * LdsM<D>::VS + ch]) + 4 * half;
    const v4s_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)(b0));
    const v4s_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)(b1));
    uint4 w;
    __builtin_memcpy(&w.x, &t0, 8);
    __builtin_memcpy(&w.z, &t1, 8);
    return w;
  };
  // Per tile: S^T = K Q^T, the weights, then O^T += V^T P^T.  Each K and
  // each V operand read from LDS serves every row block of the wave.
  float u[RB][2][4];        // score - reference (log2 units), -inf if not visible
  uint32_t vmask[RB];       // visibility bits of a masked tile (bit 4 cg + j: slot 16 cg + 4 g + j)
  bf16x8_t ph[RB], pl[RB];  // weights as bf16 hi + lo
  f16x8_t pw[RB];           // weights as binary16
  // S^T = K Q^T of the tile in buffer buf; the 2 RB accumulators are
  // independent, so consecutive MFMAs never wait for each other.
  auto qk = [&](int buf, f32x4_t (&sc)[RB][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) sc[rb][0] = sc[rb][1] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
#pragma unroll
      for (int cg = 0; cg < 2; ++cg) {
        const bf16x8_t kv = u32x4_as_bf16x8(L.k[buf][(cg * 16 + col) * LdsM<D>::KS + 4 * kk + g]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) sc[rb][cg] = mfma16x16x32(kv, qb[rb][kk], sc[rb][cg]);
      }
  };
  // Scores and u of tile t; returns whether some row's reference must move
  // (a visible score above reference + kSlack, or the first visible one).
  auto scores = [&](int buf, int t, auto full_c) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_c)::value;
    f32x4_t sc[RB][2];
    qk(buf, sc);
    f32x4_t kf[2];  // per-slot score factors (fp8 caches)
    if (KV8)
#pragma unroll
      for (int cg = 0; cg < 2; ++cg) kf[cg] = *reinterpret_cast<const f32x4_t*>(&L.ksc[buf][cg * 16 + 4 * g]);
    const bool heavy = t < nht;
    const int64_t cb = heavy ? int64_t(t) * kTB : wlo + int64_t(t - nht) * kTB;  // slot 0's coordinate
    float umax = -INFINITY;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      uint32_t vm = 0xffu;
      if (!FULL) {
        int64_t lo = heavy ? 0 : wlr[rb], hi = heavy ? cr[rb] : tr[rb] + 1;
        lo -= cb;
        hi -= cb;
        const int vl = int(lo < 0 ? 0 : (lo > kTB ? kTB : lo));
        const int vh = int(hi < 0 ? 0 : (hi > kTB ? kTB : hi));
        vm = 0;
#pragma unroll
        for (int cg = 0; cg < 2; ++cg)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            vm |= uint32_t(uint32_t(16 * cg + 4 * g + j - vl) < uint32_t(vh - vl)) << (4 * cg + j);
        vmask[rb] = vm;
      }
      const float nref = -mref[rb];
#pragma unroll
      for (int cg = 0; cg < 2; ++cg)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x = fmaf(sc[rb][cg][j], KV8 ? kf[cg][j] : sl2, nref);
          u[rb][cg][j] = FULL ? x : (((vm >> (4 * cg + j)) & 1u) ? x : -INFINITY);
          umax = fmaxf(umax, u[rb][cg][j]);
        }
    }
    return __ballot(umax > kSlack) != 0;
  };
  // Slow path of the lazy reference: the scores are recomputed (rather than
  // kept in registers), every row's reference moves to its running maximum,
  // O and the partial sum are rescaled, u is recomputed.
  auto rescale = [&](int buf, bool full) __attribute__((always_inline)) {
    f32x4_t sc[RB][2];
    qk(buf, sc);
    f32x4_t kf[2];
#pragma unroll
    for (int cg = 0; cg < 2; ++cg)
      kf[cg] = KV8 ? *reinterpret_cast<const f32x4_t*>(&L.ksc[buf][cg * 16 + 4 * g])
                   : f32x4_t{sl2, sl2, sl2, sl2};
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float tmax = -INFINITY;
#pragma unroll
      for (int cg = 0; cg < 2; ++cg)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x = sc[rb][cg][j] * kf[cg][j];
          u[rb][cg][j] = (full || ((vmask[rb] >> (4 * cg + j)) & 1u)) ? x : -INFINITY;
          tmax = fmaxf(tmax, u[rb][cg][j]);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float mnew = fmaxf(mref[rb], tmax);
      // With no visible slot yet everything is zero: subtract 0, not -inf.
      const float msafe = (mnew == -INFINITY) ? 0.0f : mnew;
      const float corr = exp2f(mref[rb] - msafe);
      mref[rb] = mnew;
      lpart[rb] *= corr;
#pragma unroll
      for (int v = 0; v < DVT; ++v)
#pragma unroll
        for (int j = 0; j < 4; ++j) o[rb][v][j] *= corr;
#pragma unroll
      for (int cg = 0; cg < 2; ++cg)
#pragma unroll
        for (int j = 0; j < 4; ++j) u[rb][cg][j] -= msafe;
    }
  };
  // Weights 2^u as bf16 hi + lo pairs (hardware exp2 and round-to-nearest
  // conversions) and their sums.
  auto weights = [&](int buf) __attribute__((always_inline)) {
    f32x4_t vf[2];  // per-slot V scales (fp8 caches)
    if (KV8)
#pragma unroll
      for (int cg = 0; cg < 2; ++cg) vf[cg] = *reinterpret_cast<const f32x4_t*>(&L.vsc[buf][cg * 16 + 4 * g]);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      f32x2_t ps = {0.0f, 0.0f};
      uint32_t whi[4], wlo[4];
#pragma unroll
      for (int cg = 0; cg < 2; ++cg)
#pragma unroll
        for (int j = 0; j < 4; j += 2) {
          f32x2_t pp = {__builtin_amdgcn_exp2f(u[rb][cg][j]), __builtin_amdgcn_exp2f(u[rb][cg][j + 1])};
          ps = (cg == 0 && j == 0) ? pp : ps + pp;
          if (KV8) pp = f32x2_t{pp[0] * vf[cg][j], pp[1] * vf[cg][j + 1]};  // the slot's V scale
          const uint32_t hi = bf16x2_bits(pp);
          const f32x2_t back = {u32_as_f32(hi << 16), u32_as_f32(hi & 0xffff0000u)};
          whi[cg * 2 + j / 2] = hi;
          wlo[cg * 2 + j / 2] = bf16x2_bits(pp - back);
        }
      lpart[rb] += ps[0] + ps[1];
      ph[rb] = u32x4_as_bf16x8(make_uint4(whi[0], whi[1], whi[2], whi[3]));
      pl[rb] = u32x4_as_bf16x8(make_uint4(wlo[0], wlo[1], wlo[2], wlo[3]));
    }
  };
  // Weights 2^u as binary16 (one round-to-nearest conversion per pair) and
  // their sums, for tiles staged as binary16.
  auto weights16 = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      f32x2_t ps = {0.0f, 0.0f};
      uint32_t w[4];
#pragma unroll
      for (int cg = 0; cg < 2; ++cg)
#pragma unroll
        for (int j = 0; j < 4; j += 2) {
          const f32x2_t pp = {__builtin_amdgcn_exp2f(u[rb][cg][j]), __builtin_amdgcn_exp2f(u[rb][cg][j + 1])};
          ps = (cg == 0 && j == 0) ? pp : ps + pp;
          w[cg * 2 + j / 2] = f16x2_bits(pp);
        }
      lpart[rb] += ps[0] + ps[1];
      pw[rb] = u32x4_as_f16x8(make_uint4(w[0], w[1], w[2], w[3]));
    }
  };
  auto products16 = [&](const f16x8_t (&va)[DVT]) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int v = 0; v < DVT; ++v) o[rb][v] = mfma16x16x32_f16(va[v], pw[rb], o[rb][v]);
  };
  // O^T += V^T P^T (V^T operands va): every hi product, then every lo
  // product, so that the two updates of one accumulator are RB * DVT MFMAs
  // apart.
  auto products = [&](const bf16x8_t (&va)[DVT]) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int v = 0; v < DVT; ++v) o[rb][v] = mfma16x16x32(va[v], ph[rb], o[rb][v]);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int v = 0; v < DVT; ++v) o[rb][v] = mfma16x16x32(va[v], pl[rb], o[rb][v]);
  };

  // Two LDS buffers and one tile in flight in registers: tile t + 1 loads
  // while tile t computes.  Buffer t & 1 is rewritten at tile t + 2, after
  // every wave passed the barrier of tile t + 1 and hence finished tile t.
  // Tiles [0, nfull) are visible to every token of the workgroup and run
  // without visibility tests; the rest (the newest heavy tile, the windows)
  // test each slot.
  const int64_t cf = div64(t_first + 1, a.m);
  const int nfull = int((cf < a.N_alloc ? cf : a.N_alloc) / kTB);
  Pre P;
  fetch(P, 0);
  // Stages tile t (with W16, V also as binary16 and its range flags) and
  // starts loading tile t + 1.
  auto head = [&](int t, auto w16_c) __attribute__((always_inline)) {
    const int buf = t & 1;
    stage(P, buf, w16_c);
    __syncthreads();
    fetch(P, t + 1);
  };
  // Whether a staged tile, whose range flags (one byte per wave) are fl, may
  // take the binary16 path.
  auto in_range = [&](uint2 fl) __attribute__((always_inline)) {
    uint32_t f = fl.x | fl.y;
    f |= f >> 16;
    f = (f | (f >> 8)) & 0xffu;
    // In range: no |V| above 65280, and either some |V| >= 2^-10 or all zero
    // (the flags of the waves or to 0 or 3).  One bit test: a compare pair
    // here changes the register allocation of the loops enough to spill.
    f = __builtin_amdgcn_readfirstlane(f);
    return ((9u >> f) & 1u) != 0u;  // f = 0 or 3
  };
  // The math of staged tile t, on the binary16 or the bf16 hi + lo path.
  // The binary16 path tests the range only once the scores are formed (so
  // that the flag reads overlap the products) and returns false, before any
  // weight is added, for a tile outside it; the caller then does the tile
  // again on the bf16 path (a repeated score pass finds the reference already
  // moved and changes nothing).
  auto body = [&](int t, auto full_c, auto w16_c) __attribute__((always_inline)) {
    constexpr bool W16 = decltype(w16_c)::value;
    const int buf = t & 1;
    uint2 fl = make_uint2(0u, 0u);  // range flags, read first: used after the scores
    if (W16) fl = *reinterpret_cast<const uint2*>(L.vflag[buf]);
    if (__builtin_expect(scores(buf, t, full_c), 0)) rescale(buf, decltype(full_c)::value);
    // V^T operands, read after the scores (read before them, the reads of the
    // 8 waves, which leave the barrier together, queue on LDS).
    uint4 vbits[DVT];
#pragma unroll
    for (int v = 0; v < DVT; ++v) vbits[v] = vfrag_bits(W16 ? L.vh[buf] : L.v[buf], v);
    if (W16 && !in_range(fl)) return false;
    if (W16) {
      f16x8_t va[DVT];
#pragma unroll
      for (int v = 0; v < DVT; ++v) va[v] = u32x4_as_f16x8(vbits[v]);
      weights16();
      products16(va);
    } else {
      bf16x8_t va[DVT];
#pragma unroll
      for (int v = 0; v < DVT; ++v) va[v] = u32x4_as_bf16x8(vbits[v]);
      weights(buf);
      products(va);
    }
    return true;
  };
  // Binary16 tiles first; the first tile outside the binary16 range (already
  // staged) and every later one take the bf16 loops.  Each loop has one path,
  // which keeps the register allocation of either (a per-tile choice inside
  // one loop spills).
  int t = 0;
  bool staged = false;  // tile t is staged and its successor is loading
  if (F16) {
    for (; t < nfull && !staged; ++t) {
      head(t, std::true_type{});
      if (!body(t, std::true_type{}, std::true_type{})) {
        staged = true;
        break;
      }
    }
    for (; t < nt && !staged; ++t) {
      head(t, std::true_type{});
      if (!body(t, std::false_type{}, std::true_type{})) {
        staged = true;
        break;
      }
    }
  }
  for (; t < nfull; ++t) {
    if (!staged) head(t, std::false_type{});
    staged = false;
    body(t, std::true_type{}, std::false_type{});
  }
  for (; t < nt; ++t) {
    if (!staged) head(t, std::false_type{});
    staged = false;
    body(t, std::false_type{}, std::false_type{});
  }

#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float lt = lpart[rb];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const int64_t i = iw + rb;
    if (i > ilast) continue;
    const int64_t row = b * T + i;
    const int h = h0 + col;
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
#pragma unroll
    for (int v = 0; v < DVT; ++v) {
      const int64_t oi = (row * H + h) * int64_t(D) + v * 16 + 4 * g;
      if (a.out_bf16) {
        const uint32_t w0 = uint32_t(f32_to_bf16(o[rb][v][0] * inv)) | (uint32_t(f32_to_bf16(o[rb][v][1] * inv)) << 16);
        const uint32_t w1 = uint32_t(f32_to_bf16(o[rb][v][2] * inv)) | (uint32_t(f32_to_bf16(o[rb][v][3] * inv)) << 16);
        *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(a.out) + oi) = make_uint2(w0, w1);
      } else {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + oi) =
            make_float4(o[rb][v][0] * inv, o[rb][v][1] * inv, o[rb][v][2] * inv, o[rb][v][3] * inv);
      }
    }
    if (a.lse && g == 0) a.lse[row * H + h] = lt > 0.0f ? (mref[rb] + log2f(lt)) * kLn2 : -INFINITY;
  }
}

// Log-sum-exp merge of the split partials: one thread per (row, head, 16-byte
// column chunk).  The (max, sum) pairs and partial rows of up to 16 splits are
// loaded together, so every load of a thread is in flight at once; longer rows
// fold further groups of 16 in with an online rescale.
template <int D>
__global__ __launch_bounds__(256) void attend_merge_kernel(AttendArgs a, AttendPlan p) {
  constexpr int CPH = D / 4;  // float4 chunks per head
  constexpr int G = 16;       // splits per load group
  const int H = a.H;
  const int64_t gi = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (gi >= p.rows * H * CPH) return;
  const int cc = int(gi % CPH) * 4;
  const int64_t rh = gi / CPH;
  const int64_t r = div64(rh, H);
  const int h = int(rh - r * H);
  const RowSlots x = row_slots(a, p, r, 0);
  if (x.S <= 1) return;  // written directly by the attention kernel
  const int S = int(x.S);
  const uint8_t* ws = reinterpret_cast<const uint8_t*>(a.ws);
  const float* part = reinterpret_cast<const float*>(ws + p.off_part) + (r * p.splits * H + h) * int64_t(D) + cc;
  const float* ml = reinterpret_cast<const float*>(ws + p.off_ml) + (r * p.splits * H + h) * 2;
  // 32-bit strides (the workspace offsets of one row fit; checked at launch).
  const uint32_t pstride = uint32_t(H) * D, mstride = uint32_t(H) * 2;
  float M = -INFINITY, Lsum = 0.0f;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int s0 = 0; s0 < S; s0 += G) {
    float2 m2[G];
    float4 v[G];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const uint32_t sp = uint32_t((s0 + u) < S ? s0 + u : S - 1);  // clamped: every load is issued
      m2[u] = *reinterpret_cast<const float2*>(ml + sp * mstride);
      v[u] = *reinterpret_cast<const float4*>(part + sp * pstride);
    }
    // Every load above is issued before any result is used (otherwise the
    // compiler interleaves the weights' arithmetic with the loads and waits
    // for each partial in turn, serialising their latencies).
    __builtin_amdgcn_sched_barrier(0);
    float mc = M;
#pragma unroll
    for (int u = 0; u < G; ++u)
      if (s0 + u < S) mc = fmaxf(mc, m2[u].x);
    // With no live slot so far everything is zero: subtract 0 instead of -inf.
    const float ms = (mc == -INFINITY) ? 0.0f : mc;
    const float corr = exp2f(M - ms);
    Lsum *= corr;
    acc.x *= corr; acc.y *= corr; acc.z *= corr; acc.w *= corr;
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const float w = (s0 + u < S) ? exp2f(m2[u].x - ms) : 0.0f;
      Lsum = fmaf(w, m2[u].y, Lsum);
      acc.x = fmaf(w, v[u].x, acc.x); acc.y = fmaf(w, v[u].y, acc.y);
      acc.z = fmaf(w, v[u].z, acc.z); acc.w = fmaf(w, v[u].w, acc.w);
    }
    M = mc;
  }
  const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
  acc.x *= inv; acc.y *= inv; acc.z *= inv; acc.w *= inv;
  const int64_t oi = rh * D + cc;
  if (a.out_bf16) {
    const uint32_t w0 = uint32_t(f32_to_bf16(acc.x)) | (uint32_t(f32_to_bf16(acc.y)) << 16);
    const uint32_t w1 = uint32_t(f32_to_bf16(acc.z)) | (uint32_t(f32_to_bf16(acc.w)) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(a.out) + oi) = make_uint2(w0, w1);
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + oi) = acc;
  }
  if (a.lse && cc == 0) a.lse[rh] = Lsum > 0.0f ? (M + log2f(Lsum)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------- fp32 kernel
//
// One workgroup = one (row, split) of at most 32 heads, four waves: wave w owns
// heads w, w + 4, ... (HPW of them).  Tiles of 64 slots go through LDS, K as
// rows (scores: lane = slot) and V transposed (O: lane = output column), while
// the next tile's rows are already being loaded into registers.  Each K or V
// value read from LDS serves every head of the wave, and each dot product runs
// as two interleaved partial sums.  LDS traffic and vector instructions bound
// it (16-byte accesses throughout; the tile arrays are 16-byte aligned, which
// the compiler needs in order to emit them).

template <int D, int HPW>
struct TileF32 {
  static constexpr int KS = D + 4;         // K row stride in floats: 16-byte reads of 16 lanes hit distinct banks
  static constexpr int VS = kTileF32 + 4;  // V^T row stride in floats
  alignas(16) float k[kTileF32][KS];  // 16-byte aligned rows: one 16-byte LDS access per float4
  alignas(16) float vt[D][VS];
  alignas(16) float q[4 * HPW][D];
  alignas(16) float pr[4 * HPW][kTileF32];
  uint32_t live[kTileF32];  // all ones for a live slot, 0 for a skipped one
};

template <int D, int HPW>
struct LdsF32 {
  union U {
    TileF32<D, HPW> t;
    MergeLds merge;  // used once every wave is past the last tile (arrive_last synchronises first)
  } u;
  uint32_t flag[4];
};

template <int D, int HPW>
__global__ __launch_bounds__(kThreads) void attend_f32_kernel(AttendArgs a, AttendPlan p) {
  __shared__ LdsF32<D, HPW> L;
  debug_poison_lds(L);
  int64_t hg, r, s;
  if (!decode_block(p, hg, r, s)) return;
  const RowSlots x = row_slots(a, p, r, s);
  if (s >= x.S) return;
  TileF32<D, HPW>& T = L.u.t;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int H = a.H;  // <= 4 * HPW
  constexpr int DPL = (D + 63) / 64;               // output columns per lane
  constexpr int CPR = D / 4;                       // float4 chunks per row
  constexpr int NCH = kTileF32 * CPR / kThreads;   // chunks per thread per tensor per tile
  static_assert(NCH >= 1 && NCH * kThreads == kTileF32 * CPR && kTileF32 == 64, "a lane per slot, whole chunks per wave");
  const float* qrow = reinterpret_cast<const float*>(a.q) + r * int64_t(H) * D;
  // Query rows of the heads; the rows past H are zeros, so that the loops below
  // run every head slot of a wave without a branch (their results are dropped).
  for (int i = tid; i < 4 * HPW * D; i += kThreads) T.q[i / D][i % D] = i < H * D ? qrow[i] : 0.0f;
  const float sl2 = a.scale * kLog2e;
  const float* kc = reinterpret_cast<const float*>(a.k_cmp);
  const float* vc = reinterpret_cast<const float*>(a.v_cmp);
  const float* kr = reinterpret_cast<const float*>(a.k_raw);
  const float* vr = reinterpret_cast<const float*>(a.v_raw);

  // Tile rows in flight: lane l of every wave loads slot t0 + l, wave w its
  // chunks w * NCH .. w * NCH + NCH - 1 (so a thread finds one source row per
  // tile, and the transposing V writes of a wave hit 64 distinct banks).  A
  // skipped slot or one past the split holds zeros.
  float4 pk[NCH], pv[NCH];
  bool plive = false;
  auto fetch = [&](int64_t t0) __attribute__((always_inline)) {
    const int64_t slot = t0 + lane;
    int64_t off = -1;
    bool cmp = false;
    if (slot < x.hi) off = slot_offset(a, x, slot, cmp);
    plive = off >= 0;
    // A dead slot reads the query row instead (at least D floats), so that every
    // load is issued unconditionally; its values are replaced by zeros when staged.
    const float* kp = (plive ? (cmp ? kc : kr) + off : qrow) + wid * NCH * 4;
    const float* vp = (plive ? (cmp ? vc : vr) + off : qrow) + wid * NCH * 4;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      pk[c] = *reinterpret_cast<const float4*>(kp + c * 4);
      pv[c] = *reinterpret_cast<const float4*>(vp + c * 4);
    }
  };
  auto stage = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ch = wid * NCH + c;
      const float4 z = make_float4(0, 0, 0, 0);
      const float4 kw = plive ? pk[c] : z, vw = plive ? pv[c] : z;
      *reinterpret_cast<float4*>(&T.k[lane][ch * 4]) = kw;
      T.vt[ch * 4][lane] = vw.x;
      T.vt[ch * 4 + 1][lane] = vw.y;
      T.vt[ch * 4 + 2][lane] = vw.z;
      T.vt[ch * 4 + 3][lane] = vw.w;
    }
    if (wid == 0) T.live[lane] = plive ? 0xffffffffu : 0u;
  };

  float o[HPW][DPL];
  float mrun[HPW], lpart[HPW];
#pragma unroll
  for (int u = 0; u < HPW; ++u) {
    mrun[u] = -INFINITY;
    lpart[u] = 0.0f;
#pragma unroll
    for (int c = 0; c < DPL; ++c) o[u][c] = 0.0f;
  }
  fetch(x.lo);
  for (int64_t t0 = x.lo; t0 < x.hi; t0 += kTileF32) {
    __syncthreads();  // every wave is done with the previous tile
    stage();
    __syncthreads();
    if (t0 + kTileF32 < x.hi) fetch(t0 + kTileF32);
    // Scores of slot `lane` for the wave's heads.
    const bool live = T.live[lane] != 0u;
    float d0[HPW], d1[HPW];
#pragma unroll
    for (int u = 0; u < HPW; ++u) d0[u] = d1[u] = 0.0f;
#pragma unroll
    for (int dd = 0; dd < D; dd += 8) {
      const float4 k0 = *reinterpret_cast<const float4*>(&T.k[lane][dd]);
      const float4 k1 = *reinterpret_cast<const float4*>(&T.k[lane][dd + 4]);
#pragma unroll
      for (int u = 0; u < HPW; ++u) {
        const int h = wid + 4 * u;
        const float4 q0 = *reinterpret_cast<const float4*>(&T.q[h][dd]);
        const float4 q1 = *reinterpret_cast<const float4*>(&T.q[h][dd + 4]);
        d0[u] = fmaf(q0.x, k0.x, d0[u]); d1[u] = fmaf(q1.x, k1.x, d1[u]);
        d0[u] = fmaf(q0.y, k0.y, d0[u]); d1[u] = fmaf(q1.y, k1.y, d1[u]);
        d0[u] = fmaf(q0.z, k0.z, d0[u]); d1[u] = fmaf(q1.z, k1.z, d1[u]);
        d0[u] = fmaf(q0.w, k0.w, d0[u]); d1[u] = fmaf(q1.w, k1.w, d1[u]);
      }
    }
    // Online softmax per head (log2 units); the weights go to LDS for O.
#pragma unroll
    for (int u = 0; u < HPW; ++u) {
      const int h = wid + 4 * u;
      const float sv = live ? (d0[u] + d1[u]) * sl2 : -INFINITY;
      const float mnew = fmaxf(mrun[u], wave_max_dpp(sv));
      // Hardware 2^x: results below the normal range flush to 0, far below what
      // can matter next to the row maximum's weight of 1.
      const float corr = (mnew == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(mrun[u] - mnew);
      const float pw = (mnew == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(sv - mnew);
      mrun[u] = mnew;
      lpart[u] = lpart[u] * corr + pw;
      T.pr[h][lane] = pw;
#pragma unroll
      for (int c = 0; c < DPL; ++c) o[u][c] *= corr;
    }
    // O += P V for output column lane + 64 c (the weights were written by this
    // same wave, whose LDS accesses complete in order).
    float oa[HPW][DPL], ob[HPW][DPL];
#pragma unroll
    for (int u = 0; u < HPW; ++u)
#pragma unroll
      for (int c = 0; c < DPL; ++c) {
        oa[u][c] = o[u][c];
        ob[u][c] = 0.0f;
      }
#pragma unroll 2
    for (int e = 0; e < kTileF32; e += 8) {
      float4 v0[DPL], v1[DPL];
#pragma unroll
      for (int c = 0; c < DPL; ++c) {
        const int dv = lane + 64 * c;
        v0[c] = v1[c] = make_float4(0, 0, 0, 0);
        if (dv < D) {
          v0[c] = *reinterpret_cast<const float4*>(&T.vt[dv][e]);
          v1[c] = *reinterpret_cast<const float4*>(&T.vt[dv][e + 4]);
        }
      }
#pragma unroll
      for (int u = 0; u < HPW; ++u) {
        const int h = wid + 4 * u;
        const float4 p0 = *reinterpret_cast<const float4*>(&T.pr[h][e]);
        const float4 p1 = *reinterpret_cast<const float4*>(&T.pr[h][e + 4]);
#pragma unroll
        for (int c = 0; c < DPL; ++c) {
          oa[u][c] = fmaf(p0.x, v0[c].x, oa[u][c]); ob[u][c] = fmaf(p1.x, v1[c].x, ob[u][c]);
          oa[u][c] = fmaf(p0.y, v0[c].y, oa[u][c]); ob[u][c] = fmaf(p1.y, v1[c].y, ob[u][c]);
          oa[u][c] = fmaf(p0.z, v0[c].z, oa[u][c]); ob[u][c] = fmaf(p1.z, v1[c].z, ob[u][c]);
          oa[u][c] = fmaf(p0.w, v0[c].w, oa[u][c]); ob[u][c] = fmaf(p1.w, v1[c].w, ob[u][c]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < HPW; ++u)
#pragma unroll
      for (int c = 0; c < DPL; ++c) o[u][c] = oa[u][c] + ob[u][c];
  }
  float lt[HPW];
#pragma unroll
  for (int u = 0; u < HPW; ++u) lt[u] = wave_sum(lpart[u]);
  if (x.S == 1) {
#pragma unroll
    for (int u = 0; u < HPW; ++u) {
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
  for (int u = 0; u < HPW; ++u) {
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
  finish_split(a, p, x, unit, 0, H, H, L.flag, L.u.merge);
}

}  // namespace

AttendPlan plan_attend(bool bf16, int B, int64_t T, int H, int d, int64_t max_entries, int window) {
  AttendPlan p{};
  p.rows = int64_t(B) * T;
  p.slots = max_entries + window;
  size_t off = kHeaderBytes;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (bytes + 255) & ~size_t(255);
    return o;
  };
  if (bf16) {
    // Split the slots until there are about 256 workgroups, keeping at least 4
    // tiles of 32 per split (2 with at most 64 heads, whose split partials are
    // half the size to merge).  Every head of a row in one workgroup, except
    // for split rows with few workgroups (kFewSplitHeadGroups).
    auto split_plan = [&](int64_t target) {
      int64_t splits = target;
      const int64_t min_slots = (H > 64 ? 4 : 2) * kTB;
      const int64_t max_splits = (p.slots + min_slots - 1) / min_slots;
      if (splits > max_splits) splits = max_splits;
      if (splits > kMaxSplits) splits = kMaxSplits;
      if (splits < 1) splits = 1;
      int64_t per = (p.slots + splits - 1) / splits;
      per = ((per + kTB - 1) / kTB) * kTB;
      if (per < kTB) per = kTB;
      p.per_split = per;
      p.splits = (p.slots + per - 1) / per;
      if (p.splits < 1) p.splits = 1;
    };
    p.groups = 1;
    split_plan((p.rows > 0 && p.rows < 256) ? (256 + p.rows - 1) / p.rows : 1);
    if (p.splits > 1 && p.rows * p.splits < 128 && H % (16 * kFewSplitHeadGroups) == 0)
      p.groups = kFewSplitHeadGroups;
    // Head groups of one (row, split) get block ids equal modulo 8 (one XCD).
    p.group_stride = p.groups > 1 ? (p.rows * p.splits + 7) / 8 * 8 : p.rows * p.splits;
    p.off_part = take(size_t(p.rows * p.splits) * size_t(H) * size_t(d) * 4);
    p.off_ml = take(size_t(p.rows * p.splits) * size_t(H) * 2 * 4);
    p.ws_bytes = p.splits > 1 ? off : 0;
    return p;
  }
  p.groups = (H + kAttendGroupHeads - 1) / kAttendGroupHeads;
  const int64_t tile = 64;  // fp32 tile
  // Split rows until there are about 256 workgroups, keeping >= 2 tiles per split.
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
  const size_t U = size_t(units);
  const size_t nh = size_t(H < kAttendGroupHeads ? H : kAttendGroupHeads);
  p.off_part = take(U * size_t(p.splits) * nh * d * 4);
  p.off_ml = take(U * size_t(p.splits) * nh * 2 * 4);
  p.ws_bytes = p.splits > 1 ? off : 0;
  return p;
}

int64_t attend_grid(const AttendPlan& p, bool bf16) {
  (void)bf16;
  return p.groups * p.group_stride;
}

template <int D, bool HCA, int PAIR, bool KV8>
static void launch_bf16_nw(const AttendArgs& a, const AttendPlan& p, dim3 grid) {
  const int nw = int((a.H / p.groups + 15) / 16);  // waves: 16 heads each, the heads of one group
  // Split rows of at most 4 head waves: two tile halves (twice the waves).
  constexpr int TH = PAIR == 2 ? 2 : 1;
  if (nw <= 2) hipLaunchKernelGGL((attend_bf16_kernel<D, 2, HCA, PAIR, KV8, TH>), grid, dim3(128 * TH), 0, a.stream, a, p);
  else if (nw <= 4) hipLaunchKernelGGL((attend_bf16_kernel<D, 4, HCA, PAIR, KV8, TH>), grid, dim3(256 * TH), 0, a.stream, a, p);
  else hipLaunchKernelGGL((attend_bf16_kernel<D, 8, HCA, PAIR, KV8>), grid, dim3(512), 0, a.stream, a, p);
}

template <int D, bool HCA>
static void launch_bf16(const AttendArgs& a, const AttendPlan& p) {
  const dim3 grid(unsigned(attend_grid(p, true)));
  {
    ProfScope prof(HCA ? "hca_attend" : "csa_attend", a.stream);
    // Split rows (decode) have one workgroup per CU: stage tiles in pairs.  Many
    // unsplit rows (prefill) keep the smaller LDS footprint for occupancy.
    if (p.splits > 1) a.kv8 ? launch_bf16_nw<D, HCA, 2, true>(a, p, grid) : launch_bf16_nw<D, HCA, 2, false>(a, p, grid);
    else a.kv8 ? launch_bf16_nw<D, HCA, 1, true>(a, p, grid) : launch_bf16_nw<D, HCA, 1, false>(a, p, grid);
  }
  if (p.splits > 1) {
    ProfScope prof(HCA ? "hca_attend_merge" : "csa_attend_merge", a.stream);
    const int64_t threads = p.rows * a.H * (D / 4);
    hipLaunchKernelGGL((attend_merge_kernel<D>), dim3(unsigned((threads + 255) / 256)), dim3(256), 0,
                       a.stream, a, p);
  }
}

// fp32: heads per wave from the head count (at most 32 heads, four waves).
template <int D>
static void launch_f32(const AttendArgs& a, const AttendPlan& p, dim3 grid, dim3 block) {
  if (a.H <= 4) hipLaunchKernelGGL((attend_f32_kernel<D, 1>), grid, block, 0, a.stream, a, p);
  else if (a.H <= 8) hipLaunchKernelGGL((attend_f32_kernel<D, 2>), grid, block, 0, a.stream, a, p);
  else if (a.H <= 16) hipLaunchKernelGGL((attend_f32_kernel<D, 4>), grid, block, 0, a.stream, a, p);
  else hipLaunchKernelGGL((attend_f32_kernel<D, 8>), grid, block, 0, a.stream, a, p);
}

// HCA prefill: QT = RB * NW / (H / 16) consecutive tokens per workgroup.
template <int D, int NW, int RB>
static bool launch_hca_multi(const AttendArgs& a) {
  const int HW = a.H / 16;
  if (HW > NW || NW % HW != 0) return false;
  const int QT = RB * (NW / HW);
  const int64_t gps = (a.T + QT - 1) / QT;
  const dim3 grid(unsigned(int64_t(a.B) * gps)), block(NW * 64);
  if (a.kv8) hipLaunchKernelGGL((hca_multi_kernel<D, NW, RB, true>), grid, block, 0, a.stream, a, gps);
  else hipLaunchKernelGGL((hca_multi_kernel<D, NW, RB, false>), grid, block, 0, a.stream, a, gps);
  return true;
}

template <int D>
static bool hca_multi(const AttendArgs& a) {
  return launch_hca_multi<D, 8, 2>(a);
}

// Rows per sequence from which HCA uses the multi-token kernel (when the rows
// are numerous enough not to need slot splits).
constexpr int64_t kHcaMultiMinT = 16;

hipError_t launch_attend(const AttendArgs& a, const AttendPlan& p) {
  if (p.rows == 0) return hipSuccess;
  CSA_HOST_CHECK(p.splits >= 1 && p.per_split >= 1 && p.splits * p.per_split >= p.slots);
  CSA_HOST_CHECK(p.splits == 1 || (a.ws != nullptr && p.off_part >= kHeaderBytes && p.off_ml > p.off_part &&
                                   p.off_ml <= p.ws_bytes));
  if (kDebug && p.splits > 1 && p.ws_bytes > kHeaderBytes) {
    const hipError_t e = debug_poison(static_cast<uint8_t*>(a.ws) + kHeaderBytes, p.ws_bytes - kHeaderBytes, a.stream);
    if (e != hipSuccess) return e;
  }
  const bool multi = a.bf16 && a.hca && p.splits == 1 && a.T >= kHcaMultiMinT && 8 % (a.H / 16) == 0;
  log_dispatch("%s: B=%d T=%lld H=%d d=%d %s -> %s, %lld rows x %lld splits of %lld slots%s", a.hca ? "hca_attend" : "csa_attend",
               a.B, (long long)a.T, a.H, a.d, a.bf16 ? (a.kv8 ? "bf16, fp8 cache" : "bf16") : "fp32",
               multi ? "multi-token kernel" : (a.bf16 ? "bf16 kernel" : "fp32 kernel"), (long long)p.rows,
               (long long)p.splits, (long long)p.per_split, p.splits > 1 ? " + merge" : "");
  // The multi-token kernel takes 8 / (H / 16) tokens per wave pair: H / 16 must divide 8.
  if (a.bf16 && a.hca && p.splits == 1 && a.T >= kHcaMultiMinT && 8 % (a.H / 16) == 0) {
    ProfScope prof("hca_attend", a.stream);
    if (a.d == 128 ? hca_multi<128>(a) : hca_multi<64>(a)) return hipGetLastError();
  }
  if (a.bf16) {
    if (a.d == 128) a.hca ? launch_bf16<128, true>(a, p) : launch_bf16<128, false>(a, p);
    else a.hca ? launch_bf16<64, true>(a, p) : launch_bf16<64, false>(a, p);
  } else {
    ProfScope prof(a.hca ? "hca_attend" : "csa_attend", a.stream);
    dim3 grid(unsigned(p.groups * p.group_stride)), block(kThreads);
    if (a.d == 128) launch_f32<128>(a, p, grid, block);
    else if (a.d == 64) launch_f32<64>(a, p, grid, block);
    else launch_f32<32>(a, p, grid, block);
  }
  return hipGetLastError();
}

}  // namespace csa

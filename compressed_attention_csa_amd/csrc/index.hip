// Lightning-Indexer scoring and exact per-query top-k for gfx950 (rows x slices path).
//
// V4 report digest, section 三: an indexer scores the compressed entries and only
// the top-k enter the core attention; section 七: the indexer keys are cached in
// low precision.  Score of entry j for query row r (position t):
//     I(r, j) = sum_h w[r,h] * max(0, q[r,h] . k[j]),  j < c(t) = min(N, (t+1)/m)
// The selection is the min(k, c(t)) best entries by (score desc, index asc).
//
// Design.  A row's visible entries are cut into slices; one workgroup scores one
// slice of one row.  Every WG keeps its fp32 scores as order-preserving uint32
// keys in LDS.
//   * A row with one slice is finished by that WG: an LDS radix select finds
//     the kk-th best (score, index) and the winners are written in index order.
//   * A longer row uses two kernels.  Kernel 1: each WG adds its 4096-bin
//     histogram of the top 12 key bits to the row histogram and stores its
//     keys; the last WG of the row to arrive locates the bin holding the kk-th
//     best score.  Kernel 2: each WG compacts its entries above that bin and
//     its entries inside it (in index order) into per-slice staging; the last
//     WG concatenates the slices in order and radix-selects the boundary bin.
// The output order is deterministic: the winners above the boundary bin in
// increasing entry index, then the boundary winners in increasing entry index.
// bf16 / e4m3 keys are scored with 16x16x32 bf16 MFMA (query heads as rows,
// entries as columns; e4m3 codes are widened exactly to bf16 in registers);
// fp32 keys use fp32 FMA with one entry per lane.
#include "common.hpp"
#include "kernels.h"

namespace csa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

struct RowCtrl {
  uint32_t arrive1, arrive2, bin, above;
};

struct RowInfo {
  int64_t r, b, i, t, c, kk, S, lo, hi;
};

__device__ __forceinline__ RowInfo row_info(const IndexArgs& a, const IndexPlan& p, int64_t r,
                                            int64_t s) {
  RowInfo ri;
  ri.r = r;
  ri.b = r / a.T;
  ri.i = r % a.T;
  ri.t = a.t0 + ri.i;
  int64_t c = (ri.t + 1) / a.m;
  ri.c = c < a.N_alloc ? c : a.N_alloc;
  ri.kk = ri.c < a.top_k ? ri.c : a.top_k;
  int64_t S = (ri.c + p.slice - 1) / p.slice;
  ri.S = S < 1 ? 1 : S;
  ri.lo = s * p.slice;
  int64_t hi = ri.lo + p.slice;
  ri.hi = hi < ri.c ? hi : ri.c;
  if (ri.hi < ri.lo) ri.hi = ri.lo;
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

// ---------------------------------------------------------------- scoring

// Scores of entries [lo, hi) of row ri into keys[0 .. hi-lo).
template <int KK>
__device__ void score_slice(const IndexArgs& a, const RowInfo& ri, uint32_t* keys, float* s_q) {
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
    for (int64_t e = tid; e < n; e += kThreads) {
      float kv[64];
      const float4* kp = reinterpret_cast<const float4*>(kbase + e * d_I);
      for (int v = 0; v < d_I / 4; ++v) {
        float4 x = kp[v];
        kv[4 * v] = x.x; kv[4 * v + 1] = x.y; kv[4 * v + 2] = x.z; kv[4 * v + 3] = x.w;
      }
      float score = 0.0f;
      for (int h = 0; h < H_I; ++h) {
        const float* qh = s_q + h * d_I;
        float dot = 0.0f;
        for (int dd = 0; dd < d_I; ++dd) dot = fmaf(qh[dd], kv[dd], dot);
        score = fmaf(s_q[16 * 64 + h], fmaxf(dot, 0.0f), score);
      }
      keys[e] = score_key(score);
    }
    __syncthreads();
    return;
  } else {
    const int lane = tid & 63, wid = tid >> 6, g = lane >> 4, col = lane & 15;
    const bf16_t* q = reinterpret_cast<const bf16_t*>(a.q_idx) + qrow * d_I;
    // A operands: row = head col (zero past H_I), k-slots 8g..8g+7.
    bf16x8_t qa0, qa1;
    {
      uint4 v0 = make_uint4(0, 0, 0, 0), v1 = make_uint4(0, 0, 0, 0);
      if (col < H_I) {
        if (d_I == 64) {
          v0 = *reinterpret_cast<const uint4*>(q + col * 64 + 16 * g);
          v1 = *reinterpret_cast<const uint4*>(q + col * 64 + 16 * g + 8);
        } else {
          v0 = *reinterpret_cast<const uint4*>(q + col * 32 + 8 * g);
        }
      }
      qa0 = u32x4_as_bf16x8(v0);
      qa1 = u32x4_as_bf16x8(v1);
    }
    float wr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int h = 4 * g + j;
      wr[j] = (h < H_I) ? (a.w ? a.w[qrow + h] : 1.0f) : 0.0f;
    }
    const int64_t kb = ri.b * a.N_alloc + ri.lo;
    const int64_t ngroups = (n + 15) / 16;
    for (int64_t gi = wid; gi < ngroups; gi += kWaves) {
      const int64_t e = gi * 16 + col;
      const bool valid = e < n;
      uint4 k0 = make_uint4(0, 0, 0, 0), k1 = make_uint4(0, 0, 0, 0);
      float ksc = 1.0f;
      if (valid) {
        if (KK == kKeyBF16) {
          const bf16_t* kp = reinterpret_cast<const bf16_t*>(a.k_idx) + (kb + e) * d_I;
          if (d_I == 64) {
            k0 = *reinterpret_cast<const uint4*>(kp + 16 * g);
            k1 = *reinterpret_cast<const uint4*>(kp + 16 * g + 8);
          } else {
            k0 = *reinterpret_cast<const uint4*>(kp + 8 * g);
          }
        } else {
          const uint8_t* kp = reinterpret_cast<const uint8_t*>(a.k_idx) + (kb + e) * d_I;
          ksc = a.k_scale[kb + e];
          if (d_I == 64) {
            uint4 raw = *reinterpret_cast<const uint4*>(kp + 16 * g);
            e4m3x4_to_bf16x4(raw.x, k0.x, k0.y);
            e4m3x4_to_bf16x4(raw.y, k0.z, k0.w);
            e4m3x4_to_bf16x4(raw.z, k1.x, k1.y);
            e4m3x4_to_bf16x4(raw.w, k1.z, k1.w);
          } else {
            uint2 raw = *reinterpret_cast<const uint2*>(kp + 8 * g);
            e4m3x4_to_bf16x4(raw.x, k0.x, k0.y);
            e4m3x4_to_bf16x4(raw.y, k0.z, k0.w);
          }
        }
      }
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
      acc = mfma16x16x32(qa0, u32x4_as_bf16x8(k0), acc);
      if (d_I == 64) acc = mfma16x16x32(qa1, u32x4_as_bf16x8(k1), acc);
      float part = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) part = fmaf(wr[j], fmaxf(acc[j], 0.0f), part);
      part += __shfl_xor(part, 16);
      part += __shfl_xor(part, 32);
      if (KK == kKeyE4M3) part *= ksc;
      if (valid && g == 0) keys[e] = score_key(part);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- radix selection

// The need-th largest 64-bit rank key among n candidates whose top `fixed_bits`
// bits equal `prefix` (callers guarantee that).  get(i) returns candidate i.
// All threads call it; the result is uniform.
template <typename Get>
__device__ uint64_t kth_largest(int64_t n, int64_t need, uint64_t prefix, int fixed_bits, Get get,
                                uint32_t* hist, uint32_t* s_misc) {
  const int tid = threadIdx.x;
  int hi_bit = 64 - fixed_bits;  // bits [0, hi_bit) still open
  while (hi_bit > 0) {
    const int width = hi_bit >= 8 ? 8 : hi_bit;
    const int shift = hi_bit - width;
    for (int x = tid; x < 256; x += kThreads) hist[x] = 0;
    __syncthreads();
    const uint64_t hi_mask = (hi_bit >= 64) ? 0ull : (~0ull << hi_bit);
    for (int64_t i = tid; i < n; i += kThreads) {
      uint64_t v = get(i);
      if ((v & hi_mask) == (prefix & hi_mask))
        atomicAdd(&hist[uint32_t(v >> shift) & ((1u << width) - 1u)], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      int64_t cum = 0;
      int dstar = 0;
      for (int dd = (1 << width) - 1; dd >= 0; --dd) {
        if (cum + hist[dd] >= need) { dstar = dd; break; }
        cum += hist[dd];
      }
      s_misc[0] = uint32_t(dstar);
      s_misc[1] = uint32_t(cum);
    }
    __syncthreads();
    prefix |= uint64_t(s_misc[0]) << shift;
    need -= int64_t(s_misc[1]);
    hi_bit = shift;
    __syncthreads();
  }
  return prefix;
}

__device__ __forceinline__ void write_pads(const IndexArgs& a, int64_t r, int64_t from) {
  for (int64_t x = from + threadIdx.x; x < a.top_k; x += kThreads) {
    a.out_idx[r * a.top_k + x] = -1;
    if (a.out_score) a.out_score[r * a.top_k + x] = -INFINITY;
  }
}

struct LdsSel {
  uint32_t keys[kMaxSlice];
  uint32_t hist[kHistBins];
  float q[16 * 64 + 16];
  int wave[kWaves];
  uint32_t misc[4];
};

// ---------------------------------------------------------------- kernel 1

template <int KK>
__global__ __launch_bounds__(kThreads) void idx_score_kernel(IndexArgs a, IndexPlan p, int64_t row0) {
  __shared__ LdsSel L;
  const int64_t lr = blockIdx.x / p.slices;  // row within this launch
  const int64_t r = row0 + lr;
  const int64_t s = blockIdx.x % p.slices;
  const RowInfo ri = row_info(a, p, r, s);
  if (s >= ri.S) return;
  const int tid = threadIdx.x;
  const int64_t n = ri.hi - ri.lo;

  score_slice<KK>(a, ri, L.keys, L.q);

  if (ri.S == 1) {
    // Whole row in this WG.
    const int64_t kk = ri.kk;
    if (kk < n) {
      const uint32_t base = uint32_t(ri.lo);
      auto get = [&](int64_t x) { return rank_key(L.keys[x], base + uint32_t(x)); };
      const uint64_t kstar = kth_largest(n, kk, 0ull, 0, get, L.hist, L.misc);
      int64_t done = 0;
      for (int64_t x0 = 0; x0 < n; x0 += kThreads) {
        const int64_t x = x0 + tid;
        const bool win = x < n && get(x) >= kstar;
        int total;
        const int pos = block_rank(win, L.wave, total);
        if (win) {
          a.out_idx[r * a.top_k + done + pos] = int32_t(ri.lo + x);
          if (a.out_score) a.out_score[r * a.top_k + done + pos] = key_score(L.keys[x]);
        }
        done += total;
      }
    } else {
      for (int64_t x = tid; x < n; x += kThreads) {
        a.out_idx[r * a.top_k + x] = int32_t(ri.lo + x);
        if (a.out_score) a.out_score[r * a.top_k + x] = key_score(L.keys[x]);
      }
    }
    write_pads(a, r, kk);
    return;
  }

  // Multi-slice row: publish keys and histogram.
  uint8_t* ws = reinterpret_cast<uint8_t*>(a.ws);
  RowCtrl* ctrl = reinterpret_cast<RowCtrl*>(ws + kIndexCtrlOff) + lr;
  uint32_t* ghist = reinterpret_cast<uint32_t*>(ws + kIndexHistOff) + lr * kHistBins;
  uint32_t* gkeys = reinterpret_cast<uint32_t*>(ws + p.off_keys) + lr * a.N_alloc;
  for (int x = tid; x < kHistBins; x += kThreads) L.hist[x] = 0;
  __syncthreads();
  for (int64_t x = tid; x < n; x += kThreads) {
    const uint32_t k = L.keys[x];
    gkeys[ri.lo + x] = k;
    atomicAdd(&L.hist[k >> 20], 1u);
  }
  __syncthreads();
  for (int x = tid; x < kHistBins; x += kThreads)
    if (L.hist[x]) atomicAdd(&ghist[x], L.hist[x]);
  __threadfence();
  __syncthreads();
  if (tid == 0) L.misc[0] = (atomicAdd(&ctrl->arrive1, 1u) == uint32_t(ri.S - 1)) ? 1u : 0u;
  __syncthreads();
  if (!L.misc[0]) return;
  __threadfence();
  // Last WG of the row: find the bin that holds the kk-th best key.
  for (int x = tid; x < kHistBins; x += kThreads) {
    L.hist[x] = __hip_atomic_load(&ghist[x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ghist[x] = 0;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t cum = 0, bin = kHistBins;
    const uint32_t kk = uint32_t(ri.kk);
    if (kk > 0) {
      for (int x = kHistBins - 1; x >= 0; --x) {
        if (cum + L.hist[x] >= kk) { bin = uint32_t(x); break; }
        cum += L.hist[x];
      }
    }
    ctrl->bin = bin;
    ctrl->above = cum;
    ctrl->arrive1 = 0;
  }
}

// ---------------------------------------------------------------- kernel 2

__global__ __launch_bounds__(kThreads) void idx_select_kernel(IndexArgs a, IndexPlan p, int64_t row0) {
  __shared__ uint32_t hist[256];
  __shared__ int s_wave[kWaves];
  __shared__ uint32_t misc[4];
  __shared__ int64_t s_pref_a[1025], s_pref_b[1025];
  const int64_t lr = blockIdx.x / p.slices;
  const int64_t r = row0 + lr;
  const int64_t s = blockIdx.x % p.slices;
  const RowInfo ri = row_info(a, p, r, s);
  if (ri.S == 1 || s >= ri.S) return;
  const int tid = threadIdx.x;
  uint8_t* ws = reinterpret_cast<uint8_t*>(a.ws);
  RowCtrl* ctrl = reinterpret_cast<RowCtrl*>(ws + kIndexCtrlOff) + lr;
  const uint32_t* gkeys = reinterpret_cast<const uint32_t*>(ws + p.off_keys) + lr * a.N_alloc;
  uint32_t* stage_a = reinterpret_cast<uint32_t*>(ws + p.off_stage_a) + lr * a.N_alloc;
  uint64_t* stage_b = reinterpret_cast<uint64_t*>(ws + p.off_stage_b) + lr * a.N_alloc;
  uint32_t* counts = reinterpret_cast<uint32_t*>(ws + p.off_counts) + lr * p.slices * 2;
  const uint32_t bin = ctrl->bin;

  int64_t na = 0, nb = 0;
  for (int64_t x0 = ri.lo; x0 < ri.hi; x0 += kThreads) {
    const int64_t j = x0 + tid;
    const bool in = j < ri.hi;
    const uint32_t k = in ? gkeys[j] : 0u;
    const bool isa = in && (k >> 20) > bin;
    const bool isb = in && (k >> 20) == bin;
    int ta, tb;
    const int pa = block_rank(isa, s_wave, ta);
    const int pb = block_rank(isb, s_wave, tb);
    if (isa) stage_a[ri.lo + na + pa] = uint32_t(j);
    if (isb) stage_b[ri.lo + nb + pb] = rank_key(k, uint32_t(j));
    na += ta;
    nb += tb;
  }
  if (tid == 0) {
    counts[2 * s] = uint32_t(na);
    counts[2 * s + 1] = uint32_t(nb);
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) misc[0] = (atomicAdd(&ctrl->arrive2, 1u) == uint32_t(ri.S - 1)) ? 1u : 0u;
  __syncthreads();
  if (!misc[0]) return;
  __threadfence();

  // Last WG: concatenate the slices in order.
  const int64_t S = ri.S;
  if (tid == 0) {
    int64_t ca = 0, cb = 0;
    for (int64_t x = 0; x < S; ++x) {
      s_pref_a[x] = ca;
      s_pref_b[x] = cb;
      ca += __hip_atomic_load(&counts[2 * x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      cb += __hip_atomic_load(&counts[2 * x + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    s_pref_a[S] = ca;
    s_pref_b[S] = cb;
  }
  __syncthreads();
  const int64_t tot_a = s_pref_a[S], tot_b = s_pref_b[S];
  auto slice_of = [&](const int64_t* pref, int64_t g) {
    int64_t lo = 0, hi = S - 1;  // last x with pref[x] <= g
    while (lo < hi) {
      int64_t mid = (lo + hi + 1) >> 1;
      if (pref[mid] <= g) lo = mid; else hi = mid - 1;
    }
    return lo;
  };
  for (int64_t gidx = tid; gidx < tot_a; gidx += kThreads) {
    const int64_t x = slice_of(s_pref_a, gidx);
    const uint32_t j = stage_a[x * p.slice + (gidx - s_pref_a[x])];
    a.out_idx[r * a.top_k + gidx] = int32_t(j);
    if (a.out_score) a.out_score[r * a.top_k + gidx] = key_score(gkeys[j]);
  }
  const int64_t need = ri.kk - tot_a;
  if (need > 0) {
    auto get = [&](int64_t gidx) {
      const int64_t x = slice_of(s_pref_b, gidx);
      return stage_b[x * p.slice + (gidx - s_pref_b[x])];
    };
    uint64_t kstar = 0;
    if (need < tot_b) kstar = kth_largest(tot_b, need, uint64_t(bin) << 52, 12, get, hist, misc);
    int64_t done = 0;
    for (int64_t g0 = 0; g0 < tot_b; g0 += kThreads) {
      const int64_t gidx = g0 + tid;
      const uint64_t v = gidx < tot_b ? get(gidx) : 0ull;
      const bool win = gidx < tot_b && v >= kstar;
      int total;
      const int pos = block_rank(win, s_wave, total);
      if (win) {
        a.out_idx[r * a.top_k + tot_a + done + pos] = int32_t(rank_key_idx(v));
        if (a.out_score) a.out_score[r * a.top_k + tot_a + done + pos] = key_score(uint32_t(v >> 32));
      }
      done += total;
    }
  }
  write_pads(a, r, ri.kk);
  if (tid == 0) {
    ctrl->arrive2 = 0;
    ctrl->bin = 0;
    ctrl->above = 0;
  }
}

}  // namespace

IndexPlan plan_index(int B, int64_t T, int64_t N_alloc, int top_k) {
  (void)top_k;
  IndexPlan p{};
  p.rows = int64_t(B) * T;
  p.c_max = N_alloc;
  // Aim for about 512 workgroups over the chip (256 CUs), slices of 256..4096 entries.
  int64_t want = (p.rows > 0) ? (p.c_max * p.rows + 511) / 512 : 1;
  int64_t slice = ((want + 255) / 256) * 256;
  if (slice < 256) slice = 256;
  if (slice > kMaxSlice) slice = kMaxSlice;
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
  p.off_keys = take(R * size_t(N_alloc) * 4);
  p.off_stage_a = take(R * size_t(N_alloc) * 4);
  p.off_stage_b = take(R * size_t(N_alloc) * 8);
  p.off_counts = take(R * size_t(p.slices) * 8);
  p.ws_bytes = multi ? off : 0;
  return p;
}

hipError_t launch_index_topk(const IndexArgs& a, const IndexPlan& p) {
  if (p.rows == 0) return hipSuccess;
  const dim3 block(kThreads);
  for (int64_t row0 = 0; row0 < p.rows; row0 += p.chunk_rows) {
    const int64_t nr = (p.rows - row0) < p.chunk_rows ? (p.rows - row0) : p.chunk_rows;
    const dim3 grid(unsigned(nr * p.slices));
    if (a.key_kind == kKeyF32)
      hipLaunchKernelGGL(idx_score_kernel<kKeyF32>, grid, block, 0, a.stream, a, p, row0);
    else if (a.key_kind == kKeyBF16)
      hipLaunchKernelGGL(idx_score_kernel<kKeyBF16>, grid, block, 0, a.stream, a, p, row0);
    else
      hipLaunchKernelGGL(idx_score_kernel<kKeyE4M3>, grid, block, 0, a.stream, a, p, row0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (p.slices > 1) {
      hipLaunchKernelGGL(idx_select_kernel, grid, block, 0, a.stream, a, p, row0);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace csa
